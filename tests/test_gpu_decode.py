"""GPU parity of the SAMU generation step (samu_scan_decode through the C ABI)
against the FP64 oracle: one step is the scan's recurrence at L = 1 from the
given state, and T steps in a row are the scan over T tokens."""
import numpy as np
import pytest
import torch

import oracle
from linear_recurrence_sequence_amd import inputs
from tests.helpers import dev_tensor, rel_l2, say, to_f64

pytestmark = pytest.mark.gpu

TOL_OUT = 1e-5


def _dev(inp):
    return {k: dev_tensor(v) for k, v in inp.items()}


def _params(d):
    return (d["w_phi"], d["w_r"], d["a_phi"], d["a_r"], d["nu"], d["theta"])


@pytest.mark.parametrize("table", [False, True], ids=["per_step_constants", "prepared_table"])
# an odd batch with a mode count that leaves the last 256-mode workgroup partial,
# and the widest state the library accepts (2^20 channels)
@pytest.mark.parametrize("B,D,std", [(3, 64, 0.5), (1, 2048, 0.1), (256, 2048, 0.1), (5, 1032, None),
                                     (67, 1032, 0.5), (2, 1 << 20, 0.1)])
def test_decode_step_matches_oracle(B, D, std, table):
    from linear_recurrence_sequence_amd import scan
    inp = inputs.samu_inputs(B, 1, D, 500 + D + B, z0_std=std, with_dy=False)
    say(f"[samu decode] B={B} D={D} z_in={'yes' if std else 'zero'} table={table}: oracle")
    rf = oracle.samu_fwd(inp["x_sel"], inp["b"], inp["w_phi"], inp["w_r"], inp["a_phi"], inp["a_r"],
                         inp["nu"], inp["theta"], inp["z0"])
    d = _dev(inp)
    tab = scan.samu_scan_decode_prepare(d["w_phi"], d["w_r"], d["a_phi"], d["a_r"], d["nu"], d["theta"]) if table else None
    say(f"[samu decode] B={B} D={D}: samu_scan_decode f32 and bf16")
    y, z = scan.samu_scan_decode(d["x_sel"][:, 0].contiguous(), d["b"][:, 0].contiguous(), *_params(d),
                                 d["z0"], y_dtype=torch.float32, table=tab)
    yb, zb = scan.samu_scan_decode(d["x_sel"][:, 0].contiguous(), d["b"][:, 0].contiguous(), *_params(d),
                                   d["z0"], y_dtype=torch.bfloat16, table=tab)
    torch.cuda.synchronize()
    ey = rel_l2(to_f64(y), rf["y"][:, 0])
    ez = rel_l2(to_f64(z), rf["z_final"])
    say(f"   errors: y {ey:.2e} z {ez:.2e}")
    assert ey <= TOL_OUT and ez <= TOL_OUT
    assert torch.equal(yb, y.to(torch.bfloat16)) and torch.equal(zb, z)


@pytest.mark.parametrize("table", [False, True], ids=["per_step_constants", "prepared_table"])
def test_decode_steps_in_place_equal_the_scan(table):
    """T = 200 steps with the state updated in place reproduce the oracle's
    scan over the same 200 tokens (every output and the final state)."""
    from linear_recurrence_sequence_amd import scan
    B, T, D = 2, 200, 256
    inp = inputs.samu_inputs(B, T, D, 77, z0_std=0.1, with_dy=False)
    say(f"[samu decode] {T} steps in place, B={B} D={D} table={table}: oracle scan")
    rf = oracle.samu_fwd(inp["x_sel"], inp["b"], inp["w_phi"], inp["w_r"], inp["a_phi"], inp["a_r"],
                         inp["nu"], inp["theta"], inp["z0"])
    d = _dev(inp)
    tab = scan.samu_scan_decode_prepare(d["w_phi"], d["w_r"], d["a_phi"], d["a_r"], d["nu"], d["theta"]) if table else None
    z = d["z0"].clone()
    ys = []
    say(f"[samu decode] {T} steps in place: samu_scan_decode")
    for t in range(T):
        y, z2 = scan.samu_scan_decode(d["x_sel"][:, t].contiguous(), d["b"][:, t].contiguous(),
                                      *_params(d), z, y_dtype=torch.float32, z_out=z, table=tab)
        assert z2.data_ptr() == z.data_ptr()
        ys.append(y)
    torch.cuda.synchronize()
    yall = torch.stack(ys, dim=1)
    ey = rel_l2(to_f64(yall), rf["y"])
    ez = rel_l2(to_f64(z), rf["z_final"])
    say(f"   errors: y {ey:.2e} z_final {ez:.2e}")
    assert ey <= TOL_OUT and ez <= TOL_OUT


def test_decode_bitwise_deterministic():
    from linear_recurrence_sequence_amd import scan
    inp = inputs.samu_inputs(4, 1, 512, 91, z0_std=0.3, with_dy=False)
    d = _dev(inp)
    say("[samu decode] determinism B=4 D=512")
    a = scan.samu_scan_decode(d["x_sel"][:, 0].contiguous(), d["b"][:, 0].contiguous(), *_params(d),
                              d["z0"], y_dtype=torch.float32)
    b = scan.samu_scan_decode(d["x_sel"][:, 0].contiguous(), d["b"][:, 0].contiguous(), *_params(d),
                              d["z0"], y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_graph_replays_match_eager():
    """32 in-place steps captured in a HIP graph: every replay, started from
    the same state (restored eagerly between replays), equals the eager run."""
    from linear_recurrence_sequence_amd import scan
    B, D, T = 4, 512, 32
    inp = inputs.samu_inputs(B, T, D, 123, z0_std=0.1, with_dy=False)
    d = _dev(inp)
    xs = [d["x_sel"][:, t].contiguous() for t in range(T)]
    bs = [d["b"][:, t].contiguous() for t in range(T)]
    z = d["z0"].clone()
    y = torch.empty((B, D // 2, 2), dtype=torch.float32, device="cuda")
    tab = scan.samu_scan_decode_prepare(d["w_phi"], d["w_r"], d["a_phi"], d["a_r"], d["nu"], d["theta"])

    def steps():
        for t in range(T):
            scan.samu_scan_decode(xs[t], bs[t], *_params(d), z, y=y, z_out=z, table=tab if t % 2 else None)

    say("[samu decode] graph: eager reference")
    steps()
    torch.cuda.synchronize()
    z_ref, y_ref = z.clone(), y.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        z.copy_(d["z0"])
        steps()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("[samu decode] graph: capture")
    g = torch.cuda.CUDAGraph()
    z.copy_(d["z0"])
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        steps()
    for r in range(4):
        say(f"[samu decode] graph: replay {r}")
        z.copy_(d["z0"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(z, z_ref) and torch.equal(y, y_ref), r


def test_decode_table_and_per_step_constants_agree():
    """The prepared table holds the same FP32 hi + lo phasors the per-step
    path forms; only the direction norms are summed in another order, so
    the two states agree to FP32 rounding (each is within 1e-5 of the
    oracle, checked above)."""
    from linear_recurrence_sequence_amd import scan
    inp = inputs.samu_inputs(16, 1, 2048, 92, z0_std=0.1, with_dy=False)
    d = _dev(inp)
    tab = scan.samu_scan_decode_prepare(d["w_phi"], d["w_r"], d["a_phi"], d["a_r"], d["nu"], d["theta"])
    say("[samu decode] table against per-step constants B=16 D=2048")
    a = scan.samu_scan_decode(d["x_sel"][:, 0].contiguous(), d["b"][:, 0].contiguous(), *_params(d), d["z0"],
                              y_dtype=torch.float32)
    b = scan.samu_scan_decode(d["x_sel"][:, 0].contiguous(), d["b"][:, 0].contiguous(), *_params(d), d["z0"],
                              y_dtype=torch.float32, table=tab)
    torch.cuda.synchronize()
    ea = rel_l2(to_f64(a[1]), to_f64(b[1]))
    say(f"   table vs per-step state: rel {ea:.2e}")
    assert ea <= 1e-6
