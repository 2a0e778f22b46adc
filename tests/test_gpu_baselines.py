"""GPU parity of the two comparison scans (per-channel sequential and
recursive associative, forward only) against the FP64 oracle, for SAMU and
RG-LRU, including the largest shape of the scan-latency sweep (B=8, D=1024,
L=16384)."""
import pytest
import torch

import oracle
from linear_recurrence_sequence_amd import inputs
from tests.helpers import dev_tensor, rel_l2, say, to_f64

pytestmark = pytest.mark.gpu

TOL_OUT = 1e-5
VARIANTS = ["sequential", "associative"]
SHAPES = [(2, 300, 64, 0.1), (1, 777, 40, 0.1), (3, 1, 16, 0.1), (1, 4099, 128, None), (8, 16384, 1024, None)]


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("B,L,D,std", SHAPES)
def test_samu_baseline_parity(variant, B, L, D, std):
    from linear_recurrence_sequence_amd import scan
    inp = inputs.samu_inputs(B, L, D, 31 + L, z0_std=std, with_dy=False)
    say(f"[samu {variant}] B={B} L={L} D={D}: oracle")
    rf = oracle.samu_fwd(inp["x_sel"], inp["b"], inp["w_phi"], inp["w_r"], inp["a_phi"], inp["a_r"],
                         inp["nu"], inp["theta"], inp["z0"])
    d = {k: dev_tensor(v) for k, v in inp.items()}
    say(f"[samu {variant}] B={B} L={L} D={D}: samu_scan_baseline_fwd f32")
    y, zf = scan.samu_scan_baseline_fwd(variant, d["x_sel"], d["b"], d["w_phi"], d["w_r"], d["a_phi"],
                                        d["a_r"], d["nu"], d["theta"], d["z0"], y_dtype=torch.float32)
    yb, zb = scan.samu_scan_baseline_fwd(variant, d["x_sel"], d["b"], d["w_phi"], d["w_r"], d["a_phi"],
                                         d["a_r"], d["nu"], d["theta"], d["z0"], y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ey, ez = rel_l2(to_f64(y), rf["y"]), rel_l2(to_f64(zf), rf["z_final"])
    say(f"   errors: y {ey:.2e} z_final {ez:.2e}")
    assert ey <= TOL_OUT and ez <= TOL_OUT
    assert torch.equal(yb, y.to(torch.bfloat16)) and torch.equal(zb, zf)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("B,L,D,std,reset_p", [(2, 300, 64, 0.1, 1 / 32), (1, 777, 10, 0.1, 0.0),
                                               (3, 1, 8, 0.1, 0.0), (8, 16384, 1024, None, 0.0)])
def test_rglru_baseline_parity(variant, B, L, D, std, reset_p):
    from linear_recurrence_sequence_amd import scan
    inp = inputs.rglru_inputs(B, L, D, 57 + L, reset_p=reset_p, h0_std=std, with_dy=False)
    say(f"[rglru {variant}] B={B} L={L} D={D} resets p={reset_p}: oracle")
    rf = oracle.rglru_fwd(inp["x"], inp["lx"], inp["la"], inp["alpha"], inp["reset"], inp["h0"])
    d = {k: dev_tensor(v) for k, v in inp.items()}
    say(f"[rglru {variant}] B={B} L={L} D={D}: rglru_scan_baseline_fwd f32")
    y, hf = scan.rglru_scan_baseline_fwd(variant, d["x"], d["lx"], d["la"], d["alpha"], d["reset"], d["h0"],
                                         y_dtype=torch.float32)
    yb, hb = scan.rglru_scan_baseline_fwd(variant, d["x"], d["lx"], d["la"], d["alpha"], d["reset"],
                                          d["h0"], y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ey, eh = rel_l2(to_f64(y), rf["y"]), rel_l2(to_f64(hf), rf["h_final"])
    say(f"   errors: y {ey:.2e} h_final {eh:.2e}")
    assert ey <= TOL_OUT and eh <= TOL_OUT
    assert torch.equal(yb, y.to(torch.bfloat16)) and torch.equal(hb, hf)
