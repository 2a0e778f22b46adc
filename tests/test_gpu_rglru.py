"""GPU parity of the RG-LRU scan (C ABI through the thin binding) against the
FP64 oracle, on the same seeded inputs; same tolerances and BF16 criterion as
the SAMU parity tests."""
import numpy as np
import pytest
import torch

import oracle
from linear_recurrence_sequence_amd import inputs
from tests.helpers import bf16_floor, dev_tensor, rel_l2, say, to_f64

pytestmark = pytest.mark.gpu

TOL_OUT, TOL_GRAD = 1e-5, 1e-4

# (name, B, L, D, K, G, reset_p, state_std)
CASES = [
    ("packed_small", 4, 600, 256, 16, 0, 1.0 / 64, 0.1),
    ("ragged_groups", 2, 77, 6, 16, 2, 0.1, 0.1),
    ("k32_groups", 1, 1000, 64, 32, 4, 0.0, 0.1),
    ("shorter_than_chunk", 1, 5, 10, 16, 0, 0.0, 0.1),
    ("serial_prefix", 2, 500, 130, 16, 1000, 0.02, None),
    ("resets_everywhere", 1, 40, 8, 16, 1, 1.0, 0.1),
]


def _inputs(name, B, L, D, reset_p, std):
    seed = 9000 + sum(map(ord, name))
    inp = inputs.rglru_inputs(B, L, D, seed, reset_p=reset_p, h0_std=std, dh_final_std=std)
    if inp["reset"] is not None and name == "ragged_groups":
        inp["reset"][0, 0] = 1
        inp["reset"][1, 20:22] = 1
    return inp, seed


def _oracle(inp):
    f = oracle.rglru_fwd(inp["x"], inp["lx"], inp["la"], inp["alpha"], inp["reset"], inp["h0"])
    h0 = inp["h0"] if inp["h0"] is not None else np.zeros(inp["x"].shape[::2], np.float32)
    g = oracle.rglru_bwd(inp["x"], inp["lx"], inp["la"], inp["alpha"], inp["reset"], h0, inp["dy"],
                         inp["dh_final"])
    return f, g


def _gpu(inp, K, G, dtype):
    from linear_recurrence_sequence_amd import scan
    d = {k: dev_tensor(v) for k, v in inp.items()}
    y, hf, saved = scan.rglru_scan_fwd(d["x"], d["lx"], d["la"], d["alpha"], d["reset"], d["h0"],
                                       K=K, G=G, y_dtype=dtype)
    g = scan.rglru_scan_bwd(d["x"], d["lx"], d["la"], d["alpha"], d["reset"], saved, d["dy"],
                            d["dh_final"], K=K, G=G, grad_dtype=dtype)
    torch.cuda.synchronize()
    return y, hf, g


def _check(name, inp, K, G, bf16=True):
    say(f"[rglru parity] {name}: oracle")
    rf, rg = _oracle(inp)
    say(f"[rglru parity] {name}: rglru_scan_fwd/bwd f32 K={K} G={G}")
    y, hf, g = _gpu(inp, K, G, torch.float32)
    errs = {"y": rel_l2(to_f64(y), rf["y"]), "h_final": rel_l2(to_f64(hf), rf["h_final"])}
    for k in ("dx", "dlx", "dla", "dalpha", "dh0"):
        errs[k] = rel_l2(to_f64(g[k]), rg[k])
    say("   errors:", {k: f"{v:.2e}" for k, v in errs.items()})
    for k in ("y", "h_final"):
        assert errs[k] <= TOL_OUT, (k, errs[k])
    for k in ("dx", "dlx", "dla", "dalpha", "dh0"):
        assert errs[k] <= TOL_GRAD, (k, errs[k])
    if not bf16:
        return
    say(f"[rglru parity] {name}: rglru_scan_fwd/bwd bf16")
    yb, hfb, gb = _gpu(inp, K, G, torch.bfloat16)
    assert torch.equal(yb, y.to(torch.bfloat16))
    assert torch.equal(hfb, hf)
    for k in ("dx", "dlx", "dla"):
        assert torch.equal(gb[k], g[k].to(torch.bfloat16)), k
        assert rel_l2(to_f64(gb[k]), rg[k]) <= bf16_floor(rg[k]) + TOL_GRAD, k
    for k in ("dalpha", "dh0"):
        assert torch.equal(gb[k], g[k]), k
    assert rel_l2(to_f64(yb), rf["y"]) <= bf16_floor(rf["y"]) + TOL_OUT


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_rglru_parity(case):
    name, B, L, D, K, G, p, std = case
    inp, _ = _inputs(name, B, L, D, p, std)
    _check(name, inp, K, G)


def test_rglru_bitwise_deterministic():
    inp, _ = _inputs("det", 2, 900, 96, 1.0 / 100, 0.1)
    say("[rglru determinism] B=2 L=900 D=96 twice")
    a = _gpu(inp, 16, 4, torch.float32)
    b = _gpu(inp, 16, 4, torch.float32)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    for k in a[2]:
        assert torch.equal(a[2][k], b[2][k]), k


def test_rglru_packed_full_size_parity():
    """The packed-sequence workload at full size: B=4, L=8192, D=2560,
    segment starts with p = 1/512, nonzero initial state."""
    name = "packed_b4_l8192_d2560"
    inp = inputs.rglru_inputs(4, 8192, 2560, 4000, reset_p=1.0 / 512, h0_std=0.1)
    _check(name, inp, 16, 0, bf16=False)


# The pages' other full-size RG-LRU workloads (no segment starts): the long
# sequence at D=1024 and the widest state at L=32768 with an initial state.
FULL_CASES = [
    ("long_b1_l131072_d1024", 1, 131072, 1024, None, 2102),
    ("wide_b1_l32768_d2560", 1, 32768, 2560, 0.1, 3103),
]


@pytest.mark.parametrize("case", FULL_CASES, ids=[c[0] for c in FULL_CASES])
def test_rglru_full_size_parity(case):
    name, B, L, D, std, seed = case
    inp = inputs.rglru_inputs(B, L, D, seed, h0_std=std)
    _check(name, inp, 16, 0, bf16=False)


@pytest.mark.parametrize("L", [2048, 16384])
def test_rglru_forward_sweep_parity(L):
    """Forward-only latency sweep workload: B=8, D=1024, no resets, zero
    initial state."""
    B, D, K = 8, 1024, 16
    inp = inputs.rglru_inputs(B, L, D, 1100 + L // 2048, with_dy=False)
    say(f"[rglru parity] sweep_b8_l{L}_d1024: oracle forward")
    rf = oracle.rglru_fwd(inp["x"], inp["lx"], inp["la"], inp["alpha"], None, None)
    d = {k: dev_tensor(v) for k, v in inp.items()}
    from linear_recurrence_sequence_amd import scan
    say(f"[rglru parity] sweep_b8_l{L}_d1024: rglru_scan_fwd f32")
    y, hf, _ = scan.rglru_scan_fwd(d["x"], d["lx"], d["la"], d["alpha"], None, None, K=K, G=0,
                                   y_dtype=torch.float32)
    torch.cuda.synchronize()
    ey, eh = rel_l2(to_f64(y), rf["y"]), rel_l2(to_f64(hf), rf["h_final"])
    say(f"   errors: y {ey:.2e} h_final {eh:.2e}")
    assert ey <= TOL_OUT and eh <= TOL_OUT
