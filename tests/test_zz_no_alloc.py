"""samu_scan_fwd_noalloc, the forward that takes its workspace from a static
device array instead of a caller buffer, called through the C ABI: its y,
z_final and saved record must give exactly what samu_scan_fwd gives with a
caller workspace (the same kernels), on two calls in a row where the second
is smaller than the first (so stale contents of the shared array from the
first call must not leak into the second), and must match the FP64 oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from linear_recurrence_sequence_amd import inputs, scan
from tests.helpers import bf16_floor, dev_tensor, rel_l2, say, to_f64

pytestmark = pytest.mark.gpu


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _noalloc(d, B, L, D, K, G, dtype):
    M = D // 2
    y = torch.empty((B, L, M, 2), dtype=dtype, device="cuda")
    zf = torch.empty((B, M, 2), dtype=torch.float32, device="cuda")
    saved = torch.empty(scan.samu_scan_saved_bytes(B, L, D, K), dtype=torch.uint8, device="cuda")
    code = scan.SCAN_F32 if dtype == torch.float32 else scan.SCAN_BF16
    st = scan.lib().samu_scan_fwd_noalloc(
        B, L, D, K, G, _ptr(d["x_sel"]), _ptr(d["b"]), _ptr(d["w_phi"]), _ptr(d["w_r"]), _ptr(d["a_phi"]),
        _ptr(d["a_r"]), _ptr(d["nu"]), _ptr(d["theta"]), _ptr(d["z0"]), _ptr(y), code, _ptr(zf), _ptr(saved),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, scan.lib().scan_last_error().decode()
    return y, zf, saved


def _bwd(d, saved, K, G):
    return scan.samu_scan_bwd(d["x_sel"], d["b"], d["w_phi"], d["w_r"], d["a_phi"], d["a_r"], d["nu"],
                              d["theta"], saved, d["dy"], d["dz_final"], K=K, G=G, grad_dtype=torch.float32)


# first the metric shape (the larger workspace), then a smaller ragged one
CALLS = [("metric_b1_l32768_d2048", 1, 32768, 2048, 32, 0, torch.bfloat16),
         ("ragged_b2_l1000_d520", 2, 1000, 520, 32, 3, torch.float32)]


def test_noalloc_forward_matches_allocating_forward():
    for name, B, L, D, K, G, dtype in CALLS:
        inp = inputs.samu_inputs(B, L, D, 7700 + L, z0_std=0.1, dz_final_std=0.1)
        d = {k: dev_tensor(v) for k, v in inp.items()}
        say(f"[noalloc] {name}: samu_scan_fwd_noalloc B={B} L={L} D={D} K={K} G={G} {dtype}")
        y, zf, saved = _noalloc(d, B, L, D, K, G, dtype)
        say(f"[noalloc] {name}: samu_scan_fwd with a caller workspace")
        y2, zf2, saved2 = scan.samu_scan_fwd(d["x_sel"], d["b"], d["w_phi"], d["w_r"], d["a_phi"], d["a_r"],
                                             d["nu"], d["theta"], d["z0"], K=K, G=G, y_dtype=dtype)
        torch.cuda.synchronize()
        assert torch.equal(y, y2) and torch.equal(zf, zf2)
        # the saved records drive identical backward passes
        say(f"[noalloc] {name}: samu_scan_bwd from both saved records")
        g1 = _bwd(d, saved, K, G)
        g2 = _bwd(d, saved2, K, G)
        torch.cuda.synchronize()
        for k in g1:
            assert torch.equal(g1[k], g2[k]), k
        say(f"[noalloc] {name}: oracle forward")
        rf = oracle.samu_fwd(inp["x_sel"], inp["b"], inp["w_phi"], inp["w_r"], inp["a_phi"], inp["a_r"],
                             inp["nu"], inp["theta"], inp["z0"])
        ey, ez = rel_l2(to_f64(y), rf["y"]), rel_l2(to_f64(zf), rf["z_final"])
        say(f"   errors: y {ey:.2e} z_final {ez:.2e}")
        floor = bf16_floor(rf["y"]) if dtype == torch.bfloat16 else 0.0
        assert ey <= floor + 1e-5 and ez <= 1e-5
        del d, y, zf, saved, y2, zf2, saved2, g1, g2


def test_noalloc_rejects_shapes_beyond_its_scratch():
    B, L, D, K = 16, 131072, 2048, 32      # forward workspace well above 32 MiB
    need = scan.samu_scan_workspace_bytes(B, L, D, K, 0, False)
    assert need > (32 << 20)
    x = torch.empty(16, dtype=torch.uint8, device="cuda")
    p = ctypes.c_void_p(x.data_ptr())
    st = scan.lib().samu_scan_fwd_noalloc(B, L, D, K, 0, *([p] * 8), None, p, 0, None, p, None)
    assert st == -4
    assert b"static scratch" in scan.lib().scan_last_error()
