"""The Python binding refuses, before any pointer reaches the C ABI, every
tensor whose dtype, shape or size the kernels would misread: the library sees
raw pointers only and cannot check allocation sizes itself.  These run on the
CPU (host tensors are enough: the checks come before the device check)."""
import os

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "linear_recurrence_sequence_amd", "libsamu_scan.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libsamu_scan.so not built")

B, L, D = 2, 40, 16
M = D // 2
bf, f32 = torch.bfloat16, torch.float32


def _samu():
    return dict(x_sel=torch.zeros(B, L, D, dtype=bf), b=torch.zeros(B, L, M, 2, dtype=bf),
                w_phi=torch.ones(D + 1), w_r=torch.ones(D + 1), a_phi=torch.zeros(1), a_r=torch.zeros(1),
                nu=torch.ones(M), theta=torch.zeros(M))


def _fwd(**over):
    from linear_recurrence_sequence_amd import scan
    a = _samu()
    kw = {k: over.pop(k) for k in list(over) if k in ("y", "z_final", "saved", "workspace", "K", "z0")}
    a.update(over)
    return scan.samu_scan_fwd(a["x_sel"], a["b"], a["w_phi"], a["w_r"], a["a_phi"], a["a_r"], a["nu"],
                              a["theta"], **kw)


@pytest.mark.parametrize("over,msg", [
    (dict(x_sel=torch.zeros(B, L, D)), "x_sel has dtype"),                    # FP32 read as BF16 words
    (dict(b=torch.zeros(B, L, M, 2)), "b has dtype"),
    (dict(b=torch.zeros(B, L - 1, M, 2, dtype=bf)), "b has shape"),           # short drive
    (dict(w_phi=torch.ones(D)), "w_phi has shape"),                           # D entries, not D+1
    (dict(w_r=torch.ones(D + 1, dtype=torch.float64)), "w_r has dtype"),
    (dict(nu=torch.ones(M + 1)), "nu has shape"),
    (dict(a_r=torch.zeros(2)), "a_r has shape"),
    (dict(z0=torch.zeros(B, M, 2, dtype=bf)), "z0 has dtype"),
    (dict(y=torch.empty(B, L, M, 2, dtype=torch.float16)), "y has dtype"),
    (dict(y=torch.empty(B, L - 1, M, 2, dtype=bf)), "y has shape"),           # undersized output
    (dict(z_final=torch.empty(B, M)), "z_final has shape"),
    (dict(saved=torch.empty(64, dtype=torch.uint8)), "saved holds"),
    (dict(workspace=torch.empty(64, dtype=torch.uint8)), "workspace holds"),
    (dict(K=24), "saved: unsupported shape"),
])
def test_samu_fwd_binding_rejects(over, msg):
    with pytest.raises(ValueError, match=msg):
        _fwd(**over)


def test_samu_fwd_binding_passes_valid_host_tensors_to_the_device_check():
    # everything well formed: the only complaint left is that the tensors are on the host
    with pytest.raises(ValueError, match="device tensor"):
        _fwd()


def test_samu_bwd_binding_rejects_wrong_record_and_cotangent():
    from linear_recurrence_sequence_amd import scan
    a = _samu()
    n16 = scan.samu_scan_saved_bytes(B, L, D, 16)
    n32 = scan.samu_scan_saved_bytes(B, L, D, 32)
    rec = torch.empty(max(n16, n32), dtype=torch.uint8)
    rec._lrs_record = ("samu", B, L, D, 16)          # as a K=16 forward would tag it
    args = [a[k] for k in ("x_sel", "b", "w_phi", "w_r", "a_phi", "a_r", "nu", "theta")]
    dy = torch.zeros(B, L, M, 2, dtype=bf)
    with pytest.raises(ValueError, match="written by a forward"):
        scan.samu_scan_bwd(*args, rec, dy, K=32)
    with pytest.raises(ValueError, match="saved holds"):
        scan.samu_scan_bwd(*args, torch.empty(16, dtype=torch.uint8), dy, K=32)
    with pytest.raises(ValueError, match="dy has dtype"):
        scan.samu_scan_bwd(*args, torch.empty(n32, dtype=torch.uint8), dy.float(), K=32)
    with pytest.raises(ValueError, match="dy has shape"):
        scan.samu_scan_bwd(*args, torch.empty(n32, dtype=torch.uint8), dy[:, 1:].contiguous(), K=32)
    out = dict(dx_sel=torch.empty(B, L, D, dtype=bf), db=torch.empty(B, L, M, 2, dtype=f32),
               dz0=None, dw_phi=torch.empty(D + 1), dw_r=torch.empty(D + 1), da_phi=torch.empty(1),
               da_r=torch.empty(1), dnu=torch.empty(M), dtheta=torch.empty(M))
    with pytest.raises(ValueError, match="db has dtype"):   # gradients share one dtype
        scan.samu_scan_bwd(*args, torch.empty(n32, dtype=torch.uint8), dy, K=32, out=out)


def test_rglru_bindings_reject():
    from linear_recurrence_sequence_amd import scan
    x = torch.zeros(B, L, D, dtype=bf)
    al = torch.zeros(D)
    with pytest.raises(ValueError, match="lx has dtype"):
        scan.rglru_scan_fwd(x, torch.zeros(B, L, D), x, al)
    with pytest.raises(ValueError, match="alpha has shape"):
        scan.rglru_scan_fwd(x, x, x, torch.zeros(D + 1))
    with pytest.raises(ValueError, match="reset has shape"):
        scan.rglru_scan_fwd(x, x, x, al, torch.zeros(B, L + 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="h0 has shape"):
        scan.rglru_scan_fwd(x, x, x, al, None, torch.zeros(B, D + 2))
    n = scan.rglru_scan_saved_bytes(B, L, D, 16)
    rec = torch.empty(n, dtype=torch.uint8)
    rec._lrs_record = ("rglru", B, L, D, 32)
    with pytest.raises(ValueError, match="written by a forward"):
        scan.rglru_scan_bwd(x, x, x, al, None, rec, x, K=16)
    with pytest.raises(ValueError, match="dy has dtype"):
        scan.rglru_scan_bwd(x, x, x, al, None, torch.empty(n, dtype=torch.uint8), x.float(), K=16)


def test_projection_and_decode_bindings_reject():
    from linear_recurrence_sequence_amd import scan
    Dp = 256
    x = torch.zeros(1, 8, Dp, dtype=bf)
    w = torch.zeros(16, Dp // 16, Dp // 16, dtype=bf)
    bb = torch.zeros(Dp)
    with pytest.raises(ValueError, match="w_x has dtype"):
        scan.rglru_gate_proj_fwd(x, w.float(), bb, w, bb)
    with pytest.raises(ValueError, match="w_a has shape"):
        scan.rglru_gate_proj_fwd(x, w, bb, w[:8].contiguous(), bb)
    dl = torch.zeros(1, 8, Dp)
    with pytest.raises(ValueError, match="dla has dtype"):
        scan.rglru_gate_proj_bwd(x, w, w, dl, dl.to(bf), dl)
    a = _samu()
    with pytest.raises(ValueError, match="b has shape"):
        scan.samu_scan_decode(a["x_sel"][:, 0].contiguous(), a["b"][:, :2].contiguous(), a["w_phi"], a["w_r"],
                              a["a_phi"], a["a_r"], a["nu"], a["theta"])
