"""Thin Python binding of the C ABI in include/samu_scan.h.

Argument marshalling only: every step of the scans runs in the HIP kernels of
libsamu_scan.so.  PyTorch provides device memory and the current stream.  The
functions keep the C names; they allocate outputs, the saved record and the
workspace with torch when the caller does not pass them.  If the library is
missing (not built) every call raises -- there is no CPU fallback.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsamu_scan.so")

SCAN_BF16, SCAN_F32 = 0, 1
_STATUS = {0: "SCAN_OK", -1: "SCAN_ERR_NULL", -2: "SCAN_ERR_SHAPE", -3: "SCAN_ERR_ALIGN",
           -4: "SCAN_ERR_WORKSPACE", -5: "SCAN_ERR_DEVICE", -6: "SCAN_ERR_ALIAS"}


class ScanError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib():
    """The loaded libsamu_scan.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m linear_recurrence_sequence_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i, sz, vp, fp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p
    L.scan_last_error.restype = ctypes.c_char_p
    for n in ("samu_scan_saved_bytes", "rglru_scan_saved_bytes"):
        getattr(L, n).argtypes = [i, i, i, i]
        getattr(L, n).restype = sz
    for n in ("samu_scan_workspace_bytes", "rglru_scan_workspace_bytes"):
        getattr(L, n).argtypes = [i, i, i, i, i, i]
        getattr(L, n).restype = sz
    L.scan_prefix_scratch_bytes.argtypes = [i, i, i, i, i, i]
    L.scan_prefix_scratch_bytes.restype = sz
    L.samu_scan_fwd.argtypes = [i] * 5 + [vp] * 9 + [vp, i, vp, vp, vp, sz, vp]
    L.samu_scan_fwd.restype = i
    L.samu_scan_bwd.argtypes = [i] * 5 + [vp] * 8 + [vp, vp, vp, vp, vp, i, vp] + [vp] * 6 + [vp, sz, vp]
    L.samu_scan_bwd.restype = i
    for n in ("samu_scan_baseline_workspace_bytes", "rglru_scan_baseline_workspace_bytes"):
        getattr(L, n).argtypes = [i, i, i, i]
        getattr(L, n).restype = sz
    L.samu_scan_baseline_fwd.argtypes = [i] * 4 + [vp] * 9 + [vp, i, vp, vp, sz, vp]
    L.samu_scan_baseline_fwd.restype = i
    L.rglru_scan_baseline_fwd.argtypes = [i] * 4 + [vp] * 6 + [vp, i, vp, vp, sz, vp]
    L.rglru_scan_baseline_fwd.restype = i
    L.rglru_gate_proj_fwd.argtypes = [i, i, i] + [vp] * 8
    L.rglru_gate_proj_fwd.restype = i
    L.rglru_gate_proj_bwd_workspace_bytes.argtypes = [i, i, i]
    L.rglru_gate_proj_bwd_workspace_bytes.restype = sz
    L.rglru_gate_proj_bwd.argtypes = [i, i, i] + [vp] * 5 + [i] + [vp] * 7 + [sz, vp]
    L.rglru_gate_proj_bwd.restype = i
    L.samu_scan_decode.argtypes = [i, i] + [vp] * 10 + [vp, i, vp]
    L.samu_scan_decode.restype = i
    L.rglru_scan_fwd.argtypes = [i] * 5 + [vp] * 6 + [vp, i, vp, vp, vp, sz, vp]
    L.rglru_scan_fwd.restype = i
    L.rglru_scan_bwd.argtypes = [i] * 5 + [vp] * 5 + [vp, vp, vp, vp, vp, vp, i, vp, vp, vp, sz, vp]
    L.rglru_scan_bwd.restype = i
    L.scan_profile_enable.argtypes = [i]
    L.scan_profile_enable.restype = None
    L.scan_profile_kernel_count.restype = i
    L.scan_profile_kernel_name.argtypes = [i]
    L.scan_profile_kernel_name.restype = ctypes.c_char_p
    L.scan_profile_collect.argtypes = [vp, vp]
    L.scan_profile_collect.restype = i
    _lib = L
    return L


def _p(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(st, what):
    if st != 0:
        raise ScanError(st, f"{what}: {lib().scan_last_error().decode()}")


def _code(dtype):
    if dtype == torch.bfloat16:
        return SCAN_BF16
    if dtype == torch.float32:
        return SCAN_F32
    raise ValueError("output dtype must be torch.bfloat16 or torch.float32")


def _bytes(n, device):
    return torch.empty(max(int(n), 16), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ sizes ---
def samu_scan_saved_bytes(B, L, D, K=32):
    return lib().samu_scan_saved_bytes(B, L, D, K)


def samu_scan_workspace_bytes(B, L, D, K=32, G=0, backward=False):
    return lib().samu_scan_workspace_bytes(B, L, D, K, G, int(bool(backward)))


def rglru_scan_saved_bytes(B, L, D, K=16):
    return lib().rglru_scan_saved_bytes(B, L, D, K)


def rglru_scan_workspace_bytes(B, L, D, K=16, G=0, backward=False):
    return lib().rglru_scan_workspace_bytes(B, L, D, K, G, int(bool(backward)))


def scan_prefix_scratch_bytes(B, L, D, K, G=0, rglru=False):
    return lib().scan_prefix_scratch_bytes(B, L, D, K, G, int(bool(rglru)))


# ------------------------------------------------------------------- SAMU ---
def samu_scan_fwd(x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, z0=None, *, K=32, G=0,
                  y_dtype=torch.bfloat16, y=None, z_final=None, saved=None, workspace=None,
                  stream=None):
    """Returns (y [B,L,M,2], z_final [B,M,2] f32, saved uint8)."""
    B, L, D = x_sel.shape
    M = D // 2
    dev = x_sel.device
    if y is None:
        y = torch.empty((B, L, M, 2), dtype=y_dtype, device=dev)
    if z_final is None:
        z_final = torch.empty((B, M, 2), dtype=torch.float32, device=dev)
    if saved is None:
        saved = _bytes(samu_scan_saved_bytes(B, L, D, K), dev)
    ws_n = samu_scan_workspace_bytes(B, L, D, K, G, False)
    if workspace is None:
        workspace = _bytes(ws_n, dev)
    st = lib().samu_scan_fwd(B, L, D, K, G, _p(x_sel), _p(b), _p(w_phi), _p(w_r), _p(a_phi),
                             _p(a_r), _p(nu), _p(theta), _p(z0), _p(y), _code(y.dtype),
                             _p(z_final), _p(saved), _p(workspace), workspace.numel(),
                             _stream(stream))
    _check(st, "samu_scan_fwd")
    return y, z_final, saved


def samu_scan_bwd(x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, saved, dy, dz_final=None, *,
                  K=32, G=0, grad_dtype=torch.bfloat16, want_dz0=True, out=None,
                  workspace=None, stream=None):
    """Returns dict(dx_sel, db, dz0, dw_phi, dw_r, da_phi, da_r, dnu, dtheta)."""
    B, L, D = x_sel.shape
    M = D // 2
    dev = x_sel.device
    if out is None:
        f = dict(dtype=torch.float32, device=dev)
        out = dict(dx_sel=torch.empty((B, L, D), dtype=grad_dtype, device=dev),
                   db=torch.empty((B, L, M, 2), dtype=grad_dtype, device=dev),
                   dz0=torch.empty((B, M, 2), **f) if want_dz0 else None,
                   dw_phi=torch.empty(D + 1, **f), dw_r=torch.empty(D + 1, **f),
                   da_phi=torch.empty(1, **f), da_r=torch.empty(1, **f),
                   dnu=torch.empty(M, **f), dtheta=torch.empty(M, **f))
    ws_n = samu_scan_workspace_bytes(B, L, D, K, G, True)
    if workspace is None:
        workspace = _bytes(ws_n, dev)
    st = lib().samu_scan_bwd(B, L, D, K, G, _p(x_sel), _p(b), _p(w_phi), _p(w_r), _p(a_phi),
                             _p(a_r), _p(nu), _p(theta), _p(saved), _p(dy), _p(dz_final),
                             _p(out["dx_sel"]), _p(out["db"]), _code(out["dx_sel"].dtype),
                             _p(out["dz0"]), _p(out["dw_phi"]), _p(out["dw_r"]), _p(out["da_phi"]),
                             _p(out["da_r"]), _p(out["dnu"]), _p(out["dtheta"]), _p(workspace),
                             workspace.numel(), _stream(stream))
    _check(st, "samu_scan_bwd")
    return out


# ----------------------------------------------------------------- RG-LRU ---
def samu_scan_decode(x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, z=None, *,
                     y_dtype=torch.bfloat16, y=None, z_out=None, stream=None):
    """One generation step.  x_sel [B, D] bf16, b [B, M, 2] bf16, z [B, M, 2]
    f32 or None (= 0).  Returns (y [B, M, 2], z_out [B, M, 2] f32); pass
    z_out=z to update the state in place."""
    B, D = x_sel.shape
    M = D // 2
    dev = x_sel.device
    if y is None:
        y = torch.empty((B, M, 2), dtype=y_dtype, device=dev)
    if z_out is None:
        z_out = torch.empty((B, M, 2), dtype=torch.float32, device=dev)
    st = lib().samu_scan_decode(B, D, _p(x_sel), _p(b), _p(w_phi), _p(w_r), _p(a_phi), _p(a_r),
                                _p(nu), _p(theta), _p(z), _p(z_out), _p(y), _code(y.dtype),
                                _stream(stream))
    _check(st, "samu_scan_decode")
    return y, z_out


def rglru_gate_proj_fwd(x, w_x, b_x, w_a, b_a, *, lx=None, la=None, stream=None):
    """Gate logits of the two 16-block block-diagonal projections (BF16).
    Returns (lx, la) [B, L, D]."""
    B, L, D = x.shape
    if lx is None:
        lx = torch.empty_like(x)
    if la is None:
        la = torch.empty_like(x)
    st = lib().rglru_gate_proj_fwd(B, L, D, _p(x), _p(w_x), _p(b_x), _p(w_a), _p(b_a), _p(lx), _p(la),
                                   _stream(stream))
    _check(st, "rglru_gate_proj_fwd")
    return lx, la


def rglru_gate_proj_bwd(x, w_x, w_a, dlx, dla, dx, *, dx_out=None, workspace=None, stream=None):
    """Adjoint of the projections: returns dict(dx = dx + W^T dl, dw_x, db_x,
    dw_a, db_a); pass dx_out=dx to accumulate in place."""
    B, L, D = x.shape
    dev = x.device
    if dx_out is None:
        dx_out = torch.empty_like(dx)
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dx=dx_out, dw_x=torch.empty((16, D // 16, D // 16), **f32), db_x=torch.empty(D, **f32),
               dw_a=torch.empty((16, D // 16, D // 16), **f32), db_a=torch.empty(D, **f32))
    if workspace is None:
        workspace = _bytes(lib().rglru_gate_proj_bwd_workspace_bytes(B, L, D), dev)
    st = lib().rglru_gate_proj_bwd(B, L, D, _p(x), _p(w_x), _p(w_a), _p(dlx), _p(dla), _code(dlx.dtype), _p(dx),
                                   _p(dx_out), _p(out["dw_x"]), _p(out["db_x"]), _p(out["dw_a"]),
                                   _p(out["db_a"]), _p(workspace), workspace.numel(), _stream(stream))
    _check(st, "rglru_gate_proj_bwd")
    return out


BASELINES = {"sequential": 0, "associative": 1}


def samu_scan_baseline_fwd(variant, x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, z0=None, *,
                           y_dtype=torch.bfloat16, y=None, z_final=None, workspace=None, stream=None):
    """Comparison scan (variant "sequential" or "associative"), forward only.
    Returns (y [B,L,M,2], z_final [B,M,2] f32)."""
    v = BASELINES[variant]
    B, L, D = x_sel.shape
    M = D // 2
    dev = x_sel.device
    if y is None:
        y = torch.empty((B, L, M, 2), dtype=y_dtype, device=dev)
    if z_final is None:
        z_final = torch.empty((B, M, 2), dtype=torch.float32, device=dev)
    n = lib().samu_scan_baseline_workspace_bytes(v, B, L, D)
    if workspace is None:
        workspace = _bytes(n, dev)
    st = lib().samu_scan_baseline_fwd(v, B, L, D, _p(x_sel), _p(b), _p(w_phi), _p(w_r), _p(a_phi),
                                      _p(a_r), _p(nu), _p(theta), _p(z0), _p(y), _code(y.dtype),
                                      _p(z_final), _p(workspace), workspace.numel(), _stream(stream))
    _check(st, "samu_scan_baseline_fwd")
    return y, z_final


def rglru_scan_baseline_fwd(variant, x, lx, la, alpha, reset=None, h0=None, *, y_dtype=torch.bfloat16,
                            y=None, h_final=None, workspace=None, stream=None):
    """Comparison scan (variant "sequential" or "associative"), forward only.
    Returns (y [B,L,D], h_final [B,D] f32)."""
    v = BASELINES[variant]
    B, L, D = x.shape
    dev = x.device
    if y is None:
        y = torch.empty((B, L, D), dtype=y_dtype, device=dev)
    if h_final is None:
        h_final = torch.empty((B, D), dtype=torch.float32, device=dev)
    n = lib().rglru_scan_baseline_workspace_bytes(v, B, L, D)
    if workspace is None and n > 0:
        workspace = _bytes(n, dev)
    st = lib().rglru_scan_baseline_fwd(v, B, L, D, _p(x), _p(lx), _p(la), _p(alpha), _p(reset), _p(h0),
                                       _p(y), _code(y.dtype), _p(h_final), _p(workspace),
                                       0 if workspace is None else workspace.numel(), _stream(stream))
    _check(st, "rglru_scan_baseline_fwd")
    return y, h_final


def rglru_scan_fwd(x, lx, la, alpha, reset=None, h0=None, *, K=16, G=0, y_dtype=torch.bfloat16,
                   y=None, h_final=None, saved=None, workspace=None, stream=None):
    """Returns (y [B,L,D], h_final [B,D] f32, saved uint8)."""
    B, L, D = x.shape
    dev = x.device
    if y is None:
        y = torch.empty((B, L, D), dtype=y_dtype, device=dev)
    if h_final is None:
        h_final = torch.empty((B, D), dtype=torch.float32, device=dev)
    if saved is None:
        saved = _bytes(rglru_scan_saved_bytes(B, L, D, K), dev)
    if workspace is None:
        workspace = _bytes(rglru_scan_workspace_bytes(B, L, D, K, G, False), dev)
    st = lib().rglru_scan_fwd(B, L, D, K, G, _p(x), _p(lx), _p(la), _p(alpha), _p(reset), _p(h0),
                              _p(y), _code(y.dtype), _p(h_final), _p(saved), _p(workspace),
                              workspace.numel(), _stream(stream))
    _check(st, "rglru_scan_fwd")
    return y, h_final, saved


def rglru_scan_bwd(x, lx, la, alpha, reset, saved, dy, dh_final=None, *, K=16, G=0,
                   grad_dtype=torch.bfloat16, want_dh0=True, out=None, workspace=None,
                   stream=None):
    """Returns dict(dx, dlx, dla, dalpha, dh0)."""
    B, L, D = x.shape
    dev = x.device
    if out is None:
        out = dict(dx=torch.empty((B, L, D), dtype=grad_dtype, device=dev),
                   dlx=torch.empty((B, L, D), dtype=grad_dtype, device=dev),
                   dla=torch.empty((B, L, D), dtype=grad_dtype, device=dev),
                   dalpha=torch.empty(D, dtype=torch.float32, device=dev),
                   dh0=torch.empty((B, D), dtype=torch.float32, device=dev) if want_dh0 else None)
    if workspace is None:
        workspace = _bytes(rglru_scan_workspace_bytes(B, L, D, K, G, True), dev)
    st = lib().rglru_scan_bwd(B, L, D, K, G, _p(x), _p(lx), _p(la), _p(alpha), _p(reset),
                              _p(saved), _p(dy), _p(dh_final), _p(out["dx"]), _p(out["dlx"]),
                              _p(out["dla"]), _code(out["dx"].dtype), _p(out["dalpha"]),
                              _p(out["dh0"]), _p(workspace), workspace.numel(), _stream(stream))
    _check(st, "rglru_scan_bwd")
    return out


# --------------------------------------------------------------- profiler ---
def scan_profile_enable(on=True):
    lib().scan_profile_enable(int(bool(on)))


def scan_profile_collect():
    """{kernel name: (total ms, launches)} for the launches recorded since the
    last collect (synchronizes on the recorded events)."""
    L = lib()
    n = L.scan_profile_kernel_count()
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int * n)()
    _check(L.scan_profile_collect(ctypes.cast(ms, ctypes.c_void_p), ctypes.cast(cnt, ctypes.c_void_p)),
           "scan_profile_collect")
    return {L.scan_profile_kernel_name(k).decode(): (ms[k], cnt[k]) for k in range(n) if cnt[k]}
