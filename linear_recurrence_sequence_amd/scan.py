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
    L.samu_scan_fwd_noalloc.argtypes = [i] * 5 + [vp] * 9 + [vp, i, vp, vp, vp]
    L.samu_scan_fwd_noalloc.restype = i
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
    L.samu_scan_decode.argtypes = [i, i] + [vp] * 11 + [vp, i, vp]
    L.samu_scan_decode.restype = i
    L.samu_scan_decode_table_bytes.argtypes = [i]
    L.samu_scan_decode_table_bytes.restype = sz
    L.samu_scan_decode_prepare.argtypes = [i] + [vp] * 7 + [vp]
    L.samu_scan_decode_prepare.restype = i
    L.rglru_scan_fwd.argtypes = [i] * 5 + [vp] * 6 + [vp, i, vp, vp, vp, sz, vp]
    L.rglru_scan_fwd.restype = i
    L.rglru_scan_bwd.argtypes = [i] * 5 + [vp] * 5 + [vp, vp, vp, vp, vp, vp, i, vp, vp, vp, sz, vp]
    L.rglru_scan_bwd.restype = i
    L.scan_profile_enable.argtypes = [i]
    L.scan_profile_enable.restype = None
    L.scan_set_handoff_poll_limit.argtypes = [i]
    L.scan_set_handoff_poll_limit.restype = i
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


def _nbytes(t):
    return t.numel() * t.element_size()


def _want(t, name, dtypes, shape=None, optional=False):
    """Check a tensor the C ABI will read or write through a raw pointer:
    device, dtype and exact shape (the library cannot see allocation sizes,
    so this is the only place a mismatch can be caught)."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected " + " or ".join(str(d) for d in dtypes))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _want_bytes(t, name, need):
    """A caller-provided byte buffer (saved record, workspace) of at least `need` bytes."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if need == 0:
        raise ValueError(f"{name}: unsupported shape (the size query returned 0)")
    if _nbytes(t) < need:
        raise ValueError(f"{name} holds {_nbytes(t)} bytes, the call needs {need}")


_BF16, _F32 = torch.bfloat16, torch.float32
_OUT_DTYPES = (torch.bfloat16, torch.float32)


def _tag_saved(saved, kind, B, L, D, K):
    """Remember which forward wrote a saved record, so that a backward of
    another shape or chunk length is refused (the record's layout depends
    on B, L, D and K; its size alone does not always tell them apart)."""
    try:
        saved._lrs_record = (kind, B, L, D, K)
    except (AttributeError, RuntimeError):
        pass


def _check_saved(saved, kind, B, L, D, K, need):
    _want_bytes(saved, "saved", need)
    tag = getattr(saved, "_lrs_record", None)
    if tag is not None and tag != (kind, B, L, D, K):
        raise ValueError(f"saved was written by a forward with (scan, B, L, D, K) = {tag}, "
                         f"the backward call has {(kind, B, L, D, K)}")


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
def _samu_params(x_sel, w_phi, w_r, a_phi, a_r, nu, theta):
    if x_sel.dim() != 3:
        raise ValueError(f"x_sel must be [B, L, D], got shape {tuple(x_sel.shape)}")
    B, L, D = x_sel.shape
    M = D // 2
    _want(x_sel, "x_sel", _BF16)
    for t, n in ((w_phi, "w_phi"), (w_r, "w_r")):
        _want(t, n, _F32, (D + 1,))
    for t, n in ((a_phi, "a_phi"), (a_r, "a_r")):
        _want(t, n, _F32, (1,))
    for t, n in ((nu, "nu"), (theta, "theta")):
        _want(t, n, _F32, (M,))
    return B, L, D, M


def samu_scan_fwd(x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, z0=None, *, K=32, G=0,
                  y_dtype=torch.bfloat16, y=None, z_final=None, saved=None, workspace=None,
                  stream=None):
    """Returns (y [B,L,M,2], z_final [B,M,2] f32, saved uint8)."""
    B, L, D, M = _samu_params(x_sel, w_phi, w_r, a_phi, a_r, nu, theta)
    _want(b, "b", _BF16, (B, L, M, 2))
    _want(z0, "z0", _F32, (B, M, 2), optional=True)
    dev = x_sel.device
    if y is None:
        y = torch.empty((B, L, M, 2), dtype=y_dtype, device=dev)
    _want(y, "y", _OUT_DTYPES, (B, L, M, 2))
    if z_final is None:
        z_final = torch.empty((B, M, 2), dtype=torch.float32, device=dev)
    _want(z_final, "z_final", _F32, (B, M, 2))
    sv_n = samu_scan_saved_bytes(B, L, D, K)
    if saved is None:
        saved = _bytes(sv_n, dev)
    _want_bytes(saved, "saved", sv_n)
    ws_n = samu_scan_workspace_bytes(B, L, D, K, G, False)
    if workspace is None:
        workspace = _bytes(ws_n, dev)
    _want_bytes(workspace, "workspace", ws_n)
    st = lib().samu_scan_fwd(B, L, D, K, G, _p(x_sel), _p(b), _p(w_phi), _p(w_r), _p(a_phi),
                             _p(a_r), _p(nu), _p(theta), _p(z0), _p(y), _code(y.dtype),
                             _p(z_final), _p(saved), _p(workspace), _nbytes(workspace),
                             _stream(stream))
    _check(st, "samu_scan_fwd")
    _tag_saved(saved, "samu", B, L, D, K)
    return y, z_final, saved


def samu_scan_bwd(x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, saved, dy, dz_final=None, *,
                  K=32, G=0, grad_dtype=torch.bfloat16, want_dz0=True, out=None,
                  workspace=None, stream=None):
    """Returns dict(dx_sel, db, dz0, dw_phi, dw_r, da_phi, da_r, dnu, dtheta)."""
    B, L, D, M = _samu_params(x_sel, w_phi, w_r, a_phi, a_r, nu, theta)
    _want(b, "b", _BF16, (B, L, M, 2))
    _want(dy, "dy", _BF16, (B, L, M, 2))
    _want(dz_final, "dz_final", _F32, (B, M, 2), optional=True)
    _check_saved(saved, "samu", B, L, D, K, samu_scan_saved_bytes(B, L, D, K))
    dev = x_sel.device
    if out is None:
        f = dict(dtype=torch.float32, device=dev)
        out = dict(dx_sel=torch.empty((B, L, D), dtype=grad_dtype, device=dev),
                   db=torch.empty((B, L, M, 2), dtype=grad_dtype, device=dev),
                   dz0=torch.empty((B, M, 2), **f) if want_dz0 else None,
                   dw_phi=torch.empty(D + 1, **f), dw_r=torch.empty(D + 1, **f),
                   da_phi=torch.empty(1, **f), da_r=torch.empty(1, **f),
                   dnu=torch.empty(M, **f), dtheta=torch.empty(M, **f))
    gd = out["dx_sel"].dtype if isinstance(out.get("dx_sel"), torch.Tensor) else None
    _want(out.get("dx_sel"), "dx_sel", _OUT_DTYPES, (B, L, D))
    _want(out.get("db"), "db", gd, (B, L, M, 2))
    _want(out.get("dz0"), "dz0", _F32, (B, M, 2), optional=True)
    for n, shp in (("dw_phi", (D + 1,)), ("dw_r", (D + 1,)), ("da_phi", (1,)), ("da_r", (1,)),
                   ("dnu", (M,)), ("dtheta", (M,))):
        _want(out.get(n), n, _F32, shp)
    ws_n = samu_scan_workspace_bytes(B, L, D, K, G, True)
    if workspace is None:
        workspace = _bytes(ws_n, dev)
    _want_bytes(workspace, "workspace", ws_n)
    st = lib().samu_scan_bwd(B, L, D, K, G, _p(x_sel), _p(b), _p(w_phi), _p(w_r), _p(a_phi),
                             _p(a_r), _p(nu), _p(theta), _p(saved), _p(dy), _p(dz_final),
                             _p(out["dx_sel"]), _p(out["db"]), _code(out["dx_sel"].dtype),
                             _p(out["dz0"]), _p(out["dw_phi"]), _p(out["dw_r"]), _p(out["da_phi"]),
                             _p(out["da_r"]), _p(out["dnu"]), _p(out["dtheta"]), _p(workspace),
                             _nbytes(workspace), _stream(stream))
    _check(st, "samu_scan_bwd")
    return out


# ---------------------------------------------------------- SAMU decode ---
def samu_scan_decode_prepare(w_phi, w_r, a_phi, a_r, nu, theta, *, table=None, stream=None):
    """The decode step's constant table for these parameters (uint8 tensor)."""
    D = w_phi.shape[0] - 1
    M = D // 2
    _want(w_phi, "w_phi", _F32, (D + 1,))
    _want(w_r, "w_r", _F32, (D + 1,))
    _want(a_phi, "a_phi", _F32, (1,))
    _want(a_r, "a_r", _F32, (1,))
    _want(nu, "nu", _F32, (M,))
    _want(theta, "theta", _F32, (M,))
    n = lib().samu_scan_decode_table_bytes(D)
    if table is None:
        table = _bytes(n, w_phi.device)
    _want_bytes(table, "table", n)
    st = lib().samu_scan_decode_prepare(D, _p(w_phi), _p(w_r), _p(a_phi), _p(a_r), _p(nu), _p(theta), _p(table),
                                        _stream(stream))
    _check(st, "samu_scan_decode_prepare")
    return table


def samu_scan_decode(x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, z=None, *,
                     y_dtype=torch.bfloat16, y=None, z_out=None, table=None, stream=None):
    """One generation step.  x_sel [B, D] bf16, b [B, M, 2] bf16, z [B, M, 2]
    f32 or None (= 0); table from samu_scan_decode_prepare (or None: the
    step forms its constants itself).  Returns (y [B, M, 2], z_out [B, M, 2]
    f32); pass z_out=z to update the state in place."""
    if x_sel.dim() != 2:
        raise ValueError(f"x_sel must be [B, D], got shape {tuple(x_sel.shape)}")
    B, L, D, M = _samu_params(x_sel.unsqueeze(1), w_phi, w_r, a_phi, a_r, nu, theta)
    _want(b, "b", _BF16, (B, M, 2))
    _want(z, "z", _F32, (B, M, 2), optional=True)
    dev = x_sel.device
    if y is None:
        y = torch.empty((B, M, 2), dtype=y_dtype, device=dev)
    _want(y, "y", _OUT_DTYPES, (B, M, 2))
    if z_out is None:
        z_out = torch.empty((B, M, 2), dtype=torch.float32, device=dev)
    _want(z_out, "z_out", _F32, (B, M, 2))
    if table is not None:
        _want_bytes(table, "table", lib().samu_scan_decode_table_bytes(D))
    st = lib().samu_scan_decode(B, D, _p(x_sel), _p(b), _p(w_phi), _p(w_r), _p(a_phi), _p(a_r),
                                _p(nu), _p(theta), _p(table), _p(z), _p(z_out), _p(y), _code(y.dtype),
                                _stream(stream))
    _check(st, "samu_scan_decode")
    return y, z_out


# ------------------------------------------------ RG-LRU gate projections ---
def _proj_weights(x, w_x, w_a):
    if x.dim() != 3:
        raise ValueError(f"x must be [B, L, D], got shape {tuple(x.shape)}")
    B, L, D = x.shape
    _want(x, "x", _BF16)
    for t, n in ((w_x, "w_x"), (w_a, "w_a")):
        _want(t, n, _BF16, (16, D // 16, D // 16))
    return B, L, D


def rglru_gate_proj_fwd(x, w_x, b_x, w_a, b_a, *, lx=None, la=None, stream=None):
    """Gate logits of the two 16-block block-diagonal projections (BF16).
    Returns (lx, la) [B, L, D]."""
    B, L, D = _proj_weights(x, w_x, w_a)
    for t, n in ((b_x, "b_x"), (b_a, "b_a")):
        _want(t, n, _F32, (D,))
    if lx is None:
        lx = torch.empty_like(x)
    if la is None:
        la = torch.empty_like(x)
    _want(lx, "lx", _BF16, (B, L, D))
    _want(la, "la", _BF16, (B, L, D))
    st = lib().rglru_gate_proj_fwd(B, L, D, _p(x), _p(w_x), _p(b_x), _p(w_a), _p(b_a), _p(lx), _p(la),
                                   _stream(stream))
    _check(st, "rglru_gate_proj_fwd")
    return lx, la


def rglru_gate_proj_bwd(x, w_x, w_a, dlx, dla, dx, *, dx_out=None, workspace=None, stream=None):
    """Adjoint of the projections: returns dict(dx = dx + W^T dl, dw_x, db_x,
    dw_a, db_a); pass dx_out=dx to accumulate in place.  dlx, dla, dx and
    dx_out share one dtype (BF16 or FP32)."""
    B, L, D = _proj_weights(x, w_x, w_a)
    _want(dlx, "dlx", _OUT_DTYPES, (B, L, D))
    for t, n in ((dla, "dla"), (dx, "dx")):
        _want(t, n, dlx.dtype, (B, L, D))
    dev = x.device
    if dx_out is None:
        dx_out = torch.empty_like(dx)
    _want(dx_out, "dx_out", dlx.dtype, (B, L, D))
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dx=dx_out, dw_x=torch.empty((16, D // 16, D // 16), **f32), db_x=torch.empty(D, **f32),
               dw_a=torch.empty((16, D // 16, D // 16), **f32), db_a=torch.empty(D, **f32))
    ws_n = lib().rglru_gate_proj_bwd_workspace_bytes(B, L, D)
    if workspace is None:
        workspace = _bytes(ws_n, dev)
    _want_bytes(workspace, "workspace", ws_n)
    st = lib().rglru_gate_proj_bwd(B, L, D, _p(x), _p(w_x), _p(w_a), _p(dlx), _p(dla), _code(dlx.dtype), _p(dx),
                                   _p(dx_out), _p(out["dw_x"]), _p(out["db_x"]), _p(out["dw_a"]),
                                   _p(out["db_a"]), _p(workspace), _nbytes(workspace), _stream(stream))
    _check(st, "rglru_gate_proj_bwd")
    return out


# ------------------------------------------------------ comparison scans ---
BASELINES = {"sequential": 0, "associative": 1}


def samu_scan_baseline_fwd(variant, x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, z0=None, *,
                           y_dtype=torch.bfloat16, y=None, z_final=None, workspace=None, stream=None):
    """Comparison scan (variant "sequential" or "associative"), forward only.
    Returns (y [B,L,M,2], z_final [B,M,2] f32)."""
    v = BASELINES[variant]
    B, L, D, M = _samu_params(x_sel, w_phi, w_r, a_phi, a_r, nu, theta)
    _want(b, "b", _BF16, (B, L, M, 2))
    _want(z0, "z0", _F32, (B, M, 2), optional=True)
    dev = x_sel.device
    if y is None:
        y = torch.empty((B, L, M, 2), dtype=y_dtype, device=dev)
    _want(y, "y", _OUT_DTYPES, (B, L, M, 2))
    if z_final is None:
        z_final = torch.empty((B, M, 2), dtype=torch.float32, device=dev)
    _want(z_final, "z_final", _F32, (B, M, 2))
    n = lib().samu_scan_baseline_workspace_bytes(v, B, L, D)
    if workspace is None:
        workspace = _bytes(n, dev)
    _want_bytes(workspace, "workspace", n)
    st = lib().samu_scan_baseline_fwd(v, B, L, D, _p(x_sel), _p(b), _p(w_phi), _p(w_r), _p(a_phi),
                                      _p(a_r), _p(nu), _p(theta), _p(z0), _p(y), _code(y.dtype),
                                      _p(z_final), _p(workspace), _nbytes(workspace), _stream(stream))
    _check(st, "samu_scan_baseline_fwd")
    return y, z_final


def _rglru_inputs(x, lx, la, alpha, reset):
    if x.dim() != 3:
        raise ValueError(f"x must be [B, L, D], got shape {tuple(x.shape)}")
    B, L, D = x.shape
    _want(x, "x", _BF16)
    _want(lx, "lx", _BF16, (B, L, D))
    _want(la, "la", _BF16, (B, L, D))
    _want(alpha, "alpha", _F32, (D,))
    _want(reset, "reset", (torch.uint8, torch.bool), (B, L), optional=True)
    return B, L, D


def rglru_scan_baseline_fwd(variant, x, lx, la, alpha, reset=None, h0=None, *, y_dtype=torch.bfloat16,
                            y=None, h_final=None, workspace=None, stream=None):
    """Comparison scan (variant "sequential" or "associative"), forward only.
    Returns (y [B,L,D], h_final [B,D] f32)."""
    v = BASELINES[variant]
    B, L, D = _rglru_inputs(x, lx, la, alpha, reset)
    _want(h0, "h0", _F32, (B, D), optional=True)
    dev = x.device
    if y is None:
        y = torch.empty((B, L, D), dtype=y_dtype, device=dev)
    _want(y, "y", _OUT_DTYPES, (B, L, D))
    if h_final is None:
        h_final = torch.empty((B, D), dtype=torch.float32, device=dev)
    _want(h_final, "h_final", _F32, (B, D))
    n = lib().rglru_scan_baseline_workspace_bytes(v, B, L, D)
    if workspace is None and n > 0:
        workspace = _bytes(n, dev)
    if n > 0:
        _want_bytes(workspace, "workspace", n)
    st = lib().rglru_scan_baseline_fwd(v, B, L, D, _p(x), _p(lx), _p(la), _p(alpha), _p(reset), _p(h0),
                                       _p(y), _code(y.dtype), _p(h_final), _p(workspace),
                                       0 if workspace is None else _nbytes(workspace), _stream(stream))
    _check(st, "rglru_scan_baseline_fwd")
    return y, h_final


# ----------------------------------------------------------------- RG-LRU ---
def rglru_scan_fwd(x, lx, la, alpha, reset=None, h0=None, *, K=16, G=0, y_dtype=torch.bfloat16,
                   y=None, h_final=None, saved=None, workspace=None, stream=None):
    """Returns (y [B,L,D], h_final [B,D] f32, saved uint8)."""
    B, L, D = _rglru_inputs(x, lx, la, alpha, reset)
    _want(h0, "h0", _F32, (B, D), optional=True)
    dev = x.device
    if y is None:
        y = torch.empty((B, L, D), dtype=y_dtype, device=dev)
    _want(y, "y", _OUT_DTYPES, (B, L, D))
    if h_final is None:
        h_final = torch.empty((B, D), dtype=torch.float32, device=dev)
    _want(h_final, "h_final", _F32, (B, D))
    sv_n = rglru_scan_saved_bytes(B, L, D, K)
    if saved is None:
        saved = _bytes(sv_n, dev)
    _want_bytes(saved, "saved", sv_n)
    ws_n = rglru_scan_workspace_bytes(B, L, D, K, G, False)
    if workspace is None:
        workspace = _bytes(ws_n, dev)
    _want_bytes(workspace, "workspace", ws_n)
    st = lib().rglru_scan_fwd(B, L, D, K, G, _p(x), _p(lx), _p(la), _p(alpha), _p(reset), _p(h0),
                              _p(y), _code(y.dtype), _p(h_final), _p(saved), _p(workspace),
                              _nbytes(workspace), _stream(stream))
    _check(st, "rglru_scan_fwd")
    _tag_saved(saved, "rglru", B, L, D, K)
    return y, h_final, saved


def rglru_scan_bwd(x, lx, la, alpha, reset, saved, dy, dh_final=None, *, K=16, G=0,
                   grad_dtype=torch.bfloat16, want_dh0=True, out=None, workspace=None,
                   stream=None):
    """Returns dict(dx, dlx, dla, dalpha, dh0)."""
    B, L, D = _rglru_inputs(x, lx, la, alpha, reset)
    _want(dy, "dy", _BF16, (B, L, D))
    _want(dh_final, "dh_final", _F32, (B, D), optional=True)
    _check_saved(saved, "rglru", B, L, D, K, rglru_scan_saved_bytes(B, L, D, K))
    dev = x.device
    if out is None:
        out = dict(dx=torch.empty((B, L, D), dtype=grad_dtype, device=dev),
                   dlx=torch.empty((B, L, D), dtype=grad_dtype, device=dev),
                   dla=torch.empty((B, L, D), dtype=grad_dtype, device=dev),
                   dalpha=torch.empty(D, dtype=torch.float32, device=dev),
                   dh0=torch.empty((B, D), dtype=torch.float32, device=dev) if want_dh0 else None)
    _want(out.get("dx"), "dx", _OUT_DTYPES, (B, L, D))
    for n in ("dlx", "dla"):
        _want(out.get(n), n, out["dx"].dtype, (B, L, D))
    _want(out.get("dalpha"), "dalpha", _F32, (D,))
    _want(out.get("dh0"), "dh0", _F32, (B, D), optional=True)
    ws_n = rglru_scan_workspace_bytes(B, L, D, K, G, True)
    if workspace is None:
        workspace = _bytes(ws_n, dev)
    _want_bytes(workspace, "workspace", ws_n)
    st = lib().rglru_scan_bwd(B, L, D, K, G, _p(x), _p(lx), _p(la), _p(alpha), _p(reset),
                              _p(saved), _p(dy), _p(dh_final), _p(out["dx"]), _p(out["dlx"]),
                              _p(out["dla"]), _code(out["dx"].dtype), _p(out["dalpha"]),
                              _p(out["dh0"]), _p(workspace), _nbytes(workspace), _stream(stream))
    _check(st, "rglru_scan_bwd")
    return out


# --------------------------------------------------------------- profiler ---
def scan_set_handoff_poll_limit(polls):
    """Polls a single-pass scan's hand-off wait makes before it gives up
    (its words then read as NaN); negative restores the default.  Returns
    the previous limit."""
    return int(lib().scan_set_handoff_poll_limit(int(polls)))


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
