"""FP64 CPU oracle for the SAMU complex scan and the RG-LRU real scan.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP library
never loads it and shares no code with it.

Every function follows the pages' equations one token at a time in FP64 (see
``oracle.c`` for the citations and the readings adopted).  Tensor arguments
may be given as

* ``numpy.uint16`` arrays -- BF16 bit patterns, the form the GPU receives;
* ``numpy.float32`` arrays -- FP32 values as the GPU receives them;
* ``numpy.float64`` arrays -- used directly (finite-difference checks).

BF16 and FP32 values are widened to FP64 exactly before the C code runs.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB points the pins at a deliberately broken build (mutation checks).
_LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")


class _Nullable:
    """ctypes argtype accepting a C-contiguous array of one dtype, or None."""

    def __init__(self, dtype):
        self.dtype = np.dtype(dtype)

    def from_param(self, obj):
        if obj is None:
            return None
        if not isinstance(obj, np.ndarray) or obj.dtype != self.dtype or not obj.flags.c_contiguous:
            raise TypeError(f"expected C-contiguous {self.dtype} array or None")
        return obj.ctypes.data_as(ctypes.c_void_p)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    i, d = ctypes.c_int, ctypes.c_double
    n64, n8 = _Nullable(np.float64), _Nullable(np.uint8)
    P = _f64p
    lib.oracle_rglru_gate_proj.argtypes = [i, i, i, P, P, P, P]
    lib.oracle_rglru_gate_proj_bwd.argtypes = [i, i, i, P, P, P, P, P, P]
    lib.oracle_max_threads.restype = i
    lib.oracle_set_threads.argtypes = [i]
    lib.oracle_samu_controller.argtypes = [i, i, i, P, P, P, d, d] + [P] * 7
    lib.oracle_samu_fwd.argtypes = [i, i, i, P, P, P, P, d, d, P, P, n64, P, n64, n64, n64]
    lib.oracle_samu_bwd.argtypes = [i, i, i, P, P, P, P, d, d, P, P, n64, P, n64,
                                    P, P, n64, P, P, P, P, P, P]
    lib.oracle_rglru_fwd.argtypes = [i, i, i, P, P, P, P, n8, n64, P, n64]
    lib.oracle_rglru_bwd.argtypes = [i, i, i, P, P, P, P, n8, n64, P, n64, P, P, P, P, n64]
    _lib = lib
    return lib


def widen(a):
    """Exact FP64 copy of a BF16-bits (uint16), FP32 or FP64 array (None passes)."""
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.uint16:
        a = (a.astype(np.uint32) << 16).view(np.float32)
    return np.ascontiguousarray(a, dtype=np.float64)


def _scalar(v):
    return float(np.asarray(v, dtype=np.float64).reshape(-1)[0])


def max_threads() -> int:
    return _load().oracle_max_threads()


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def samu_controller(x_sel, w_phi, w_r, a_phi, a_r):
    """Per-token controller values p, r, d, c, E, C, S (each [B, L], FP64)."""
    lib = _load()
    x = widen(x_sel)
    B, L, D = x.shape
    outs = [np.empty((B, L), np.float64) for _ in range(7)]
    lib.oracle_samu_controller(B, L, D, x, widen(w_phi), widen(w_r), _scalar(a_phi),
                               _scalar(a_r), *outs)
    return dict(zip("p r d c E C S".split(), outs))


def samu_fwd(x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, z0=None):
    """Returns dict(y=[B,L,M,2], z_final=[B,M,2], p=[B,L], r=[B,L]) in FP64."""
    lib = _load()
    x = widen(x_sel)
    B, L, D = x.shape
    M = D // 2
    bb = widen(b)
    assert bb.shape == (B, L, M, 2)
    y = np.empty((B, L, M, 2), np.float64)
    zf = np.empty((B, M, 2), np.float64)
    p = np.empty((B, L), np.float64)
    r = np.empty((B, L), np.float64)
    lib.oracle_samu_fwd(B, L, D, x, bb, widen(w_phi), widen(w_r), _scalar(a_phi), _scalar(a_r),
                        widen(nu), widen(theta), widen(z0), y, zf, p, r)
    return dict(y=y, z_final=zf, p=p, r=r)


def samu_bwd(x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, z0, dy, dz_final=None):
    """Exact adjoint.  Returns dx_sel, db, dz0 (None if z0 is None), dw_phi,
    dw_r, da_phi, da_r, dnu, dtheta in FP64."""
    lib = _load()
    x = widen(x_sel)
    B, L, D = x.shape
    M = D // 2
    dx = np.empty((B, L, D), np.float64)
    db = np.empty((B, L, M, 2), np.float64)
    dz0 = np.empty((B, M, 2), np.float64) if z0 is not None else None
    dwp = np.empty(D + 1, np.float64)
    dwr = np.empty(D + 1, np.float64)
    dap = np.empty(1, np.float64)
    dar = np.empty(1, np.float64)
    dnu = np.empty(M, np.float64)
    dth = np.empty(M, np.float64)
    lib.oracle_samu_bwd(B, L, D, x, widen(b), widen(w_phi), widen(w_r), _scalar(a_phi),
                        _scalar(a_r), widen(nu), widen(theta), widen(z0), widen(dy),
                        widen(dz_final), dx, db, dz0, dwp, dwr, dap, dar, dnu, dth)
    return dict(dx_sel=dx, db=db, dz0=dz0, dw_phi=dwp, dw_r=dwr, da_phi=float(dap[0]),
                da_r=float(dar[0]), dnu=dnu, dtheta=dth)


def _reset_u8(reset):
    if reset is None:
        return None
    return np.ascontiguousarray(np.asarray(reset) != 0, dtype=np.uint8)


def rglru_fwd(x, lx, la, alpha, reset=None, h0=None):
    """Returns dict(y=[B,L,D], h_final=[B,D]) in FP64."""
    lib = _load()
    xx = widen(x)
    B, L, D = xx.shape
    y = np.empty((B, L, D), np.float64)
    hf = np.empty((B, D), np.float64)
    lib.oracle_rglru_fwd(B, L, D, xx, widen(lx), widen(la), widen(alpha), _reset_u8(reset),
                         widen(h0), y, hf)
    return dict(y=y, h_final=hf)


def rglru_bwd(x, lx, la, alpha, reset, h0, dy, dh_final=None):
    """Exact adjoint (with the capped square-root derivative).  Returns dx,
    dlx, dla, dalpha, dh0 (None if h0 is None) in FP64."""
    lib = _load()
    xx = widen(x)
    B, L, D = xx.shape
    dx = np.empty((B, L, D), np.float64)
    dlx = np.empty((B, L, D), np.float64)
    dla = np.empty((B, L, D), np.float64)
    dal = np.empty(D, np.float64)
    dh0 = np.empty((B, D), np.float64) if h0 is not None else None
    lib.oracle_rglru_bwd(B, L, D, xx, widen(lx), widen(la), widen(alpha), _reset_u8(reset),
                         widen(h0), widen(dy), widen(dh_final), dx, dlx, dla, dal, dh0)
    return dict(dx=dx, dlx=dlx, dla=dla, dalpha=dal, dh0=dh0)


def rglru_gate_proj(x, w, bias):
    """Block-diagonal gate projection (16 blocks): x [B, L, D], w [16, D/16,
    D/16] as (block, output, input), bias [D] -> FP64 logits [B, L, D]."""
    x, w, bias = widen(x), widen(w), widen(bias)
    B, L, D = x.shape
    if D % 16 or w.shape != (16, D // 16, D // 16) or bias.shape != (D,):
        raise ValueError("expected D % 16 == 0, w [16, D/16, D/16] and bias [D]")
    out = np.empty((B, L, D), np.float64)
    _load().oracle_rglru_gate_proj(B, L, D, x, w, bias, out)
    return out


def rglru_gate_proj_bwd(x, w, dl, dx=None):
    """Adjoint of rglru_gate_proj for the logit cotangent dl [B, L, D]:
    returns (dx + W^T dl per block, dW [16, D/16, D/16], dbias [D]); dx
    (FP64, optional) is the gradient already collected for x."""
    x, w, dl = widen(x), widen(w), widen(dl)
    B, L, D = x.shape
    dxo = np.zeros((B, L, D), np.float64) if dx is None else np.array(widen(dx), np.float64, copy=True)
    dw = np.empty((16, D // 16, D // 16), np.float64)
    db = np.empty((D,), np.float64)
    _load().oracle_rglru_gate_proj_bwd(B, L, D, x, w, dl, dxo, dw, db)
    return dxo, dw, db
