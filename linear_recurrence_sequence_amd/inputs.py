"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module draws random numbers and rounds them to the storage formats; it
holds none of the scan's arithmetic.  BF16 tensors are returned as
``numpy.uint16`` bit patterns (round-to-nearest-even of an FP32 draw), FP32
tensors as ``numpy.float32``.  Both the HIP path and the oracle read exactly
these arrays.

Value distributions follow the workloads the pages measure: selector and
drive ~ N(0, 1); theta ~ U[0, 2 pi); exp(-nu) ~ U[0.9, 0.999]; direction
vectors ~ N(0, 1); amplitudes a_phi = a_r = 0.5; initial state ~ N(0, 0.1^2);
dense output cotangent ~ N(0, 1).  RG-LRU: x, gate logits ~ N(0, 1);
softplus(alpha) ~ U[0.1, 1]; segment starts Bernoulli(p) at every position.
"""
import math

import numpy as np


def bf16_bits(a) -> np.ndarray:
    """Round FP32 values to BF16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """Exact FP32 value of BF16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _normal_bf16(rng, shape, chunk=1 << 24):
    """N(0, 1) FP32 draws rounded to BF16, generated in slices to bound memory."""
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = bf16_bits(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


def samu_inputs(B, L, D, seed, *, z0_std=None, dz_final_std=None, amp=0.5,
                with_dy=True):
    """Inputs of one SAMU forward+backward.

    Returns a dict with x_sel [B,L,D] bf16, b [B,L,M,2] bf16, w_phi/w_r [D+1]
    f32, a_phi/a_r [1] f32, nu/theta [M] f32, z0 [B,M,2] f32 or None, dy
    [B,L,M,2] bf16 (if with_dy) and dz_final [B,M,2] f32 or None.
    """
    if D % 2:
        raise ValueError("D must be even (M = D/2 complex modes)")
    M = D // 2
    rng = _rng(seed)
    out = {}
    out["x_sel"] = _normal_bf16(rng, (B, L, D))
    out["b"] = _normal_bf16(rng, (B, L, M, 2))
    out["theta"] = rng.uniform(0.0, 2.0 * math.pi, M).astype(np.float32)
    out["nu"] = (-np.log(rng.uniform(0.9, 0.999, M))).astype(np.float32)
    out["w_phi"] = rng.standard_normal(D + 1, dtype=np.float32)
    out["w_r"] = rng.standard_normal(D + 1, dtype=np.float32)
    out["a_phi"] = np.array([amp], np.float32)
    out["a_r"] = np.array([amp], np.float32)
    out["z0"] = (None if z0_std is None else
                 (z0_std * rng.standard_normal((B, M, 2))).astype(np.float32))
    out["dy"] = _normal_bf16(rng, (B, L, M, 2)) if with_dy else None
    out["dz_final"] = (None if dz_final_std is None else
                       (dz_final_std * rng.standard_normal((B, M, 2))).astype(np.float32))
    return out


def rglru_inputs(B, L, D, seed, *, reset_p=0.0, h0_std=None, dh_final_std=None,
                 with_dy=True):
    """Inputs of one RG-LRU forward+backward.

    Returns x, lx, la [B,L,D] bf16, alpha [D] f32, reset [B,L] uint8 or None,
    h0 [B,D] f32 or None, dy [B,L,D] bf16 and dh_final [B,D] f32 or None.
    """
    rng = _rng(seed)
    out = {}
    out["x"] = _normal_bf16(rng, (B, L, D))
    out["lx"] = _normal_bf16(rng, (B, L, D))
    out["la"] = _normal_bf16(rng, (B, L, D))
    s = rng.uniform(0.1, 1.0, D)                   # target softplus(alpha)
    out["alpha"] = np.log(np.expm1(s)).astype(np.float32)
    out["reset"] = ((rng.random((B, L)) < reset_p).astype(np.uint8)
                    if reset_p > 0 else None)
    out["h0"] = (None if h0_std is None else
                 (h0_std * rng.standard_normal((B, D))).astype(np.float32))
    out["dy"] = _normal_bf16(rng, (B, L, D)) if with_dy else None
    out["dh_final"] = (None if dh_final_std is None else
                       (dh_final_std * rng.standard_normal((B, D))).astype(np.float32))
    return out


def rglru_proj_inputs(D, seed):
    """Weights of the two 16-block block-diagonal gate projections: w_x, w_a
    bf16 [16, D/16, D/16] (block, output, input) ~ N(0, 1/(D/16)) so the
    logits keep unit scale for unit inputs; b_x, b_a f32 [D] ~ N(0, 0.1^2)."""
    if D % 16:
        raise ValueError("D must be a multiple of 16")
    Db = D // 16
    rng = _rng(seed)
    out = {}
    for g in ("x", "a"):
        w = rng.standard_normal((16, Db, Db), dtype=np.float32) / np.float32(math.sqrt(Db))
        out["w_" + g] = bf16_bits(w)
        out["b_" + g] = (0.1 * rng.standard_normal(D)).astype(np.float32)
    return out


def proj_cotangents(B, L, D, seed, *, bf16=False, std=0.01):
    """Logit cotangents dlx, dla and an incoming input gradient dx, all
    [B, L, D] ~ N(0, std^2): FP32, or BF16 bits when bf16 is set."""
    rng = _rng(seed)
    out = {}
    for k in ("dlx", "dla", "dx"):
        a = (std * rng.standard_normal((B, L, D), dtype=np.float32)).astype(np.float32)
        out[k] = bf16_bits(a) if bf16 else a
    return out


# Workloads the pages measure (seed = 1000 * workload index + row index).
WORKLOADS = {
    "samu_b1_l2048_d1024": dict(kind="samu", B=1, L=2048, D=1024, seed=0),
    "scan_sweep_b8_d1024": dict(kind="both", B=8, D=1024, L=(2048, 4096, 8192, 16384),
                                seed=1000, forward_only=True),
    "long_b1_d1024": dict(kind="both", B=1, D=1024, L=(32768, 65536, 131072), seed=2000),
    "wide_b1_l32768": dict(kind="both", B=1, L=32768, D=(1024, 1536, 2048, 2560), seed=3000,
                           state_std=0.1),
    "rglru_packed_b4_l8192_d2560": dict(kind="rglru", B=4, L=8192, D=2560, seed=4000,
                                        reset_p=1.0 / 512, state_std=0.1),
}
