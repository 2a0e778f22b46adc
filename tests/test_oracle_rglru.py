"""Pins of the FP64 RG-LRU oracle against things other than itself.

Equations: page 'SAMU 与 RG-LRU 的 H800 训练性能对比', section 04 (gates,
retention, normalized write, recurrence, segment reset, backward); reset
semantics also on page 'Griffin 第 4、5 节 H800 对照协议', 'RG-LRU 的固定方程'.
"""
import math

import numpy as np
import pytest
from scipy.signal import lfilter

import oracle


def _f64_inputs(B, L, D, seed, reset_p=0.0, h0=True, dhf=True):
    rng = np.random.default_rng(seed)
    return dict(
        x=rng.standard_normal((B, L, D)),
        lx=rng.standard_normal((B, L, D)),
        la=rng.standard_normal((B, L, D)),
        alpha=np.log(np.expm1(rng.uniform(0.1, 1.0, D))),
        reset=(rng.random((B, L)) < reset_p).astype(np.uint8) if reset_p > 0 else None,
        h0=rng.standard_normal((B, D)) * 0.5 if h0 else None,
        dy=rng.standard_normal((B, L, D)),
        dh_final=rng.standard_normal((B, D)) if dhf else None,
    )


def _fwd(inp):
    return oracle.rglru_fwd(inp["x"], inp["lx"], inp["la"], inp["alpha"], inp["reset"], inp["h0"])


def _bwd(inp):
    return oracle.rglru_bwd(inp["x"], inp["lx"], inp["la"], inp["alpha"], inp["reset"],
                            inp["h0"], inp["dy"], inp["dh_final"])


def test_reset_everywhere_gives_gated_input():
    """Every token a segment start: a = 0 and multiplier 1, so h_t = x_t sigmoid(l^x_t)
    and the initial state never leaks."""
    inp = _f64_inputs(2, 30, 5, 1)
    inp["reset"] = np.ones((2, 30), np.uint8)
    out = _fwd(inp)
    ref = inp["x"] / (1.0 + np.exp(-inp["lx"]))
    np.testing.assert_allclose(out["y"], ref, rtol=1e-14)
    g = _bwd(inp)
    assert np.all(g["dh0"] == 0.0)
    assert np.all(g["dla"] == 0.0) and np.all(g["dalpha"] == 0.0)


def test_constant_gates_are_a_geometric_filter():
    """softplus(alpha) = 1, l^a = 0, l^x = 0: a = exp(-4), multiplier
    sqrt(1 - exp(-8)), g^x = 1/2 -> h_t = a h_{t-1} + beta x_t (scipy lfilter)."""
    B, L, D = 1, 64, 3
    inp = _f64_inputs(B, L, D, 2)
    inp["alpha"] = np.full(D, math.log(math.e - 1.0))
    inp["lx"] = np.zeros((B, L, D))
    inp["la"] = np.zeros((B, L, D))
    a = math.exp(-4.0)
    beta = 0.5 * math.sqrt(1.0 - math.exp(-8.0))
    out = _fwd(inp)
    for dd in range(D):
        ref, _ = lfilter([beta], [1.0, -a], inp["x"][0, :, dd], zi=[a * inp["h0"][0, dd]])
        np.testing.assert_allclose(out["y"][0, :, dd], ref, rtol=1e-13, atol=1e-15)


def test_segment_start_cuts_the_state():
    """After a reset at position s the outputs equal a run of the suffix that
    starts with a segment start, from any initial state."""
    B, L, D, s = 1, 40, 4, 17
    inp = _f64_inputs(B, L, D, 3)
    inp["reset"] = np.zeros((B, L), np.uint8)
    inp["reset"][0, s] = 1
    full = _fwd(inp)["y"]
    suf = dict(inp)
    for k in ("x", "lx", "la"):
        suf[k] = inp[k][:, s:]
    suf["reset"] = np.zeros((B, L - s), np.uint8)
    suf["reset"][0, 0] = 1
    suf["h0"] = np.full((B, D), 123.0)
    np.testing.assert_allclose(full[:, s:], _fwd(suf)["y"], rtol=1e-14, atol=1e-15)


def _loss(inp):
    out = _fwd(inp)
    L = np.sum(inp["dy"] * out["y"])
    if inp["dh_final"] is not None:
        L += np.sum(inp["dh_final"] * out["h_final"])
    return L


def _fd(inp, key, idx, h):
    base = np.array(inp[key], dtype=np.float64, copy=True)
    vals = []
    for s in (+1, -1):
        pert = base.copy()
        pert[idx] += s * h
        vals.append(_loss(dict(inp, **{key: pert})))
    return (vals[0] - vals[1]) / (2 * h)


@pytest.mark.parametrize("reset_p", [0.0, 0.2])
def test_gradients_match_finite_differences(reset_p):
    B, L, D = 2, 19, 5
    inp = _f64_inputs(B, L, D, 4, reset_p=reset_p)
    if reset_p:
        inp["reset"][0, 0] = 1          # also a reset at t = 0
        inp["reset"][1, 5:7] = 1        # and two consecutive ones
    g = _bwd(inp)
    rng = np.random.default_rng(5)
    idx3 = [tuple(rng.integers(0, s) for s in (B, L, D)) for _ in range(8)]
    checks = {"x": ("dx", idx3), "lx": ("dlx", idx3), "la": ("dla", idx3),
              "alpha": ("dalpha", [(d,) for d in range(D)]),
              "h0": ("dh0", [(b, d) for b in range(B) for d in range(D)])}
    for key, (gkey, idxs) in checks.items():
        for idx in idxs:
            fd = _fd(inp, key, idx, 1e-6)
            an = g[gkey][idx]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (key, idx, fd, an)


def test_adjoint_dot_product_identity():
    """Gates fixed, y and h_L are linear in (x, h0)."""
    inp = _f64_inputs(3, 33, 6, 6, reset_p=0.1)
    out = _fwd(inp)
    g = _bwd(inp)
    lhs = np.sum(inp["dy"] * out["y"]) + np.sum(inp["dh_final"] * out["h_final"])
    rhs = np.sum(g["dx"] * inp["x"]) + np.sum(g["dh0"] * inp["h0"])
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def test_square_root_derivative_is_capped():
    """When 1 - a^2 underflows the cap, d sqrt(u)/du is limited to 1000: the
    a-gradient uses -a / sqrt(2.5e-7) instead of the (huge) exact value."""
    alpha = np.array([-30.0])                 # softplus ~ 9.4e-14, a ~ 1 - 3.7e-13
    x = np.array([[[0.7]]])
    lx = np.array([[[0.3]]])
    la = np.array([[[0.0]]])
    dy = np.array([[[1.0]]])
    g = oracle.rglru_bwd(x, lx, la, alpha, None, None, dy, None)
    sp = math.log1p(math.exp(-30.0))
    ga, gx = 0.5, 1.0 / (1.0 + math.exp(-0.3))
    a = math.exp(-8.0 * ga * sp)
    abar = 1.0 * 0.7 * gx * (-a / math.sqrt(2.5e-7))
    expected = abar * a * (-8.0 * sp) * ga * (1 - ga)
    assert g["dla"][0, 0, 0] == pytest.approx(expected, rel=1e-12)
    uncapped = 1.0 * 0.7 * gx * (-a / math.sqrt(1 - a * a)) * a * (-8.0 * sp) * ga * (1 - ga)
    assert abs(uncapped) > 100 * abs(expected)
