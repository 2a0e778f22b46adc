"""Pins of the FP64 SAMU oracle against things other than itself.

Each test checks the oracle against a closed form, a textbook identity, a
library routine, finite differences or an invariant fixed by the mathematics
of the pages ('SAMU 与 RG-LRU 的 H800 训练性能对比', section 05), so that a
dropped term, a wrong sign, a wrong index or a transposed operand anywhere in
the oracle fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle
from linear_recurrence_sequence_amd import inputs

RNG = np.random.default_rng(12345)


def _f64_inputs(B, L, D, seed, amp_phi=0.8, amp_r=-0.6, z0=True, dzf=True):
    rng = np.random.default_rng(seed)
    M = D // 2
    return dict(
        x_sel=rng.standard_normal((B, L, D)),
        b=rng.standard_normal((B, L, M, 2)),
        w_phi=rng.standard_normal(D + 1),
        w_r=rng.standard_normal(D + 1),
        a_phi=np.array([amp_phi]), a_r=np.array([amp_r]),
        nu=-np.log(rng.uniform(0.5, 0.999, M)),
        theta=rng.uniform(0, 2 * np.pi, M),
        z0=rng.standard_normal((B, M, 2)) * 0.5 if z0 else None,
        dy=rng.standard_normal((B, L, M, 2)),
        dz_final=rng.standard_normal((B, M, 2)) if dzf else None,
    )


def _fwd(inp):
    return oracle.samu_fwd(inp["x_sel"], inp["b"], inp["w_phi"], inp["w_r"], inp["a_phi"],
                           inp["a_r"], inp["nu"], inp["theta"], inp["z0"])


def _bwd(inp):
    return oracle.samu_bwd(inp["x_sel"], inp["b"], inp["w_phi"], inp["w_r"], inp["a_phi"],
                           inp["a_r"], inp["nu"], inp["theta"], inp["z0"], inp["dy"],
                           inp["dz_final"])


def _cplx(a):
    return a[..., 0] + 1j * a[..., 1]


# --------------------------------------------------------------------------
# Controller: designed inputs whose projections are known in closed form.
# --------------------------------------------------------------------------
def test_controller_designed_values():
    D, M = 4, 2
    w_phi = np.array([3.0, 0.0, 0.0, 0.0, 4.0])   # norm 5 over all D+1 entries
    w_r = np.array([0.0, 2.0, 0.0, 0.0, 0.0])     # unit direction e_1
    x = np.zeros((1, 2, D))
    x[0, 0] = [1.0, 0.5, 0.0, 0.0]               # u_phi = 3/5 + 4/5 = 1.4, u_r = 0.5
    # token 1: x = 0 -> u_phi = 4/5 (the appended 1 hits the bias), u_r = 0
    a_phi, a_r = 0.3, -1.1
    ctl = oracle.samu_controller(x, w_phi, w_r, np.array([a_phi]), np.array([a_r]))
    u_phi = np.array([1.4, 0.8])
    u_r = np.array([0.5, 0.0])
    p = np.tanh(u_phi)
    # q(tanh u) = tanh(u)/(1+tanh(u)^2) = tanh(2u)/2 (double-angle identity)
    q = np.tanh(2 * u_r) / 2
    d = math.tanh(a_phi) / math.sqrt(M) * p
    c = math.tanh(a_r) / math.sqrt(M) * q
    np.testing.assert_allclose(ctl["p"][0], p, rtol=1e-14)
    np.testing.assert_allclose(ctl["r"][0], np.tanh(u_r), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(ctl["d"][0], d, rtol=1e-14)
    np.testing.assert_allclose(ctl["c"][0], c, rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(ctl["E"][0], np.exp(c), rtol=1e-14)
    np.testing.assert_allclose(ctl["C"][0], np.cos(d), rtol=1e-14)
    np.testing.assert_allclose(ctl["S"][0], np.sin(d), rtol=1e-14)


def test_controller_direction_scale_invariance():
    inp = _f64_inputs(2, 9, 8, 1)
    c1 = oracle.samu_controller(inp["x_sel"], inp["w_phi"], inp["w_r"], inp["a_phi"], inp["a_r"])
    c2 = oracle.samu_controller(inp["x_sel"], 3.7 * inp["w_phi"], 0.01 * inp["w_r"],
                                inp["a_phi"], inp["a_r"])
    for k in "prdc":
        np.testing.assert_allclose(c1[k], c2[k], rtol=1e-12, atol=1e-15)


# --------------------------------------------------------------------------
# Transition + recurrence.
# --------------------------------------------------------------------------
def test_impulse_response_is_exact_chunk_product():
    """Unit impulse at the first token: y_t = prod_{s=2..t} lambda_s, whose
    closed form is exp(-nu sum E) exp(i((t-1) theta + sum d))  (the exact
    chunk-product closed form of section 05, 'G_c, D_c')."""
    B, L, D = 1, 37, 8
    M = D // 2
    inp = _f64_inputs(B, L, D, 2, amp_phi=1.3, amp_r=-0.9, z0=False)
    for drive in (1.0, 1j):
        b = np.zeros((B, L, M, 2))
        b[0, 0, :, 0] = np.real(drive)
        b[0, 0, :, 1] = np.imag(drive)
        inp["b"] = b
        y = _cplx(_fwd(inp)["y"])[0]                      # [L, M]
        ctl = oracle.samu_controller(inp["x_sel"], inp["w_phi"], inp["w_r"], inp["a_phi"],
                                     inp["a_r"])
        E, d = ctl["E"][0], ctl["d"][0]
        G = np.concatenate([[0.0], np.cumsum(E[1:])])      # sum_{s=2..t} E_s
        Dsum = np.concatenate([[0.0], np.cumsum(d[1:])])
        k = np.arange(L)[:, None]
        ref = drive * np.exp(-inp["nu"][None, :] * G[:, None]) * \
            np.exp(1j * (k * inp["theta"][None, :] + Dsum[:, None]))
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)
    # the controls really vary, so the test above is not the static case
    assert np.ptp(d) > 1e-2 and np.ptp(E) > 1e-2


def test_rtu_degeneration_closed_form():
    """a_phi = a_r = 0: lambda_m = exp(-nu_m) exp(i theta_m) is static and
    z_t = lambda^t z0 + sum_{s<=t} lambda^{t-s} b_s (numpy.convolve)."""
    B, L, D = 2, 50, 12
    M = D // 2
    inp = _f64_inputs(B, L, D, 3, amp_phi=0.0, amp_r=0.0)
    out = _fwd(inp)
    y = _cplx(out["y"])
    lam = np.exp(-inp["nu"]) * np.exp(1j * inp["theta"])
    for bb in range(B):
        for m in range(M):
            bs = _cplx(inp["b"])[bb, :, m]
            z0 = _cplx(inp["z0"])[bb, m]
            kern = lam[m] ** np.arange(L)
            ref = np.convolve(bs, kern)[:L] + z0 * lam[m] ** np.arange(1, L + 1)
            np.testing.assert_allclose(y[bb, :, m], ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(_cplx(out["z_final"]), y[:, -1], rtol=0, atol=0)


def test_cumsum_special_case():
    """nu = 0, theta = 0, zero amplitudes: lambda = 1 and z = z0 + cumsum(b)."""
    B, L, D = 2, 40, 6
    inp = _f64_inputs(B, L, D, 4, amp_phi=0.0, amp_r=0.0)
    inp["nu"] = np.zeros(D // 2)
    inp["theta"] = np.zeros(D // 2)
    y = _cplx(_fwd(inp)["y"])
    ref = _cplx(inp["z0"])[:, None, :] + np.cumsum(_cplx(inp["b"]), axis=1)
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_forgetful_modes_return_the_drive():
    """nu -> large: |lambda| = exp(-nu E) underflows, so z_t = b_t."""
    inp = _f64_inputs(1, 20, 8, 5)
    inp["nu"] = np.full(4, 1.0e4)
    y = _fwd(inp)["y"]
    np.testing.assert_array_equal(y, inp["b"])


# --------------------------------------------------------------------------
# Adjoint.
# --------------------------------------------------------------------------
def _loss(inp):
    out = _fwd(inp)
    L = np.sum(inp["dy"] * out["y"])
    if inp["dz_final"] is not None:
        L += np.sum(inp["dz_final"] * out["z_final"])
    return L


def _fd(inp, key, idx, h):
    base = np.array(inp[key], dtype=np.float64, copy=True)
    vals = []
    for s in (+1, -1):
        pert = base.copy()
        pert[idx] += s * h
        q = dict(inp)
        q[key] = pert
        vals.append(_loss(q))
    return (vals[0] - vals[1]) / (2 * h)


@pytest.mark.parametrize("amps", [(0.8, -0.6), (2.0, 1.5)])
def test_gradients_match_finite_differences(amps):
    B, L, D = 2, 13, 8
    inp = _f64_inputs(B, L, D, 6, amp_phi=amps[0], amp_r=amps[1])
    g = _bwd(inp)
    rng = np.random.default_rng(7)
    checks = {
        "x_sel": ("dx_sel", [tuple(rng.integers(0, s) for s in (B, L, D)) for _ in range(6)]),
        "b": ("db", [tuple(rng.integers(0, s) for s in (B, L, D // 2, 2)) for _ in range(6)]),
        "z0": ("dz0", [tuple(rng.integers(0, s) for s in (B, D // 2, 2)) for _ in range(4)]),
        "w_phi": ("dw_phi", [(j,) for j in (0, 3, D)]),
        "w_r": ("dw_r", [(j,) for j in (1, 5, D)]),
        "nu": ("dnu", [(m,) for m in range(D // 2)]),
        "theta": ("dtheta", [(m,) for m in range(D // 2)]),
        "a_phi": ("da_phi", [(0,)]),
        "a_r": ("da_r", [(0,)]),
    }
    for key, (gkey, idxs) in checks.items():
        for idx in idxs:
            fd = _fd(inp, key, idx, 1e-6)
            an = g[gkey] if np.isscalar(g[gkey]) else g[gkey][idx]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (key, idx, fd, an)


def test_adjoint_dot_product_identity():
    """Controls fixed, y and z_L are linear in (b, z0):
    <dy, y> + <dz_L, z_L> = <db, b> + <dz0, z0>."""
    inp = _f64_inputs(3, 41, 10, 8)
    out = _fwd(inp)
    g = _bwd(inp)
    lhs = np.sum(inp["dy"] * out["y"]) + np.sum(inp["dz_final"] * out["z_final"])
    rhs = np.sum(g["db"] * inp["b"]) + np.sum(g["dz0"] * inp["z0"])
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def test_direction_gradient_invariants():
    inp = _f64_inputs(2, 17, 8, 9)
    g1 = _bwd(inp)
    # dw is orthogonal to w (the loss is invariant to the scale of w)
    for k, w in (("dw_phi", inp["w_phi"]), ("dw_r", inp["w_r"])):
        assert abs(np.dot(g1[k], w)) <= 1e-12 * np.linalg.norm(g1[k]) * np.linalg.norm(w)
        assert np.linalg.norm(g1[k]) > 1e-6
    s = 3.7
    q = dict(inp, w_phi=s * inp["w_phi"], w_r=s * inp["w_r"])
    np.testing.assert_allclose(_fwd(q)["y"], _fwd(inp)["y"], rtol=1e-12, atol=1e-12)
    g2 = _bwd(q)
    np.testing.assert_allclose(g2["dw_phi"], g1["dw_phi"] / s, rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(g2["dw_r"], g1["dw_r"] / s, rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(g2["dx_sel"], g1["dx_sel"], rtol=1e-10, atol=1e-14)


def test_rtu_controller_gradients_vanish_exactly():
    """At zero amplitude d and c do not depend on x_sel or w, so their
    gradients are exactly zero; the amplitude gradients are not."""
    inp = _f64_inputs(2, 15, 8, 10, amp_phi=0.0, amp_r=0.0)
    g = _bwd(inp)
    assert np.all(g["dx_sel"] == 0.0)
    assert np.all(g["dw_phi"] == 0.0) and np.all(g["dw_r"] == 0.0)
    assert abs(g["da_phi"]) > 1e-6 and abs(g["da_r"]) > 1e-6
    fd = _fd(inp, "a_phi", (0,), 1e-6)
    assert abs(fd - g["da_phi"]) <= 1e-6 * max(1.0, abs(fd))


# --------------------------------------------------------------------------
# Chunked composition: a test-only FP64 evaluator of the pages' hierarchy
# (S_c, L_c, U_g, O_g, Q_c = L_c o O_g) must reproduce the serial oracle for
# any chunk length K and group size G, and the order of composition matters.
# --------------------------------------------------------------------------
def _compose(second, first, swap=False):
    """(l2, b2) o (l1, b1) = (l2 l1, l2 b1 + b2): `first` runs first."""
    (l2, b2), (l1, b1) = second, first
    if swap:
        (l2, b2), (l1, b1) = (l1, b1), (l2, b2)
    return (l2 * l1, l2 * b1 + b2)


def _chunked_scan(lam, drv, z0, K, G, swap=False, outer_swap=False):
    """lam, drv: [L, M] complex; z0 [M].  Returns all states [L, M]."""
    L, M = lam.shape
    C = -(-L // K)
    ident = (np.ones(M, complex), np.zeros(M, complex))
    S = []
    for c in range(C):
        acc = ident
        for t in range(c * K, min(L, (c + 1) * K)):
            acc = _compose((lam[t], drv[t]), acc, swap)
        S.append(acc)
    NG = -(-C // G)
    U = []
    for g in range(NG):
        acc = ident
        for c in range(g * G, min(C, (g + 1) * G)):
            acc = _compose(S[c], acc, swap)
        U.append(acc)
    out = np.empty((L, M), complex)
    O = ident
    for g in range(NG):
        Lc = ident
        for c in range(g * G, min(C, (g + 1) * G)):
            Q = _compose(Lc, O, outer_swap)          # Q_c = L_c o O_g
            h = Q[0] * z0 + Q[1]
            for t in range(c * K, min(L, (c + 1) * K)):
                h = lam[t] * h + drv[t]
                out[t] = h
            Lc = _compose(S[c], Lc, swap)
        O = _compose(U[g], O, swap)
    return out


def _lambda(inp):
    ctl = oracle.samu_controller(inp["x_sel"], inp["w_phi"], inp["w_r"], inp["a_phi"], inp["a_r"])
    E, C, S = ctl["E"][0], ctl["C"][0], ctl["S"][0]
    rho = np.exp(-inp["nu"][None, :] * E[:, None])
    ct, st = np.cos(inp["theta"])[None, :], np.sin(inp["theta"])[None, :]
    return rho * ((ct * C[:, None] - st * S[:, None]) + 1j * (st * C[:, None] + ct * S[:, None]))


@pytest.mark.parametrize("K,G", [(1, 1), (2, 4), (3, 2), (5, 64), (32, 1), (32, 2), (7, 3)])
def test_chunked_hierarchy_equals_serial(K, G):
    L, D = 101, 8
    inp = _f64_inputs(1, L, D, 11)
    ref = _cplx(_fwd(inp)["y"])[0]
    got = _chunked_scan(_lambda(inp), _cplx(inp["b"])[0], _cplx(inp["z0"])[0], K, G)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_composition_order_is_not_commutative():
    L, D = 101, 8
    inp = _f64_inputs(1, L, D, 11)
    ref = _cplx(_fwd(inp)["y"])[0]
    lam, drv, z0 = _lambda(inp), _cplx(inp["b"])[0], _cplx(inp["z0"])[0]
    bad1 = _chunked_scan(lam, drv, z0, 5, 4, swap=True)
    bad2 = _chunked_scan(lam, drv, z0, 5, 4, outer_swap=True)
    for bad in (bad1, bad2):
        assert np.max(np.abs(bad - ref)) > 1e-2 * np.max(np.abs(ref))


def _reverse_chunked_adjoint(lam, dy, dzf, K, G, forward_order=False):
    """Reverse affine hierarchy on conj(lambda): per chunk the map from the
    cotangent arriving after the chunk to the one leaving before it.  Returns
    (db [L, M], dz0 [M])."""
    L, M = lam.shape
    C = -(-L // K)
    ident = (np.ones(M, complex), np.zeros(M, complex))
    R = []
    for c in range(C):
        acc = ident
        for t in range(min(L, (c + 1) * K) - 1, c * K - 1, -1):
            # carry -> conj(lambda_t) (dy_t + carry)
            step = (np.conj(lam[t]), np.conj(lam[t]) * dy[t])
            acc = _compose(step, acc)
        R.append(acc)
    order = list(range(C)) if forward_order else list(range(C - 1, -1, -1))
    groups = [order[i:i + G] for i in range(0, C, G)]
    U = []
    for grp in groups:
        acc = ident
        for c in grp:
            acc = _compose(R[c], acc)
        U.append(acc)
    db = np.empty((L, M), complex)
    O = ident
    carry_out = None
    for gi, grp in enumerate(groups):
        Lc = ident
        for c in grp:
            Q = _compose(Lc, O)
            carry = Q[0] * dzf + Q[1]
            for t in range(min(L, (c + 1) * K) - 1, c * K - 1, -1):
                gt = dy[t] + carry
                db[t] = gt
                carry = np.conj(lam[t]) * gt
            carry_out = carry
            Lc = _compose(R[c], Lc)
        O = _compose(U[gi], O)
    return db, carry_out


@pytest.mark.parametrize("K,G", [(1, 3), (4, 2), (32, 64), (6, 1)])
def test_reverse_hierarchy_equals_serial_adjoint(K, G):
    L, D = 77, 8
    inp = _f64_inputs(1, L, D, 12)
    g = _bwd(inp)
    db, dz0 = _reverse_chunked_adjoint(_lambda(inp), _cplx(inp["dy"])[0],
                                       _cplx(inp["dz_final"])[0], K, G)
    np.testing.assert_allclose(db, _cplx(g["db"])[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dz0, _cplx(g["dz0"])[0], rtol=1e-12, atol=1e-12)
    bad_db, _ = _reverse_chunked_adjoint(_lambda(inp), _cplx(inp["dy"])[0],
                                         _cplx(inp["dz_final"])[0], 4, 2, forward_order=True)
    assert np.max(np.abs(bad_db - _cplx(g["db"])[0])) > 1e-2


# --------------------------------------------------------------------------
# BF16 / FP32 bit patterns reach the oracle exactly.
# --------------------------------------------------------------------------
def test_bf16_inputs_are_widened_exactly():
    inp = inputs.samu_inputs(1, 33, 16, seed=13, z0_std=0.1)
    f = {k: (oracle.widen(v) if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    a = oracle.samu_fwd(inp["x_sel"], inp["b"], inp["w_phi"], inp["w_r"], inp["a_phi"],
                        inp["a_r"], inp["nu"], inp["theta"], inp["z0"])
    b = oracle.samu_fwd(f["x_sel"], f["b"], f["w_phi"], f["w_r"], f["a_phi"], f["a_r"],
                        f["nu"], f["theta"], f["z0"])
    np.testing.assert_array_equal(a["y"], b["y"])
    # bf16 RNE of the generator: spot values
    bits = inputs.bf16_bits(np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e38], np.float32))
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x7F62]
