"""Pins of the oracle's RG-LRU gate projections (16-block block-diagonal
linear layers, page "Griffin 第 4、5 节 H800 对照协议", "RG-LRU 的固定方程")
against computations it does not share: a dense block-diagonal matrix
product, identity weights, block locality, the adjoint identity and
per-block outer-product sums."""
import numpy as np
import scipy.linalg

import oracle
from linear_recurrence_sequence_amd import inputs


def _setup(B=2, L=7, D=64, seed=5):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, L, D))
    w = rng.standard_normal((16, D // 16, D // 16))
    b = rng.standard_normal(D)
    return x, w, b


def test_matches_dense_block_diagonal_product():
    x, w, b = _setup()
    dense = scipy.linalg.block_diag(*w)                       # [D, D] as (output, input)
    ref = x @ dense.T + b
    got = oracle.rglru_gate_proj(x, w, b)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_identity_blocks_pass_the_input_through():
    x, _, _ = _setup(D=48)
    w = np.stack([np.eye(3)] * 16)
    got = oracle.rglru_gate_proj(x, w, np.zeros(48))
    assert np.array_equal(got, x)


def test_blocks_are_independent():
    x, w, b = _setup(D=128)
    base = oracle.rglru_gate_proj(x, w, b)
    x2 = x.copy()
    x2[..., 40:48] += 1.0                                    # inside block 5 (channels 40..47)
    diff = np.abs(oracle.rglru_gate_proj(x2, w, b) - base).max(axis=(0, 1))
    assert np.all(diff[:40] == 0) and np.all(diff[48:] == 0) and np.all(diff[40:48] > 0)


def test_adjoint_identity_and_parameter_gradients():
    x, w, b = _setup(B=3, L=11, D=64, seed=9)
    rng = np.random.default_rng(10)
    dl = rng.standard_normal(x.shape)
    dx0 = rng.standard_normal(x.shape)
    dx, dw, db = oracle.rglru_gate_proj_bwd(x, w, dl, dx0)
    lin = oracle.rglru_gate_proj(x, w, np.zeros(64))         # the linear part W x
    # <dl, W x> = <W^T dl, x>
    assert abs(np.sum(dl * lin) - np.sum((dx - dx0) * x)) <= 1e-10 * np.sum(np.abs(dl * lin))
    Db = 4
    xb = x.reshape(-1, 16, Db)
    dlb = dl.reshape(-1, 16, Db)
    assert np.allclose(dw, np.einsum("tio,tik->iok", dlb, xb), rtol=1e-12, atol=1e-12)
    assert np.allclose(db, dl.reshape(-1, 64).sum(0), rtol=1e-12, atol=1e-12)


def test_weight_inputs_have_unit_logit_scale():
    p = inputs.rglru_proj_inputs(256, 3)
    x = inputs.rglru_inputs(1, 64, 256, 4, with_dy=False)["x"]
    lx = oracle.rglru_gate_proj(x, p["w_x"], p["b_x"])
    assert 0.7 < np.std(lx) < 1.3
