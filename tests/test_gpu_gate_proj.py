"""GPU parity of the RG-LRU gate projections (16-block block-diagonal,
matrix cores) and of the whole input-to-output RG-LRU layer against the FP64
oracle.

The logits are rounded to BF16, a rounding decision: the GPU (FP32
accumulation) must return the BF16 rounding of the exact FP64 logit except
within FP32 accumulation error of a rounding tie.  The scan and the
projection adjoint are then compared against the oracle fed the GPU's own
BF16 logits, so both sides share that decision."""
import numpy as np
import pytest
import torch

import oracle
from linear_recurrence_sequence_amd import inputs
from tests.helpers import dev_tensor, rel_l2, say, to_f64

pytestmark = pytest.mark.gpu

TOL_OUT, TOL_GRAD = 1e-5, 1e-4


def _check_logits(name, gpu_bf16, x, w, b):
    exact = oracle.rglru_gate_proj(x, w, b)
    mag = oracle.rglru_gate_proj(np.abs(oracle.widen(x)), np.abs(oracle.widen(w)), np.zeros(exact.shape[-1]))
    g = to_f64(gpu_bf16)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(exact), 1e-30))) - 7)
    err = np.abs(g - exact)
    slack = 1e-6 * mag + 1e-30
    assert np.all(err <= 0.5 * ulp + slack), (name, float(np.max(err / (0.5 * ulp + slack))))
    rne = torch.from_numpy(exact).to(torch.bfloat16).double().numpy()
    frac = np.mean(g != rne)
    say(f"   {name}: logits differing from the FP64 rounding (near ties): {frac:.2e}")
    assert frac < 1e-3


def _layer(B, L, D, seed, reset_p, std):
    inp = inputs.rglru_inputs(B, L, D, seed, reset_p=reset_p, h0_std=std, dh_final_std=std)
    prm = inputs.rglru_proj_inputs(D, seed + 1)
    return inp, prm


def _run(B, L, D, seed, reset_p=0.0, std=0.1, dtype=torch.float32):
    from linear_recurrence_sequence_amd import scan
    inp, prm = _layer(B, L, D, seed, reset_p, std)
    d = {k: dev_tensor(v) for k, v in {**inp, **prm}.items()}
    lx, la = scan.rglru_gate_proj_fwd(d["x"], d["w_x"], d["b_x"], d["w_a"], d["b_a"])
    y, hf, saved = scan.rglru_scan_fwd(d["x"], lx, la, d["alpha"], d["reset"], d["h0"], y_dtype=dtype)
    g = scan.rglru_scan_bwd(d["x"], lx, la, d["alpha"], d["reset"], saved, d["dy"], d["dh_final"],
                            grad_dtype=dtype)
    p = scan.rglru_gate_proj_bwd(d["x"], d["w_x"], d["w_a"], g["dlx"], g["dla"], g["dx"])
    torch.cuda.synchronize()
    return inp, prm, lx, la, y, hf, g, p


@pytest.mark.parametrize("B,L,D,reset_p", [(2, 300, 256, 1 / 64), (1, 1000, 2560, 0.0), (3, 77, 512, 0.1)])
def test_layer_parity(B, L, D, reset_p):
    say(f"[gate proj] B={B} L={L} D={D}: projections, scan F+B, projection adjoint (f32)")
    inp, prm, lx, la, y, hf, g, p = _run(B, L, D, 700 + L, reset_p)
    _check_logits("l^x", lx, inp["x"], prm["w_x"], prm["b_x"])
    _check_logits("l^a", la, inp["x"], prm["w_a"], prm["b_a"])
    lxg = lx.view(torch.int16).cpu().numpy().view(np.uint16)
    lag = la.view(torch.int16).cpu().numpy().view(np.uint16)
    say(f"[gate proj] B={B} L={L} D={D}: oracle on the GPU's logits")
    rf = oracle.rglru_fwd(inp["x"], lxg, lag, inp["alpha"], inp["reset"], inp["h0"])
    rg = oracle.rglru_bwd(inp["x"], lxg, lag, inp["alpha"], inp["reset"], inp["h0"], inp["dy"], inp["dh_final"])
    dx, dw_x, db_x = oracle.rglru_gate_proj_bwd(inp["x"], prm["w_x"], rg["dlx"], rg["dx"])
    dx, dw_a, db_a = oracle.rglru_gate_proj_bwd(inp["x"], prm["w_a"], rg["dla"], dx)
    errs = {"y": rel_l2(to_f64(y), rf["y"]), "h_final": rel_l2(to_f64(hf), rf["h_final"]),
            "dx": rel_l2(to_f64(p["dx"]), dx), "dw_x": rel_l2(to_f64(p["dw_x"]), dw_x),
            "db_x": rel_l2(to_f64(p["db_x"]), db_x), "dw_a": rel_l2(to_f64(p["dw_a"]), dw_a),
            "db_a": rel_l2(to_f64(p["db_a"]), db_a), "dalpha": rel_l2(to_f64(g["dalpha"]), rg["dalpha"])}
    say("   errors:", {k: f"{v:.2e}" for k, v in errs.items()})
    assert errs["y"] <= TOL_OUT and errs["h_final"] <= TOL_OUT
    for k in ("dx", "dw_x", "db_x", "dw_a", "db_a", "dalpha"):
        assert errs[k] <= TOL_GRAD, (k, errs[k])


def _u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def test_layer_full_size_and_bf16_mode():
    """B=1, L=32768, D=2048 (the metric shape): every output of the layer
    against the oracle fed the GPU's BF16 logits (a rounding decision both
    sides then share).
      * FP32 mode: y, h_final at 1e-5; dx (scan and projection adjoints
        summed), dW, db, d alpha, dh0 at 1e-4.
      * BF16 mode: y within the BF16 floor + 1e-5, h_final, d alpha, dh0 at
        1e-5 / 1e-4; the projection adjoint against the oracle fed the same
        BF16 cotangents the GPU multiplied: dx_out within half a BF16 ulp of
        the exact sum plus FP32 accumulation slack, dW and db at 1e-5."""
    from tests.helpers import bf16_floor
    B, L, D = 1, 32768, 2048
    for mode, dt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        say(f"[gate proj] full size B={B} L={L} D={D}, {mode} mode")
        inp, prm, lx, la, y, hf, g, p = _run(B, L, D, 3103, 0.0, dtype=dt)
        _check_logits("l^x", lx, inp["x"], prm["w_x"], prm["b_x"])
        _check_logits("l^a", la, inp["x"], prm["w_a"], prm["b_a"])
        say(f"[gate proj] full size {mode}: oracle on the GPU's logits")
        lxg, lag = _u16(lx), _u16(la)
        rf = oracle.rglru_fwd(inp["x"], lxg, lag, inp["alpha"], inp["reset"], inp["h0"])
        rg = oracle.rglru_bwd(inp["x"], lxg, lag, inp["alpha"], inp["reset"], inp["h0"], inp["dy"],
                              inp["dh_final"])
        e = {"y": rel_l2(to_f64(y), rf["y"]), "h_final": rel_l2(to_f64(hf), rf["h_final"]),
             "dalpha": rel_l2(to_f64(g["dalpha"]), rg["dalpha"]), "dh0": rel_l2(to_f64(g["dh0"]), rg["dh0"])}
        if mode == "f32":
            dl_x, dl_a, dx_in = rg["dlx"], rg["dla"], rg["dx"]
        else:
            dl_x, dl_a, dx_in = _u16(g["dlx"]), _u16(g["dla"]), _u16(g["dx"])
        dx, dw_x, db_x = oracle.rglru_gate_proj_bwd(inp["x"], prm["w_x"], dl_x, dx_in)
        dx, dw_a, db_a = oracle.rglru_gate_proj_bwd(inp["x"], prm["w_a"], dl_a, dx)
        for k, ref in (("dw_x", dw_x), ("db_x", db_x), ("dw_a", dw_a), ("db_a", db_a)):
            e[k] = rel_l2(to_f64(p[k]), ref)
        if mode == "f32":
            e["dx"] = rel_l2(to_f64(p["dx"]), dx)
        say("   errors:", {k: f"{v:.2e}" for k, v in e.items()})
        assert e["y"] <= (bf16_floor(rf["y"]) if mode == "bf16" else 0.0) + TOL_OUT
        assert e["h_final"] <= TOL_OUT
        for k in ("dalpha", "dh0") + (("dx",) if mode == "f32" else ()):
            assert e[k] <= TOL_GRAD, (k, e[k])
        for k in ("dw_x", "db_x", "dw_a", "db_a"):
            assert e[k] <= (TOL_GRAD if mode == "f32" else TOL_OUT), (k, e[k])
        if mode == "bf16":
            # |dx_in| + sum |W| |dl| bounds the FP32 accumulation error
            ax = np.abs(oracle.widen(inp["x"]))
            mx, _, _ = oracle.rglru_gate_proj_bwd(ax, np.abs(oracle.widen(prm["w_x"])),
                                                  np.abs(oracle.widen(dl_x)), np.abs(oracle.widen(dx_in)))
            mag, _, _ = oracle.rglru_gate_proj_bwd(ax, np.abs(oracle.widen(prm["w_a"])),
                                                   np.abs(oracle.widen(dl_a)), mx)
            _check_bf16_output("dx", p["dx"], dx, mag)
            del ax, mx, mag
        del inp, prm, lx, la, y, hf, g, p, rf, rg, dx


def test_projection_in_place_and_deterministic():
    from linear_recurrence_sequence_amd import scan
    inp, prm = _layer(2, 500, 512, 41, 0.0, 0.1)
    d = {k: dev_tensor(v) for k, v in {**inp, **prm}.items()}
    say("[gate proj] in-place accumulation and determinism B=2 L=500 D=512")
    dl1 = torch.randn(2, 500, 512, device="cuda")
    dl2 = torch.randn(2, 500, 512, device="cuda")
    dx = torch.randn(2, 500, 512, device="cuda")
    a = scan.rglru_gate_proj_bwd(d["x"], d["w_x"], d["w_a"], dl1, dl2, dx)
    b = scan.rglru_gate_proj_bwd(d["x"], d["w_x"], d["w_a"], dl1, dl2, dx)
    dx2 = dx.clone()
    c = scan.rglru_gate_proj_bwd(d["x"], d["w_x"], d["w_a"], dl1, dl2, dx2, dx_out=dx2)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]) and torch.equal(a[k], c[k]), k


def _check_bf16_output(name, gpu_bf16, exact, mag):
    """A BF16 result rounded from an FP32 sum: within half a BF16 ulp of the
    exact value plus FP32 accumulation slack, and RNE of it off ties."""
    g = to_f64(gpu_bf16)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(exact), 1e-30))) - 7)
    slack = 1e-6 * mag + 1e-30
    err = np.abs(g - exact)
    assert np.all(err <= 0.5 * ulp + slack), (name, float(np.max(err / (0.5 * ulp + slack))))
    rne = torch.from_numpy(exact).to(torch.bfloat16).double().numpy()
    frac = np.mean(g != rne)
    say(f"   {name}: values differing from the FP64 rounding (near ties): {frac:.2e}")
    assert frac < 1e-3


@pytest.mark.parametrize("D", [768, 1024, 1280, 1536, 1792, 2304])
@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_projection_odd_tiles_and_modes(D, mode):
    """Every block width the other tests do not reach (3 to 9 tiles of 16
    channels, the odd ones with a half-used last pair), a ragged token count,
    both cotangent precisions: logits, dx, dW and db against the FP64
    oracle."""
    from linear_recurrence_sequence_amd import scan
    B, L = 2, 333
    say(f"[gate proj] B={B} L={L} D={D} cotangents {mode}")
    x = inputs.rglru_inputs(B, L, D, 900 + D)["x"]
    prm = inputs.rglru_proj_inputs(D, 901 + D)
    ct = inputs.proj_cotangents(B, L, D, 902 + D, bf16=(mode == "bf16"))
    d = {k: dev_tensor(v) for k, v in {"x": x, **prm, **ct}.items()}
    lx, la = scan.rglru_gate_proj_fwd(d["x"], d["w_x"], d["b_x"], d["w_a"], d["b_a"])
    p = scan.rglru_gate_proj_bwd(d["x"], d["w_x"], d["w_a"], d["dlx"], d["dla"], d["dx"])
    torch.cuda.synchronize()
    _check_logits("l^x", lx, x, prm["w_x"], prm["b_x"])
    _check_logits("l^a", la, x, prm["w_a"], prm["b_a"])
    dx, dw_x, db_x = oracle.rglru_gate_proj_bwd(x, prm["w_x"], ct["dlx"], ct["dx"])
    dx, dw_a, db_a = oracle.rglru_gate_proj_bwd(x, prm["w_a"], ct["dla"], dx)
    errs = {"dw_x": rel_l2(to_f64(p["dw_x"]), dw_x), "db_x": rel_l2(to_f64(p["db_x"]), db_x),
            "dw_a": rel_l2(to_f64(p["dw_a"]), dw_a), "db_a": rel_l2(to_f64(p["db_a"]), db_a)}
    if mode == "f32":
        errs["dx"] = rel_l2(to_f64(p["dx"]), dx)
    else:
        # |dx_in| + sum |W| |dl| bounds the FP32 accumulation error
        mx, _, _ = oracle.rglru_gate_proj_bwd(np.abs(oracle.widen(x)), np.abs(oracle.widen(prm["w_x"])),
                                              np.abs(oracle.widen(ct["dlx"])), np.abs(oracle.widen(ct["dx"])))
        mag, _, _ = oracle.rglru_gate_proj_bwd(np.abs(oracle.widen(x)), np.abs(oracle.widen(prm["w_a"])),
                                               np.abs(oracle.widen(ct["dla"])), mx)
        _check_bf16_output("dx", p["dx"], dx, mag)
    say("   errors:", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= TOL_OUT, (k, v)


@pytest.mark.parametrize("D", [256, 512, 2048, 2560])
def test_projection_adjoint_bf16_ranges(D):
    """BF16 cotangents over several 2048-token dW ranges with a ragged last
    range and tile (B=3, L=1500: 4500 tokens), at the block widths the odd
    widths test leaves out (1, 2, 8 and 10 tiles of 16 channels; up to 8 the
    adjoint runs as one pass, dx and dW from shared tiles): dx within half a
    BF16 ulp of the exact sum plus FP32 accumulation slack, dW and db at
    1e-5 against the FP64 oracle; accumulating in place gives the same bits."""
    from linear_recurrence_sequence_amd import scan
    B, L = 3, 1500
    say(f"[gate proj] adjoint B={B} L={L} D={D} bf16 cotangents, several ranges")
    x = inputs.rglru_inputs(B, L, D, 910 + D)["x"]
    prm = inputs.rglru_proj_inputs(D, 911 + D)
    ct = inputs.proj_cotangents(B, L, D, 912 + D, bf16=True)
    d = {k: dev_tensor(v) for k, v in {"x": x, **prm, **ct}.items()}
    p = scan.rglru_gate_proj_bwd(d["x"], d["w_x"], d["w_a"], d["dlx"], d["dla"], d["dx"])
    dx2 = d["dx"].clone()
    q = scan.rglru_gate_proj_bwd(d["x"], d["w_x"], d["w_a"], d["dlx"], d["dla"], dx2, dx_out=dx2)
    torch.cuda.synchronize()
    for k in p:
        assert torch.equal(p[k], q[k]), k
    dx, dw_x, db_x = oracle.rglru_gate_proj_bwd(x, prm["w_x"], ct["dlx"], ct["dx"])
    dx, dw_a, db_a = oracle.rglru_gate_proj_bwd(x, prm["w_a"], ct["dla"], dx)
    mx, _, _ = oracle.rglru_gate_proj_bwd(np.abs(oracle.widen(x)), np.abs(oracle.widen(prm["w_x"])),
                                          np.abs(oracle.widen(ct["dlx"])), np.abs(oracle.widen(ct["dx"])))
    mag, _, _ = oracle.rglru_gate_proj_bwd(np.abs(oracle.widen(x)), np.abs(oracle.widen(prm["w_a"])),
                                           np.abs(oracle.widen(ct["dla"])), mx)
    _check_bf16_output("dx", p["dx"], dx, mag)
    errs = {"dw_x": rel_l2(to_f64(p["dw_x"]), dw_x), "db_x": rel_l2(to_f64(p["db_x"]), db_x),
            "dw_a": rel_l2(to_f64(p["dw_a"]), dw_a), "db_a": rel_l2(to_f64(p["db_a"]), db_a)}
    say("   errors:", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= TOL_OUT, (k, v)
