"""The differentiable wrappers: gradients through torch.autograd equal the
direct adjoint calls (the same kernels on the same inputs), and the
input-to-output RG-LRU layer agrees with the explicit composition."""
import pytest
import torch

from linear_recurrence_sequence_amd import autograd as ag
from linear_recurrence_sequence_amd import inputs, scan
from tests.helpers import dev_tensor, rel_l2, say, to_f64

pytestmark = pytest.mark.gpu


def test_samu_scan_autograd_matches_direct_adjoint():
    B, L, D = 2, 300, 64
    say(f"[autograd] SAMU B={B} L={L} D={D}")
    inp = inputs.samu_inputs(B, L, D, 51, z0_std=0.1, dz_final_std=0.1)
    d = {k: dev_tensor(v) for k, v in inp.items()}
    leaves = {k: d[k].clone().requires_grad_(True)
              for k in ("x_sel", "b", "w_phi", "w_r", "a_phi", "a_r", "nu", "theta", "z0")}
    y, zf = ag.samu_scan(*(leaves[k] for k in ("x_sel", "b", "w_phi", "w_r", "a_phi", "a_r", "nu", "theta",
                                                "z0")), K=32, G=4)
    torch.autograd.backward([y, zf], [d["dy"], d["dz_final"]])
    y2, zf2, saved = scan.samu_scan_fwd(d["x_sel"], d["b"], d["w_phi"], d["w_r"], d["a_phi"], d["a_r"],
                                        d["nu"], d["theta"], d["z0"], K=32, G=4)
    g = scan.samu_scan_bwd(d["x_sel"], d["b"], d["w_phi"], d["w_r"], d["a_phi"], d["a_r"], d["nu"],
                           d["theta"], saved, d["dy"], d["dz_final"], K=32, G=4)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(zf, zf2)
    pairs = {"x_sel": "dx_sel", "b": "db", "w_phi": "dw_phi", "w_r": "dw_r", "a_phi": "da_phi",
             "a_r": "da_r", "nu": "dnu", "theta": "dtheta", "z0": "dz0"}
    for leaf, name in pairs.items():
        assert torch.equal(leaves[leaf].grad, g[name]), leaf


def test_rglru_layer_autograd_matches_composition_and_oracle():
    """The layer's gradients through autograd: equal bit for bit to the
    entry-point composition (scan adjoint in FP32, projection adjoint
    accumulated into that dx, one rounding to BF16), and within the BF16
    floor + 1e-4 (1e-5 for y) of the FP64 oracle fed the GPU's logits."""
    import numpy as np

    import oracle
    from tests.helpers import bf16_floor

    B, L, D = 2, 200, 512
    say(f"[autograd] RG-LRU layer B={B} L={L} D={D}")
    inp = inputs.rglru_inputs(B, L, D, 52, reset_p=0.05, h0_std=0.1, dh_final_std=0.1)
    prm = inputs.rglru_proj_inputs(D, 53)
    d = {k: dev_tensor(v) for k, v in {**inp, **prm}.items()}
    leaves = {k: d[k].clone().requires_grad_(True) for k in ("x", "w_x", "b_x", "w_a", "b_a", "alpha", "h0")}
    y, hf = ag.rglru_layer(leaves["x"], leaves["w_x"], leaves["b_x"], leaves["w_a"], leaves["b_a"],
                           leaves["alpha"], d["reset"], leaves["h0"])
    torch.autograd.backward([y, hf], [d["dy"], d["dh_final"]])
    # the same layer from the entry points
    lx, la = scan.rglru_gate_proj_fwd(d["x"], d["w_x"], d["b_x"], d["w_a"], d["b_a"])
    y2, hf2, saved = scan.rglru_scan_fwd(d["x"], lx, la, d["alpha"], d["reset"], d["h0"])
    g = scan.rglru_scan_bwd(d["x"], lx, la, d["alpha"], d["reset"], saved, d["dy"], d["dh_final"],
                            grad_dtype=torch.float32)
    p = scan.rglru_gate_proj_bwd(d["x"], d["w_x"], d["w_a"], g["dlx"], g["dla"], g["dx"])
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(hf, hf2)
    assert torch.equal(leaves["alpha"].grad, g["dalpha"]) and torch.equal(leaves["h0"].grad, g["dh0"])
    assert torch.equal(leaves["b_x"].grad, p["db_x"]) and torch.equal(leaves["b_a"].grad, p["db_a"])
    assert torch.equal(leaves["x"].grad, p["dx"].to(torch.bfloat16))
    assert torch.equal(leaves["w_x"].grad, p["dw_x"].to(torch.bfloat16))
    assert torch.equal(leaves["w_a"].grad, p["dw_a"].to(torch.bfloat16))
    # against the oracle, on the GPU's own BF16 logits (a rounding decision both sides share)
    lxg = lx.view(torch.int16).cpu().numpy().view(np.uint16)
    lag = la.view(torch.int16).cpu().numpy().view(np.uint16)
    rf = oracle.rglru_fwd(inp["x"], lxg, lag, inp["alpha"], inp["reset"], inp["h0"])
    rg = oracle.rglru_bwd(inp["x"], lxg, lag, inp["alpha"], inp["reset"], inp["h0"], inp["dy"], inp["dh_final"])
    dx, dw_x, db_x = oracle.rglru_gate_proj_bwd(inp["x"], prm["w_x"], rg["dlx"], rg["dx"])
    dx, dw_a, db_a = oracle.rglru_gate_proj_bwd(inp["x"], prm["w_a"], rg["dla"], dx)
    e = {"y": rel_l2(to_f64(y), rf["y"]), "h_final": rel_l2(to_f64(hf), rf["h_final"]),
         "x": rel_l2(to_f64(leaves["x"].grad), dx), "w_x": rel_l2(to_f64(leaves["w_x"].grad), dw_x),
         "w_a": rel_l2(to_f64(leaves["w_a"].grad), dw_a), "b_x": rel_l2(to_f64(leaves["b_x"].grad), db_x),
         "b_a": rel_l2(to_f64(leaves["b_a"].grad), db_a), "alpha": rel_l2(to_f64(leaves["alpha"].grad), rg["dalpha"]),
         "h0": rel_l2(to_f64(leaves["h0"].grad), rg["dh0"])}
    say("   errors:", {k: f"{v:.2e}" for k, v in e.items()})
    assert e["y"] <= bf16_floor(rf["y"]) + 1e-5 and e["h_final"] <= 1e-5
    for k, ref in (("x", dx), ("w_x", dw_x), ("w_a", dw_a)):
        assert e[k] <= bf16_floor(ref) + 1e-4, (k, e[k])
    for k in ("b_x", "b_a", "alpha", "h0"):
        assert e[k] <= 1e-4, (k, e[k])


def test_autograd_refuses_non_bf16_streams():
    inp = inputs.samu_inputs(1, 40, 16, 54)
    d = {k: dev_tensor(v) for k, v in inp.items()}
    with pytest.raises(ValueError, match="bfloat16"):
        ag.samu_scan(d["x_sel"].float(), d["b"], d["w_phi"], d["w_r"], d["a_phi"], d["a_r"], d["nu"],
                     d["theta"])
    with pytest.raises(ValueError, match="bfloat16"):
        ag.samu_scan(d["x_sel"], d["b"].float(), d["w_phi"], d["w_r"], d["a_phi"], d["a_r"], d["nu"],
                     d["theta"])
