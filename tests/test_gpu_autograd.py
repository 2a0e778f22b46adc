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


def test_rglru_layer_autograd_matches_composition():
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
    g = scan.rglru_scan_bwd(d["x"], lx, la, d["alpha"], d["reset"], saved, d["dy"], d["dh_final"])
    p = scan.rglru_gate_proj_bwd(d["x"], d["w_x"], d["w_a"], g["dlx"], g["dla"], g["dx"])
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(hf, hf2)
    assert torch.equal(leaves["alpha"].grad, g["dalpha"]) and torch.equal(leaves["h0"].grad, g["dh0"])
    assert torch.equal(leaves["b_x"].grad, p["db_x"]) and torch.equal(leaves["b_a"].grad, p["db_a"])
    # weight gradients come back in the weights' BF16; dx is summed by autograd in BF16 from its two paths
    for k, ref in (("w_x", p["dw_x"]), ("w_a", p["dw_a"]), ("x", p["dx"])):
        e = rel_l2(to_f64(leaves[k].grad), to_f64(ref))
        say(f"   {k}: rel-L2 {e:.2e} against the composition")
        assert e <= 1e-2, (k, e)
