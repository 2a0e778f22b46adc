"""The single-pass scans' bounded hand-off waits, forced to expire from the
host (a poll limit of 0): a workgroup that would wait for another
workgroup's words then takes NaN instead, so every output downstream of an
expired wait is NaN while the first group, which waits for nothing, is
bitwise the same as in a normal run.  Restoring the default limit restores
the normal results.  No kernel waits longer than it does normally, so
nothing here can hang.
"""
import numpy as np
import pytest
import torch

from linear_recurrence_sequence_amd import inputs
from tests.helpers import dev_tensor, say

pytestmark = pytest.mark.gpu


def _scan():
    from linear_recurrence_sequence_amd import scan
    return scan


def _split_check(normal, expired, first, name):
    """Along the token axis (dim 1): tokens in `first` (a slice) equal the
    normal run bitwise, every other token is NaN in every element."""
    n, e = normal.float().cpu(), expired.float().cpu()
    L = n.shape[1]
    keep = torch.zeros(L, dtype=torch.bool)
    keep[first] = True
    assert torch.equal(e[:, keep], n[:, keep]), f"{name}: the first group changed"
    assert torch.isfinite(n).all(), f"{name}: the normal run is not finite"
    assert torch.isnan(e[:, ~keep]).all(), f"{name}: an expired wait did not reach every later token"


def test_samu_expired_waits_are_nan():
    scan = _scan()
    # K=32, groups of 8 chunks: 256 tokens per group, 16 groups in two
    # segments of the hand-off chain; two 64-mode tiles, two batch rows
    B, L, D, K, G = 2, 4096, 256, 32, 8
    per_group = K * G
    inp = inputs.samu_inputs(B, L, D, 9101, z0_std=0.1, dz_final_std=0.1)
    d = {k: dev_tensor(v) for k, v in inp.items()}
    say(f"[handoff expiry] samu B={B} L={L} D={D} K={K} G={G}: default limit")

    def fwd():
        return scan.samu_scan_fwd(d["x_sel"], d["b"], d["w_phi"], d["w_r"], d["a_phi"], d["a_r"], d["nu"],
                                  d["theta"], d["z0"], K=K, G=G, y_dtype=torch.float32)

    def bwd(saved):
        return scan.samu_scan_bwd(d["x_sel"], d["b"], d["w_phi"], d["w_r"], d["a_phi"], d["a_r"], d["nu"],
                                  d["theta"], saved, d["dy"], d["dz_final"], K=K, G=G,
                                  grad_dtype=torch.float32)

    y0, zf0, saved0 = fwd()
    g0 = bwd(saved0)
    torch.cuda.synchronize()
    say("[handoff expiry] samu: poll limit 0")
    prev = scan.scan_set_handoff_poll_limit(0)
    try:
        y1, zf1, _ = fwd()
        g1 = bwd(saved0)  # the backward from the normal forward's saved record
        torch.cuda.synchronize()
    finally:
        scan.scan_set_handoff_poll_limit(prev)
    # forward: group 0 holds the first 256 tokens
    _split_check(y0, y1, slice(0, per_group), "samu y")
    assert torch.isnan(zf1).all()
    # backward: processing order runs from the last chunk, so group 0 holds
    # the last 256 tokens
    _split_check(g0["db"], g1["db"], slice(L - per_group, L), "samu db")
    say("[handoff expiry] samu: default limit again")
    y2, zf2, saved2 = fwd()
    g2 = bwd(saved2)
    torch.cuda.synchronize()
    assert torch.equal(y2, y0) and torch.equal(zf2, zf0)
    for k in ("db", "dx_sel", "dnu", "dtheta", "dz0"):
        assert torch.equal(g2[k], g0[k]), k


def test_rglru_expired_waits_are_nan():
    scan = _scan()
    # K=16, groups of 8 chunks: 128 tokens per group, 16 groups; three
    # 64-lane channel tiles (the last one partial), two rows
    B, L, D, K, G = 2, 2048, 320, 16, 8
    per_group = K * G
    inp = inputs.rglru_inputs(B, L, D, seed=9102, reset_p=1.0 / 128, h0_std=0.1, dh_final_std=0.1)
    d = {k: dev_tensor(v) for k, v in inp.items()}
    say(f"[handoff expiry] rglru B={B} L={L} D={D} K={K} G={G}: default limit")

    def fwd():
        return scan.rglru_scan_fwd(d["x"], d["lx"], d["la"], d["alpha"], d["reset"], d["h0"], K=K, G=G,
                                   y_dtype=torch.float32)

    def bwd(saved):
        return scan.rglru_scan_bwd(d["x"], d["lx"], d["la"], d["alpha"], d["reset"], saved, d["dy"],
                                   d["dh_final"], K=K, G=G, grad_dtype=torch.float32)

    y0, hf0, saved0 = fwd()
    g0 = bwd(saved0)
    torch.cuda.synchronize()
    say("[handoff expiry] rglru: poll limit 0")
    prev = scan.scan_set_handoff_poll_limit(0)
    try:
        y1, hf1, _ = fwd()
        g1 = bwd(saved0)
        torch.cuda.synchronize()
    finally:
        scan.scan_set_handoff_poll_limit(prev)
    _split_check(y0, y1, slice(0, per_group), "rglru y")
    assert torch.isnan(hf1).all()
    for k in ("dx", "dlx", "dla"):
        n, e = g0[k].float().cpu(), g1[k].float().cpu()
        keep = torch.zeros(L, dtype=torch.bool)
        keep[L - per_group:] = True
        assert torch.equal(e[:, keep], n[:, keep]), k
        # dl^a is exactly 0 at a segment start whatever the carry (the
        # retention there is a constant), so only the other tokens must be NaN
        later = e[:, ~keep]
        if k == "dla":
            rs = torch.from_numpy(np.asarray(inp["reset"]).astype(bool))[:, ~keep]
            later = later[~rs]
        assert torch.isnan(later).all(), k
    say("[handoff expiry] rglru: default limit again")
    y2, hf2, saved2 = fwd()
    g2 = bwd(saved2)
    torch.cuda.synchronize()
    assert torch.equal(y2, y0) and torch.equal(hf2, hf0)
    for k in ("dx", "dlx", "dla", "dalpha", "dh0"):
        assert torch.equal(g2[k], g0[k]), k
