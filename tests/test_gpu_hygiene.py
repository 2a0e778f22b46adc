"""Memory and ordering hygiene of the C ABI on the GPU.

* Guard bytes: every output, the saved record and both workspaces are handed
  to the library as exact-size windows inside larger buffers whose padding
  holds a known byte pattern.  After a forward+backward the padding must be
  untouched, at ragged shapes (L not a multiple of K, mode or channel counts
  that leave the last workgroup and the last 64-mode tile partly empty), and
  the results must equal those of ordinary allocations bit for bit.
* Determinism under load: the same forward+backward while another stream
  keeps the device busy gives bitwise the same results as on a quiet device.
* Concurrency: single-pass scans of independent calls on several streams at
  once give bitwise the results of the same calls run one at a time.
"""
import numpy as np
import pytest
import torch

from linear_recurrence_sequence_amd import inputs, scan
from tests.helpers import dev_tensor, say

pytestmark = pytest.mark.gpu

PAD = 4096          # guard bytes on each side
FILL = 0xA5


class Guarded:
    """Exact-size tensors carved out of padded byte buffers."""

    def __init__(self):
        self.bufs = []

    def tensor(self, shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        buf = torch.full((PAD + n + PAD,), FILL, dtype=torch.uint8, device="cuda")
        self.bufs.append((buf, n))
        return buf[PAD:PAD + n].view(dtype).view(shape)

    def bytes(self, n):
        return self.tensor((int(n),), torch.uint8)

    def intact(self):
        bad = []
        for i, (buf, n) in enumerate(self.bufs):
            head, tail = buf[:PAD], buf[PAD + n:]
            if not (bool(torch.all(head == FILL)) and bool(torch.all(tail == FILL))):
                bad.append(i)
        return bad


def _samu_run(d, B, L, D, K, G, dtype, gd=None):
    """One SAMU F+B; every output in exact-size guarded windows when gd is given."""
    M = D // 2
    mk = (lambda s, t: gd.tensor(s, t)) if gd else (lambda s, t: torch.empty(s, dtype=t, device="cuda"))
    mb = (lambda n: gd.bytes(n)) if gd else (lambda n: torch.empty(int(n), dtype=torch.uint8, device="cuda"))
    f = torch.float32
    y, zf = mk((B, L, M, 2), dtype), mk((B, M, 2), f)
    saved = mb(scan.samu_scan_saved_bytes(B, L, D, K))
    wf = mb(scan.samu_scan_workspace_bytes(B, L, D, K, G, False))
    wb = mb(scan.samu_scan_workspace_bytes(B, L, D, K, G, True))
    out = dict(dx_sel=mk((B, L, D), dtype), db=mk((B, L, M, 2), dtype), dz0=mk((B, M, 2), f),
               dw_phi=mk((D + 1,), f), dw_r=mk((D + 1,), f), da_phi=mk((1,), f), da_r=mk((1,), f),
               dnu=mk((M,), f), dtheta=mk((M,), f))
    scan.samu_scan_fwd(d["x_sel"], d["b"], d["w_phi"], d["w_r"], d["a_phi"], d["a_r"], d["nu"], d["theta"],
                       d["z0"], K=K, G=G, y=y, z_final=zf, saved=saved, workspace=wf)
    scan.samu_scan_bwd(d["x_sel"], d["b"], d["w_phi"], d["w_r"], d["a_phi"], d["a_r"], d["nu"], d["theta"],
                       saved, d["dy"], d["dz_final"], K=K, G=G, out=out, workspace=wb)
    return dict(y=y, z_final=zf, **out)


def _rglru_run(d, B, L, D, K, G, dtype, gd=None):
    mk = (lambda s, t: gd.tensor(s, t)) if gd else (lambda s, t: torch.empty(s, dtype=t, device="cuda"))
    mb = (lambda n: gd.bytes(n)) if gd else (lambda n: torch.empty(int(n), dtype=torch.uint8, device="cuda"))
    f = torch.float32
    y, hf = mk((B, L, D), dtype), mk((B, D), f)
    saved = mb(scan.rglru_scan_saved_bytes(B, L, D, K))
    wf = mb(scan.rglru_scan_workspace_bytes(B, L, D, K, G, False))
    wb = mb(scan.rglru_scan_workspace_bytes(B, L, D, K, G, True))
    out = dict(dx=mk((B, L, D), dtype), dlx=mk((B, L, D), dtype), dla=mk((B, L, D), dtype),
               dalpha=mk((D,), f), dh0=mk((B, D), f))
    scan.rglru_scan_fwd(d["x"], d["lx"], d["la"], d["alpha"], d["reset"], d["h0"], K=K, G=G, y=y, h_final=hf,
                        saved=saved, workspace=wf)
    scan.rglru_scan_bwd(d["x"], d["lx"], d["la"], d["alpha"], d["reset"], saved, d["dy"], d["dh_final"], K=K,
                        G=G, out=out, workspace=wb)
    return dict(y=y, h_final=hf, **out)


def _equal(a, b):
    for k in a:
        assert torch.equal(a[k], b[k]), k


# (B, L, D, K, G): L % K != 0; M = 260 modes leave the last 256-mode
# workgroup and the last 64-mode tile partly empty; serial and grouped prefix
SAMU_SHAPES = [(2, 1000, 520, 32, 3), (1, 777, 40, 16, 0), (2, 45, 1032, 32, 1000)]
RGLRU_SHAPES = [(3, 333, 1030, 16, 4), (1, 1001, 70, 32, 0)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", SAMU_SHAPES, ids=[f"B{s[0]}_L{s[1]}_D{s[2]}_K{s[3]}" for s in SAMU_SHAPES])
def test_samu_guard_bytes(shape, dtype):
    B, L, D, K, G = shape
    inp = inputs.samu_inputs(B, L, D, 6100 + L, z0_std=0.1, dz_final_std=0.1)
    d = {k: dev_tensor(v) for k, v in inp.items()}
    say(f"[hygiene] SAMU guard bytes B={B} L={L} D={D} K={K} G={G} {dtype}")
    gd = Guarded()
    got = _samu_run(d, B, L, D, K, G, dtype, gd)
    ref = _samu_run(d, B, L, D, K, G, dtype)
    torch.cuda.synchronize()
    assert gd.intact() == []
    _equal(got, ref)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", RGLRU_SHAPES, ids=[f"B{s[0]}_L{s[1]}_D{s[2]}_K{s[3]}" for s in RGLRU_SHAPES])
def test_rglru_guard_bytes(shape, dtype):
    B, L, D, K, G = shape
    inp = inputs.rglru_inputs(B, L, D, 6200 + L, reset_p=1.0 / 64, h0_std=0.1, dh_final_std=0.1)
    d = {k: dev_tensor(v) for k, v in inp.items()}
    say(f"[hygiene] RG-LRU guard bytes B={B} L={L} D={D} K={K} G={G} {dtype}")
    gd = Guarded()
    got = _rglru_run(d, B, L, D, K, G, dtype, gd)
    ref = _rglru_run(d, B, L, D, K, G, dtype)
    torch.cuda.synchronize()
    assert gd.intact() == []
    _equal(got, ref)


def test_deterministic_with_another_stream_busy():
    """The same SAMU and RG-LRU F+B, first on a quiet device, then while a
    second stream runs device copies of 256 MiB the whole time: bitwise
    equal (no reduction order depends on timing)."""
    B, L, D = 1, 8192, 1024
    si = inputs.samu_inputs(B, L, D, 6300, z0_std=0.1)
    ri = inputs.rglru_inputs(B, L, D, 6301, reset_p=1.0 / 512, h0_std=0.1)
    sd = {k: dev_tensor(v) for k, v in si.items()}
    rd = {k: dev_tensor(v) for k, v in ri.items()}
    say(f"[hygiene] determinism with a busy stream B={B} L={L} D={D}: quiet run")
    quiet_s = _samu_run(sd, B, L, D, 32, 0, torch.bfloat16)
    quiet_r = _rglru_run(rd, B, L, D, 16, 0, torch.bfloat16)
    torch.cuda.synchronize()
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    side = torch.cuda.Stream()
    say("[hygiene] determinism: runs while the side stream copies")
    for _ in range(3):
        with torch.cuda.stream(side):
            for _ in range(40):
                dst.copy_(src)
        busy_s = _samu_run(sd, B, L, D, 32, 0, torch.bfloat16)
        busy_r = _rglru_run(rd, B, L, D, 16, 0, torch.bfloat16)
        torch.cuda.synchronize()
        _equal(busy_s, quiet_s)
        _equal(busy_r, quiet_r)


def test_single_pass_scans_concurrent_on_three_streams():
    """Two SAMU and one RG-LRU forward+backward, each with its own outputs
    and workspaces, enqueued on three streams at once, so the workgroups of
    their single-pass launches share the device: bitwise equal to the same
    calls run one at a time.  A workgroup of these launches waits only for
    earlier workgroups of its own launch, which were dispatched before it,
    so sharing the device delays the waits but cannot stall them."""
    B, L, D = 2, 16384, 1024
    s1 = {k: dev_tensor(v) for k, v in inputs.samu_inputs(B, L, D, 6400, z0_std=0.1, dz_final_std=0.1).items()}
    s2 = {k: dev_tensor(v) for k, v in inputs.samu_inputs(B, L, D, 6401, z0_std=0.1).items()}
    rr = {k: dev_tensor(v) for k, v in inputs.rglru_inputs(B, L, D, 6402, reset_p=1.0 / 512, h0_std=0.1,
                                                          dh_final_std=0.1).items()}
    say(f"[hygiene] concurrent streams B={B} L={L} D={D}: one at a time")
    ref1 = _samu_run(s1, B, L, D, 32, 0, torch.bfloat16)
    ref2 = _samu_run(s2, B, L, D, 32, 0, torch.bfloat16)
    refr = _rglru_run(rr, B, L, D, 16, 0, torch.bfloat16)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    for rep in range(3):
        say(f"[hygiene] concurrent streams: round {rep}")
        with torch.cuda.stream(streams[0]):
            got1 = _samu_run(s1, B, L, D, 32, 0, torch.bfloat16)
        with torch.cuda.stream(streams[1]):
            got2 = _samu_run(s2, B, L, D, 32, 0, torch.bfloat16)
        with torch.cuda.stream(streams[2]):
            gotr = _rglru_run(rr, B, L, D, 16, 0, torch.bfloat16)
        torch.cuda.synchronize()
        _equal(got1, ref1)
        _equal(got2, ref2)
        _equal(gotr, refr)
