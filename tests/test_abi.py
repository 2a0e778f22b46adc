"""The C ABI: every function include/samu_scan.h declares is exported by the
built library, size queries follow the documented layouts, and invalid
arguments return their status before anything is enqueued.

The rejection tests pass made-up device addresses.  They only ever run in a
process that sees no GPU: if a validation check regressed and let a call
through, its launch would then fail for want of a device instead of touching
those addresses.  Where a GPU is visible, the module re-runs itself in a child
process with HIP_VISIBLE_DEVICES and ROCR_VISIBLE_DEVICES empty."""
import ctypes
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "samu_scan.h")
LIB = os.path.join(ROOT, "linear_recurrence_sequence_amd", "libsamu_scan.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libsamu_scan.so not built")


def _gpu_visible():
    import torch
    return torch.cuda.device_count() > 0    # counts devices without initializing them


fake_pointers = pytest.mark.skipif(_gpu_visible(), reason="made-up device addresses run only where no GPU "
                                                          "is visible (see test_rejections_in_a_gpu_free_child)")


@pytest.mark.skipif(not _gpu_visible(), reason="the rejection tests run in this process")
def test_rejections_in_a_gpu_free_child():
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", __file__],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("extern",)))


def test_every_declared_symbol_is_exported():
    from linear_recurrence_sequence_amd import scan
    lib = scan.lib()
    names = declared_functions()
    assert len(names) >= 14, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in samu_scan.h but not exported"


def test_handoff_poll_limit_round_trip():
    # host state only: the limit the next single-pass launches take
    from linear_recurrence_sequence_amd import scan
    prev = scan.scan_set_handoff_poll_limit(7)
    try:
        assert scan.scan_set_handoff_poll_limit(0) == 7
        assert scan.scan_set_handoff_poll_limit(-5) == 0
        assert scan.scan_set_handoff_poll_limit(-1) == 16384
    finally:
        scan.scan_set_handoff_poll_limit(prev)


def test_prefix_scratch_matches_pages_table():
    from linear_recurrence_sequence_amd import scan
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_tables.json")))
    f = gold["prefix_scratch_formula"]
    for row in gold["prefix_scratch_mib"]:
        B, L, D = row["B"], row["L"], row["D"]
        G = 10**6 if row["samu_serial"] else f["samu_group_chunks"]
        s = scan.scan_prefix_scratch_bytes(B, L, D, f["samu_chunk"], G, rglru=False)
        r = scan.scan_prefix_scratch_bytes(B, L, D, f["rglru_chunk"], f["rglru_group_chunks"], rglru=True)
        assert round(s / 2**20, 3) == row["samu"]
        assert round(r / 2**20, 3) == row["rglru"]


def test_saved_and_workspace_sizes():
    from linear_recurrence_sequence_amd import scan
    B, L, D, K = 1, 32768, 2048, 32
    M, C = D // 2, L // K
    sv = scan.samu_scan_saved_bytes(B, L, D, K)
    # p, r, (u_phi, u_r), per-token (E, C, S, d) record, mode table (four
    # float4 per mode), chunk entry states, and the state entering the second
    # 16-token half of every 32-token chunk, and one (G_c, cos D_c, sin D_c)
    # record per chunk
    need = B * L * (4 + 4 + 8 + 16) + M * 64 + B * C * M * 8 + B * C * M * 8 + B * C * 16
    assert need <= sv < need + 9 * 256
    # forward workspace, grouped path (G <= 16): the single-pass forward's
    # hand-off words, two 8-byte words per (group, mode)
    G = 4
    NG = C // G
    need = B * NG * M * 16
    assert need <= scan.samu_scan_workspace_bytes(B, L, D, K, G, False) < need + 256
    # three-kernel prefix (G > 16): compressed chunk summaries (8 B per mode
    # plus a 16 B record per chunk), group summaries (16 B per mode) and group
    # entry states (8 B per mode)
    G = 32
    NG = C // G
    need = B * C * M * 8 + B * C * 16 + B * NG * M * 24
    assert need <= scan.samu_scan_workspace_bytes(B, L, D, K, G, False) < need + 4 * 256
    # backward adds the per-tile controller partials [B, M/64 tiles, L, 2]
    assert scan.samu_scan_workspace_bytes(B, L, D, K, G, True) > B * (M // 64) * L * 8
    assert scan.samu_scan_workspace_bytes(B, L, D, K, 0, False) > 0
    assert scan.samu_scan_workspace_bytes(B, L, 1001, K, 0, False) == 0      # D % 8
    assert scan.samu_scan_workspace_bytes(B, L, D, 24, 0, False) == 0        # K
    assert scan.rglru_scan_saved_bytes(4, 8192, 2560, 16) >= 4 * 512 * 2560 * 4
    assert scan.rglru_scan_workspace_bytes(1, 10, 3, 16, 0, False) == 0     # D odd
    # the widest state accepted (every chunk's rows stay inside 32-bit byte
    # ranges): 2^20 channels
    assert scan.samu_scan_workspace_bytes(1, 64, 1 << 20, K, 0, False) > 0
    assert scan.samu_scan_workspace_bytes(1, 64, (1 << 20) + 8, K, 0, False) == 0
    assert scan.rglru_scan_workspace_bytes(1, 64, 1 << 20, 16, 0, False) > 0
    assert scan.rglru_scan_workspace_bytes(1, 64, (1 << 20) + 2, 16, 0, False) == 0
    assert scan.lib().samu_scan_decode_table_bytes((1 << 20) + 8) == 0


def _fake(addr):
    return ctypes.c_void_p(addr)


def _samu_fwd_args(**over):
    a = dict(B=1, L=64, D=16, K=32, G=0, x_sel=0x100000, b=0x200000, w_phi=0x300000,
             w_r=0x300100, a_phi=0x300200, a_r=0x300210, nu=0x300300, theta=0x300400, z0=None,
             y=0x400000, y_dtype=0, z_final=None, saved=0x500000, workspace=0x600000,
             ws=1 << 20, stream=None)
    a.update(over)
    return a


def _call_samu_fwd(a):
    from linear_recurrence_sequence_amd import scan
    L = scan.lib()
    v = lambda x: None if x is None else _fake(x)
    return L.samu_scan_fwd(a["B"], a["L"], a["D"], a["K"], a["G"], v(a["x_sel"]), v(a["b"]),
                           v(a["w_phi"]), v(a["w_r"]), v(a["a_phi"]), v(a["a_r"]), v(a["nu"]),
                           v(a["theta"]), v(a["z0"]), v(a["y"]), a["y_dtype"], v(a["z_final"]),
                           v(a["saved"]), v(a["workspace"]), a["ws"], None)


@pytest.mark.parametrize("over,status", [
    (dict(D=12), -2), (dict(D=0), -2), (dict(D=(1 << 20) + 8), -2), (dict(K=8), -2), (dict(L=0), -2),
    (dict(B=0), -2),
    (dict(G=-1), -2), (dict(L=32 * 65536), -2), (dict(y_dtype=3), -2),
    (dict(x_sel=None), -1), (dict(saved=None), -1), (dict(nu=None), -1),
    (dict(b=0x200004), -3), (dict(z0=0x700008), -3),
    (dict(ws=16), -4),
    (dict(y=0x100000), -6), (dict(z_final=0x300300), -6), (dict(workspace=0x400000), -6),
])
@fake_pointers
def test_samu_fwd_rejects_before_enqueue(over, status):
    from linear_recurrence_sequence_amd import scan
    assert _call_samu_fwd(_samu_fwd_args(**over)) == status
    assert scan.lib().scan_last_error().decode()


@fake_pointers
def test_rglru_fwd_rejects_before_enqueue():
    from linear_recurrence_sequence_amd import scan
    L = scan.lib()
    f = _fake
    ok = dict(x=f(0x100000), lx=f(0x200000), la=f(0x300000), al=f(0x400000))
    # odd D
    assert L.rglru_scan_fwd(1, 8, 3, 16, 0, ok["x"], ok["lx"], ok["la"], ok["al"], None, None,
                            f(0x500000), 0, None, f(0x600000), f(0x700000), 1 << 20, None) == -2
    # missing alpha
    assert L.rglru_scan_fwd(1, 8, 4, 16, 0, ok["x"], ok["lx"], ok["la"], None, None, None,
                            f(0x500000), 0, None, f(0x600000), f(0x700000), 1 << 20, None) == -1
    # y overlaps x
    assert L.rglru_scan_fwd(1, 8, 4, 16, 0, ok["x"], ok["lx"], ok["la"], ok["al"], None, None,
                            f(0x100000), 0, None, f(0x600000), f(0x700000), 1 << 20, None) == -6
    # workspace too small
    assert L.rglru_scan_fwd(1, 8, 4, 16, 0, ok["x"], ok["lx"], ok["la"], ok["al"], None, None,
                            f(0x500000), 0, None, f(0x600000), f(0x700000), 8, None) == -4


def _call_decode(**over):
    from linear_recurrence_sequence_amd import scan
    a = dict(B=2, D=16, x_sel=0x100000, b=0x200000, w_phi=0x300000, w_r=0x300100, a_phi=0x300200,
             a_r=0x300210, nu=0x300300, theta=0x300400, table=None, z_in=0x500000, z_out=0x600000,
             y=0x700000, y_dtype=0)
    a.update(over)
    v = lambda x: None if x is None else _fake(x)
    return scan.lib().samu_scan_decode(a["B"], a["D"], v(a["x_sel"]), v(a["b"]), v(a["w_phi"]),
                                       v(a["w_r"]), v(a["a_phi"]), v(a["a_r"]), v(a["nu"]),
                                       v(a["theta"]), v(a["table"]), v(a["z_in"]), v(a["z_out"]), v(a["y"]),
                                       a["y_dtype"], None)


@pytest.mark.parametrize("over,status", [
    (dict(D=12), -2), (dict(B=0), -2), (dict(B=70000), -2), (dict(y_dtype=2), -2),
    (dict(z_out=None), -1), (dict(y=None), -1), (dict(theta=None), -1),
    (dict(b=0x200008), -3),
    (dict(y=0x100000), -6),                 # y overlaps x_sel
    (dict(z_out=0x500020), -6),             # z_out partly overlaps z_in
    (dict(z_out=0x700000), -6),             # z_out overlaps y
    (dict(table=0x800008), -3),             # misaligned table
    (dict(y=0x800000, table=0x800000), -6),  # y overlaps the table
])
@fake_pointers
def test_samu_decode_rejects_before_enqueue(over, status):
    from linear_recurrence_sequence_amd import scan
    assert _call_decode(**over) == status
    assert scan.lib().scan_last_error().decode()


@fake_pointers
def test_baseline_scans_reject_before_enqueue():
    from linear_recurrence_sequence_amd import scan
    L = scan.lib()
    f = _fake
    # sizes: the associative scan keeps its level arrays; the sequential RG-LRU scan needs none
    assert L.samu_scan_baseline_workspace_bytes(2, 1, 64, 16) == 0               # unknown variant
    assert L.samu_scan_baseline_workspace_bytes(0, 1, 64, 12) == 0               # D % 8
    assert L.samu_scan_baseline_workspace_bytes(1, 2, 64, 16) > L.samu_scan_baseline_workspace_bytes(0, 2, 64, 16)
    assert L.rglru_scan_baseline_workspace_bytes(0, 2, 64, 16) == 0
    assert L.rglru_scan_baseline_workspace_bytes(1, 2, 64, 16) == (32 + 16 + 8 + 4 + 2 + 1) * 2 * 16 * 8
    p = [f(0x100000), f(0x200000), f(0x300000), f(0x300100), f(0x300200), f(0x300210), f(0x300300),
         f(0x300400)]
    ws = L.samu_scan_baseline_workspace_bytes(1, 1, 64, 16)
    assert L.samu_scan_baseline_fwd(5, 1, 64, 16, *p, None, f(0x400000), 0, None, f(0x600000), ws, None) == -2
    assert L.samu_scan_baseline_fwd(1, 1, 64, 16, *p, None, f(0x400000), 0, None, f(0x600000), 8, None) == -4
    assert L.samu_scan_baseline_fwd(1, 1, 64, 16, *p, None, f(0x100000), 0, None, f(0x600000), ws, None) == -6
    r = [f(0x100000), f(0x200000), f(0x300000), f(0x400000)]
    assert L.rglru_scan_baseline_fwd(0, 1, 8, 3, *r, None, None, f(0x500000), 0, None, None, 0, None) == -2
    assert L.rglru_scan_baseline_fwd(1, 1, 8, 4, *r, None, None, f(0x500000), 0, None, None, 0, None) == -4
    assert L.rglru_scan_baseline_fwd(0, 1, 8, 4, *r, None, None, f(0x200000), 0, None, None, 0, None) == -6


@fake_pointers
def test_gate_projection_rejects_before_enqueue():
    from linear_recurrence_sequence_amd import scan
    L = scan.lib()
    f = _fake
    assert L.rglru_gate_proj_bwd_workspace_bytes(1, 64, 384) == 0           # D % 256
    assert L.rglru_gate_proj_bwd_workspace_bytes(1, 64, 2816) == 0          # D > 2560
    n = L.rglru_gate_proj_bwd_workspace_bytes(1, 4096, 512)
    # two range partials of [2][16][32][32] plus [2][512] floats, 256-byte aligned
    assert 2 * (2 * 16 * 32 * 32 + 2 * 512) * 4 <= n < 2 * (2 * 16 * 32 * 32 + 2 * 512) * 4 + 512
    args = [f(0x100000), f(0x300000), f(0x310000), f(0x320000), f(0x330000)]
    assert L.rglru_gate_proj_bwd_workspace_bytes(0, 64, 512) == 0            # empty batch
    assert L.rglru_gate_proj_bwd_workspace_bytes(1, 0, 512) == 0             # empty sequence
    assert L.rglru_gate_proj_fwd(1, 8, 384, *args, f(0x500000), f(0x600000), None) == -2
    assert L.rglru_gate_proj_fwd(0, 8, 256, *args, f(0x500000), f(0x600000), None) == -2
    assert L.rglru_gate_proj_fwd(1, 0, 256, *args, f(0x500000), f(0x600000), None) == -2
    assert L.rglru_gate_proj_fwd(1, 8, 256, *args, f(0x500008), f(0x600000), None) == -3   # misaligned
    assert L.rglru_gate_proj_fwd(1, 8, 256, *args, None, f(0x600000), None) == -1
    assert L.rglru_gate_proj_fwd(1, 8, 256, *args, f(0x100000), f(0x600000), None) == -6     # lx over x
    bw = [f(0x100000), f(0x300000), f(0x320000), f(0x400000), f(0x500000)]
    outs = [f(0x700000), f(0x710000), f(0x720000), f(0x730000)]
    ws = L.rglru_gate_proj_bwd_workspace_bytes(1, 8, 256)
    assert L.rglru_gate_proj_bwd(1, 8, 256, *bw, 0, f(0x600000), f(0x600000), *outs, f(0x800000), 8, None) == -4
    assert L.rglru_gate_proj_bwd(1, 8, 256, *bw, 3, f(0x600000), f(0x600000), *outs, f(0x800000), ws, None) == -2
    assert L.rglru_gate_proj_bwd(1, 8, 256, *bw, 0, f(0x600000), f(0x600010), *outs, f(0x800000), ws, None) == -6
    assert L.rglru_gate_proj_bwd(1, 8, 256, *bw, 0, f(0x600000), f(0x400000), *outs, f(0x800000), ws, None) == -6


@fake_pointers
def test_noalloc_forward_rejects_before_enqueue():
    from linear_recurrence_sequence_amd import scan
    L = scan.lib()
    f = _fake
    p = [f(0x100000), f(0x200000), f(0x300000), f(0x300100), f(0x300200), f(0x300210), f(0x300300),
         f(0x300400)]
    # a forward workspace above the 32 MiB static scratch
    assert L.samu_scan_fwd_noalloc(16, 131072, 2048, 32, 0, *p, None, f(0x400000), 0, None, f(0x500000),
                                   None) == -4
    assert b"static scratch" in L.scan_last_error()
    # an unsupported shape is named by the forward's own check
    assert L.samu_scan_fwd_noalloc(1, 64, 12, 32, 0, *p, None, f(0x400000), 0, None, f(0x500000), None) == -2


@fake_pointers
def test_decode_prepare_rejects_before_enqueue():
    from linear_recurrence_sequence_amd import scan
    L = scan.lib()
    f = _fake
    assert L.samu_scan_decode_table_bytes(12) == 0
    assert L.samu_scan_decode_table_bytes(16) == (8 * 4 + 1) * 16     # 4 float4 per mode + the norms
    p = [f(0x300000), f(0x300100), f(0x300200), f(0x300210), f(0x300300), f(0x300400)]
    assert L.samu_scan_decode_prepare(12, *p, f(0x800000), None) == -2
    assert L.samu_scan_decode_prepare(16, *p, None, None) == -1
    assert L.samu_scan_decode_prepare(16, *p, f(0x800004), None) == -3
    assert L.samu_scan_decode_prepare(16, *p, f(0x300300), None) == -6      # table over nu
