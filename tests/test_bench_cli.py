"""The benchmark's host side, without a GPU: its refusal of more than one GPU
and the byte counts its roofline divides by, pinned to the sizes the
metric workload's tensors have (B=1, L=32768, D=2048, K=32, groups of 8)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_default_grouping():
    assert bench.effective_groups(32768, 32, 0) == 8
    assert bench.effective_groups(32768, 16, 0, min_group=16, samu=False) == 8
    assert bench.effective_groups(100, 32, 0) == 4      # fewer chunks than a group
    assert bench.effective_groups(32768, 32, 64) == 64


def test_backward_scan_bytes_at_the_metric_shape():
    B, L, D, K, G = 1, 32768, 2048, 32, 0
    M, C = D // 2, L // K
    method, design = bench.samu_kernel_bytes(B, L, D, K, G)["samu_backward_scan"]
    stream = B * L * M * 4                    # one [B, L, M] word tensor (a BF16 complex pair per mode)
    tiles = M // 64
    # dy and b read once, db written; per (token, tile) the two partials; per
    # (chunk, mode) the entry state and the (d nu, d theta) partial; the
    # per-token controls (E, C, S) and the mode constants
    expect = 3 * stream + 12 * B * L + 8 * M + 8 * B * C * M + 8 * B * tiles * L + 8 * B * C * M
    assert method == expect == 424026112
    assert design > method


def test_forward_scan_and_floor_bytes():
    B, L, D, K, G = 1, 32768, 2048, 32, 0
    M, C = D // 2, L // K
    method, _ = bench.samu_kernel_bytes(B, L, D, K, G)["samu_forward_scan"]
    stream = B * L * M * 4
    # b read once, y written; the controls, the mode constants, z_final and
    # the entry states
    assert method == 2 * stream + 12 * B * L + 8 * M + 8 * B * M + 8 * B * C * M
    # the headline's floor: 16 bytes per (token x real channel) over the
    # whole forward + backward
    assert bench.FLOOR_SAMU * B * L * D == 16 * B * L * D
