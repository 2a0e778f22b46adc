"""Benchmark: SAMU mixer forward+backward at B=1, L=32768, D=2048 on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = samu_scan_fwd + samu_scan_bwd (the whole hot path: controller,
chunk summary, grouped prefix, replay; reverse summary, reverse prefix,
backward replay, controller backward, parameter reductions) over one batch of
seeded synthetic inputs already resident in HBM.  Prints ONE JSON line on
stdout; progress goes to stderr.

value = algorithmic floor bytes of the mixer F+B (16 B per token x real
channel: x_sel, b, y forward; dy, b, x_sel, dx_sel, db backward) / F+B time,
in GB/s.  The timed steps are the K steps captured once into a HIP graph and
replayed (median of three replays, each exactly K steps between device
synchronizations; the replayed gradients are checked bit for bit against an
eager step's); ms_per_step_eager is the same K steps launched one call at a
time.  The roofline object reports the dominant kernel's algorithmic bytes
per launch over its average launch time, timed with HIP events recorded by the
library around every launch on the bench stream, over a separate eager run of
the same steps (the event records themselves cost a few microseconds per
launch, so no step time comes from that run).

Besides the headline, the line carries every other workload of the pages'
measurement plan, each F+B timed the same way with per-kernel rates:
  configs.cfg0   SAMU and RG-LRU, B=1, L=2048, D=1024
  configs.cfg2   SAMU and RG-LRU, B=1, D=1024, L = 32768, 65536, 131072
  configs.cfg3   SAMU and RG-LRU, B=1, L=32768, D = 1024, 1536, 2048, 2560
                 (initial state and its gradient)
  configs.cfg4   RG-LRU packed sequences, B=4, L=8192, D=2560, resets p=1/512
and the forward scan-latency sweep (B=8, D=1024, L = 2K..16K).
"""
import argparse
import hashlib
import json
import statistics
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
WORKLOAD = dict(B=1, L=32768, D=2048, K=32, G=0)   # G=0: library default grouping
METRIC = "mixer F+B ms and achieved HBM GB/s (% of peak) at B=1,L=32768,D=2048"
FLOOR_SAMU, FLOOR_RGLRU = 16.0, 22.0   # F+B floor bytes per (token x real channel)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def effective_groups(L, K, G, min_group=8, samu=None):
    """Chunks per group the library uses for G (0 = its choice: groups of 8
    chunks, one workgroup each, for SAMU and for RG-LRU at K=16; RG-LRU at
    K=32 serial up to 128 chunks, else about 128 groups of >= min_group
    chunks)."""
    C = -(-L // K)
    if samu is None:
        samu = min_group == 8
    if G == 0:
        if samu or K == 16:
            G = 8
        else:
            G = C if C <= 128 else max(min_group, -(-C // 128))
    return min(G, C)


def samu_kernel_bytes_unfused(B, L, D, K, G):
    """samu_kernel_bytes with the separate summary, prefix and replay passes."""
    return samu_kernel_bytes(B, L, D, K, G, unfused=True)


def samu_kernel_bytes(B, L, D, K, G, unfused=False):
    """Bytes one launch of each SAMU kernel moves at this shape, as
    (method, design):
      method  the streams the method's step itself reads and writes (the
              tensors the hot-path table lists for that step: BF16 streams,
              FP32 summaries (A, B), entry states, carries, per-tile and
              per-(chunk, mode) partials), each counted once;
      design  what this implementation's kernel reads and writes: the same
              streams in its own formats (compressed summaries: 8 B per
              (chunk, mode) plus 16 B per chunk), plus its own records (the
              per-token (E, C, S, d) record, the mode table, the mid-chunk
              states the forward replay keeps for the backward)."""
    M = D // 2
    C = -(-L // K)
    NG = -(-C // effective_groups(L, K, G))
    BL, BLD, BCM, BC = B * L, B * L * D, B * C * M, B * C
    n_tiles = -(-M // 64)
    NMID = K // 16 - 1 if K > 16 else 0
    BMID = B * C * NMID * M
    n_blk = -(-BL // 64)
    tab = {
        # x_sel, both directions -> p, r (saved) and E, C, S per token
        "samu_controller": (2 * BLD + 8 * (D + 1) + 8 * BL + 12 * BL,
                            2 * BLD + 8 * (D + 1) + 32 * BL + 64 * M),
        # b, (E, C, S), (nu, theta) -> (A, B) per (chunk, mode)
        "samu_chunk_summary": (2 * BLD + 12 * BL + 8 * M + 16 * BCM,
                               2 * BLD + 16 * BL + 32 * M + 8 * BCM + 16 * BC),
        "samu_reverse_summary": (2 * BLD + 12 * BL + 8 * M + 16 * BCM,
                                 2 * BLD + 16 * BL + 32 * M + 8 * BCM + 16 * BC),
        # the grouped prefix's three launches (compose U_g, scan over groups,
        # chunk entries); method: summaries in, entry states out
        "prefix_group_compose": (16 * BCM + 32 * B * NG * M,
                                 8 * BCM + 16 * BC + 48 * M + 16 * B * NG * M),
        "prefix_group_scan": (32 * B * NG * M + 8 * B * M,
                              16 * B * NG * M + 8 * B * M + 8 * B * NG * M),
        "prefix_chunk_entries": (16 * BCM + 8 * B * NG * M + 8 * BCM,
                                 8 * B * NG * M + 8 * BCM + 16 * BC + 48 * M + 8 * BCM),
        # entries, b -> y, z_L
        "samu_replay": (8 * BCM + 2 * BLD + 12 * BL + 8 * M + 2 * BLD + 8 * B * M,
                        2 * BLD + 16 * BL + 32 * M + 8 * BCM + 2 * BLD + 8 * B * M + 8 * BMID),
        # entries, carries, b, dy -> db, per-tile (c-bar, d-bar), per-(chunk, mode) (nu-bar, theta-bar)
        "samu_bwd_replay": (8 * BCM + 8 * BCM + 2 * BLD + 2 * BLD + 2 * BLD + 8 * B * n_tiles * L + 8 * BCM,
                            2 * BLD + 2 * BLD + 16 * BL + 32 * M + 8 * BCM + 8 * BMID + 8 * BCM + 2 * BLD
                            + 8 * B * n_tiles * L + 8 * BCM),
    }
    if effective_groups(L, K, G) <= 16 and not unfused:
        # the grouped path: one single-pass kernel per direction (chunk
        # summaries, the state or carry entering each group, replay), the
        # groups handing states on through 16 B per (group, mode)
        NGM = B * NG * M
        G_ = effective_groups(L, K, G)
        for k in ("samu_chunk_summary", "samu_replay", "samu_reverse_summary", "samu_bwd_replay",
                  "prefix_group_compose", "prefix_group_scan", "prefix_chunk_entries"):
            tab.pop(k, None)
        # what one group reads of its segment's earlier groups, on average:
        # (G - 1) / 2 published words of 16 B and one 16 B state
        handoff = 16 * NGM + (8 * (G_ - 1) + 16) * NGM
        tab.update({
            # the controller also writes one (G_c, e^{i D_c}) record per chunk
            # and clears the forward's hand-off words
            "samu_controller": (tab["samu_controller"][0], tab["samu_controller"][1] + 16 * BC + 16 * NGM),
            # b read once, y and the entry states written; the design adds the
            # token and chunk records, the mode table, the mid-chunk states
            # and the hand-off
            "samu_forward_scan": (2 * BLD + 12 * BL + 8 * M + 2 * BLD + 8 * B * M + 8 * BCM,
                                  2 * BLD + 16 * BL + 64 * M + 16 * BC + 2 * BLD + 8 * B * M + 8 * BMID
                                  + 8 * BCM + handoff),
            # dy read once (the reverse summary and the replay), b, the entry
            # states, db, the per-tile controller partials and the (d nu,
            # d theta) partials; the design reads the mid-chunk states, the
            # records and the mode table, writes one (d nu, d theta) row per
            # group, and the hand-off
            "samu_backward_scan": (2 * BLD + 2 * BLD + 2 * BLD + 12 * BL + 8 * M + 8 * BCM
                                   + 8 * B * n_tiles * L + 8 * BCM,
                                   2 * BLD + 2 * BLD + 2 * BLD + 16 * BL + 64 * M + 16 * BC + 8 * BCM
                                   + 8 * BMID + 8 * B * n_tiles * L + 8 * NGM + handoff),
            "clear": (0, 16 * NGM),
        })
    tab.update({
        # x_sel, p, r, per-tile partials -> dx_sel, per-block direction partials
        "samu_controller_bwd": (2 * BLD + 8 * BL + 8 * B * n_tiles * L + 2 * BLD + 8 * n_blk * (D + 1),
                                2 * BLD + 16 * BL + 8 * B * n_tiles * L + 2 * BLD + 8 * n_blk * (D + 4)),
        # block and chunk partials -> dw_phi, dw_r, da, dnu, dtheta
        "samu_params": (8 * n_blk * (D + 1) + 8 * BCM + 8 * (D + 1) + 8 * (D + 1) + 8 * M,
                        8 * n_blk * (D + 4) + 8 * BCM + 8 * (D + 1) + 16 + 8 * (D + 1) + 8 + 8 * M),
    })
    if effective_groups(L, K, G) <= 16 and not unfused:
        # the grouped backward writes one (d nu, d theta) row per group
        dif = 8 * BCM - 8 * B * NG * M
        tab["samu_params"] = (tab["samu_params"][0] - dif, tab["samu_params"][1] - dif)
    return tab


def rglru_kernel_bytes(B, L, D, K, G, resets, unfused=False):
    """(method, design) bytes per launch of each RG-LRU kernel (the real
    scan keeps full FP32 (A, B) summaries, so both agree but for the
    per-token reset flags)."""
    C = -(-L // K)
    NG = -(-C // effective_groups(L, K, G, 16))
    BLD, BCD = B * L * D, B * C * D
    rs = B * L if resets else 0
    tab = {
        "rglru_chunk_summary": 6 * BLD + 4 * D + rs + 8 * BCD,
        "rglru_replay": 6 * BLD + 4 * D + rs + 4 * BCD + 2 * BLD + 4 * B * D,
        "rglru_reverse_summary": 4 * BLD + 4 * D + rs + 8 * BCD,
        "rglru_bwd_replay": 8 * BLD + 4 * D + rs + 8 * BCD + 6 * BLD + 4 * BCD + 4 * B * D,
        "rglru_alpha": 4 * BCD + 4 * D,
        "prefix_group_compose": 8 * BCD + 8 * B * NG * D,
        "prefix_group_scan": 8 * B * NG * D + 4 * B * D + 4 * B * NG * D,
        "prefix_chunk_entries": 4 * B * NG * D + 8 * BCD + 4 * BCD,
    }
    tab = {k: (v, v) for k, v in tab.items()}
    G_ = effective_groups(L, K, G, 16)
    if K == 16 and G_ <= 16 and not unfused:
        # the single-pass path: x, l^x, l^a (and dy) read once per direction;
        # the design adds the hand-off (one 8 B word per (group, channel)
        # published, about (G - 1) / 2 maps and one state read per group) and
        # writes one alpha row per group
        NGD = B * NG * D
        handoff = 8 * NGD + (4 * (G_ - 1) + 8) * NGD
        for k in ("rglru_chunk_summary", "rglru_replay", "rglru_reverse_summary", "rglru_bwd_replay",
                  "prefix_group_compose", "prefix_group_scan", "prefix_chunk_entries"):
            tab.pop(k, None)
        fwd = 6 * BLD + 4 * D + rs + 2 * BLD + 4 * BCD + 4 * B * D
        bwd = 8 * BLD + 4 * D + rs + 4 * BCD + 6 * BLD + 4 * B * D
        tab.update({
            "rglru_forward_scan": (fwd, fwd + handoff),
            "rglru_backward_scan": (bwd + 4 * BCD, bwd + 4 * NGD + handoff),
            "rglru_alpha": (4 * BCD + 4 * D, 4 * NGD + 4 * D),
            "clear": (0, 8 * NGD),
        })
    return tab


def rglru_fused_step_bytes(B, L, D, K, G, resets):
    """The bytes of the method's separate steps (summary, prefix, replay)
    each RG-LRU single-pass kernel does the work of."""
    full = rglru_kernel_bytes(B, L, D, K, G, resets, unfused=True)
    return {"rglru_forward_scan": full["rglru_chunk_summary"][0] + full["prefix_group_scan"][0]
            + full["rglru_replay"][0],
            "rglru_backward_scan": full["rglru_reverse_summary"][0] + full["prefix_group_scan"][0]
            + full["rglru_bwd_replay"][0]}


def sources_digest(paths):
    """First 16 hex digits of the SHA-256 of the given repository files, in order."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_record(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE passes, scaled by a 512 MiB device
    copy), if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1)).get(kernel)
    if not rec:
        return None
    try:
        if sources_digest(rec["sources"]) != rec["sources_sha256_16"]:
            return None
    except OSError:
        return None
    return rec["bytes_per_launch"]


def copy_probe(torch, nbytes=512 << 20, reps=10):
    """Device-to-device copy of a 512 MiB buffer: achievable HBM GB/s (read +
    write bytes), the second denominator of the roofline."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    return 2 * nbytes / (ms * 1e-3) / 1e9


# ---------------------------------------------------------------- CPU leg ---
def _oracle_samu_fb(oracle, inp):
    oracle.samu_fwd(inp["x_sel"], inp["b"], inp["w_phi"], inp["w_r"], inp["a_phi"], inp["a_r"],
                    inp["nu"], inp["theta"], inp["z0"])
    z0 = inp["z0"]
    if z0 is None:
        z0 = np.zeros((inp["b"].shape[0], inp["b"].shape[2], 2), np.float32)
    oracle.samu_bwd(inp["x_sel"], inp["b"], inp["w_phi"], inp["w_r"], inp["a_phi"], inp["a_r"],
                    inp["nu"], inp["theta"], z0, inp["dy"], None)


def _oracle_rglru_fb(oracle, inp):
    oracle.rglru_fwd(inp["x"], inp["lx"], inp["la"], inp["alpha"], inp["reset"], inp["h0"])
    h0 = inp["h0"] if inp["h0"] is not None else np.zeros(inp["x"].shape[::2], np.float32)
    oracle.rglru_bwd(inp["x"], inp["lx"], inp["la"], inp["alpha"], inp["reset"], h0, inp["dy"])


def _median_time(fn, reps):
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return sorted(times)[len(times) // 2]


def cpu_baseline(sample_L, t1_sample_L, reps=3, by_config=True):
    """The FP64 oracle, as it stands, on the host cores.
      * headline: forward+backward over the first `sample_L` tokens of the
        metric workload (all of it by default), all OpenMP threads, median of
        `reps` runs;
      * t1: the same on one thread over the first `t1_sample_L` tokens;
      * by_config: one F+B of each other workload at all threads (one run
        each, the long and wide rows at a quarter of their length)."""
    import oracle
    from linear_recurrence_sequence_amd import inputs
    B, D = WORKLOAD["B"], WORKLOAD["D"]
    nthreads = oracle.max_threads()
    inp = inputs.samu_inputs(B, sample_L, D, seed=3002, z0_std=0.1)
    dt = _median_time(lambda: _oracle_samu_fb(oracle, inp), reps)
    floor = FLOOR_SAMU * B * sample_L * D
    whole = sample_L == WORKLOAD["L"]
    out = {"value": round(floor / dt / 1e9, 4), "unit": "GB/s", "cores": nthreads,
           "kind": "oracle", "ms_per_step": round(dt * 1e3, 1),
           "sample": (f"{'the whole workload' if whole else 'a prefix of the workload'}: one "
                      f"forward+backward of B={B}, L={sample_L} (of {WORKLOAD['L']}), D={D}, same "
                      f"seed and distributions; floor bytes / median wall time of {reps} runs")}
    inp1 = inputs.samu_inputs(B, t1_sample_L, D, seed=3002, z0_std=0.1)
    oracle.set_threads(1)
    try:
        dt1 = _median_time(lambda: _oracle_samu_fb(oracle, inp1), 1)
    finally:
        oracle.set_threads(nthreads)
    out["t1"] = {"cores": 1, "value": round(FLOOR_SAMU * B * t1_sample_L * D / dt1 / 1e9, 4), "unit": "GB/s",
                 "ms": round(dt1 * 1e3, 1),
                 "sample": f"one forward+backward of B={B}, L={t1_sample_L} (a prefix), D={D}, one thread"}
    if by_config:
        rows = {}
        plan = [("cfg0_samu_b1_l2048_d1024", "samu", 1, 2048, 1024, None, 0.0),
                ("cfg0_rglru_b1_l2048_d1024", "rglru", 1, 2048, 1024, None, 0.0),
                ("cfg2_samu_b1_l131072_d1024", "samu", 1, 32768, 1024, None, 0.0),
                ("cfg2_rglru_b1_l131072_d1024", "rglru", 1, 32768, 1024, None, 0.0),
                ("cfg3_samu_b1_l32768_d2560", "samu", 1, 8192, 2560, 0.1, 0.0),
                ("cfg3_rglru_b1_l32768_d2560", "rglru", 1, 8192, 2560, 0.1, 0.0),
                ("cfg4_rglru_b4_l8192_d2560", "rglru", 4, 2048, 2560, 0.1, 1.0 / 512)]
        for name, kind, Bc, Lc, Dc, std, p in plan:
            if kind == "samu":
                ci = inputs.samu_inputs(Bc, Lc, Dc, seed=5000, z0_std=std)
                t = _median_time(lambda: _oracle_samu_fb(oracle, ci), 1)
                fl = FLOOR_SAMU
            else:
                ci = inputs.rglru_inputs(Bc, Lc, Dc, seed=5001, reset_p=p, h0_std=std)
                t = _median_time(lambda: _oracle_rglru_fb(oracle, ci), 1)
                fl = FLOOR_RGLRU
            rows[name] = {"sample_L": Lc, "B": Bc, "D": Dc, "ms": round(t * 1e3, 1),
                          "token_channels_per_s": round(Bc * Lc * Dc / t, 1),
                          "floor_gbs": round(fl * Bc * Lc * Dc / t / 1e9, 4)}
            del ci
        out["by_config"] = {"cores": nthreads, "rows": rows,
                            "note": "one F+B per row at all threads; L is the sampled prefix length"}
    return out


# ------------------------------------------------------------- GPU cases ---
class Timer:
    """Steps timed between device synchronizations, without and with the
    library's per-launch events."""

    def __init__(self, torch, scan):
        self.torch, self.scan = torch, scan

    def __call__(self, step, steps, warmup, profile):
        torch, scan = self.torch, self.scan
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        scan.scan_profile_collect()
        scan.scan_profile_enable(profile)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        scan.scan_profile_enable(False)
        prof = scan.scan_profile_collect()
        return e0.elapsed_time(e1) / steps, prof

    def graph(self, step, steps, warmup, repeats=3):
        """The same `steps` steps captured once into a HIP graph, then
        replayed `repeats` times; each replay (exactly `steps` steps) is
        timed between device synchronizations.  Returns the median ms per
        step and every replay's.  No library call allocates or clears device
        memory, so the whole step captures."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(max(1, warmup)):
                step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                step()
        g.replay()  # untimed
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        runs = []
        for _ in range(repeats):
            torch.cuda.synchronize()
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            runs.append(e0.elapsed_time(e1) / steps)
        del g
        return statistics.median(runs), runs


def _dev(torch):
    def dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()
    return dev


def samu_case(torch, scan, inputs, B, L, D, K, G, seed, z0_std):
    """Device inputs, outputs and workspaces of one SAMU F+B; returns the
    step function (forward then backward, BF16 I/O) and its buffers."""
    dev = _dev(torch)
    inp = inputs.samu_inputs(B, L, D, seed=seed, z0_std=z0_std)
    d = {k: dev(v) for k, v in inp.items()}
    del inp
    M = D // 2
    cu = torch.device("cuda")
    f32 = dict(dtype=torch.float32, device=cu)
    y = torch.empty((B, L, M, 2), dtype=torch.bfloat16, device=cu)
    zf = torch.empty((B, M, 2), **f32)
    saved = torch.empty(scan.samu_scan_saved_bytes(B, L, D, K), dtype=torch.uint8, device=cu)
    ws_f = torch.empty(scan.samu_scan_workspace_bytes(B, L, D, K, G, False), dtype=torch.uint8, device=cu)
    ws_b = torch.empty(scan.samu_scan_workspace_bytes(B, L, D, K, G, True), dtype=torch.uint8, device=cu)
    out = dict(dx_sel=torch.empty((B, L, D), dtype=torch.bfloat16, device=cu),
               db=torch.empty((B, L, M, 2), dtype=torch.bfloat16, device=cu),
               dz0=torch.empty((B, M, 2), **f32) if z0_std else None, dw_phi=torch.empty(D + 1, **f32),
               dw_r=torch.empty(D + 1, **f32), da_phi=torch.empty(1, **f32),
               da_r=torch.empty(1, **f32), dnu=torch.empty(M, **f32), dtheta=torch.empty(M, **f32))

    def fwd():
        scan.samu_scan_fwd(d["x_sel"], d["b"], d["w_phi"], d["w_r"], d["a_phi"], d["a_r"], d["nu"],
                           d["theta"], d["z0"], K=K, G=G, y=y, z_final=zf, saved=saved, workspace=ws_f)

    def bwd():
        scan.samu_scan_bwd(d["x_sel"], d["b"], d["w_phi"], d["w_r"], d["a_phi"], d["a_r"], d["nu"],
                           d["theta"], saved, d["dy"], None, K=K, G=G, out=out, workspace=ws_b)

    def step():
        fwd()
        bwd()

    return step, dict(d=d, y=y, zf=zf, saved=saved, ws_f=ws_f, ws_b=ws_b, out=out, fwd=fwd, bwd=bwd)


def rglru_case(torch, scan, inputs, B, L, D, K, G, seed, h0_std, reset_p=0.0, d=None):
    """As samu_case for the RG-LRU scan; `d` reuses device inputs already made."""
    if d is None:
        dev = _dev(torch)
        inp = inputs.rglru_inputs(B, L, D, seed=seed, reset_p=reset_p, h0_std=h0_std)
        d = {k: dev(v) for k, v in inp.items()}
        del inp
    cu = torch.device("cuda")
    f32 = dict(dtype=torch.float32, device=cu)
    y = torch.empty((B, L, D), dtype=torch.bfloat16, device=cu)
    hf = torch.empty((B, D), **f32)
    saved = torch.empty(scan.rglru_scan_saved_bytes(B, L, D, K), dtype=torch.uint8, device=cu)
    wf = torch.empty(scan.rglru_scan_workspace_bytes(B, L, D, K, G, False), dtype=torch.uint8, device=cu)
    wb = torch.empty(scan.rglru_scan_workspace_bytes(B, L, D, K, G, True), dtype=torch.uint8, device=cu)
    out = dict(dx=torch.empty((B, L, D), dtype=torch.bfloat16, device=cu),
               dlx=torch.empty((B, L, D), dtype=torch.bfloat16, device=cu),
               dla=torch.empty((B, L, D), dtype=torch.bfloat16, device=cu),
               dalpha=torch.empty(D, **f32), dh0=torch.empty((B, D), **f32) if h0_std else None)

    def step():
        scan.rglru_scan_fwd(d["x"], d["lx"], d["la"], d["alpha"], d["reset"], d["h0"], K=K, G=G, y=y,
                            h_final=hf, saved=saved, workspace=wf)
        scan.rglru_scan_bwd(d["x"], d["lx"], d["la"], d["alpha"], d["reset"], saved, d["dy"], None, K=K, G=G,
                            out=out, workspace=wb)

    return step, dict(d=d, y=y, hf=hf, saved=saved, wf=wf, wb=wb, out=out)


# A single-pass kernel does the work of several of the method's steps; the
# bytes those steps move as separate passes (summary, prefix, replay) are
# reported beside its own, as what the same work costs without the fusion.
def fused_step_bytes(B, L, D, K, G):
    full = samu_kernel_bytes_unfused(B, L, D, K, G)
    return {"samu_forward_scan": full["samu_chunk_summary"][0] + full["prefix_group_scan"][0]
            + full["samu_replay"][0],
            "samu_backward_scan": full["samu_reverse_summary"][0] + full["prefix_group_scan"][0]
            + full["samu_bwd_replay"][0]}


def kernel_rates(prof, steps, table, fused=None):
    """Per-kernel us/launch and GB/s from a profiled run (prefix kernels of
    both directions share one name): gbs_design and gbs_method from the two
    byte counts, and frac, the fraction of peak on the smaller of the two
    (the conservative rate: the compressed summaries move fewer bytes than
    the method's FP32 (A, B) pairs, the replays more than its streams).  A
    single-pass kernel also gets frac_method_steps: the bytes of the
    method's separate steps it does the work of, over its time."""
    fused = fused or {}
    ks = {}
    for n, (t, c) in prof.items():
        us = t / c * 1e3
        row = {"us_per_launch": round(us, 2), "launches_per_step": c // steps}
        if n in table:
            meth, des = table[n]
            row["gbs_design"] = round(des / (us * 1e-6) / 1e9, 1)
            row["gbs_method"] = round(meth / (us * 1e-6) / 1e9, 1)
            row["frac"] = round(min(meth, des) / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        if n in fused:
            row["method_steps_bytes"] = fused[n]
            row["frac_method_steps"] = round(fused[n] / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        ks[n] = row
    return ks


# prefix launches stream only summaries (a few MB); the bar applies to the
# kernels that stream the [B, L, D] tensors
STREAM_KERNELS = ("samu_controller", "samu_chunk_summary", "samu_replay", "samu_forward_scan", "samu_reverse_summary",
                  "samu_bwd_replay", "samu_backward_scan", "samu_controller_bwd", "rglru_chunk_summary", "rglru_replay",
                  "rglru_reverse_summary", "rglru_bwd_replay", "rglru_forward_scan", "rglru_backward_scan")


def run_case(timer, kind, step, B, L, D, K, G, steps, warmup, resets=False, repeats=3):
    """F+B of one workload: the median of `repeats` replays of a HIP graph
    holding `steps` steps (ms_per_step), the median of `repeats` eager runs
    of `steps` steps (ms_per_step_eager), then one eager run with per-launch
    events for the kernel rates."""
    runs = []
    for r in range(repeats):
        t, _ = timer(step, steps, warmup if r == 0 else 1, False)
        runs.append(t)
    ms_eager = statistics.median(runs)
    ms, gruns = timer.graph(step, steps, 1, repeats)
    _, prof = timer(step, steps, 1, True)
    floor = (FLOOR_SAMU if kind == "samu" else FLOOR_RGLRU) * B * L * D
    table = samu_kernel_bytes(B, L, D, K, G) if kind == "samu" else rglru_kernel_bytes(B, L, D, K, G, resets)
    ks = kernel_rates(prof, steps, table, fused_step_bytes(B, L, D, K, G) if kind == "samu"
                      else rglru_fused_step_bytes(B, L, D, K, G, resets))
    row = {"B": B, "L": L, "D": D, "K": K,
           "G": effective_groups(L, K, G, 8 if kind == "samu" else 16),
           "ms_per_step": round(ms, 4), "ms_runs": [round(t, 4) for t in gruns],
           "ms_per_step_eager": round(ms_eager, 4), "ms_runs_eager": [round(t, 4) for t in runs],
           "token_channels_per_s": round(B * L * D / (ms * 1e-3), 1),
           "floor_gbs": round(floor / (ms * 1e-3) / 1e9, 1),
           "floor_pct_of_peak": round(100 * floor / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
           "launches_per_step": sum(c for _, c in prof.values()) / steps, "kernels": ks}
    if L >= 32768:
        low = {n: r["frac"] for n, r in ks.items() if n in STREAM_KERNELS and r["frac"] < 0.6}
        row["stream_kernels_below_60pct_of_peak"] = low
    return row


def config_sweep(torch, scan, inputs, timer, steps, warmup):
    """Every F+B workload of the pages' plan besides the headline (see the
    module docstring), SAMU and RG-LRU, each with its own seeded inputs."""
    plan = {
        "cfg0": [("samu", 1, 2048, 1024, None, 0.0), ("rglru", 1, 2048, 1024, None, 0.0)],
        "cfg2": [(k, 1, L, 1024, None, 0.0) for L in (32768, 65536, 131072) for k in ("samu", "rglru")],
        "cfg3": [(k, 1, 32768, D, 0.1, 0.0) for D in (1024, 1536, 2048, 2560) for k in ("samu", "rglru")],
        "cfg4": [("rglru", 4, 8192, 2560, 0.1, 1.0 / 512)],
    }
    seeds = {"cfg0": 0, "cfg2": 2000, "cfg3": 3000, "cfg4": 4000}
    out = {}
    for cfg, rows in plan.items():
        res = {}
        for i, (kind, B, L, D, std, p) in enumerate(rows):
            K, G = (32, 0) if kind == "samu" else (16, 0)
            log(f"[bench] {cfg} {kind} F+B B={B} L={L} D={D}")
            if kind == "samu":
                step, bufs = samu_case(torch, scan, inputs, B, L, D, K, G, seeds[cfg] + i, std)
            else:
                step, bufs = rglru_case(torch, scan, inputs, B, L, D, K, G, seeds[cfg] + i, std, p)
            r = run_case(timer, kind, step, B, L, D, K, G, steps, warmup, resets=p > 0)
            res[f"{kind}_b{B}_l{L}_d{D}"] = r
            log(f"    {r['ms_per_step']:.4f} ms/step, floor {r['floor_gbs']:.0f} GB/s"
                + (f", below 60%: {r['stream_kernels_below_60pct_of_peak']}"
                   if r.get("stream_kernels_below_60pct_of_peak") else ""))
            del step, bufs
            torch.cuda.empty_cache()
        for L_or_D in sorted({k.split("_")[2] + "_" + k.split("_")[3] for k in res}):
            s, g = res.get(f"samu_b1_{L_or_D}"), res.get(f"rglru_b1_{L_or_D}")
            if s and g:
                res[f"samu_fb_time_reduction_{L_or_D}"] = round(1 - s["ms_per_step"] / g["ms_per_step"], 4)
        out[cfg] = res
    return out


def scan_latency_sweep(torch, inputs, scan, dev, timed, B=8, D=1024, Ls=(2048, 4096, 8192, 16384)):
    """Forward scan latency at B=8, D=1024 over L (the pages' Fig. 8(a)
    shapes): the chunked scan against the per-channel sequential and the
    recursive associative comparison scans, for SAMU and RG-LRU, in ms."""
    log("[bench] scan-latency sweep (forward, B=8, D=1024)")
    Lmax = max(Ls)
    si = inputs.samu_inputs(B, Lmax, D, seed=1004, with_dy=False)
    ri = inputs.rglru_inputs(B, Lmax, D, seed=1104, with_dy=False)
    sd = {k: dev(v) for k, v in si.items()}
    rd = {k: dev(v) for k, v in ri.items()}
    M = D // 2
    out = {}
    for L in Ls:
        xs, bs = sd["x_sel"][:, :L].contiguous(), sd["b"][:, :L].contiguous()
        pr = (sd["w_phi"], sd["w_r"], sd["a_phi"], sd["a_r"], sd["nu"], sd["theta"])
        x, lx, la = (rd[k][:, :L].contiguous() for k in ("x", "lx", "la"))
        y = torch.empty((B, L, M, 2), dtype=torch.bfloat16, device="cuda")
        ry = torch.empty((B, L, D), dtype=torch.bfloat16, device="cuda")
        zf = torch.empty((B, M, 2), dtype=torch.float32, device="cuda")
        hf = torch.empty((B, D), dtype=torch.float32, device="cuda")
        saved = torch.empty(scan.samu_scan_saved_bytes(B, L, D, 32), dtype=torch.uint8, device="cuda")
        ws = torch.empty(scan.samu_scan_workspace_bytes(B, L, D, 32, 0, False), dtype=torch.uint8, device="cuda")
        rsaved = torch.empty(scan.rglru_scan_saved_bytes(B, L, D, 16), dtype=torch.uint8, device="cuda")
        rws = torch.empty(scan.rglru_scan_workspace_bytes(B, L, D, 16, 0, False), dtype=torch.uint8, device="cuda")
        row = {}
        row["samu_chunked"] = timed(lambda: scan.samu_scan_fwd(xs, bs, *pr, None, K=32, G=0, y=y, z_final=zf,
                                                                saved=saved, workspace=ws), 10, 2, False)[0]
        row["rglru_chunked"] = timed(lambda: scan.rglru_scan_fwd(x, lx, la, rd["alpha"], None, None, K=16, G=0,
                                                                 y=ry, h_final=hf, saved=rsaved, workspace=rws),
                                     10, 2, False)[0]
        for v in ("sequential", "associative"):
            sw = torch.empty(max(1, scan.lib().samu_scan_baseline_workspace_bytes(scan.BASELINES[v], B, L, D)),
                             dtype=torch.uint8, device="cuda")
            n = scan.lib().rglru_scan_baseline_workspace_bytes(scan.BASELINES[v], B, L, D)
            rw = torch.empty(n, dtype=torch.uint8, device="cuda") if n else None
            row[f"samu_{v}"] = timed(lambda: scan.samu_scan_baseline_fwd(v, xs, bs, *pr, None, y=y, z_final=zf,
                                                                          workspace=sw), 5, 1, False)[0]
            row[f"rglru_{v}"] = timed(lambda: scan.rglru_scan_baseline_fwd(v, x, lx, la, rd["alpha"], None, None,
                                                                           y=ry, h_final=hf, workspace=rw),
                                      5, 1, False)[0]
            del sw, rw
        out[f"L{L}"] = {k: round(v, 4) for k, v in row.items()}
        log(f"    L={L}: " + " ".join(f"{k}={v:.3f}" for k, v in row.items()) + " ms")
        del y, ry, saved, ws, rsaved, rws
    return {"B": B, "D": D, "unit": "ms", "direction": "forward", "by_L": out}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-sample-L", type=int, default=WORKLOAD["L"])
    ap.add_argument("--cpu-t1-sample-L", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rglru", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the scan library has no multi-GPU path "
              "(no collectives, no sequence or mode sharding); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_recurrence_sequence_amd import inputs, scan
    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    scan.lib()  # fail loudly if the HIP library is missing
    timed = Timer(torch, scan)
    dev = _dev(torch)

    B, L, D, K, G = (WORKLOAD[k] for k in ("B", "L", "D", "K", "G"))
    M = D // 2
    G_eff = effective_groups(L, K, G)
    log(f"[bench] generating inputs B={B} L={L} D={D}")
    samu_step, sb = samu_case(torch, scan, inputs, B, L, D, K, G, 3002, 0.1)
    d, out = sb["d"], sb["out"]

    log(f"[bench] SAMU F+B: warmup {args.warmup}, timing {args.steps} steps")
    ms_eager, _ = timed(samu_step, args.steps, args.warmup, False)
    log(f"[bench] SAMU F+B {ms_eager:.4f} ms/step, eager launches")
    # the same steps again with an event pair around every kernel launch
    ms_ev, prof = timed(samu_step, args.steps, 1, True)
    log(f"[bench] SAMU F+B {ms_ev:.4f} ms/step with per-kernel events")
    launches_per_step = sum(c for _, c in prof.values()) / args.steps
    for name, (tot, cnt) in sorted(prof.items(), key=lambda kv: -kv[1][0]):
        log(f"    {name:24s} {tot / cnt * 1e3:9.2f} us/launch  x{cnt // args.steps}/step")
    # the same kernels with the memory-side cache emptied before each pass (a
    # 1 GiB read ahead of the forward and of the backward): no stream one pass
    # reads is then still cached from the other pass or from the step before,
    # as in a network where other layers run between a layer's passes
    flush = torch.ones(256 << 20, dtype=torch.float32, device="cuda")

    def cold_step():
        flush.sum()
        sb["fwd"]()
        flush.sum()
        sb["bwd"]()

    _, prof_cold = timed(cold_step, args.steps, 1, True)
    del flush
    kern_us = sum(t for t, _ in prof.values()) / args.steps * 1e3
    kern_us_cold = sum(t for t, _ in prof_cold.values()) / args.steps * 1e3
    log(f"[bench] SAMU F+B kernels {kern_us:.1f} us/step, {kern_us_cold:.1f} us/step with the cache emptied "
        f"before each pass")

    ms, graph_runs, graph_equal = ms_eager, None, None
    if not args.no_graph:
        # the timed steps: the same K steps captured into one HIP graph and
        # replayed (three replays, median); the gradients left by the replays
        # must equal an eager step's bit for bit
        samu_step()
        torch.cuda.synchronize()
        db_ref = out["db"].clone()
        ms, graph_runs = timed.graph(samu_step, args.steps, args.warmup)
        graph_equal = bool(torch.equal(out["db"], db_ref))
        del db_ref
        log(f"[bench] SAMU F+B {ms:.4f} ms/step replayed from a graph of {args.steps} steps "
            f"(runs {[round(t, 4) for t in graph_runs]}; db equal to eager: {graph_equal})")

    floor_bytes = FLOOR_SAMU * B * L * D
    value = floor_bytes / (ms * 1e-3) / 1e9

    # dominant kernel and its roofline (method bytes; the design's own extra
    # records are reported beside them)
    table = samu_kernel_bytes(B, L, D, K, G)
    dom = max(prof.items(), key=lambda kv: kv[1][0])[0]
    dom_ms = prof[dom][0] / prof[dom][1]
    meth_bytes, des_bytes = table[dom]
    achieved = meth_bytes / (dom_ms * 1e-3) / 1e9
    traffic = traffic_record(dom)
    fused = fused_step_bytes(B, L, D, K, G)
    kernels = kernel_rates(prof, args.steps, table, fused)

    log("[bench] copy probe (512 MiB)")
    copy_gbs = copy_probe(torch)

    rg = None
    if not args.no_rglru:
        log("[bench] RG-LRU F+B at the same shape (comparison variant): K and G sweep")
        variants = {}
        best = None
        rd = None
        for RK in (16, 32):
            for RG in (0, 4, 8, 16, 32, 64):
                step, rb = rglru_case(torch, scan, inputs, B, L, D, RK, RG, 3003, 0.1, d=rd)
                rd = rb["d"]
                t = timed.graph(step, args.steps, args.warmup)[0]
                geff = effective_groups(L, RK, RG, 16)
                key = f"K{RK}_G{geff}"
                if key in variants:
                    del step, rb
                    continue
                variants[key] = round(t, 4)
                log(f"    K={RK} G={geff}: {t:.4f} ms/step")
                if best is None or t < best[0]:
                    best = (t, RK, RG)
                del step, rb
        rg_ms, RK, RG = best
        rg_step, rb = rglru_case(torch, scan, inputs, B, L, D, RK, RG, 3003, 0.1, d=rd)
        rd, rout = rb["d"], rb["out"]
        rg_row = run_case(timed, "rglru", rg_step, B, L, D, RK, RG, args.steps, args.warmup)
        rg_ms = rg_row["ms_per_step"]

        # the same F+B from the input: the two block-diagonal gate projections
        # (matrix cores) in front, their adjoint behind
        prm = {k: dev(v) for k, v in inputs.rglru_proj_inputs(D, 3005).items()}
        pws = torch.empty(scan.lib().rglru_gate_proj_bwd_workspace_bytes(B, L, D), dtype=torch.uint8,
                          device="cuda")

        def layer_step():
            scan.rglru_gate_proj_fwd(rd["x"], prm["w_x"], prm["b_x"], prm["w_a"], prm["b_a"], lx=rd["lx"],
                                     la=rd["la"])
            rg_step()
            scan.rglru_gate_proj_bwd(rd["x"], prm["w_x"], prm["w_a"], rout["dlx"], rout["dla"], rout["dx"],
                                     dx_out=rout["dx"], workspace=pws)

        layer_ms_eager, _ = timed(layer_step, args.steps, args.warmup, False)
        layer_ms, _ = timed.graph(layer_step, args.steps, 1)
        _, lprof = timed(layer_step, args.steps, 1, True)
        BLD = B * L * D
        pbytes = {"gate_projection": 6 * BLD, "gate_projection_dx": 8 * BLD, "gate_projection_dw": 6 * BLD,
                  "gate_projection_adjoint": 10 * BLD}
        proj = {}
        for n, (t, c) in lprof.items():
            if n.startswith("gate_projection"):
                us = t / c * 1e3
                proj[n] = {"us_per_launch": round(us, 2)}
                if n in pbytes:
                    proj[n]["gbs"] = round(pbytes[n] / (us * 1e-6) / 1e9, 1)
                    proj[n]["frac"] = round(pbytes[n] / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        rg = {"ms_per_step": rg_ms, "K": RK, "G": effective_groups(L, RK, RG, 16),
              "chosen_as": "fastest of the K x G sweep below",
              "k_g_sweep_ms": variants, "kernels": rg_row["kernels"],
              "ms_per_step_eager": rg_row["ms_per_step_eager"],
              "layer_ms_per_step": round(layer_ms, 4), "layer_ms_per_step_eager": round(layer_ms_eager, 4),
              "gate_projection": proj,
              "gbs_floor": round(FLOOR_RGLRU * B * L * D / (rg_ms * 1e-3) / 1e9, 1),
              "samu_fb_time_reduction": round((rg_ms - ms) / rg_ms, 4),
              "samu_fb_time_reduction_eager": round(1 - ms_eager / rg_row["ms_per_step_eager"], 4)}
        log(f"[bench] RG-LRU F+B {rg_ms:.4f} ms/step (K={RK}, G={rg['G']}); SAMU reduction "
            f"{(rg_ms - ms) / rg_ms:.1%}; with gate projections {layer_ms:.4f} ms/step {proj}")

        # the pages' sampling protocol: after warmups, two rounds of five
        # individually timed F+B samples per variant, the order of the
        # variants swapped between rounds; median, [min, max] and every sample
        log("[bench] paired protocol: 2 rounds x 5 samples, order swapped between rounds")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

        def one(step):
            torch.cuda.synchronize()
            e0.record()
            step()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1)

        samples = {"samu": [], "rglru": []}
        steps_by = {"samu": samu_step, "rglru": rg_step}
        for _ in range(3):
            samu_step()
            rg_step()
        for rnd in range(2):
            for name in (("samu", "rglru") if rnd == 0 else ("rglru", "samu")):
                samples[name] += [round(one(steps_by[name]), 4) for _ in range(5)]
        paired = {n: {"median_ms": round(statistics.median(v), 4), "min_ms": min(v), "max_ms": max(v),
                      "samples_ms": v} for n, v in samples.items()}
        paired["samu_time_reduction_median"] = round(
            (paired["rglru"]["median_ms"] - paired["samu"]["median_ms"]) / paired["rglru"]["median_ms"], 4)
        rg["paired_protocol"] = paired
        log(f"[bench] paired medians: SAMU {paired['samu']['median_ms']} ms, RG-LRU {paired['rglru']['median_ms']} ms")
        del rg_step, rb, prm, pws

    dec = None
    if not args.no_decode:
        log("[bench] SAMU decode step (one token, state in place) at D=%d" % D)
        dec = {}
        for Bd in (1, 16, 256):
            di = inputs.samu_inputs(Bd, 1, D, seed=3004, z0_std=0.1, with_dy=False)
            dd = {k: dev(v) for k, v in di.items()}
            xs, bs, z = dd["x_sel"][:, 0].contiguous(), dd["b"][:, 0].contiguous(), dd["z0"]
            yd = torch.empty((Bd, M, 2), dtype=torch.bfloat16, device="cuda")
            tab = scan.samu_scan_decode_prepare(d["w_phi"], d["w_r"], d["a_phi"], d["a_r"], d["nu"], d["theta"])

            def dec_step(tab=tab):
                scan.samu_scan_decode(xs, bs, d["w_phi"], d["w_r"], d["a_phi"], d["a_r"], d["nu"],
                                      d["theta"], z, y=yd, z_out=z, table=tab)

            n = 200
            dms, _ = timed(dec_step, n, 10, False)
            _, dprof = timed(dec_step, n, 1, True)
            kus = dprof["samu_decode"][0] / dprof["samu_decode"][1] * 1e3
            # the same step forming its constants itself (no prepared table)
            _, dprof0 = timed(lambda: dec_step(None), n, 10, True)
            kus0 = dprof0["samu_decode"][0] / dprof0["samu_decode"][1] * 1e3
            # the same steps replayed from a captured HIP graph (32 steps per graph)
            gs = torch.cuda.Stream()
            gs.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(gs):
                for _ in range(3):
                    dec_step()
            torch.cuda.current_stream().wait_stream(gs)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(32):
                    dec_step()
            gms, _ = timed(graph.replay, 20, 3, False)
            # x_sel, b, state in and out, y per row; both directions and the
            # constant table (64 B per mode) once
            nbytes = Bd * (2 * D + 4 * M + 16 * M + 4 * M) + 8 * (D + 1) + 64 * M + 16
            dec[f"B{Bd}"] = {"us_per_step": round(dms * 1e3, 2),
                             "us_per_step_graph": round(gms * 1e3 / 32, 2), "kernel_us": round(kus, 2),
                             "bytes_per_step": nbytes,
                             "kernel_gbs": round(nbytes / (kus * 1e-6) / 1e9, 1),
                             "kernel_us_without_table": round(kus0, 2)}
            log(f"    B={Bd}: {dms * 1e3:.2f} us/step eager, {gms * 1e3 / 32:.2f} us/step from a graph "
                f"({kus:.2f} us kernel with events, {nbytes} B)")
            del graph

    sweep = None
    if not args.no_sweep:
        sweep = scan_latency_sweep(torch, inputs, scan, dev, timed)

    configs = None
    if not args.no_configs:
        del samu_step, sb, d, out
        torch.cuda.empty_cache()
        configs = config_sweep(torch, scan, inputs, timed, 10, 5)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] CPU baseline: oracle F+B over L={args.cpu_sample_L}, one thread over "
            f"L={args.cpu_t1_sample_L}, and the other workloads")
        cpu = cpu_baseline(args.cpu_sample_L, args.cpu_t1_sample_L)
        log(f"[bench] CPU baseline {cpu}")

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; distributions of the pages' workloads)",
        "config": {"workload": "samu_mixer_fwd_bwd_b1_l32768_d2048", "B": B, "L": L, "D": D,
                   "M": M, "K": K, "G": G_eff, "io_dtype": "bf16", "state_dtype": "f32",
                   "initial_state": "N(0, 0.1^2) with gradient"},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "ms_per_step_with_kernel_events": round(ms_ev, 4),
        "kernel_us_per_step": round(kern_us, 1),
        "kernel_us_per_step_cold_passes": round(kern_us_cold, 1),
        "launches_per_step": launches_per_step,
        "token_channels_per_s": round(B * L * D / (ms * 1e-3), 1),
        "workspace_bytes": {"saved": scan.samu_scan_saved_bytes(B, L, D, K),
                            "forward": scan.samu_scan_workspace_bytes(B, L, D, K, G, False),
                            "backward": scan.samu_scan_workspace_bytes(B, L, D, K, G, True),
                            "pages_prefix_scratch_formula": scan.scan_prefix_scratch_bytes(B, L, D, K, G)},
        "timing": "HIP graph replay of the K steps" if graph_runs else "eager launches",
        "ms_per_step_runs": [round(t, 4) for t in graph_runs] if graph_runs else None,
        "ms_per_step_eager": round(ms_eager, 4), "graph_replay_equal": graph_equal,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": meth_bytes,
                     "design_bytes_per_launch": des_bytes,
                     "design_frac": round(des_bytes / (dom_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "method_steps_bytes_per_launch": fused.get(dom),
                     "method_steps_frac": (round(fused[dom] / (dom_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                                           if dom in fused else None),
                     "us_per_launch": round(dom_ms * 1e3, 2)},
        "copy_probe_gbs": round(copy_gbs, 1),
        "kernels": kernels,
        "rglru": rg,
        "configs": configs,
        "decode": dec,
        "scan_latency_sweep": sweep,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
