"""Benchmark: SAMU mixer forward+backward at B=1, L=32768, D=2048 on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = samu_scan_fwd + samu_scan_bwd (the whole hot path: controller,
chunk summary, grouped prefix, replay; reverse summary, reverse prefix,
backward replay, controller backward, parameter reductions) over one batch of
seeded synthetic inputs already resident in HBM.  Prints ONE JSON line on
stdout; progress goes to stderr.

value = algorithmic floor bytes of the mixer F+B (16 B per token x real
channel: x_sel, b, y forward; dy, b, x_sel, dx_sel, db backward) / F+B time,
in GB/s.  The roofline object reports the dominant kernel's algorithmic bytes
per launch over its average launch time, timed with HIP events recorded by the
library around every launch on the bench stream, over a second run of the
same timed steps (the event records themselves cost a few microseconds per
launch, so ms_per_step comes from the first run, without them).
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def effective_groups(L, K, G, min_group=8):
    """Chunks per group the library uses for G (0 = its choice by shape:
    serial up to 128 chunks, else about 128 groups of >= min_group chunks)."""
    C = -(-L // K)
    if G == 0:
        G = C if C <= 128 else max(min_group, -(-C // 128))
    return min(G, C)


def kernel_bytes(name, B, L, D, K, G):
    """Algorithmic bytes one launch of `name` must move at this shape: the
    streams its job reads and writes, each counted once."""
    M = D // 2
    C = -(-L // K)
    NG = -(-C // effective_groups(L, K, G))
    BL, BLD, BCM = B * L, B * L * D, B * C * M
    n_tiles = -(-M // 64)
    BC = B * C
    NMID = K // 16 - 1 if K > 16 else 0  # states entering the later 16-token halves of a chunk
    BMID = B * C * NMID * M
    table = {
        # x_sel, both direction vectors -> p, r, (u_phi, u_r), (E, C, S, d), mode table
        "samu_controller": 2 * BLD + 8 * (D + 1) + 32 * BL + 64 * M,
        # b, (E, C, S, d), mode table -> B part per (chunk, mode), (G_c, e^{i D_c}) per chunk
        "samu_chunk_summary": 2 * BLD + 16 * BL + 32 * M + 8 * BCM + 16 * BC,
        "samu_reverse_summary": 2 * BLD + 16 * BL + 32 * M + 8 * BCM + 16 * BC,
        # compressed chunk summaries, mode constants -> group summaries
        "prefix_group_compose": 8 * BCM + 16 * BC + 48 * M + 16 * B * NG * M,
        # group summaries, initial state -> state entering every group
        "prefix_group_scan": 16 * B * NG * M + 8 * B * M + 8 * B * NG * M,
        # group entry states, compressed chunk summaries -> state entering every chunk
        "prefix_chunk_entries": 8 * B * NG * M + 8 * BCM + 16 * BC + 48 * M + 8 * BCM,
        # b, (E, C, S, d), entry states -> y, final state, mid-chunk states
        "samu_replay": 2 * BLD + 16 * BL + 32 * M + 8 * BCM + 2 * BLD + 8 * B * M + 8 * BMID,
        # dy, b, (E, C, S, d), entry and mid-chunk states, adjoint carries -> db,
        # per-tile controller partials, per-(chunk, mode) spectrum partials
        "samu_bwd_replay": 2 * BLD + 2 * BLD + 16 * BL + 32 * M + 8 * BCM + 8 * BMID + 8 * BCM + 2 * BLD
        + 8 * B * n_tiles * L + 8 * BCM,
        # x_sel, p, r, u, per-tile partials -> dx_sel, per-block direction partials
        "samu_controller_bwd": 2 * BLD + 16 * BL + 8 * B * n_tiles * L + 2 * BLD
        + 8 * (-(-BL // 64)) * (D + 4),
        # per-block direction partials, per-(chunk, mode) spectrum partials, both
        # directions and their squared norms -> dw_phi, dw_r, da, dnu, dtheta
        "samu_params": 8 * (-(-BL // 64)) * (D + 4) + 8 * BCM + 8 * (D + 1) + 16 + 8 * (D + 1) + 8 + 8 * M,
    }
    return table.get(name)


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


def cpu_baseline(sample_L, reps=3):
    """The FP64 oracle, as it stands, on the host cores: forward+backward over
    the first `sample_L` tokens of the same workload (all of it by default),
    median wall time of `reps` runs."""
    import oracle
    from linear_recurrence_sequence_amd import inputs
    B, D = WORKLOAD["B"], WORKLOAD["D"]
    inp = inputs.samu_inputs(B, sample_L, D, seed=3002, z0_std=0.1)
    z0 = inp["z0"]
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.samu_fwd(inp["x_sel"], inp["b"], inp["w_phi"], inp["w_r"], inp["a_phi"], inp["a_r"],
                        inp["nu"], inp["theta"], z0)
        oracle.samu_bwd(inp["x_sel"], inp["b"], inp["w_phi"], inp["w_r"], inp["a_phi"], inp["a_r"],
                        inp["nu"], inp["theta"], z0, inp["dy"], None)
        times.append(time.perf_counter() - t0)
    dt = sorted(times)[len(times) // 2]
    floor = 16.0 * B * sample_L * D
    whole = sample_L == WORKLOAD["L"]
    return {"value": round(floor / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.max_threads(),
            "kind": "oracle", "ms_per_step": round(dt * 1e3, 1),
            "sample": (f"{'the whole workload' if whole else 'a prefix of the workload'}: one "
                       f"forward+backward of B={B}, L={sample_L} (of {WORKLOAD['L']}), D={D}, same "
                       f"seed and distributions; floor bytes / median wall time of {reps} runs")}


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
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rglru", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
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

    B, L, D, K, G = (WORKLOAD[k] for k in ("B", "L", "D", "K", "G"))
    M = D // 2
    G_eff = effective_groups(L, K, G)
    log(f"[bench] generating inputs B={B} L={L} D={D}")
    inp = inputs.samu_inputs(B, L, D, seed=3002, z0_std=0.1)

    def dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    d = {k: dev(v) for k, v in inp.items()}
    dev_ = torch.device("cuda")
    f32 = dict(dtype=torch.float32, device=dev_)
    y = torch.empty((B, L, M, 2), dtype=torch.bfloat16, device=dev_)
    zf = torch.empty((B, M, 2), **f32)
    saved = torch.empty(scan.samu_scan_saved_bytes(B, L, D, K), dtype=torch.uint8, device=dev_)
    ws_f = torch.empty(scan.samu_scan_workspace_bytes(B, L, D, K, G, False), dtype=torch.uint8, device=dev_)
    ws_b = torch.empty(scan.samu_scan_workspace_bytes(B, L, D, K, G, True), dtype=torch.uint8, device=dev_)
    out = dict(dx_sel=torch.empty((B, L, D), dtype=torch.bfloat16, device=dev_),
               db=torch.empty((B, L, M, 2), dtype=torch.bfloat16, device=dev_),
               dz0=torch.empty((B, M, 2), **f32), dw_phi=torch.empty(D + 1, **f32),
               dw_r=torch.empty(D + 1, **f32), da_phi=torch.empty(1, **f32),
               da_r=torch.empty(1, **f32), dnu=torch.empty(M, **f32), dtheta=torch.empty(M, **f32))

    def samu_step():
        scan.samu_scan_fwd(d["x_sel"], d["b"], d["w_phi"], d["w_r"], d["a_phi"], d["a_r"], d["nu"],
                           d["theta"], d["z0"], K=K, G=G, y=y, z_final=zf, saved=saved, workspace=ws_f)
        scan.samu_scan_bwd(d["x_sel"], d["b"], d["w_phi"], d["w_r"], d["a_phi"], d["a_r"], d["nu"],
                           d["theta"], saved, d["dy"], None, K=K, G=G, out=out, workspace=ws_b)

    def timed(step, steps, warmup, profile):
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

    log(f"[bench] SAMU F+B: warmup {args.warmup}, timing {args.steps} steps")
    ms, _ = timed(samu_step, args.steps, args.warmup, False)
    log(f"[bench] SAMU F+B {ms:.4f} ms/step")
    # the same steps again with an event pair around every kernel launch
    ms_ev, prof = timed(samu_step, args.steps, 1, True)
    log(f"[bench] SAMU F+B {ms_ev:.4f} ms/step with per-kernel events")
    launches_per_step = sum(c for _, c in prof.values()) / args.steps
    for name, (tot, cnt) in sorted(prof.items(), key=lambda kv: -kv[1][0]):
        log(f"    {name:24s} {tot / cnt * 1e3:9.2f} us/launch  x{cnt // args.steps}/step")

    # the same step replayed from a captured HIP graph (8 steps per graph; no
    # library call allocates or clears memory, so the whole pass captures);
    # the replayed gradients must equal an eager step's bit for bit
    log("[bench] SAMU F+B replayed from a HIP graph")
    samu_step()
    torch.cuda.synchronize()
    db_ref = out["db"].clone()
    gs = torch.cuda.Stream()
    gs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(gs):
        for _ in range(2):
            samu_step()
    torch.cuda.current_stream().wait_stream(gs)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(8):
            samu_step()
    gms, _ = timed(graph.replay, max(2, args.steps // 8), 1, False)
    ms_graph = gms / 8
    graph_equal = bool(torch.equal(out["db"], db_ref))
    del graph
    log(f"[bench] SAMU F+B {ms_graph:.4f} ms/step from a graph (replayed db equal to eager: {graph_equal})")

    floor_bytes = 16.0 * B * L * D
    value = floor_bytes / (ms * 1e-3) / 1e9

    # dominant kernel and its roofline
    dom = max(prof.items(), key=lambda kv: kv[1][0])[0]
    dom_ms = prof[dom][0] / prof[dom][1]
    dom_bytes = kernel_bytes(dom, B, L, D, K, G)
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic = traffic_record(dom)
    kernels = {n: {"us_per_launch": round(t / c * 1e3, 2),
                   "launches_per_step": c // args.steps,
                   "gbs": (round(kernel_bytes(n, B, L, D, K, G) / (t / c * 1e-3) / 1e9, 1)
                           if kernel_bytes(n, B, L, D, K, G) else None)}
               for n, (t, c) in prof.items()}

    log("[bench] copy probe (512 MiB)")
    copy_gbs = copy_probe(torch)

    rg = None
    if not args.no_rglru:
        log("[bench] RG-LRU F+B at the same shape (comparison variant)")
        ri = inputs.rglru_inputs(B, L, D, seed=3003, h0_std=0.1)
        rd = {k: dev(v) for k, v in ri.items()}
        RK, RG = 16, 0
        ry = torch.empty((B, L, D), dtype=torch.bfloat16, device=dev_)
        rhf = torch.empty((B, D), **f32)
        rsv = torch.empty(scan.rglru_scan_saved_bytes(B, L, D, RK), dtype=torch.uint8, device=dev_)
        rwf = torch.empty(scan.rglru_scan_workspace_bytes(B, L, D, RK, RG, False), dtype=torch.uint8, device=dev_)
        rwb = torch.empty(scan.rglru_scan_workspace_bytes(B, L, D, RK, RG, True), dtype=torch.uint8, device=dev_)
        rout = dict(dx=torch.empty((B, L, D), dtype=torch.bfloat16, device=dev_),
                    dlx=torch.empty((B, L, D), dtype=torch.bfloat16, device=dev_),
                    dla=torch.empty((B, L, D), dtype=torch.bfloat16, device=dev_),
                    dalpha=torch.empty(D, **f32), dh0=torch.empty((B, D), **f32))

        def rg_step():
            scan.rglru_scan_fwd(rd["x"], rd["lx"], rd["la"], rd["alpha"], None, rd["h0"], K=RK, G=RG,
                                y=ry, h_final=rhf, saved=rsv, workspace=rwf)
            scan.rglru_scan_bwd(rd["x"], rd["lx"], rd["la"], rd["alpha"], None, rsv, rd["dy"], None,
                                K=RK, G=RG, out=rout, workspace=rwb)

        rg_ms, rg_prof = timed(rg_step, args.steps, args.warmup, False)

        # the same F+B from the input: the two block-diagonal gate projections
        # (matrix cores) in front, their adjoint behind
        prm = {k: dev(v) for k, v in inputs.rglru_proj_inputs(D, 3005).items()}
        pws = torch.empty(scan.lib().rglru_gate_proj_bwd_workspace_bytes(B, L, D), dtype=torch.uint8, device=dev_)

        def layer_step():
            scan.rglru_gate_proj_fwd(rd["x"], prm["w_x"], prm["b_x"], prm["w_a"], prm["b_a"], lx=rd["lx"],
                                     la=rd["la"])
            rg_step()
            scan.rglru_gate_proj_bwd(rd["x"], prm["w_x"], prm["w_a"], rout["dlx"], rout["dla"], rout["dx"],
                                     dx_out=rout["dx"], workspace=pws)

        layer_ms, _ = timed(layer_step, args.steps, args.warmup, False)
        _, lprof = timed(layer_step, args.steps, 1, True)
        proj = {n: round(t / c * 1e3, 2) for n, (t, c) in lprof.items() if n.startswith("gate_projection")}
        rg = {"ms_per_step": round(rg_ms, 4), "K": RK, "G": effective_groups(L, RK, RG, 16),
              "layer_ms_per_step": round(layer_ms, 4), "gate_projection_us": proj,
              "gbs_floor": round(22.0 * B * L * D / (rg_ms * 1e-3) / 1e9, 1),
              "samu_fb_time_reduction": round((rg_ms - ms) / rg_ms, 4)}
        log(f"[bench] RG-LRU F+B {rg_ms:.4f} ms/step; SAMU reduction {(rg_ms - ms) / rg_ms:.1%}; "
            f"with gate projections {layer_ms:.4f} ms/step {proj}")

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

    dec = None
    if not args.no_decode:
        log("[bench] SAMU decode step (one token, state in place) at D=%d" % D)
        dec = {}
        for Bd in (1, 16, 256):
            di = inputs.samu_inputs(Bd, 1, D, seed=3004, z0_std=0.1, with_dy=False)
            dd = {k: dev(v) for k, v in di.items()}
            xs, bs, z = dd["x_sel"][:, 0].contiguous(), dd["b"][:, 0].contiguous(), dd["z0"]
            yd = torch.empty((Bd, M, 2), dtype=torch.bfloat16, device=dev_)

            def dec_step():
                scan.samu_scan_decode(xs, bs, d["w_phi"], d["w_r"], d["a_phi"], d["a_r"], d["nu"],
                                      d["theta"], z, y=yd, z_out=z)

            n = 200
            dms, _ = timed(dec_step, n, 10, False)
            _, dprof = timed(dec_step, n, 1, True)
            kus = dprof["samu_decode"][0] / dprof["samu_decode"][1] * 1e3
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
            # x_sel, b, state in and out, y, both directions, nu and theta
            nbytes = Bd * (2 * D + 4 * M + 16 * M + 4 * M) + 8 * (D + 1) + 8 * M
            dec[f"B{Bd}"] = {"us_per_step": round(dms * 1e3, 2),
                             "us_per_step_graph": round(gms * 1e3 / 32, 2), "kernel_us": round(kus, 2),
                             "bytes_per_step": nbytes,
                             "kernel_gbs": round(nbytes / (kus * 1e-6) / 1e9, 1)}
            log(f"    B={Bd}: {dms * 1e3:.2f} us/step eager, {gms * 1e3 / 32:.2f} us/step from a graph "
                f"({kus:.2f} us kernel with events, {nbytes} B)")

    sweep = None
    if not args.no_sweep:
        sweep = scan_latency_sweep(torch, inputs, scan, dev, timed)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] CPU baseline: oracle F+B over L={args.cpu_sample_L}")
        cpu = cpu_baseline(args.cpu_sample_L)
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
                   "M": M, "K": K, "G": G_eff, "io": "bf16", "state": "f32",
                   "initial_state": "N(0, 0.1^2) with gradient"},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "ms_per_step_with_kernel_events": round(ms_ev, 4),
        "launches_per_step": launches_per_step,
        "token_channels_per_s": round(B * L * D / (ms * 1e-3), 1),
        "workspace_bytes": {"saved": scan.samu_scan_saved_bytes(B, L, D, K),
                            "forward": scan.samu_scan_workspace_bytes(B, L, D, K, G, False),
                            "backward": scan.samu_scan_workspace_bytes(B, L, D, K, G, True),
                            "pages_prefix_scratch_formula": scan.scan_prefix_scratch_bytes(B, L, D, K, G)},
        "ms_per_step_graph": round(ms_graph, 4), "graph_replay_equal": graph_equal,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": dom_bytes,
                     "us_per_launch": round(dom_ms * 1e3, 2)},
        "copy_probe_gbs": round(copy_gbs, 1),
        "kernels": kernels,
        "rglru": rg,
        "decode": dec,
        "scan_latency_sweep": sweep,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
