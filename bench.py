#!/usr/bin/env python3
"""Decode-step benchmark of index-selected sparse attention on one MI355X.

One step = the whole Decode hot path for a batch: indexer scores over every cached token,
Top-K selection and sparse attention over the selected rows (sa_decode_step). Inputs are
seeded synthetic tensors already resident in HBM; R replicas of the caches are rotated so that
no step finds its inputs in the 256 MB last-level cache left warm by the previous step.

Prints one JSON line (rank 0) with the throughput, the roofline of the dominant kernel, and the
CPU oracle's throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode tokens/s (indexer+TopK+sparse attn), B=32 ctx=32K; % HBM peak"
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the kernel sources with comments and blank space removed (code changes only)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "indexer_top_sparse_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f)) as fh:
            code = re.sub(r"//[^\n]*", "", fh.read())
        h.update(f.encode() + " ".join(code.split()).encode())
    return h.hexdigest()[:16]


def host_info():
    """CPU model of the host (the oracle baseline runs there)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "logical_cpus": os.cpu_count()}


def step_distribution(step, n, stream, rotate):
    """Per-step durations (us) of n back-to-back steps, each bracketed by its own pair of events
    on the launch stream: median, p10 and p90. rotate=False runs every step on replica 0
    (inputs possibly still in the last-level cache: "warm"), rotate=True rotates the replicas
    as the headline loop does ("cold")."""
    import numpy as np
    import torch

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(n):
        step(i if rotate else 0)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    t = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(n)]) * 1e3
    return {"steps": n, "median_us": float(np.median(t)), "p10_us": float(np.percentile(t, 10)),
            "p90_us": float(np.percentile(t, 90)), "min_us": float(t.min()),
            "max_us": float(t.max())}


def algorithmic_bytes(wl):
    """Bytes each kernel must move at least once (inputs read once, outputs written once)."""
    P, K = wl.page_size, wl.topk
    key_row = {"bf16": 2 * wl.idx_dim, "fp8": wl.idx_dim + 4,            # codes + fp32 row scale
               "mxfp8": wl.idx_dim + wl.idx_dim // 32}[wl.idx_dtype]    # codes + E8M0 per 32
    kv_row = {"bf16": 2 * wl.k_row, "fp8": wl.k_row + 4,                     # codes + row scale
              "fp8t128": wl.k_row + 4 * -(-wl.k_row // 128)}[wl.kv_dtype]   # + tile scales
    sel = attn = 0
    for n in wl.ctx_lens:
        npg = math.ceil(n / P)
        k_eff = min(K, n)
        if wl.block_topk:
            # two-level: one pooled summary row per block, then the keys of the kept blocks
            keys = npg * wl.idx_dim * 2 + min(n, min(wl.block_topk, npg) * P) * key_row
        else:
            keys = n * key_row
        sel += (keys + wl.idx_heads * wl.idx_dim * 2 + wl.idx_heads * 4 + npg * 4 + 4 + K * 4)
        attn += (k_eff * kv_row + wl.heads_q * wl.dim_qk * 2 + wl.heads_q * wl.dim_v * 2
                 + K * 4 + npg * 4)
    # the fused step: everything above except the index set, which never has to leave the op
    step = sel + attn - 2 * 4 * K * wl.num_seqs
    return {"select": sel, "attention": attn, "step": step}


# kernels of each launch the bench times (a launch may consist of several kernels; the latent
# attention kernel merges inside the launch, the other one is followed by k_attn_merge). Decode
# times select and attention, prefill index_score, topk and sparse_attn.
_ATTN_KERNELS = ("k_attn_latent", "k_sparse_attn", "k_attn_merge")
LAUNCH_KERNELS = {"select": ("k_decode_select",), "attention": _ATTN_KERNELS,
                  "index_score": ("k_prefill_score", "k_index_score"),
                  "topk": ("k_topk_rows",), "sparse_attn": _ATTN_KERNELS}


def write_traffic(workload, csvs, copy_gib):
    """HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE counters (KiB per dispatch).

    Each counter is scaled by the ratio between the bytes a plain device copy of known size moves
    and what the same counter reads for that copy (the largest __amd_rocclr_copyBuffer dispatch,
    made by --copy-calibration-gib)."""
    import csv
    assert copy_gib > 0, "--copy-calibration-gib must name the calibration copy size"
    known = copy_gib * 2**30
    res = {"workload": workload, "source_hash": kernel_source_hash(), "calibration": {},
           "kernels": {}}
    per = {}
    for counter, path in zip(("FETCH_SIZE", "WRITE_SIZE"), csvs):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        copies = [float(r["Counter_Value"]) for r in rows
                  if "copyBuffer" in r["Kernel_Name"]]
        factor = known / (max(copies) * 1024.0)
        res["calibration"][counter] = {"copy_bytes": known, "counter_kib": max(copies),
                                       "factor": factor}
        for launch, names in LAUNCH_KERNELS.items():
            tot, seen = 0.0, False
            for n in names:  # the kernels of this launch that the run dispatched
                vals = [float(r["Counter_Value"]) for r in rows if n in r["Kernel_Name"]]
                if vals:
                    tot += sum(vals) / len(vals) * 1024.0 * factor
                    seen = True
            if seen:
                per.setdefault(launch, {})[counter] = tot
    for launch, d in per.items():
        if len(d) == 2:
            res["kernels"][launch] = {"fetch_bytes": d["FETCH_SIZE"],
                                      "write_bytes": d["WRITE_SIZE"],
                                      "hbm_bytes_per_launch": d["FETCH_SIZE"] + d["WRITE_SIZE"]}
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, f"traffic_{workload}.json")
    with open(out, "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res, indent=1))


MFMA_BF16_PEAK_TFLOPS = 2500.0


def prefill_flops(wl):
    """Indexer and attention flops of a prefill batch (causal: row i sees positions 0..p_i)."""
    pos = wl.q_pos()
    vis = int((pos + 1).sum())
    idx = 2 * wl.idx_heads * wl.idx_dim * vis
    k_eff = int(sum(min(wl.topk, int(p) + 1) for p in pos))
    attn = 2 * wl.heads_q * (wl.dim_qk + wl.dim_v) * k_eff
    return idx, attn


def run_prefill(args):
    """Prefill: sa_index_score -> sa_topk -> sa_sparse_attn over every query row. Prints one
    JSON line with the step time and the indexer's MFMA utilisation."""
    import torch

    from indexer_top_sparse_amd import binding as B
    from indexer_top_sparse_amd import device, inputs

    B.load()
    torch.cuda.set_device(0)
    wl = inputs.make(args.workload)
    d = device.to_device(wl, "cuda:0")
    ws = device.new_workspace(d)
    ncols = max(wl.ctx_lens)
    rows = wl.num_queries
    scores = torch.empty((rows, ncols), dtype=torch.float32, device="cuda")
    idx = torch.empty((rows, wl.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((rows, wl.heads_q, wl.dim_v), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    if args.copy_calibration_gib > 0:  # the counters' reference copy (see write_traffic)
        nc = int(args.copy_calibration_gib * 2**30) // 4
        ca = torch.empty(nc, dtype=torch.float32, device="cuda").fill_(1.0)
        cb = torch.empty_like(ca)
        cb.copy_(ca)
        torch.cuda.synchronize()
        del ca, cb

    def step():
        B.index_score(d.batch, d.ix, d.t["q_idx"], d.t["w"], scores)
        B.topk(d.batch, scores, wl.topk, idx)
        B.sparse_attn(d.batch, d.kv, d.t["q"], idx, out, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    import numpy as np
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    per = {"index_score": [], "topk": [], "sparse_attn": [], "step": []}
    for _ in range(args.steps):
        ev[0].record(stream)
        B.index_score(d.batch, d.ix, d.t["q_idx"], d.t["w"], scores)
        ev[1].record(stream)
        B.topk(d.batch, scores, wl.topk, idx)
        ev[2].record(stream)
        B.sparse_attn(d.batch, d.kv, d.t["q"], idx, out, ws)
        ev[3].record(stream)
        torch.cuda.synchronize()
        per["index_score"].append(ev[0].elapsed_time(ev[1]))
        per["topk"].append(ev[1].elapsed_time(ev[2]))
        per["sparse_attn"].append(ev[2].elapsed_time(ev[3]))
        per["step"].append(ev[0].elapsed_time(ev[3]))
    n = args.steps
    mean = {k: float(np.mean(v)) for k, v in per.items()}
    t_s, t_k, t_a, tot = mean["index_score"], mean["topk"], mean["sparse_attn"], mean["step"]
    fi, fa = prefill_flops(wl)
    pos = wl.q_pos()
    # row Top-K: the visible scores read once, the index rows written once
    topk_bytes = 4 * int((pos + 1).sum()) + 4 * rows * wl.topk
    roof = {
        "index_score": {"bound": "mfma", "achieved": fi / (t_s * 1e-3) / 1e12,
                        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "flops": fi},
        "topk": {"bound": "hbm", "achieved": topk_bytes / (t_k * 1e-3) / 1e9,
                 "peak": HBM_PEAK_GBS, "unit": "GB/s", "algorithmic_bytes": topk_bytes},
        "sparse_attn": {"bound": "mfma", "achieved": fa / (t_a * 1e-3) / 1e12,
                        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "flops": fa},
    }
    # measured HBM bytes per launch, when the counters were taken on the current sources
    tr = {}
    tfile = os.path.join(PROFILES, f"traffic_{args.workload}.json")
    if os.path.exists(tfile):
        t = json.load(open(tfile))
        if t.get("source_hash") == kernel_source_hash():
            tr = {k: v["hbm_bytes_per_launch"] for k, v in t["kernels"].items()}
    for k, r in roof.items():
        r["frac"] = r["achieved"] / r["peak"]
        r["avg_launch_ms"] = mean[k]
        r["traffic"] = tr.get(k)
    dominant = max(("index_score", "topk", "sparse_attn"), key=lambda k: mean[k])
    res = {
        "metric": "prefill query tokens/s (indexer GEMM + row Top-K + sparse attn)",
        "value": rows / (tot * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": n,
        "warmup": args.warmup, "ms_per_step": tot, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.kv_dtype, "data": "synthetic",
        "config": {"workload": f"{args.workload}: {rows} query rows after a "
                               f"{max(wl.ctx_lens) - rows}-token prefix, K={wl.topk}"},
        "roofline": dict(kernel=dominant, **roof[dominant]),
        "rooflines": roof,
        "kernels_ms": {"index_score": t_s, "topk": t_k, "sparse_attn": t_a},
        "step_distribution": {"steps": n, "median_ms": float(np.median(per["step"])),
                              "p10_ms": float(np.percentile(per["step"], 10)),
                              "p90_ms": float(np.percentile(per["step"], 90))},
        "mfma": {"indexer_tflops": fi / (t_s * 1e-3) / 1e12, "indexer_flops": fi,
                 "attention_tflops": fa / (t_a * 1e-3) / 1e12, "attention_flops": fa,
                 "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                 "indexer_frac": fi / (t_s * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                 "attention_frac": fa / (t_a * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
        "host": host_info(),
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # about 300 steps (some 30 ms of work) bring the GPU to its steady clocks; launches timed
    # before that run several percent slower
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--settle-ms", type=float, default=30.0,
                    help="after the warm-up, run untimed steps for this long (their count is "
                         "reported as settle_steps)")
    ap.add_argument("--workload", default="decode32k",
                    help="input preset (decode32k is the headline configuration)")
    ap.add_argument("--replicas", type=int, default=3)
    ap.add_argument("--dist-steps", type=int, default=200,
                    help="single steps timed one by one for the median / p10 / p90 (at least "
                         "--steps)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-gib", type=float, default=0.0,
                    help="also run a plain device copy of this size (counter calibration)")
    ap.add_argument("--traffic-csv", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU run: turn two rocprofv3 --pmc counter_collection.csv files "
                         "(FETCH_SIZE, WRITE_SIZE) of a run with --copy-calibration-gib into "
                         "profiles/traffic_<workload>.json")
    args = ap.parse_args()
    if args.traffic_csv:
        write_traffic(args.workload, args.traffic_csv, args.copy_calibration_gib)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    if args.workload.startswith("prefill"):
        run_prefill(args)
        return

    import numpy as np
    import torch

    from indexer_top_sparse_amd import binding as B
    from indexer_top_sparse_amd import device, inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.load()
    torch.cuda.set_device(0)
    t0 = time.time()
    wl = inputs.make(args.workload)
    log(f"[bench] generated {args.workload} in {time.time() - t0:.1f}s")

    # replicas: same content at different addresses
    reps = [device.to_device(wl, "cuda:0")]
    for r in range(1, args.replicas):
        d = device.to_device(wl, "cuda:0")
        reps.append(d)
    ws = device.new_workspace(reps[0])
    out = torch.empty((wl.num_seqs, wl.heads_q, wl.dim_v), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((wl.num_seqs, wl.topk), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] {args.replicas} replicas resident, "
        f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated")

    if args.copy_calibration_gib > 0:
        n = int(args.copy_calibration_gib * 2**30) // 4
        a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {n * 4 / 2**30:.2f} GiB read + written")
        del a, b

    def step(i):
        d = reps[i % len(reps)]
        device.decode_step(d, ws, out=out, idx=idx)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    assert B.workspace_error(ws) == 0, "device-side wait failed"
    log(f"[bench] warmup {args.warmup} done")

    # the clocks settle after some 30 ms of sustained work; a short warm-up leaves the first
    # timed steps several percent slower, so untimed steps run for that long after it
    settle, s0 = 0, time.perf_counter()
    while settle < 100000 and (time.perf_counter() - s0) * 1e3 < args.settle_ms:
        for j in range(10):
            step(args.warmup + settle + j)
        settle += 10
        torch.cuda.synchronize()
    assert B.workspace_error(ws) == 0, "device-side wait failed"
    log(f"[bench] settle: {settle} more untimed steps")

    # ---- headline: K fused decode steps
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = e0.elapsed_time(e1) / args.steps
    log(f"[bench] timed {args.steps} steps: {ms_step * 1e3:.1f} us/step (wall {wall * 1e3 / args.steps:.1f})")

    # ---- distribution of single steps (after the headline, so the GPU is at steady clocks):
    #      rotated replicas (cold, as timed above) and one replica (warm)
    nd = max(args.dist_steps, args.steps)
    dist = {"cold": step_distribution(step, nd, stream, rotate=True),
            "warm": step_distribution(step, nd, stream, rotate=False)}
    log(f"[bench] per-step distribution: {dist}")

    # ---- per-kernel durations, measured live on the same stream: K launches of the selection
    #      alone, then K launches of the attention (plus its split merge) alone, each loop
    #      bracketed by events; the average includes only the gaps between back-to-back launches
    idxs = [torch.empty_like(idx) for _ in reps]
    for r, d in enumerate(reps):
        device.index_select(d, ws, idx=idxs[r])
    torch.cuda.synchronize()

    def timed(fn):
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a0.record(stream)
        for i in range(args.steps):
            fn(i)
        a1.record(stream)
        torch.cuda.synchronize()
        return a0.elapsed_time(a1) / args.steps

    sel_avg = timed(lambda i: device.index_select(reps[i % len(reps)], ws,
                                                  idx=idxs[i % len(reps)]))
    att_avg = timed(lambda i: B.sparse_attn(reps[i % len(reps)].batch, reps[i % len(reps)].kv,
                                            reps[i % len(reps)].t["q"], idxs[i % len(reps)],
                                            out, ws))
    assert B.workspace_error(ws) == 0
    log(f"[bench] per launch: select {sel_avg * 1e3:.1f} us, attention {att_avg * 1e3:.1f} us")

    # ---- the step before the path (reported beside it, not part of it): appending one new
    #      token per sequence to the caches (after the timings above, since it changes them)
    g = torch.Generator().manual_seed(7)
    k_new = torch.randn((wl.num_seqs, wl.idx_dim), generator=g).to(torch.bfloat16).cuda()
    kv_new = torch.randn((wl.num_seqs, wl.heads_kv, wl.dim_qk), generator=g).to(torch.bfloat16).cuda()
    v_new = None
    if wl.v_cache is not None:
        v_new = torch.randn((wl.num_seqs, wl.heads_kv, wl.dim_v), generator=g).to(torch.bfloat16).cuda()
    def app(i):
        d = reps[i % len(reps)]
        B.cache_append(d.batch, d.ix, d.kv, k_new, kv_new, v_new)

    # a few microseconds of GPU work per call: K calls are captured in one HIP graph and replayed,
    # so that the host's per-call cost does not hide the kernels' own time
    app(0)
    gph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(gph, stream=side):
            for i in range(args.steps):
                app(i)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    gph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    app_avg = g0.elapsed_time(g1) / args.steps
    log(f"[bench] cache append of {wl.num_seqs} tokens: {app_avg * 1e3:.1f} us (graph replay)")

    # ---- the indexer prolog of the same tokens (synthetic weights; query input 1536 wide,
    #      hidden 7168 wide), timed the same way
    pi = inputs.make_prolog(wl.num_seqs, wl.idx_heads, wl.idx_dim)
    pt = {k: getattr(pi, k).cuda().contiguous() for k in ("x_q", "x", "w_q", "w_k", "w_w", "gamma", "beta")}
    pdesc = B.prolog_desc(wl.idx_heads, wl.idx_dim, pt["w_q"], pt["w_k"], pt["w_w"], pt["gamma"],
                          pt["beta"])
    q_o = torch.empty((wl.num_seqs, wl.idx_heads, wl.idx_dim), dtype=torch.bfloat16, device="cuda")
    k_o = torch.empty((wl.num_seqs, wl.idx_dim), dtype=torch.bfloat16, device="cuda")
    w_o = torch.empty((wl.num_seqs, wl.idx_heads), dtype=torch.float32, device="cuda")
    pws = B.prolog_workspace(pdesc, wl.num_seqs)
    B.indexer_prolog(pdesc, pt["x_q"], pt["x"], q_o, k_o, w_o, pws)
    gp = torch.cuda.CUDAGraph()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(gp, stream=side):
            for i in range(args.steps):
                B.indexer_prolog(pdesc, pt["x_q"], pt["x"], q_o, k_o, w_o, pws)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g0.record(stream)
    gp.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    pro_avg = g0.elapsed_time(g1) / args.steps
    pro_bytes = 2 * (pi.w_q.numel() + pi.w_k.numel() + pi.w_w.numel() + pi.x_q.numel() + pi.x.numel())
    log(f"[bench] indexer prolog of {wl.num_seqs} tokens: {pro_avg * 1e3:.1f} us "
        f"({pro_bytes / (pro_avg * 1e-3) / 1e9:.0f} GB/s of weights and inputs)")

    ab = algorithmic_bytes(wl)
    tokens_per_s = wl.num_seqs / (ms_step * 1e-3)
    step_gbs = ab["step"] / (ms_step * 1e-3) / 1e9

    dominant = "select" if sel_avg >= att_avg else "attention"
    dom_ms = sel_avg if dominant == "select" else att_avg
    achieved = ab[dominant] / (dom_ms * 1e-3) / 1e9
    traffic = None
    tfile = os.path.join(PROFILES, f"traffic_{args.workload}.json")
    if os.path.exists(tfile):
        t = json.load(open(tfile))
        if t.get("source_hash") == kernel_source_hash() and dominant in t.get("kernels", {}):
            traffic = t["kernels"][dominant]["hbm_bytes_per_launch"]

    # ---- CPU baseline: the oracle (plain C, OpenMP) on a bounded sample of the same workload,
    #      in fp32 (the reported value) and in fp64 beside it
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        def oracle_rate(real):
            t1 = time.perf_counter()
            oracle.decode_step(wl, rows=[0], real=real)
            one = time.perf_counter() - t1
            n_rows = max(1, min(wl.num_seqs, int(args.cpu_seconds / max(one, 1e-3))))
            t1 = time.perf_counter()
            oracle.decode_step(wl, rows=list(range(n_rows)), real=real)
            return n_rows, time.perf_counter() - t1

        n32, el32 = oracle_rate("f32")
        n64, el64 = oracle_rate("f64")
        threads = oracle.max_threads("f32")
        cpu = {"value": n32 / el32, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"{n32} of {wl.num_seqs} sequences of the same workload, full path "
                         f"(scores, Top-K, attention), fp32 oracle, {el32:.1f}s",
               "fp64": {"value": n64 / el64, "sample": f"{n64} sequences, {el64:.1f}s"},
               "omp_max_threads": threads, **host_info()}
        log(f"[bench] cpu baseline {cpu}")

    res = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.kv_dtype,
        "data": "synthetic: seeded N(0,1) caches and queries, randomly permuted pages, "
                f"{args.replicas} rotating replicas resident in HBM",
        "config": {
            "workload": f"{args.workload}: decode B={wl.num_seqs} ctx={max(wl.ctx_lens)} "
                        f"page={wl.page_size} indexer {wl.idx_heads}x{wl.idx_dim} {wl.idx_dtype} "
                        f"K={wl.topk} heads_q={wl.heads_q} qk/v={wl.dim_qk}/{wl.dim_v} "
                        f"{wl.kv_dtype}",
            "global_batch": wl.num_seqs, "seq_len": max(wl.ctx_lens), "parallelism": "none",
        },
        "step_hbm": {"algorithmic_bytes": ab["step"], "achieved_gbs": step_gbs,
                     "frac_of_peak": step_gbs / HBM_PEAK_GBS},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes": ab[dominant],
                     "avg_launch_us": dom_ms * 1e3},
        "kernels_us": {"select": sel_avg * 1e3, "attention": att_avg * 1e3,
                       "cache_append": app_avg * 1e3, "indexer_prolog": pro_avg * 1e3},
        "step_distribution": dist,
        "cpu_baseline": cpu,
        "host": host_info(),
        "source_hash": kernel_source_hash(),
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
