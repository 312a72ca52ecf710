#!/usr/bin/env python3
"""MLA decode on one MI355X: microseconds per call and effective KV HBM bandwidth.

Prints ONE JSON line. The headline workload is fp8-KV decode, batch 32 x kv_len
1024 (16 heads, 576/512 dims, page size 1, seeded synthetic inputs resident in
HBM). A "step" is one decode call over the whole batch. Timing:

  * cold (headline): before every timed call a 1 GiB buffer is read (not
    written: a write flush leaves up to 256 MB of dirty MALL lines whose
    write-back would be charged to the timed call), which evicts the 8 x 4 MB
    L2 and the 256 MB MALL, so the cache rows come from HBM; the call is
    bracketed by a pair of HIP events on the stream it runs on (the flush keeps
    the GPU busy while the call is queued, so host submission time is not
    inside the bracket). value = median over --steps.
  * warm (secondary, labelled): --steps calls back to back between one event
    pair; the inputs then sit partly in MALL.

The other four workloads are timed the same way and reported under "grid".
`roofline` refers to the decode call of the headline workload; `cpu_baseline`
is the fp64 CPU oracle on a bounded sample of the same workload.
"""
import os

os.environ.setdefault("HIP_FORCE_DEV_KERNARG", "1")

import argparse  # noqa: E402
import hashlib  # noqa: E402
import json  # noqa: E402
import platform  # noqa: E402
import statistics  # noqa: E402
import sys  # noqa: E402
import time  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
HEADLINE = "fp8_b32_kv1024"
FLUSH_BYTES = 1 << 30
KERNEL_SOURCE = os.path.join(ROOT, "mla_decode_02_amd", "csrc", "mla_decode.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse_args():
    import synthetic as syn

    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE,
                    choices=sorted(set(syn.WORKLOADS) | set(syn.SWEEP) | set(syn.PAGED) | set(syn.RAGGED)))
    ap.add_argument("--flags", type=int, default=0, help="MLA_FLAG_* word (0 = library heuristic)")
    ap.add_argument("--no-grid", action="store_true", help="time only the headline workload")
    ap.add_argument("--sweep", action="store_true",
                    help="also time the full batch {4,32,64,256} x kv_len {1k,8k} x format grid (reported under 'sweep')")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--only-gpu-loop", type=int, default=0,
                    help="skip measurement; run this many back-to-back calls of --workload (for profilers)")
    ap.add_argument("--cold", action="store_true",
                    help="with --only-gpu-loop: read-flush the caches before every call")
    ap.add_argument("--q8", choices=["static", "dynamic"], default=None,
                    help="with --only-gpu-loop: the fp8-query entry point (mla_decode_q8) with this Q scale mode")
    ap.add_argument("--no-q8-grid", action="store_true", help="skip timing the fp8-query variants")
    ap.add_argument("--mtp", type=int, default=0,
                    help="with --only-gpu-loop: this many causal query tokens per sequence (mla_decode_mtp)")
    ap.add_argument("--no-mtp-grid", action="store_true", help="skip timing the several-query-token variants")
    ap.add_argument("--no-mixed-grid", action="store_true", help="skip timing the mixed-length batches")
    return ap.parse_args()


def source_hash():
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def flush_read(buf):
    """Evict L2 and MALL by reading (not writing) a 1 GiB buffer: the caches are left
    holding clean lines, so the timed call pays no write-back of the flush itself."""
    return buf.view(-1, 1 << 20).amax(dim=1)


def upload(case, dev):
    import numpy as np
    import torch

    import synthetic as syn

    q = torch.from_numpy(case.q.view(np.int16)).view(torch.bfloat16).to(dev)
    if case.kv_dtype == syn.KV_BF16:
        kv = torch.from_numpy(case.kv.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        kv = torch.from_numpy(case.kv).to(dev)
    sc = None if case.kv_scales is None else torch.from_numpy(case.kv_scales).to(dev)
    return q, kv, sc, torch.from_numpy(case.kv_indptr).to(dev), torch.from_numpy(case.kv_indices).to(dev)


# The pages' static fp8 query scale: absmax 6 over the e4m3fn maximum 448.
STATIC_Q_SCALE = 6.0 / 448.0


def prepare(mla, case, q, kv, sc, indptr, indices, out, lse, flags, dev, q8=None, mtp=0):
    """The pre-marshalled decode call: mla_decode, or mla_decode_paged for a paged workload,
    or mla_decode_q8 (fp8 query, `q8` = "static" / "dynamic" scale), or mla_decode_mtp
    (`mtp` causal query tokens per sequence; q, out and lse then have B * mtp rows)."""
    import torch

    paged = case.meta.get("paged")
    if mtp:
        extra = {}
        if paged is not None:
            t = {k: torch.from_numpy(paged[k]).to(dev) for k in ("kv_indptr", "kv_indices", "kv_last_page_len")}
            indptr, indices = t["kv_indptr"], t["kv_indices"]
            extra = dict(kv_last_page_len=t["kv_last_page_len"], page_size=paged["page_size"])
        return mla.prepare_decode_mtp(q, None, kv, sc, indptr, indices, out, lse, total_q=q.shape[0], causal=True,
                                      total_kv=case.total_kv, kv_dtype=case.kv_dtype, uni_q_len=mtp, flags=flags,
                                      **extra)
    if q8 is not None:
        mode = mla.Q_SCALE_STATIC if q8 == "static" else mla.Q_SCALE_DYNAMIC
        q_scale = torch.tensor([STATIC_Q_SCALE], dtype=torch.float32, device=dev)
        extra = {}
        if paged is not None:
            t = {k: torch.from_numpy(paged[k]).to(dev) for k in ("kv_indptr", "kv_indices", "kv_last_page_len")}
            indptr, indices = t["kv_indptr"], t["kv_indices"]
            extra = dict(kv_last_page_len=t["kv_last_page_len"], page_size=paged["page_size"])
        return mla.prepare_decode_q8(q, q_scale, kv, sc, indptr, indices, out, lse, q_scale_mode=mode,
                                     total_kv=case.total_kv, kv_dtype=case.kv_dtype, flags=flags, **extra)
    if paged is None:
        return mla.prepare_decode(q, kv, sc, indptr, indices, out, lse, total_kv=case.total_kv,
                                  kv_dtype=case.kv_dtype, flags=flags)
    t = {k: torch.from_numpy(paged[k]).to(dev) for k in ("kv_indptr", "kv_indices", "kv_last_page_len")}
    return mla.prepare_decode_paged(q, kv, sc, t["kv_indptr"], t["kv_indices"], t["kv_last_page_len"], out, lse,
                                    page_size=paged["page_size"], total_kv=case.total_kv, kv_dtype=case.kv_dtype,
                                    flags=flags)


def mtp_query(case, mtp, dev):
    """bf16 query of `mtp` tokens per sequence, seeded from the workload's own seed."""
    import numpy as np
    import torch

    import synthetic as syn

    qb, _ = syn.make_mtp_query([mtp] * case.batch, seed=case.meta.get("seed", 0) + 1000 * mtp)
    return torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).to(dev)


def measure(name, args, dev, flush, q8=None, mtp=0):
    import torch

    import mla_decode_02_amd as mla
    import synthetic as syn

    case = syn.make_workload(name)
    q, kv, sc, indptr, indices = upload(case, dev)
    B = case.batch
    rows = B * mtp if mtp else B
    if mtp:
        q = mtp_query(case, mtp, dev)
    out = torch.empty((rows, 16, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((rows, 16), dtype=torch.float32, device=dev)
    call = prepare(mla, case, q, kv, sc, indptr, indices, out, lse, args.flags, dev, q8=q8, mtp=mtp)
    paged = case.meta.get("paged")
    plan_flags = args.flags | (mla.FLAG_FORCE_SPLIT if (paged and paged["page_size"] > 1) or mtp else 0)
    if mtp:  # the plan runs over the query rows, each seeing its sequence
        plan = mla.mla_decode_plan(rows, min(case.total_kv * mtp, 2**31 - 1), case.kv_dtype, plan_flags)
    else:
        plan = mla.mla_decode_plan(B, case.total_kv, case.kv_dtype, plan_flags)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()

    # cold: flush, then one bracketed call per step
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    for i in range(args.steps):
        flush_read(flush)
        ev[i][0].record()
        call()
        ev[i][1].record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    cold_us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)

    # warm: back to back behind a fill that lets the queue build up
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    flush_read(flush)
    e0.record()
    for _ in range(args.steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    warm_us = e0.elapsed_time(e1) * 1e3 / args.steps

    med = statistics.median(cold_us)
    kv_bytes, tot_bytes = case.kv_bytes(), case.total_bytes()
    if mtp:  # the extra query rows: q, out and lse of each
        tot_bytes += (rows - B) * (2 * 16 * 576 + 2 * 16 * 512 + 4 * 16)
    return {
        "workload": name,
        "query": ("bf16" if q8 is None else f"fp8 ({q8} per-tensor scale)")
                 + (f", {mtp} causal tokens per sequence" if mtp else ""),
        "kv_format": syn.KV_NAMES[case.kv_dtype],
        "page_size": case.meta.get("paged", {}).get("page_size", 1),
        "batch": B,
        "kv_len": int(case.kv_indptr[1] - case.kv_indptr[0]),
        "plan": {"mode": "split" if plan.mode == 0 else "persistent", "splits": plan.num_splits,
                 "grid": plan.grid, "combine_launch": plan.combine == 1,
                 "merge": ("none", "combine launch", "last-arriving split workgroup")[plan.combine]},
        "cold_us_median": med,
        "cold_us_p10": cold_us[len(cold_us) // 10],
        "cold_us_p90": cold_us[(9 * len(cold_us)) // 10],
        "cold_us_mean": statistics.fmean(cold_us),
        "warm_us": warm_us,
        "kv_bytes": kv_bytes,
        "algorithmic_bytes": tot_bytes,
        "effective_kv_GBps": kv_bytes / (med * 1e-6) / 1e9,
        "pct_hbm_peak_kv": 100.0 * kv_bytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS,
        "algorithmic_GBps": tot_bytes / (med * 1e-6) / 1e9,
        "wall_ms_per_step_incl_flush": 1e3 * t_wall / args.steps,
        "_case": case,
    }


def measure_graph(name, args, dev, flush):
    """The same call captured once in a HIP graph and replayed: cold median per replay (events around each
    replay, read flush before it), as a serving loop that captures its decode step would run it."""
    import torch

    import mla_decode_02_amd as mla
    import synthetic as syn

    case = syn.make_workload(name)
    q, kv, sc, indptr, indices = upload(case, dev)
    B = case.batch
    out = torch.empty((B, 16, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, 16), dtype=torch.float32, device=dev)
    ws = mla.new_workspace(mla.mla_decode_workspace_size(B, case.total_kv, case.kv_dtype, args.flags), dev)

    def call():
        mla.mla_decode(q, kv, sc, indptr, indices, out, lse, total_kv=case.total_kv, kv_dtype=case.kv_dtype,
                       workspace=ws, flags=args.flags)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        flush_read(flush)
        ev[i][0].record()
        g.replay()
        ev[i][1].record()
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    return {"workload": name, "cold_us_median": statistics.median(us), "cold_us_p10": us[len(us) // 10],
            "cold_us_p90": us[(9 * len(us)) // 10],
            "effective_kv_GBps": case.kv_bytes() / (statistics.median(us) * 1e-6) / 1e9}


def cpu_baseline(case, target_s):
    """Time the fp64 oracle on a bounded sample of sequences; scale to the whole call."""
    import oracle

    oracle.build(force=False)
    B = case.batch
    t0 = time.perf_counter()
    oracle.mla_decode(case.q, case.kv_dtype, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices, batches=[0])
    t_one = time.perf_counter() - t0
    n = int(max(1, min(B, target_s / max(t_one, 1e-6))))
    batches = list(range(n))
    # repeat the sample until about a fifth of the target time has accumulated
    # (small workloads finish in well under a second)
    reps, t = 0, 0.0
    while reps == 0 or (t < target_s / 5 and reps < 50):
        t0 = time.perf_counter()
        oracle.mla_decode(case.q, case.kv_dtype, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices,
                          batches=batches)
        t += time.perf_counter() - t0
        reps += 1
    t /= reps
    threads = oracle.max_threads()
    # the same oracle on one thread, on a sample of at most a few sequences
    n1 = max(1, min(n, 4))
    t0 = time.perf_counter()
    oracle.mla_decode(case.q, case.kv_dtype, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices,
                      batches=list(range(n1)), nthreads=1)
    t1 = time.perf_counter() - t0
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": t * 1e6 * B / n,
        "unit": "us/call",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{n} of {B} sequences of {case.meta['workload']} (fp64 C oracle, OpenMP over heads), "
                  f"mean of {reps} runs of {t:.3f} s, scaled by {B}/{n}",
        "host_cpu": cpu,
        "host_nproc": os.cpu_count(),
        "single_thread": {"value": t1 * 1e6 * B / n1, "unit": "us/call", "cores": 1,
                          "sample": f"{n1} of {B} sequences, one run of {t1:.3f} s, scaled by {B}/{n1}"},
    }


def read_ceiling(dev, flush, nbytes=302 << 20, steps=10):
    """Practical HBM read reference on this machine: a plain cold streaming read of nbytes (a torch
    row-wise max over 4 KiB rows, the fastest plain torch read measured here), after the same
    1 GiB read flush, HIP events around it, median GB/s."""
    import torch

    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    rows = buf.view(-1, 1024)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    rows.amax(dim=1)
    for i in range(steps):
        flush_read(flush)
        ev[i][0].record()
        rows.amax(dim=1)
        ev[i][1].record()
    torch.cuda.synchronize()
    us = statistics.median(a.elapsed_time(b) * 1e3 for a, b in ev)
    del rows, buf
    return {"bytes": nbytes, "cold_us_median": us, "GBps": nbytes / (us * 1e-6) / 1e9,
            "kernel": "torch amax over 4 KiB rows of a contiguous fp32 buffer"}


def load_traffic(name):
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    ent = d.get(name)
    if not ent or ent.get("source_hash") != source_hash():
        return None  # counters were taken on a different kernel build
    return ent.get("bytes_per_call")


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the decode path runs on a "
              "single MI355X (decode would shard by batch, one share per GPU).", file=sys.stderr)
        sys.exit(2)
    import torch

    import mla_decode_02_amd as mla
    import synthetic as syn

    dev = torch.device("cuda:0")
    if args.only_gpu_loop:
        case = syn.make_workload(args.workload)
        q, kv, sc, indptr, indices = upload(case, dev)
        out = torch.empty((case.batch, 16, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((case.batch, 16), dtype=torch.float32, device=dev)
        if args.mtp:
            q = mtp_query(case, args.mtp, dev)
            out = torch.empty((q.shape[0], 16, 512), dtype=torch.bfloat16, device=dev)
            lse = torch.empty((q.shape[0], 16), dtype=torch.float32, device=dev)
        call = prepare(mla, case, q, kv, sc, indptr, indices, out, lse, args.flags, dev, q8=args.q8, mtp=args.mtp)
        flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev) if args.cold else None
        for _ in range(args.only_gpu_loop):
            if flush is not None:
                flush_read(flush)
            call()
        torch.cuda.synchronize()
        print(json.dumps({"workload": args.workload, "q8": args.q8, "mtp": args.mtp, "calls": args.only_gpu_loop}),
              flush=True)
        return

    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    names = [args.workload] + ([] if args.no_grid else [n for n in syn.WORKLOADS if n != args.workload])
    results = {}
    for n in names:
        results[n] = measure(n, args, dev, flush)
        r = results[n]
        print(f"# {n}: cold {r['cold_us_median']:.2f} us (p10 {r['cold_us_p10']:.2f}, p90 {r['cold_us_p90']:.2f}), "
              f"warm {r['warm_us']:.2f} us, {r['effective_kv_GBps']:.0f} GB/s KV ({r['pct_hbm_peak_kv']:.1f}% of 8 TB/s)",
              file=sys.stderr, flush=True)
    # The fp8-query entry point (the pages' a8w8 path) on the same workloads,
    # with the static and with the dynamic query scale.
    grid_q8 = None
    if not args.no_q8_grid:
        grid_q8 = {}
        todo = [(n, mode) for n in names for mode in ("static", "dynamic")]
        for n, mode in todo:
            r = measure(n, args, dev, flush, q8=mode)
            r.pop("_case", None)
            grid_q8[f"{n}/{mode}"] = r
            print(f"# q8 {mode} {n}: cold {r['cold_us_median']:.2f} us, warm {r['warm_us']:.2f} us, "
                  f"{r['effective_kv_GBps']:.0f} GB/s KV ({r['pct_hbm_peak_kv']:.1f}% of 8 TB/s)",
                  file=sys.stderr, flush=True)
    # Mixed-length batches (lengths uniform in [256, 16128]): the default plan (split-K) and the
    # mixed-lengths hint (persistent grid).
    grid_mixed = None
    if not args.no_mixed_grid:
        grid_mixed = {}
        base_flags = args.flags
        for n in syn.RAGGED:
            for hint in (False, True):
                args.flags = base_flags | (mla.FLAG_MIXED_LENGTHS if hint else 0)
                r = measure(n, args, dev, flush)
                r.pop("_case", None)
                key = f"{n}/{'mixed_lengths_hint' if hint else 'default'}"
                grid_mixed[key] = r
                print(f"# mixed {key}: cold {r['cold_us_median']:.2f} us, {r['effective_kv_GBps']:.0f} GB/s KV "
                      f"({r['pct_hbm_peak_kv']:.1f}% of 8 TB/s), plan {r['plan']}", file=sys.stderr, flush=True)
        args.flags = base_flags
        torch.cuda.empty_cache()
    # Several causal query tokens per sequence (mla_decode_mtp): 2 and 4 tokens on the headline
    # workload and on the bandwidth-bound fp8 64 x 8192 workload. Effective GB/s counts the cache once.
    grid_mtp = None
    if not args.no_mtp_grid:
        grid_mtp = {}
        for n in dict.fromkeys([args.workload, "fp8_b64_kv8192"]):
            for k in (2, 4):
                r = measure(n, args, dev, flush, mtp=k)
                r.pop("_case", None)
                grid_mtp[f"{n}/q{k}"] = r
                print(f"# mtp q{k} {n}: cold {r['cold_us_median']:.2f} us, warm {r['warm_us']:.2f} us, "
                      f"{r['effective_kv_GBps']:.0f} GB/s KV counted once ({r['pct_hbm_peak_kv']:.1f}% of 8 TB/s)",
                      file=sys.stderr, flush=True)
    graph = None
    if args.workload not in syn.PAGED:  # the graph leg replays mla_decode (page size 1)
        graph = measure_graph(args.workload, args, dev, flush)
        print(f"# graph replay {args.workload}: cold {graph['cold_us_median']:.2f} us "
              f"(p10 {graph['cold_us_p10']:.2f}, p90 {graph['cold_us_p90']:.2f})", file=sys.stderr, flush=True)
    head = results[args.workload]
    case = head.pop("_case")
    for r in results.values():
        r.pop("_case", None)
    sweep = None
    if args.sweep:
        sweep = {}
        for n in list(syn.SWEEP) + list(syn.PAGED):
            r = dict(results[n]) if n in results else measure(n, args, dev, flush)
            r.pop("_case", None)
            sweep[n] = r
            print(f"# sweep {n}: cold {r['cold_us_median']:.2f} us, warm {r['warm_us']:.2f} us, "
                  f"{r['effective_kv_GBps']:.0f} GB/s KV ({r['pct_hbm_peak_kv']:.1f}% of 8 TB/s), plan {r['plan']}",
                  file=sys.stderr, flush=True)
            torch.cuda.empty_cache()

    achieved = head["algorithmic_bytes"] / (head["cold_us_mean"] * 1e-6) / 1e9
    traffic = load_traffic(args.workload)
    roofline = {
        "bound": "hbm",
        "achieved": achieved,
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": achieved / HBM_PEAK_GBPS,
        "traffic": traffic,
        "kernel": "mla decode call (stage-1 kernel, plus the combine kernel when the plan merges in a launch)",
        "bytes_per_launch": head["algorithmic_bytes"],
        "timing": "HIP events on the launch stream, cold cache, mean over steps",
    }
    cpu = None if args.no_cpu_baseline else cpu_baseline(case, args.cpu_seconds)
    ceiling = read_ceiling(dev, flush)
    print(f"# plain cold read of {ceiling['bytes'] / 1e6:.0f} MB: {ceiling['cold_us_median']:.1f} us, "
          f"{ceiling['GBps']:.0f} GB/s", file=sys.stderr, flush=True)
    line = {
        "metric": "us/call and effective KV HBM GB/s (% of peak), MLA decode bs x kv grid",
        "value": head["cold_us_median"],
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["cold_us_median"] / 1e3,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "dtype_detail": f"{syn.KV_NAMES[case.kv_dtype]} cache decoded exactly to bf16; bf16 MFMA, fp32 accumulate",
        "data": "synthetic (seeded N(0,1) q and cache rows, quantised per format)",
        "config": {"workload": args.workload, "batch": head["batch"], "kv_len": head["kv_len"],
                   "kv_format": head["kv_format"], "heads": 16, "qk_dim": 576, "v_dim": 512, "page_size": 1,
                   "plan": head["plan"]},
        "effective_kv_GBps": head["effective_kv_GBps"],
        "pct_hbm_peak_kv": head["pct_hbm_peak_kv"],
        "warm_us": head["warm_us"],
        "roofline": roofline,
        "hbm_read_ceiling": ceiling,
        "graph_replay": graph,
        "cpu_baseline": cpu,
        "grid": results,
        "grid_q8": grid_q8,
        "grid_mtp": grid_mtp,
        "grid_mixed": grid_mixed,
        "sweep": sweep,
        "kernel_source_hash": source_hash(),
        "host": platform.node(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
