#!/usr/bin/env python3
"""MLA decode on one MI355X: microseconds per call and effective KV HBM bandwidth.

Prints ONE JSON line. The headline workload is fp8-KV decode, batch 64 x kv_len
8192 (16 heads, 576/512 dims, page size 1, seeded synthetic inputs resident in
HBM; 302 MB of cache), the largest of the measured configurations that fits
one GPU. A "step" is one decode call over the whole batch. Timing:

  * cold (headline): before every timed call a 1 GiB buffer is read (not
    written: a write flush leaves up to 256 MB of dirty MALL lines whose
    write-back would be charged to the timed call), which evicts the 8 x 4 MB
    L2 and the 256 MB MALL, so the cache rows come from HBM; the call is
    bracketed by a pair of HIP events on the stream it runs on (the flush keeps
    the GPU busy while the call is queued, so host submission time is not
    inside the bracket). value = median over --steps.
  * warm (secondary, labelled): --steps calls back to back between one event
    pair; the inputs then sit partly in MALL.

The other measured workloads (fp8 32x1k, bf16 4x1k, fp8 4x8k, MXFP4 32x8k) are
timed the same way under "grid", and the pages' whole shape grid (batch
{4, 32, 64, 256} x kv_len {1024, 8192} x the three formats, plus the 8-row-page
caches) under "sweep" with --sweep-steps calls each. `roofline` refers to the
headline call; `roofline_grid` gives the same figures for every grid workload.
`cpu_baseline` is the fp64 CPU oracle on a bounded sample of the headline.

`python bench.py --summarise DIR` (no GPU) turns the rocprofv3 runs under DIR
into the summaries under profiles/ (see summarise()).
"""
import os

os.environ.setdefault("HIP_FORCE_DEV_KERNARG", "1")

import argparse  # noqa: E402
import csv  # noqa: E402
import json  # noqa: E402
import platform  # noqa: E402
import statistics  # noqa: E402
import sys  # noqa: E402
import time  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
HEADLINE = "fp8_b64_kv8192"
FLUSH_BYTES = 1 << 30
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic.json")
KERNEL_TIMES_FILE = os.path.join(PROFILES, "kernel_times.json")
FLOP_PER_TOKEN = 34816  # 2 * 16 * 576 (scores) + 2 * 16 * 512 (P.V)


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
    ap.add_argument("--no-sweep", action="store_true", help="skip the full batch x kv_len x format grid")
    ap.add_argument("--sweep-steps", type=int, default=20, help="cold (and warm) calls per sweep shape")
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
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay leg")
    ap.add_argument("--phases", nargs="*", metavar="WORKLOAD", default=None,
                    help="load the measurement build (phase timestamps) and print the per-phase timeline of "
                         "these workloads' cold calls (default: the five measured workloads)")
    ap.add_argument("--summarise", metavar="DIR", default=None,
                    help="write the profiles/ summaries from the rocprofv3 runs under DIR and exit (no GPU)")
    return ap.parse_args()


def source_hash():
    """Digest of the sources the loaded library was built from; importing the
    package has already checked that it is the digest of the tree's sources."""
    import mla_decode_02_amd as mla

    return mla.mla_source_digest()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


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
    extra = {}
    if paged is not None:
        t = {k: torch.from_numpy(paged[k]).to(dev) for k in ("kv_indptr", "kv_indices", "kv_last_page_len")}
        indptr, indices = t["kv_indptr"], t["kv_indices"]
        extra = dict(kv_last_page_len=t["kv_last_page_len"], page_size=paged["page_size"])
    if mtp:
        return mla.prepare_decode_mtp(q, None, kv, sc, indptr, indices, out, lse, total_q=q.shape[0], causal=True,
                                      total_kv=case.total_kv, kv_dtype=case.kv_dtype, uni_q_len=mtp, flags=flags,
                                      **extra)
    if q8 is not None:
        mode = mla.Q_SCALE_STATIC if q8 == "static" else mla.Q_SCALE_DYNAMIC
        q_scale = torch.tensor([STATIC_Q_SCALE], dtype=torch.float32, device=dev)
        return mla.prepare_decode_q8(q, q_scale, kv, sc, indptr, indices, out, lse, q_scale_mode=mode,
                                     total_kv=case.total_kv, kv_dtype=case.kv_dtype, flags=flags, **extra)
    if paged is None:
        return mla.prepare_decode(q, kv, sc, indptr, indices, out, lse, total_kv=case.total_kv,
                                  kv_dtype=case.kv_dtype, flags=flags)
    return mla.prepare_decode_paged(q, kv, sc, indptr, indices, extra["kv_last_page_len"], out, lse,
                                    page_size=paged["page_size"], total_kv=case.total_kv, kv_dtype=case.kv_dtype,
                                    flags=flags)


def mtp_query(case, mtp, dev):
    """bf16 query of `mtp` tokens per sequence, seeded from the workload's own seed."""
    import numpy as np
    import torch

    import synthetic as syn

    qb, _ = syn.make_mtp_query([mtp] * case.batch, seed=case.meta.get("seed", 0) + 1000 * mtp)
    return torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).to(dev)


def plan_of(mla, case, flags, mtp=0):
    paged = case.meta.get("paged")
    plan_flags = flags | (mla.FLAG_FORCE_SPLIT if (paged and paged["page_size"] > 1) or mtp else 0)
    if mtp:  # split-K over the query rows (or, on the bf16 cache, row pairs), each seeing its sequence
        return mla.mla_decode_mtp_plan(case.batch, case.batch * mtp, case.total_kv, case.kv_dtype, plan_flags, mtp)
    return mla.mla_decode_plan(case.batch, case.total_kv, case.kv_dtype, plan_flags)


def launches(plan, q8=None):
    """Kernel launches of one call, in order."""
    k = ["q_amax"] if q8 == "dynamic" else []
    k.append("stage1")
    if plan.combine == 1:
        k.append("combine")
    return k


def measure(name, args, dev, flush, q8=None, mtp=0, steps=None):
    import torch

    import mla_decode_02_amd as mla
    import synthetic as syn

    steps = steps or args.steps
    case = syn.make_workload(name)
    q, kv, sc, indptr, indices = upload(case, dev)
    B = case.batch
    rows = B * mtp if mtp else B
    if mtp:
        q = mtp_query(case, mtp, dev)
    out = torch.empty((rows, 16, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((rows, 16), dtype=torch.float32, device=dev)
    call = prepare(mla, case, q, kv, sc, indptr, indices, out, lse, args.flags, dev, q8=q8, mtp=mtp)
    plan = plan_of(mla, case, args.flags, mtp)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()

    # cold: flush, then one bracketed call per step
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    for i in range(steps):
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
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    warm_us = e0.elapsed_time(e1) * 1e3 / steps

    med = statistics.median(cold_us)
    kv_bytes, tot_bytes = case.kv_bytes(), case.total_bytes()
    if mtp:  # the extra query rows: q, out and lse of each
        tot_bytes += (rows - B) * (2 * 16 * 576 + 2 * 16 * 512 + 4 * 16)
    mean = statistics.fmean(cold_us)
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
                 "merge": ("none", "combine launch", "last-arriving split workgroup")[plan.combine],
                 "rows_per_wg": plan.rows_per_wg},
        "launches": launches(plan, q8),
        "steps": steps,
        "calls": 1 + args.warmup + 2 * steps,  # the prepared call's checked first call, warm-up, cold, warm
        "cold_us_median": med,
        "cold_us_p10": cold_us[len(cold_us) // 10],
        "cold_us_p90": cold_us[(9 * len(cold_us)) // 10],
        "cold_us_mean": mean,
        "warm_us": warm_us,
        "kv_bytes": kv_bytes,
        "algorithmic_bytes": tot_bytes,
        "effective_kv_GBps": kv_bytes / (med * 1e-6) / 1e9,
        "pct_hbm_peak_kv": 100.0 * kv_bytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS,
        "algorithmic_GBps": tot_bytes / (mean * 1e-6) / 1e9,
        "frac_hbm_peak_call": tot_bytes / (mean * 1e-6) / 1e9 / HBM_PEAK_GBPS,
        "wall_ms_per_step_incl_flush": 1e3 * t_wall / steps,
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
    plan = plan_of(mla, case, args.flags)
    return {"workload": name, "cold_us_median": statistics.median(us), "cold_us_p10": us[len(us) // 10],
            "cold_us_p90": us[(9 * len(us)) // 10], "launches": launches(plan),
            "calls": 1 + args.warmup + args.steps,  # the eager call before capture, warm-up and timed replays
            "effective_kv_GBps": case.kv_bytes() / (statistics.median(us) * 1e-6) / 1e9}


TICK_US = 0.01  # s_memrealtime runs at 100 MHz


def phases(args):
    """The stage-1 and combine workgroups' timelines from the measurement build
    (include/mla_decode_phases.h): cold calls as in measure(), each workgroup's
    phase stamps read back after the call. Per call, times are relative to the
    first stage-1 workgroup's entry; each figure is the median over calls of a
    median or maximum over the workgroups. Prints a markdown table."""
    import numpy as np
    import torch

    import mla_decode_02_amd as mla
    import synthetic as syn

    assert mla.LIB_PATH.endswith("libmla_decode_phases.so"), mla.LIB_PATH
    dev = torch.device("cuda:0")
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    names = args.phases or list(syn.WORKLOADS)
    steps = min(args.steps, 30)
    print(f"Phase timeline of the stage-1 and combine workgroups (measurement build, source digest "
          f"`{mla.mla_source_digest()}`; {steps} cold calls each, after {args.warmup} warm-up calls; "
          "us from the first stage-1 workgroup's entry; med / max over the workgroups, median over calls)\n")
    print("| workload | plan | entry skew med / max | query + index med | first rows landed med | token steps med / "
          "max | epilogue stores med | stage-1 merge med / max | stage-1 end med / max | combine start | "
          "combine end |")
    print("|" + "---|" * 11)
    for name in names:
        case = syn.make_workload(name)
        q, kv, sc, indptr, indices = upload(case, dev)
        out = torch.empty((case.batch, 16, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((case.batch, 16), dtype=torch.float32, device=dev)
        plan = plan_of(mla, case, args.flags)
        st = torch.zeros(plan.grid * 8, dtype=torch.int64, device=dev)
        comb = torch.zeros(64 * case.batch * 2, dtype=torch.int64, device=dev)
        mla.mla_phase_buffers(st, comb)
        call = prepare(mla, case, q, kv, sc, indptr, indices, out, lse, args.flags, dev)
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        rows = []
        for _ in range(steps):
            st.zero_()
            comb.zero_()
            flush_read(flush)
            call()
            torch.cuda.synchronize()
            s = st.view(-1, 8).cpu().numpy().astype(np.int64)
            c = comb.view(-1, 2).cpu().numpy().astype(np.int64)
            t0 = s[:, 0].min()
            ok = s[:, 2] > 0  # workgroups that attended tokens
            d = lambda a, b: (s[ok, b] - s[ok, a]) * TICK_US  # noqa: E731
            cw = c[:, 0] > 0
            rows.append([np.median((s[:, 0] - t0) * TICK_US), np.max((s[:, 0] - t0) * TICK_US),
                         np.median(d(0, 1)), np.median(d(1, 2)), np.median(d(2, 3)), np.max(d(2, 3)),
                         np.median(d(3, 4)), np.median(d(4, 5)), np.max(d(4, 5)),
                         np.median((s[:, 5] - t0) * TICK_US), np.max((s[:, 5] - t0) * TICK_US),
                         (c[cw, 0].min() - t0) * TICK_US if cw.any() else float("nan"),
                         (c[cw, 1].max() - t0) * TICK_US if cw.any() else float("nan")])
        mla.mla_phase_buffers(None, None)
        r = np.median(np.array(rows), axis=0)
        pl = f"{plan.num_splits} splits, {plan.grid} WGs, " + ("none", "combine launch", "merged in stage 1")[plan.combine]
        cs = "—" if np.isnan(r[11]) else f"{r[11]:.2f}"
        ce = "—" if np.isnan(r[12]) else f"{r[12]:.2f}"
        print(f"| {name} | {pl} | {r[0]:.2f} / {r[1]:.2f} | {r[2]:.2f} | {r[3]:.2f} | {r[4]:.2f} / {r[5]:.2f} | "
              f"{r[6]:.2f} | {r[7]:.2f} / {r[8]:.2f} | {r[9]:.2f} / {r[10]:.2f} | {cs} | {ce} |", flush=True)
        del q, kv, sc, indptr, indices, out, lse, st, comb, call
        torch.cuda.empty_cache()


def cpu_baseline(case, target_s):
    """Time the fp64 oracle on a bounded sample of sequences; scale to the whole call."""
    import oracle

    oracle.build(force=False)
    B = case.batch
    t0 = time.perf_counter()
    oracle.mla_decode(case.q, case.kv_dtype, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices, batches=[0])
    t_one = time.perf_counter() - t0
    n = int(max(1, min(B, target_s / 3 / max(t_one, 1e-6))))
    batches = list(range(n))
    # repeat the sample until about a third of the target time has accumulated
    # (small workloads finish in well under a second)
    reps, t = 0, 0.0
    while reps == 0 or (t < target_s / 3 and reps < 50):
        t0 = time.perf_counter()
        oracle.mla_decode(case.q, case.kv_dtype, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices,
                          batches=batches)
        t += time.perf_counter() - t0
        reps += 1
    t /= reps
    threads = oracle.max_threads()
    # the same oracle on one thread, on a sample of at most two sequences
    n1 = max(1, min(n, 2))
    t0 = time.perf_counter()
    oracle.mla_decode(case.q, case.kv_dtype, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices,
                      batches=list(range(n1)), nthreads=1)
    t1 = time.perf_counter() - t0
    oracle.mla_decode(case.q, case.kv_dtype, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices,
                      batches=[0], nthreads=threads)  # restore the thread count
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


def read_ceiling(dev, flush, nbytes, steps=20):
    """Practical HBM read ceiling on this machine: the library's streaming read (mla_hbm_read_probe: the
    gathers' own LDS-DMA loads and cache hint, each workgroup one contiguous share) of nbytes, cold
    (same 1 GiB read flush first), HIP events around it, median GB/s."""
    import torch

    import mla_decode_02_amd as mla

    nbytes = nbytes // 16 * 16
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    mla.mla_hbm_read_probe(buf)
    for i in range(steps):
        flush_read(flush)
        ev[i][0].record()
        mla.mla_hbm_read_probe(buf)
        ev[i][1].record()
    torch.cuda.synchronize()
    us = statistics.median(a.elapsed_time(b) * 1e3 for a, b in ev)
    del buf
    return {"bytes": nbytes, "cold_us_median": us, "GBps": nbytes / (us * 1e-6) / 1e9,
            "frac_of_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
            "kernel": "mla_hbm_read_probe (stream_read_kernel: LDS-DMA, non-temporal, 512 workgroups)"}


def _load_profile_json(path, name):
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    ent = d.get(name)
    if not ent or ent.get("source_hash") != source_hash():
        return None  # taken on a different kernel build
    return ent


def roofline_of(r):
    """Roofline figures of one measured workload: the call (HIP events, cold mean) and, when
    the call is one launch, the stage-1 kernel (the same events time exactly that launch);
    for a two-launch plan the stage-1 kernel time comes from the committed kernel trace of
    the same kernel build (profiles/kernel_times.json), else null."""
    bytes_ = r["algorithmic_bytes"]
    call_gbps = bytes_ / (r["cold_us_mean"] * 1e-6) / 1e9
    kt = _load_profile_json(KERNEL_TIMES_FILE, r["workload"])
    if r["launches"] == ["stage1"]:
        k_us, k_src = r["cold_us_mean"], "HIP events around the call, which is this one launch"
    elif kt is not None:
        k_us, k_src = kt["stage1_cold_avg_us"], "profiles/kernel_times.json (rocprofv3 kernel trace, same build)"
    else:
        k_us, k_src = None, None
    ent = {"call_us_mean": r["cold_us_mean"], "call_GBps": call_gbps, "call_frac": call_gbps / HBM_PEAK_GBPS,
           "launches": r["launches"], "kernel_us": k_us, "kernel_time_source": k_src,
           "kernel_frac": (bytes_ / (k_us * 1e-6) / 1e9 / HBM_PEAK_GBPS) if k_us else None,
           "kv_frac_median": r["pct_hbm_peak_kv"] / 100.0}
    return ent


def main():
    args = parse_args()
    if args.summarise:
        summarise(args.summarise)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the decode path runs on a "
              "single MI355X (decode would shard by batch, one share per GPU).", file=sys.stderr)
        sys.exit(2)
    if args.phases is not None:
        os.environ["MLA_DECODE_LIBRARY"] = "phases"  # before the package is imported
        phases(args)
        return
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
        print(json.dumps({"workload": args.workload, "q8": args.q8, "mtp": args.mtp, "calls": args.only_gpu_loop,
                          "kernel_source_hash": source_hash()}), flush=True)
        return

    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    legs = []  # measured legs in launch order (the kernel-trace summary walks them)
    names = [args.workload] + ([] if args.no_grid else [n for n in syn.WORKLOADS if n != args.workload])
    results = {}
    for n in names:
        results[n] = measure(n, args, dev, flush)
        r = results[n]
        legs.append({"label": n, "calls": r["calls"], "launches": r["launches"], "steps": r["steps"]})
        log(f"# {n}: cold {r['cold_us_median']:.2f} us (p10 {r['cold_us_p10']:.2f}, p90 {r['cold_us_p90']:.2f}), "
            f"warm {r['warm_us']:.2f} us, {r['effective_kv_GBps']:.0f} GB/s KV ({r['pct_hbm_peak_kv']:.1f}% of 8 TB/s), "
            f"plan {r['plan']}")
    # The fp8-query entry point (the pages' a8w8 path) on the same workloads,
    # with the static and with the dynamic query scale.
    grid_q8 = None
    if not args.no_q8_grid:
        grid_q8 = {}
        for n in names:
            for mode in ("static", "dynamic"):
                r = measure(n, args, dev, flush, q8=mode)
                r.pop("_case", None)
                grid_q8[f"{n}/{mode}"] = r
                legs.append({"label": f"q8 {n}/{mode}", "calls": r["calls"], "launches": r["launches"],
                             "steps": r["steps"]})
                log(f"# q8 {mode} {n}: cold {r['cold_us_median']:.2f} us, warm {r['warm_us']:.2f} us, "
                    f"{r['effective_kv_GBps']:.0f} GB/s KV ({r['pct_hbm_peak_kv']:.1f}% of 8 TB/s)")
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
                legs.append({"label": f"mixed {key}", "calls": r["calls"], "launches": r["launches"],
                             "steps": r["steps"]})
                log(f"# mixed {key}: cold {r['cold_us_median']:.2f} us, {r['effective_kv_GBps']:.0f} GB/s KV "
                    f"({r['pct_hbm_peak_kv']:.1f}% of 8 TB/s), plan {r['plan']}")
        args.flags = base_flags
        torch.cuda.empty_cache()
    # Several causal query tokens per sequence (mla_decode_mtp): 2 and 4 tokens on fp8 32 x 1k,
    # fp8 64 x 8k and bf16 64 x 8k. On the bf16 cache the default plan carries two query rows per
    # workgroup; its "rows" legs force one row per workgroup, and "q1" is the one-token mla_decode
    # call on the same cache. Effective GB/s counts the cache once.
    grid_mtp = None
    if not args.no_mtp_grid:
        grid_mtp = {}
        base_flags = args.flags
        mtp_legs = [("fp8_b32_kv1024", k, "") for k in (2, 4)] + [("fp8_b64_kv8192", k, "") for k in (2, 4)] + \
            [("bf16_b64_kv8192", 1, ""), ("bf16_b64_kv8192", 2, ""), ("bf16_b64_kv8192", 4, ""),
             ("bf16_b64_kv8192", 2, "rows"), ("bf16_b64_kv8192", 4, "rows")]
        for n, k, variant in mtp_legs:
            args.flags = base_flags | (mla.FLAG_ROW_PER_WG if variant == "rows" else 0)
            r = measure(n, args, dev, flush, mtp=k if k > 1 else 0)
            r.pop("_case", None)
            key = f"{n}/q{k}" + (f"/{variant}" if variant else "")
            grid_mtp[key] = r
            legs.append({"label": f"mtp {key}", "calls": r["calls"], "launches": r["launches"],
                         "steps": r["steps"]})
            log(f"# mtp {key}: cold {r['cold_us_median']:.2f} us, warm {r['warm_us']:.2f} us, "
                f"{r['effective_kv_GBps']:.0f} GB/s KV counted once ({r['pct_hbm_peak_kv']:.1f}% of 8 TB/s), "
                f"plan {r['plan']}")
        args.flags = base_flags
    graph = None
    if not args.no_graph and args.workload not in syn.PAGED:  # the graph leg replays mla_decode (page size 1)
        graph = measure_graph(args.workload, args, dev, flush)
        legs.append({"label": f"graph {args.workload}", "calls": graph["calls"], "launches": graph["launches"],
                     "steps": args.steps})
        log(f"# graph replay {args.workload}: cold {graph['cold_us_median']:.2f} us "
            f"(p10 {graph['cold_us_p10']:.2f}, p90 {graph['cold_us_p90']:.2f})")
    # The pages' whole shape grid and the 8-row-page caches, --sweep-steps calls each.
    sweep = None
    if not args.no_sweep:
        sweep = {}
        for n in list(syn.SWEEP) + list(syn.PAGED):
            r = measure(n, args, dev, flush, steps=args.sweep_steps)
            r.pop("_case", None)
            sweep[n] = r
            legs.append({"label": f"sweep {n}", "calls": r["calls"], "launches": r["launches"], "steps": r["steps"]})
            log(f"# sweep {n}: cold {r['cold_us_median']:.2f} us, warm {r['warm_us']:.2f} us, "
                f"{r['effective_kv_GBps']:.0f} GB/s KV ({r['pct_hbm_peak_kv']:.1f}% of 8 TB/s), plan {r['plan']}")
            torch.cuda.empty_cache()
    head = results[args.workload]
    case = head.pop("_case")
    for r in results.values():
        r.pop("_case", None)

    rf = roofline_of(head)
    traffic = _load_profile_json(TRAFFIC_FILE, args.workload)
    kernel_name = "mla decode call: the stage-1 kernel" + (
        "" if head["launches"] == ["stage1"] else ", then the combine kernel")
    roofline = {
        "bound": "hbm",
        "achieved": rf["call_GBps"],
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": rf["call_frac"],
        "traffic": None if traffic is None else traffic["bytes_per_call"],
        "kernel": kernel_name,
        "launches_per_call": len(head["launches"]),
        "bytes_per_launch": head["algorithmic_bytes"],
        "kernel_frac": rf["kernel_frac"],
        "kernel_time_source": rf["kernel_time_source"],
        "timing": "HIP events on the launch stream, cold cache (1 GiB read flush before each call), mean over steps",
    }
    roofline_grid = {n: roofline_of(r) for n, r in results.items()}
    cpu = None if args.no_cpu_baseline else cpu_baseline(case, args.cpu_seconds)
    ceiling = read_ceiling(dev, flush, head["kv_bytes"])
    log(f"# library streaming read of {ceiling['bytes'] / 1e6:.0f} MB: {ceiling['cold_us_median']:.1f} us, "
        f"{ceiling['GBps']:.0f} GB/s ({100 * ceiling['frac_of_peak']:.1f}% of 8 TB/s)")
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
        "roofline_grid": roofline_grid,
        "hbm_read_ceiling": ceiling,
        "graph_replay": graph,
        "cpu_baseline": cpu,
        "grid": results,
        "grid_q8": grid_q8,
        "grid_mtp": grid_mtp,
        "grid_mixed": grid_mixed,
        "sweep": sweep,
        "legs": legs,
        "kernel_source_hash": source_hash(),
        "argv": " ".join(sys.argv[1:]),
        "host": platform.node(),
    }
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------------------
# --summarise: rocprofv3 outputs -> profiles/
# ---------------------------------------------------------------------------
# Expected layout under DIR (the commands are written into each summary):
#   DIR/trace.log, DIR/trace/run_kernel_trace.csv
#       rocprofv3 --kernel-trace --stats --output-format csv -d DIR/trace -o run -- python3 bench.py <args>
#       (bench.py's JSON line in trace.log lists the measured legs in launch order)
#   DIR/pmc/<workload>_<FETCH_SIZE|WRITE_SIZE>/run_counter_collection.csv (+ .log)
#       rocprofv3 --pmc <counter> --output-format csv -d DIR/pmc/<workload>_<counter> -o run --
#           python3 bench.py --workload <workload> --only-gpu-loop 3
#   DIR/pmc/copy_<FETCH_SIZE|WRITE_SIZE>/run_counter_collection.csv: the copy calibration
#   DIR/pmc/<workload>_sq1, DIR/pmc/<workload>_sq2: the two SQ counter groups, --cold
# Each part is summarised when present. Every bench.py output read must carry the
# current kernel source hash.

SQ_GROUP1 = "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_WAVES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU GRBM_GUI_ACTIVE"
SQ_GROUP2 = ("SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_WAIT_INST_LDS SQ_WAIT_INST_ANY SQ_LDS_BANK_CONFLICT "
             "SQ_INSTS_VALU_CVT SQ_WAVE_CYCLES SQ_ACTIVE_INST_ANY")
COPY_CMD = ("python3 -c \"import torch; a=torch.ones(256<<20,dtype=torch.uint8,device='cuda'); b=torch.empty_like(a); "
            "[b.copy_(a) for _ in range(3)]; torch.cuda.synchronize()\"")


def _short(n):
    return n.replace("void ", "").split("(")[0]


def _kind(n):
    if "mla::split_kernel" in n or "mla::persistent_kernel" in n:
        return "stage1"
    if "mla::combine_kernel" in n:
        return "combine"
    if "mla::q_amax_kernel" in n:
        return "q_amax"
    return None


def _json_line(path):
    with open(path) as f:
        for line in f:
            if line.startswith("{"):
                return json.loads(line)
    raise ValueError(f"{path}: no JSON line")


def _check_hash(path, h):
    got = _json_line(path).get("kernel_source_hash")
    if got != h:
        raise SystemExit(f"{path} was made by kernel build {got}, the source is now {h}: profile again")


def _pct(v, p):
    return sorted(v)[min(len(v) - 1, int(p * len(v)))]


def _summarise_trace(d, h):
    bench = _json_line(os.path.join(d, "trace.log"))
    _check_hash(os.path.join(d, "trace.log"), h)
    with open(os.path.join(d, "trace", "run_kernel_trace.csv")) as f:
        rows = list(csv.DictReader(f))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    by_kind = {k: [r for r in rows if _kind(r["Kernel_Name"]) == k] for k in ("stage1", "combine", "q_amax")}
    pos = {k: 0 for k in by_kind}
    warm = bench["warmup"]
    results = dict(bench["grid"])
    for key, grp in (("grid_q8", "q8 "), ("grid_mixed", "mixed "), ("grid_mtp", "mtp "), ("sweep", "sweep ")):
        for k, v in (bench.get(key) or {}).items():
            results[grp + k] = v
    out = ["# MLA decode kernels: durations under a bench run\n",
           "Command (one MI355X, from the repository root):\n",
           f"    cd /tmp && export TMPDIR=/tmp && cd <repo> && rocprofv3 --kernel-trace --stats --output-format csv "
           f"-d DIR/trace -o run -- python3 bench.py {bench.get('argv', '')}".rstrip() + " > DIR/trace.log",
           "    python3 bench.py --summarise DIR\n",
           f"Kernel source sha256[:16] = `{h}`. Each leg: one checked call, {warm} warm-up calls, its cold calls (each",
           "after a 1 GiB read flush), then as many back-to-back warm calls. Durations are rocprofv3 kernel-dispatch",
           "times (begin to end of each kernel); `call (events)` is bench.py's own HIP-event time of the whole call in",
           "the same profiled run, which adds the gaps between a call's launches. Tracing adds some overhead.\n"]
    times = {}
    for leg in bench["legs"]:
        lab, calls, kinds = leg["label"], leg["calls"], leg["launches"]
        steps = leg["steps"]
        got = {}
        for k in kinds:
            got[k] = by_kind[k][pos[k]:pos[k] + calls]
            if len(got[k]) != calls:
                raise SystemExit(f"trace: leg {lab} has {len(got[k])} {k} dispatches, expected {calls}")
            pos[k] += calls
        if lab.startswith("graph "):
            cold = {k: v[1 + warm:1 + warm + steps] for k, v in got.items()}
            hot = None
        else:
            cold = {k: v[1 + warm:1 + warm + steps] for k, v in got.items()}
            hot = {k: v[1 + warm + steps:1 + warm + 2 * steps] for k, v in got.items()}
        r = results.get(lab)
        out.append(f"## {lab}\n")
        if r is not None:
            out.append(f"Plan: {r['plan']}\n")
        out.append("| kernel | workgroups | LDS B | VGPR | AGPR | scratch | cold calls | cold avg us | cold median | "
                   "cold p10 | cold p90 | warm avg us |")
        out.append("|---|---|---|---|---|---|---|---|---|---|---|---|")
        tot = 0.0
        for k in kinds:
            ks = cold[k]
            k0 = ks[0]
            cd = [(int(x["End_Timestamp"]) - int(x["Start_Timestamp"])) / 1e3 for x in ks]
            wd = [(int(x["End_Timestamp"]) - int(x["Start_Timestamp"])) / 1e3 for x in hot[k]] if hot else None
            tot += statistics.fmean(cd)
            wg = int(k0["Grid_Size_X"]) // int(k0["Workgroup_Size_X"])
            out.append(f"| `{_short(k0['Kernel_Name'])}` | {wg} | {k0['LDS_Block_Size']} | {k0['VGPR_Count']} | "
                       f"{k0['Accum_VGPR_Count']} | {k0['Scratch_Size']} | {len(cd)} | {statistics.fmean(cd):.2f} | "
                       f"{statistics.median(cd):.2f} | {_pct(cd, .1):.2f} | {_pct(cd, .9):.2f} | "
                       f"{statistics.fmean(wd):.2f} |" if wd else " - |")
            if k == "stage1" and r is not None and lab in bench["grid"]:
                times.setdefault(lab, {"source_hash": h, "kernels": {}})
                times[lab]["stage1_cold_avg_us"] = statistics.fmean(cd)
            if lab in bench["grid"]:
                times[lab]["kernels"][_short(k0["Kernel_Name"])] = statistics.fmean(cd)
        line = f"\nSum of the cold kernel averages: {tot:.2f} us"
        if r is not None:
            line += f"; call (events) in the same profiled run: mean {r['cold_us_mean']:.2f} us, " \
                    f"median {r['cold_us_median']:.2f} us"
            if lab in times:
                times[lab]["call_events_mean_us"] = r["cold_us_mean"]
                times[lab]["algorithmic_bytes"] = r["algorithmic_bytes"]
        out.append(line + ".\n")
    with open(os.path.join(PROFILES, "mla_decode_kernels_bench_trace.md"), "w") as f:
        f.write("\n".join(out) + "\n")
    with open(KERNEL_TIMES_FILE, "w") as f:
        json.dump(times, f, indent=1)
    log(f"trace: {len(bench['legs'])} legs summarised")


def _pmc(path, counter):
    dd = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            dd.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return {k: statistics.fmean(v) for k, v in dd.items()}


def _summarise_traffic(d, h):
    import synthetic as syn

    pm = os.path.join(d, "pmc")
    cf = _pmc(os.path.join(pm, "copy_FETCH_SIZE", "run_counter_collection.csv"), "FETCH_SIZE")
    cw = _pmc(os.path.join(pm, "copy_WRITE_SIZE", "run_counter_collection.csv"), "WRITE_SIZE")
    copy_k = [k for k in cf if "copyBuffer" in k][0]
    fill_k = [k for k in cw if "FillFunctor" in k][0]
    fetch_scale, write_scale = 262144.0 / cf[copy_k], 262144.0 / cw[fill_k]
    md = ["# MLA decode: HBM traffic per call from FETCH_SIZE and WRITE_SIZE\n",
          "Commands (one MI355X, from the repository root, one counter per run):\n",
          "    cd /tmp && export TMPDIR=/tmp && cd <repo>",
          "    rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/pmc/<w>_FETCH_SIZE -o run -- "
          "python3 bench.py --workload <w> --only-gpu-loop 3 > DIR/pmc/<w>_FETCH_SIZE.log",
          "    rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/pmc/<w>_WRITE_SIZE -o run -- "
          "python3 bench.py --workload <w> --only-gpu-loop 3 > DIR/pmc/<w>_WRITE_SIZE.log",
          "    python3 bench.py --summarise DIR\n",
          "Calibration: the same two counters on a torch fill and copy of a 256 MiB buffer, 3 copies:\n",
          f"    rocprofv3 --pmc <counter> --output-format csv -d DIR/pmc/copy_<counter> -o run -- {COPY_CMD}\n",
          f"- `{copy_k}`: FETCH_SIZE {cf[copy_k]:.0f} KiB per dispatch for 262144 KiB read -> fetch scale {fetch_scale:.4f}",
          f"- `{fill_k}`: WRITE_SIZE {cw[fill_k]:.0f} KiB per dispatch for 262144 KiB written -> write scale "
          f"{write_scale:.4f}\n",
          f"Kernel source sha256[:16] = `{h}`. Counts are per dispatch, averaged over the dispatches of each kernel (the",
          "run is warm: three back-to-back calls, so this measures what the L2 fetches and writes, wherever it is served",
          "from). Scaled bytes = KiB x 1024 x scale.\n",
          "| workload | kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB |",
          "|---|---|---|---|---|---|"]
    summ, tj = [], {}
    for w in syn.WORKLOADS:
        fp = os.path.join(pm, f"{w}_FETCH_SIZE", "run_counter_collection.csv")
        if not os.path.exists(fp):
            continue
        _check_hash(os.path.join(pm, f"{w}_FETCH_SIZE.log"), h)
        _check_hash(os.path.join(pm, f"{w}_WRITE_SIZE.log"), h)
        f = _pmc(fp, "FETCH_SIZE")
        wr = _pmc(os.path.join(pm, f"{w}_WRITE_SIZE", "run_counter_collection.csv"), "WRITE_SIZE")
        alg = syn.make_workload(w).total_bytes()
        ent = {"source_hash": h, "kernels": {}, "algorithmic_bytes": alg, "fetch_scale": fetch_scale,
               "write_scale": write_scale}
        tot = 0.0
        for k in sorted(k for k in f if k.startswith("mla::")):
            rb, wb = f[k] * 1024 * fetch_scale, wr.get(k, 0.0) * 1024 * write_scale
            ent["kernels"][k] = {"read_bytes": rb, "write_bytes": wb}
            tot += rb + wb
            md.append(f"| {w} | `{k}` | {f[k]:.0f} | {wr.get(k, 0.0):.0f} | {rb / 1e6:.2f} | {wb / 1e6:.2f} |")
        ent["bytes_per_call"] = tot
        tj[w] = ent
        summ.append(f"| {w} | {tot / 1e6:.2f} | {alg / 1e6:.2f} | {tot / alg:.3f} |")
    md += ["", "| workload | traffic per call MB (read + write, all kernels of the call) | algorithmic bytes MB | ratio |",
           "|---|---|---|---|"] + summ
    with open(os.path.join(PROFILES, "mla_decode_hbm_traffic.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(tj, f, indent=1)
    log(f"traffic: {len(tj)} workloads summarised")


def _summarise_sq(d, h):
    import synthetic as syn

    pm = os.path.join(d, "pmc")

    def load(path):
        dd = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if _kind(r["Kernel_Name"]) != "stage1":
                    continue
                e = dd.setdefault(r["Dispatch_Id"], [_short(r["Kernel_Name"]),
                                                     (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3, {}])
                e[2][r["Counter_Name"]] = float(r["Counter_Value"])
        return dd

    rows = []
    for w in syn.WORKLOADS:
        p1 = os.path.join(pm, f"{w}_sq1", "run_counter_collection.csv")
        if not os.path.exists(p1):
            continue
        _check_hash(os.path.join(pm, f"{w}_sq1.log"), h)
        _check_hash(os.path.join(pm, f"{w}_sq2.log"), h)
        a = load(p1)
        b = load(os.path.join(pm, f"{w}_sq2", "run_counter_collection.csv"))
        name = next(iter(a.values()))[0]

        def avg(dd, c):
            return statistics.fmean(v[2][c] for v in dd.values())

        dur = statistics.fmean(v[1] for v in a.values())
        waves = avg(a, "SQ_WAVES")
        cfg = syn.WORKLOADS[w]
        tokens = cfg["batch"] * cfg["kv_lens"]
        mfma_busy = avg(a, "SQ_VALU_MFMA_BUSY_CYCLES") / (1024 * dur * 1e-6 * 2.4e9)
        util = FLOP_PER_TOKEN * tokens / (dur * 1e-6) / 2.5e15
        wc = avg(b, "SQ_WAVE_CYCLES")
        rows.append(
            f"| {w} | `{name}` | {dur:.1f} | {waves:.0f} | {avg(a, 'SQ_INSTS_VALU') / waves:.0f} / "
            f"{avg(a, 'SQ_INSTS_MFMA') / waves:.0f} / {avg(a, 'SQ_INSTS_LDS') / waves:.0f} / "
            f"{avg(a, 'SQ_INSTS_SALU') / waves:.0f} | {avg(b, 'SQ_INSTS_VALU_CVT') / waves:.0f} | {100 * mfma_busy:.1f}% | "
            f"{100 * util:.1f}% | {100 * avg(b, 'SQ_ACTIVE_INST_VALU') / wc:.1f}% | "
            f"{100 * avg(b, 'SQ_WAIT_INST_LDS') / wc:.1f}% | "
            f"{avg(b, 'SQ_LDS_BANK_CONFLICT') / avg(a, 'SQ_INSTS_LDS'):.2f} |")
    md = ["# MLA decode stage-1 kernel: MFMA, VALU and LDS counters (cold calls)\n",
          "Commands (one MI355X, from the repository root, two counter groups, one run each):\n",
          "    cd /tmp && export TMPDIR=/tmp && cd <repo>",
          f"    rocprofv3 --pmc {SQ_GROUP1} --output-format csv -d DIR/pmc/<w>_sq1 -o run -- "
          "python3 bench.py --workload <w> --only-gpu-loop 3 --cold > DIR/pmc/<w>_sq1.log",
          f"    rocprofv3 --pmc {SQ_GROUP2} --output-format csv -d DIR/pmc/<w>_sq2 -o run -- "
          "python3 bench.py --workload <w> --only-gpu-loop 3 --cold > DIR/pmc/<w>_sq2.log",
          "    python3 bench.py --summarise DIR\n",
          f"Kernel source sha256[:16] = `{h}`. Values are averages over the stage-1 dispatches of the run (counter",
          "mode serialises dispatches, so `dur` is a little longer than an unprofiled call). Units:\n",
          "- `SQ_VALU_MFMA_BUSY_CYCLES` counts 16 cycles per `v_mfma_f32_16x16x32_bf16` / fp8 and 32 per",
          "  `v_mfma_scale_f32_16x16x128_f8f6f4`; MFMA pipe busy = that / (1024 SIMDs x dur x 2.4 GHz).",
          "- `SQ_WAVE_CYCLES` and `SQ_ACTIVE_INST_*` count in units of 4 cycles (a wave64 VALU instruction is one",
          "  unit); the VALU and LDS-wait shares are per wave.",
          "- MFMA flop utilisation = 34,816 flop per token x tokens / dur against the 2.5 PFLOP/s dense bf16 peak.\n",
          "| workload | kernel | dur us | waves | VALU / MFMA / LDS / SALU instructions per wave | of which cvt | "
          "MFMA pipe busy | MFMA flop util | VALU active per wave | LDS wait per wave | bank conflicts per LDS "
          "instruction |",
          "|---|---|---|---|---|---|---|---|---|---|---|"] + rows
    with open(os.path.join(PROFILES, "mla_decode_counters_mfma_valu.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    log(f"SQ counters: {len(rows)} workloads summarised")


def summarise(d):
    """Write the profiles/ summaries from the rocprofv3 runs under directory d (layout above)."""
    h = source_hash()
    done = 0
    if os.path.exists(os.path.join(d, "trace", "run_kernel_trace.csv")):
        _summarise_trace(d, h)
        done += 1
    if os.path.exists(os.path.join(d, "pmc", "copy_FETCH_SIZE", "run_counter_collection.csv")):
        _summarise_traffic(d, h)
        done += 1
    if any(n.endswith("_sq1") for n in (os.listdir(os.path.join(d, "pmc")) if os.path.isdir(os.path.join(d, "pmc"))
                                         else [])):
        _summarise_sq(d, h)
        done += 1
    if not done:
        raise SystemExit(f"{d}: no rocprofv3 output found")


if __name__ == "__main__":
    main()
