"""Benchmark: single-token MLA decode on one MI355X.

    python bench.py [--steps K] [--warmup W] [--warmup-ms T] [--workload NAME]
                    [--targets A,B|none] [--cold-calls N] [--no-cpu-baseline]

A step is one decode call (the split kernel, plus the LSE merge kernel when
the plan needs one) over one batch of seeded synthetic inputs already
resident in HBM; the split plan is made once beforehand (plan_us).  The
headline workload is the largest listed one: 256 sequences of 1024-8192
tokens (uniform draw) in an fp8 cache of 2-token pages, shuffled.  Every
timed step is cold: the steps cycle through copies of the inputs totalling
at least 1 GiB, so no step finds its KV in the 256 MB last-level (MALL)
cache.  The `steps` calls run back to back between two events; ms_per_step =
elapsed / steps and value = algorithmic KV bytes / ms_per_step.  Before them,
untimed, at least W calls and then back-to-back calls until T ms (default 60)
have run: after an idle spell the chip holds a lower core clock through the
first ~25 ms of sustained load, and the timed calls are meant to see the clock
it sustains.  "warmup" in the line is the number of warm-up calls made.

Beside that: cold_single_us, the median and the mean without the fastest and
slowest of calls timed one at a time (events around each call, the GPU idle
before it); us_per_call_warm, back-to-back calls on one copy of the inputs;
plan.replan_us, the host time of re-planning the live handle between runs
(plan.replan_loop_us: the same in a plan/run loop that runs ahead of the GPU);
and, under "targets", the same record for 32 and 64 sequences of 8192 tokens
in an fp8 cache (the target shapes).

Algorithmic bytes = tokens x stored bytes per row (bf16 1152, fp8 576, MXFP4
288 + 18 scale bytes); query, output, partials and page ids are overhead.

Prints one JSON line.  Also reports the roofline of the dominant kernel
(stage 1, timed with HIP events recorded by the library around its own launch
on the same stream) and the fp64 oracle timed on the host cores on a
bounded sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
DEFAULT_WORKLOAD = "bs256_ragged1024-8192_fp8_paged2"  # the largest listed workload
# The target shapes (at least 32 sequences of 8192 tokens, fp8 cache), measured in
# the same run and reported under "targets".
TARGETS = ("bs32_kv8192_fp8", "bs64_kv8192_fp8")
ROTATION_BYTES = 1 << 30  # inputs cycled per timed pass: 4x the 256 MB MALL
METRIC = "µs/call and effective KV HBM GB/s (% of peak), MLA decode bs×kv_len"
# Times the pages report for one of these workloads on MI355X (µs per call;
# the page states no unit, µs is the plain reading): submission 727205
# ("v25: LEAN"), the notes at the head of its source, give 244 -> 236.6 for
# its v24 MXFP4 split kernel at 256 sequences x 8192 tokens once iglp_opt
# scheduling was added.  vs_baseline = that time / ours (the same bytes, so
# also our GB/s over the page's).
PAGE_US = {"bs256_kv8192_mxfp4": 236.6}
# Sources of each cache format's split kernel: a traffic record holds for
# them as hashed.
CSRC = os.path.join(ROOT, "latent_attention_decode_amd", "csrc")
KERNEL_SRCS = {
    "fp8": ("mla_stage1_fp8.hip", "mla_device.h", "mla_internal.h"),
    "mxfp4": ("mla_stage1_mxfp4.hip", "mla_device.h", "mla_internal.h"),
    "bf16": ("mla_kernels.hip", "mla_device.h", "mla_internal.h"),
}


def kernel_hash(kv_dtype: str = "fp8") -> str:
    h = hashlib.sha256()
    for name in KERNEL_SRCS[kv_dtype]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_record(workload: str, kv_dtype: str):
    """HBM bytes per stage-1 launch from a committed rocprofv3 --pmc summary,
    if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"stage1_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sha256_16") != kernel_hash(kv_dtype):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(case, budget_s: float = 10.0):
    """The oracle as it stands, on a bounded sample: whole sequences from the
    start of the batch (as many as fit the budget with every thread busy),
    passed over repeatedly until about budget_s of wall time is spent."""
    import oracle
    threads = max(1, len(os.sched_getaffinity(0)))
    t0 = time.perf_counter()
    oracle.decode_case(case, batches=[0], nthreads=1)
    one = max(time.perf_counter() - t0, 1e-4)
    n = int(min(case.batch, max(threads, (budget_s / one) * threads * 0.8)))
    n = max(1, min(n, case.batch))
    batches = list(range(n))
    tokens = int(sum(int(case.lens[b]) for b in batches))
    sample_bytes = tokens * (case.kv_algorithmic_bytes() / case.total_tokens)
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.decode_case(case, batches=batches, nthreads=threads)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or dt / passes * (passes + 1) > 3 * budget_s:
            break
    gbs = sample_bytes * passes / dt / 1e9
    full_us = case.kv_algorithmic_bytes() / (gbs * 1e9) * 1e6
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {case.batch} sequences ({tokens} tokens) x {passes} passes, "
                      f"{dt:.2f} s wall, fp64 C oracle",
            "us_per_call_extrapolated": round(full_us, 1)}


def measure(name, args, dev, torch, binding, synth, full=True):
    """One workload: plan once, then the cold back-to-back pass (steps calls
    between two events), the same calls with the library's kernel events
    (stage-1 and merge durations), individually event-timed cold calls
    (median and the mean without the fastest and slowest), warm calls, and
    the cost of re-planning the live handle."""
    kv_dtype, batch, kv_len, ps, shuffled, seed = synth.CONFIGS[name][:6]
    print(f"[bench] generating {name}", file=sys.stderr, flush=True)
    case = synth.config_case(name)
    base = binding.case_to_device(case, dev)
    out = torch.empty((case.rows, 16, 512), dtype=torch.bfloat16, device=dev)
    alg_bytes = case.kv_algorithmic_bytes()  # the cache once, whatever the query tokens per sequence

    # Cold-cache protocol: consecutive calls read different copies of the
    # inputs (same bytes, other addresses), cycling through at least 1 GiB, so
    # each call finds none of its data in the 256 MB last-level (MALL) cache;
    # no flush kernel and no per-call event sits inside the timed region.
    per_copy = sum(v.numel() * v.element_size() for v in base.values() if v is not None)
    n_copies = max(2, -(-ROTATION_BYTES // per_copy))
    copies = [base] + [{k: (None if v is None else v.clone()) for k, v in base.items()}
                       for _ in range(n_copies - 1)]

    dec = binding.MlaDecode(kv_dtype, ps, device=0)
    if args.query_format != "exact":
        dec.set_query_format(args.query_format)
    t0 = time.perf_counter()
    ws_bytes = dec.plan(case.kv_indptr, case.kv_last_page_len, args.split, case.qo_indptr)
    plan_us = (time.perf_counter() - t0) * 1e6
    n_items, max_splits, n_partials = binding.mla_decode_plan_info(dec.h)
    res1 = binding.mla_decode_kernel_resources(dec.h, 0)

    # Each copy's call is marshalled once (binding.PreparedRun), so that a
    # step costs the host one foreign call and the loop measures the GPU.
    calls = [dec.prepare(t["q"], t["kv"], t["kv_scales"], t["kv_indptr"], out, t["kv_page_indices"],
                         t["kv_last_page_len"]) for t in copies]

    def run(i):
        calls[i % n_copies]()

    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)

    # Untimed warm-up: at least `warmup` calls and one pass over the copies,
    # then back-to-back calls until `warmup_ms` of them have run.  After an
    # idle spell the chip runs the first ~25 ms of back-to-back calls at a
    # lower core clock (1.5-2.0 GHz, against the 2.2-2.4 GHz it then
    # sustains), so the timed region starts once that has passed.
    # The first chunk also pays one-time costs (first launches), so the
    # sustained time is counted from the second chunk on.
    n_warm = 0
    chunk = max(args.warmup, n_copies)
    sustained_ms = -1.0
    while True:
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(chunk):
            run(n_warm + i)
        ev1.record(stream)
        torch.cuda.synchronize()
        dt = ev0.elapsed_time(ev1)
        n_warm += chunk
        sustained_ms = 0.0 if sustained_ms < 0 else sustained_ms + dt
        if sustained_ms >= args.warmup_ms:
            break
        per_call_ms = max(dt / chunk, 1e-3)
        chunk = max(8, int(np.ceil((args.warmup_ms - sustained_ms) / per_call_ms)))

    # Timed region: exactly `steps` calls back to back, each on the next copy.
    print(f"[bench] {name}: timing {args.steps} cold steps over {n_copies} input copies",
          file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        run(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    mean_ms = ev0.elapsed_time(ev1) / args.steps

    # Kernel durations: the same calls again with the library recording HIP
    # events around each of its kernel launches on the same stream (the event
    # packets add their own dispatch latency, so these read slightly long).
    binding.mla_decode_set_profiling(dec.h, True)
    s1_ms, mg_ms = [], []
    for i in range(args.steps):
        run(i)
        s1_ms.append(binding.mla_decode_kernel_time_ms(dec.h, 0))
        mg_ms.append(binding.mla_decode_kernel_time_ms(dec.h, 1))
    binding.mla_decode_set_profiling(dec.h, False)

    # Cold calls one at a time: events around each call, the GPU idle before
    # it, the call's inputs last read n_copies calls earlier.
    single = []
    for i in range(args.cold_calls):
        torch.cuda.synchronize()
        ev0.record(stream)
        run(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        single.append(ev0.elapsed_time(ev1) * 1e3)
    single = np.sort(np.array(single))
    trimmed = float(single[1:-1].mean()) if single.size > 2 else float(single.mean())

    # warm: back-to-back calls on one copy (its KV may sit in the MALL)
    run(0)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.warm_iters):
        run(0)
    ev1.record(stream)
    torch.cuda.synchronize()
    warm_us = ev0.elapsed_time(ev1) / args.warm_iters * 1e3

    # Re-planning the live handle for the same batch, as a decode loop does
    # each step (lengths change by one token): the host time of a plan call
    # with the GPU idle (the planner and the enqueued upload), and in a loop of
    # plan, run, plan, run, ... with runs in flight, where a plan also waits for
    # the run two plans back, whose plan buffer it reuses, whenever the host
    # is that far ahead of the GPU.
    replan, replan_loop = [], []
    t = copies[0]
    for i in range(20):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        dec.plan(case.kv_indptr, case.kv_last_page_len, args.split, case.qo_indptr)
        replan.append((time.perf_counter() - t0) * 1e6)
        dec.run(t["q"], t["kv"], t["kv_scales"], t["kv_indptr"], out, t["kv_page_indices"],
                t["kv_last_page_len"])
    torch.cuda.synchronize()
    for i in range(20):
        t0 = time.perf_counter()
        dec.plan(case.kv_indptr, case.kv_last_page_len, args.split, case.qo_indptr)
        replan_loop.append((time.perf_counter() - t0) * 1e6)
        dec.run(t["q"], t["kv"], t["kv_scales"], t["kv_indptr"], out, t["kv_page_indices"],
                t["kv_last_page_len"])
    torch.cuda.synchronize()

    s1 = np.array(s1_ms)
    value = alg_bytes / (mean_ms * 1e-3) / 1e9
    s1_mean = float(s1.mean())
    achieved = alg_bytes / (s1_mean * 1e-3) / 1e9
    rec = {
        "us_per_call": round(mean_ms * 1e3, 2),
        "gbs": round(value, 2),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "cold_single_us": {"median": round(float(np.median(single)), 2), "trimmed_mean": round(trimmed, 2),
                           "min": round(float(single[0]), 2), "max": round(float(single[-1]), 2),
                           "calls": int(single.size)},
        "us_per_call_warm": round(warm_us, 2),
        "kernels": {"stage1_us": round(s1_mean * 1e3, 2),
                    "merge_us": round(float(np.mean(mg_ms)) * 1e3, 2),
                    "stage1_vgprs": res1["vgprs"], "stage1_lds_bytes": res1["lds_bytes"],
                    "stage1_scratch_bytes": res1["scratch_bytes"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_record(name, kv_dtype) if args.query_format == "exact" else None},
        "plan": {"items": n_items, "max_splits": max_splits, "partials": n_partials,
                 "workspace_bytes": int(ws_bytes), "plan_us": round(plan_us, 1),
                 "replan_us": round(float(np.median(replan)), 1),
                 "replan_loop_us": round(float(np.median(replan_loop)), 1)},
    }
    if full:
        rec["config"] = {"workload": name, "kv_dtype": kv_dtype, "batch": int(case.batch),
                         "query_rows": int(case.rows),
                         "kv_len": kv_len if isinstance(kv_len, int) else list(kv_len),
                         "total_tokens": int(case.total_tokens), "page_size": ps,
                         "query_format": args.query_format, "algorithmic_kv_bytes": int(alg_bytes)}
        rec["input_copies"] = n_copies
        rec["timed_wall_s"] = round(wall, 3)
        rec["mean_ms"] = mean_ms
        rec["kv_dtype"] = kv_dtype
    else:
        rec["algorithmic_kv_bytes"] = int(alg_bytes)
    rec["warmup_calls"] = n_warm
    del calls
    dec.close()
    del copies, base
    torch.cuda.empty_cache()
    return rec, case


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-ms", type=float, default=60.0,
                    help="after the `warmup` calls, keep calling back to back until this much GPU time has run")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--targets", default=",".join(TARGETS),
                    help="comma-separated workloads measured in the same run and reported under "
                         "'targets' ('none' for none)")
    ap.add_argument("--warm-iters", type=int, default=100)
    ap.add_argument("--cold-calls", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--split", type=int, default=0, help="split override (0 = planner)")
    ap.add_argument("--query-format", choices=("exact", "e4m3"), default="exact",
                    help="the query in the scores: exact (e4m3 hi + lo, default) or one e4m3 code per element")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device 5 times (a kernel of known traffic "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this decode path "
              "shards by sequence with no exchange, so run one process per GPU.", file=sys.stderr)
        sys.exit(2)

    import torch
    from latent_attention_decode_amd import binding, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), flush=True)
        return

    name = args.workload
    rec, case = measure(name, args, dev, torch, binding, synth, full=True)
    kv_dtype = rec.pop("kv_dtype")
    mean_ms = rec.pop("mean_ms")
    line = {
        "metric": METRIC,
        "value": rec["gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": rec.pop("warmup_calls"),
        "ms_per_step": round(mean_ms, 5),
        "us_per_call": rec["us_per_call"],
        "input_copies": rec["input_copies"],
        "cold_single_us": rec["cold_single_us"],
        "us_per_call_warm": rec["us_per_call_warm"],
        "pct_of_hbm_peak": rec["pct_of_hbm_peak"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(PAGE_US[name] / (mean_ms * 1e3), 3) if name in PAGE_US else None,
        "dtype": {"bf16": "bf16 (bf16 MFMA, fp32 acc)",
                  "fp8": "fp8-e4m3 (fp8 / MX MFMA on the codes, fp32 acc)",
                  "mxfp4": "mxfp4 (MX MFMA: e2m1 scores, e4m3 values, fp32 acc)"}[kv_dtype],
        "data": "synthetic",
        "config": rec["config"],
        "plan": rec["plan"],
        "kernels": rec["kernels"],
        "roofline": rec["roofline"],
        "timed_wall_s": rec["timed_wall_s"],
    }
    targets = [t for t in args.targets.split(",") if t and t != "none" and t != name]
    if targets:
        line["targets"] = {}
        for t in targets:
            sub, _ = measure(t, args, dev, torch, binding, synth, full=False)
            line["targets"][t] = sub
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(case)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
