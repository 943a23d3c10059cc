#!/usr/bin/env python3
"""Benchmark of the MI355X mixed-precision partial-sum reduce (one GPU).

A step is one ``ar_reduce`` call over one batch of synthetic input: the
prefill-shaped reduce of R=2 fp32 partials [2048 x 4096] through a bf16 wire
into an fp32 destination, CHUNKED schedule with 4 MiB chunks (validation,
plan, load, cast-to-wire, ordered fp32 fold, store -- all in one launch).
Inputs are resident in HBM before the timed region and rotate over several
sets so that the 256 MiB Infinity Cache cannot serve them.

Before the timed steps: the ceiling kernels over the same buffers (reported),
the warmup steps, and three lead-in calls (reported).  The K timed steps lie
between two HIP events on the launch stream.  Afterwards: per-step times in a
pass of their own, parity against the oracle, the oracle's own throughput on
the host cores, decode-size latency (fp32 and bf16 wire), and the other
configurations beside their own ceilings (skipped with --quick).

Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--sets S]
                    [--no-cpu-baseline] [--no-decode] [--quick]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic_prefill_bf16.json")
CSRC = os.path.join(ROOT, "mixed_precision_partial_amd", "csrc")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class HipEvent:
    """A HIP event created with hipEventDisableSystemFence, recorded on a given
    stream.  HIP's own documentation gives this flag for events that only
    measure time: recording it skips the system-scope cache writeback and
    invalidation that a default event performs, which on this part costs
    ~2.6 us per event (measured: an empty interval between two default events
    reads 4.3-7.3 us, between two of these 3.2 us) and would otherwise sit
    inside every timed interval.  Uses the HIP runtime torch has loaded."""

    FLAG_DISABLE_SYSTEM_FENCE = 0x20000000
    _hip = None

    def __init__(self):
        import ctypes

        if HipEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so.7")   # the runtime already loaded by torch
            vp = ctypes.c_void_p
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [vp, vp]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
            hip.hipEventDestroy.argtypes = [vp]
            HipEvent._hip = hip
        self._ct = ctypes
        self.h = ctypes.c_void_p()
        rc = HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.h), self.FLAG_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream) -> None:
        rc = HipEvent._hip.hipEventRecord(self.h, self._ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, end: "HipEvent") -> float:
        """Milliseconds from this event to `end` (both complete: call after a synchronize)."""
        f = self._ct.c_float()
        rc = HipEvent._hip.hipEventElapsedTime(self._ct.byref(f), self.h, end.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(f.value)

    def __del__(self):
        if HipEvent._hip is not None and self.h:
            HipEvent._hip.hipEventDestroy(self.h)


def timed_us(torch, stream, fn, reps: int, lead: int = 1) -> float:
    """Mean microseconds per call of `fn(k)` over `reps` back-to-back calls on
    `stream`, between two HipEvents.  `lead` untimed calls are enqueued just
    before the start event so that the GPU queue is not empty when it is
    reached (otherwise the first timed call's host-side enqueue lands inside
    the interval)."""
    torch.cuda.synchronize()
    for k in range(lead):
        fn(k)
    a, b = HipEvent(), HipEvent()
    a.record(stream)
    for k in range(reps):
        fn(lead + k)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_ms(b) * 1e3 / reps


def code_tokens(text: str) -> str:
    """C/C++ source text without its comments, whitespace runs collapsed to one space: what
    the compiler sees, so that an edited comment does not count as a changed kernel.  String
    and character literals are kept verbatim (a "//" inside one is not a comment)."""
    out = []
    i, n = 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of every device-code source of the reduce library (the kernel templates and their
    instance files; the benchmark's own ceiling kernels are not part of it), over the code
    tokens only: comments and layout do not change it."""
    import glob

    h = hashlib.sha256()
    paths = glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h"))
    for path in sorted(p for p in paths if os.path.basename(p) != "bench_ceiling.hip"):
        with open(path, encoding="utf-8") as fh:
            h.update(os.path.basename(path).encode() + b"\0" + code_tokens(fh.read()).encode())
    return h.hexdigest()[:16]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measured_traffic(algo_bytes: int):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when absent or taken on a different kernel source."""
    try:
        with open(PROFILE_TRAFFIC) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return int(t["hbm_bytes_per_launch"])


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--sets", type=int, default=8, help="rotated input/output sets (>= 6 defeats the MALL)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--quick", action="store_true",
                   help="skip the other configurations (slice + broadcast, R=8 from HBM and from host memory, "
                        "residual, narrow and row-strided forms) that the default run also measures")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--summarize-trace", metavar="DIR",
                   help="write profiles/ summary of a rocprofv3 --kernel-trace --stats output dir")
    p.add_argument("--summarize-pass-trace", metavar="DIR",
                   help="the same for a traced --profile-pass of the prefill reduce (the prefill's own "
                        "summary describes the traced default run), written as "
                        "profiles/kernel_trace_prefill_bf16_profile_pass.md")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="write profiles/ HBM-traffic summary from two rocprofv3 --pmc runs "
                        "(FETCH_SIZE, WRITE_SIZE) of --profile-pass")
    p.add_argument("--timing-study", action="store_true",
                   help="instead of the benchmark: how the timing method changes a 20-step figure of the prefill "
                        "reduce (default events vs fence-free events, with and without a lead-in call, the cost "
                        "of an empty event interval, and the first steps after the GPU idled); one JSON line")
    p.add_argument("--family-study", action="store_true",
                   help="instead of the benchmark: the prefill call, plain and with an element-wise or a "
                        "4096-element broadcast-row residual, on the automatically chosen kernel against the "
                        "register- and LDS-staged general kernels and against the hardware's workgroup "
                        "placement, interleaved in one process (bit-identical outputs checked); one JSON line")
    p.add_argument("--hold-study", action="store_true",
                   help="instead of the benchmark: the two-rank calls (prefill plain / residual / row and the "
                        "row-strided block) and three general-kernel calls (cfg 4, the bf16 -> bf16 prefill "
                        "shape, R = 8 fp32) by occupancy hold, interleaved in one process (bit-identical "
                        "outputs checked); one JSON line")
    p.add_argument("--size-study", action="store_true",
                   help="instead of the benchmark: the prefill call's reduce and its 2 : 1 ceiling kernel at "
                        "n = 2^20 ... 2^26 elements, with a fitted fixed per-call cost and streaming rate; "
                        "one JSON line")
    p.add_argument("--summarize-footprint", metavar="ROOT",
                   help="write profiles/counters_prefill_footprint.md from the FOOTPRINT_PASSES runs and "
                        "kernel traces under ROOT (8 and 16 rotated sets)")
    p.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                   help="write profiles/counters_<workload>.md from the rocprofv3 --pmc runs of COUNTER_PASSES")
    p.add_argument("--profile-pass", action="store_true",
                   help="short run for hardware-counter collection: a few reduce steps, then a "
                        "plain elementwise copy of known size used to calibrate the counters")
    p.add_argument("--profile-workload", default="prefill_bf16", choices=sorted(PROFILE_CASES),
                   help="configuration the profile pass runs and the summaries describe")
    return p.parse_args()


# untimed calls enqueued right before the timed region's start event
LEAD_IN_CALLS = 3


def main() -> int:
    args = parse()
    if (args.summarize_trace or args.summarize_pass_trace or args.summarize_pmc or args.summarize_counters or
            args.summarize_footprint):
        if args.summarize_footprint:
            summarize_footprint(args.summarize_footprint)
        if args.summarize_trace:
            summarize_trace(args.summarize_trace, args.profile_workload)
        if args.summarize_pass_trace:
            summarize_trace(args.summarize_pass_trace, "prefill_bf16", bench_run=False)
        if args.summarize_pmc:
            summarize_pmc(*args.summarize_pmc, args.profile_workload)
        if args.summarize_counters:
            summarize_counters(args.summarize_counters, args.profile_workload)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the reduce is run with every "
              "rank simulated on a single MI355X, so there is no multi-GPU figure", file=sys.stderr)
        return 2

    import torch

    import mixed_precision_partial_amd as ar
    import workloads as wl

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    ar.load_library()   # fails loudly when the HIP library was not built
    if args.profile_pass:
        return profile_pass(torch, ar, wl, args)
    if args.timing_study:
        return timing_study(torch, ar, wl, args)
    if args.family_study:
        return family_study(torch, ar, wl, args)
    if args.hold_study:
        return hold_study(torch, ar, wl, args)
    if args.size_study:
        return size_study(torch, ar, wl, args)
    w = wl.WORKLOADS["prefill_bf16"]
    R, n = w.R, w.n
    S = max(1, args.sets)

    log(f"generating {S} sets of R={R} x n={n} fp32 partials")
    host_sets = [wl.partials(w, s) for s in range(S)]
    dev_src = [[torch.from_numpy(p).cuda() for p in srcs] for srcs in host_sets]
    dev_dst = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(S)]
    torch.cuda.synchronize()

    ctx = ar.ar_init(0)
    mode = ar.AR_MODE_CHUNKED
    rc, plan = ar.ar_plan_query([dev_dst[0]], dev_src[0], n, ar.AR_F32, w.wire, mode)
    assert rc == ar.AR_OK
    algo_bytes = int(plan.algo_bytes)
    stream = torch.cuda.current_stream()

    def step(k: int) -> None:
        s = k % S
        ar.ar_reduce(ctx, [dev_dst[s]], dev_src[s], n, ar.AR_F32, w.wire, mode, stream=stream)

    # Reported measurement before the timed steps: the achievable ceilings of
    # this call's access pattern on the same rotated buffers (plain 16-byte
    # copy and 2-read / 1-write kernels of the benchmark's own, and the
    # runtime's device-to-device copy).  It also brings the GPU out of its idle
    # clocks, which a cold start costs (measured: the first 20 steps after 1 s
    # idle ran at 20.2 us/step, the next 20 at 16.1).
    ceil = ceilings(torch, stream, dev_src, dev_dst, n, S)

    log(f"warmup {args.warmup} steps")
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    # LEAD_IN_CALLS more untimed calls, enqueued just before the start event
    # (reported as lead_in_calls): the timed calls then find the GPU busy, so the
    # interval holds K whole calls -- host path and kernel -- and not also an idle
    # gap before the first ones reach the queue.  After the synchronize the host
    # can be slow to start (the first timed call's enqueue measured up to 20 us,
    # the second 9 us, then 6-7 us, on one box), longer than one call of queued
    # GPU work (15 us).
    log(f"timing {args.steps} steps ({LEAD_IN_CALLS} lead-in calls)")
    start, end = HipEvent(), HipEvent()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(LEAD_IN_CALLS):
        step(args.warmup + k)
    host_t = [0.0] * (args.steps + 1)
    start.record(stream)
    host_t[0] = time.perf_counter()
    for k in range(args.steps):
        step(args.warmup + LEAD_IN_CALLS + k)
        host_t[k + 1] = time.perf_counter()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_ms(end)
    ms_per_step = ms_total / args.steps
    gbs = algo_bytes / (ms_per_step * 1e-3) / 1e9
    enqueue_us = [round((host_t[i + 1] - host_t[i]) * 1e6, 2) for i in range(args.steps)]
    log(f"{ms_per_step * 1e3:.3f} us/step, {gbs:.1f} GB/s effective (wall {wall:.4f} s); host enqueue per "
        f"step: median {np.median(enqueue_us):.2f} us, max {max(enqueue_us):.2f} us")

    # Per-step times, in a pass of their own after the timed one (an event
    # between every two steps adds its own cost to each step, so these are
    # not the timed figure): the same K steps, each between two events.
    per_step = per_step_times(torch, stream, step, args.steps)
    log("per-step us (own pass, an event between steps): " + " ".join(f"{x:.2f}" for x in per_step))

    # parity of the timed path on set 0 against the oracle (outside the timed region)
    parity = None
    cpu_baseline = None
    if not args.no_cpu_baseline:
        import oracle

        step(0)
        torch.cuda.synchronize()
        got = dev_dst[0].cpu().numpy()
        log("oracle on one full set (parity of the timed path)")
        t = time.perf_counter()
        want = oracle.reduce(host_sets[0], w.wire)[0]
        one = time.perf_counter() - t
        parity = "bit-exact" if np.array_equal(got.view(np.uint32), want.view(np.uint32)) else "MISMATCH"
        reps = max(1, int(args.cpu_seconds / max(one, 1e-3)))
        log(f"cpu baseline: oracle x{reps} (one call {one:.3f} s)")
        t = time.perf_counter()
        for _ in range(reps):
            oracle.reduce(host_sets[0], w.wire)
        cpu_s = time.perf_counter() - t
        # the same oracle on T host threads, each over its own contiguous element range
        # (the C oracle runs with the interpreter lock released)
        from concurrent.futures import ThreadPoolExecutor

        T = max(1, min(16, os.cpu_count() or 1))
        bounds = [(n * k // T, n * (k + 1) // T) for k in range(T)]
        mt_reps = max(1, min(reps, int(args.cpu_seconds / 2 / max(one / T, 1e-3))))
        with ThreadPoolExecutor(max_workers=T) as pool:
            t = time.perf_counter()
            for _ in range(mt_reps):
                list(pool.map(lambda b: oracle.reduce([x[b[0]:b[1]] for x in host_sets[0]], w.wire), bounds))
            mt_s = time.perf_counter() - t
        cpu_baseline = {
            "value": round(algo_bytes * reps / cpu_s / 1e9, 3),
            "unit": "GB/s",
            "cores": 1,
            "kind": "oracle",
            "cpu_model": cpu_model(),
            "host_cores_visible": os.cpu_count(),
            "all_threads": {"value": round(algo_bytes * mt_reps / mt_s / 1e9, 3), "threads": T,
                            "sample": f"{mt_reps} full calls split over {T} threads"},
            "sample": f"{reps + 1} full calls of the same 2048x4096 R=2 bf16-wire reduce "
                      f"({cpu_s + one:.1f} s, single-threaded scalar C oracle)",
            "decode_us_per_call": oracle_decode_latency(oracle, wl),
        }

    extras = {"ceilings_prefill_size": ceil}
    best_2r1w = max(v for k, v in ceil.items() if k.startswith("kernel_2r1w"))
    extras["value_over_ceiling_2r1w"] = round(gbs / best_2r1w, 4)
    extras["timing"] = {
        "method": "HIP events created with hipEventDisableSystemFence, recorded on the launch stream",
        "lead_in_calls": LEAD_IN_CALLS,
        "host_enqueue_us_per_step": enqueue_us,
        "per_step_us_separate_pass": [round(x, 3) for x in per_step],
        "before_timed_steps": "ceiling kernels over the same rotated buffers (reported in "
                              "ceilings_prefill_size), then the warmup steps, then the lead-in calls",
    }
    if not args.no_decode:
        extras["decode_f32"] = decode_latency(torch, ar, wl, "decode_f32", floors=False)
        extras["decode_bf16"] = decode_latency(torch, ar, wl)
    if not args.quick:
        extras.update(other_schedules(torch, ar, wl))

    traffic = measured_traffic(algo_bytes)
    torch.cuda.synchronize()
    ar.ar_free(ctx)

    result = {
        "metric": "effective GB/s and % of HBM peak (prefill reduce); us/call (decode-size)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "prefill reduce: R=2 fp32 partials [2048x4096] N(0,1)+0.1% x100 outliers, "
                        "bf16 wire, fp32 dst, CHUNKED 4 MiB chunks",
            "R": R, "n": n, "wire": "bf16", "dst": "f32", "rotated_sets": S,
            "algo_bytes_per_step": algo_bytes,
        },
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": cpu_baseline,
        "parity": parity,
        "extras": extras,
    }
    print(json.dumps(result), flush=True)
    if parity == "MISMATCH":
        log("the timed path's output differs from the oracle: failing the run")
        return 3
    return 0


CALIBRATION_BYTES = 64 << 20   # read and written once per calibration launch
# the prefill reduce's kernel instance: the two-rank contiguous kernel, bf16 wire
# (two fp32 sources, one fp32 destination, no residual)
REDUCE_KERNEL = "k_pair<2>"


def _plain_name(name: str) -> str:
    return name.replace("(anonymous namespace)::", "").replace("mpp::", "").replace(" ", "")


def is_reduce_kernel(name: str) -> bool:
    return _plain_name(REDUCE_KERNEL) in _plain_name(name)


def is_library_kernel(name: str) -> bool:
    """Any kernel of the reduce library (every streaming and single-shot instance)."""
    plain = _plain_name(name)
    return "k_stream_" in plain or "k_single_shot" in plain or "k_pair" in plain or "k_few" in plain


CALIBRATION_KERNEL = "neg_kernel"   # torch.neg, the calibration copy (other elementwise kernels may run)

# Configurations a profile pass can run: ranks, elements, wire type, schedule,
# source element bytes, destinations, rotated sets, and whether the sources sit
# in pinned host memory (read by the kernel through their device mapping).
PROFILE_CASES = {
    "prefill_bf16": dict(R=2, n=2048 * 4096, wire="bf16", mode="chunked", src_bytes=4, n_dst=1, sets=8,
                         host=False, what="prefill reduce: R=2 fp32 partials [2048x4096], bf16 wire, CHUNKED"),
    "prefill_bf16_one_set": dict(R=2, n=2048 * 4096, wire="bf16", mode="chunked", src_bytes=4, n_dst=1,
                                 sets=1, host=False,
                                 what="prefill reduce without rotation (one input set, MALL-resident)"),
    "prefill_bf16_16_sets": dict(R=2, n=2048 * 4096, wire="bf16", mode="chunked", src_bytes=4, n_dst=1,
                                 sets=16, host=False,
                                 what="prefill reduce over 16 rotated sets (1.5 GiB touched; run with --sets 16)"),
    "slice_bcast_f16": dict(R=4, n=2048 * 8192, wire="f16", mode="rs_bcast", src_bytes=4, n_dst=4, sets=2,
                            host=False, what="slice + broadcast: R=4 fp32 partials [2048x8192], fp16 wire, "
                                             "4 destinations, RS_BCAST"),
    "r8_hbm_bf16": dict(R=8, n=8192 * 8192, wire="bf16", mode="chunked", src_bytes=4, n_dst=1, sets=1,
                        host=False, what="R=8 fp32 partials [8192x8192] in HBM, bf16 wire, CHUNKED"),
    "r8_hbm_bf16_src": dict(R=8, n=8192 * 8192, wire="bf16", mode="chunked", src_bytes=2, n_dst=1, sets=1,
                            host=False, what="R=8 bf16 partials [8192x8192] in HBM (AR_SRC_WIRE), CHUNKED"),
    "r8_host_direct_bf16": dict(R=8, n=8192 * 8192, wire="bf16", mode="host_staged", src_bytes=2, n_dst=1,
                                sets=1, host=True,
                                what="R=8 bf16 partials [8192x8192] in pinned host memory, HOST_STAGED, "
                                     "kernel reads them directly over PCIe"),
    # the adjacent forms: residual add, narrow destination, row-strided view
    "prefill_residual": dict(R=2, n=2048 * 4096, wire="bf16", mode="chunked", src_bytes=4, n_dst=1, sets=4,
                             host=False, res="elementwise",
                             what="prefill reduce + element-wise fp32 residual (CHUNKED)"),
    "prefill_row_residual": dict(R=2, n=2048 * 4096, wire="bf16", mode="chunked", src_bytes=4, n_dst=1, sets=8,
                                 host=False, res=4096,
                                 what="prefill reduce + broadcast row of 4096 (CHUNKED)"),
    "prefill_bf16_dst": dict(R=2, n=2048 * 4096, wire="bf16", mode="chunked", src_bytes=2, n_dst=1, sets=8,
                             host=False, dst_bytes=2,
                             what="prefill shape, bf16 partials into a bf16 destination (CHUNKED)"),
    "slice_bcast_f16_dst": dict(R=4, n=2048 * 8192, wire="f16", mode="rs_bcast", src_bytes=2, n_dst=4, sets=4,
                                host=False, dst_bytes=2,
                                what="slice + broadcast: R=4 fp16 partials [2048x8192] into 4 fp16 "
                                     "destinations, RS_BCAST"),
    "slice_bcast_f16_residual": dict(R=4, n=2048 * 8192, wire="f16", mode="rs_bcast", src_bytes=4, n_dst=4,
                                     sets=2, host=False, res="elementwise",
                                     what="slice + broadcast to 4 destinations + element-wise fp32 residual"),
    "prefill_r4_one_inactive": dict(R=4, n=2048 * 4096, wire="bf16", mode="chunked", src_bytes=4, n_dst=1, sets=4,
                                    host=False, inactive=(2,),
                                    what="4 ranks on the prefill shape, rank 2 inactive (+0.0), CHUNKED"),
    "rows_prefill_block_bias": dict(R=2, n=2048 * 4096, wire="bf16", mode="chunked", src_bytes=4, n_dst=1,
                                    sets=6, host=False, res=4096, rows=(2048, 4096, 4608, 4352),
                                    what="row-strided prefill block (2048 x 4096 in rows of 4608 / 4352) "
                                         "+ bias row"),
}


def case_algo_bytes(case: dict) -> int:
    db = case.get("dst_bytes", 4)
    res = case.get("res")
    res_b = 0 if res is None else (case["n"] if res == "elementwise" else res) * db
    active = case["R"] - len(case.get("inactive", ()))   # an inactive rank is not read
    return active * case["n"] * case["src_bytes"] + case["n_dst"] * case["n"] * db + res_b


TRACE_CMD = "cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o trace -- python3 /root/repo/bench.py"
TRACE_PASS_CMD = ("cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o trace -- "
                  "python3 /root/repo/bench.py --profile-pass --profile-workload {wl}")
PMC_CMD = ("cd /tmp && rocprofv3 --pmc {counter} --output-format csv -d <dir> -o {tag} -- "
           "python3 /root/repo/bench.py --profile-pass{extra}")


def _csv_rows(directory: str, suffix: str):
    import csv
    import glob

    files = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    with open(files[0]) as fh:
        return list(csv.DictReader(fh))


def _dispatch_rows(directory: str):
    """Per-dispatch records of a rocprofv3 --kernel-trace output (kernel name, start and
    end timestamps in ns, grid size in work-items)."""
    try:
        return _csv_rows(directory, "kernel_trace.csv")
    except FileNotFoundError:
        return []


def prefill_grid_items(n: int) -> int:
    """Work-items of the prefill call's launch: one 64-lane wave per 512-element wave tile
    (the two-rank kernel's one-wave workgroups, the remainder in one more wave)."""
    return (n + 511) // 512 * 64


def _short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("mpp::", "").replace("|", "/")
    return name if len(name) <= 90 else name[:87] + "..."


def summarize_trace(directory: str, wl: str = "prefill_bf16", bench_run: bool | None = None) -> None:
    """profiles/kernel_trace_<wl>.md from a rocprofv3 kernel-trace directory: the traced
    default bench run for the prefill reduce, a traced --profile-pass otherwise
    (``bench_run=False`` for a profile pass of the prefill reduce, written under its
    own name)."""
    case = PROFILE_CASES[wl]
    bench_run = wl == "prefill_bf16" if bench_run is None else bench_run
    rows = _csv_rows(directory, "kernel_stats.csv")
    name = wl if bench_run or wl != "prefill_bf16" else f"{wl}_profile_pass"
    out = os.path.join(ROOT, "profiles", f"kernel_trace_{name}.md")
    if bench_run:
        title = "# rocprofv3 kernel trace: bench.py default run (prefill reduce + decode calls)"
        cmd = TRACE_CMD
    else:
        title = f"# rocprofv3 kernel trace: profile pass of {case['what']}"
        cmd = TRACE_PASS_CMD.format(wl=wl)
    lines = [title, "", f"Command: `{cmd}`", "",
             "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows[:8]:
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                     f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} | {float(r['Percentage']):.1f} |")
    algo = case_algo_bytes(case)
    if bench_run:
        # the default run also launches the same kernel for decode-sized calls and a 768 MiB
        # call: the prefill call's own dispatches are those of its grid, taken from the
        # per-dispatch records of the same trace
        grid = prefill_grid_items(case["n"])
        disp = [r for r in _dispatch_rows(directory)
                if is_reduce_kernel(r["Kernel_Name"]) and int(r["Grid_Size_X"]) == grid]
        if disp:
            dur = np.array([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in disp])
            avg_us = float(dur.mean())
            lines += ["", f"Prefill reduce kernel `{REDUCE_KERNEL}` at the prefill call's grid ({grid} work-items): "
                          f"{dur.size} dispatches, average {avg_us:.3f} us (median {float(np.median(dur)):.3f}, "
                          f"min {float(dur.min()):.3f}, max {float(dur.max()):.3f}) = "
                          f"{algo / avg_us / 1e3:.1f} GB/s of algorithmic bytes ({algo} B per launch). The "
                          f"table's row for the kernel also holds its decode-sized and 768 MiB calls."]
    else:
        ours = [r for r in rows if is_library_kernel(r["Name"])]
        if ours:
            top = max(ours, key=lambda r: float(r["TotalDurationNs"]))
            avg_us = float(top["AverageNs"]) / 1e3
            lines += ["", f"Reduce kernel `{_short(top['Name'])}`: average {avg_us:.3f} us per launch = "
                          f"{algo / avg_us / 1e3:.1f} GB/s of algorithmic bytes ({algo} B per launch: "
                          f"{case['R'] - len(case.get('inactive', ()))} x {case['n']} x {case['src_bytes']} B read, "
                          f"{case['n_dst']} x "
                          f"{case['n']} x {case.get('dst_bytes', 4)} B written"
                          + ("" if case.get("res") is None else
                             f", residual {case['res'] if case['res'] != 'elementwise' else case['n']} x "
                             f"{case.get('dst_bytes', 4)} B read") + ")."]
            if case["host"]:
                host_b = case["R"] * case["n"] * case["src_bytes"]
                lines += ["", f"The sources cross PCIe: {host_b} B read from pinned host memory per launch = "
                              f"{host_b / avg_us / 1e3:.1f} GB/s host-to-device."]
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(out)


# Further counter passes, each within one pass's hardware limits (at most 4 TCC,
# 4 TCP, 2 TA, 2 TD, 8 SQ and 2 GRBM counters), for locating where a kernel's
# time goes beyond its byte counts.
COUNTER_PASSES = {
    "l2": "TCC_HIT_sum TCC_MISS_sum TCC_REQ_sum",
    "l2_mem": "TCC_EA0_RDREQ_sum TCC_EA0_WRREQ_sum TCC_TAG_STALL_sum TCC_BUSY_sum",
    "core": "TCP_TCC_READ_REQ_LATENCY_sum TCP_TCC_READ_REQ_sum TA_TA_BUSY_sum TD_TD_BUSY_sum SQ_WAVE_CYCLES "
            "SQ_BUSY_CYCLES SQ_WAIT_INST_ANY SQ_INSTS_VMEM_RD GRBM_GUI_ACTIVE",
}
COUNTER_CMD = ("cd /tmp && rocprofv3 --pmc {counters} --output-format csv -d <dir> -o {tag} -- "
               "python3 /root/repo/bench.py --profile-pass --profile-workload {wl}")


# Counter passes that compare the prefill call at two footprints (the default 8
# rotated sets, 768 MiB touched per cycle, and 16 sets, 1.5 GiB): per-CU address
# translation (UTCL1) and the shared translation cache's activity, and the L2's
# memory requests.  Each pass, and a kernel trace, runs once per footprint.
FOOTPRINT_PASSES = {
    "utcl": "TCP_UTCL1_TRANSLATION_MISS_sum TCP_UTCL1_TRANSLATION_HIT_sum TCP_UTCL1_REQUEST_sum "
            "TCP_UTCL1_PERMISSION_MISS_sum",
    "utcl_stall": "TCP_CLIENT_UTCL1_INFLIGHT_sum TCP_UTCL1_TRANSLATION_MISS_UNDER_MISS_sum "
                  "TCP_UTCL1_STALL_MULTI_MISS_sum TCP_UTCL1_STALL_UTCL2_REQ_OUT_OF_CREDITS_sum GRBM_UTCL2_BUSY "
                  "GRBM_GUI_ACTIVE",
    "dram": "TCC_EA0_RDREQ_DRAM_sum TCC_EA0_RDREQ_sum TCC_EA0_WRREQ_DRAM_sum TCC_EA0_WRREQ_sum "
            "TCP_UTCL1_STALL_INFLIGHT_MAX_sum TCP_UTCL1_STALL_LRU_INFLIGHT_sum TCP_UTCL1_THRASHING_STALL_sum "
            "TCP_UTCL1_LFIFO_FULL_sum",
}
FOOTPRINT_SETS = {8: "prefill_bf16", 16: "prefill_bf16_16_sets"}
FOOTPRINT_CMD = ("cd /tmp && rocprofv3 {what} --output-format csv -d <root>/{tag}{sets} -o {tag} -- "
                 "python3 /root/repo/bench.py --profile-pass --profile-workload {wl} --sets {sets}")


def summarize_footprint(root: str) -> str:
    """profiles/counters_prefill_footprint.md from <root>/<pass><sets> directories
    (FOOTPRINT_PASSES and a kernel trace "trace", for 8 and 16 sets): the prefill
    kernel's per-dispatch counters and traced duration at both footprints."""
    vals = {}
    for sets in FOOTPRINT_SETS:
        for tag in FOOTPRINT_PASSES:
            for r in _csv_rows(os.path.join(root, f"{tag}{sets}"), "counter_collection.csv"):
                if is_reduce_kernel(r["Kernel_Name"]):
                    vals.setdefault(r["Counter_Name"], {}).setdefault(sets, []).append(float(r["Counter_Value"]))
    durs = {}
    for sets in FOOTPRINT_SETS:
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
             for r in _dispatch_rows(os.path.join(root, f"trace{sets}")) if is_reduce_kernel(r["Kernel_Name"])]
        if not d:
            raise RuntimeError(f"no prefill dispatches in {root}/trace{sets}")
        durs[sets] = (sum(d) / len(d), len(d))
    if not vals:
        raise RuntimeError(f"no prefill dispatches in the counter passes under {root}")
    lines = ["# Prefill reduce at two footprints: 8 rotated sets (768 MiB touched) against 16 (1.5 GiB)", "",
             "Commands (one per footprint; `{sets}` 8 with workload `prefill_bf16`, 16 with "
             "`prefill_bf16_16_sets`):", ""]
    lines.append(f"- `{FOOTPRINT_CMD.format(what='--kernel-trace --stats', tag='trace', sets='{sets}', wl='<workload>')}`")
    for tag, counters in FOOTPRINT_PASSES.items():
        lines.append(f"- `{FOOTPRINT_CMD.format(what='--pmc ' + counters, tag=tag, sets='{sets}', wl='<workload>')}`")
    lines += ["", f"Kernel `{REDUCE_KERNEL}`; kernel source hash {kernel_source_hash()}.", "",
              "| per dispatch (mean) | 8 sets | 16 sets | 16 / 8 |", "|---|---|---|---|"]
    a, b = durs[8][0], durs[16][0]
    lines.append(f"| traced duration, us ({durs[8][1]} / {durs[16][1]} dispatches) | {a:.3f} | {b:.3f} | {b / a:.3f} |")
    for c in sorted(vals):
        v8, v16 = vals[c].get(8), vals[c].get(16)
        if not v8 or not v16:
            continue
        m8, m16 = sum(v8) / len(v8), sum(v16) / len(v16)
        ratio = f"{m16 / m8:.3f}" if m8 else "—"
        lines.append(f"| {c} | {m8:.1f} | {m16:.1f} | {ratio} |")
    out = os.path.join(ROOT, "profiles", "counters_prefill_footprint.md")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(out)
    return out


def summarize_counters(dirs: list, wl: str) -> None:
    """profiles/counters_<wl>.md: per-dispatch averages of the COUNTER_PASSES counters
    for the reduce kernel of a profile pass (one directory per pass, in order)."""
    case = PROFILE_CASES[wl]
    match = is_reduce_kernel if wl == "prefill_bf16" else is_library_kernel
    vals, names = {}, set()
    for d in dirs:
        for r in _csv_rows(d, "counter_collection.csv"):
            if match(r["Kernel_Name"]):
                names.add(_short(r["Kernel_Name"]))
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not vals:
        raise RuntimeError(f"no reduce-kernel dispatches in {dirs}")
    out = os.path.join(ROOT, "profiles", f"counters_{wl}.md")
    lines = [f"# Hardware counters of the reduce kernel: {case['what']}", ""]
    for tag, counters in COUNTER_PASSES.items():
        lines.append(f"- `{COUNTER_CMD.format(counters=counters, tag=tag, wl=wl)}`")
    lines += ["", "Kernel " + ", ".join(f"`{k}`" for k in sorted(names)) +
              f"; kernel source hash {kernel_source_hash()}.", "",
              "| counter | per dispatch (mean) | dispatches |", "|---|---|---|"]
    for c in sorted(vals):
        v = vals[c]
        lines.append(f"| {c} | {sum(v) / len(v):.1f} | {len(v)} |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(out)


def summarize_pmc(fetch_dir: str, write_dir: str, wl: str = "prefill_bf16") -> None:
    case = PROFILE_CASES[wl]
    match = is_reduce_kernel if wl == "prefill_bf16" else is_library_kernel

    def per_kernel(directory):
        rows = _csv_rows(directory, "counter_collection.csv")
        red = [float(r["Counter_Value"]) for r in rows if match(r["Kernel_Name"])]
        names = sorted({_short(r["Kernel_Name"]) for r in rows if match(r["Kernel_Name"])})
        cal = [float(r["Counter_Value"]) for r in rows if CALIBRATION_KERNEL in r["Kernel_Name"]]
        if not red or not cal:
            raise RuntimeError(f"missing dispatches in {directory}")
        return sum(red) / len(red), len(red), sum(cal) / len(cal), len(cal), names

    f_red, nf, f_cal, ncf, names = per_kernel(fetch_dir)
    w_red, nw, w_cal, ncw, _ = per_kernel(write_dir)
    known_kib = CALIBRATION_BYTES / 1024
    f_scale, w_scale = known_kib / f_cal, known_kib / w_cal
    fetch_b = f_red * f_scale * 1024
    write_b = w_red * w_scale * 1024
    algo = case_algo_bytes(case)
    extra = "" if wl == "prefill_bf16" else f" --profile-workload {wl}"
    traffic = {
        "workload": case["what"],
        "kernel": REDUCE_KERNEL if wl == "prefill_bf16" else names,
        "kernel_source_sha256_16": kernel_source_hash(),
        "fetch_size_kib_per_dispatch": round(f_red, 1), "fetch_dispatches": nf,
        "write_size_kib_per_dispatch": round(w_red, 1), "write_dispatches": nw,
        "calibration": {"kernel": "torch.neg on 64 MiB (reads and writes CALIBRATION_BYTES)",
                        "fetch_kib": round(f_cal, 1), "write_kib": round(w_cal, 1),
                        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
        "hbm_bytes_per_launch": int(round(fetch_b + write_b)),
        "algo_bytes_per_launch": algo,
        "traffic_over_algo": round((fetch_b + write_b) / algo, 4),
        "commands": [PMC_CMD.format(counter="FETCH_SIZE", tag="fetch", extra=extra),
                     PMC_CMD.format(counter="WRITE_SIZE", tag="write", extra=extra)],
    }
    js = PROFILE_TRAFFIC if wl == "prefill_bf16" else os.path.join(ROOT, "profiles", f"traffic_{wl}.json")
    with open(js, "w") as fh:
        json.dump(traffic, fh, indent=1)
    md = os.path.join(ROOT, "profiles", f"traffic_{wl}.md")
    with open(md, "w") as fh:
        fh.write(f"# HBM traffic of the reduce kernel (rocprofv3 --pmc): {case['what']}\n\n")
        for c in traffic["commands"]:
            fh.write(f"- `{c}`\n")
        kn = ", ".join(f"`{k}`" for k in ([REDUCE_KERNEL] if wl == "prefill_bf16" else names))
        fh.write(f"\nKernel {kn}, {nf} dispatches (rotated input sets).\n\n")
        fh.write("| counter | reduce KiB/dispatch | calibration KiB/dispatch (64 MiB known) | scale | "
                 "reduce bytes after scaling |\n|---|---|---|---|---|\n")
        fh.write(f"| FETCH_SIZE | {f_red:.1f} | {f_cal:.1f} | {f_scale:.4f} | {fetch_b:.0f} |\n")
        fh.write(f"| WRITE_SIZE | {w_red:.1f} | {w_cal:.1f} | {w_scale:.4f} | {write_b:.0f} |\n\n")
        fh.write(f"HBM traffic per launch {fetch_b + write_b:.0f} B against {algo} algorithmic B "
                 f"(ratio {(fetch_b + write_b) / algo:.4f}); kernel source hash "
                 f"{traffic['kernel_source_sha256_16']}.\n")
        if case["host"]:
            fh.write("\nThe sources are pinned host memory: FETCH_SIZE counts the L2's fetches from "
                     "memory whether HBM or PCIe serves them, so here it is the host bytes that crossed "
                     "PCIe; HBM sees only the writes.\n")
    print(js, md)


def profile_pass(torch, ar, wl, args):
    """Counter / trace pass: ~20 ms of fill kernels (clock warm-up), rotated reduces
    of one configuration (at least 48 launches), then 8 torch.neg launches that
    read and write CALIBRATION_BYTES each (a plain copy-shaped kernel)."""
    case = PROFILE_CASES[args.profile_workload]
    R, n = case["R"], case["n"]
    S = max(1, min(args.sets, case["sets"]))
    wire = {"bf16": ar.AR_BF16, "f16": ar.AR_F16}[case["wire"]]
    mode = {"chunked": ar.AR_MODE_CHUNKED, "rs_bcast": ar.AR_MODE_RS_BCAST,
            "host_staged": ar.AR_MODE_HOST_STAGED}[case["mode"]]
    sdt = torch.float32 if case["src_bytes"] == 4 else {"bf16": torch.bfloat16, "f16": torch.float16}[case["wire"]]
    if case["src_bytes"] == 2:
        mode |= ar.AR_SRC_WIRE

    def make_src():
        t = torch.randn(n, device="cuda").to(sdt)
        if case["host"]:
            h = torch.empty(n, dtype=sdt, pin_memory=True)
            h.copy_(t)
            return h
        return t

    narrow = case.get("dst_bytes", 4) == 2
    ddt = torch.int16 if narrow else torch.float32
    dst_type = wire if narrow else ar.AR_F32
    if narrow:
        mode &= ~ar.AR_SRC_WIRE          # a narrow destination's sources hold its type anyway
    rows = case.get("rows")
    src_len = n if rows is None else rows[0] * rows[2]
    dst_len = n if rows is None else rows[0] * rows[3]

    def make(length, dt):
        t = torch.randn(length, device="cuda").to(dt)
        if case["host"]:
            h = torch.empty(length, dtype=dt, pin_memory=True)
            h.copy_(t)
            return h
        return t

    inactive = set(case.get("inactive", ()))
    if inactive:
        mode |= ar.AR_SRC_INACTIVE_NULL
    srcs = [[None if r in inactive else (make(src_len, sdt).view(torch.int16) if narrow else make(src_len, sdt))
             for r in range(R)] for _ in range(S)]
    dsts = [[torch.empty(dst_len, device="cuda", dtype=ddt) for _ in range(case["n_dst"])] for _ in range(S)]
    res = case.get("res")
    ress = None
    if res is not None:
        rl = n if res == "elementwise" else res
        ress = [torch.randn(rl, device="cuda") for _ in range(S)]
    torch.cuda.synchronize()
    ctx = ar.ar_init(0)
    stream = torch.cuda.current_stream()
    # bring the GPU out of its idle clocks first (the first calls after idle run
    # up to 25 % slower), with kernels that are not the reduce's: ~20 ms of fills
    # of a 64 MiB buffer
    scratch = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    for _ in range(200):
        scratch.fill_(1)
    torch.cuda.synchronize()
    del scratch
    launches = max(6 * S, 48)
    for k in range(launches):
        i = k % S
        if rows is not None:
            ar.ar_reduce_rows(ctx, dsts[i], srcs[i], rows[0], rows[1], rows[2], rows[3], dst_type, wire, mode,
                              residual=ress[i] if ress else None, res_stride=0, stream=stream)
        elif ress is not None:
            ar.ar_reduce_add(ctx, dsts[i], srcs[i], n, dst_type, wire, mode, ress[i], stream=stream)
        else:
            ar.ar_reduce(ctx, dsts[i], srcs[i], n, dst_type, wire, mode, stream=stream)
    torch.cuda.synchronize()
    ar.ar_free(ctx)
    del srcs, dsts, ress
    nc = CALIBRATION_BYTES // 4
    a = [torch.randn(nc, device="cuda") for _ in range(4)]
    b = [torch.empty(nc, device="cuda") for _ in range(4)]
    for k in range(8):
        torch.neg(a[k % 4], out=b[k % 4])
    torch.cuda.synchronize()
    log(f"profile pass done ({args.profile_workload}): {launches} reduces of R={R} x {n} elements, "
        f"8 calibration copies of {CALIBRATION_BYTES} B")
    return 0


CEILING_LIB = os.path.join(ROOT, "mixed_precision_partial_amd", "libmpp_ceiling.so")


def family_study(torch, ar, wl, args, reps: int = 7, calls: int = 1000) -> int:
    """The kernel choice of the prefill call, measured: the automatic plan (the two-rank
    kernels) against forced register-staged (stream_kernel 1) and LDS-staged (2) general
    kernels, and against the hardware's own workgroup placement (xcd_run_elems 1), for the
    plain call, an element-wise residual and a 4096-element broadcast row.  Every context's
    output is compared bit for bit with the automatic plan's before timing; contexts are
    timed interleaved, rep by rep, with pre-converted calls (ar.bind_reduce).  The plain call
    is also timed with every second source moved 1 MiB into a larger allocation (the kernels'
    sensitivity to where the buffers sit relative to each other), and two bf16 partials
    into a bf16 destination (the two-rank 16-bit kernel) with and without a ragged tail, and
    three or four fp32 partials (the kernels for a few active partials: three ranks, four with
    rank 2 inactive, four, three and four with an element-wise residual).  One JSON line."""
    w = wl.WORKLOADS["prefill_bf16"]
    n, S = w.n, max(1, args.sets)
    src = [[torch.from_numpy(p).cuda() for p in wl.partials(w, s)] for s in range(S)]
    dst = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(S)]
    res = [torch.from_numpy(wl.residual(w.case, s, n)).cuda() for s in range(S)]
    row = torch.from_numpy(wl.residual(w.case, S, 4096)).cuda()
    stream = torch.cuda.current_stream()
    configs = {"auto": None, "register": {"stream_kernel": 1}, "lds": {"stream_kernel": 2},
               "auto_hw_placement": {"xcd_run_elems": 1}}
    ctxs = {k: ar.ar_init(0, v) for k, v in configs.items()}
    forms = {"plain": (None, 12 * n), "residual": ("elementwise", 16 * n), "row": ("row", 12 * n + 4 * 4096)}
    out = {"metric": "prefill call us by kernel choice", "n": n, "wire": "bf16", "rotated_sets": S,
           "calls_per_rep": calls, "reps": reps}
    for form, (rk, nbytes) in forms.items():
        def bound(c, s):
            r = None if rk is None else (res[s] if rk == "elementwise" else row)
            return ar.bind_reduce(c, [dst[s]], src[s], n, ar.AR_F32, w.wire, ar.AR_MODE_CHUNKED, stream=stream,
                                  residual=r)
        fns = {k: [bound(c, s) for s in range(S)] for k, c in ctxs.items()}
        plans = {}
        for k, c in ctxs.items():
            r = None if rk is None else (res[0] if rk == "elementwise" else row)
            if r is None:
                rc, plan = ar.ar_plan_query([dst[0]], src[0], n, ar.AR_F32, w.wire, ar.AR_MODE_CHUNKED,
                                            config=configs[k])
            else:
                rc, plan = ar.ar_plan_query_add([dst[0]], src[0], n, ar.AR_F32, w.wire, ar.AR_MODE_CHUNKED, r,
                                                r.numel(), config=configs[k])
            assert rc == ar.AR_OK
            plans[k] = int(plan.stream_kernel)
        ref = None
        for k in ctxs:
            dst[0].fill_(float("nan"))
            if fns[k][0]() != ar.AR_OK:
                raise RuntimeError(f"{form} {k}: call failed")
            torch.cuda.synchronize()
            bits = dst[0].view(torch.int32).clone()
            if ref is None:
                ref = bits
            elif not torch.equal(bits, ref):
                raise RuntimeError(f"{form}: {k} differs from the automatic plan's output")
        times = {k: [] for k in ctxs}
        for _ in range(reps):
            for k in ctxs:
                f = fns[k]
                times[k].append(timed_us(torch, stream, lambda i: f[i % S](), calls))
        out[form] = {k: {"stream_kernel": plans[k], "us_median": round(float(np.median(v)), 3),
                         "us_min": round(min(v), 3), "us_max": round(max(v), 3),
                         "GB/s": round(nbytes / float(np.median(v)) / 1e3, 1)} for k, v in times.items()}
        log(f"{form}: " + ", ".join(f"{k} {v['us_median']} us (kernel {v['stream_kernel']})"
                                    for k, v in out[form].items()))
    # the plain call with the second sources shifted by 1 MiB
    shift = (1 << 20) // 4
    big = [torch.empty(n + shift, dtype=torch.float32, device="cuda") for _ in range(S)]
    moved = [b[shift:shift + n] for b in big]
    for s in range(S):
        moved[s].copy_(src[s][1])
    fns = {k: [ar.bind_reduce(c, [dst[s]], [src[s][0], moved[s]], n, ar.AR_F32, w.wire, ar.AR_MODE_CHUNKED,
                              stream=stream) for s in range(S)] for k, c in ctxs.items()}
    times = {k: [] for k in ctxs}
    for _ in range(reps):
        for k in ctxs:
            f = fns[k]
            times[k].append(timed_us(torch, stream, lambda i: f[i % S](), calls))
    out["plain_second_source_shifted_1MiB"] = {k: {"us_median": round(float(np.median(v)), 3),
                                                   "GB/s": round(12 * n / float(np.median(v)) / 1e3, 1)}
                                               for k, v in times.items()}
    log("plain, second sources shifted 1 MiB: " + ", ".join(
        f"{k} {v['us_median']} us" for k, v in out["plain_second_source_shifted_1MiB"].items()))
    del big, moved
    # two bf16 partials into a bf16 destination (the two-rank 16-bit kernel on the automatic
    # plan), on the prefill shape and with a 1000-element ragged tail
    for name, m in (("narrow_bf16", n), ("narrow_bf16_ragged", n + 1000)):
        hs = [[torch.randn(m, device="cuda").bfloat16() for _ in range(2)] for _ in range(S)]
        hd = [torch.empty(m, dtype=torch.bfloat16, device="cuda") for _ in range(S)]
        fns = {k: [ar.bind_reduce(c, [hd[s]], hs[s], m, ar.AR_BF16, ar.AR_BF16, ar.AR_MODE_CHUNKED, stream=stream)
                   for s in range(S)] for k, c in ctxs.items()}
        ref = None
        for k in ctxs:
            hd[0].fill_(0)
            if fns[k][0]() != ar.AR_OK:
                raise RuntimeError(f"{name} {k}: call failed")
            torch.cuda.synchronize()
            bits = hd[0].view(torch.int16).clone()
            if ref is None:
                ref = bits
            elif not torch.equal(bits, ref):
                raise RuntimeError(f"{name}: {k} differs from the automatic plan's output")
        times = {k: [] for k in ctxs}
        for _ in range(reps):
            for k in ctxs:
                f = fns[k]
                times[k].append(timed_us(torch, stream, lambda i: f[i % S](), calls))
        out[name] = {k: {"us_median": round(float(np.median(v)), 3),
                         "GB/s": round(6 * m / float(np.median(v)) / 1e3, 1)} for k, v in times.items()}
        log(f"{name}: " + ", ".join(f"{k} {v['us_median']} us" for k, v in out[name].items()))
        del hs, hd, fns
    # three or four fp32 partials on the prefill shape: the kernels for a few active partials
    del src, res
    torch.cuda.empty_cache()
    fsrc = [[torch.randn(n, device="cuda") for _ in range(4)] for _ in range(S)]
    fres = [torch.randn(n, device="cuda") for _ in range(S)]
    inact = ar.AR_SRC_INACTIVE_NULL
    for name, pick, flags, with_res, nbytes in (
            ("few_r3", lambda q: q[:3], 0, False, 16 * n),
            ("few_r4_rank2_inactive", lambda q: [q[0], q[1], None, q[3]], inact, False, 16 * n),
            ("few_r4", lambda q: q, 0, False, 20 * n),
            ("few_r3_residual", lambda q: q[:3], 0, True, 20 * n),
            ("few_r4_residual", lambda q: q, 0, True, 24 * n)):
        fns = {k: [ar.bind_reduce(c, [dst[s]], pick(fsrc[s]), n, ar.AR_F32, w.wire, ar.AR_MODE_CHUNKED | flags,
                                  stream=stream, residual=fres[s] if with_res else None) for s in range(S)]
               for k, c in ctxs.items()}
        ref = None
        for k in ctxs:
            dst[0].fill_(float("nan"))
            if fns[k][0]() != ar.AR_OK:
                raise RuntimeError(f"{name} {k}: call failed")
            torch.cuda.synchronize()
            bits = dst[0].view(torch.int32).clone()
            if ref is None:
                ref = bits
            elif not torch.equal(bits, ref):
                raise RuntimeError(f"{name}: {k} differs from the automatic plan's output")
        times = {k: [] for k in ctxs}
        for _ in range(reps):
            for k in ctxs:
                f = fns[k]
                times[k].append(timed_us(torch, stream, lambda i: f[i % S](), calls))
        out[name] = {k: {"us_median": round(float(np.median(v)), 3),
                         "GB/s": round(nbytes / float(np.median(v)) / 1e3, 1)} for k, v in times.items()}
        log(f"{name}: " + ", ".join(f"{k} {v['us_median']} us" for k, v in out[name].items()))
        del fns
    torch.cuda.synchronize()
    for c in ctxs.values():
        ar.ar_free(c)
    print(json.dumps(out), flush=True)
    return 0


def hold_study(torch, ar, wl, args, reps: int = 7) -> int:
    """The occupancy hold (ar_config.occupancy_hold), measured: the prefill call (plain,
    element-wise residual, 4096-element broadcast row) and the row-strided prefill block
    (2048 x 4096 in rows of 4608 / 4352: plain, strided residual, bias row), each on the
    two-rank kernels unheld (-1), held to 14, 16, 18 or 20 waves per CU, and automatic (0);
    the prefill shape with three ranks, four with rank 2 inactive, four, and two active of
    four, and with an element-wise residual, on the kernels for a few active partials unheld,
    held to 8, 10, 14 or 18, and automatic;
    the 4-rank broadcast (cfg 4), the bf16 -> bf16 prefill shape and R = 8 fp32 partials on
    their automatic general kernels unheld and held to 8, 12 or 16 waves.  Outputs are
    compared bit for bit across holds before timing; holds are timed interleaved, rep by
    rep, medians reported.  One JSON line."""
    stream = torch.cuda.current_stream()
    holds = sorted({-1, 0, 8, 10, 12, 14, 16, 18, 20})
    ctxs = {h: ar.ar_init(0, {"occupancy_hold": h} if h else None) for h in holds}
    out = {"metric": "us per call by occupancy hold (waves per CU; -1 none, 0 automatic)", "reps": reps}

    def measure(name, hs, calls, fn, nbytes, check):
        """fn(h, k) enqueues call k under hold h; check() returns the output bits of call 0."""
        ref = None
        for h in hs:
            fn(h, 0)
            torch.cuda.synchronize()
            bits = check().clone()
            if ref is None:
                ref = bits
            elif not torch.equal(bits, ref):
                raise RuntimeError(f"{name}: hold {h} changes the output")
        times = {h: [] for h in hs}
        for _ in range(reps):
            for h in hs:
                times[h].append(timed_us(torch, stream, lambda k, h=h: fn(h, k), calls))
        out[name] = {str(h): {"us_median": round(float(np.median(v)), 3), "us_min": round(min(v), 3),
                              "GB/s": round(nbytes / float(np.median(v)) / 1e3, 1)} for h, v in times.items()}
        log(f"{name}: " + ", ".join(f"{h}: {out[name][str(h)]['us_median']}" for h in hs))

    pair_holds = [-1, 14, 16, 18, 20, 0]
    w = wl.WORKLOADS["prefill_bf16"]
    n, S = w.n, max(1, args.sets)
    src = [[torch.from_numpy(p).cuda() for p in wl.partials(w, s)] for s in range(S)]
    dst = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(S)]
    res = [torch.from_numpy(wl.residual(w.case, s, n)).cuda() for s in range(S)]
    row = torch.from_numpy(wl.residual(w.case, S, 4096)).cuda()
    bound = {}
    for h, c in ctxs.items():
        for form in ("plain", "residual", "row"):
            bound[(h, form)] = [ar.bind_reduce(c, [dst[s]], src[s], n, ar.AR_F32, w.wire, ar.AR_MODE_CHUNKED,
                                               stream=stream,
                                               residual={"plain": None, "residual": res[s], "row": row}[form])
                                for s in range(S)]
    for form, nbytes in (("plain", 12 * n), ("residual", 16 * n), ("row", 12 * n + 4 * 4096)):
        measure(f"prefill_{form}", pair_holds, 1000, lambda h, k, form=form: bound[(h, form)][k % S](), nbytes,
                lambda: dst[0].view(torch.int32))
    del src, dst, res, bound
    torch.cuda.empty_cache()
    few_holds = [-1, 8, 10, 14, 18, 0]
    f_src = [[torch.randn(n, device="cuda") for _ in range(4)] for _ in range(S)]
    f_dst = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(S)]
    inact = ar.AR_SRC_INACTIVE_NULL
    f_res = [torch.randn(n, device="cuda") for _ in range(S)]
    for form, pick, flags, nbytes, with_res in (
            ("r3", lambda q: q[:3], 0, 16 * n, False),
            ("r4_rank2_inactive", lambda q: [q[0], q[1], None, q[3]], inact, 16 * n, False),
            ("r4", lambda q: q, 0, 20 * n, False),
            ("r4_two_active", lambda q: [None, q[1], None, q[3]], inact, 12 * n, False),
            ("r4_two_active_residual", lambda q: [None, q[1], None, q[3]], inact, 16 * n, True),
            ("r3_residual", lambda q: q[:3], 0, 20 * n, True),
            ("r4_residual", lambda q: q, 0, 24 * n, True)):
        fb = {h: [ar.bind_reduce(ctxs[h], [f_dst[i]], pick(f_src[i]), n, ar.AR_F32, w.wire,
                                 ar.AR_MODE_CHUNKED | flags, stream=stream,
                                 residual=f_res[i] if with_res else None) for i in range(S)]
              for h in few_holds}
        measure(f"few_{form}", few_holds, 1000, lambda h, k, fb=fb: fb[h][k % S](), nbytes,
                lambda: f_dst[0].view(torch.int32))
    del f_src, f_dst, f_res
    torch.cuda.empty_cache()
    rows, cols, ss, ds = 2048, 4096, 4608, 4352
    R6 = 6
    rs_src = [[torch.randn(rows * ss, device="cuda") for _ in range(2)] for _ in range(R6)]
    rs_dst = [torch.empty(rows * ds, device="cuda") for _ in range(R6)]
    rs_res = [torch.randn(rows * ss, device="cuda") for _ in range(R6)]
    bias = torch.randn(cols, device="cuda")
    for form, nbytes in (("plain", 12 * rows * cols), ("residual", 16 * rows * cols),
                         ("bias_row", 12 * rows * cols + 4 * cols)):
        def call(h, k, form=form):
            i = k % R6
            r = {"plain": None, "residual": rs_res[i], "bias_row": bias}[form]
            ar.ar_reduce_rows(ctxs[h], [rs_dst[i]], rs_src[i], rows, cols, ss, ds, ar.AR_F32, ar.AR_BF16,
                              ar.AR_MODE_CHUNKED, residual=r, res_stride=ss if form == "residual" else 0,
                              stream=stream)
        measure(f"rows_block_{form}", pair_holds, 1000, call, nbytes, lambda: rs_dst[0].view(torch.int32))
    del rs_src, rs_dst, rs_res
    torch.cuda.empty_cache()
    gen_holds = [-1, 8, 12, 16]
    n4 = 2048 * 8192
    b4_src = [[torch.randn(n4, device="cuda") for _ in range(4)] for _ in range(2)]
    b4_dst = [[torch.empty(n4, device="cuda") for _ in range(4)] for _ in range(2)]
    measure("slice_bcast_f16", gen_holds, 50,
            lambda h, k: ar.ar_reduce(ctxs[h], b4_dst[k % 2], b4_src[k % 2], n4, ar.AR_F32, ar.AR_F16,
                                      ar.AR_MODE_RS_BCAST, stream=stream),
            8 * n4 * 4, lambda: b4_dst[0][3].view(torch.int32))
    del b4_src, b4_dst
    torch.cuda.empty_cache()
    h_src = [[torch.randn(n, device="cuda").bfloat16() for _ in range(2)] for _ in range(S)]
    h_dst = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(S)]
    measure("prefill_bf16_dst", gen_holds, 500,
            lambda h, k: ar.ar_reduce(ctxs[h], [h_dst[k % S]], h_src[k % S], n, ar.AR_BF16, ar.AR_BF16,
                                      ar.AR_MODE_CHUNKED, stream=stream),
            6 * n, lambda: h_dst[0].view(torch.int16))
    del h_src, h_dst
    torch.cuda.empty_cache()
    n8 = 8192 * 8192
    s8 = [torch.randn(n8, device="cuda") for _ in range(8)]
    d8 = torch.empty(n8, device="cuda")
    measure("r8_hbm_fp32_src", gen_holds, 20,
            lambda h, k: ar.ar_reduce(ctxs[h], [d8], s8, n8, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED,
                                      stream=stream),
            9 * n8 * 4, lambda: d8.view(torch.int32))
    del s8, d8
    torch.cuda.synchronize()
    for c in ctxs.values():
        ar.ar_free(c)
    print(json.dumps(out), flush=True)
    return 0


def size_study(torch, ar, wl, args, reps: int = 5) -> int:
    """How the prefill call's time splits into a fixed per-call cost and streaming: the
    two-rank reduce (R = 2 fp32 partials, bf16 wire, CHUNKED) and the 2 : 1 ceiling kernel
    (write-through, XCD runs, one-wave workgroups, held to 18 waves: the reduce's own
    launch) at n = 2^20 ... 2^26 elements, each size over 768 MiB of rotated sets (the
    headline's footprint: past the Infinity Cache, below the ~1 GiB where every kernel
    slows), back to back between two HIP events; a least-squares line
    us = fixed + bytes / rate over the sizes from 2^22 up (smaller calls can be limited by
    the Python enqueue).  Then the prefill size by footprint: the reduce and the ceiling
    kernel over 4 ... 24 rotated sets, and the reduce over 8 or 16 sets touching only the
    first half of every buffer (is it the bytes touched or the allocations?).  Then the
    cost of a ragged tail (n = 2^23 + k) on each kernel family.  Last, the 768 MiB call and
    its ceiling with the three buffers at five relative placements.  One JSON line."""
    import ctypes

    stream = torch.cuda.current_stream()
    ctx = ar.ar_init(0)
    lib = ceiling_lib()
    vp = ctypes.c_void_p
    sh = vp(stream.cuda_stream)
    out = {"metric": "us per call by size (R = 2 fp32 partials, bf16 wire)", "reps": reps, "sizes": {}}
    xs, ys, yc = [], [], []
    for k in range(20, 27):
        n = 1 << k
        nbytes = 12 * n
        sets = max(1, (768 << 20) // nbytes)   # 768 MiB touched at every size, as in the headline
        src = [[torch.randn(n, device="cuda") for _ in range(2)] for _ in range(sets)]
        dst = [torch.empty(n, device="cuda") for _ in range(sets)]
        calls = max(20, min(2000, int(30e3 / (nbytes / 6.5e6 + 2.0))))
        fns = [ar.bind_reduce(ctx, [dst[i]], src[i], n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED, stream=stream)
               for i in range(sets)]
        arrs = [((vp * 2)(src[i][0].data_ptr(), src[i][1].data_ptr()), (vp * 1)(dst[i].data_ptr()))
                for i in range(sets)]

        def ceil_call(i):
            a, b = arrs[i % sets]
            if lib.mpp_ceiling_launch(2, 1, 2, 64, a, b, n * 4, 512 << 10, 18, sh) != 0:
                raise RuntimeError("ceiling kernel launch failed")
        tr, tc = [], []
        for _ in range(reps):
            tr.append(timed_us(torch, stream, lambda i: fns[i % sets](), calls))
            tc.append(timed_us(torch, stream, ceil_call, calls))
        r, c = float(np.median(tr)), float(np.median(tc))
        out["sizes"][str(n)] = {"bytes": nbytes, "sets": sets, "calls": calls, "reduce_us": round(r, 3),
                                "reduce_GB/s": round(nbytes / r / 1e3, 1), "ceiling_us": round(c, 3),
                                "ceiling_GB/s": round(nbytes / c / 1e3, 1)}
        log(f"n = 2^{k}: reduce {r:.3f} us ({nbytes / r / 1e3:.0f} GB/s), ceiling {c:.3f} us "
            f"({nbytes / c / 1e3:.0f} GB/s), {sets} sets")
        if k >= 22:    # below ~10 us per call the Python enqueue can be the limit
            xs.append(nbytes)
            ys.append(r)
            yc.append(c)
        del src, dst, fns, arrs
        torch.cuda.empty_cache()
    for name, y in (("reduce", ys), ("ceiling", yc)):
        slope, fixed = np.polyfit(np.array(xs, dtype=float), np.array(y), 1)
        out[f"{name}_fit"] = {"fixed_us": round(float(fixed), 3), "streaming_GB/s": round(1e-3 / float(slope), 1)}
        log(f"{name}: us = {fixed:.3f} + bytes / {1e-3 / slope:.1f} GB/s")
    # the prefill size by footprint: 4 ... 24 rotated sets (384 MiB ... 2.25 GiB touched), and
    # 8 or 16 sets of which each call touches only the first half of every buffer
    n = 1 << 23
    smax = 24
    src = [[torch.randn(n, device="cuda") for _ in range(2)] for _ in range(smax)]
    dst = [torch.empty(n, device="cuda") for _ in range(smax)]
    full = [ar.bind_reduce(ctx, [dst[i]], src[i], n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED, stream=stream)
            for i in range(smax)]
    half = [ar.bind_reduce(ctx, [dst[i][:n // 2]], [t[:n // 2] for t in src[i]], n // 2, ar.AR_F32, ar.AR_BF16,
                           ar.AR_MODE_CHUNKED, stream=stream) for i in range(smax)]
    arrs = [((vp * 2)(src[i][0].data_ptr(), src[i][1].data_ptr()), (vp * 1)(dst[i].data_ptr()))
            for i in range(smax)]

    def ceil_at(i):
        a, b = arrs[i]
        if lib.mpp_ceiling_launch(2, 1, 2, 64, a, b, n * 4, 512 << 10, 18, sh) != 0:
            raise RuntimeError("ceiling kernel launch failed")
    cases = {}
    for sets in (4, 8, 12, 16, 24):
        cases[f"reduce_{sets}_sets"] = (lambda k, sets=sets: full[k % sets](), 12 * n, sets * 96)
        cases[f"ceiling_{sets}_sets"] = (lambda k, sets=sets: ceil_at(k % sets), 12 * n, sets * 96)
    for sets in (8, 16):
        cases[f"reduce_half_touched_{sets}_sets"] = (lambda k, sets=sets: half[k % sets](), 6 * n, sets * 48)
    times = {k: [] for k in cases}
    for _ in range(reps):
        for k, (fn, _, _) in cases.items():
            times[k].append(timed_us(torch, stream, fn, 1000))
    out["footprint"] = {}
    for k, (fn, nbytes, mib) in cases.items():
        m = float(np.median(times[k]))
        out["footprint"][k] = {"touched_MiB": mib, "us": round(m, 3), "GB/s": round(nbytes / m / 1e3, 1)}
        log(f"{k} ({mib} MiB touched): {m:.3f} us, {nbytes / m / 1e3:.0f} GB/s")
    del src, dst, full, half, arrs
    torch.cuda.empty_cache()
    # the tail: the prefill call with n = 2^23 + k on the automatic plan (the two-rank kernel)
    # and on the forced register- and LDS-staged kernels (the LDS-staged kernels keep the
    # per-element tail)
    tail_ctx = {"auto": ctx, "register": ar.ar_init(0, {"stream_kernel": 1}),
                "lds": ar.ar_init(0, {"stream_kernel": 2})}
    n = 1 << 23
    src = [[torch.randn(n + 512, device="cuda") for _ in range(2)] for _ in range(8)]
    dst = [torch.empty(n + 512, device="cuda") for _ in range(8)]
    out["tail"] = {}
    for k in (0, 200, 488):
        m = n + k
        row = {}
        for name, c in tail_ctx.items():
            fns = [ar.bind_reduce(c, [dst[i][:m]], [t[:m] for t in src[i]], m, ar.AR_F32, ar.AR_BF16,
                                  ar.AR_MODE_CHUNKED, stream=stream) for i in range(8)]
            row[name] = round(float(np.median([timed_us(torch, stream, lambda i: fns[i % 8](), 1000)
                                               for _ in range(reps)])), 3)
        out["tail"][str(k)] = row
        log(f"n = 2^23 + {k}: " + ", ".join(f"{name} {v:.3f} us" for name, v in row.items()))
    for name in ("register", "lds"):
        ar.ar_free(tail_ctx[name])
    del src, dst
    torch.cuda.empty_cache()
    # the 768 MiB call with its three buffers carved from one pool at different relative
    # offsets (the second source and the destination moved by d1, d1 + d2 bytes)
    n = 1 << 26
    out["placement_768MiB"] = {}
    for d1, d2 in ((0, 0), (1 << 18, 1 << 19), (1 << 20, 3 << 20), (5 << 20, 1 << 22), (3 << 12, 7 << 12)):
        pool = torch.empty(3 * n + (16 << 20) // 4, device="cuda")
        a, b = pool[:n], pool[n + d1 // 4:2 * n + d1 // 4]
        d = pool[2 * n + (d1 + d2) // 4:3 * n + (d1 + d2) // 4]
        a.normal_()
        b.normal_()
        fn = ar.bind_reduce(ctx, [d], [a, b], n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED, stream=stream)
        pa = ((vp * 2)(a.data_ptr(), b.data_ptr()), (vp * 1)(d.data_ptr()))

        def ceil_p(i, pa=pa):
            if lib.mpp_ceiling_launch(2, 1, 2, 64, pa[0], pa[1], n * 4, 512 << 10, 18, sh) != 0:
                raise RuntimeError("ceiling kernel launch failed")
        tr, tc = [], []
        for _ in range(reps):
            tr.append(timed_us(torch, stream, lambda i: fn(), 100))
            tc.append(timed_us(torch, stream, ceil_p, 100))
        key = f"offsets_{d1}_{d1 + d2}"
        out["placement_768MiB"][key] = {"reduce_us": round(float(np.median(tr)), 3),
                                        "ceiling_us": round(float(np.median(tc)), 3)}
        log(f"768 MiB call, second source +{d1} B, destination +{d1 + d2} B: reduce "
            f"{np.median(tr):.2f} us, ceiling {np.median(tc):.2f} us")
        del pool, a, b, d, fn
    ar.ar_free(ctx)
    print(json.dumps(out), flush=True)
    return 0


def timing_study(torch, ar, wl, args, reps: int = 6) -> int:
    """The 20-step prefill figure under each timing method, interleaved rep by rep
    on the same rotated buffers, plus what an event costs on its own and what an
    idle GPU costs the first steps.  Prints one JSON line."""
    w = wl.WORKLOADS["prefill_bf16"]
    n, S = w.n, max(1, args.sets)
    src = [[torch.from_numpy(p).cuda() for p in wl.partials(w, s)] for s in range(S)]
    dst = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(S)]
    ctx = ar.ar_init(0)
    stream = torch.cuda.current_stream()

    def step(k):
        ar.ar_reduce(ctx, [dst[k % S]], src[k % S], n, ar.AR_F32, w.wire, ar.AR_MODE_CHUNKED, stream=stream)

    def block(K, lead, fenced):
        torch.cuda.synchronize()
        for k in range(lead):
            step(k)
        if fenced:   # torch's events: default HIP events (system-scope fence on record)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        else:
            a, b = HipEvent(), HipEvent()
        a.record(stream)
        for k in range(K):
            step(lead + k)
        b.record(stream)
        torch.cuda.synchronize()
        return (a.elapsed_time(b) if fenced else a.elapsed_ms(b)) * 1e3 / max(K, 1)

    for k in range(200):
        step(k)
    methods = {"default_events_no_lead_in": (0, True), "default_events_lead_in": (1, True),
               "fence_free_events_no_lead_in": (0, False), "fence_free_events_lead_in": (1, False),
               "fence_free_events_3_lead_in": (LEAD_IN_CALLS, False)}
    res = {m: [] for m in methods}
    for _ in range(reps):
        for m, (lead, fenced) in methods.items():
            res[m].append(block(args.steps, lead, fenced))
    out = {"metric": "prefill reduce us/step by timing method", "steps": args.steps, "reps": reps,
           "k20_us_per_step": {m: {"median": round(float(np.median(v)), 3), "min": round(min(v), 3),
                                   "max": round(max(v), 3)} for m, v in res.items()},
           "k2000_fence_free_lead_in_us": round(block(2000, 1, False), 3),
           "empty_interval_us": {"default_events": round(float(np.median([block(0, 0, True) for _ in range(5)])), 2),
                                 "fence_free_events": round(float(np.median([block(0, 0, False) for _ in range(5)])), 2)}}
    idle = {}
    for sec in (0.2, 1.0):
        torch.cuda.synchronize()
        time.sleep(sec)
        first = block(args.steps, 1, False)
        second = block(args.steps, 1, False)
        idle[f"after_{sec}s_idle"] = {"first_block_us": round(first, 3), "second_block_us": round(second, 3)}
    out["idle_then_20_steps"] = idle
    torch.cuda.synchronize()
    ar.ar_free(ctx)
    print(json.dumps(out), flush=True)
    return 0


def ceiling_lib():
    import ctypes

    if not os.path.exists(CEILING_LIB):
        raise RuntimeError(f"{CEILING_LIB} is missing: build with `python -m mixed_precision_partial_amd.build`")
    lib = ctypes.CDLL(CEILING_LIB)
    vp = ctypes.c_void_p
    lib.mpp_ceiling_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(vp),
                                       ctypes.POINTER(vp), ctypes.c_size_t, ctypes.c_size_t, ctypes.c_int, vp]
    lib.mpp_ceiling_launch.restype = ctypes.c_int
    return lib


# resident waves per CU the ceiling kernels are also timed at (0: not held); the
# reduce's two-rank kernels are held to 18 (no residual) and 14 (residual)
CEILING_HOLDS = (0, 10, 14, 18)


def pattern_ceiling(torch, stream, R, D, src_sets, dst_sets, nbytes, reps):
    """Best GB/s (bytes moved) of the ceiling kernel with the (R reads, D writes)
    pattern over the given rotated tensors, `nbytes` per stream: 256- and
    64-thread workgroups, every store policy, without and with XCD runs of
    512 KiB and 1 MiB, each CU unheld and held to CEILING_HOLDS resident waves."""
    import ctypes

    lib = ceiling_lib()
    vp = ctypes.c_void_p
    sh = vp(stream.cuda_stream)
    arrays = [((vp * R)(*[t.data_ptr() for t in srcs]), (vp * D)(*[t.data_ptr() for t in dsts]))
              for srcs, dsts in zip(src_sets, dst_sets)]
    best = 0.0
    for block in (256, 64):
        for sp in (0, 1, 2):
            for run in (0, 512 << 10, 1 << 20):
                for hold in CEILING_HOLDS:
                    def fn(k, sp=sp, run=run, block=block, hold=hold):
                        a, b = arrays[k % len(arrays)]
                        if lib.mpp_ceiling_launch(R, D, sp, block, a, b, nbytes, run, hold, sh) != 0:
                            raise RuntimeError("ceiling kernel launch failed")
                    best = max(best, (R + D) * nbytes / timed_us(torch, stream, fn, reps) / 1e3)
    return round(best, 1)


def ceilings(torch, stream, dev_src, dev_dst, n, sets, reps=300):
    """Achievable rates at the prefill size over the benchmark's own rotated
    buffers (GB/s of bytes moved): the reference kernels of libmpp_ceiling.so --
    a 16-byte copy (1 read : 1 write) and a 2-read : 1-write stream, each with
    every store policy, with the hardware's placement and with the reduce's XCD
    runs, in 256-thread workgroups and in the one-wave workgroups the prefill's
    own kernel uses, each CU unheld and held to CEILING_HOLDS resident waves
    (key suffix _hold<waves>) -- and the runtime's device-to-device copy (torch
    copy_).  The reduce is compared with the best 2-read : 1-write figure."""
    import ctypes

    lib = ceiling_lib()
    vp = ctypes.c_void_p
    sh = vp(stream.cuda_stream)
    arrays = [((vp * 2)(dev_src[i][0].data_ptr(), dev_src[i][1].data_ptr()), (vp * 1)(dev_dst[i].data_ptr()))
              for i in range(sets)]
    out = {}
    for R, name in ((1, "copy_1r1w"), (2, "2r1w")):
        for sp, sp_name in ((0, "wb"), (1, "nt"), (2, "wt")):
            for run, run_name in ((0, "hw"), (512 << 10, "xcd512k")):
                for block, wg_name in ((256, ""), (64, "_wg64")):
                    for hold in CEILING_HOLDS:
                        def fn(k, R=R, sp=sp, run=run, block=block, hold=hold):
                            src, dst = arrays[k % sets]
                            rc = lib.mpp_ceiling_launch(R, 1, sp, block, src, dst, n * 4, run, hold, sh)
                            if rc != 0:
                                raise RuntimeError(f"ceiling kernel launch failed ({rc})")
                        us = timed_us(torch, stream, fn, reps)
                        key = f"kernel_{name}_{sp_name}_{run_name}{wg_name}{f'_hold{hold}' if hold else ''}_GB/s"
                        out[key] = round((R + 1) * 4 * n / us / 1e3, 1)
    us = timed_us(torch, stream, lambda k: dev_dst[k % sets].copy_(dev_src[k % sets][0]), reps)
    out["runtime_d2d_copy_GB/s"] = round(2 * 4 * n / us / 1e3, 1)
    log(f"ceilings at the prefill size: {out}")
    return out


def per_step_times(torch, stream, step, K):
    """Microseconds of each of K steps, each step between two HipEvents (a
    pass of its own: the events between steps add their own cost)."""
    torch.cuda.synchronize()
    step(0)
    ev = [HipEvent() for _ in range(K + 1)]
    ev[0].record(stream)
    for k in range(K):
        step(1 + k)
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[k].elapsed_ms(ev[k + 1]) * 1e3 for k in range(K)]


def oracle_decode_latency(oracle, wl):
    """The CPU oracle at decode size: microseconds per call over all 10,000
    seeded calls of the bf16-wire decode configuration, and over 2,000 calls
    of the fp32-wire one, single-threaded (the host arrays of each call are
    generated beforehand, outside the timing)."""
    res = {}
    for name, calls in (("decode_bf16", 10_000), ("decode_f32", 2_000)):
        w = wl.WORKLOADS[name]
        inputs = [wl.partials(w, c) for c in range(calls)]
        t = time.perf_counter()
        for srcs in inputs:
            oracle.reduce(srcs, w.wire)
        res[f"{name}_us_per_call"] = round((time.perf_counter() - t) * 1e6 / calls, 2)
        res[f"{name}_calls"] = calls
    log(f"oracle at decode size: {res}")
    return res


def decode_latency(torch, ar, wl, name="decode_bf16", floors=True):
    """10,000 sequential single-shot calls on fresh seeded data (all pre-staged in HBM);
    `floors` adds the smallest torch kernel timed the same way."""
    w = wl.WORKLOADS[name]
    calls, n, R = max(w.calls, 10_000), w.n, w.R
    log(f"{name}: staging {calls} calls of R={R} x n={n}")
    host = np.empty((calls, R, n), dtype=np.float32)
    for c in range(calls):
        for r, p in enumerate(wl.partials(w, c)):
            host[c, r] = p
    dev = torch.from_numpy(host).cuda()
    out = torch.empty((calls, n), dtype=torch.float32, device="cuda")
    ctx = ar.ar_init(0)
    stream = torch.cuda.current_stream()
    bi, bo = dev.data_ptr(), out.data_ptr()
    # pointer arrays built once (the binding passes ready-made arrays through)
    srcs = [ar.ptr_array([bi + (c * R + r) * n * 4 for r in range(R)]) for c in range(calls)]
    dsts = [ar.ptr_array([bo + c * n * 4]) for c in range(calls)]

    def call(c):
        ar.ar_reduce(ctx, dsts[c], srcs[c], n, ar.AR_F32, w.wire, ar.AR_MODE_SINGLE_SHOT, stream=stream)

    # the same calls with their arguments converted to C types once (ar.bind_reduce)
    bound = [ar.bind_reduce(ctx, dsts[c], srcs[c], n, ar.AR_F32, w.wire, ar.AR_MODE_SINGLE_SHOT, stream=stream)
             for c in range(calls)]

    for c in range(200):
        call(c)
        bound[c]()
    torch.cuda.synchronize()
    start, end = HipEvent(), HipEvent()
    t0 = time.perf_counter()
    start.record(stream)
    for c in range(calls):
        call(c)
    end.record(stream)
    torch.cuda.synchronize()
    host_s = time.perf_counter() - t0
    us_async = start.elapsed_ms(end) * 1e3 / calls
    t0 = time.perf_counter()
    start.record(stream)
    for fn in bound:
        if fn():
            raise RuntimeError("bound decode call failed")
    end.record(stream)
    torch.cuda.synchronize()
    host_bound_s = time.perf_counter() - t0
    us_async_bound = start.elapsed_ms(end) * 1e3 / calls
    # the same calls captured once into a HIP graph and replayed: the
    # per-call cost without Python or runtime launch overhead
    graph_calls = 1000
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        gs = torch.cuda.current_stream()
        for c in range(graph_calls):
            ar.ar_reduce(ctx, dsts[c], srcs[c], n, ar.AR_F32, w.wire, ar.AR_MODE_SINGLE_SHOT, stream=gs)
    g.replay()
    torch.cuda.synchronize()
    reps = calls // graph_calls
    start.record(stream)
    for _ in range(reps):
        g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    us_graph = start.elapsed_ms(end) * 1e3 / (reps * graph_calls)
    del g
    # per-call round trip, wall clock: enqueue + hipStreamSynchronize on the launch stream
    lat = np.empty(2000)
    for i in range(lat.size):
        t = time.perf_counter()
        call(i)
        stream.synchronize()
        lat[i] = (time.perf_counter() - t) * 1e6
    ar.ar_free(ctx)
    res = {
        "us_per_call_async": round(us_async, 3),
        "us_per_call_async_bound": round(us_async_bound, 3),
        "host_enqueue_us_per_call_bound": round(host_bound_s * 1e6 / calls, 3),
        "us_per_call_graph_replay": round(us_graph, 3),
        "host_enqueue_us_per_call": round(host_s * 1e6 / calls, 3),
        "us_per_call_sync_p50": round(float(np.percentile(lat, 50)), 2),
        "us_per_call_sync_p99": round(float(np.percentile(lat, 99)), 2),
        "calls": calls,
    }
    if not floors:
        log(f"{name}: {res}")
        return res
    # launch floor for context: the smallest torch kernel (a 1-element fill) issued
    # the same way, async and replayed from a graph
    one = torch.empty(1, device="cuda")
    for _ in range(200):
        one.fill_(1.0)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(calls):
        one.fill_(1.0)
    end.record(stream)
    torch.cuda.synchronize()
    floor_async = start.elapsed_ms(end) * 1e3 / calls
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        for _ in range(graph_calls):
            one.fill_(1.0)
    g.replay()
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(reps):
        g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    floor_graph = start.elapsed_ms(end) * 1e3 / (reps * graph_calls)
    del g
    res = {"floor_1elem_fill_us_async": round(floor_async, 3),
           "floor_1elem_fill_us_graph_replay": round(floor_graph, 3), **res}
    log(f"{name}: {res}")
    return res


def with_ceiling(entry: dict, ceiling_gbs: float) -> None:
    entry["ceiling_GB/s"] = ceiling_gbs
    entry["frac_of_ceiling"] = round(entry["GB/s"] / ceiling_gbs, 4)
    entry["frac_of_hbm_peak"] = round(entry["GB/s"] / HBM_PEAK_GBS, 4)


def other_schedules(torch, ar, wl):
    """The other configurations and adjacent forms: the 4-rank slice + broadcast,
    residual adds, narrow destinations, inactive ranks, row-strided tensors, R=8
    from HBM (fp32 and bf16 partials) and from pinned host memory (direct reads,
    copy-engine pipeline, static staging), the two-rank reduce on a 768 MiB
    call, and the headline call over 1.5 GiB of rotated sets -- each beside the
    ceiling kernel run at its own bytes and access pattern where one exists
    (stderr + extras)."""
    out = {}
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        """milliseconds per call (one warm-up call, the headline's lead-in calls, HipEvents
        on the stream)"""
        fn()
        return timed_us(torch, stream, lambda k: fn(), reps, lead=LEAD_IN_CALLS) / 1e3

    def rotating(calls):
        """One call of a rotation over pre-bound calls (arguments converted to C types once,
        as in the headline's timed region); a failed status raises."""
        k = [0]

        def call():
            rc = calls[k[0] % len(calls)]()
            k[0] += 1
            if rc != ar.AR_OK:
                raise ar.ArError(rc, "bound reduce")
        return call

    ctx = ar.ar_init(0)
    # the 4-rank broadcast over two rotated sets (1 GiB, beyond the Infinity Cache)
    w = wl.WORKLOADS["slice_bcast_f16"]
    bsets = 2
    srcs = [[torch.from_numpy(p).cuda() for p in wl.partials(w, k)] for k in range(bsets)]
    dsts = [[torch.empty(w.n, dtype=torch.float32, device="cuda") for _ in range(w.R)] for _ in range(bsets)]

    ms = timed(rotating([ar.bind_reduce(ctx, dsts[i], srcs[i], w.n, ar.AR_F32, w.wire, ar.AR_MODE_RS_BCAST,
                                        stream=stream) for i in range(bsets)]), 50)
    b = 2 * w.R * w.n * 4
    out["slice_bcast_f16"] = {"us": round(ms * 1e3, 2), "GB/s": round(b / ms / 1e6, 1)}
    with_ceiling(out["slice_bcast_f16"], pattern_ceiling(torch, stream, 4, 4, srcs, dsts, w.n * 4, 30))
    log(f"slice_bcast_f16: {out['slice_bcast_f16']}")
    # the same broadcast with an element-wise fp32 residual (the receiving rank's hidden state)
    ress = [torch.from_numpy(wl.residual(w.case, 5 + k, w.n)).cuda() for k in range(bsets)]
    ms = timed(rotating([ar.bind_reduce(ctx, dsts[i], srcs[i], w.n, ar.AR_F32, w.wire, ar.AR_MODE_RS_BCAST,
                                        stream=stream, residual=ress[i]) for i in range(bsets)]), 50)
    b = 2 * w.R * w.n * 4 + w.n * 4
    out["slice_bcast_f16_residual"] = {"us": round(ms * 1e3, 2), "GB/s": round(b / ms / 1e6, 1)}
    log(f"slice_bcast_f16_residual: {out['slice_bcast_f16_residual']}")
    del srcs, dsts, ress
    torch.cuda.empty_cache()

    # fused residual add on the prefill shape (element-wise hidden state, and a
    # broadcast row of 4096), and narrow destinations; rotated sets so the
    # Infinity Cache cannot serve them
    w = wl.WORKLOADS["prefill_bf16"]
    sets = 4
    srcs = [[torch.from_numpy(p).cuda() for p in wl.partials(w, k)] for k in range(sets)]
    dsts = [torch.empty(w.n, dtype=torch.float32, device="cuda") for _ in range(sets)]
    ress = [torch.from_numpy(wl.residual(w.case, k, w.n)).cuda() for k in range(sets)]
    row = torch.from_numpy(wl.residual(w.case, 9, 4096)).cuda()

    # the same reduce with an fp32 wire: the difference to the headline is the narrowing's cost
    ms = timed(rotating([ar.bind_reduce(ctx, [dsts[i]], srcs[i], w.n, ar.AR_F32, ar.AR_F32, ar.AR_MODE_CHUNKED,
                                        stream=stream) for i in range(sets)]), 200)
    b = w.R * w.n * 4 + w.n * 4
    out["prefill_f32_wire"] = {"us": round(ms * 1e3, 2), "GB/s": round(b / ms / 1e6, 1)}
    log(f"prefill_f32_wire: {out['prefill_f32_wire']}")
    ms = timed(rotating([ar.bind_reduce(ctx, [dsts[i]], srcs[i], w.n, ar.AR_F32, w.wire, ar.AR_MODE_CHUNKED,
                                        stream=stream, residual=ress[i], residual_len=w.n)
                         for i in range(sets)]), 200)
    b = w.R * w.n * 4 + w.n * 4 + w.n * 4
    out["prefill_residual"] = {"us": round(ms * 1e3, 2), "GB/s": round(b / ms / 1e6, 1)}
    # its ceiling: three read streams (the partials and the residual) and one write
    with_ceiling(out["prefill_residual"],
                 pattern_ceiling(torch, stream, 3, 1, [srcs[i] + [ress[i]] for i in range(sets)],
                                 [[d] for d in dsts], w.n * 4, 200))
    log(f"prefill_residual: {out['prefill_residual']}")
    ms = timed(rotating([ar.bind_reduce(ctx, [dsts[i]], srcs[i], w.n, ar.AR_F32, w.wire, ar.AR_MODE_CHUNKED,
                                        stream=stream, residual=row, residual_len=4096) for i in range(sets)]), 200)
    b = w.R * w.n * 4 + w.n * 4 + 4096 * 4
    out["prefill_row_residual"] = {"us": round(ms * 1e3, 2), "GB/s": round(b / ms / 1e6, 1)}
    log(f"prefill_row_residual: {out['prefill_row_residual']}")
    del srcs, dsts, ress
    # the headline call over 16 rotated sets (1.5 GiB touched): past about 1 GiB of touched
    # memory every streaming kernel here, the ceiling kernel included, runs ~8 % slower than
    # at the headline's 768 MiB (not the 256 MiB Infinity Cache: the step lies between 768 MiB
    # and 1152 MiB and does not move when only half of each buffer is touched; not extra DRAM
    # requests or translation misses either, by the counters of --summarize-footprint);
    # reported beside its own ceiling kernel
    big = 16
    srcs = [[torch.randn(w.n, device="cuda") for _ in range(2)] for _ in range(big)]
    dsts = [torch.empty(w.n, device="cuda") for _ in range(big)]

    ms = timed(rotating([ar.bind_reduce(ctx, [dsts[i]], srcs[i], w.n, ar.AR_F32, w.wire, ar.AR_MODE_CHUNKED,
                                        stream=stream) for i in range(big)]), 400)
    b = w.R * w.n * 4 + w.n * 4
    out["prefill_footprint_1536MiB"] = {"us": round(ms * 1e3, 2), "GB/s": round(b / ms / 1e6, 1), "sets": big}
    with_ceiling(out["prefill_footprint_1536MiB"],
                 pattern_ceiling(torch, stream, 2, 1, srcs, [[d] for d in dsts], w.n * 4, 400))
    log(f"prefill_footprint_1536MiB: {out['prefill_footprint_1536MiB']}")
    del srcs, dsts
    torch.cuda.empty_cache()
    # 48 MiB per call: 8 rotated sets (384 MiB) to stay beyond the Infinity Cache
    sets = 8
    srcs = [[torch.from_numpy(wl.as_wire_typed(p, ar.AR_BF16).view(np.int16)).cuda() for p in wl.partials(w, k)]
            for k in range(sets)]
    dsts = [torch.empty(w.n, dtype=torch.int16, device="cuda") for _ in range(sets)]
    ms = timed(rotating([ar.bind_reduce(ctx, [dsts[i]], srcs[i], w.n, ar.AR_BF16, ar.AR_BF16, ar.AR_MODE_CHUNKED,
                                        stream=stream) for i in range(sets)]), 200)
    b = w.R * w.n * 2 + w.n * 2
    out["prefill_bf16_dst"] = {"us": round(ms * 1e3, 2), "GB/s": round(b / ms / 1e6, 1)}
    with_ceiling(out["prefill_bf16_dst"],
                 pattern_ceiling(torch, stream, 2, 1, srcs, [[d] for d in dsts], w.n * 2, 200))
    log(f"prefill_bf16_dst: {out['prefill_bf16_dst']}")
    del srcs, dsts
    # four ranks on the prefill shape with rank 2 inactive (it contributes +0.0 and is not read)
    srcs = [[None if r == 2 else torch.randn(w.n, device="cuda") for r in range(4)] for _ in range(sets)]
    dsts = [torch.empty(w.n, dtype=torch.float32, device="cuda") for _ in range(sets)]
    ms = timed(rotating([ar.bind_reduce(ctx, [dsts[i]], srcs[i], w.n, ar.AR_F32, w.wire,
                                        ar.AR_MODE_CHUNKED | ar.AR_SRC_INACTIVE_NULL, stream=stream)
                         for i in range(sets)]), 200)
    b = 3 * w.n * 4 + w.n * 4
    out["prefill_r4_one_inactive"] = {"us": round(ms * 1e3, 2), "GB/s": round(b / ms / 1e6, 1)}
    with_ceiling(out["prefill_r4_one_inactive"],
                 pattern_ceiling(torch, stream, 3, 1, [[t for t in s if t is not None] for s in srcs],
                                 [[d] for d in dsts], w.n * 4, 200))
    log(f"prefill_r4_one_inactive: {out['prefill_r4_one_inactive']}")
    del srcs, dsts
    # row-strided: the prefill block as a view of wider rows (2048 x 4096 in rows of
    # 4608 for the partials, 4352 for the destination) with a broadcast bias row
    rows, cols, ss, ds = 2048, 4096, 4608, 4352
    sets = 6
    srcs = [[torch.randn(rows * ss, device="cuda") for _ in range(2)] for _ in range(sets)]
    dsts = [torch.empty(rows * ds, device="cuda") for _ in range(sets)]
    bias = torch.randn(cols, device="cuda")
    ms = timed(rotating([ar.bind_reduce_rows(ctx, [dsts[i]], srcs[i], rows, cols, ss, ds, ar.AR_F32, ar.AR_BF16,
                                             ar.AR_MODE_CHUNKED, residual=bias, res_stride=0, stream=stream)
                         for i in range(sets)]), 200)
    b = 2 * rows * cols * 4 + rows * cols * 4 + cols * 4
    out["rows_prefill_block_bias"] = {"us": round(ms * 1e3, 2), "GB/s": round(b / ms / 1e6, 1)}
    log(f"rows_prefill_block_bias: {out['rows_prefill_block_bias']}")
    del srcs, dsts

    # 16-bit partials and destinations: a set is half the fp32 one's 512 MiB, so four
    # sets keep the rotation at 1 GiB (with two, write-through variants read 10-15 %
    # faster than cold because the Infinity Cache still holds part of the set)
    w = wl.WORKLOADS["slice_bcast_f16"]
    bsets = 4
    srcs = [[torch.from_numpy(wl.as_wire_typed(p, ar.AR_F16).view(np.int16)).cuda() for p in wl.partials(w, k)]
            for k in range(bsets)]
    dsts = [[torch.empty(w.n, dtype=torch.int16, device="cuda") for _ in range(w.R)] for _ in range(bsets)]
    ms = timed(rotating([ar.bind_reduce(ctx, dsts[i], srcs[i], w.n, ar.AR_F16, ar.AR_F16, ar.AR_MODE_RS_BCAST,
                                        stream=stream) for i in range(bsets)]), 50)
    b = w.R * w.n * 2 + w.R * w.n * 2
    out["slice_bcast_f16_dst"] = {"us": round(ms * 1e3, 2), "GB/s": round(b / ms / 1e6, 1)}
    with_ceiling(out["slice_bcast_f16_dst"], pattern_ceiling(torch, stream, 4, 4, srcs, dsts, w.n * 2, 50))
    log(f"slice_bcast_f16_dst: {out['slice_bcast_f16_dst']}")
    del srcs, dsts

    w = wl.WORKLOADS["host_staged_bf16"]
    parts = wl.partials(w, 0)
    srcs32 = [torch.from_numpy(p).cuda() for p in parts]
    dst = torch.empty(w.n, dtype=torch.float32, device="cuda")
    ms = timed(rotating([ar.bind_reduce(ctx, [dst], srcs32, w.n, ar.AR_F32, w.wire, ar.AR_MODE_CHUNKED,
                                        stream=stream)]), 20)
    b = w.R * w.n * 4 + w.n * 4
    out["r8_hbm_fp32_src"] = {"us": round(ms * 1e3, 2), "GB/s": round(b / ms / 1e6, 1)}
    with_ceiling(out["r8_hbm_fp32_src"], pattern_ceiling(torch, stream, 8, 1, [srcs32], [[dst]], w.n * 4, 10))
    log(f"r8_hbm_fp32_src: {out['r8_hbm_fp32_src']}")
    # the prefill reduce's kernel on a call 8 x larger (two of the same [8192 x 8192] fp32
    # partials, 768 MiB per call): the per-call fixed cost amortised, beside its ceiling kernel
    ms = timed(rotating([ar.bind_reduce(ctx, [dst], srcs32[:2], w.n, ar.AR_F32, w.wire, ar.AR_MODE_CHUNKED,
                                        stream=stream)]), 30)
    b = 2 * w.n * 4 + w.n * 4
    out["r2_large_fp32_src"] = {"us": round(ms * 1e3, 2), "GB/s": round(b / ms / 1e6, 1), "n": w.n}
    with_ceiling(out["r2_large_fp32_src"], pattern_ceiling(torch, stream, 2, 1, [srcs32[:2]], [[dst]], w.n * 4, 10))
    log(f"r2_large_fp32_src: {out['r2_large_fp32_src']}")
    del srcs32
    pre = [wl.as_wire_typed(p, w.wire) for p in parts]
    srcs16 = [torch.from_numpy(p.view(np.int16)).cuda() for p in pre]
    ms = timed(rotating([ar.bind_reduce(ctx, [dst], srcs16, w.n, ar.AR_F32, w.wire,
                                        ar.AR_MODE_CHUNKED | ar.AR_SRC_WIRE, stream=stream)]), 20)
    b = w.R * w.n * 2 + w.n * 4
    out["r8_hbm_bf16_src"] = {"us": round(ms * 1e3, 2), "GB/s": round(b / ms / 1e6, 1)}
    log(f"r8_hbm_bf16_src: {out['r8_hbm_bf16_src']}")
    del srcs16
    pinned = []
    for p in pre:
        t = torch.empty(p.size, dtype=torch.int16, pin_memory=True)
        t.copy_(torch.from_numpy(p.view(np.int16)))
        pinned.append(t)
    ctx_copy = ar.ar_init(0, {"host_path": 1})
    ms = timed(lambda: ar.ar_reduce(ctx_copy, [dst], pinned, w.n, ar.AR_F32, w.wire,
                                    ar.AR_MODE_HOST_STAGED | ar.AR_SRC_WIRE, stream=stream), 5)
    ms_direct = timed(lambda: ar.ar_reduce(ctx, [dst], pinned, w.n, ar.AR_F32, w.wire,
                                           ar.AR_MODE_HOST_STAGED | ar.AR_SRC_WIRE, stream=stream), 5)
    # the allocation-free entry point: the same copy-engine pipeline staged in the
    # library's 64 MiB static array (one slot: smaller copies than the context's ring)
    ms_static = timed(lambda: ar.ar_reduce_staged_static(ctx_copy, [dst], pinned, w.n, ar.AR_F32, w.wire,
                                                         ar.AR_MODE_HOST_STAGED | ar.AR_SRC_WIRE, stream=stream), 5)
    torch.cuda.synchronize()
    ar.ar_free(ctx_copy)
    pcie_bytes = w.R * w.n * 2
    # plain pinned H2D copy of the same byte count, for the achievable PCIe ceiling
    big = torch.empty(pcie_bytes // 2, dtype=torch.int16, pin_memory=True)
    dev_big = torch.empty_like(big, device="cuda")
    ms_copy = timed(lambda: dev_big.copy_(big, non_blocking=True), 5)
    out["host_staged_bf16"] = {"ms": round(ms, 3), "pcie_GB/s": round(pcie_bytes / ms / 1e6, 2),
                               "h2d_copy_GB/s": round(pcie_bytes / ms_copy / 1e6, 2),
                               "frac_of_h2d_copy": round(ms_copy / ms, 3), "path": "copy engine",
                               # time beyond one plain copy of the same bytes, against the adds'
                               # own time on the same data in HBM (kernel time left exposed <= this)
                               "over_plain_copy_ms": round(ms - ms_copy, 3),
                               "adds_from_hbm_ms": round(out["r8_hbm_bf16_src"]["us"] / 1e3, 3)}
    out["host_direct_bf16"] = {"ms": round(ms_direct, 3), "pcie_GB/s": round(pcie_bytes / ms_direct / 1e6, 2),
                               "frac_of_h2d_copy": round(ms_copy / ms_direct, 3), "path": "kernel reads pinned memory"}
    out["host_static_staging_bf16"] = {"ms": round(ms_static, 3), "pcie_GB/s": round(pcie_bytes / ms_static / 1e6, 2),
                                       "frac_of_h2d_copy": round(ms_copy / ms_static, 3),
                                       "path": "copy engine into the static 64 MiB array, one slot (ar_reduce_staged_static)"}
    log(f"host_static_staging_bf16: {out['host_static_staging_bf16']}")
    log(f"host_staged_bf16: {out['host_staged_bf16']}")
    log(f"host_direct_bf16: {out['host_direct_bf16']}")
    # decode-sized host-staged calls (one hidden vector per rank): latency of each path
    hw = wl.WORKLOADS["decode_bf16"]
    hsrc = []
    for p in wl.partials(hw, 0):
        t = torch.empty(hw.n, dtype=torch.int16, pin_memory=True)
        t.copy_(torch.from_numpy(wl.as_wire_typed(p, hw.wire).view(np.int16)))
        hsrc.append(t)
    hdst = torch.empty(hw.n, dtype=torch.float32, device="cuda")
    ctx_copy = ar.ar_init(0, {"host_path": 1})
    us_copy = timed(lambda: ar.ar_reduce(ctx_copy, [hdst], hsrc, hw.n, ar.AR_F32, hw.wire,
                                         ar.AR_MODE_HOST_STAGED | ar.AR_SRC_WIRE, stream=stream), 500) * 1e3
    us_direct = timed(lambda: ar.ar_reduce(ctx, [hdst], hsrc, hw.n, ar.AR_F32, hw.wire,
                                           ar.AR_MODE_HOST_STAGED | ar.AR_SRC_WIRE, stream=stream), 500) * 1e3
    torch.cuda.synchronize()
    ar.ar_free(ctx_copy)
    out["host_decode_bf16"] = {"us_copy_engine": round(us_copy, 2), "us_direct": round(us_direct, 2)}
    log(f"host_decode_bf16: {out['host_decode_bf16']}")
    ar.ar_free(ctx)
    return out


if __name__ == "__main__":
    sys.exit(main())
