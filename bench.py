#!/usr/bin/env python3
"""Benchmark of the MI355X GEMM library on one GPU.

    python bench.py [--gpus 1] [--steps 100] [--warmup 100] [--workload sgemm_4096]

One step is one library call on the named workload (default: FP32
C = alpha*A*B + beta*C at M = N = K = 4096, alpha = 1, beta = 0.5, inputs
U[-1, 1] from seed 1).  C is restored from a pristine copy before every call,
outside the timed events.  Each call is bracketed by HIP events on the stream
it is launched on (created without the system-scope fence, which would write
back and invalidate the caches at every record inside the timed interval);
TFLOP/s = 2*M*N*K / mean call time.  Before its --warmup calls each workload
runs untimed until its call time stops falling (the card's clock settles over
the first tens of calls; at most --settle-seconds).  The default run also times the
inference-FFN product (M = 4096, N = 14336, K = 4096, bias + GELU) in binary16
and in bfloat16, for the percentage of the matrix peak of each dtype.  After
the GPU phase, every element of each workload's first timed output is compared
with the CPU oracle.  The run prints ONE JSON line with the throughput, the
roofline position of the GEMM kernel, the per-dtype figures, the parity result
and the CPU oracle's own throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOPS at 4096³ FP32 (α,β) + % of MI355X matrix peak per dtype"
PROFILES = os.path.join(ROOT, "profiles")

class HipTimer:
    """Timing events of the HIP runtime the process already uses (torch's), created
    with hipEventDisableSystemFence: a record then only marks the point in the
    stream, without the system-scope cache write-back and invalidation that the
    default event flags add around it (which the HIP runtime documents as
    distorting short timings)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, count: int):
        import ctypes
        self._ct = ctypes
        self._hip = ctypes.CDLL("libamdhip64.so.7")
        self._hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self._hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                  ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []
        for _ in range(count):
            ev = ctypes.c_void_p()
            self._check(self._hip.hipEventCreateWithFlags(ctypes.byref(ev), self.DISABLE_SYSTEM_FENCE),
                        "hipEventCreateWithFlags")
            self.events.append(ev.value)

    def _check(self, err, what):
        if err != 0:
            raise RuntimeError("%s failed with HIP error %d" % (what, err))

    def record(self, i: int, stream_handle: int):
        self._check(self._hip.hipEventRecord(self.events[i], stream_handle), "hipEventRecord")

    def elapsed_ms(self, i: int, j: int) -> float:
        out = self._ct.c_float()
        self._check(self._hip.hipEventElapsedTime(self._ct.byref(out), self.events[i],
                                                  self.events[j]), "hipEventElapsedTime")
        return float(out.value)

    def close(self):
        for ev in self.events:
            self._hip.hipEventDestroy(ev)
        self.events = []


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    # The card raises its clocks over the first tens of milliseconds of load: 100
    # untimed calls (about 0.1 s at 4096^3) reach the steady state.
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--workload", default="sgemm_4096")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target CPU time of the oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-parity", action="store_true",
                   help="skip the oracle comparison of the first timed call's output")
    p.add_argument("--swizzle", default=None, metavar="GROUP,REMAP",
                   help="tile order for a counter comparison: rows per group (0 = each "
                        "launch's own) and the XCD renumbering (1 on, 0 off)")
    p.add_argument("--settle-seconds", type=float, default=SETTLE_MAX_S,
                   help="longest untimed settling phase per workload before its warm-up "
                        "calls (0 = none); it ends once the call time stops falling")
    p.add_argument("--headline-first", action="store_true",
                   help="time --workload before the per-dtype workloads instead of after them")
    p.add_argument("--no-extras", action="store_true",
                   help="time only --workload (by default the 4096^3 FP32 run also times the "
                        "binary16 and bfloat16 FFN products)")
    return p.parse_args()


def profiled_figures(workload: str, op: str):
    """Figures per call from the committed rocprofv3 counter summary of this workload:
    HBM bytes ("traffic"), the effective clock and MfmaUtil under the counter passes;
    None when there is no summary or the sources that decide what the call runs
    changed since it was taken."""
    path = os.path.join(PROFILES, "%s_counters.md" % workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    if not m_src:
        return None
    from linear_algebra_sgemm_amd.profile_summary import source_digest
    if m_src.group(1) != source_digest(op):
        return None
    out = {}
    for key, name in (("traffic", "hbm_bytes_per_launch"), ("effective_clock_ghz",
                                                           "effective_clock_ghz"),
                      ("mfma_util_pct", "mfma_util_pct")):
        m = re.search(r"%s:\s*([0-9.eE+]+)" % name, text)
        out[key] = float(m.group(1)) if m else None
    return out


def profiled_traffic(workload: str, op: str):
    """HBM bytes per call from the committed counter summary, or None (see profiled_figures)."""
    f = profiled_figures(workload, op)
    return None if f is None else f["traffic"]


def cpu_baseline(w, A, B, C, target_seconds: float):
    """Time the CPU oracle (as it stands) on the first rows of the same workload."""
    import torch

    import oracle
    from linear_algebra_sgemm_amd import cost
    threads = oracle.max_threads()
    M, N, K = w.M, w.N, w.K

    def run(rows):
        t0 = time.perf_counter()
        if w.op == "sgemm":
            oracle.sgemm(rows, N, K, w.alpha, A[:rows].numpy(), K, B.numpy(), N, w.beta,
                         C[:rows].numpy(), N, with_den=False)
        else:
            a = A[:rows].contiguous().view(torch.int16).numpy().view("uint16")
            b = B.contiguous().view(torch.int16).numpy().view("uint16")
            oracle.hgemm_bias_act(rows, N, K, w.alpha, a, K, b, N, C.numpy(),
                                  oracle.ACT_GELU_TANH, with_den=False,
                                  fmt="bf16" if w.op == "bgemm_bias_gelu" else "f16")
        return time.perf_counter() - t0

    probe = min(M, 16)
    t_probe = run(probe)
    rows = int(max(probe, min(M, probe * target_seconds / max(t_probe, 1e-6))))
    rows = max(probe, (rows // 8) * 8) if rows < M else M
    t = run(rows)
    tf = cost.gemm_flops(rows, N, K) / t / 1e12
    return {"value": tf, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d output rows (%d x %d x %d), fp64 accumulation, %.1f s"
                      % (rows, M, rows, N, K, t),
            "cpu_model": cpu_model()}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def parity(w, A, B, C, got):
    """Every element of the first timed call's output against the CPU oracle: the largest
    normalised error |C - ref| / (|alpha| sum_k |a||b| + |beta||c| or |bias|) and where."""
    import numpy as np
    import torch

    import oracle
    M, N, K = w.M, w.N, w.K
    t0 = time.perf_counter()
    floor = 0.0
    if w.op == "sgemm":
        ref, den = oracle.sgemm(M, N, K, w.alpha, A.numpy(), K, B.numpy(), N, w.beta, C.numpy(), N)
        tol = 1e-5
    else:
        bits = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
        fmt = "bf16" if w.op == "bgemm_bias_gelu" else "f16"
        ref, den = oracle.hgemm_bias_act(M, N, K, w.alpha, bits(A), K, bits(B), N, C.numpy(),
                                         oracle.ACT_GELU_TANH, fmt=fmt)
        tol = 1e-2
        floor = oracle.OUTPUT_FLOOR[fmt]
    e = oracle.normalized_error(got.float().numpy(), ref, den, floor)
    k = int(np.argmax(e))
    return {"max_err": float(e[k // N, k % N]), "where": [k // N, k % N], "tol": tol,
            "entries": M * N, "pass": bool(e.max() <= tol),
            "oracle_s": round(time.perf_counter() - t0, 2)}


# Settling: untimed calls before the warm-up calls, in groups of SETTLE_GROUP, until
# the median call time of a group is no longer SETTLE_DROP below the previous
# group's (at least SETTLE_MIN_GROUPS groups, at most SETTLE_MAX_S seconds).  A card
# that has been idle raises its clock over the first tens of calls, and one that
# has just run power-limited 16-bit work starts the next workload at a lower clock;
# five warm-up calls do not cover that (4096^3 FP32: 1.08 ms for the first calls,
# 0.94 ms once settled).
#
# The first group has SETTLE_GROUP calls; every later one enough calls for about
# SETTLE_GROUP_MS of call time (at most SETTLE_GROUP_MAX calls).  The clock rises over
# tens of milliseconds of load, not over a number of calls, so a short call needs
# large groups for the rule to see the rise: 1000 x 3000 x 777 took 51.5 us per call
# after three groups of ten calls, and 47 us after about 70 ms of calls.
SETTLE_GROUP = 10
SETTLE_GROUP_MS = 20.0
SETTLE_GROUP_MAX = 2000
SETTLE_MIN_GROUPS = 3
SETTLE_DROP = 0.005
SETTLE_MAX_S = 3.0


def settle_groups(time_group, max_s: float, clock=time.perf_counter):
    """The settling rule: time_group() runs one group of untimed calls and returns
    their times (ms); groups run until a group's median is no longer
    SETTLE_DROP below the previous group's (after at least SETTLE_MIN_GROUPS groups) or
    max_s seconds have passed.  Returns the number of calls and each group's median."""
    if max_s <= 0:
        return 0, []
    medians = []
    t0 = clock()
    calls = 0
    while True:
        times = time_group()
        medians.append(statistics.median(times))
        calls += len(times)
        settled = (len(medians) >= SETTLE_MIN_GROUPS and
                   medians[-1] >= (1.0 - SETTLE_DROP) * medians[-2])
        if settled or clock() - t0 > max_s:
            break
    return calls, [round(m, 4) for m in medians]


def settle_group_size(call_ms: float) -> int:
    """Calls in a settling group after the first, for calls of call_ms each."""
    want = int(math.ceil(SETTLE_GROUP_MS / max(call_ms, 1e-6)))
    return min(SETTLE_GROUP_MAX, max(SETTLE_GROUP, want))


def settle(call, reset, handle, max_s: float):
    """Untimed calls of one workload until the per-call time has stopped falling
    (settle_groups), each call between two HIP events on the launch stream."""
    import torch

    if max_s <= 0:
        return 0, []
    state = {"n": SETTLE_GROUP, "timer": HipTimer(2 * SETTLE_GROUP)}

    def time_group():
        n, timer = state["n"], state["timer"]
        for i in range(n):
            reset()
            timer.record(2 * i, handle)
            call()
            timer.record(2 * i + 1, handle)
        torch.cuda.synchronize()
        ms = [timer.elapsed_ms(2 * i, 2 * i + 1) for i in range(n)]
        want = settle_group_size(statistics.median(ms))
        if want != n:
            timer.close()
            state["n"], state["timer"] = want, HipTimer(2 * want)
        return ms

    try:
        return settle_groups(time_group, max_s)
    finally:
        state["timer"].close()


def time_workload(w, steps: int, warmup: int, settle_s: float = SETTLE_MAX_S):
    """Settling calls, warm-up calls, then `steps` timed calls of one workload on the
    current stream.  Returns the per-call times (ms), the settling record, the host
    inputs and a copy of the first timed call's output (taken after its end event,
    outside the timed interval)."""
    import torch

    import linear_algebra_sgemm_amd as lib
    from linear_algebra_sgemm_amd import inputs

    A, B, C = inputs.workload_inputs(w)   # C is the bias vector for the half-precision product
    M, N, K = w.M, w.N, w.K
    dev = torch.device("cuda:0")
    dA, dB = A.to(dev), B.to(dev)
    stream = torch.cuda.current_stream()
    if w.op == "sgemm":
        dC0 = C.to(dev)
        dC = dC0.clone()

        def call():
            lib.sgemm(M, N, K, w.alpha, dA, K, dB, N, w.beta, dC, N, stream=stream)

        def reset():
            dC.copy_(dC0)
    else:
        bf16 = w.op == "bgemm_bias_gelu"
        dbias = C.to(dev)
        dC = torch.empty((M, N), dtype=torch.bfloat16 if bf16 else torch.float16, device=dev)
        fn = lib.bgemm_bias_act if bf16 else lib.hgemm_bias_act

        def call():
            fn(M, N, K, w.alpha, dA, K, dB, N, dbias, lib.ACT_GELU_TANH, dC, N, stream=stream)

        def reset():
            pass

    handle = stream.cuda_stream
    settle_calls, settle_ms = settle(call, reset, handle, settle_s)
    for _ in range(warmup):
        reset()
        call()
    torch.cuda.synchronize()

    timer = HipTimer(2 * steps)
    first = torch.empty_like(dC)
    if w.op != "sgemm":
        dC.fill_(float("nan"))   # the first timed call must write every element itself
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        reset()
        timer.record(2 * i, handle)
        call()
        timer.record(2 * i + 1, handle)
        if i == 0:
            first.copy_(dC)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [timer.elapsed_ms(2 * i, 2 * i + 1) for i in range(steps)]
    timer.close()
    out = first.cpu()
    del dA, dB, dC, first
    return {"ms": ms, "wall_s": wall, "inputs": (A, B, C), "first": out,
            "settle": {"calls": settle_calls, "group_median_ms": settle_ms}}


def call_stats(ms):
    srt = sorted(ms)
    p90 = srt[min(len(srt) - 1, int(round(0.9 * (len(srt) - 1))))]
    return {"mean": round(statistics.fmean(ms), 5), "median": round(statistics.median(ms), 5),
            "min": round(min(ms), 5), "p90": round(p90, 5), "max": round(max(ms), 5),
            "stdev": round(statistics.stdev(ms), 5) if len(ms) > 1 else 0.0,
            "first": [round(x, 4) for x in ms[:8]], "last": [round(x, 4) for x in ms[-8:]]}


def kernel_label(w, dtype: str) -> str:
    import torch

    import linear_algebra_sgemm_amd as lib
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if w.op == "sgemm":
        tile, splits = lib.gemm_debug_pick_config(0, w.M, w.N, w.K, cus)
        name = "%s, tile config %d" % ("sgemm_dma_kernel" if tile >= 7 else "sgemm_mfma_kernel",
                                       tile)
        if splits > 1:
            name += ", split-K x%d + sgemm_splitk_reduce_kernel (timed together)" % splits
        return name
    tile, splits = lib.gemm_debug_pick_config(1, w.M, w.N, w.K, cus)
    name = "%s, %s, tile config %d" % ("hgemm_dma_kernel" if tile >= 3 else "hgemm_mfma_kernel",
                                       dtype, tile)
    if splits > 1:
        name += ", split-K x%d + half_splitk_reduce_kernel (timed together)" % splits
    return name


# The half-precision workloads measured beside the FP32 headline ("% of MI355X matrix
# peak per dtype"): the FFN product in binary16 and in bfloat16.
PER_DTYPE_EXTRAS = ("hgemm_ffn", "bgemm_ffn")
EXTRA_MIN_STEPS = 50
EXTRA_MIN_WARMUP = 10


def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this library has no multi-GPU path "
              "(--gpus %d was asked for)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import linear_algebra_sgemm_amd as lib
    from linear_algebra_sgemm_amd import cost, inputs

    if args.workload not in inputs.WORKLOADS:
        sys.exit("unknown workload %s (known: %s)" % (args.workload, ", ".join(inputs.WORKLOADS)))
    w = inputs.WORKLOADS[args.workload]
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    steps = max(1, args.steps)
    extras = [] if (args.no_extras or args.workload != "sgemm_4096") else list(PER_DTYPE_EXTRAS)

    cpu = None
    if not args.no_cpu_baseline:
        A, B, C = inputs.workload_inputs(w)
        cpu = cpu_baseline(w, A, B, C, args.cpu_seconds)
        del A, B, C

    lib.gemm_create()
    if args.swizzle:
        g, r = (int(x) for x in args.swizzle.split(","))
        if lib.gemm_debug_force_swizzle(g, bool(r)) != lib.STATUS_SUCCESS:
            sys.exit("invalid --swizzle %s" % args.swizzle)
    # GPU phase: every timed workload, the headline one last; the CPU checks follow.
    # The per-dtype workloads take at least 50 timed calls after at least 10 warm-up
    # calls (the reporting rule of these workloads); the headline takes exactly
    # --steps after --warmup.
    runs = {}
    if args.headline_first:
        runs[w.name] = time_workload(w, steps, args.warmup, args.settle_seconds)
    for name in extras:
        runs[name] = time_workload(inputs.WORKLOADS[name], max(steps, EXTRA_MIN_STEPS),
                                   max(args.warmup, EXTRA_MIN_WARMUP), args.settle_seconds)
    if not args.headline_first:
        runs[w.name] = time_workload(w, steps, args.warmup, args.settle_seconds)
    lib.gemm_destroy()

    def dtype_of(wl):
        return {"sgemm": "f32", "hgemm_bias_gelu": "f16", "bgemm_bias_gelu": "bf16"}[wl.op]

    per_dtype = {}
    for name, r in runs.items():
        wl = inputs.WORKLOADS[name]
        dt = dtype_of(wl)
        st = call_stats(r["ms"])
        tf = cost.gemm_flops(wl.M, wl.N, wl.K) / (st["mean"] * 1e-3) / 1e12
        entry = {"workload": name, "steps": len(r["ms"]), "tflops": round(tf, 3),
                 "pct_of_peak": round(100.0 * tf / cost.PEAK_TFLOPS[dt], 2),
                 "peak_tflops": cost.PEAK_TFLOPS[dt], "call_ms": st, "settle": r["settle"],
                 "kernel": kernel_label(wl, dt)}
        if not args.no_parity:
            A, B, C = r["inputs"]
            entry["parity"] = parity(wl, A, B, C, r["first"])
        per_dtype[dt] = entry

    main_run = runs[w.name]
    dtype = dtype_of(w)
    st = call_stats(main_run["ms"])
    mean_ms = st["mean"]
    flops = cost.gemm_flops(w.M, w.N, w.K)
    tflops = flops / (mean_ms * 1e-3) / 1e12
    peak = cost.PEAK_TFLOPS[dtype]
    nbytes = (cost.sgemm_bytes(w.M, w.N, w.K, w.beta) if w.op == "sgemm"
              else cost.hgemm_bias_act_bytes(w.M, w.N, w.K))
    A, B, C = main_run["inputs"]
    par = per_dtype[dtype].get("parity")
    line = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "settle": main_run["settle"],
        "ms_per_step": round(main_run["wall_s"] / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "op": w.op, "M": w.M, "N": w.N, "K": w.K,
                   "alpha": w.alpha, "beta": w.beta, "layout": "row-major, packed",
                   "inputs": "%s, seed %d" % (w.dist_ab, w.seed),
                   "inputs_sha256": inputs.sha256(A, B, C),
                   "tile_order": args.swizzle or "default",
                   "timing": "per-call HIP events (no system-scope fence) on the launch "
                             "stream, C reset before each call outside the events; "
                             "untimed settling calls until the call time stops falling, "
                             "then the warm-up calls; ms_per_step is wall time per step "
                             "including that reset"},
        "pct_of_peak": round(100.0 * tflops / peak, 2),
        "call_ms": st,
        "parity_max_err": None if par is None else par["max_err"],
        "parity": par,
        "per_dtype": per_dtype,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                     "traffic": profiled_traffic(w.name, w.op),
                     "profiled": profiled_figures(w.name, w.op),
                     "algorithmic_bytes": nbytes,
                     "kernel": kernel_label(w, dtype)},
        "cpu_baseline": cpu,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line), flush=True)
    if par is not None and not par["pass"]:
        sys.exit("parity failed: max normalised error %.3g > %g" % (par["max_err"], par["tol"]))


if __name__ == "__main__":
    main()
