#!/usr/bin/env python3
"""Benchmark of the MI355X GEMM library on one GPU.

    python bench.py [--gpus 1] [--steps 100] [--warmup 100] [--workload sgemm_4096]

One step is one library call on the named workload (default: FP32
C = alpha*A*B + beta*C at M = N = K = 4096, alpha = 1, beta = 0.5, inputs
U[-1, 1] from seed 1).  C is restored from a pristine copy before every call,
outside the timed events.  Each call is bracketed by HIP events on the stream
it is launched on (created without the system-scope fence, which would write
back and invalidate the caches at every record inside the timed interval);
TFLOP/s = 2*M*N*K / mean call time.  The run prints ONE JSON
line with the throughput, the roofline position of the GEMM kernel and the CPU
oracle's own throughput on a bounded sample of the same workload (parity of
this exact launch configuration is checked by the GPU test suite).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOPS at 4096³ FP32 (α,β) + % of MI355X matrix peak per dtype"
PROFILES = os.path.join(ROOT, "profiles")
_CSRC = os.path.join(ROOT, "linear_algebra_sgemm_amd", "csrc")
# The sources that decide what one call of each op runs: its kernels, the shared
# copy helpers and the shape -> configuration choice with its tuned table.
_CHOICE = [os.path.join(_CSRC, f) for f in ("dma_common.h", "gemm_config.cpp", "gemm_tuned.inc")]
KERNEL_SOURCES = {
    "sgemm": [os.path.join(_CSRC, "sgemm_kernels.hip")] + _CHOICE,
    "hgemm_bias_gelu": [os.path.join(_CSRC, "hgemm_kernels.hip")] + _CHOICE,
    "bgemm_bias_gelu": [os.path.join(_CSRC, "hgemm_kernels.hip")] + _CHOICE,
}


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
    return p.parse_args()


def source_digest(paths) -> str:
    """First 16 hex digits of the SHA-256 of the files' contents, in order."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profiled_traffic(workload: str, op: str):
    """HBM bytes per call (all kernels of one call) from the committed rocprofv3 counter
    summary of this workload, or None when there is none or the sources that decide
    what the call runs changed since it was taken."""
    path = os.path.join(PROFILES, "%s_counters.md" % workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_src and m_bytes):
        return None
    if m_src.group(1) != source_digest(KERNEL_SOURCES[op]):
        return None
    return float(m_bytes.group(1))


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
                      % (rows, M, rows, N, K, t)}


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

    A, B, C = inputs.workload_inputs(w)   # C is the bias vector for the half-precision product
    M, N, K = w.M, w.N, w.K

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, A, B, C, args.cpu_seconds)

    lib.gemm_create()
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
        dtype, flops_dtype = "f32", "f32"
        nbytes = cost.sgemm_bytes(M, N, K, w.beta)
    else:
        bf16 = w.op == "bgemm_bias_gelu"
        dbias = C.to(dev)
        dC = torch.empty((M, N), dtype=torch.bfloat16 if bf16 else torch.float16, device=dev)
        fn = lib.bgemm_bias_act if bf16 else lib.hgemm_bias_act

        def call():
            fn(M, N, K, w.alpha, dA, K, dB, N, dbias, lib.ACT_GELU_TANH, dC, N, stream=stream)

        def reset():
            pass
        dtype = flops_dtype = "bf16" if bf16 else "f16"
        nbytes = cost.hgemm_bias_act_bytes(M, N, K)
    flops = cost.gemm_flops(M, N, K)

    for _ in range(args.warmup):
        reset()
        call()
    torch.cuda.synchronize()

    timer = HipTimer(2 * steps)
    handle = stream.cuda_stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        reset()
        timer.record(2 * i, handle)
        call()
        timer.record(2 * i + 1, handle)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [timer.elapsed_ms(2 * i, 2 * i + 1) for i in range(steps)]
    timer.close()
    mean_ms = statistics.fmean(ms)
    tflops = flops / (mean_ms * 1e-3) / 1e12
    peak = cost.PEAK_TFLOPS[flops_dtype]

    traffic = profiled_traffic(w.name, w.op)
    if w.op == "sgemm":
        tile, splits = lib.gemm_debug_pick_config(
            0, M, N, K, torch.cuda.get_device_properties(0).multi_processor_count)
        kernel_name = "%s, tile config %d" % (
            "sgemm_dma_kernel" if tile >= 7 else "sgemm_mfma_kernel", tile)
        if splits > 1:
            kernel_name += ", split-K x%d + sgemm_splitk_reduce_kernel (timed together)" % splits
    else:
        tile, _ = lib.gemm_debug_pick_config(
            1, M, N, K, torch.cuda.get_device_properties(0).multi_processor_count)
        kernel_name = "%s, %s, tile config %d" % (
            "hgemm_dma_kernel" if tile >= 3 else "hgemm_mfma_kernel", dtype, tile)
        if tile == 7:
            kernel_name += " (256x256 head + 128x256 tail launches, timed together)"
    line = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "op": w.op, "M": M, "N": N, "K": K, "alpha": w.alpha,
                   "beta": w.beta, "layout": "row-major, packed",
                   "inputs": "%s, seed %d" % (w.dist_ab, w.seed),
                   "timing": "per-call HIP events (no system-scope fence) on the launch "
                             "stream, C reset before each call outside the events; "
                             "ms_per_step is wall time per step including that reset"},
        "pct_of_peak": round(100.0 * tflops / peak, 2),
        "call_ms": {"mean": round(mean_ms, 5), "median": round(statistics.median(ms), 5),
                    "min": round(min(ms), 5), "max": round(max(ms), 5)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                     "traffic": traffic,
                     "algorithmic_bytes": nbytes,
                     "kernel": kernel_name},
        "cpu_baseline": cpu,
        "device": torch.cuda.get_device_name(0),
    }
    lib.gemm_destroy()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
