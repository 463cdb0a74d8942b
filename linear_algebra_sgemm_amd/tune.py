"""Offline tuner and size sweep for the GEMM library (run on an MI355X).

    python -m linear_algebra_sgemm_amd.tune [--ops sgemm,half] [--min-class 7]
        [--max-class 13] [--table PATH] [--report PATH] [--margin 0.03]

For every size class (M, N, K) = (2^a, 2^b, 2^c), a, b, c in [min, max], and
each op (plus the --extra shapes whose class lies outside that cube, timed at
their own sizes), every legal configuration is timed: each (tile, split count) pair is
forced through the test hooks, the library reports what it would actually run
for the shape (split counts reduced to what K and the workspace allow, direct-
to-LDS tiles replaced where the shape does not suit them) and each distinct
configuration is timed once.  The built-in rule's choice is the baseline; a
class enters the table only when the fastest configuration beats it by more
than the margin.  This is the search of the SGEMM page's kernel k9 (tile
parameters timed on the target GPU, the best kept; section "k7、k8、k9") and
the offline tuning with run-time table lookup of the DeepGEMM page (5.3).

Outputs:
  * the C table `csrc/gemm_tuned.inc` that gemm_config.cpp compiles in (rebuild
    the library afterwards);
  * a markdown report: the square-size sweep 128 ... 8192 per configuration
    (TFLOP/s, the form of the SGEMM page's size heat map, section 尺寸维度) and
    the tuned entries with their gains.

Timing: HIP events around R back-to-back calls on the current stream (median
of three such batches), each batch queued behind about 2 ms of other GPU work
so that the events time the GPU and not the host's launch rate; inputs are seeded U[-1, 1] (FP32) and N(0, 0.02^2)
(fp16) views of one large buffer per operand, beta = 0.5 so repeated calls
stay bounded without resetting C.
"""
from __future__ import annotations

import argparse
import datetime
import json
import os
import statistics
import sys
import time

import torch

import linear_algebra_sgemm_amd as lib
from linear_algebra_sgemm_amd import inputs

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
DEFAULT_TABLE = os.path.join(HERE, "csrc", "gemm_tuned.inc")
DEFAULT_REPORT = os.path.join(ROOT, "profiles", "size_sweep.md")

OPS = {"sgemm": 0, "half": 1}
SGEMM_TILES = (0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13)
HALF_TILES = (0, 1, 2, 3, 4, 5, 6, 7, 8, 9)
SPLITS = (1, 2, 4, 8, 16, 32)
TILE_NAMES = {
    0: {0: "256x256", 1: "128x128", 2: "64x64", 3: "256x256 (BK 32)", 4: "128x256 (2 WG/CU)",
        5: "256x256 (16x16 MFMA)", 6: "128x256 (2 WG/CU, 16x16 MFMA)", 7: "256x256 direct",
        8: "128x256 direct (2 WG/CU)", 9: "256x256 direct, 8 waves",
        10: "128x128 direct (2 WG/CU)", 11: "64x64 direct (4 WG/CU)",
        12: "32x32 (16x16 MFMA, BK 32)", 13: "16x16, K split over 8 waves"},
    1: {0: "256x256 reg", 1: "128x128 reg", 2: "64x64 reg", 3: "256x256 direct",
        4: "128x256 direct", 5: "256x256 direct, 5 stages", 6: "256x256 direct, 8 waves",
        7: "256x256 direct, 8 waves + 128x256 tail", 8: "128x128 direct (2 WG/CU)",
        9: "16x16, K split over 8 waves"},
}


def timed(fn, busy, target_s=0.02, max_reps=50):
    """Mean GPU time per call in ms: median of three batches of back-to-back calls.

    Each batch is queued behind `busy` (about 2 ms of GPU work), so the host has
    enqueued the whole batch before the first call starts and the events measure
    GPU time, not the host's launch rate."""
    def batch(reps):
        busy()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps

    fn()
    torch.cuda.synchronize()
    est = max(batch(3) * 1e-3, 1e-7)
    reps = int(min(max_reps, max(3, target_s / est)))
    return statistics.median(batch(reps) for _ in range(3))


def make_busy(dev):
    """About 2 ms of GPU work: two 4096^3 FP32 products on buffers of their own."""
    n = 4096
    A = torch.rand((n, n), device=dev)
    B = torch.rand((n, n), device=dev)
    C = torch.zeros((n, n), device=dev)
    pa, pb, pc = A.data_ptr(), B.data_ptr(), C.data_ptr()
    keep = (A, B, C)

    def busy():
        _ = keep
        lib.sgemm(n, n, n, 1.0, pa, n, pb, n, 0.0, pc, n)
        lib.sgemm(n, n, n, 1.0, pa, n, pb, n, 0.0, pc, n)
    return busy


class Buffers:
    """One device buffer per operand, large enough for the biggest class."""

    def __init__(self, op, nmax, dev):
        if op == 0:
            A, B, C = inputs.sgemm_inputs(nmax, nmax, nmax, seed=97)
            self.A, self.B, self.C = A.to(dev), B.to(dev), C.to(dev)
        else:
            A, B, bias = inputs.hgemm_inputs(nmax, nmax, nmax, seed=98)
            self.A, self.B = A.to(dev), B.to(dev)
            self.bias = bias.to(dev)
            self.C = torch.empty((nmax, nmax), dtype=torch.float16, device=dev)


def call_for(op, buf, M, N, K):
    if op == 0:
        A, B, C = buf.A.data_ptr(), buf.B.data_ptr(), buf.C.data_ptr()
        return lambda: lib.sgemm(M, N, K, 1.0, A, K, B, N, 0.5, C, N)
    A, B, C, bias = buf.A.data_ptr(), buf.B.data_ptr(), buf.C.data_ptr(), buf.bias.data_ptr()
    return lambda: lib.hgemm_bias_act(M, N, K, 1.0, A, K, B, N, bias, lib.ACT_GELU_TANH, C, N)


def candidates(op, M, N, K, cus):
    """Distinct (tile, splits) the library would run, over every forced pair."""
    seen = []
    tiles = SGEMM_TILES if op == 0 else HALF_TILES
    try:
        for t in tiles:
            lib.gemm_debug_force_tile(op, t)
            for s in SPLITS:
                lib.gemm_debug_force_splits(op, s)
                cfg = lib.gemm_debug_pick_config(op, M, N, K, cus)
                if cfg not in seen:
                    seen.append(cfg)
    finally:
        lib.gemm_debug_force_tile(op, -1)
        lib.gemm_debug_force_splits(op, -1)
    return seen


def force(op, cfg):
    lib.gemm_debug_force_tile(op, cfg[0])
    lib.gemm_debug_force_splits(op, cfg[1])


def unforce(op):
    lib.gemm_debug_force_tile(op, -1)
    lib.gemm_debug_force_splits(op, -1)


def size_class(x):
    """The library's size class of a dimension: log2 rounded, clamped to 7..14."""
    import math
    c = round(math.log2(x)) if x > 1 else 7
    return min(max(c, 7), 14)


def tune_op(op, lo, hi, margin, cus, dev, log, busy, extra=()):
    """Time every class of the cube [lo, hi]^3 (aligned power-of-two shapes) and the
    extra shapes whose class lies outside it (timed at their own sizes)."""
    buf = Buffers(op, 1 << hi, dev)
    results = {}      # class (a, b, c) -> {cfg: ms}
    rule = {}         # class -> cfg
    dims = {}         # class -> (M, N, K) that was timed
    entries = []
    shapes = [(1 << a, 1 << b, 1 << c) for a in range(lo, hi + 1) for b in range(lo, hi + 1)
              for c in range(lo, hi + 1)]
    for (M, N, K) in extra:
        key = (size_class(M), size_class(N), size_class(K))
        if all(lo <= k <= hi for k in key):
            continue
        if (M * K > buf.A.numel()) or (K * N > buf.B.numel()) or (M * N > buf.C.numel()):
            raise ValueError("extra shape %dx%dx%d does not fit the %d^2 buffers" % (M, N, K, 1 << hi))
        shapes.append((M, N, K))
    for (M, N, K) in shapes:
        key = (size_class(M), size_class(N), size_class(K))
        fn = call_for(op, buf, M, N, K)
        lib.gemm_debug_use_tuned_table(False)
        base = lib.gemm_debug_pick_config(op, M, N, K, cus)
        times = {}
        for cfg in candidates(op, M, N, K, cus):
            force(op, cfg)
            try:
                times[cfg] = timed(fn, busy)
            finally:
                unforce(op)
        lib.gemm_debug_use_tuned_table(True)
        results[key] = times
        rule[key] = base
        dims[key] = (M, N, K)
        best = min(times, key=times.get)
        gain = times[base] / times[best] - 1.0
        if best != base and times[best] < times[base] * (1.0 - margin):
            entries.append((op,) + key + (best[0], best[1], times[base], times[best]))
        log("op %d %5d x %5d x %5d  rule %s %.4f ms  best %s %.4f ms  (%+.1f%%)"
            % (op, M, N, K, base, times[base], best, times[best], 100 * gain))
    del buf
    torch.cuda.empty_cache()
    return results, rule, entries, dims


def write_table(path, entries, header):
    lines = ["// Offline-tuned shape -> configuration entries, written by",
             "// linear_algebra_sgemm_amd/tune.py; do not edit by hand.",
             "// " + header,
             "// {op, class of M, class of N, class of K, tile, splits}: class = log2 of the",
             "// size rounded to the nearest integer; op 0 = sgemm, 1 = the half products."]
    for (op, a, b, c, t, s, _, _) in entries:
        lines.append("{%d, %d, %d, %d, %d, %d}," % (op, a, b, c, t, s))
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def flops(dims):
    M, N, K = dims
    return 2.0 * M * N * K


def write_report(path, all_results, header, command, margin):
    out = ["# Size sweep and tuned configurations", "",
           "Written by `linear_algebra_sgemm_amd/tune.py` (%s)." % header, "",
           "Command ($REPO = repository root on the MI355X machine that ran it):", "", "    " + command, "",
           "TFLOP/s = 2·M·N·K / mean GPU time per call (HIP events around back-to-back calls "
           "queued behind other GPU work, so host launch time is excluded; median of three "
           "batches). FP32: α = 1, β = 0.5. Half: fp16, bias + GELU(tanh). "
           "A class enters the tuned table when its best configuration beats the built-in rule "
           "by more than %.0f %%." % (100 * margin), ""]
    for op, (results, rule, entries, dims) in all_results.items():
        name = "FP32 sgemm" if op == 0 else "FP16 bias + GELU (the BF16 product runs the same kernels)"
        squares = sorted(k for k in results if k[0] == k[1] == k[2])
        out += ["## %s: square sizes" % name, ""]
        out.append("| Configuration | " + " | ".join(str(1 << k[0]) for k in squares) + " |")
        out.append("|---|" + "---|" * len(squares))
        cfgs = sorted({cfg for k in squares for cfg in results[k]})
        for cfg in cfgs:
            if cfg[1] != 1:
                continue
            row = []
            for k in squares:
                ms = results[k].get(cfg)
                row.append("%.1f" % (flops(dims[k]) / ms / 1e9) if ms else "—")
            out.append("| tile %d %s | " % (cfg[0], TILE_NAMES[op][cfg[0]]) + " | ".join(row) + " |")
        for label, choose in (("built-in rule", lambda k: rule[k]),
                              ("best (any split)", lambda k: min(results[k], key=results[k].get))):
            row = []
            for k in squares:
                cfg = choose(k)
                row.append("%.1f %s" % (flops(dims[k]) / results[k][cfg] / 1e9, _cfg_str(cfg)))
            out.append("| %s | " % label + " | ".join(row) + " |")
        out += ["", "## %s: tuned entries (%d of %d classes)" % (name, len(entries), len(results)),
                "", "| M | N | K | rule | rule TFLOP/s | tuned | tuned TFLOP/s | gain |",
                "|---|---|---|---|---|---|---|---|"]
        for (o, a, b, c, t, s, tb, tt) in sorted(entries, key=lambda e: e[6] / e[7], reverse=True):
            d = dims[(a, b, c)]
            out.append("| %d | %d | %d | %s | %.1f | %s | %.1f | %+.1f %% |" % (
                d[0], d[1], d[2], _cfg_str(rule[(a, b, c)]), flops(d) / tb / 1e9,
                _cfg_str((t, s)), flops(d) / tt / 1e9, 100 * (tb / tt - 1)))
        extra_keys = [k for k in results if max(k) > max(squares)[0] or min(k) < min(squares)[0]]
        if extra_keys:
            out += ["", "## %s: extra shapes (size classes outside the cube)" % name, "",
                    "| M | N | K | TFLOP/s per configuration | rule |", "|---|---|---|---|---|"]
            for k in extra_keys:
                d = dims[k]
                cells = ", ".join("%s %.1f" % (_cfg_str(c), flops(d) / results[k][c] / 1e9)
                                  for c in sorted(results[k]))
                out.append("| %d | %d | %d | %s | %s |" % (d + (cells, _cfg_str(rule[k]))))
        out.append("")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")


def _cfg_str(cfg):
    return "t%d" % cfg[0] + ("×%d" % cfg[1] if cfg[1] > 1 else "")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--ops", default="sgemm,half")
    ap.add_argument("--min-class", type=int, default=7)
    ap.add_argument("--max-class", type=int, default=13)
    ap.add_argument("--margin", type=float, default=0.03)
    ap.add_argument("--table", default=DEFAULT_TABLE)
    ap.add_argument("--report", default=DEFAULT_REPORT)
    ap.add_argument("--dump", default=None, help="also write every timing as JSON here")
    ap.add_argument("--extra", default="half:4096x14336x4096",
                    help="comma-separated op:MxNxK shapes tuned at their own sizes when their "
                         "size class lies outside the cube")
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        sys.exit("the tuner times kernels and needs a GPU")
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    lib.gemm_create()
    header = "%s, %d CUs, %s, classes %d..%d" % (
        props.name, cus, datetime.date.today().isoformat(), args.min_class, args.max_class)
    command = "python -m linear_algebra_sgemm_amd.tune " + " ".join(argv if argv is not None
                                                                   else sys.argv[1:])
    t0 = time.time()

    def log(msg):
        print("[%6.1fs] %s" % (time.time() - t0, msg), flush=True)

    all_results = {}
    entries = []
    try:
        busy = make_busy(dev)
        for name in args.ops.split(","):
            op = OPS[name]
            extra = [tuple(int(x) for x in e.split(":")[1].split("x"))
                     for e in args.extra.split(",") if e and e.split(":")[0] == name]
            res = tune_op(op, args.min_class, args.max_class, args.margin, cus, dev, log, busy,
                          extra)
            all_results[op] = res
            entries += res[2]
    finally:
        lib.gemm_destroy()
    for p in (args.table, args.report):
        d = os.path.dirname(os.path.abspath(p))
        os.makedirs(d, exist_ok=True)
    if args.dump:
        dump = {str(op): {"%d,%d,%d" % k: {"rule": list(rule[k]),
                                            "ms": {"%d,%d" % cfg: ms for cfg, ms in times.items()}}
                          for k, times in results.items()}
                for op, (results, rule, _, _) in all_results.items()}
        with open(args.dump, "w") as f:
            json.dump(dump, f)
    # Ops not tuned in this run keep their entries from the compiled-in table.
    tuned_ops = set(all_results)
    kept = []
    if os.path.exists(DEFAULT_TABLE):
        for line in open(DEFAULT_TABLE):
            line = line.strip()
            if line.startswith("{") and line.endswith("},"):
                vals = [int(x) for x in line[1:-2].split(",")]
                if vals[0] not in tuned_ops:
                    kept.append(tuple(vals) + (0.0, 0.0))
    write_table(args.table, kept + entries, header)
    write_report(args.report, all_results, header, command, args.margin)
    log("wrote %s (%d entries) and %s" % (args.table, len(entries), args.report))


if __name__ == "__main__":
    main()
