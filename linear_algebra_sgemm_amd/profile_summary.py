"""Markdown summaries of rocprofv3 output for the files under profiles/.

    python -m linear_algebra_sgemm_amd.profile_summary trace --workload W \
        --stats DIR/run_kernel_stats.csv --command "CMD" --out profiles/W_kernel_trace.md
    python -m linear_algebra_sgemm_amd.profile_summary counters --workload W \
        --pass DIR1/run_counter_collection.csv --pass DIR2/... --command "CMD1" --command ... \
        [--resources] --out profiles/W_counters.md

Host-side text processing only (no GPU).  A kernel trace summary tabulates
rocprofv3's per-kernel statistics.  A counter summary averages each counter
over the dispatches of every library kernel (names in the ``lasg::`` namespace)
and sums those averages over the kernels of one call; it converts the cache
counters FETCH_SIZE and WRITE_SIZE (KiB) into HBM bytes with scale factors
measured in the same runs on the plain device copy (``__amd_rocclr_copyBuffer``)
of the workload's output, whose size is known; it derives the effective clock
(GRBM_GUI_ACTIVE summed over the eight XCDs, over the dispatch duration), the
FLOPs the matrix cores executed (MOPS x 512, which equals 2 M N K for a product
on whole tiles) and the LDS bank-conflict rate; and it records the digest of the
sources that decide what one call runs, so that a summary taken before a kernel
or the configuration choice changed is recognised as stale (the benchmark then
reports no traffic figure).  Register and scratch counts come from the
compiler's resource remarks (``resource_usage``).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
import statistics
import sys
from collections import defaultdict

_HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(_HERE, "csrc")
ROOT = os.path.dirname(_HERE)

# The sources that decide what one call of each op runs: its kernels, the copy
# kernels, the shared device helpers (copies, tile order), the C entry points with
# their planning, and the shape -> configuration choice with its tuned table.
_SHARED = ["pack_kernels.hip", "dma_common.h", "gemm_common.h", "gemm_launch.h", "gemm_capi.cpp",
           "gemm_config.cpp", "gemm_tuned.inc"]
KERNEL_SOURCES = {
    "sgemm": ["sgemm_kernels.hip"] + _SHARED,
    "hgemm_bias_gelu": ["hgemm_kernels.hip"] + _SHARED,
    "bgemm_bias_gelu": ["hgemm_kernels.hip"] + _SHARED,
}

LIB_PREFIX = "lasg::"
COPY_KERNEL = "__amd_rocclr_copyBuffer"
XCDS = 8
# Shortest dispatch whose effective clock is reported.
MIN_CLOCK_NS = 100e3


_COMMENT = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def code_only(text: str) -> str:
    """C++ source without its comments and with runs of whitespace collapsed: what the
    compiler sees, so that an edit of a comment leaves the digest alone.  (The sources
    hold no string literal with a comment marker in it.)"""
    return " ".join(_COMMENT.sub(" ", text).split())


def source_digest(op: str) -> str:
    """First 16 hex digits of the SHA-256 of the op's deciding sources (code only,
    comments removed), in order."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[op]:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_csv(path: str):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _col(row, *names, default=None):
    for n in names:
        if n in row and row[n] not in (None, ""):
            return row[n]
    return default


def _num(x):
    try:
        return float(x)
    except (TypeError, ValueError):
        return None


# ---------------------------------------------------------------------------
# Kernel trace statistics
# ---------------------------------------------------------------------------

def trace_table(stats_csv: str):
    """(kernel, calls, average ns, min ns, max ns, percent) rows, most time first."""
    rows = []
    for r in read_csv(stats_csv):
        rows.append((_col(r, "Name", "KERNEL_NAME", "Kernel_Name"),
                     int(float(_col(r, "Calls", "CALLS", default=0))),
                     _num(_col(r, "AverageNs", "AVERAGE_NS")),
                     _num(_col(r, "MinNs", "MIN_NS")),
                     _num(_col(r, "MaxNs", "MAX_NS")),
                     _num(_col(r, "Percentage", "PERCENTAGE"))))
    rows.sort(key=lambda t: -(t[5] or 0.0))
    return rows


def trace_markdown(workload: str, stats_csv: str, command: str, note: str = "") -> str:
    lines = ["# Kernel trace: workload `%s`" % workload, "",
             "Command ($REPO = repository root on the MI355X machine that ran it):", "", "    " + command, ""]
    if note:
        lines += [note, ""]
    lines += ["`%s` (durations in ns):" % os.path.basename(stats_csv), "",
              "| Kernel | Calls | Average ns | Min ns | Max ns | % of GPU time |",
              "|---|---|---|---|---|---|"]
    for name, calls, avg, mn, mx, pct in trace_table(stats_csv):
        lines.append("| `%s` | %d | %.0f | %.0f | %.0f | %.2f |" % (name, calls, avg or 0, mn or 0,
                                                                    mx or 0, pct or 0))
    return "\n".join(lines) + "\n"


# ---------------------------------------------------------------------------
# Counter passes
# ---------------------------------------------------------------------------

def dispatches(counter_csv: str):
    """Dispatch id -> {"kernel", "grid", "duration_ns", "counters": {name: value}}."""
    out = {}
    for r in read_csv(counter_csv):
        did = _col(r, "Dispatch_Id", "DISPATCH_ID", "Correlation_Id")
        d = out.get(did)
        if d is None:
            start = _num(_col(r, "Start_Timestamp", "BEGIN_NS"))
            end = _num(_col(r, "End_Timestamp", "END_NS"))
            grid = _col(r, "Grid_Size", "GRID_SIZE")
            if grid is None:
                grid = "x".join(str(_col(r, "Grid_Size_%s" % a, default="1")) for a in "XYZ")
            d = {"kernel": _col(r, "Kernel_Name", "KERNEL_NAME"), "grid": str(grid),
                 "duration_ns": (end - start) if (start is not None and end is not None) else None,
                 "counters": defaultdict(float)}
            out[did] = d
        name = _col(r, "Counter_Name", "COUNTER_NAME")
        val = _num(_col(r, "Counter_Value", "COUNTER_VALUE"))
        if name is not None and val is not None:
            d["counters"][name] += val
    return out


def library_kernels(disp):
    """Kernel name -> list of dispatches, for the library's kernels only."""
    by = defaultdict(list)
    for d in disp.values():
        if d["kernel"] and LIB_PREFIX in d["kernel"]:
            by[d["kernel"]].append(d)
    return by


def copy_scale(write_disp, fetch_disp, copy_bytes: int):
    """(fetch scale, write scale, copies used): known-size device copies of the output.

    The copies whose WRITE_SIZE is within 2 % of copy_bytes fix the write scale;
    the copies with the same grid in the FETCH_SIZE pass fix the fetch scale (medians,
    so that an upload of the same size from host memory cannot skew them)."""
    kib = copy_bytes / 1024.0
    w_ok = [d for d in write_disp.values() if d["kernel"] and COPY_KERNEL in d["kernel"]
            and abs(d["counters"].get("WRITE_SIZE", 0.0) - kib) <= 0.02 * kib]
    if not w_ok:
        raise ValueError("no %s dispatch of %d bytes in the WRITE_SIZE pass" % (COPY_KERNEL,
                                                                                 copy_bytes))
    grids = {d["grid"] for d in w_ok}
    f_ok = [d for d in fetch_disp.values() if d["kernel"] and COPY_KERNEL in d["kernel"]
            and d["grid"] in grids and d["counters"].get("FETCH_SIZE", 0.0) > 0]
    if not f_ok:
        raise ValueError("no matching %s dispatch in the FETCH_SIZE pass" % COPY_KERNEL)
    wmean = statistics.median(d["counters"]["WRITE_SIZE"] for d in w_ok)
    fmean = statistics.median(d["counters"]["FETCH_SIZE"] for d in f_ok)
    return kib / fmean, kib / wmean, (len(f_ok), len(w_ok), fmean, wmean)


def per_call(passes):
    """Counter -> (per-call value, per-kernel averages): every library kernel's average
    over its dispatches, summed over the kernels (each runs once per call)."""
    merged = {}
    kernels = {}
    durations = {}
    for disp in passes:
        for name, ds in library_kernels(disp).items():
            kernels.setdefault(name, {})
            durations.setdefault(name, {})
            dur = [d["duration_ns"] for d in ds if d["duration_ns"] is not None]
            counters = set().union(*[set(d["counters"]) for d in ds])
            for c in counters:
                kernels[name][c] = statistics.fmean(d["counters"].get(c, 0.0) for d in ds)
                kernels[name]["dispatches"] = len(ds)
                if dur:   # duration of the dispatches of the pass that counted c
                    durations[name][c] = statistics.fmean(dur)
    for name, cs in kernels.items():
        for c, v in cs.items():
            if c in ("dispatches", "_durations", "duration_ns"):
                continue
            merged[c] = merged.get(c, 0.0) + v
        if durations[name]:
            cs["duration_ns"] = statistics.fmean(durations[name].values())
            cs["_durations"] = durations[name]
    return merged, kernels


def counters_markdown(workload: str, op: str, flops: int, algo_bytes: int, copy_bytes: int,
                      pass_csvs, commands, resources=None, note: str = "") -> str:
    """The counter summary of one workload (see the module docstring)."""
    passes = [dispatches(p) for p in pass_csvs]
    merged, kernels = per_call(passes)
    fetch_pass = next((d for d in passes if any("FETCH_SIZE" in x["counters"] for x in d.values())),
                      None)
    write_pass = next((d for d in passes if any("WRITE_SIZE" in x["counters"] for x in d.values())),
                      None)
    lines = ["# Counters: workload `%s`" % workload, "",
             "Each counter set ran in its own pass ($REPO = repository root on the MI355X machine that ran them):", ""]
    lines += ["    " + c for c in commands]
    lines += [""]
    if note:
        lines += [note, ""]
    lines += ["Per-dispatch averages of each library kernel:", "",
              "| Kernel | Dispatches | Counter | Value |", "|---|---|---|---|"]
    for name, cs in kernels.items():
        for c in sorted(k for k in cs if k not in ("dispatches", "_durations")):
            lines.append("| `%s` | %d | %s | %.6g |" % (name, cs["dispatches"], c, cs[c]))
    lines.append("")
    hbm = None
    if fetch_pass is not None and write_pass is not None:
        fs, ws, (nf, nw, fmean, wmean) = copy_scale(write_pass, fetch_pass, copy_bytes)
        lines.append("Calibration: the plain device copy `%s` of the output (a known %d KiB) reads "
                     "FETCH_SIZE %.0f KiB (%d dispatches) and WRITE_SIZE %.0f KiB (%d), so fetch "
                     "counts are scaled by %.4f and write counts by %.4f."
                     % (COPY_KERNEL, copy_bytes // 1024, fmean, nf, wmean, nw, fs, ws))
        fetch_b = merged.get("FETCH_SIZE", 0.0) * 1024 * fs
        write_b = merged.get("WRITE_SIZE", 0.0) * 1024 * ws
        hbm = fetch_b + write_b
        lines.append("")
        lines.append("HBM bytes per call: read %.4g + written %.4g = %.4g bytes against %d "
                     "algorithmic (%.2fx)." % (fetch_b, write_b, hbm, algo_bytes, hbm / algo_bytes))
    lines.append("")
    mops = sum(merged.get(c, 0.0) for c in ("SQ_INSTS_VALU_MFMA_MOPS_F32",
                                            "SQ_INSTS_VALU_MFMA_MOPS_F16",
                                            "SQ_INSTS_VALU_MFMA_MOPS_BF16"))
    if mops:
        lines.append("MFMA work counted by the hardware: MOPS x 512 = %.6g FLOP per call; "
                     "2 M N K = %d, ratio useful / executed = %.4f."
                     % (mops * 512, flops, flops / (mops * 512)))
    for name, cs in kernels.items():
        dur = cs.get("_durations", {}).get("GRBM_GUI_ACTIVE")
        if "GRBM_GUI_ACTIVE" in cs and dur and dur < MIN_CLOCK_NS:
            lines.append("Effective clock of `%s`: not derived (a %.1f us dispatch; "
                         "GRBM_GUI_ACTIVE also counts its launch and drain)." % (name, dur / 1e3))
        elif "GRBM_GUI_ACTIVE" in cs and dur:
            lines.append("Effective clock of `%s`: GRBM_GUI_ACTIVE / %d XCDs / dispatch duration "
                         "= %.3f GHz (under the counter pass; the published peaks assume 2.4 GHz)."
                         % (name, XCDS, cs["GRBM_GUI_ACTIVE"] / XCDS / dur))
        if "SQ_LDS_BANK_CONFLICT" in cs and cs.get("SQ_LDS_IDX_ACTIVE"):
            lines.append("LDS bank conflicts of `%s`: %.4g of %.4g active LDS cycles (%.2f %%)."
                         % (name, cs["SQ_LDS_BANK_CONFLICT"], cs["SQ_LDS_IDX_ACTIVE"],
                            100.0 * cs["SQ_LDS_BANK_CONFLICT"] / cs["SQ_LDS_IDX_ACTIVE"]))
    if resources:
        lines += ["", "Kernel resources (compiler remarks, -Rpass-analysis=kernel-resource-usage):",
                  "", "| Kernel | VGPR | AGPR | SGPR | scratch B/lane | LDS B | waves/SIMD |",
                  "|---|---|---|---|---|---|---|"]
        for name in kernels:
            r = match_resources(name, resources)
            if r is not None:
                lines.append("| `%s` | %s | %s | %s | %s | %s | %s |"
                             % (name, r.get("vgprs"), r.get("agprs"), r.get("sgprs"),
                                r.get("scratch"), r.get("lds"), r.get("occupancy")))
    # Call-level figures (duration-weighted over the call's kernels): the effective
    # clock where the dispatches are long enough, and MfmaUtil.
    clk_cycles = clk_ns = util_ns = util_sum = 0.0
    for cs in kernels.values():
        durs = cs.get("_durations", {})
        d = durs.get("GRBM_GUI_ACTIVE")
        if "GRBM_GUI_ACTIVE" in cs and d and d >= MIN_CLOCK_NS:
            clk_cycles += cs["GRBM_GUI_ACTIVE"] / XCDS
            clk_ns += d
        d = durs.get("MfmaUtil")
        if "MfmaUtil" in cs and d:
            util_sum += cs["MfmaUtil"] * d
            util_ns += d
    lines += ["", "kernel_source_sha256: %s" % source_digest(op)]
    if hbm is not None:
        lines.append("hbm_bytes_per_launch: %.0f" % hbm)
    if clk_ns > 0:
        lines.append("effective_clock_ghz: %.3f" % (clk_cycles / clk_ns))
    if util_ns > 0:
        lines.append("mfma_util_pct: %.2f" % (util_sum / util_ns))
    return "\n".join(lines) + "\n"


def tile_order_markdown(cases, commands, note: str = "") -> str:
    """A/B of tile orders: per case (workload, label, FETCH csv, WRITE csv, kernel-stats
    csv), the HBM bytes per call (copy-calibrated as in counters_markdown) and the
    library kernels' summed average duration per call."""
    from . import cost, inputs
    lines = ["# Tile order A/B: HBM traffic and kernel time per call", "",
             "Commands ($REPO = repository root on the MI355X machine that ran them; W = workload, G,R = rows per "
             "group and XCD renumbering, as passed to bench.py --swizzle):", ""]
    lines += ["    " + c for c in commands]
    lines += [""]
    if note:
        lines += [note, ""]
    lines += ["| Workload | group rows | XCD renumbering | HBM bytes per call | vs algorithmic | "
              "kernel time per call (us) |", "|---|---|---|---|---|---|"]
    for workload, label, fetch_csv, write_csv, stats_csv in cases:
        w = inputs.WORKLOADS[workload]
        half = w.op != "sgemm"
        algo = (cost.hgemm_bias_act_bytes(w.M, w.N, w.K) if half
                else cost.sgemm_bytes(w.M, w.N, w.K, w.beta))
        f, wr = dispatches(fetch_csv), dispatches(write_csv)
        fs, ws, _ = copy_scale(wr, f, w.M * w.N * (2 if half else 4))
        merged, _ = per_call([f, wr])
        hbm = (merged.get("FETCH_SIZE", 0.0) * fs + merged.get("WRITE_SIZE", 0.0) * ws) * 1024
        us = sum(r[2] for r in trace_table(stats_csv) if LIB_PREFIX in (r[0] or "")) / 1e3
        g, r = label.split(",")
        lines.append("| `%s` | %s | %s | %.4g | %.2fx | %.1f |"
                     % (workload, g if g != "0" else "launch's own", "on" if r == "1" else "off",
                        hbm, hbm / algo, us))
    return "\n".join(lines) + "\n"


def _norm(name: str) -> str:
    return re.sub(r"\s+", "", name)


def match_resources(kernel: str, resources):
    """The compiler record of a kernel named as rocprofv3 prints it (demangled)."""
    k = _norm(kernel)
    for r in resources:
        if _norm(r["demangled"]) == k:
            return r
    return None


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--workload", required=True)
    t.add_argument("--stats", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--note", default="")
    t.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--workload", required=True)
    c.add_argument("--pass", dest="passes", action="append", required=True)
    c.add_argument("--command", dest="commands", action="append", required=True)
    c.add_argument("--resources", action="store_true",
                   help="compile the HIP sources for the compiler's register remarks")
    c.add_argument("--remarks", action="append", default=[],
                   help="a file holding those remarks (instead of compiling)")
    c.add_argument("--note", default="")
    c.add_argument("--out", required=True)
    o = sub.add_parser("tile-order")
    o.add_argument("--case", dest="cases", action="append", required=True,
                   metavar="WORKLOAD:G,R:FETCH_CSV:WRITE_CSV:STATS_CSV")
    o.add_argument("--command", dest="commands", action="append", required=True)
    o.add_argument("--note", default="")
    o.add_argument("--out", required=True)
    return ap.parse_args(argv)


def _self_command(argv) -> str:
    import shlex
    return "python -m linear_algebra_sgemm_amd.profile_summary " + " ".join(
        shlex.quote(a) for a in argv)


def main(argv=None):
    argv = sys.argv[1:] if argv is None else argv
    args = parse_args(argv)
    if args.what == "trace":
        text = trace_markdown(args.workload, args.stats, args.command, args.note)
    elif args.what == "tile-order":
        text = tile_order_markdown([tuple(c.split(":")) for c in args.cases], args.commands,
                                   args.note)
    else:
        sys.path.insert(0, ROOT)
        from . import cost, inputs
        w = inputs.WORKLOADS[args.workload]
        half = w.op != "sgemm"
        algo = (cost.hgemm_bias_act_bytes(w.M, w.N, w.K) if half
                else cost.sgemm_bytes(w.M, w.N, w.K, w.beta))
        copy_bytes = w.M * w.N * (2 if half else 4)
        res = None
        if args.remarks:
            from . import resource_usage
            res = []
            for path in args.remarks:
                with open(path) as f:
                    res += resource_usage.parse(f.read())
        elif args.resources:
            from . import resource_usage
            res = [r for _, r in resource_usage.all_kernels()]
        text = counters_markdown(args.workload, w.op, cost.gemm_flops(w.M, w.N, w.K), algo,
                                 copy_bytes, args.passes, args.commands, res, args.note)
    text += "\nSummary written from the rocprofv3 CSV files by (repository root):\n\n    %s\n" % (
        _self_command(argv))
    with open(args.out, "w") as f:
        f.write(text)
    print(text)


if __name__ == "__main__":
    main()
