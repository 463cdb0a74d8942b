"""Register, LDS and scratch use of every kernel instance, from the compiler.

    python -m linear_algebra_sgemm_amd.resource_usage [--spills-only]

Each HIP source of the library is compiled for gfx950 with the library's own
flags plus ``-Rpass-analysis=kernel-resource-usage``; the compiler then reports,
per kernel instance, its SGPR, VGPR and AGPR counts, scratch bytes per lane,
spilled registers, LDS bytes per workgroup and occupancy.  A kernel whose
register arrays do not fit spills them to scratch memory in HBM, the "local
memory" trap of the register-array and register-accounting sections of
"SGEMM优化，从naive到warptiling" (kernels k5 and k10); the host test built on
this module holds every instance to zero scratch.
"""
from __future__ import annotations

import argparse
import os
import re
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

from . import build as _build

# gfx950 register files: 512 VGPRs + AGPRs per lane for one wave per SIMD, 160 KiB
# of LDS per compute unit.
MAX_REGS = 512
MAX_LDS = 160 * 1024

_FIELD = re.compile(r"remark:\s+([A-Za-z][A-Za-z /]*?)(?: \[[^\]]*\])?: (\S+) \[-Rpass-analysis")
_NAME = re.compile(r"remark: Function Name: (\S+) \[-Rpass-analysis")

KEYS = {
    "TotalSGPRs": "sgprs", "VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize": "scratch",
    "Occupancy": "occupancy", "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill",
    "LDS Size": "lds",
}


def parse(text: str):
    """Kernel records (dicts) from the compiler's kernel-resource-usage remarks."""
    out = []
    cur = None
    for line in text.splitlines():
        m = _NAME.search(line)
        if m:
            cur = {"name": m.group(1)}
            out.append(cur)
            continue
        m = _FIELD.search(line)
        if m and cur is not None:
            key = KEYS.get(m.group(1).strip())
            if key is not None:
                v = m.group(2)
                cur[key] = int(v) if v.lstrip("-").isdigit() else v
    for r in out:
        r["demangled"] = demangle(r["name"])
    return out


_demangle_cache: dict = {}


def demangle(name: str) -> str:
    if name in _demangle_cache:
        return _demangle_cache[name]
    tool = shutil.which("c++filt") or shutil.which("llvm-cxxfilt")
    res = name
    if tool:
        try:
            res = subprocess.run([tool, name], capture_output=True, text=True,
                                 timeout=30).stdout.strip() or name
        except (OSError, subprocess.SubprocessError):
            res = name
    _demangle_cache[name] = res
    return res


def hip_sources():
    return [os.path.join(_build.CSRC, s) for s in _build.SOURCES if s.endswith(".hip")]


def compile_remarks(src: str) -> str:
    """Compile one source's device code with the library's flags and return the remarks."""
    cc = _build.hipcc()
    tmp = tempfile.mkdtemp(prefix="lasg_res_")
    try:
        cmd = [cc] + _build.DEVICE_FLAGS + ["-I", _build.INCLUDE, "-I", _build.CSRC,
                                            "--cuda-device-only", "-c", src, "-o",
                                            os.path.join(tmp, "dev.o"),
                                            "-Rpass-analysis=kernel-resource-usage"]
        p = subprocess.run(cmd, capture_output=True, text=True)
        if p.returncode != 0:
            raise RuntimeError("hipcc failed on %s:\n%s" % (src, p.stderr[-4000:]))
        return p.stderr + p.stdout
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def all_remarks(jobs: int = 3):
    """(source path, remark text) of every HIP source, compiled in parallel."""
    srcs = hip_sources()
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        return list(zip(srcs, ex.map(compile_remarks, srcs)))


def all_kernels(jobs: int = 3):
    """(source file name, record) for every kernel instance of every HIP source."""
    out = []
    for src, text in all_remarks(jobs):
        out += [(os.path.basename(src), r) for r in parse(text)]
    return out


def over_budget(r) -> list:
    """Reasons this instance breaks the register / scratch / LDS budget (empty: none)."""
    bad = []
    if r.get("scratch", 0) != 0:
        bad.append("scratch %s bytes/lane" % r.get("scratch"))
    if r.get("vgpr_spill", 0) != 0:
        bad.append("%s VGPRs spilled" % r.get("vgpr_spill"))
    occ = r.get("occupancy", 1)
    occ = occ if isinstance(occ, int) and occ > 0 else 1
    regs = r.get("vgprs", 0) + r.get("agprs", 0)
    if regs > MAX_REGS // occ:
        bad.append("%d registers at %d waves per SIMD" % (regs, occ))
    if r.get("lds", 0) > MAX_LDS:
        bad.append("LDS %s bytes" % r.get("lds"))
    return bad


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--spills-only", action="store_true")
    ap.add_argument("--save", default=None,
                    help="also write the raw remarks of every source to this directory")
    args = ap.parse_args()
    rows = []
    for src, text in all_remarks():
        if args.save:
            os.makedirs(args.save, exist_ok=True)
            with open(os.path.join(args.save, os.path.basename(src) + ".remarks.txt"), "w") as f:
                f.write(text)
        rows += [(os.path.basename(src), r) for r in parse(text)]
    for src, r in rows:
        bad = over_budget(r)
        if args.spills_only and not bad:
            continue
        print("%-20s VGPR %3s AGPR %3s SGPR %3s scratch %3s spill v%s/s%s LDS %6s occ %s  %s%s"
              % (src, r.get("vgprs"), r.get("agprs"), r.get("sgprs"), r.get("scratch"),
                 r.get("vgpr_spill"), r.get("sgpr_spill"), r.get("lds"), r.get("occupancy"),
                 r["demangled"][:150], ("  <-- " + "; ".join(bad)) if bad else ""))
    sys.exit(1 if any(over_budget(r) for _, r in rows) else 0)


if __name__ == "__main__":
    main()
