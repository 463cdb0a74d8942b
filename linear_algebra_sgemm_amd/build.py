"""Build the HIP library libgemm.so in-tree with hipcc for gfx950.

    python -m linear_algebra_sgemm_amd.build

Every kernel source is compiled for gfx950 only.  Packed FP32 instructions are
disabled for all device code (-Xclang -target-feature -Xclang -packed-fp32-ops).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libgemm.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = ["gemm_capi.cpp", "gemm_config.cpp", "sgemm_kernels.hip", "hgemm_kernels.hip",
           "pack_kernels.hip"]
ARCH = "gfx950"

DEVICE_FLAGS = [
    "--offload-arch=%s" % ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library needs ROCm's hipcc")
    return path


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source to an object (in parallel) and link libgemm.so; return its path."""
    cc = hipcc()
    tmpdir = tempfile.mkdtemp(prefix="lasg_build_")
    try:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmpdir, src + ".o")
            objs.append(obj)
            lang = ["-x", "hip"] if src.endswith(".cpp") else []
            cmd = [cc] + DEVICE_FLAGS + ["-I", INCLUDE, "-I", CSRC] + lang + [
                "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
            if len(procs) >= jobs:
                _drain(procs[:1])
                procs = procs[1:]
        _drain(procs)
        tmp_lib = LIB_PATH + ".tmp%d" % os.getpid()
        link = [cc, "--offload-arch=%s" % ARCH, "-shared", "-fPIC", "-o", tmp_lib] + objs
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
        os.replace(tmp_lib, LIB_PATH)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB_PATH


def _drain(procs):
    for src, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            sys.stderr.write(out)
            raise RuntimeError("hipcc failed on %s" % src)
        # hipcc's host pass does not know the device-only feature flag; drop that note.
        lines = [l for l in out.splitlines() if "is not a recognized feature for this target" not in l]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
