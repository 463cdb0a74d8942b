#!/usr/bin/env python3
"""Parity report of the library's configurations against the CPU oracle.

    python tests/parity_report.py [--out FILE]

Runs every workload (the five configurations of the benchmark plus the
bfloat16 twin of the FFN product) once through the C ABI on the configuration
the library picks, compares every output element with the oracle and prints
one markdown table: the number of entries compared, the largest normalised
error |C - ref| / (|alpha| sum_k |a||b| + |beta||c| or
|bias|) with its position, its 50th, 99th and 99.99th percentiles, and the
bar (1e-5 for FP32, 1e-2 for the 16-bit products).  Test infrastructure: it
imports the oracle; the GPU tests assert the same bars.
"""
from __future__ import annotations

import argparse
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--out", default=None, help="also write the table to this file")
    args = ap.parse_args()

    import torch

    import linear_algebra_sgemm_amd as lib
    import oracle
    from linear_algebra_sgemm_amd import inputs

    if not torch.cuda.is_available():
        sys.exit("parity_report.py needs a GPU")
    lib.gemm_create()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    bits = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    rows_out = []
    for name, w in inputs.WORKLOADS.items():
        M, N, K = w.M, w.N, w.K
        op = 0 if w.op == "sgemm" else 1
        tile, splits = lib.gemm_debug_pick_config(op, M, N, K, cus)
        print("[case] %s %dx%dx%d tile %d x%d" % (name, M, N, K, tile, splits), flush=True)
        A, B, C = inputs.workload_inputs(w)
        dA, dB = A.cuda(), B.cuda()
        if w.op == "sgemm":
            dC = C.cuda()
            lib.sgemm(M, N, K, w.alpha, dA, K, dB, N, w.beta, dC, N)
            torch.cuda.synchronize()
            got = dC.cpu().numpy()
            ref, den = oracle.sgemm(M, N, K, w.alpha, A.numpy(), K, B.numpy(), N, w.beta,
                                    C.numpy(), N)
            tol, dtype = 1e-5, "f32"
        else:
            bf16 = w.op == "bgemm_bias_gelu"
            dt = torch.bfloat16 if bf16 else torch.float16
            dC = torch.empty((M, N), dtype=dt, device="cuda")
            fn = lib.bgemm_bias_act if bf16 else lib.hgemm_bias_act
            fn(M, N, K, w.alpha, dA, K, dB, N, C.cuda(), lib.ACT_GELU_TANH, dC, N)
            torch.cuda.synchronize()
            got = dC.cpu().float().numpy()
            fmt = "bf16" if bf16 else "f16"
            ref, den = oracle.hgemm_bias_act(M, N, K, w.alpha, bits(A), K, bits(B), N, C.numpy(),
                                             oracle.ACT_GELU_TANH, fmt=fmt)
            tol, dtype = 1e-2, fmt
        e = oracle.normalized_error(got, ref, den,
                                    oracle.OUTPUT_FLOOR[dtype] if dtype in oracle.OUTPUT_FLOOR
                                    else 0.0).reshape(-1)
        k = int(np.argmax(e))
        ki, kj = divmod(k, N)
        q = np.quantile(e, [0.5, 0.99, 0.9999])
        rows_out.append("| `%s` %d×%d×%d | %s | tile %d ×%d | %s | %.3g at (%d, %d) | %.3g | %.3g "
                        "| %.3g | %g | %s |"
                        % (name, M, N, K, dtype, tile, splits,
                           "all %d" % e.size, e[k], ki, kj,
                           q[0], q[1], q[2], tol, "pass" if e.max() <= tol else "FAIL"))
    lib.gemm_destroy()
    table = ["| Workload | dtype | configuration | entries | max error (where) | p50 | p99 | "
             "p99.99 | bar | |", "|---|---|---|---|---|---|---|---|---|---|"] + rows_out
    text = "\n".join(table)
    print(text, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text + "\n")


if __name__ == "__main__":
    main()
