"""Work and traffic accounting for one GEMM call (host-side arithmetic only).

* FLOPs: every output element is a K-term dot product, one multiply and one add
  per term, so a call performs 2*M*N*K floating-point operations
  ("SGEMM优化，从naive到warptiling", section 问题与估算; lecture 24, section 1.1).
  Epilogue work (alpha/beta scaling, bias, activation) is not counted, as on
  both pages.
* Algorithmic bytes: each operand crosses HBM exactly once: A and B are read,
  C is written, and C is also read when beta != 0.  With beta != 0 this is the
  "4 x 4096^2 x 4 B ~ 268 MB" figure of the SGEMM page; with C counted once it
  is lecture 24's "4 (MK + KN + MN) ~ 201.3 MB".  The half-precision product
  reads fp16 A and B plus an fp32 bias vector and writes fp16 C.
* Peaks are MI355X's published dense figures (256 CUs at 2.4 GHz): FP32 matrix
  157.3 TFLOP/s, FP16/BF16 dense matrix 2516.6 TFLOP/s, HBM3E 8 TB/s.
"""
from __future__ import annotations

PEAK_TFLOPS = {"f32": 157.3, "f16": 2516.6, "bf16": 2516.6}
PEAK_HBM_GBS = 8000.0
CU_COUNT = 256
CLOCK_GHZ = 2.4


def gemm_flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def sgemm_bytes(M: int, N: int, K: int, beta: float) -> int:
    c_passes = 2 if beta != 0 else 1
    return 4 * (M * K + K * N + c_passes * M * N)


def hgemm_bias_act_bytes(M: int, N: int, K: int, has_bias: bool = True) -> int:
    return 2 * (M * K + K * N) + (4 * N if has_bias else 0) + 2 * M * N


def arithmetic_intensity(flops: float, nbytes: float) -> float:
    return flops / nbytes


def tile_intensity(bm: int, bn: int) -> float:
    """FLOP per byte of fp32 operand traffic for one BM x BN output tile: per k step it
    loads BM + BN floats (4 bytes each) and does 2*BM*BN FLOP, so BM*BN / (2 (BM + BN))
    (lecture 24, block-tiling and register-tiling sections; the same ratio holds for
    a per-thread TM x TN register tile)."""
    return bm * bn / (2.0 * (bm + bn))


def tflops(flops: float, seconds: float) -> float:
    return flops / seconds / 1e12


def machine_balance(dtype: str) -> float:
    """FLOP per HBM byte at which MI355X turns compute-bound for this dtype."""
    return PEAK_TFLOPS[dtype] * 1e12 / (PEAK_HBM_GBS * 1e9)
