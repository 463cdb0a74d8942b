"""Seeded synthetic inputs for the GEMM workloads.

This module only draws random numbers; it holds none of the product's
arithmetic.  The oracle side (tests, CPU baseline) and the GPU side take the
same host arrays from here, so both see identical bytes.

Recipe (the pages fix no values, only shapes: square FP32 matrices at 4096 in
"SGEMM优化，从naive到warptiling" section 问题与估算, an FP16-in/FP32-accumulate
product with a fused bias + GELU epilogue on the DeepGEMM page):

* one CPU ``torch.Generator`` seeded with the workload's seed;
* draws in the order A, B, C (or A, B, bias for the half-precision product);
* U[-1, 1] is ``rand * 2 - 1`` in float32 (covers [-1, 1));
* N(0, 1) is ``randn`` in float32;
* the 16-bit operands are ``(randn * 0.02)`` rounded to float16 or bfloat16 (round to
  nearest even);
* matrices are packed row-major (leading dimension = column count) unless a
  caller asks for padding, which is filled with NaN so that any read of it
  shows up in the result.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    op: str            # "sgemm", "hgemm_bias_gelu" or "bgemm_bias_gelu"
    M: int
    N: int
    K: int
    seed: int
    alpha: float
    beta: float = 0.0
    dist_ab: str = "uniform"     # "uniform" U[-1,1], "normal" N(0,1), "normal002_f16"/"_bf16"
    dist_c: str = "uniform"      # distribution of C (sgemm) -- bias is always N(0,1)
    note: str = field(default="", compare=False)


# The five workloads: a small square case, the 4096^3 headline case, a ragged
# case whose sizes are not tile multiples (and whose K = lda = 777 leaves A's
# rows only 4-byte aligned), the inference-FFN half-precision case and a large
# square case.
WORKLOADS = {
    "sgemm_256": Workload("sgemm_256", "sgemm", 256, 256, 256, seed=0, alpha=1.0, beta=0.0),
    "sgemm_4096": Workload("sgemm_4096", "sgemm", 4096, 4096, 4096, seed=1, alpha=1.0, beta=0.5,
                           note="C reset before every timed repetition"),
    "sgemm_ragged": Workload("sgemm_ragged", "sgemm", 1000, 3000, 777, seed=2, alpha=1.5,
                             beta=-0.25),
    "hgemm_ffn": Workload("hgemm_ffn", "hgemm_bias_gelu", 4096, 14336, 4096, seed=3, alpha=1.0,
                          dist_ab="normal002_f16"),
    "sgemm_8192": Workload("sgemm_8192", "sgemm", 8192, 8192, 8192, seed=4, alpha=1.0, beta=1.0,
                           dist_ab="normal", dist_c="uniform"),
    # the FFN product again with bfloat16 operands and output
    "bgemm_ffn": Workload("bgemm_ffn", "bgemm_bias_gelu", 4096, 14336, 4096, seed=5, alpha=1.0,
                          dist_ab="normal002_bf16"),
}


def _draw(gen: torch.Generator, rows: int, cols: int, dist: str) -> torch.Tensor:
    if dist == "uniform":
        return torch.rand((rows, cols), generator=gen, dtype=torch.float32) * 2 - 1
    if dist == "normal":
        return torch.randn((rows, cols), generator=gen, dtype=torch.float32)
    if dist == "normal002_f16":
        return (torch.randn((rows, cols), generator=gen, dtype=torch.float32) * 0.02).to(torch.float16)
    if dist == "normal002_bf16":
        return (torch.randn((rows, cols), generator=gen, dtype=torch.float32) * 0.02).to(torch.bfloat16)
    raise ValueError("unknown distribution %r" % dist)


def _pad(x: torch.Tensor, ld: int) -> torch.Tensor:
    """Return a (rows, ld) tensor whose first cols columns are x and the rest NaN."""
    rows, cols = x.shape
    if ld == cols:
        return x.contiguous()
    if ld < cols:
        raise ValueError("leading dimension smaller than the column count")
    out = torch.full((rows, ld), float("nan"), dtype=x.dtype)
    out[:, :cols] = x
    return out


def sgemm_inputs(M: int, N: int, K: int, seed: int, dist_ab: str = "uniform",
                 dist_c: str = "uniform", lda: int | None = None, ldb: int | None = None,
                 ldc: int | None = None):
    """Host float32 tensors A (M x lda), B (K x ldb), C (M x ldc), drawn in the order A, B, C."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    A = _draw(gen, M, K, dist_ab)
    B = _draw(gen, K, N, dist_ab)
    C = _draw(gen, M, N, dist_c)
    return _pad(A, lda or max(K, 1)), _pad(B, ldb or max(N, 1)), _pad(C, ldc or max(N, 1))


def hgemm_inputs(M: int, N: int, K: int, seed: int, lda: int | None = None,
                 ldb: int | None = None, fmt: str = "f16"):
    """Host tensors A (M x lda), B (K x ldb) in fp16 (fmt "f16") or bfloat16 ("bf16") and
    bias (N fp32 ~ N(0,1)), drawn in the order A, B, bias."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    dist = {"f16": "normal002_f16", "bf16": "normal002_bf16"}[fmt]
    A = _draw(gen, M, K, dist)
    B = _draw(gen, K, N, dist)
    bias = torch.randn((N,), generator=gen, dtype=torch.float32)
    return _pad(A, lda or max(K, 1)), _pad(B, ldb or max(N, 1)), bias


def workload_inputs(w: Workload):
    if w.op == "sgemm":
        return sgemm_inputs(w.M, w.N, w.K, w.seed, w.dist_ab, w.dist_c)
    return hgemm_inputs(w.M, w.N, w.K, w.seed, fmt="bf16" if w.op == "bgemm_bias_gelu" else "f16")


def sha256(*tensors: torch.Tensor) -> str:
    h = hashlib.sha256()
    for t in tensors:
        h.update(t.contiguous().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()


def sample_indices(M: int, N: int, count: int, seed: int):
    """Deterministic (rows, cols) sample that always includes the four corners and the
    last row / column (where ragged tiles end), then uniform picks."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed + 7919)
    fixed_r = [0, 0, M - 1, M - 1]
    fixed_c = [0, N - 1, 0, N - 1]
    r = torch.randint(0, M, (count,), generator=gen)
    c = torch.randint(0, N, (count,), generator=gen)
    rows = torch.cat([torch.tensor(fixed_r), r, torch.full((count // 8,), M - 1),
                      torch.randint(0, M, (count // 8,), generator=gen)])
    cols = torch.cat([torch.tensor(fixed_c), c, torch.randint(0, N, (count // 8,), generator=gen),
                      torch.full((count // 8,), N - 1)])
    return rows.numpy().astype("int64"), cols.numpy().astype("int64")
