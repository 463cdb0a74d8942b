"""Seeded random problems on the configuration the library picks, on the GPU through
the C ABI, against the CPU oracle.

Each case draws M, N, K (from 1 up to a few hundred, some large enough that copies
to the pack buffer and K splits pay), padded leading dimensions (padding NaN, never
read or written), alpha and beta (zero included), and a base offset of one element
for A, B and C (rows then only 4- or 2-byte aligned), so that the automatic choice
walks through the direct-to-LDS tiles with ragged edges and 4-byte copies of A,
the register-staged tiles with bounds checks or padded copies, packing of B, the
small tiles and split-K.  Bars: the FP32 and half-precision bars of the other
parity tests; nothing outside C's M x N window changes.
"""
import random

import pytest
import torch

import linear_algebra_sgemm_amd as lib
from linear_algebra_sgemm_amd import inputs
from tests.gpu_helpers import FP16_TOL, FP32_TOL, hgemm_error, note, sgemm_error

pytestmark = pytest.mark.gpu

FMTS = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def library():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.gemm_create()
    yield
    torch.cuda.synchronize()
    lib.gemm_destroy()


def draw_shape(rng):
    big = rng.random() < 0.3
    hi = 900 if big else 300
    M, N, K = rng.randint(1, hi), rng.randint(1, hi), rng.randint(1, hi if not big else 1200)
    return M, N, K


def draw_ld(rng, cols):
    return cols + rng.choice([0, 0, 0, 1, 3, 4, 8, 13])


def place(host, offset, dtype):
    """A device buffer holding `host` (flattened) `offset` elements past its start, and
    the address of that element."""
    flat = host.reshape(-1)
    buf = torch.full((flat.numel() + offset + 8,), float("nan"), dtype=dtype)
    buf[offset:offset + flat.numel()] = flat
    dbuf = buf.cuda()
    return dbuf, dbuf.data_ptr() + offset * dbuf.element_size()


@pytest.mark.parametrize("case", range(96))
def test_random_sgemm(case):
    rng = random.Random(20000 + case)
    M, N, K = draw_shape(rng)
    lda, ldb, ldc = draw_ld(rng, K), draw_ld(rng, N), draw_ld(rng, N)
    alpha = rng.choice([1.0, -0.5, 1.75, 0.0])
    beta = rng.choice([0.0, 1.0, -0.25, 0.5])
    offs = [rng.choice([0, 0, 1]) for _ in range(3)]
    A, B, C = inputs.sgemm_inputs(M, N, K, 20000 + case, lda=lda, ldb=ldb, ldc=ldc)
    if beta == 0.0:
        C[:, :N] = float("nan")   # beta = 0: C is not read
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tile, splits = lib.gemm_debug_pick_config(0, M, N, K, cus)
    note("sgemm random case %d: M=%d N=%d K=%d lda=%d ldb=%d ldc=%d alpha=%g beta=%g offsets=%s "
         "(packed-operand choice tile %d x%d)" % (case, M, N, K, lda, ldb, ldc, alpha, beta, offs,
                                                  tile, splits))
    dA, pA = place(A, offs[0], torch.float32)
    dB, pB = place(B, offs[1], torch.float32)
    dC, pC = place(C, offs[2], torch.float32)
    lib.sgemm(M, N, K, alpha, pA, lda, pB, ldb, beta, pC, ldc)
    torch.cuda.synchronize()
    out = dC.cpu()
    body = out[offs[2]:offs[2] + M * ldc].reshape(M, ldc)
    assert torch.isnan(out[:offs[2]]).all() and torch.isnan(out[offs[2] + M * ldc:]).all()
    if ldc > N:
        assert torch.isnan(body[:, N:]).all(), "wrote outside the N columns"
    C0 = torch.zeros_like(C) if beta == 0.0 else C
    err, where = sgemm_error(M, N, K, alpha, A, lda, B, ldb, beta, C0, ldc, body.reshape(-1))
    assert err <= FP32_TOL, (err, where)


@pytest.mark.parametrize("case", range(48))
def test_random_half(case):
    rng = random.Random(30000 + case)
    fmt = rng.choice(list(FMTS))
    M, N, K = draw_shape(rng)
    lda, ldb, ldc = draw_ld(rng, K), draw_ld(rng, N), draw_ld(rng, N)
    alpha = rng.choice([1.0, -0.5, 1.75])
    act = rng.choice([lib.ACT_NONE, lib.ACT_GELU_TANH])
    with_bias = rng.random() < 0.8
    offs = [rng.choice([0, 0, 1]) for _ in range(3)]
    A, B, bias = inputs.hgemm_inputs(M, N, K, 30000 + case, lda=lda, ldb=ldb, fmt=fmt)
    b = bias if with_bias else None
    C = torch.full((M, ldc), float("nan"), dtype=FMTS[fmt])
    note("half random case %d: %s M=%d N=%d K=%d lda=%d ldb=%d ldc=%d alpha=%g act=%d bias=%s "
         "offsets=%s" % (case, fmt, M, N, K, lda, ldb, ldc, alpha, act, with_bias, offs))
    dA, pA = place(A, offs[0], FMTS[fmt])
    dB, pB = place(B, offs[1], FMTS[fmt])
    dC, pC = place(C, offs[2], FMTS[fmt])
    dbias = None if b is None else b.cuda()
    fn = lib.bgemm_bias_act if fmt == "bf16" else lib.hgemm_bias_act
    fn(M, N, K, alpha, pA, lda, pB, ldb, dbias, act, pC, ldc)
    torch.cuda.synchronize()
    out = dC.cpu()
    body = out[offs[2]:offs[2] + M * ldc].reshape(M, ldc)
    assert torch.isnan(out[:offs[2]].float()).all()
    assert torch.isnan(out[offs[2] + M * ldc:].float()).all()
    if ldc > N:
        assert torch.isnan(body[:, N:].float()).all(), "wrote outside the N columns"
    err, where = hgemm_error(M, N, K, alpha, A, lda, B, ldb, b, act, body.reshape(-1), ldc)
    assert err <= FP16_TOL, (err, where)
