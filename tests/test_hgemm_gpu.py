"""FP16-input / FP32-accumulate GEMM with fused bias + GELU(tanh) on the GPU through
the C ABI, against the CPU oracle.

Bar: max |C - ref| / (|alpha| sum_k |a||b| + |bias_j|) <= 1e-2 (C is stored in
fp16; its rounding alone is at most 2^-11 of |C|).  Cases with exactly
representable results (identity and permutation operands, no activation) must
match bit for bit.
"""
import itertools

import pytest
import torch

import linear_algebra_sgemm_amd as lib
from linear_algebra_sgemm_amd import inputs
from tests.gpu_helpers import FP16_TOL, hgemm_error, note, run_hgemm

pytestmark = pytest.mark.gpu

TILES = (0, 1, 2, 3, 4, 5, 6, 7, 8, 9)   # register-staged 256, 128, 64; direct-to-LDS 256x256,
#      128x256, 256x256 5-stage, 256x256 eight waves, eight waves + tail, 128x128; 16x16 K-split


@pytest.fixture(scope="module", autouse=True)
def library():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.gemm_create()
    yield
    lib.gemm_debug_force_tile(1, -1)
    torch.cuda.synchronize()
    lib.gemm_destroy()


@pytest.fixture
def tile_forced():
    yield
    lib.gemm_debug_force_tile(1, -1)


def check_full(M, N, K, alpha, act, seed, with_bias=True, lda=None, ldb=None, ldc=None, label=""):
    A, B, bias = inputs.hgemm_inputs(M, N, K, seed, lda, ldb)
    lda, ldb = A.shape[1], B.shape[1]
    ldc = ldc or max(N, 1)
    C = torch.full((M, ldc), float("nan"), dtype=torch.float16)
    b = bias if with_bias else None
    note("hgemm %s M=%d N=%d K=%d lda=%d ldb=%d ldc=%d alpha=%g act=%d bias=%s seed=%d"
         % (label, M, N, K, lda, ldb, ldc, alpha, act, with_bias, seed))
    got = run_hgemm(M, N, K, alpha, A, lda, B, ldb, b, act, C, ldc)
    err, where = hgemm_error(M, N, K, alpha, A, lda, B, ldb, b, act, got, ldc)
    assert err <= FP16_TOL, "max normalised error %.3g at %s (%s)" % (err, where, label)
    out = got.cpu()
    if ldc > N:
        assert torch.isnan(out[:, N:]).all(), "wrote outside the N columns"
    return out


def test_ffn_shape_tile_rows():
    """A 512-row slice of the inference-FFN workload (N = 14336, K = 4096) in full."""
    w = inputs.WORKLOADS["hgemm_ffn"]
    check_full(512, w.N, w.K, w.alpha, lib.ACT_GELU_TANH, w.seed, label="ffn slice")


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("shape", [(512, 512, 128), (256, 768, 320), (300, 520, 100),
                                   (257, 129, 33), (64, 64, 64)])
def test_every_tile_fast_and_edge(tile, shape, tile_forced):
    lib.gemm_debug_force_tile(1, tile)
    M, N, K = shape
    check_full(M, N, K, 1.0, lib.ACT_GELU_TANH, seed=101 + tile, label="tile %d" % tile)


@pytest.mark.parametrize("act", [lib.ACT_NONE, lib.ACT_GELU_TANH])
@pytest.mark.parametrize("with_bias", [False, True])
def test_bias_and_activation_options(act, with_bias):
    check_full(384, 640, 192, 0.5, act, seed=7, with_bias=with_bias, label="options")


# The size checklist of the DeepGEMM page (section 6.5): every combination of
# m, n, k in {1, 3, 17, 32, 64, 128, 129, 1024}.
EDGE_SIZES = (1, 3, 17, 32, 64, 128, 129, 1024)


@pytest.mark.parametrize("M,N,K", list(itertools.product(EDGE_SIZES, repeat=3)))
def test_edge_grid(M, N, K):
    check_full(M, N, K, 1.5, lib.ACT_GELU_TANH, seed=M * 7919 + N * 31 + K, label="edge grid")


@pytest.mark.parametrize("K", [32, 64, 128, 192, 256, 1024])
@pytest.mark.parametrize("tile", [3, 4, 5, 6, 8])
def test_direct_to_lds_pipeline_depths(K, tile, tile_forced):
    """Whole tiles with K a multiple of 64 take the direct-to-LDS kernels; K from 2 to 32
    tiles of 32 exercises every prologue / drain case of their 4-, 3- and 5-stage pipelines
    (K = 32 is one bounds-checked tail step)."""
    lib.gemm_debug_force_tile(1, tile)
    check_full(512, 256, K, 1.0, lib.ACT_GELU_TANH, seed=K, label="dma%d K=%d" % (tile, K))


@pytest.mark.parametrize("tile", [3, 4, 5, 6, 8])
def test_direct_to_lds_unaligned_ldc(tile, tile_forced):
    lib.gemm_debug_force_tile(1, tile)
    check_full(256, 512, 64, 0.5, lib.ACT_GELU_TANH, seed=77, ldc=515, label="dma ldc=515")
    check_full(256, 512, 64, 0.5, lib.ACT_NONE, seed=78, with_bias=False, lda=72, ldb=520,
               label="dma padded lda/ldb")


def test_padded_leading_dimensions():
    check_full(200, 136, 88, 1.0, lib.ACT_GELU_TANH, seed=12, lda=88 + 8, ldb=136 + 5,
               ldc=136 + 3, label="padded ld")


@pytest.mark.parametrize("tile", TILES)
def test_exact_identity_and_permutation(tile, tile_forced):
    lib.gemm_debug_force_tile(1, tile)
    g = torch.Generator().manual_seed(17)
    M, N = 256, (512 if tile in (3, 4, 5, 6, 8) else 320)
    B = (torch.randn((M, N), generator=g)).half()
    C = torch.zeros((M, N), dtype=torch.float16)
    note("hgemm identity tile=%d" % tile)
    eye = torch.eye(M).half()
    got = run_hgemm(M, N, M, 1.0, eye, M, B, N, None, lib.ACT_NONE, C, N).cpu()
    assert torch.equal(got, B), "I x B must equal B bit for bit"
    p = torch.randperm(M, generator=g)
    P = torch.zeros((M, M))
    P[torch.arange(M), p] = 1.0
    got = run_hgemm(M, N, M, 1.0, P.half(), M, B, N, None, lib.ACT_NONE, C, N).cpu()
    assert torch.equal(got, B[p]), "P x B must permute rows exactly"
    q = torch.randperm(N, generator=g)
    Q = torch.zeros((N, N))
    Q[q, torch.arange(N)] = 1.0
    A = torch.randn((M, N), generator=g).half()
    got = run_hgemm(M, N, N, 1.0, A, N, Q.half(), N, None, lib.ACT_NONE, C, N).cpu()
    assert torch.equal(got, A[:, q]), "A x Q must permute columns exactly"
    # bias only adds per column: I x B + bias with small integers is exact too
    Bi = torch.randint(-50, 50, (M, N), generator=g).half()
    bias = torch.randint(-50, 50, (N,), generator=g).float()
    got = run_hgemm(M, N, M, 1.0, eye, M, Bi, N, bias, lib.ACT_NONE, C, N).cpu()
    assert torch.equal(got, (Bi.float() + bias).half()), "bias must be added per column"


def test_alpha_zero_and_k_zero():
    M, N, K = 70, 90, 40
    A, B, bias = inputs.hgemm_inputs(M, N, K, 23)
    nanA = torch.full_like(A, float("nan"))
    nanB = torch.full_like(B, float("nan"))
    C = torch.zeros((M, N), dtype=torch.float16)
    want = torch.nn.functional.gelu(bias.double(), approximate="tanh")
    note("hgemm alpha=0")
    got = run_hgemm(M, N, K, 0.0, nanA, K, nanB, N, bias, lib.ACT_GELU_TANH, C, N).cpu()
    e = (got.double() - want).abs() / bias.double().abs().clamp_min(1e-30)
    assert torch.isfinite(got).all() and float(e.max()) <= FP16_TOL
    note("hgemm K=0")
    dC = C.cuda()
    lib.hgemm_bias_act(M, N, 0, 1.0, None, 1, None, N, bias.cuda(), lib.ACT_GELU_TANH, dC, N)
    torch.cuda.synchronize()
    got = dC.cpu()
    e = (got.double() - want).abs() / bias.double().abs().clamp_min(1e-30)
    assert float(e.max()) <= FP16_TOL
    note("hgemm K=0 no bias")
    lib.hgemm_bias_act(M, N, 0, 1.0, None, 1, None, N, None, lib.ACT_NONE, dC, N)
    torch.cuda.synchronize()
    assert torch.equal(dC.cpu(), torch.zeros((M, N), dtype=torch.float16))


def test_workload_ffn_every_element():
    """The FFN workload exactly as the benchmark launches it, every output element
    against the oracle."""
    w = inputs.WORKLOADS["hgemm_ffn"]
    A, B, bias = inputs.hgemm_inputs(w.M, w.N, w.K, w.seed)
    C = torch.empty((w.M, w.N), dtype=torch.float16)
    note("hgemm full-size ffn 4096x14336x4096, every element")
    got = run_hgemm(w.M, w.N, w.K, w.alpha, A, w.K, B, w.N, bias, lib.ACT_GELU_TANH, C, w.N).cpu()
    assert torch.isfinite(got).all()
    err, where = hgemm_error(w.M, w.N, w.K, w.alpha, A, w.K, B, w.N, bias, lib.ACT_GELU_TANH,
                             got, w.N)
    assert err <= FP16_TOL, "max normalised error %.3g at %s" % (err, where)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", [(4096, 5120, 128), (2048, 10240, 192)])
def test_head_and_tail_split(fmt, M, N, K, tile_forced):
    """Tile 7: eight-wave 256x256 tiles on the columns that fill whole rounds of
    workgroups, 128x256 tiles on the rest; every entry checked."""
    lib.gemm_debug_force_tile(1, 7)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert lib.gemm_debug_pick_config(1, M, N, K, cus)[0] == 7, "no split for this shape"
    A, B, bias = inputs.hgemm_inputs(M, N, K, 41 + K, fmt=fmt)
    dt = torch.bfloat16 if fmt == "bf16" else torch.float16
    C = torch.full((M, N), float("nan"), dtype=dt)
    note("hgemm head+tail split %s %dx%dx%d" % (fmt, M, N, K))
    got = run_hgemm(M, N, K, 1.25, A, K, B, N, bias, lib.ACT_GELU_TANH, C, N).cpu().float()
    assert torch.isfinite(got).all(), "every output written"
    err, where = hgemm_error(M, N, K, 1.25, A, K, B, N, bias, lib.ACT_GELU_TANH, got, N)
    assert err <= FP16_TOL, "max normalised error %.3g at %s" % (err, where)


def test_deterministic():
    M, N, K = 512, 1024, 512
    A, B, bias = inputs.hgemm_inputs(M, N, K, 33)
    C = torch.empty((M, N), dtype=torch.float16)
    note("hgemm determinism")
    g1 = run_hgemm(M, N, K, 1.0, A, K, B, N, bias, lib.ACT_GELU_TANH, C, N).cpu()
    g2 = run_hgemm(M, N, K, 1.0, A, K, B, N, bias, lib.ACT_GELU_TANH, C, N).cpu()
    assert torch.equal(g1, g2)


WAVE_SPLIT_CASES = [(256, 256, 256, None, None, None),
                    (100, 70, 1001, 1003, 73, 75),
                    (17, 129, 2500, 2504, None, 130),
                    (16, 16, 8, None, None, None),
                    (48, 80, 1152, None, None, None),
                    (33, 40, 129, 136, 48, 41)]


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc", WAVE_SPLIT_CASES)
def test_wave_split_tile_padded_and_odd(M, N, K, lda, ldb, ldc, tile_forced):
    """Tile 9 (16 x 16 tiles, K split over eight waves, operands loaded straight into
    registers): ragged sizes; rows of A off 16-byte boundaries (lda 1003: the 2-byte
    loads run); K = 1152 and 2500 give the waves one to three chunks and a tail; NaN
    padding that must never be read; with and without bias and GELU."""
    lib.gemm_debug_force_tile(1, 9)
    check_full(M, N, K, 1.25, lib.ACT_GELU_TANH, seed=M + N + K, lda=lda, ldb=ldb, ldc=ldc,
               label="tile 9")
    check_full(M, N, K, -0.5, lib.ACT_NONE, seed=M + N + K + 1, with_bias=False, lda=lda,
               ldb=ldb, ldc=ldc, label="tile 9, no bias")
