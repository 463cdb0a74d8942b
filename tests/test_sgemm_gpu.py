"""FP32 GEMM on the GPU through the C ABI, element by element against the CPU oracle.

Bar: max |C - ref| / (|alpha| sum_k |a||b| + |beta||c|) <= 1e-5, and bit-exact
results where every partial sum is exactly representable (identity,
permutation, all-ones and small-integer operands).
"""
import itertools

import pytest
import torch

import linear_algebra_sgemm_amd as lib
from linear_algebra_sgemm_amd import inputs
from tests.gpu_helpers import FP32_TOL, note, run_sgemm, sgemm_error

pytestmark = pytest.mark.gpu

# 256x256, 128x128, 64x64, 256x256 (K step 32), 128x256; 5, 6: 256x256 and 128x256 with
# 16x16x4 MFMA blocks; 7, 8: 256x256 and 128x256 with direct-to-LDS copies
TILES = (0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13)   # 9: tile 7 with eight waves; 10, 11: 128x128, 64x64 direct; 12: 32x32; 13: 16x16, K over 8 waves


@pytest.fixture(scope="module", autouse=True)
def library():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.gemm_create()
    yield
    lib.gemm_debug_force_tile(0, -1)
    torch.cuda.synchronize()
    lib.gemm_destroy()


@pytest.fixture
def tile_forced():
    yield
    lib.gemm_debug_force_tile(0, -1)


def check_full(M, N, K, alpha, beta, seed, lda=None, ldb=None, ldc=None, dist_ab="uniform",
               dist_c="uniform", label=""):
    A, B, C = inputs.sgemm_inputs(M, N, K, seed, dist_ab, dist_c, lda, ldb, ldc)
    lda, ldb, ldc = A.shape[1], B.shape[1], C.shape[1]
    note("sgemm %s M=%d N=%d K=%d lda=%d ldb=%d ldc=%d alpha=%g beta=%g seed=%d"
         % (label, M, N, K, lda, ldb, ldc, alpha, beta, seed))
    got = run_sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)
    err, where = sgemm_error(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, got)
    assert err <= FP32_TOL, "max normalised error %.3g at %s (%s)" % (err, where, label)
    out = got.cpu()
    if ldc > N:   # padding columns untouched (they hold NaN from the generator)
        assert torch.isnan(out[:, N:]).all(), "sgemm wrote outside the N columns"
    return out


def test_workload_256():
    w = inputs.WORKLOADS["sgemm_256"]
    check_full(w.M, w.N, w.K, w.alpha, w.beta, w.seed, label="256^3")


def test_workload_ragged():
    w = inputs.WORKLOADS["sgemm_ragged"]
    check_full(w.M, w.N, w.K, w.alpha, w.beta, w.seed, label="ragged 1000x3000x777")


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("shape", [(512, 512, 64), (768, 256, 160), (300, 520, 100),
                                   (257, 129, 33), (64, 64, 16)])
def test_every_tile_fast_and_edge(tile, shape, tile_forced):
    lib.gemm_debug_force_tile(0, tile)
    M, N, K = shape
    check_full(M, N, K, 1.25, -0.5, seed=11 + tile, label="tile %d" % tile)


# The size checklist of the DeepGEMM page (section 6.5): every combination of
# m, n, k in {1, 3, 17, 32, 64, 128, 129, 1024}.
EDGE_SIZES = (1, 3, 17, 32, 64, 128, 129, 1024)


@pytest.mark.parametrize("M,N,K", list(itertools.product(EDGE_SIZES, repeat=3)))
def test_edge_grid(M, N, K):
    check_full(M, N, K, 0.75, 0.25 if (M + N) % 2 else 0.0, seed=M * 10007 + N * 101 + K,
               label="edge grid")


def test_padded_leading_dimensions_and_guard_bands():
    M, N, K = 200, 150, 90
    A, B, C = inputs.sgemm_inputs(M, N, K, 21, lda=K + 5, ldb=N + 3, ldc=N + 7)
    lda, ldb, ldc = A.shape[1], B.shape[1], C.shape[1]
    # C sits inside a larger buffer with guard rows before and after it.
    guard = 3 * ldc
    Cbuf = torch.full((guard + M * ldc + guard,), 12345.0, dtype=torch.float32)
    Cbuf[guard:guard + M * ldc] = C.reshape(-1)
    dA, dB, dC = A.cuda(), B.cuda(), Cbuf.cuda()
    note("sgemm padded ld + guard bands")
    lib.sgemm(M, N, K, 1.0, dA, lda, dB, ldb, 0.5, dC.data_ptr() + guard * 4, ldc)
    torch.cuda.synchronize()
    out = dC.cpu()
    assert torch.all(out[:guard] == 12345.0) and torch.all(out[guard + M * ldc:] == 12345.0)
    body = out[guard:guard + M * ldc].reshape(M, ldc)
    assert torch.isnan(body[:, N:]).all()
    err, where = sgemm_error(M, N, K, 1.0, A, lda, B, ldb, 0.5, C, ldc, body.reshape(-1))
    assert err <= FP32_TOL, (err, where)


@pytest.mark.parametrize("tile", TILES)
def test_unaligned_base_pointers(tile, tile_forced):
    """Operands offset by one float (4-byte, not 16-byte aligned) with aligned shapes."""
    lib.gemm_debug_force_tile(0, tile)
    M = N = 256
    K = 64
    A, B, C = inputs.sgemm_inputs(M, N, K, 31)
    bufA = torch.zeros(M * K + 1)
    bufA[1:] = A.reshape(-1)
    bufB = torch.zeros(K * N + 1)
    bufB[1:] = B.reshape(-1)
    dA, dB, dC = bufA.cuda(), bufB.cuda(), C.cuda()
    note("sgemm unaligned base tile=%d" % tile)
    lib.sgemm(M, N, K, 1.0, dA.data_ptr() + 4, K, dB.data_ptr() + 4, N, -1.0, dC, N)
    torch.cuda.synchronize()
    err, where = sgemm_error(M, N, K, 1.0, A, K, B, N, -1.0, C, N, dC)
    assert err <= FP32_TOL, (err, where)


@pytest.mark.parametrize("tile", TILES)
def test_exact_identity_and_permutation(tile, tile_forced):
    lib.gemm_debug_force_tile(0, tile)
    g = torch.Generator().manual_seed(5)
    M, N = 256, 192
    B = torch.rand((M, N), generator=g) * 2 - 1
    C = torch.rand((M, N), generator=g) * 2 - 1
    eye = torch.eye(M)
    note("sgemm identity tile=%d" % tile)
    got = run_sgemm(M, N, M, 1.0, eye, M, B, N, 0.0, C, N).cpu()
    assert torch.equal(got, B), "I x B must equal B bit for bit"
    p = torch.randperm(M, generator=g)
    P = torch.zeros((M, M))
    P[torch.arange(M), p] = 1.0
    got = run_sgemm(M, N, M, 1.0, P, M, B, N, 0.0, C, N).cpu()
    assert torch.equal(got, B[p]), "P x B must permute rows exactly"
    q = torch.randperm(N, generator=g)
    Q = torch.zeros((N, N))
    Q[q, torch.arange(N)] = 1.0
    A = torch.rand((M, N), generator=g) * 2 - 1
    got = run_sgemm(M, N, N, 1.0, A, N, Q, N, 0.0, C, N).cpu()
    assert torch.equal(got, A[:, q]), "A x Q must permute columns exactly"


@pytest.mark.parametrize("tile", TILES)
def test_exact_ones_and_small_integers(tile, tile_forced):
    lib.gemm_debug_force_tile(0, tile)
    M, N, K = 200, 300, 1000
    ones_a, ones_b = torch.ones((M, K)), torch.ones((K, N))
    C = torch.randint(-8, 8, (M, N)).float()
    note("sgemm all-ones tile=%d" % tile)
    got = run_sgemm(M, N, K, 1.0, ones_a, K, ones_b, N, 2.0, C, N).cpu()
    assert torch.equal(got, K + 2.0 * C), "all-ones must give K + beta*C exactly"
    g = torch.Generator().manual_seed(9)
    Ai = torch.randint(-9, 10, (M, 96), generator=g)
    Bi = torch.randint(-9, 10, (96, N), generator=g)
    Ci = torch.randint(-9, 10, (M, N), generator=g)
    want = (2 * (Ai.long() @ Bi.long()) - 3 * Ci.long()).float()
    got = run_sgemm(M, N, 96, 2.0, Ai.float(), 96, Bi.float(), N, -3.0, Ci.float(), N).cpu()
    assert torch.equal(got, want), "small-integer products must be exact"


def test_alpha_zero_k_zero_and_beta_zero_nan():
    M, N, K = 130, 70, 50
    A, B, C = inputs.sgemm_inputs(M, N, K, 41)
    nanA = torch.full_like(A, float("nan"))
    nanB = torch.full_like(B, float("nan"))
    note("sgemm alpha=0")
    got = run_sgemm(M, N, K, 0.0, nanA, K, nanB, N, -0.5, C, N).cpu()
    assert torch.equal(got, -0.5 * C), "alpha = 0 must give beta*C without reading A, B"
    note("sgemm alpha=0 beta=0")
    got = run_sgemm(M, N, K, 0.0, A, K, B, N, 0.0, torch.full_like(C, float("nan")), N).cpu()
    assert torch.equal(got, torch.zeros_like(C)), "alpha = beta = 0 must zero C"
    note("sgemm K=0")
    dC = C.cuda()
    lib.sgemm(M, N, 0, 1.0, None, 1, None, N, 3.0, dC, N)
    torch.cuda.synchronize()
    assert torch.equal(dC.cpu(), 3.0 * C)
    note("sgemm beta=0 with NaN C")
    Cn = torch.full_like(C, float("nan"))
    got = run_sgemm(M, N, K, 1.0, A, K, B, N, 0.0, Cn, N)
    assert torch.isfinite(got).all(), "beta = 0 must not read C"
    err, _ = sgemm_error(M, N, K, 1.0, A, K, B, N, 0.0, Cn, N, got)
    assert err <= FP32_TOL
    note("sgemm M=0 / N=0")
    lib.sgemm(0, N, K, 1.0, None, K, None, N, 0.0, None, N)
    lib.sgemm(M, 0, K, 1.0, None, K, None, 1, 0.0, None, 1)
    torch.cuda.synchronize()


def test_invalid_arguments_enqueue_nothing():
    C = torch.ones((4, 4), device="cuda")
    st = lib.sgemm(4, 4, 4, 1.0, C, 3, C, 4, 0.0, C, 4, raise_on_error=False)
    assert st == lib.STATUS_INVALID_VALUE
    torch.cuda.synchronize()
    assert torch.equal(C.cpu(), torch.ones((4, 4)))


def _full_size_check(w):
    """The workload exactly as the benchmark launches it (packed operands, the
    configuration the library picks), every output element against the oracle."""
    A, B, C = inputs.workload_inputs(w)
    M, N, K = w.M, w.N, w.K
    note("sgemm full-size %s, every element" % w.name)
    got = run_sgemm(M, N, K, w.alpha, A, K, B, N, w.beta, C, N).cpu()
    assert torch.isfinite(got).all()
    err, where = sgemm_error(M, N, K, w.alpha, A, K, B, N, w.beta, C, N, got)
    assert err <= FP32_TOL, "max normalised error %.3g at %s" % (err, where)
    return got


def test_workload_4096_every_element():
    _full_size_check(inputs.WORKLOADS["sgemm_4096"])


def test_workload_8192_every_element():
    _full_size_check(inputs.WORKLOADS["sgemm_8192"])


def test_deterministic():
    M, N, K = 1024, 1024, 512
    A, B, C = inputs.sgemm_inputs(M, N, K, 51)
    note("sgemm determinism")
    g1 = run_sgemm(M, N, K, 1.0, A, K, B, N, 0.5, C, N).cpu()
    g2 = run_sgemm(M, N, K, 1.0, A, K, B, N, 0.5, C, N).cpu()
    assert torch.equal(g1, g2)


def test_two_streams_concurrently():
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    p1 = (512, 768, 256, 61)
    p2 = (300, 200, 700, 62)
    note("sgemm two streams")
    dev = []
    for (M, N, K, seed) in (p1, p2):
        A, B, C = inputs.sgemm_inputs(M, N, K, seed)
        dev.append((M, N, K, A, B, C, A.cuda(), B.cuda(), C.cuda()))
    torch.cuda.synchronize()
    for (M, N, K, A, B, C, dA, dB, dC), s in zip(dev, (s1, s2)):
        lib.sgemm(M, N, K, 1.0, dA, K, dB, N, 1.0, dC, N, stream=s)
    torch.cuda.synchronize()
    for (M, N, K, A, B, C, dA, dB, dC) in dev:
        err, where = sgemm_error(M, N, K, 1.0, A, K, B, N, 1.0, C, N, dC)
        assert err <= FP32_TOL, (M, N, K, err, where)


def test_long_k_repeated():
    M, N, K = 256, 256, 16384
    A, B, C = inputs.sgemm_inputs(M, N, K, 71)
    dA, dB = A.cuda(), B.cuda()
    first = None
    note("sgemm long K x5")
    for _ in range(5):
        dC = C.cuda()
        lib.sgemm(M, N, K, 1.0, dA, K, dB, N, 0.25, dC, N)
        torch.cuda.synchronize()
        out = dC.cpu()
        if first is None:
            first = out
            err, where = sgemm_error(M, N, K, 1.0, A, K, B, N, 0.25, C, N, out)
            assert err <= FP32_TOL, (err, where)
        else:
            assert torch.equal(out, first)


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc", [(256, 256, 256, None, None, None),
                                               (100, 70, 1001, 1003, 73, 75),
                                               (17, 129, 2048, 2049, None, 130),
                                               (16, 16, 4, None, None, None),
                                               (48, 80, 320, None, None, None),
                                               (64, 32, 128, 132, 40, 33),
                                               (32, 16, 1024, 1028, 17, None),
                                               (16, 48, 32, None, None, None)])
def test_wave_split_tile_padded_and_odd(M, N, K, lda, ldb, ldc, tile_forced):
    """Tile 13 (16 x 16 tiles, K split over the eight waves, operands loaded straight
    into registers): ragged sizes, odd leading dimensions (rows of A not 16-byte
    aligned, so the scalar loads run), NaN padding that must never be read; whole
    tiles (M, N multiples of 16, K of 32, rows of A 16-byte aligned) need no
    out-of-range values replaced, with K = 320 giving the waves one or two chunks
    each and K = 32 leaving seven waves without one."""
    lib.gemm_debug_force_tile(0, 13)
    check_full(M, N, K, 1.5, -0.75, seed=M + N + K, lda=lda, ldb=ldb, ldc=ldc, label="tile 13")
