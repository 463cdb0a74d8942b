"""The FP32 direct-to-LDS kernels on ragged shapes, on the GPU through the C ABI,
against the CPU oracle.

Tiles 7 to 11 copy 16-byte chunks of A and B straight into LDS.  When M or N
is not a multiple of the tile, or K not a multiple of 32, they run a
bounds-checked instantiation: copies of rows past M - 1 (columns past N - 4)
repeat the last row (chunk) inside the matrix, the last K % 32 values of k go
through one zero-filled tail step, and the epilogue stores only rows < M and
columns < N.  It needs rows of A and B on 16-byte boundaries and N a multiple
of 4; other operands resolve to the register-staged tile 4 (tile 2 for the 64x64 tile 11).  Bar: max
|C - ref| / (|alpha| sum|a||b| + |beta||c|) <= 1e-5, bit-exact on small
integers, nothing written outside C's M x N window.
"""
import pytest
import torch

import linear_algebra_sgemm_amd as lib
from linear_algebra_sgemm_amd import inputs
from tests.gpu_helpers import FP32_TOL, note, run_sgemm, sgemm_error

pytestmark = pytest.mark.gpu

DMA_TILES = (7, 8, 9, 10, 11)
# (M, N, K): ragged M and N, K below 32, K % 32 in 1..31, K a multiple of 32 on ragged M / N,
# tiles smaller than one block, several tiles with a ragged last row and column, and K % 32 > 16
# after whole K tiles (a tail of two 16-wide K tiles)
SHAPES = [(300, 520, 100), (257, 260, 33), (64, 64, 16), (1, 4, 1), (129, 132, 31),
          (511, 516, 64), (700, 900, 777), (256, 256, 40), (1000, 1000, 1000),
          (260, 4, 4100), (200, 196, 95), (130, 260, 1009)]


@pytest.fixture(scope="module", autouse=True)
def library():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.gemm_create()
    yield
    lib.gemm_debug_force_tile(0, -1)
    lib.gemm_debug_force_splits(0, -1)
    torch.cuda.synchronize()
    lib.gemm_destroy()


@pytest.fixture
def forced():
    yield
    lib.gemm_debug_force_tile(0, -1)
    lib.gemm_debug_force_splits(0, -1)


def force(tile, splits=1):
    assert lib.gemm_debug_force_tile(0, tile) == lib.STATUS_SUCCESS
    assert lib.gemm_debug_force_splits(0, splits) == lib.STATUS_SUCCESS


def check(M, N, K, alpha, beta, seed, label, lda=None, ldb=None, ldc=None):
    A, B, C = inputs.sgemm_inputs(M, N, K, seed, lda=lda, ldb=ldb, ldc=ldc)
    lda, ldb, ldc = A.shape[1], B.shape[1], C.shape[1]
    note("sgemm direct-to-LDS edge %s M=%d N=%d K=%d lda=%d ldb=%d ldc=%d alpha=%g beta=%g seed=%d"
         % (label, M, N, K, lda, ldb, ldc, alpha, beta, seed))
    got = run_sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)
    err, where = sgemm_error(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, got)
    assert err <= FP32_TOL, "max normalised error %.3g at %s (%s)" % (err, where, label)
    out = got.cpu()
    if ldc > N:
        assert torch.isnan(out.reshape(-1, ldc)[:M, N:]).all(), "wrote outside the N columns"
    return out


def lda_for(K):
    """A's leading dimension: K rounded up to a multiple of 4 (rows on 16-byte boundaries)."""
    return (K + 3) // 4 * 4


@pytest.mark.parametrize("tile", DMA_TILES)
@pytest.mark.parametrize("shape", SHAPES)
def test_ragged_shapes(tile, shape, forced):
    force(tile)
    M, N, K = shape
    # the forced direct-to-LDS tile runs for every shape (rows of A with lda = K
    # not a multiple of 4 are copied 4 bytes at a time); here lda is padded to a
    # multiple of 4, so A is copied in 16-byte chunks
    t, s = lib.gemm_debug_pick_config(0, M, N, K, 256)
    assert (t, s) == (tile, 1)
    check(M, N, K, 1.25, -0.5, seed=900 + tile + M + K, label="tile %d" % tile, lda=lda_for(K))


@pytest.mark.parametrize("tile", DMA_TILES)
def test_beta_zero_and_padded_leading_dimensions(tile, forced):
    force(tile)
    # lda, ldb, ldc padded (multiples of 4 for A and B), C padding must stay NaN
    check(333, 292, 250, 2.0, 0.0, seed=931 + tile, label="beta 0, padded", lda=256, ldb=300,
          ldc=301)
    check(333, 292, 250, -1.0, 1.0, seed=932 + tile, label="beta 1, padded", lda=260, ldb=296,
          ldc=293)


@pytest.mark.parametrize("tile", DMA_TILES)
@pytest.mark.parametrize("splits", [2, 5])
@pytest.mark.parametrize("shape", [(300, 260, 1000), (257, 516, 777), (100, 8, 4111)])
def test_ragged_split(tile, splits, shape, forced):
    force(tile, splits)
    M, N, K = shape
    t, s = lib.gemm_debug_pick_config(0, M, N, K, 256)
    assert t == tile and 1 <= s <= splits
    check(M, N, K, 0.75, 0.25, seed=940 + tile + splits, label="tile %d x%d" % (tile, s),
          lda=lda_for(K))


@pytest.mark.parametrize("tile", DMA_TILES)
def test_exact_small_integers(tile, forced):
    force(tile)
    M, N, K = 300, 260, 77
    g = torch.Generator().manual_seed(951 + tile)
    Ai = torch.randint(-9, 10, (M, K), generator=g)
    Bi = torch.randint(-9, 10, (K, N), generator=g)
    Ci = torch.randint(-9, 10, (M, N), generator=g)
    want = (2 * (Ai.long() @ Bi.long()) - 3 * Ci.long()).float()
    note("sgemm direct-to-LDS edge small integers tile %d" % tile)
    # lda = 80: rows of A on 16-byte boundaries, copied 16 bytes at a time
    Ap = torch.zeros((M, 80))
    Ap[:, :K] = Ai.float()
    got = run_sgemm(M, N, K, 2.0, Ap, 80, Bi.float(), N, -3.0, Ci.float(), N).cpu()
    assert torch.equal(got, want), "small-integer products must be exact on ragged tiles"
    # lda = 77: rows of A only 4-byte aligned, copied 4 bytes at a time into the same layout
    got = run_sgemm(M, N, K, 2.0, Ai.float().contiguous(), K, Bi.float(), N, -3.0, Ci.float(),
                    N).cpu()
    assert torch.equal(got, want), "4-byte copies of A must give the same exact result"


@pytest.mark.parametrize("tile", DMA_TILES)
def test_guard_bands_untouched(tile, forced):
    """C sits inside a larger buffer; nothing before, after or between its rows changes."""
    force(tile)
    M, N, K = 270, 140, 72   # K % 32 = 8: the tail step runs
    A, B, C = inputs.sgemm_inputs(M, N, K, 961 + tile, ldc=N + 6)
    ldc = C.shape[1]
    guard = 2 * ldc
    buf = torch.full((guard + M * ldc + guard,), 4321.0)
    buf[guard:guard + M * ldc] = C.reshape(-1)
    dA, dB, dbuf = A.cuda(), B.cuda(), buf.cuda()
    note("sgemm direct-to-LDS edge guard bands tile %d" % tile)
    lib.sgemm(M, N, K, 1.0, dA, K, dB, N, 0.5, dbuf.data_ptr() + guard * 4, ldc)
    torch.cuda.synchronize()
    out = dbuf.cpu()
    assert torch.all(out[:guard] == 4321.0) and torch.all(out[guard + M * ldc:] == 4321.0)
    body = out[guard:guard + M * ldc].reshape(M, ldc)
    assert torch.isnan(body[:, N:]).all()
    err, where = sgemm_error(M, N, K, 1.0, A, K, B, N, 0.5, C, ldc, body.reshape(-1))
    assert err <= FP32_TOL, (err, where)


@pytest.mark.parametrize("tile", DMA_TILES)
@pytest.mark.parametrize("shape", [(300, 520, 101), (513, 260, 777), (256, 256, 255), (64, 128, 33)])
def test_four_byte_copies_of_a(tile, shape, forced):
    """lda not a multiple of 4 and A's base 4 bytes past a 16-byte boundary: the
    direct-to-LDS tile copies A 4 bytes at a time, with no packing."""
    force(tile)
    M, N, K = shape
    lda = K if K % 4 else K + 1
    A, B, C = inputs.sgemm_inputs(M, N, K, 1010 + tile + M, lda=lda, ldc=N + 2)
    ldc = C.shape[1]
    buf = torch.zeros(M * lda + 1)
    buf[1:] = A.reshape(-1)
    dbuf, dB, dC = buf.cuda(), B.cuda(), C.cuda()
    note("sgemm direct-to-LDS 4-byte A copies tile %d M=%d N=%d K=%d lda=%d" % (tile, M, N, K, lda))
    lib.sgemm(M, N, K, 0.75, dbuf.data_ptr() + 4, lda, dB, N, 0.5, dC, ldc)
    torch.cuda.synchronize()
    err, where = sgemm_error(M, N, K, 0.75, A, lda, B, N, 0.5, C, ldc, dC)
    assert err <= FP32_TOL, (err, where)
    assert torch.isnan(dC.cpu()[:, N:]).all(), "wrote outside the N columns"


def test_unaligned_operands_are_packed(forced):
    """N not a multiple of 4: B is copied into the library's pack buffer with 16-byte
    rows and the direct-to-LDS tile reads the copy; lda not a multiple of 4: A is read
    4 bytes at a time."""
    force(9)
    assert lib.gemm_debug_pick_config(0, 600, 1026, 1000, 256) == (9, 1)
    check(600, 1026, 1000, 1.0, 0.5, seed=971, label="N = 1026")
    check(600, 1024, 1001, 1.0, 0.5, seed=972, label="lda = 1001")
    # too small for the copy to pay: the register-staged tile runs on the operands as given
    assert lib.gemm_debug_pick_config(0, 300, 258, 100, 256) == (4, 1)
    check(300, 258, 100, 1.0, 0.5, seed=973, label="N = 258, not packed")


@pytest.mark.parametrize("shape,want", [((4000, 4000, 4008), (9, 1)), ((6000, 6000, 6000), (8, 1)),
                                        ((2800, 2800, 2800), (10, 1)),
                                        ((4000, 2000, 3000), (10, 1)), ((3000, 3000, 3000), (11, 1))])
def test_auto_choice_large_ragged(shape, want):
    """Full-size ragged products on the configuration the library picks, every output
    element against the oracle."""
    M, N, K = shape
    assert lib.gemm_debug_pick_config(
        0, M, N, K, torch.cuda.get_device_properties(0).multi_processor_count) == want
    A, B, C = inputs.sgemm_inputs(M, N, K, 981 + M)
    note("sgemm direct-to-LDS edge auto %dx%dx%d (expect tile %d x%d)" % (M, N, K, *want))
    got = run_sgemm(M, N, K, 1.5, A, K, B, N, -0.25, C, N).cpu()
    assert torch.isfinite(got).all()
    err, where = sgemm_error(M, N, K, 1.5, A, K, B, N, -0.25, C, N, got)
    assert err <= FP32_TOL, "max normalised error %.3g at %s" % (err, where)
