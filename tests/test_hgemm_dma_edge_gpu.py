"""The half-precision direct-to-LDS kernels (binary16 and bfloat16) on ragged shapes,
on the GPU through the C ABI, against the CPU oracle.

Tiles 3-6 and 8 copy 16-byte chunks of A and B straight into LDS.  When M or N is not
a multiple of the tile, or K not a multiple of 64, they run a bounds-checked
instantiation: copies of rows past M - 1 (8-column chunks past N - 8) repeat the
last row (chunk) inside the matrix, the last K % 64 values of k go through one
zero-filled tail step, and the epilogue (bias, GELU, 16-bit rounding) stores
only rows < M and columns < N and reads the bias only for columns < N.  It needs
rows of A and B on 16-byte boundaries (lda, ldb multiples of 8) and N a multiple
of 8; tile 7 (the column split) runs as tile 6 off whole tiles.  Bar: max
|C - ref| / (|alpha| sum|a||b| + |bias|) <= 1e-2, nothing written outside C's
M x N window, the padding of A and B (NaN) never read.
"""
import pytest
import torch

import linear_algebra_sgemm_amd as lib
from linear_algebra_sgemm_amd import inputs
from tests.gpu_helpers import FP16_TOL, hgemm_error, note, run_hgemm

pytestmark = pytest.mark.gpu

FMTS = {"f16": torch.float16, "bf16": torch.bfloat16}
DMA_TILES = (3, 4, 5, 6, 8)
SHAPES = [(300, 520, 100), (257, 264, 33), (64, 64, 16), (1, 8, 1), (129, 136, 31),
          (511, 520, 64), (700, 904, 777), (256, 256, 40), (1000, 1000, 1000), (260, 8, 4100)]


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
def forced():
    yield
    lib.gemm_debug_force_tile(1, -1)


def ld8(x):
    """A leading dimension of at least x that is a multiple of 8 (16-byte rows)."""
    return (x + 7) // 8 * 8


def check(fmt, M, N, K, alpha, act, seed, label, with_bias=True, lda=None, ldb=None, ldc=None):
    A, B, bias = inputs.hgemm_inputs(M, N, K, seed, lda=lda or ld8(K), ldb=ldb, fmt=fmt)
    lda, ldb = A.shape[1], B.shape[1]
    ldc = ldc or N
    C = torch.full((M, ldc), float("nan"), dtype=FMTS[fmt])
    b = bias if with_bias else None
    note("half direct-to-LDS edge %s %s M=%d N=%d K=%d lda=%d ldb=%d ldc=%d act=%d bias=%s seed=%d"
         % (fmt, label, M, N, K, lda, ldb, ldc, act, with_bias, seed))
    got = run_hgemm(M, N, K, alpha, A, lda, B, ldb, b, act, C, ldc)
    err, where = hgemm_error(M, N, K, alpha, A, lda, B, ldb, b, act, got, ldc)
    assert err <= FP16_TOL, "max normalised error %.3g at %s (%s)" % (err, where, label)
    out = got.cpu()
    if ldc > N:
        assert torch.isnan(out[:, N:].float()).all(), "wrote outside the N columns"
    return out


@pytest.mark.parametrize("fmt", list(FMTS))
@pytest.mark.parametrize("tile", DMA_TILES)
@pytest.mark.parametrize("shape", SHAPES)
def test_ragged_shapes(fmt, tile, shape, forced):
    assert lib.gemm_debug_force_tile(1, tile) == lib.STATUS_SUCCESS
    M, N, K = shape
    # the configuration for packed operands (lda = K): with K % 8 != 0 the rows of A
    # are packed first when that pays, else tile 0 runs; with lda padded to a
    # multiple of 8, as here, the direct-to-LDS tile runs for every shape
    t, s = lib.gemm_debug_pick_config(1, M, N, K, 256)
    assert (t, s) == (tile, 1) or (K % 8 != 0 and t == (1 if tile == 8 else 0))
    check(fmt, M, N, K, 1.25, lib.ACT_GELU_TANH, seed=1100 + tile + M + K, label="tile %d" % tile)


@pytest.mark.parametrize("fmt", list(FMTS))
@pytest.mark.parametrize("tile", DMA_TILES)
def test_epilogue_options_and_leading_dimensions(fmt, tile, forced):
    """ldc a multiple of 8 (stores staged through LDS) and odd (direct stores);
    no bias, no activation; padded lda and ldb."""
    assert lib.gemm_debug_force_tile(1, tile) == lib.STATUS_SUCCESS
    check(fmt, 333, 296, 250, 0.5, lib.ACT_NONE, seed=1131 + tile, label="no bias, ldc 304",
          with_bias=False, lda=264, ldb=304, ldc=304)
    check(fmt, 333, 296, 250, -1.0, lib.ACT_GELU_TANH, seed=1132 + tile, label="ldc 301",
          lda=256, ldb=296, ldc=301)


@pytest.mark.parametrize("fmt", list(FMTS))
def test_column_split_tile_off_whole_tiles(fmt, forced):
    """Tile 7 on a ragged shape runs the eight-wave tile alone."""
    assert lib.gemm_debug_force_tile(1, 7) == lib.STATUS_SUCCESS
    assert lib.gemm_debug_pick_config(1, 300, 5120, 128, 256) == (6, 1)
    check(fmt, 300, 5120, 128, 1.0, lib.ACT_GELU_TANH, seed=1141, label="tile 7 -> 6")


@pytest.mark.parametrize("tile", DMA_TILES)
def test_guard_bands_untouched(tile, forced):
    assert lib.gemm_debug_force_tile(1, tile) == lib.STATUS_SUCCESS
    M, N, K = 270, 136, 72
    A, B, bias = inputs.hgemm_inputs(M, N, K, 1151 + tile)
    ldc = N + 8
    guard = 2 * ldc
    buf = torch.full((guard + M * ldc + guard,), 1234.0, dtype=torch.float16)
    body0 = torch.full((M, ldc), float("nan"), dtype=torch.float16)
    buf[guard:guard + M * ldc] = body0.reshape(-1)
    dA, dB, dbias, dbuf = A.cuda(), B.cuda(), bias.cuda(), buf.cuda()
    note("half direct-to-LDS edge guard bands tile %d" % tile)
    lib.hgemm_bias_act(M, N, K, 1.0, dA, K, dB, N, dbias, lib.ACT_GELU_TANH,
                       dbuf.data_ptr() + guard * 2, ldc)
    torch.cuda.synchronize()
    out = dbuf.cpu()
    assert torch.all(out[:guard] == 1234.0) and torch.all(out[guard + M * ldc:] == 1234.0)
    body = out[guard:guard + M * ldc].reshape(M, ldc)
    assert torch.isnan(body[:, N:].float()).all()
    err, where = hgemm_error(M, N, K, 1.0, A, K, B, N, bias, lib.ACT_GELU_TANH,
                             body.reshape(-1), ldc)
    assert err <= FP16_TOL, (err, where)


def test_misaligned_operands_are_packed(forced):
    """N not a multiple of 8, or lda not a multiple of 8: the operand is copied into the
    library's pack buffer with 16-byte rows and the direct-to-LDS tile reads the copy."""
    assert lib.gemm_debug_force_tile(1, 6) == lib.STATUS_SUCCESS
    assert lib.gemm_debug_pick_config(1, 600, 1028, 1000, 256) == (6, 1)
    check("f16", 600, 1028, 1000, 1.0, lib.ACT_GELU_TANH, seed=1161, label="N = 1028")
    check("f16", 600, 1024, 1000, 1.0, lib.ACT_GELU_TANH, seed=1162, label="lda = 1004", lda=1004)
    # too small for the copy to pay: the register-staged tile runs on the operands as given
    assert lib.gemm_debug_pick_config(1, 300, 260, 100, 256) == (0, 1)
    check("f16", 300, 260, 100, 1.0, lib.ACT_GELU_TANH, seed=1163, label="N = 260, not packed")


@pytest.mark.parametrize("fmt", list(FMTS))
@pytest.mark.parametrize("shape,want", [((4000, 14000, 4000), (6, 1)), ((3000, 3000, 3000), (6, 1)),
                                        ((1000, 1000, 1000), (8, 1)), ((2000, 2000, 2000), (8, 1))])
def test_auto_choice_ragged_every_element(fmt, shape, want):
    """Ragged products on the configuration the library picks, every output element
    against the oracle."""
    M, N, K = shape
    assert lib.gemm_debug_pick_config(
        1, M, N, K, torch.cuda.get_device_properties(0).multi_processor_count) == want
    A, B, bias = inputs.hgemm_inputs(M, N, K, 1171 + M, lda=ld8(K), fmt=fmt)
    lda = A.shape[1]
    C = torch.full((M, N), float("nan"), dtype=FMTS[fmt])
    note("half direct-to-LDS edge auto %s %dx%dx%d (expect tile %d)" % (fmt, M, N, K, want[0]))
    got = run_hgemm(M, N, K, 1.0, A, lda, B, N, bias, lib.ACT_GELU_TANH, C, N).cpu().float()
    assert torch.isfinite(got).all(), "every output written"
    err, where = hgemm_error(M, N, K, 1.0, A, lda, B, N, bias, lib.ACT_GELU_TANH, got, N)
    assert err <= FP16_TOL, "max normalised error %.3g at %s" % (err, where)
