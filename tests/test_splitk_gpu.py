"""Split-K FP32 GEMM on the GPU through the C ABI, against the CPU oracle.

Split-K runs K chunks of one output tile on different workgroups, writes FP32
partials to the library's workspace and adds them in a fixed order in a second
kernel.  Same bar as the unsplit product: max |C - ref| / (|alpha| sum|a||b| +
|beta||c|) <= 1e-5; bit-exact where every partial sum is exactly representable;
bit-identical results from run to run.
"""
import pytest
import torch

import linear_algebra_sgemm_amd as lib
from linear_algebra_sgemm_amd import inputs
from tests.gpu_helpers import FP32_TOL, note, run_sgemm, sgemm_error

pytestmark = pytest.mark.gpu

TILES = (0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12)
RESOLVED = {7: 4, 8: 4, 9: 4, 10: 4, 11: 2}   # direct-to-LDS tiles fall back to their register-staged twin off whole tiles


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


def force(tile, splits):
    assert lib.gemm_debug_force_tile(0, tile) == lib.STATUS_SUCCESS
    assert lib.gemm_debug_force_splits(0, splits) == lib.STATUS_SUCCESS


def check(M, N, K, alpha, beta, seed, label, lda=None, ldb=None, ldc=None):
    A, B, C = inputs.sgemm_inputs(M, N, K, seed, lda=lda, ldb=ldb, ldc=ldc)
    lda, ldb, ldc = A.shape[1], B.shape[1], C.shape[1]
    note("sgemm split-K %s M=%d N=%d K=%d lda=%d ldb=%d ldc=%d alpha=%g beta=%g seed=%d"
         % (label, M, N, K, lda, ldb, ldc, alpha, beta, seed))
    got = run_sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)
    err, where = sgemm_error(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, got)
    assert err <= FP32_TOL, "max normalised error %.3g at %s (%s)" % (err, where, label)
    out = got.cpu()
    if ldc > N:
        assert torch.isnan(out[:, N:]).all(), "wrote outside the N columns"
    return out


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("splits", [2, 5, 32])
@pytest.mark.parametrize("shape", [(256, 256, 256), (300, 260, 1000), (128, 192, 4096),
                                   (17, 33, 515)])
def test_forced_splits_every_tile(tile, splits, shape, forced):
    force(tile, splits)
    M, N, K = shape
    t, s = lib.gemm_debug_pick_config(0, M, N, K, 256)
    assert t in (tile, RESOLVED.get(tile)) and 1 <= s <= splits
    check(M, N, K, 1.25, -0.5, seed=300 + 7 * tile + splits, label="tile %d x%d" % (tile, s))


@pytest.mark.parametrize("shape", [(256, 256, 256), (128, 128, 16384), (64, 1000, 3000),
                                   (129, 129, 129)])
def test_automatic_choice(shape):
    M, N, K = shape
    t, s = lib.gemm_debug_pick_config(0, M, N, K, torch.cuda.get_device_properties(0).multi_processor_count)
    check(M, N, K, 0.75, 0.5, seed=M + N + K, label="auto tile %d x%d" % (t, s))


def test_beta_zero_leaves_c_unread(forced):
    force(2, 8)
    M, N, K = 200, 136, 600
    A, B, _ = inputs.sgemm_inputs(M, N, K, 311)
    Cn = torch.full((M, N), float("nan"))
    note("sgemm split-K beta=0 NaN C")
    got = run_sgemm(M, N, K, 2.0, A, K, B, N, 0.0, Cn, N)
    assert torch.isfinite(got).all(), "beta = 0 must not read C"
    err, where = sgemm_error(M, N, K, 2.0, A, K, B, N, 0.0, Cn, N, got)
    assert err <= FP32_TOL, (err, where)


def test_padded_leading_dimensions_and_guard_bands(forced):
    force(1, 4)
    M, N, K = 190, 150, 333
    A, B, C = inputs.sgemm_inputs(M, N, K, 313, lda=K + 5, ldb=N + 3, ldc=N + 7)
    lda, ldb, ldc = A.shape[1], B.shape[1], C.shape[1]
    guard = 3 * ldc
    Cbuf = torch.full((guard + M * ldc + guard,), 12345.0, dtype=torch.float32)
    Cbuf[guard:guard + M * ldc] = C.reshape(-1)
    dA, dB, dC = A.cuda(), B.cuda(), Cbuf.cuda()
    note("sgemm split-K padded ld + guard bands")
    lib.sgemm(M, N, K, 1.0, dA, lda, dB, ldb, 0.5, dC.data_ptr() + guard * 4, ldc)
    torch.cuda.synchronize()
    out = dC.cpu()
    assert torch.all(out[:guard] == 12345.0) and torch.all(out[guard + M * ldc:] == 12345.0)
    body = out[guard:guard + M * ldc].reshape(M, ldc)
    assert torch.isnan(body[:, N:]).all()
    err, where = sgemm_error(M, N, K, 1.0, A, lda, B, ldb, 0.5, C, ldc, body.reshape(-1))
    assert err <= FP32_TOL, (err, where)


@pytest.mark.parametrize("tile", [2, 4])
def test_unaligned_base_pointers(tile, forced):
    force(tile, 4)
    M, N, K = 128, 256, 512
    A, B, C = inputs.sgemm_inputs(M, N, K, 317)
    bufA = torch.zeros(M * K + 1)
    bufA[1:] = A.reshape(-1)
    bufB = torch.zeros(K * N + 1)
    bufB[1:] = B.reshape(-1)
    dA, dB, dC = bufA.cuda(), bufB.cuda(), C.cuda()
    note("sgemm split-K unaligned base tile=%d" % tile)
    lib.sgemm(M, N, K, 1.0, dA.data_ptr() + 4, K, dB.data_ptr() + 4, N, -1.0, dC, N)
    torch.cuda.synchronize()
    err, where = sgemm_error(M, N, K, 1.0, A, K, B, N, -1.0, C, N, dC)
    assert err <= FP32_TOL, (err, where)


def test_exact_small_integers(forced):
    force(2, 7)
    M, N, K = 96, 160, 700
    g = torch.Generator().manual_seed(319)
    Ai = torch.randint(-9, 10, (M, K), generator=g)
    Bi = torch.randint(-9, 10, (K, N), generator=g)
    Ci = torch.randint(-9, 10, (M, N), generator=g)
    want = (2 * (Ai.long() @ Bi.long()) - 3 * Ci.long()).float()
    note("sgemm split-K small integers")
    got = run_sgemm(M, N, K, 2.0, Ai.float(), K, Bi.float(), N, -3.0, Ci.float(), N).cpu()
    assert torch.equal(got, want), "small-integer products must be exact with split-K too"


def test_deterministic_and_close_to_unsplit(forced):
    M, N, K = 256, 384, 2048
    A, B, C = inputs.sgemm_inputs(M, N, K, 321)
    force(2, 8)
    note("sgemm split-K determinism")
    g1 = run_sgemm(M, N, K, 1.0, A, K, B, N, 0.5, C, N).cpu()
    g2 = run_sgemm(M, N, K, 1.0, A, K, B, N, 0.5, C, N).cpu()
    assert torch.equal(g1, g2), "split-K must give the same bits on every run"
    force(2, 1)
    g0 = run_sgemm(M, N, K, 1.0, A, K, B, N, 0.5, C, N).cpu()
    for g in (g0, g1):
        err, where = sgemm_error(M, N, K, 1.0, A, K, B, N, 0.5, C, N, g)
        assert err <= FP32_TOL, (err, where)


def test_streams_take_turns_on_the_workspace(forced):
    """Back-to-back split-K calls on three streams share one workspace; the library
    orders them, so every result is right."""
    force(2, 8)
    streams = [torch.cuda.Stream() for _ in range(3)]
    cases = []
    for i in range(9):
        M, N, K = 192 + 32 * (i % 3), 256 - 64 * (i % 2), 512 + 128 * i
        A, B, C = inputs.sgemm_inputs(M, N, K, 330 + i)
        cases.append((M, N, K, A, B, C, A.cuda(), B.cuda(), C.cuda()))
    torch.cuda.synchronize()
    note("sgemm split-K 9 calls over 3 streams")
    for i, (M, N, K, A, B, C, dA, dB, dC) in enumerate(cases):
        lib.sgemm(M, N, K, 1.0, dA, K, dB, N, 1.0, dC, N, stream=streams[i % 3])
    torch.cuda.synchronize()
    for (M, N, K, A, B, C, dA, dB, dC) in cases:
        err, where = sgemm_error(M, N, K, 1.0, A, K, B, N, 1.0, C, N, dC)
        assert err <= FP32_TOL, (M, N, K, err, where)
