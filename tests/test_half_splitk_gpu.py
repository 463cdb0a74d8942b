"""Split-K of the half products (binary16 and bfloat16) on the GPU through the C ABI,
against the CPU oracle.

K chunks of one output tile run on different workgroups of the register-staged
kernel and write FP32 partials to the library's workspace; a second kernel adds
them in a fixed order, applies alpha, the bias and GELU, and rounds to the 16-bit
format.  Bar: max |C - ref| / (|alpha| sum|a||b| + |bias|) <= 1e-2; identical bits
from run to run.
"""
import pytest
import torch

import linear_algebra_sgemm_amd as lib
from linear_algebra_sgemm_amd import inputs
from tests.gpu_helpers import FP16_TOL, FP32_TOL, hgemm_error, note, run_hgemm, sgemm_error

pytestmark = pytest.mark.gpu

FMTS = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def library():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.gemm_create()
    yield
    for op in (0, 1):
        lib.gemm_debug_force_tile(op, -1)
        lib.gemm_debug_force_splits(op, -1)
    torch.cuda.synchronize()
    lib.gemm_destroy()


@pytest.fixture
def forced():
    yield
    lib.gemm_debug_force_tile(1, -1)
    lib.gemm_debug_force_splits(1, -1)


def force(tile, splits):
    assert lib.gemm_debug_force_tile(1, tile) == lib.STATUS_SUCCESS
    assert lib.gemm_debug_force_splits(1, splits) == lib.STATUS_SUCCESS


def check(fmt, M, N, K, alpha, act, seed, with_bias=True, ldc=None, label=""):
    A, B, bias = inputs.hgemm_inputs(M, N, K, seed, fmt=fmt)
    ldc = ldc or N
    C = torch.full((M, ldc), float("nan"), dtype=FMTS[fmt])
    b = bias if with_bias else None
    note("half split-K %s %s M=%d N=%d K=%d ldc=%d act=%d seed=%d" % (fmt, label, M, N, K, ldc, act,
                                                                       seed))
    got = run_hgemm(M, N, K, alpha, A, K, B, N, b, act, C, ldc)
    err, where = hgemm_error(M, N, K, alpha, A, K, B, N, b, act, got, ldc)
    assert err <= FP16_TOL, "max normalised error %.3g at %s (%s)" % (err, where, label)
    out = got.cpu()
    if ldc > N:
        assert torch.isnan(out[:, N:].float()).all(), "wrote outside the N columns"
    return out


@pytest.mark.parametrize("fmt", list(FMTS))
@pytest.mark.parametrize("tile", [0, 1, 2])
@pytest.mark.parametrize("splits", [2, 7, 32])
@pytest.mark.parametrize("shape", [(256, 256, 1024), (300, 260, 1000), (64, 192, 2048)])
def test_forced_splits(fmt, tile, splits, shape, forced):
    force(tile, splits)
    M, N, K = shape
    t, s = lib.gemm_debug_pick_config(1, M, N, K, 256)
    assert t == tile and 1 <= s <= splits
    check(fmt, M, N, K, 1.25, lib.ACT_GELU_TANH, seed=700 + tile + splits,
          label="tile %d x%d" % (tile, s))


@pytest.mark.parametrize("fmt", list(FMTS))
@pytest.mark.parametrize("splits", [2, 7, 32])
@pytest.mark.parametrize("shape", [(256, 256, 1024), (300, 264, 1000), (128, 640, 2048),
                                   (1000, 520, 2000), (129, 136, 776)])
def test_forced_splits_direct_tile(fmt, splits, shape, forced):
    """The 128x128 direct-to-LDS tile with K split: whole and ragged tiles, K chunks
    of whole 64-wide steps, the last chunk ragged (its bounds-checked tail step)."""
    force(8, splits)
    M, N, K = shape
    t, s = lib.gemm_debug_pick_config(1, M, N, K, 256)
    assert t == 8 and 1 <= s <= splits
    check(fmt, M, N, K, 0.75, lib.ACT_GELU_TANH, seed=760 + splits + M,
          label="tile 8 x%d" % s)


@pytest.mark.parametrize("fmt", list(FMTS))
def test_epilogue_options_and_padded_ldc(fmt, forced):
    force(2, 6)
    check(fmt, 200, 136, 768, 0.5, lib.ACT_NONE, seed=711, with_bias=False, ldc=141,
          label="no bias, no act, ldc 141")
    check(fmt, 200, 136, 768, -1.0, lib.ACT_GELU_TANH, seed=712, ldc=136, label="alpha -1")


@pytest.mark.parametrize("shape", [(512, 512, 4096), (300, 500, 4096), (128, 256, 8192)])
def test_automatic_choice(shape):
    M, N, K = shape
    t, s = lib.gemm_debug_pick_config(1, M, N, K,
                                      torch.cuda.get_device_properties(0).multi_processor_count)
    check("f16", M, N, K, 1.0, lib.ACT_GELU_TANH, seed=M + N + K, label="auto tile %d x%d" % (t, s))


def test_deterministic(forced):
    force(2, 8)
    M, N, K = 256, 384, 2048
    A, B, bias = inputs.hgemm_inputs(M, N, K, 721)
    C = torch.zeros((M, N), dtype=torch.float16)
    note("half split-K determinism")
    g1 = run_hgemm(M, N, K, 1.0, A, K, B, N, bias, lib.ACT_GELU_TANH, C, N).cpu()
    g2 = run_hgemm(M, N, K, 1.0, A, K, B, N, bias, lib.ACT_GELU_TANH, C, N).cpu()
    assert torch.equal(g1, g2), "split-K must give the same bits on every run"


def test_fp32_and_half_share_the_workspace(forced):
    """Split-K calls of both products on two streams take turns on the one workspace."""
    force(2, 8)
    assert lib.gemm_debug_force_tile(0, 2) == lib.STATUS_SUCCESS
    assert lib.gemm_debug_force_splits(0, 8) == lib.STATUS_SUCCESS
    try:
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        Mh, Nh, Kh = 256, 320, 1536
        Ah, Bh, bias = inputs.hgemm_inputs(Mh, Nh, Kh, 731)
        Ms, Ns, Ks = 192, 256, 2048
        As, Bs, Cs = inputs.sgemm_inputs(Ms, Ns, Ks, 732)
        dAh, dBh, dbias = Ah.cuda(), Bh.cuda(), bias.cuda()
        dCh = torch.empty((Mh, Nh), dtype=torch.float16, device="cuda")
        dAs, dBs, dCs = As.cuda(), Bs.cuda(), Cs.cuda()
        torch.cuda.synchronize()
        note("half + FP32 split-K on two streams")
        for _ in range(3):
            lib.hgemm_bias_act(Mh, Nh, Kh, 1.0, dAh, Kh, dBh, Nh, dbias, lib.ACT_GELU_TANH, dCh, Nh,
                               stream=s1)
            lib.sgemm(Ms, Ns, Ks, 1.0, dAs, Ks, dBs, Ns, 0.0, dCs, Ns, stream=s2)
        torch.cuda.synchronize()
        err, where = hgemm_error(Mh, Nh, Kh, 1.0, Ah, Kh, Bh, Nh, bias, lib.ACT_GELU_TANH, dCh, Nh)
        assert err <= FP16_TOL, (err, where)
        err, where = sgemm_error(Ms, Ns, Ks, 1.0, As, Ks, Bs, Ns, 0.0, Cs, Ns, dCs)
        assert err <= FP32_TOL, (err, where)
    finally:
        lib.gemm_debug_force_tile(0, -1)
        lib.gemm_debug_force_splits(0, -1)
