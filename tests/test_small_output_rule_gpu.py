"""Parity at the boundaries of the automatic choice of the 16 x 16 K-split tiles
(FP32 tile 13, half tile 9): outputs of exactly one, two and four 16 x 16 tiles
per CU and one more, K at 2048 / 2049 and 4096 / 4097, whole and ragged, each
compared element by element with the CPU oracle on whatever configuration the
library picks.  The sizes scale with the device's CU count."""
import pytest
import torch

import linear_algebra_sgemm_amd as lib
from linear_algebra_sgemm_amd import inputs
from tests.gpu_helpers import FP16_TOL, FP32_TOL, hgemm_error, note, run_hgemm, run_sgemm, \
    sgemm_error

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def library():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.gemm_create()
    yield
    torch.cuda.synchronize()
    lib.gemm_destroy()


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def shapes():
    """(M, N, K): 16-row strips of 16 x 16 tiles, per_cu tiles per CU (+1 tile), at the
    K values where the rules change."""
    out = []
    for per_cu, ks in ((1, (4096, 4097)), (2, (2048, 2049)), (4, (2048, 2049))):
        tiles = per_cu * cus()
        for extra in (0, 1):
            n_tiles = tiles + extra
            M = 16 * 4
            N = 16 * ((n_tiles + 3) // 4) - (5 if extra else 0)   # ragged N past the boundary
            for K in ks:
                out.append((M, N, K))
    return out


@pytest.mark.parametrize("i", range(12))
def test_sgemm_at_rule_boundaries(i):
    M, N, K = shapes()[i]
    tile, splits = lib.gemm_debug_pick_config(0, M, N, K, cus())
    A, B, C = inputs.sgemm_inputs(M, N, K, 40000 + i)
    note("sgemm rule boundary M=%d N=%d K=%d (tile %d x%d)" % (M, N, K, tile, splits))
    got = run_sgemm(M, N, K, 1.25, A, K, B, N, -0.5, C, N)
    err, where = sgemm_error(M, N, K, 1.25, A, K, B, N, -0.5, C, N, got)
    assert err <= FP32_TOL, (err, where, tile, splits)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("i", range(12))
def test_half_at_rule_boundaries(i, fmt):
    M, N, K = shapes()[i]
    tile, splits = lib.gemm_debug_pick_config(1, M, N, K, cus())
    A, B, bias = inputs.hgemm_inputs(M, N, K, 41000 + i, fmt=fmt)
    dt = torch.bfloat16 if fmt == "bf16" else torch.float16
    C = torch.full((M, N), float("nan"), dtype=dt)
    note("%s rule boundary M=%d N=%d K=%d (tile %d x%d)" % (fmt, M, N, K, tile, splits))
    got = run_hgemm(M, N, K, 1.0, A, K, B, N, bias, lib.ACT_GELU_TANH, C, N)
    err, where = hgemm_error(M, N, K, 1.0, A, K, B, N, bias, lib.ACT_GELU_TANH, got, N)
    assert err <= FP16_TOL, (err, where, tile, splits)
