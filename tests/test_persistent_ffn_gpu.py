"""The persistent form of the half products' column split (tile 7 with K of at least
six 32-wide K tiles): one workgroup per CU walks its 256x256 head tiles and then
its 128x256 tail tile, loading each next tile's first K tiles under the current
tile's epilogue.  Every output element against the oracle, on shapes with one to
four head tiles per workgroup, tails that reach every workgroup or only a few,
with and without bias and activation, at the smallest K it takes.

Bar: max |C - ref| / (|alpha| sum_k |a||b| + |bias_j|) <= 1e-2."""
import pytest
import torch

import linear_algebra_sgemm_amd as lib
from linear_algebra_sgemm_amd import inputs
from tests.gpu_helpers import FP16_TOL, hgemm_error, note, run_hgemm

pytestmark = pytest.mark.gpu

FMTS = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def library():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.gemm_create()
    yield
    lib.gemm_debug_force_tile(1, -1)
    torch.cuda.synchronize()
    lib.gemm_destroy()


@pytest.mark.parametrize("fmt,M,N,K,alpha,with_bias,act", [
    ("f16", 4096, 5120, 1024, 1.25, True, lib.ACT_GELU_TANH),    # one head tile per workgroup, tail on half
    ("bf16", 2048, 10240, 2048, 0.75, False, lib.ACT_NONE),      # no bias, no activation
    ("f16", 1024, 16640, 256, 1.0, True, lib.ACT_GELU_TANH),     # tail tiles on 8 workgroups only
    ("bf16", 8192, 9216, 192, 1.0, True, lib.ACT_GELU_TANH),     # four head tiles each, smallest K
])
def test_persistent_column_split(fmt, M, N, K, alpha, with_bias, act):
    lib.gemm_debug_force_tile(1, 7)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert lib.gemm_debug_pick_config(1, M, N, K, cus)[0] == 7, "the column split applies"
    A, B, bias = inputs.hgemm_inputs(M, N, K, M + N + K, fmt=fmt)
    C = torch.full((M, N), float("nan"), dtype=FMTS[fmt])
    b = bias if with_bias else None
    note("persistent split %s %dx%dx%d alpha=%g bias=%s act=%d" % (fmt, M, N, K, alpha, with_bias,
                                                                   act))
    got = run_hgemm(M, N, K, alpha, A, K, B, N, b, act, C, N).cpu()
    assert torch.isfinite(got.float()).all(), "every output written"
    err, where = hgemm_error(M, N, K, alpha, A, K, B, N, b, act, got, N)
    assert err <= FP16_TOL, "max normalised error %.3g at %s" % (err, where)


def test_persistent_split_is_deterministic():
    lib.gemm_debug_force_tile(1, 7)
    M, N, K = 4096, 5120, 512
    A, B, bias = inputs.hgemm_inputs(M, N, K, 77)
    C = torch.empty((M, N), dtype=torch.float16)
    note("persistent split determinism")
    g1 = run_hgemm(M, N, K, 1.0, A, K, B, N, bias, lib.ACT_GELU_TANH, C, N).cpu()
    g2 = run_hgemm(M, N, K, 1.0, A, K, B, N, bias, lib.ACT_GELU_TANH, C, N).cpu()
    assert torch.equal(g1, g2)
