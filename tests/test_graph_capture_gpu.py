"""Calls captured into a HIP graph and replayed, next to eager calls.

A captured call may be replayed at any time later, unordered with the eager
calls that share the library's split-K workspace and pack buffer, so the
library plans captured calls without them (no split-K, no operand copies).
Each replay is checked against the oracle, with eager split-K calls on another
stream and the program's own synchronisations between the replays."""
import pytest
import torch

import linear_algebra_sgemm_amd as lib
from linear_algebra_sgemm_amd import inputs
from tests.gpu_helpers import FP16_TOL, FP32_TOL, hgemm_error, note, sgemm_error

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def library():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.gemm_create()
    yield
    torch.cuda.synchronize()
    lib.gemm_destroy()


def test_captured_split_shape_replays_next_to_eager_split_calls():
    M, N, K = 256, 256, 8192
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert lib.gemm_debug_pick_config(0, M, N, K, cus)[1] > 1, "this shape splits K when eager"
    A, B, C = inputs.sgemm_inputs(M, N, K, 301)
    dA, dB, dC0 = A.cuda(), B.cuda(), C.cuda()
    dC = dC0.clone()
    # eager operands on a second stream: a split-K call of another shape
    m, n, k = 192, 320, 6144
    a, b, c = inputs.sgemm_inputs(m, n, k, 302)
    da, db, dc0 = a.cuda(), b.cuda(), c.cuda()
    torch.cuda.synchronize()
    note("sgemm graph capture %dx%dx%d" % (M, N, K))
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            lib.sgemm(M, N, K, 1.25, dA, K, dB, N, -0.5, dC, N, stream=s)
    torch.cuda.synchronize()
    other = torch.cuda.Stream()
    for rep in range(3):
        dC.copy_(dC0)
        dc = dc0.clone()
        torch.cuda.synchronize()
        # the replay and the eager split-K call run concurrently on two streams
        g.replay()
        lib.sgemm(m, n, k, 0.75, da, k, db, n, 0.25, dc, n, stream=other)
        torch.cuda.synchronize()
        err, where = sgemm_error(M, N, K, 1.25, A, K, B, N, -0.5, C, N, dC)
        assert err <= FP32_TOL, ("replay", rep, err, where)
        err, where = sgemm_error(m, n, k, 0.75, a, k, b, n, 0.25, c, n, dc)
        assert err <= FP32_TOL, ("eager split call", rep, err, where)


def test_captured_half_product_with_unaligned_rows():
    """K = 1001: rows of A off 16-byte boundaries, which an eager call would copy into
    the pack buffer; the captured call runs the bounds-checked kernels instead."""
    M, N, K = 1024, 2048, 1001
    A, B, bias = inputs.hgemm_inputs(M, N, K, 303)
    dA, dB, dbias = A.cuda(), B.cuda(), bias.cuda()
    dC = torch.empty((M, N), dtype=torch.float16, device="cuda")
    torch.cuda.synchronize()
    note("hgemm graph capture %dx%dx%d" % (M, N, K))
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            lib.hgemm_bias_act(M, N, K, 1.0, dA, K, dB, N, dbias, lib.ACT_GELU_TANH, dC, N, stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        dC.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        err, where = hgemm_error(M, N, K, 1.0, A, K, B, N, bias, lib.ACT_GELU_TANH, dC, N)
        assert err <= FP16_TOL, ("replay", rep, err, where)
