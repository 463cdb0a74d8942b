"""Host-side logic on the CPU: the cost model against the pages' printed figures and
the seeded input generator."""
import json
import os

import numpy as np
import pytest
import torch

from linear_algebra_sgemm_amd import cost, inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cost_model.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["entries"]


@pytest.mark.parametrize("entry", _golden(), ids=lambda e: e["what"][:40])
def test_cost_model_matches_pages(entry):
    w = entry["what"]
    if "BM" in entry:
        got = cost.tile_intensity(entry["BM"], entry["BN"])
    elif "gflops" in entry:
        got = cost.gemm_flops(entry["M"], entry["N"], entry["K"]) / (entry["gflops"] * 1e9) * 1e3
    elif w.startswith("2*M*N*K"):
        got = cost.gemm_flops(entry["M"], entry["N"], entry["K"]) / 1e9
    elif "bytes" in w or "volume" in w:
        got = cost.sgemm_bytes(entry["M"], entry["N"], entry["K"], entry["beta"]) / 1e6
    else:
        f = cost.gemm_flops(entry["M"], entry["N"], entry["K"])
        b = cost.sgemm_bytes(entry["M"], entry["N"], entry["K"], entry["beta"])
        got = cost.arithmetic_intensity(f, b)
    tol = entry["rel_tol"]
    assert abs(got - entry["value"]) <= tol * abs(entry["value"]) + 1e-12, (w, got, entry["cite"])


def test_half_bytes_and_balance():
    # fp16 A (4096x4096), B (4096x14336), fp32 bias, fp16 C (4096x14336)
    b = cost.hgemm_bias_act_bytes(4096, 14336, 4096)
    assert b == 2 * 4096 * 4096 + 2 * 4096 * 14336 + 4 * 14336 + 2 * 4096 * 14336
    assert abs(cost.machine_balance("f32") - 19.6625) < 1e-9
    assert cost.PEAK_TFLOPS["f32"] == pytest.approx(256 * 256 * 2.4e9 / 1e12, rel=1e-3)
    assert cost.PEAK_TFLOPS["f16"] == pytest.approx(256 * 4096 * 2.4e9 / 1e12, rel=1e-4)


def test_inputs_reproducible_and_ordered():
    A1, B1, C1 = inputs.sgemm_inputs(31, 17, 9, seed=3)
    A2, B2, C2 = inputs.sgemm_inputs(31, 17, 9, seed=3)
    assert inputs.sha256(A1, B1, C1) == inputs.sha256(A2, B2, C2)
    # drawn in the order A, B, C from one generator
    g = torch.Generator().manual_seed(3)
    a = torch.rand((31, 9), generator=g) * 2 - 1
    assert torch.equal(a, A1)
    assert float(A1.min()) >= -1 and float(A1.max()) < 1
    A3, _, _ = inputs.sgemm_inputs(31, 17, 9, seed=4)
    assert not torch.equal(A1, A3)


def test_inputs_padding_is_nan():
    A, B, C = inputs.sgemm_inputs(5, 6, 7, seed=0, lda=9, ldb=8, ldc=11)
    assert A.shape == (5, 9) and B.shape == (7, 8) and C.shape == (5, 11)
    assert torch.isnan(A[:, 7:]).all() and torch.isnan(B[:, 6:]).all() and torch.isnan(C[:, 6:]).all()
    assert torch.isfinite(A[:, :7]).all()


def test_half_inputs():
    A, B, bias = inputs.hgemm_inputs(64, 48, 32, seed=3)
    assert A.dtype == torch.float16 and B.dtype == torch.float16 and bias.dtype == torch.float32
    assert bias.shape == (48,)
    assert 0.01 < float(A.float().std()) < 0.03


def test_workloads_table():
    w = inputs.WORKLOADS
    assert (w["sgemm_4096"].M, w["sgemm_4096"].alpha, w["sgemm_4096"].beta) == (4096, 1.0, 0.5)
    assert (w["sgemm_ragged"].M, w["sgemm_ragged"].N, w["sgemm_ragged"].K) == (1000, 3000, 777)
    assert (w["hgemm_ffn"].N, w["hgemm_ffn"].seed) == (14336, 3)
    assert w["sgemm_8192"].dist_ab == "normal" and w["sgemm_8192"].beta == 1.0


def test_sample_indices_cover_edges():
    r, c = inputs.sample_indices(1000, 3000, 256, seed=2)
    assert r.min() >= 0 and r.max() == 999 and c.min() >= 0 and c.max() == 2999
    assert ((r == 999) & (c == 2999)).any()
    assert np.array_equal(inputs.sample_indices(1000, 3000, 256, seed=2)[0], r)
