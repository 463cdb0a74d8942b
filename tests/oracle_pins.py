"""Pins for the CPU oracle: checks against facts fixed by the mathematics, not by the
oracle's own formula.

Each pin takes an ``oracle.Oracle`` and raises AssertionError on a mismatch.  The
same pins run against the real oracle (tests/test_oracle.py) and against copies of
its source with planted mistakes, where at least one pin must fail.

What pins what:
* identity / permutation products (exact): operand indexing, leading dimensions,
  which operand is transposed, the alpha and beta terms;
* all-ones products (exact): the number of k terms summed;
* alpha = 0 and beta = 0 with NaN-filled operands: the BLAS reading that unread
  operands never reach the result;
* exact rational brute force on every shape up to 8 x 8 x 8 with padded leading
  dimensions: the whole sum, within the double-precision rounding bound, and the
  error scale ``den`` it returns;
* small-integer operands (exact): the product against Python integer arithmetic;
* binary16 decoding against numpy, bfloat16 decoding against torch, both over all
  65536 bit patterns;
* GELU(tanh) against its odd-part identity gelu(x) - gelu(-x) = x, its limits and
  torch's float64 ``gelu(approximate='tanh')``;
* the binary16 and bfloat16 products against torch.matmul in float64 and torch's GELU;
* the 16-bit products on small-integer operands with padded, NaN-filled leading
  dimensions against Python integer arithmetic (exact), and A = I giving B exactly:
  their indexing, leading dimensions and the number of k terms.
"""
from __future__ import annotations

import itertools
from fractions import Fraction

import numpy as np
import torch

import oracle as _oracle

U53 = 2.0 ** -53


def _rng(seed):
    return np.random.default_rng(seed)


def _f32(rng, shape):
    return rng.uniform(-1, 1, size=shape).astype(np.float32)


def pin_identity(o: _oracle.Oracle):
    rng = _rng(1)
    for (M, N, alpha, beta) in [(5, 7, 1.0, 0.0), (9, 4, 1.5, -0.25), (16, 33, -2.0, 0.5)]:
        K = M
        A = np.eye(M, dtype=np.float32)
        B = _f32(rng, (K, N))
        C0 = _f32(rng, (M, N))
        ref, _ = o.sgemm(M, N, K, alpha, A, K, B, N, beta, C0, N)
        want = alpha * B.astype(np.float64) + (beta * C0.astype(np.float64) if beta else 0.0)
        assert np.array_equal(ref, want), "A = I must give alpha*B + beta*C exactly"
        # B = I: alpha*A + beta*C
        A2 = _f32(rng, (M, N))
        Bi = np.eye(N, dtype=np.float32)
        ref2, _ = o.sgemm(M, N, N, alpha, A2, N, Bi, N, beta, C0, N)
        want2 = alpha * A2.astype(np.float64) + (beta * C0.astype(np.float64) if beta else 0.0)
        assert np.array_equal(ref2, want2), "B = I must give alpha*A + beta*C exactly"


def pin_permutation(o: _oracle.Oracle):
    rng = _rng(2)
    M, N = 11, 13
    p = rng.permutation(M)
    P = np.zeros((M, M), np.float32)
    P[np.arange(M), p] = 1.0            # (P B)[i] = B[p[i]]
    B = _f32(rng, (M, N))
    ref, _ = o.sgemm(M, N, M, 1.0, P, M, B, N, 0.0, None, N)
    assert np.array_equal(ref, B[p].astype(np.float64)), "row permutation of B"
    q = rng.permutation(N)
    Q = np.zeros((N, N), np.float32)
    Q[q, np.arange(N)] = 1.0            # (A Q)[:, j] = A[:, q[j]]
    A = _f32(rng, (M, N))
    ref2, _ = o.sgemm(M, N, N, 1.0, A, N, Q, N, 0.0, None, N)
    assert np.array_equal(ref2, A[:, q].astype(np.float64)), "column permutation of A"
    # A rectangular selection: M x K picks K-rows of B, with a padded lda and ldb.
    K = 7
    sel = rng.integers(0, K, size=M)
    S = np.full((M, K + 3), np.nan, np.float32)
    S[:, :K] = 0.0
    S[np.arange(M), sel] = 1.0
    Bp = np.full((K, N + 5), np.nan, np.float32)
    Bp[:, :N] = _f32(rng, (K, N))
    ref3, _ = o.sgemm(M, N, K, 1.0, S, K + 3, Bp, N + 5, 0.0, None, N)
    assert np.array_equal(ref3, Bp[sel, :N].astype(np.float64)), "selection with padded ld"


def pin_all_ones(o: _oracle.Oracle):
    rng = _rng(3)
    for (M, N, K, alpha, beta) in [(3, 4, 1, 1.0, 0.0), (6, 5, 97, 1.0, 0.0),
                                   (4, 9, 1000, 0.5, 2.0), (2, 2, 4096, 1.0, 1.0)]:
        A = np.ones((M, K), np.float32)
        B = np.ones((K, N), np.float32)
        C0 = rng.integers(-8, 8, size=(M, N)).astype(np.float32)
        ref, den = o.sgemm(M, N, K, alpha, A, K, B, N, beta, C0, N)
        want = alpha * K + beta * C0.astype(np.float64)
        assert np.array_equal(ref, want), "all-ones product must be alpha*K + beta*C"
        assert np.array_equal(den, abs(alpha) * K + abs(beta) * np.abs(C0.astype(np.float64)))


def pin_alpha_zero_and_unread(o: _oracle.Oracle):
    rng = _rng(4)
    M, N, K = 5, 6, 7
    A = np.full((M, K), np.nan, np.float32)
    B = np.full((K, N), np.nan, np.float32)
    C0 = _f32(rng, (M, N))
    ref, den = o.sgemm(M, N, K, 0.0, A, K, B, N, -0.75, C0, N)
    assert np.array_equal(ref, -0.75 * C0.astype(np.float64)), "alpha = 0 leaves beta*C"
    assert np.array_equal(den, 0.75 * np.abs(C0.astype(np.float64)))
    ref0, den0 = o.sgemm(M, N, 0, 1.0, A, 1, B, N, 2.0, C0, N)
    assert np.array_equal(ref0, 2.0 * C0.astype(np.float64)), "K = 0 leaves beta*C"
    # beta = 0: C is never read, even when it holds NaN.
    A2 = _f32(rng, (M, K))
    B2 = _f32(rng, (K, N))
    Cn = np.full((M, N), np.nan, np.float32)
    ref2, den2 = o.sgemm(M, N, K, 1.0, A2, K, B2, N, 0.0, Cn, N)
    assert np.all(np.isfinite(ref2)) and np.all(np.isfinite(den2)), "beta = 0 must not read C"
    # and the entry-wise form agrees
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    e_ref, _ = o.sgemm_entries(K, 0.0, A, K, B, N, -0.75, C0, N, rows.ravel(), cols.ravel())
    assert np.array_equal(e_ref, -0.75 * C0.astype(np.float64).ravel())


def _exact_sgemm(A, B, C0, alpha, beta, M, N, K, lda, ldb, ldc):
    """Exact rational alpha*A*B + beta*C0 and sum |alpha||a||b| + |beta||c| from the float values."""
    Af = A.ravel()
    Bf = B.ravel()
    Cf = None if C0 is None else C0.ravel()
    fa, fb = Fraction(alpha), Fraction(beta)
    out = [[None] * N for _ in range(M)]
    mag = [[None] * N for _ in range(M)]
    for i in range(M):
        arow = [Fraction(float(Af[i * lda + k])) for k in range(K)]
        for j in range(N):
            s = Fraction(0)
            m = Fraction(0)
            for k in range(K):
                b = Fraction(float(Bf[k * ldb + j]))
                s += arow[k] * b
                m += abs(arow[k] * b)
            c = Fraction(0) if beta == 0 else Fraction(float(Cf[i * ldc + j]))
            out[i][j] = fa * s + fb * c
            mag[i][j] = abs(fa) * m + abs(fb) * abs(c)
    return out, mag


def pin_brute_force_rational(o: _oracle.Oracle):
    rng = _rng(5)
    dims = range(1, 9)
    for (M, N, K) in itertools.product(dims, dims, dims):
        lda, ldb, ldc = K + (M % 3), N + (K % 2), N + 1
        alpha = float(np.float32(rng.uniform(-2, 2)))
        beta = float(np.float32(rng.uniform(-2, 2))) if (M + N + K) % 2 else 0.0
        A = np.full((M, lda), np.nan, np.float32)
        A[:, :K] = _f32(rng, (M, K))
        B = np.full((K, ldb), np.nan, np.float32)
        B[:, :N] = _f32(rng, (K, N))
        C0 = np.full((M, ldc), np.nan, np.float32)
        C0[:, :N] = _f32(rng, (M, N))
        ref, den = o.sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C0, ldc)
        exact, mag = _exact_sgemm(A, B, C0 if beta else None, alpha, beta, M, N, K, lda, ldb, ldc)
        for i in range(M):
            for j in range(N):
                m = float(mag[i][j])
                # each of the K products, K-1 sums, the alpha product and the beta terms
                # rounds once: (K + 3) u times the magnitude bounds the error (with margin)
                bound = (K + 4) * U53 * m
                err = abs(Fraction(float(ref[i, j])) - exact[i][j])
                assert err <= Fraction(bound), (M, N, K, i, j, float(err), bound)
                assert abs(den[i, j] - m) <= (K + 4) * U53 * m, "den must equal the magnitude sum"


def pin_small_integers_exact(o: _oracle.Oracle):
    rng = _rng(6)
    M, N, K = 17, 19, 23
    Ai = rng.integers(-9, 10, size=(M, K))
    Bi = rng.integers(-9, 10, size=(K, N))
    Ci = rng.integers(-9, 10, size=(M, N))
    ref, _ = o.sgemm(M, N, K, 2.0, Ai.astype(np.float32), K, Bi.astype(np.float32), N, -3.0,
                     Ci.astype(np.float32), N)
    want = [[2 * sum(int(Ai[i, k]) * int(Bi[k, j]) for k in range(K)) - 3 * int(Ci[i, j])
             for j in range(N)] for i in range(M)]
    assert np.array_equal(ref, np.array(want, dtype=np.float64)), "integer product must be exact"


def pin_entries_match_full(o: _oracle.Oracle):
    rng = _rng(7)
    M, N, K = 37, 29, 41
    A = _f32(rng, (M, K))
    B = _f32(rng, (K, N))
    C0 = _f32(rng, (M, N))
    ref, den = o.sgemm(M, N, K, 1.25, A, K, B, N, 0.5, C0, N)
    rows = rng.integers(0, M, size=200)
    cols = rng.integers(0, N, size=200)
    er, ed = o.sgemm_entries(K, 1.25, A, K, B, N, 0.5, C0, N, rows, cols)
    # both take each element's terms in ascending k, so they agree to the last bit
    assert np.array_equal(er, ref[rows, cols]) and np.array_equal(ed, den[rows, cols])


def pin_half_decoder(o: _oracle.Oracle):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = bits.view(np.float16).astype(np.float64)
    got = np.array([o.half_to_double(int(b)) for b in bits], dtype=np.float64)
    nan_w = np.isnan(want)
    assert np.array_equal(nan_w, np.isnan(got)), "NaN patterns"
    assert np.array_equal(got[~nan_w], want[~nan_w]), "binary16 decoding"
    assert np.array_equal(np.signbit(got[~nan_w]), np.signbit(want[~nan_w])), "signed zeros"


def pin_bf16_decoder(o: _oracle.Oracle):
    bits = np.arange(65536, dtype=np.int64).astype(np.int32)
    t = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([o.bf16_to_double(int(b)) for b in range(65536)], dtype=np.float64)
    nan_w = np.isnan(t)
    assert np.array_equal(nan_w, np.isnan(got)), "bfloat16 NaN patterns"
    assert np.array_equal(got[~nan_w], t[~nan_w]), "bfloat16 decoding"
    assert np.array_equal(np.signbit(got[~nan_w]), np.signbit(t[~nan_w])), "bfloat16 signed zeros"


def pin_gelu(o: _oracle.Oracle):
    assert o.gelu_tanh(0.0) == 0.0
    xs = np.concatenate([np.linspace(-8, 8, 401), [1e-6, 3.0, 0.5, 12.0, 30.0]])
    for x in xs:
        g, gm = o.gelu_tanh(float(x)), o.gelu_tanh(float(-x))
        # 0.5 x (1 + t) - 0.5 (-x)(1 - t) = x for the odd tanh: an exact identity of the form
        assert abs((g - gm) - x) <= 1e-14 * max(1.0, abs(x)), x
    assert o.gelu_tanh(30.0) == 30.0 and abs(o.gelu_tanh(-30.0)) < 1e-300 + 1e-12
    t = torch.tensor(xs, dtype=torch.float64)
    lib = torch.nn.functional.gelu(t, approximate="tanh").numpy()
    got = np.array([o.gelu_tanh(float(x)) for x in xs])
    assert np.allclose(got, lib, rtol=1e-14, atol=1e-15), "torch float64 gelu(tanh)"


def _f16(rng, shape, scale=0.5):
    return (rng.standard_normal(size=shape) * scale).astype(np.float16)


def pin_half_product_vs_torch(o: _oracle.Oracle):
    rng = _rng(8)
    for (M, N, K, alpha) in [(7, 9, 5, 1.0), (33, 20, 130, 0.75), (16, 64, 257, -1.5)]:
        A = _f16(rng, (M, K))
        B = _f16(rng, (K, N))
        bias = rng.standard_normal(N).astype(np.float32)
        prod = alpha * (torch.from_numpy(A.astype(np.float64)) @ torch.from_numpy(B.astype(np.float64)))
        mag = abs(alpha) * (torch.from_numpy(np.abs(A.astype(np.float64)))
                            @ torch.from_numpy(np.abs(B.astype(np.float64))))
        tol = (K + 4) * U53 * (mag.numpy() + np.abs(bias.astype(np.float64))) + 1e-300
        ref0, den0 = o.hgemm_bias_act(M, N, K, alpha, A, K, B, N, None, _oracle.ACT_NONE)
        assert np.all(np.abs(ref0 - prod.numpy()) <= tol), "plain fp16 product"
        assert np.allclose(den0, mag.numpy(), rtol=(K + 4) * U53, atol=0)
        x = prod + torch.from_numpy(bias.astype(np.float64))
        ref1, den1 = o.hgemm_bias_act(M, N, K, alpha, A, K, B, N, bias, _oracle.ACT_NONE)
        assert np.all(np.abs(ref1 - x.numpy()) <= tol), "bias added per column"
        assert np.allclose(den1, mag.numpy() + np.abs(bias.astype(np.float64)), rtol=(K + 4) * U53)
        ref2, _ = o.hgemm_bias_act(M, N, K, alpha, A, K, B, N, bias, _oracle.ACT_GELU_TANH)
        g = torch.nn.functional.gelu(x, approximate="tanh").numpy()
        assert np.all(np.abs(ref2 - g) <= 2 * tol + 1e-14 * np.abs(g)), "gelu(x + bias)"
        rows = rng.integers(0, M, 50)
        cols = rng.integers(0, N, 50)
        er, ed = o.hgemm_entries(K, alpha, A, K, B, N, bias, _oracle.ACT_GELU_TANH, rows, cols)
        assert np.array_equal(er, ref2[rows, cols])


def pin_bf16_product_vs_torch(o: _oracle.Oracle):
    rng = _rng(9)
    for (M, N, K, alpha) in [(9, 7, 11, 1.0), (24, 40, 200, -0.5)]:
        A = torch.from_numpy(rng.standard_normal((M, K)) * 0.5).to(torch.bfloat16)
        B = torch.from_numpy(rng.standard_normal((K, N)) * 0.5).to(torch.bfloat16)
        bias = rng.standard_normal(N).astype(np.float32)
        a64, b64 = A.to(torch.float64), B.to(torch.float64)
        x = alpha * (a64 @ b64) + torch.from_numpy(bias.astype(np.float64))
        mag = abs(alpha) * (a64.abs() @ b64.abs()) + torch.from_numpy(np.abs(bias.astype(np.float64)))
        tol = (K + 4) * U53 * mag.numpy() + 1e-300
        bits = lambda t: t.view(torch.int16).numpy()  # noqa: E731
        ref0, den0 = o.hgemm_bias_act(M, N, K, alpha, bits(A), K, bits(B), N, bias, _oracle.ACT_NONE,
                                      fmt="bf16")
        assert np.all(np.abs(ref0 - x.numpy()) <= tol), "bfloat16 product + bias"
        assert np.allclose(den0, mag.numpy(), rtol=(K + 4) * U53)
        ref1, _ = o.hgemm_bias_act(M, N, K, alpha, bits(A), K, bits(B), N, bias,
                                   _oracle.ACT_GELU_TANH, fmt="bf16")
        g = torch.nn.functional.gelu(x, approximate="tanh").numpy()
        assert np.all(np.abs(ref1 - g) <= 2 * tol + 1e-14 * np.abs(g)), "bfloat16 gelu(x + bias)"
        rows = rng.integers(0, M, 30)
        cols = rng.integers(0, N, 30)
        er, _ = o.hgemm_entries(K, alpha, bits(A), K, bits(B), N, bias, _oracle.ACT_GELU_TANH,
                                rows, cols, fmt="bf16")
        assert np.array_equal(er, ref1[rows, cols])


def pin_half_unread(o: _oracle.Oracle):
    M, N, K = 4, 6, 5
    A = np.full((M, K), np.nan, np.float16)
    B = np.full((K, N), np.nan, np.float16)
    bias = np.linspace(-3, 3, N).astype(np.float32)
    ref, _ = o.hgemm_bias_act(M, N, K, 0.0, A, K, B, N, bias, _oracle.ACT_GELU_TANH)
    want = torch.nn.functional.gelu(torch.from_numpy(bias.astype(np.float64)),
                                    approximate="tanh").numpy()
    assert np.allclose(ref, np.broadcast_to(want, (M, N)), rtol=1e-14, atol=1e-15)


def pin_half_integers_padded_exact(o: _oracle.Oracle):
    """Small integers are exact in binary16 and bfloat16 and so are their K-term sums here,
    so the 16-bit products must equal Python's integer arithmetic bit for bit, with the
    padding of A and B (NaN) never read."""
    rng = _rng(10)
    for fmt, dt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        for (M, N, K) in [(5, 7, 3), (13, 11, 29), (8, 33, 64)]:
            lda, ldb = K + 3, N + 2
            Ai = rng.integers(-6, 7, size=(M, K))
            Bi = rng.integers(-6, 7, size=(K, N))
            A = torch.full((M, lda), float("nan"), dtype=dt)
            A[:, :K] = torch.from_numpy(Ai.astype(np.float32)).to(dt)
            B = torch.full((K, ldb), float("nan"), dtype=dt)
            B[:, :N] = torch.from_numpy(Bi.astype(np.float32)).to(dt)
            bits = lambda t: t.contiguous().view(torch.int16).numpy()  # noqa: E731
            ref, den = o.hgemm_bias_act(M, N, K, 2.0, bits(A), lda, bits(B), ldb, None,
                                        _oracle.ACT_NONE, fmt=fmt)
            want = [[2 * sum(int(Ai[i, k]) * int(Bi[k, j]) for k in range(K)) for j in range(N)]
                    for i in range(M)]
            mag = [[2 * sum(abs(int(Ai[i, k]) * int(Bi[k, j])) for k in range(K))
                    for j in range(N)] for i in range(M)]
            assert np.array_equal(ref, np.array(want, np.float64)), "%s integer product" % fmt
            assert np.array_equal(den, np.array(mag, np.float64)), "%s integer magnitudes" % fmt
            # A = I (M = K): the product returns B's rows exactly, bias added per column
            eye = torch.full((K, K + 1), float("nan"), dtype=dt)
            eye[:, :K] = torch.eye(K).to(dt)
            bias = np.arange(N, dtype=np.float32) - N / 2
            refi, _ = o.hgemm_bias_act(K, N, K, 1.0, bits(eye), K + 1, bits(B), ldb, bias,
                                       _oracle.ACT_NONE, fmt=fmt)
            assert np.array_equal(refi, Bi.astype(np.float64) + bias.astype(np.float64)), \
                "%s identity product" % fmt


PINS = [pin_identity, pin_permutation, pin_all_ones, pin_alpha_zero_and_unread,
        pin_brute_force_rational, pin_small_integers_exact, pin_entries_match_full,
        pin_half_decoder, pin_bf16_decoder, pin_gelu, pin_half_product_vs_torch,
        pin_bf16_product_vs_torch, pin_half_unread, pin_half_integers_padded_exact]


def failing_pins(o: _oracle.Oracle):
    """Names of the pins that fail (or crash) on this oracle build."""
    bad = []
    for pin in PINS:
        try:
            pin(o)
        except Exception:  # noqa: BLE001 - any failure counts
            bad.append(pin.__name__)
    return bad
