"""CPU oracle for C = alpha*A*B + beta*C and the fp16 bias + GELU(tanh) product.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The GPU library never imports, links or
executes anything here, and this package imports nothing from it.

The arithmetic lives in ``oracle.c`` (plain C, IEEE double, no FMA contraction,
ascending-k sums, OpenMP over rows); this module builds it with gcc and
marshals numpy arrays through ctypes.  The definition it follows is the problem
statement of "SGEMM优化，从naive到warptiling" (section 问题与估算) and, for the
half-precision variants (binary16 and bfloat16 inputs), the fused bias/activation epilogue of the DeepGEMM page
(sections 1.1 and 3.2); the header of ``oracle.c`` states each reading.

Every function here is pinned by tests that do not reuse its own formula:
identity and permutation products, all-ones sums, alpha = 0 and beta = 0
special cases, exact rational brute force on tiny shapes, the binary16 decoder
against numpy over all 65536 bit patterns, and GELU against its odd-part
identity and torch's float64 implementation.  The pins are also run against
deliberately broken copies of ``oracle.c`` to show that they catch mistakes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

ACT_NONE = 0
ACT_GELU_TANH = 1


def build(force: bool = True, src: str = SOURCE, out: str = LIB_PATH) -> str:
    """Compile the oracle C source with gcc into a shared library; return its path."""
    if not force and os.path.exists(out):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=gnu11", "-O2", "-fno-fast-math", "-ffp-contract=off",
           "-fopenmp", "-fPIC", "-shared", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(lib):
    P = ctypes.c_void_p
    i32, f64, i64 = ctypes.c_int, ctypes.c_double, ctypes.c_int64
    lib.oracle_sgemm.argtypes = [i32, i32, i32, f64, P, i32, P, i32, f64, P, i32, P, P, i32]
    lib.oracle_sgemm.restype = None
    lib.oracle_sgemm_entries.argtypes = [i32, f64, P, i32, P, i32, f64, P, i32, P, P, i64, P, P,
                                         i32]
    lib.oracle_sgemm_entries.restype = None
    lib.oracle_hgemm_bias_act.argtypes = [i32, i32, i32, f64, P, i32, P, i32, P, i32, P, P, i32]
    lib.oracle_hgemm_bias_act.restype = None
    lib.oracle_hgemm_entries.argtypes = [i32, f64, P, i32, P, i32, P, i32, P, P, i64, P, P, i32]
    lib.oracle_hgemm_entries.restype = None
    lib.oracle_bgemm_bias_act.argtypes = [i32, i32, i32, f64, P, i32, P, i32, P, i32, P, P, i32]
    lib.oracle_bgemm_bias_act.restype = None
    lib.oracle_bgemm_entries.argtypes = [i32, f64, P, i32, P, i32, P, i32, P, P, i64, P, P, i32]
    lib.oracle_bgemm_entries.restype = None
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = f64
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = f64
    lib.oracle_gelu_tanh.argtypes = [f64]
    lib.oracle_gelu_tanh.restype = f64
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = i32
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _as_f32(a):
    a = np.asarray(a)
    if a.dtype != np.float32:
        raise TypeError("expected float32 array, got %s" % a.dtype)
    return np.ascontiguousarray(a).ravel()


def _as_f16_bits(a):
    """numpy float16 or a uint16 / int16 array of 16-bit patterns (binary16 or bfloat16)."""
    a = np.asarray(a)
    if a.dtype == np.float16 or a.dtype == np.int16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("expected float16 (or 16-bit pattern) array, got %s" % a.dtype)
    return np.ascontiguousarray(a).ravel()


def _check_ld(rows, cols, ld, arr, name):
    if ld < max(1, cols):
        raise ValueError("%s: leading dimension %d < %d" % (name, ld, cols))
    need = 0 if rows == 0 or cols == 0 else (rows - 1) * ld + cols
    if arr is not None and arr.size < need:
        raise ValueError("%s: buffer of %d elements, need %d" % (name, arr.size, need))


class Oracle:
    """The oracle's entry points bound to one compiled library: the default one, or a
    variant built from an edited copy of the source (used by the tests to show that
    their pins catch planted mistakes)."""

    def __init__(self, lib=None):
        self._lib = lib

    @classmethod
    def from_source(cls, src: str, out: str) -> "Oracle":
        build(True, src, out)
        return cls(_bind(ctypes.CDLL(out)))

    @property
    def lib(self):
        if self._lib is None:
            if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SOURCE):
                build()
            self._lib = _bind(ctypes.CDLL(LIB_PATH))
        return self._lib

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    def sgemm(self, M, N, K, alpha, A, lda, B, ldb, beta, C0, ldc, *, with_den=True, threads=0):
        """(ref, den): packed M x N float64 arrays of alpha*A*B + beta*C0 and its error scale.

        A, B, C0 are float32 arrays read flat with the given leading dimensions.
        C0 is not read when beta == 0; A and B are not read when alpha == 0 or K == 0."""
        A = _as_f32(A)
        B = _as_f32(B)
        C0 = None if (beta == 0 or C0 is None) else _as_f32(C0)
        skip = alpha == 0 or K == 0
        _check_ld(M, K, lda, None if skip else A, "A")
        _check_ld(K, N, ldb, None if skip else B, "B")
        _check_ld(M, N, ldc, C0, "C")
        if beta != 0 and C0 is None:
            raise ValueError("beta != 0 needs C0")
        ref = np.empty((M, N), np.float64)
        den = np.empty((M, N), np.float64) if with_den else None
        self.lib.oracle_sgemm(M, N, K, float(alpha), _ptr(A), lda, _ptr(B), ldb, float(beta),
                              _ptr(C0), ldc, _ptr(ref), _ptr(den), int(threads))
        return ref, den

    def sgemm_entries(self, K, alpha, A, lda, B, ldb, beta, C0, ldc, rows, cols, *, threads=0):
        """(ref, den) of the entries (rows[t], cols[t]) of alpha*A*B + beta*C0."""
        A = _as_f32(A)
        B = _as_f32(B)
        C0 = None if (beta == 0 or C0 is None) else _as_f32(C0)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        if rows.shape != cols.shape:
            raise ValueError("rows and cols differ in shape")
        ref = np.empty(rows.size, np.float64)
        den = np.empty(rows.size, np.float64)
        self.lib.oracle_sgemm_entries(K, float(alpha), _ptr(A), lda, _ptr(B), ldb, float(beta),
                                      _ptr(C0), ldc, _ptr(rows), _ptr(cols), rows.size, _ptr(ref),
                                      _ptr(den), int(threads))
        return ref, den

    def hgemm_bias_act(self, M, N, K, alpha, A, lda, B, ldb, bias, act, *, with_den=True,
                       threads=0, fmt="f16"):
        """(ref, den) of act(alpha*A*B + bias) for 16-bit A, B (fmt "f16" = binary16,
        "bf16" = bfloat16 bit patterns) and an fp32 bias of length N."""
        A = _as_f16_bits(A)
        B = _as_f16_bits(B)
        bias = None if bias is None else _as_f32(bias)
        skip = alpha == 0 or K == 0
        _check_ld(M, K, lda, None if skip else A, "A")
        _check_ld(K, N, ldb, None if skip else B, "B")
        if bias is not None and bias.size < N:
            raise ValueError("bias shorter than N")
        ref = np.empty((M, N), np.float64)
        den = np.empty((M, N), np.float64) if with_den else None
        fn = {"f16": self.lib.oracle_hgemm_bias_act, "bf16": self.lib.oracle_bgemm_bias_act}[fmt]
        fn(M, N, K, float(alpha), _ptr(A), lda, _ptr(B), ldb, _ptr(bias), int(act), _ptr(ref),
           _ptr(den), int(threads))
        return ref, den

    def hgemm_entries(self, K, alpha, A, lda, B, ldb, bias, act, rows, cols, *, threads=0,
                      fmt="f16"):
        """(ref, den) of the entries (rows[t], cols[t]) of act(alpha*A*B + bias)."""
        A = _as_f16_bits(A)
        B = _as_f16_bits(B)
        bias = None if bias is None else _as_f32(bias)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        ref = np.empty(rows.size, np.float64)
        den = np.empty(rows.size, np.float64)
        fn = {"f16": self.lib.oracle_hgemm_entries, "bf16": self.lib.oracle_bgemm_entries}[fmt]
        fn(K, float(alpha), _ptr(A), lda, _ptr(B), ldb, _ptr(bias), int(act), _ptr(rows),
           _ptr(cols), rows.size, _ptr(ref), _ptr(den), int(threads))
        return ref, den

    def half_to_double(self, bits: int) -> float:
        return float(self.lib.oracle_half_to_double(int(bits) & 0xFFFF))

    def bf16_to_double(self, bits: int) -> float:
        return float(self.lib.oracle_bf16_to_double(int(bits) & 0xFFFF))

    def gelu_tanh(self, x: float) -> float:
        return float(self.lib.oracle_gelu_tanh(float(x)))


_default = Oracle()

max_threads = _default.max_threads
sgemm = _default.sgemm
sgemm_entries = _default.sgemm_entries
hgemm_bias_act = _default.hgemm_bias_act
hgemm_entries = _default.hgemm_entries
half_to_double = _default.half_to_double
bf16_to_double = _default.bf16_to_double
gelu_tanh = _default.gelu_tanh


# Half the spacing of the subnormal numbers of each 16-bit output format: the
# least error with which a value below the format's normal range can be stored.
OUTPUT_FLOOR = {"f16": 2.0 ** -25, "bf16": 2.0 ** -134}


def normalized_error(got, ref, den, out_floor=0.0):
    """Per-element max(|got - ref| - out_floor, 0) / den, the parity measure.

    out_floor is OUTPUT_FLOOR[fmt] for a 16-bit output: an entry whose exact value
    lies below the format's normal range cannot be stored closer than that, so
    only the error beyond it counts (0 for FP32).  Where den == 0 the entry must
    match within out_floor (error 0, else inf); a non-finite output gives inf.
    The maximum over all entries is compared with the tolerance of the precision
    under test."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.asarray(den, dtype=np.float64)
    diff = np.maximum(np.abs(got - ref) - out_floor, 0.0)
    pos = den > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.where(pos, diff / np.where(pos, den, 1.0), np.where(diff == 0, 0.0, np.inf))
    return np.where(np.isfinite(got), e, np.inf)
