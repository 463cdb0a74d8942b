"""The oracle against its pins, and the pins against planted mistakes (CPU only)."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.Oracle())


# Each mutation edits one spot of a private copy of oracle.c; the pins must notice.
MUTATIONS = {
    "drop_last_k_term": ("for (int k = 0; k < K; ++k) {\n          double a = (double)A",
                         "for (int k = 0; k < K - 1; ++k) {\n          double a = (double)A"),
    "beta_sign": ("cterm = beta * c;\n          cmag", "cterm = -beta * c;\n          cmag"),
    "transposed_B_index": ("const float *brow = B + (size_t)k * ldb;",
                           "const float *brow = B + (size_t)k;"),
    "alpha_dropped": ("double r = skip_product ? 0.0 : alpha * acc[j];",
                      "double r = skip_product ? 0.0 : acc[j];"),
    "beta_zero_reads_C": ("if (beta != 0.0) {\n          double c = (double)C0[(size_t)i * ldc + j];",
                          "if (1) {\n          double c = (double)C0[(size_t)i * ldc + j];"),
    "lda_ignored": ("double a = (double)A[(size_t)i * lda + k];",
                    "double a = (double)A[(size_t)i * K + k];"),
    "gelu_cubic_constant": ("0.044715 * x * x * x", "0.04715 * x * x * x"),
    "gelu_half_factor": ("return 0.5 * x * (1.0 + tanh(inner));", "return x * (1.0 + tanh(inner));"),
    "half_exponent_bias": ("v = ldexp((double)(frac + 1024), expo - 25);",
                           "v = ldexp((double)(frac + 1024), expo - 24);"),
    "half_subnormal_scale": ("v = ldexp((double)frac, -24);", "v = ldexp((double)frac, -25);"),
    "bf16_shift": ("uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;"),
    "hgemm_bias_row_index": ("double b = bias ? (double)bias[j] : 0.0;",
                             "double b = bias ? (double)bias[i % N] : 0.0;"),
    "half_ldb_ignored": ("dec(B[(size_t)k * ldb + j]);", "dec(B[(size_t)k * N + j]);"),
    "half_lda_ignored": ("double a = dec(A[(size_t)i * lda + k]);",
                         "double a = dec(A[(size_t)i * K + k]);"),
    "half_drop_last_k": ("for (int k = 0; k < K; ++k) {\n          double a = dec(",
                         "for (int k = 0; k < K - 1; ++k) {\n          double a = dec("),
    "half_B_row_stride": ("const double *brow = bdec + (size_t)k * N;",
                          "const double *brow = bdec + (size_t)k;"),
    "den_missing_beta": ("cmag = fabs(beta) * fabs(c);\n        }\n        ref[",
                         "cmag = 0.0;\n        }\n        ref["),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(oracle.SOURCE).read()
    old, new = MUTATIONS[name]
    assert src.count(old) >= 1, "mutation anchor %r not found in oracle.c" % name
    mutated = src.replace(old, new, 1)
    path = tmp_path / "oracle_mut.c"
    path.write_text(mutated)
    lib = tmp_path / "liboracle_mut.so"
    oracle.build(True, str(path), str(lib))
    # A mutant may crash (e.g. by reading a NULL C); run it in a child process, where a
    # crash also counts as caught.
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import ctypes, json, oracle; from tests import oracle_pins; "
            "o = oracle.Oracle(oracle._bind(ctypes.CDLL(%r))); "
            "print(json.dumps(oracle_pins.failing_pins(o)))" % str(lib))
    proc = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                          timeout=600, env=dict(os.environ, OMP_NUM_THREADS="2"))
    if proc.returncode != 0:
        return  # crashed: caught
    bad = json.loads(proc.stdout.strip().splitlines()[-1])
    assert bad, "no pin noticed the planted mistake %s" % name


def test_measure_counts_16_bit_output_rounding_only_below_the_normal_range():
    # binary16: the exact value 2^-26 cannot be stored; 0 is the nearest value the
    # format has, and its error 2^-26 lies within half the subnormal spacing.
    floor = oracle.OUTPUT_FLOOR["f16"]
    assert floor == 2.0 ** -25
    tiny_ref, tiny_den = np.array([2.0 ** -26]), np.array([2.0 ** -25])
    assert oracle.normalized_error([0.0], tiny_ref, tiny_den, floor)[0] == 0.0
    # without the floor the same entry reads 0.5: the measure alone would ask for
    # a value the format does not have
    assert oracle.normalized_error([0.0], tiny_ref, tiny_den)[0] == 0.5
    # an error beyond the floor still counts in full past it
    e = oracle.normalized_error([0.0], np.array([2.0 ** -20]), np.array([2.0 ** -20]), floor)[0]
    assert e == (2.0 ** -20 - 2.0 ** -25) / 2.0 ** -20
    # in the normal range the floor changes nothing measurable: a 1e-3 error of a
    # value of 1 reads 1e-3 to within 2^-25
    e = oracle.normalized_error([1.001], np.array([1.0]), np.array([1.0]), floor)[0]
    assert abs(e - 1e-3) < 1e-7
    # bfloat16 has the exponent range of binary32: its floor is far below any value
    # these products produce
    assert oracle.OUTPUT_FLOOR["bf16"] == 2.0 ** -134
    # den == 0: exact, or within the floor
    assert oracle.normalized_error([2.0 ** -26], np.array([0.0]), np.array([0.0]), floor)[0] == 0.0
    assert oracle.normalized_error([2.0 ** -24], np.array([0.0]), np.array([0.0]), floor)[0] == np.inf
