"""The C-ABI library on the CPU: it loads, exports every declared symbol, and its
host-side argument checks answer without touching a GPU."""
import ctypes
import os
import re

import pytest

import linear_algebra_sgemm_amd as lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("gemm.h", "gemm_debug.h")]


def _declared_functions():
    names = []
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\([^;]*\)\s*;", text, flags=re.M)
    return names


@pytest.fixture(scope="module")
def so():
    if not os.path.exists(lib.library_path()):
        pytest.fail("libgemm.so is not built; run __graft_entry__.build() first")
    return lib.load_library()


def test_headers_declare_the_boundary():
    names = set(_declared_functions())
    assert {"gemm_create", "gemm_destroy", "sgemm", "hgemm_bias_act", "bgemm_bias_act",
            "gemm_status_string"} <= names
    assert names == set(lib.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(so):
    for name in _declared_functions():
        assert hasattr(so, name), name
        assert ctypes.cast(getattr(so, name), ctypes.c_void_p).value


def test_status_strings(so):
    for st in range(6):
        assert lib.gemm_status_string(st)
    assert "invalid" in lib.gemm_status_string(lib.STATUS_INVALID_VALUE)


BAD_SGEMM = [
    dict(M=-1), dict(N=-1), dict(K=-1),
    dict(lda=3),            # lda < K
    dict(ldb=4),            # ldb < N
    dict(ldc=4),            # ldc < N
    dict(C=None),
    dict(A=None), dict(B=None),
]


@pytest.mark.parametrize("bad", BAD_SGEMM, ids=lambda d: ",".join("%s=%s" % kv for kv in d.items()))
def test_sgemm_rejects_bad_arguments_without_gpu(so, bad):
    args = dict(M=8, N=5, K=4, alpha=1.0, A=0x1000, lda=4, B=0x2000, ldb=5, beta=0.0, C=0x3000,
                ldc=5)
    args.update(bad)
    st = lib.sgemm(args["M"], args["N"], args["K"], args["alpha"], args["A"], args["lda"],
                   args["B"], args["ldb"], args["beta"], args["C"], args["ldc"], stream=0,
                   raise_on_error=False)
    assert st == lib.STATUS_INVALID_VALUE


def test_sgemm_unread_operands_may_be_null(so):
    # alpha == 0: A and B are not read, so NULL is fine; the call then stops at the
    # missing gemm_create (no GPU here), not at argument validation.
    st = lib.sgemm(8, 5, 4, 0.0, None, 4, None, 5, 2.0, 0x3000, 5, stream=0, raise_on_error=False)
    assert st == lib.STATUS_NOT_INITIALIZED
    st = lib.sgemm(8, 5, 0, 1.0, None, 1, None, 5, 2.0, 0x3000, 5, stream=0, raise_on_error=False)
    assert st == lib.STATUS_NOT_INITIALIZED
    # M == 0: nothing is read or written.
    st = lib.sgemm(0, 5, 4, 1.0, None, 4, None, 5, 0.0, None, 5, stream=0, raise_on_error=False)
    assert st == lib.STATUS_NOT_INITIALIZED


def test_hgemm_rejects_bad_arguments_without_gpu(so):
    ok = dict(M=8, N=16, K=8, alpha=1.0, A=0x1000, lda=8, B=0x2000, ldb=16, bias=None, act=1,
              C=0x3000, ldc=16)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return lib.hgemm_bias_act(a["M"], a["N"], a["K"], a["alpha"], a["A"], a["lda"], a["B"],
                                  a["ldb"], a["bias"], a["act"], a["C"], a["ldc"], stream=0,
                                  raise_on_error=False)

    assert call(act=2) == lib.STATUS_INVALID_VALUE
    b = dict(ok)
    b["act"] = 7
    assert lib.bgemm_bias_act(b["M"], b["N"], b["K"], b["alpha"], b["A"], b["lda"], b["B"],
                              b["ldb"], b["bias"], b["act"], b["C"], b["ldc"], stream=0,
                              raise_on_error=False) == lib.STATUS_INVALID_VALUE
    b["act"] = 1
    assert lib.bgemm_bias_act(b["M"], b["N"], b["K"], b["alpha"], b["A"], b["lda"], b["B"],
                              b["ldb"], b["bias"], b["act"], b["C"], b["ldc"], stream=0,
                              raise_on_error=False) == lib.STATUS_NOT_INITIALIZED
    assert call(act=-1) == lib.STATUS_INVALID_VALUE
    assert call(lda=7) == lib.STATUS_INVALID_VALUE
    assert call(ldc=15) == lib.STATUS_INVALID_VALUE
    assert call(C=None) == lib.STATUS_INVALID_VALUE
    assert call(B=None) == lib.STATUS_INVALID_VALUE
    assert call() == lib.STATUS_NOT_INITIALIZED
    assert call(alpha=0.0, A=None, B=None) == lib.STATUS_NOT_INITIALIZED


def test_destroy_without_create(so):
    assert lib.gemm_destroy(raise_on_error=False) == lib.STATUS_NOT_INITIALIZED


def test_tile_choice(so):
    # largest tile when it still fills the device, smaller tiles for small outputs
    assert lib.gemm_debug_pick_tile(0, 4096, 4096, 256) == 4
    assert lib.gemm_debug_pick_tile(0, 8192, 8192, 256) == 4
    assert lib.gemm_debug_pick_tile(0, 256, 256, 256) == 2
    assert lib.gemm_debug_pick_tile(0, 1000, 3000, 256) == 2
    assert lib.gemm_debug_pick_tile(0, 2048, 2048, 256) == 2
    assert lib.gemm_debug_pick_tile(0, 4096, 4096, 64) == 4
    # the half product: whole 256-tiles take the direct-to-LDS kernel (3)
    assert lib.gemm_debug_pick_tile(1, 4096, 14336, 256) == 3
    assert lib.gemm_debug_pick_tile(1, 4096, 4000, 256) == 0
    assert lib.gemm_debug_pick_tile(1, 2048, 2000, 256) == 1
    assert lib.gemm_debug_pick_tile(1, 300, 500, 256) == 2
    assert lib.gemm_debug_pick_tile(2, 300, 500, 256) == -1
    assert lib.gemm_debug_force_tile(0, 5) == lib.STATUS_INVALID_VALUE
    assert lib.gemm_debug_force_tile(1, 5) == lib.STATUS_INVALID_VALUE
    assert lib.gemm_debug_force_tile(1, 3) == lib.STATUS_SUCCESS
    assert lib.gemm_debug_force_tile(1, -1) == lib.STATUS_SUCCESS
    assert lib.gemm_debug_force_tile(0, 4) == lib.STATUS_SUCCESS
    assert lib.gemm_debug_force_tile(5, 0) == lib.STATUS_INVALID_VALUE
    assert lib.gemm_debug_force_tile(0, -1) == lib.STATUS_SUCCESS
