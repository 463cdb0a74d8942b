"""Python binding of the MI355X GEMM library (libgemm.so, C ABI in include/gemm.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  Pointers may be given as integers (device
addresses) or as torch tensors (their ``data_ptr()`` is passed; no copy, no
dtype or layout conversion).  ``stream`` may be None (torch's current stream on
the current device), an integer ``hipStream_t`` or a ``torch.cuda.Stream``.

There is no fallback: if libgemm.so has not been built, or the device is not
gfx950, every call raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["GemmError", "gemm_create", "gemm_destroy", "sgemm", "sgemm_noalloc", "hgemm_bias_act",
           "bgemm_bias_act",
           "gemm_status_string", "gemm_debug_force_tile", "gemm_debug_force_splits",
           "gemm_debug_pick_config", "gemm_debug_use_tuned_table", "gemm_debug_force_swizzle",
           "gemm_debug_tile_map", "library_path",
           "load_library", "EXPORTED_SYMBOLS", "ACT_NONE", "ACT_GELU_TANH"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgemm.so")

STATUS_SUCCESS = 0
STATUS_NOT_INITIALIZED = 1
STATUS_INVALID_VALUE = 2
STATUS_ARCH_MISMATCH = 3
STATUS_HIP_ERROR = 4
STATUS_INTERNAL = 5

ACT_NONE = 0
ACT_GELU_TANH = 1

# Every symbol declared in include/gemm.h and include/gemm_debug.h.
EXPORTED_SYMBOLS = ("gemm_create", "gemm_destroy", "sgemm", "sgemm_noalloc", "hgemm_bias_act",
                    "bgemm_bias_act",
                    "gemm_status_string", "gemm_debug_force_tile", "gemm_debug_force_splits",
                    "gemm_debug_pick_config", "gemm_debug_use_tuned_table",
                    "gemm_debug_force_swizzle", "gemm_debug_tile_map")

_lib = None


class GemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: status %d (%s)" % (where, status, gemm_status_string(status)))


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libgemm.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libgemm.so is not built (run `python -m linear_algebra_sgemm_amd.build` "
                           "or __graft_entry__.build()); there is no non-HIP fallback")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.gemm_create.argtypes = []
    lib.gemm_create.restype = I
    lib.gemm_destroy.argtypes = []
    lib.gemm_destroy.restype = I
    lib.sgemm.argtypes = [I, I, I, F, P, I, P, I, F, P, I, P]
    lib.sgemm.restype = I
    lib.sgemm_noalloc.argtypes = [I, I, I, F, P, I, P, I, F, P, I, P]
    lib.sgemm_noalloc.restype = I
    lib.hgemm_bias_act.argtypes = [I, I, I, F, P, I, P, I, P, I, P, I, P]
    lib.hgemm_bias_act.restype = I
    lib.bgemm_bias_act.argtypes = [I, I, I, F, P, I, P, I, P, I, P, I, P]
    lib.bgemm_bias_act.restype = I
    lib.gemm_status_string.argtypes = [I]
    lib.gemm_status_string.restype = ctypes.c_char_p
    lib.gemm_debug_force_tile.argtypes = [I, I]
    lib.gemm_debug_force_tile.restype = I
    lib.gemm_debug_force_splits.argtypes = [I, I]
    lib.gemm_debug_force_splits.restype = I
    IP = ctypes.POINTER(ctypes.c_int)
    lib.gemm_debug_pick_config.argtypes = [I, I, I, I, I, IP, IP]
    lib.gemm_debug_pick_config.restype = I
    lib.gemm_debug_use_tuned_table.argtypes = [I]
    lib.gemm_debug_use_tuned_table.restype = I
    lib.gemm_debug_force_swizzle.argtypes = [I, I]
    lib.gemm_debug_force_swizzle.restype = I
    lib.gemm_debug_tile_map.argtypes = [I, I, I, I, P, P]
    lib.gemm_debug_tile_map.restype = I
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    raise TypeError("expected a device pointer (int) or a tensor, got %r" % type(x))


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    raise TypeError("expected None, an int hipStream_t or a torch.cuda.Stream")


def _check(status: int, where: str, raise_on_error: bool) -> int:
    if status != STATUS_SUCCESS and raise_on_error:
        raise GemmError(status, where)
    return status


def gemm_create(raise_on_error: bool = True) -> int:
    return _check(load_library().gemm_create(), "gemm_create", raise_on_error)


def gemm_destroy(raise_on_error: bool = True) -> int:
    return _check(load_library().gemm_destroy(), "gemm_destroy", raise_on_error)


def sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None, *, raise_on_error=True):
    """C = alpha * A x B + beta * C (FP32, row-major); see include/gemm.h."""
    st = load_library().sgemm(int(M), int(N), int(K), float(alpha), _ptr(A), int(lda), _ptr(B),
                              int(ldb), float(beta), _ptr(C), int(ldc), _stream(stream))
    return _check(st, "sgemm", raise_on_error)


def sgemm_noalloc(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None, *,
                  raise_on_error=True):
    """sgemm without device allocation on the call path; see include/gemm.h."""
    st = load_library().sgemm_noalloc(int(M), int(N), int(K), float(alpha), _ptr(A), int(lda),
                                      _ptr(B), int(ldb), float(beta), _ptr(C), int(ldc),
                                      _stream(stream))
    return _check(st, "sgemm_noalloc", raise_on_error)


def hgemm_bias_act(M, N, K, alpha, A, lda, B, ldb, bias, act, C, ldc, stream=None, *,
                   raise_on_error=True):
    """C = act(alpha * A x B + bias), fp16 A/B/C, fp32 bias and accumulation; see include/gemm.h."""
    st = load_library().hgemm_bias_act(int(M), int(N), int(K), float(alpha), _ptr(A), int(lda),
                                       _ptr(B), int(ldb), _ptr(bias), int(act), _ptr(C), int(ldc),
                                       _stream(stream))
    return _check(st, "hgemm_bias_act", raise_on_error)


def bgemm_bias_act(M, N, K, alpha, A, lda, B, ldb, bias, act, C, ldc, stream=None, *,
                   raise_on_error=True):
    """C = act(alpha * A x B + bias), bfloat16 A/B/C, fp32 bias and accumulation; see include/gemm.h."""
    st = load_library().bgemm_bias_act(int(M), int(N), int(K), float(alpha), _ptr(A), int(lda),
                                       _ptr(B), int(ldb), _ptr(bias), int(act), _ptr(C), int(ldc),
                                       _stream(stream))
    return _check(st, "bgemm_bias_act", raise_on_error)


def gemm_status_string(status: int) -> str:
    try:
        return load_library().gemm_status_string(int(status)).decode()
    except RuntimeError:
        return "status %d" % status


def gemm_debug_force_tile(op: int, tile: int) -> int:
    return load_library().gemm_debug_force_tile(int(op), int(tile))


def gemm_debug_force_splits(op: int, splits: int) -> int:
    return load_library().gemm_debug_force_splits(int(op), int(splits))


def gemm_debug_use_tuned_table(on: bool) -> int:
    return load_library().gemm_debug_use_tuned_table(1 if on else 0)


def gemm_debug_pick_config(op: int, M: int, N: int, K: int, cus: int):
    """(tile, splits) the library would run for this shape, or raise GemmError."""
    tile, splits = ctypes.c_int(-1), ctypes.c_int(-1)
    st = load_library().gemm_debug_pick_config(int(op), int(M), int(N), int(K), int(cus),
                                                ctypes.byref(tile), ctypes.byref(splits))
    _check(st, "gemm_debug_pick_config", True)
    return tile.value, splits.value


def gemm_debug_force_swizzle(group_m: int, xcd_remap: bool = True) -> int:
    """Tile order of later launches: group_m 0 = each launch's own; see include/gemm_debug.h."""
    return load_library().gemm_debug_force_swizzle(int(group_m), 1 if xcd_remap else 0)


def gemm_debug_tile_map(tiles_m: int, tiles_n: int, group_m: int, xcd_remap: bool = True):
    """(tile_m, tile_n) int arrays: the output tile of every workgroup of such a launch."""
    import numpy as np
    n = int(tiles_m) * int(tiles_n)
    tm = np.empty(max(n, 1), np.int32)
    tn = np.empty(max(n, 1), np.int32)
    st = load_library().gemm_debug_tile_map(int(tiles_m), int(tiles_n), int(group_m),
                                            1 if xcd_remap else 0, tm.ctypes.data, tn.ctypes.data)
    _check(st, "gemm_debug_tile_map", True)
    return tm[:n], tn[:n]
