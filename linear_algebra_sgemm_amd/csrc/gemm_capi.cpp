// C ABI of the GEMM library: argument validation, library state, quick
// returns and kernel dispatch.  Declared in include/gemm.h (compute calls) and
// include/gemm_debug.h (test hooks).
//
// The computation is C = alpha * A x B + beta * C of "SGEMM优化，从naive到
// warptiling" (section 问题与估算), whose kernels take (M, N, K, alpha, A, B,
// beta, C) (section k1); leading dimensions and a stream are added here.  The
// BLAS readings of the cases the pages do not discuss (beta == 0 leaves C
// unread, alpha == 0 or K == 0 leaves A and B unread, M or N == 0 is a no-op)
// are applied in this file, before any kernel is chosen.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/gemm.h"
#include "../../include/gemm_debug.h"
#include "gemm_launch.h"

namespace {

struct LibraryState {
  std::mutex mu;
  int refcount = 0;
  int device = -1;
  int cus = 256;
};

LibraryState g_state;
std::atomic<int> g_ready{0};
std::atomic<int> g_cus{256};
std::atomic<int> g_force_sgemm_tile{-1};
std::atomic<int> g_force_hgemm_tile{-1};

thread_local char t_last_error[256] = "";

int hip_failure(hipError_t e) {
  std::snprintf(t_last_error, sizeof(t_last_error), "HIP error %d: %s", (int)e,
                hipGetErrorString(e));
  return GEMM_STATUS_HIP_ERROR;
}

bool ld_ok(int ld, int cols) { return ld >= (cols > 1 ? cols : 1); }

}  // namespace

extern "C" {

int gemm_create(void) {
  std::lock_guard<std::mutex> lock(g_state.mu);
  if (g_state.refcount > 0) {
    ++g_state.refcount;
    return GEMM_STATUS_SUCCESS;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_failure(e);
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_failure(e);
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    std::snprintf(t_last_error, sizeof(t_last_error), "device %d is %s, not gfx950", dev,
                  prop.gcnArchName);
    return GEMM_STATUS_ARCH_MISMATCH;
  }
  g_state.device = dev;
  g_state.cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  g_cus.store(g_state.cus);
  g_state.refcount = 1;
  g_ready.store(1);
  return GEMM_STATUS_SUCCESS;
}

int gemm_destroy(void) {
  std::lock_guard<std::mutex> lock(g_state.mu);
  if (g_state.refcount <= 0) return GEMM_STATUS_NOT_INITIALIZED;
  if (--g_state.refcount == 0) {
    g_ready.store(0);
    g_state.device = -1;
  }
  return GEMM_STATUS_SUCCESS;
}

int sgemm(int M, int N, int K, float alpha, const float* A, int lda, const float* B, int ldb,
          float beta, float* C, int ldc, hipStream_t stream) {
  // 1. Arguments (no HIP call, nothing enqueued on failure).
  if (M < 0 || N < 0 || K < 0) return GEMM_STATUS_INVALID_VALUE;
  if (!ld_ok(lda, K) || !ld_ok(ldb, N) || !ld_ok(ldc, N)) return GEMM_STATUS_INVALID_VALUE;
  const bool empty = (M == 0 || N == 0);
  const bool reads_ab = !empty && K > 0 && alpha != 0.0f;
  if (!empty && C == nullptr) return GEMM_STATUS_INVALID_VALUE;
  if (reads_ab && (A == nullptr || B == nullptr)) return GEMM_STATUS_INVALID_VALUE;
  // 2. State.
  if (!g_ready.load()) return GEMM_STATUS_NOT_INITIALIZED;
  // 3. Quick returns.
  if (empty) return GEMM_STATUS_SUCCESS;
  hipError_t e;
  if (!reads_ab) {
    e = lasg::launch_sgemm_scale(M, N, beta, C, ldc, stream);
  } else {
    lasg::SgemmCall c{M, N, K, alpha, beta, A, lda, B, ldb, C, ldc};
    e = lasg::launch_sgemm(c, g_cus.load(), g_force_sgemm_tile.load(), stream);
  }
  return e == hipSuccess ? GEMM_STATUS_SUCCESS : hip_failure(e);
}

namespace {

int half_product(bool bf16, int M, int N, int K, float alpha, const uint16_t* A, int lda,
                 const uint16_t* B, int ldb, const float* bias, int act, uint16_t* C, int ldc,
                 hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0) return GEMM_STATUS_INVALID_VALUE;
  if (!ld_ok(lda, K) || !ld_ok(ldb, N) || !ld_ok(ldc, N)) return GEMM_STATUS_INVALID_VALUE;
  if (act != GEMM_ACT_NONE && act != GEMM_ACT_GELU_TANH) return GEMM_STATUS_INVALID_VALUE;
  const bool empty = (M == 0 || N == 0);
  const bool reads_ab = !empty && K > 0 && alpha != 0.0f;
  if (!empty && C == nullptr) return GEMM_STATUS_INVALID_VALUE;
  if (reads_ab && (A == nullptr || B == nullptr)) return GEMM_STATUS_INVALID_VALUE;
  if (!g_ready.load()) return GEMM_STATUS_NOT_INITIALIZED;
  if (empty) return GEMM_STATUS_SUCCESS;
  // alpha == 0 or K == 0: the product is zero and A, B stay unread; the kernel
  // skips its K loop and still applies bias and activation.
  lasg::HgemmCall c{M, N, reads_ab ? K : 0, alpha, A, lda, B, ldb, bias, act, C, ldc};
  const int force = g_force_hgemm_tile.load();
  hipError_t e = bf16 ? lasg::launch_bgemm(c, g_cus.load(), force, stream)
                      : lasg::launch_hgemm(c, g_cus.load(), force, stream);
  return e == hipSuccess ? GEMM_STATUS_SUCCESS : hip_failure(e);
}

}  // namespace

int hgemm_bias_act(int M, int N, int K, float alpha, const uint16_t* A, int lda,
                   const uint16_t* B, int ldb, const float* bias, int act, uint16_t* C, int ldc,
                   hipStream_t stream) {
  return half_product(false, M, N, K, alpha, A, lda, B, ldb, bias, act, C, ldc, stream);
}

int bgemm_bias_act(int M, int N, int K, float alpha, const uint16_t* A, int lda,
                   const uint16_t* B, int ldb, const float* bias, int act, uint16_t* C, int ldc,
                   hipStream_t stream) {
  return half_product(true, M, N, K, alpha, A, lda, B, ldb, bias, act, C, ldc, stream);
}

const char* gemm_status_string(int status) {
  switch (status) {
    case GEMM_STATUS_SUCCESS: return "success";
    case GEMM_STATUS_NOT_INITIALIZED: return "library not initialized (call gemm_create)";
    case GEMM_STATUS_INVALID_VALUE: return "invalid argument";
    case GEMM_STATUS_ARCH_MISMATCH:
      return t_last_error[0] ? t_last_error : "device is not gfx950";
    case GEMM_STATUS_HIP_ERROR: return t_last_error[0] ? t_last_error : "HIP error";
    case GEMM_STATUS_INTERNAL: return "internal error";
    default: return "unknown status";
  }
}

int gemm_debug_force_tile(int op, int tile) {
  const int count = op == 0 ? lasg::kSgemmTileCount : lasg::kHgemmTileCount;
  if (tile < -1 || tile >= count) return GEMM_STATUS_INVALID_VALUE;
  if (op == 0) {
    g_force_sgemm_tile.store(tile);
  } else if (op == 1) {
    g_force_hgemm_tile.store(tile);
  } else {
    return GEMM_STATUS_INVALID_VALUE;
  }
  return GEMM_STATUS_SUCCESS;
}

int gemm_debug_pick_tile(int op, int M, int N, int cus) {
  if (op == 0) return lasg::sgemm_pick_tile(M, N, cus);
  // half product: aligned operands assumed, K a multiple of 64
  if (op == 1) return lasg::hgemm_pick_tile(M, N, 64, cus, true);
  return -1;
}

}  // extern "C"
