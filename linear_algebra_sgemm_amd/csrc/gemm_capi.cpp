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
#include "gemm_common.h"
#include "gemm_launch.h"

namespace {

struct LibraryState {
  std::mutex mu;
  int refcount = 0;
  int device = -1;
  int cus = 256;
};

// Workspace: FP32 split-K partials and the buffer for packed operand copies,
// allocated by gemm_create and shared by all calls.  Calls on different
// streams take turns: each call that uses them first waits for the event
// recorded after the previous one (when that ran on another stream), then
// records the event after its own kernels.
struct Workspace {
  std::mutex mu;
  float* ptr = nullptr;
  size_t floats = 0;
  void* pack = nullptr;
  size_t pack_bytes = 0;
  hipEvent_t done = nullptr;
  hipStream_t last = nullptr;
  bool used = false;
  bool multi = false;   // a second stream has used the workspace: record `done`
};

LibraryState g_state;
Workspace g_ws;
std::atomic<int> g_ready{0};
std::atomic<int> g_cus{256};
std::atomic<int> g_force_sgemm_tile{-1};
std::atomic<int> g_force_hgemm_tile{-1};
std::atomic<int> g_force_sgemm_splits{-1};
std::atomic<int> g_force_half_splits{-1};

thread_local char t_last_error[256] = "";

// Scratch of the entry point that allocates nothing (sgemm_noalloc): the FP32
// split-K partial sums of one call, at most kScratchFloats floats.
constexpr size_t kScratchFloats = size_t(4) << 20;   // 16 MiB
constexpr int kMaxDevices = 64;

}  // namespace

// One copy per GPU, held until the process ends.  In host code `scratch` only
// names the symbol: its device address, per device, comes from
// hipGetSymbolAddress (scratch_on_current_device) and is what kernels receive.
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {

std::atomic<float*> g_scratch_ptr[kMaxDevices];

int hip_failure(hipError_t e) {
  std::snprintf(t_last_error, sizeof(t_last_error), "HIP error %d: %s", (int)e,
                hipGetErrorString(e));
  return GEMM_STATUS_HIP_ERROR;
}

bool ld_ok(int ld, int cols) { return ld >= (cols > 1 ? cols : 1); }

// Device address of `scratch` on the current device, looked up once per device
// (by gemm_create, or by the first sgemm_noalloc call on another device).
int scratch_on_current_device(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_failure(e);
  if (dev < 0 || dev >= kMaxDevices) return GEMM_STATUS_INTERNAL;
  float* ptr = g_scratch_ptr[dev].load();
  if (ptr == nullptr) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_failure(e);
    ptr = static_cast<float*>(addr);
    g_scratch_ptr[dev].store(ptr);
  }
  *out = ptr;
  return GEMM_STATUS_SUCCESS;
}

// Runs `launch(ws, pack)` with the workspace, ordered after the previous
// workspace user when that ran on another stream.  While one stream has used
// the workspace, stream order alone keeps its users apart and no event is
// recorded (an event record between two kernels costs about 4 us of GPU time
// per call).  The first user on a second stream waits, once, for all work
// queued on the device (nothing recorded the earlier users' completion); from
// then on every user records `done` and a user on another stream than the last
// waits for it.  Calls made under stream capture never get here (they are
// planned without the workspace: see capturing()).
template <class F>
int with_workspace(hipStream_t stream, F launch) {
  std::lock_guard<std::mutex> wl(g_ws.mu);
  if (g_ws.ptr == nullptr || g_ws.pack == nullptr) return GEMM_STATUS_NOT_INITIALIZED;
  hipError_t e;
  if (g_ws.used && g_ws.last != stream) {
    if (!g_ws.multi) {
      e = hipDeviceSynchronize();
      if (e != hipSuccess) return hip_failure(e);
      g_ws.multi = true;
    } else {
      e = hipStreamWaitEvent(stream, g_ws.done, 0);
      if (e != hipSuccess) return hip_failure(e);
    }
  }
  e = launch(g_ws.ptr, g_ws.pack);
  if (e != hipSuccess) return hip_failure(e);
  if (g_ws.multi) {
    e = hipEventRecord(g_ws.done, stream);
    if (e != hipSuccess) return hip_failure(e);
  }
  g_ws.last = stream;
  g_ws.used = true;
  return GEMM_STATUS_SUCCESS;
}

// Whether `stream` is being captured into a graph.  A captured call may be
// replayed at any later time, unordered with the eager calls that share the
// workspace, so such calls are planned without it: no split-K and no operand
// copies (operands off 16-byte rows then take the bounds-checked kernels).
// Sets *status on a HIP failure.
bool capturing(hipStream_t stream, int* status) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  const hipError_t e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess) {
    *status = hip_failure(e);
    return false;
  }
  return cs != hipStreamCaptureStatusNone;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Operand packing.  The direct-to-LDS kernels copy 16-byte chunks, so they need
// rows of A and B on 16-byte boundaries and B readable in whole chunks up to N;
// the register-staged kernels read such rows with 16-byte loads too.  Where an
// operand falls short, it is copied once per call into the library's pack
// buffer, rows padded to a multiple of 16 bytes with zeros, and the product
// reads the copy.  The copy costs a kernel launch and moves 2 x its bytes through HBM; it
// is made only when it fits the buffer and is small next to the product:
// 2 M N K of at least 2^28 FLOP (a few microseconds of work, the order of a
// launch) and at least 64 FLOP per byte moved.
struct Packing {
  bool a = false, b = false;
  int lda = 0, ldb = 0;    // leading dimensions of the copies (elements)
  size_t b_offset = 0;     // byte offset of B's copy in the buffer
  // Padded copies (register-staged FP32 tiles on ragged shapes): A copied to
  // `rows_a` rows and B to `k` rows, both zero-filled past the product, so the
  // kernel loads without bounds checks over K' = `k`.
  bool padded = false;
  int rows_a = 0, k = 0;
};

bool plan_packing(int M, int N, int K, bool a_ok, bool b_ok, size_t elem, size_t cap_bytes,
                  Packing& pk) {
  const size_t chunk = 16 / elem;
  pk.a = !a_ok;
  pk.b = !b_ok;
  pk.lda = (int)round_up((size_t)K, chunk);
  pk.ldb = (int)round_up((size_t)N, chunk);
  const size_t a_bytes = pk.a ? round_up((size_t)M * pk.lda * elem, 256) : 0;
  const size_t b_bytes = pk.b ? (size_t)K * pk.ldb * elem : 0;
  pk.b_offset = a_bytes;
  const double flops = 2.0 * M * N * K;
  return a_bytes + b_bytes <= cap_bytes && flops >= (double)(1 << 28) &&
         flops >= 64.0 * 2.0 * (double)(a_bytes + b_bytes);
}

// Padded copies for a register-staged FP32 tile that would otherwise run its
// bounds-checked instantiation (M, N or K off the tile, or rows of A or B off
// 16-byte boundaries): A to ceil(M / BM) BM rows of K' = ceil(K / BK) BK
// columns, B to K' rows of ceil(N / BN) BN columns.  Extra zeros add exact
// zeros to every sum.  Same cost test as the plain copies, on the padded bytes.
bool plan_padding(int M, int N, int K, int tile, bool operands_aligned, size_t cap_bytes,
                  Packing& pk) {
  if (tile < 0 || (tile > 6 && tile != 12)) return false;   // the register-staged tiles
  const int bm = lasg::sgemm_tile_bm(tile), bn = lasg::sgemm_tile_bn(tile);
  const int bk = lasg::sgemm_tile_bk(tile);
  if (operands_aligned && M % bm == 0 && N % bn == 0 && K % bk == 0) return false;
  Packing q;
  q.a = q.b = q.padded = true;
  q.rows_a = (int)round_up((size_t)M, bm);
  q.k = (int)round_up((size_t)K, bk);
  q.lda = q.k;
  q.ldb = (int)round_up((size_t)N, bn);
  const size_t a_bytes = round_up((size_t)q.rows_a * q.lda * 4, 256);
  const size_t b_bytes = (size_t)q.k * q.ldb * 4;
  q.b_offset = a_bytes;
  const double flops = 2.0 * M * N * K;
  if (!(a_bytes + b_bytes <= cap_bytes && flops >= (double)(1 << 28) &&
        flops >= 64.0 * 2.0 * (double)(a_bytes + b_bytes)))
    return false;
  pk = q;
  return true;
}

// Makes the copies `pk` asks for (elements of `elem` bytes) in the pack buffer,
// in one launch, and points the operands (`a` / `lda`, `b` / `ldb`, holding the
// caller's on entry) at them.
hipError_t pack_operands(const Packing& pk, int M, int N, int K, int elem, void* pbuf,
                         hipStream_t s, const void*& a, int& lda, const void*& b, int& ldb) {
  lasg::PackJob jobs[2];
  int n = 0;
  if (pk.a) {
    lasg::PackJob& j = jobs[n++];
    j.src = a;
    j.rows = M;
    j.cols = K;
    j.lds = lda;
    j.dst = pbuf;
    j.dst_rows = pk.padded ? pk.rows_a : M;
    j.ldd = pk.lda;
  }
  if (pk.b) {
    lasg::PackJob& j = jobs[n++];
    j.src = b;
    j.rows = K;
    j.cols = N;
    j.lds = ldb;
    j.dst = static_cast<char*>(pbuf) + pk.b_offset;
    j.dst_rows = pk.padded ? pk.k : K;
    j.ldd = pk.ldb;
  }
  if (n == 0) return hipSuccess;
  const hipError_t e = lasg::launch_pack(jobs, n, elem, s);
  if (e != hipSuccess) return e;
  if (pk.a) {
    a = jobs[0].dst;
    lda = pk.lda;
  }
  if (pk.b) {
    b = jobs[n - 1].dst;
    ldb = pk.ldb;
  }
  return hipSuccess;
}

// Operand conditions of the FP32 product.  A's rows on 16-byte boundaries (the
// register-staged tiles' 16-byte loads); A's rows on 4-byte boundaries with
// 32-bit copy offsets (the direct-to-LDS tiles, which copy A 4 bytes at a time
// where its rows are not 16-byte aligned); B's rows 16-byte aligned and
// readable in whole 4-float chunks, 32-bit copy offsets.
bool sgemm_a_rows16(const void* A, int lda) { return lda % 4 == 0 && aligned16(A); }
bool sgemm_a_ok(const void* A, int lda) {
  return (reinterpret_cast<uintptr_t>(A) & 3u) == 0 &&
         (int64_t)lda * 256 * 4 < (int64_t(1) << 31);
}
bool sgemm_b_ok(const void* B, int ldb, int N) {
  return ldb % 4 == 0 && N % 4 == 0 && aligned16(B) && (int64_t)ldb * 16 * 4 < (int64_t(1) << 31);
}
// The same for the half products (8-half chunks).
bool half_a_ok(const void* A, int lda) {
  return lda % 8 == 0 && aligned16(A) && (int64_t)lda * 256 * 2 < (int64_t(1) << 31);
}
bool half_b_ok(const void* B, int ldb, int N) {
  return ldb % 8 == 0 && N % 8 == 0 && aligned16(B) && (int64_t)ldb * 32 * 2 < (int64_t(1) << 31);
}

// The inputs a decision depends on; each thread keeps its last decision per
// product, so a loop of equal calls plans once (about half a microsecond of
// host time per call otherwise).
struct DecisionKey {
  int M, N, K, cus, ft, fs;
  bool a16, a_ok, b_ok, tuned;
  size_t ws_floats, pack_bytes;
  bool operator==(const DecisionKey& o) const {
    return M == o.M && N == o.N && K == o.K && cus == o.cus && ft == o.ft && fs == o.fs &&
           a16 == o.a16 && a_ok == o.a_ok && b_ok == o.b_ok && tuned == o.tuned &&
           ws_floats == o.ws_floats && pack_bytes == o.pack_bytes;
  }
};
template <class Plan>
struct Decision {
  bool valid = false;
  DecisionKey key{};
  Plan plan{};
  Packing pk;
  bool pack = false;
};
thread_local Decision<lasg::SgemmPlan> t_last_sgemm;
thread_local Decision<lasg::HalfPlan> t_last_half;

// The FP32 plan, and whether (and how) operands are packed for it: `a16`,
// `a_ok`, `b_ok` as above.
lasg::SgemmPlan decide_sgemm(int M, int N, int K, bool a16, bool a_ok, bool b_ok, int cus,
                             size_t ws_floats, size_t pack_bytes, Packing& pk, bool& pack) {
  const int ft = g_force_sgemm_tile.load(), fs = g_force_sgemm_splits.load();
  const DecisionKey key{M, N, K, cus, ft, fs, a16, a_ok, b_ok, lasg::use_tuned(), ws_floats,
                        pack_bytes};
  Decision<lasg::SgemmPlan>& last = t_last_sgemm;
  if (last.valid && last.key == key) {
    pk = last.pk;
    pack = last.pack;
    return last.plan;
  }
  pack = !(a_ok && b_ok) && plan_packing(M, N, K, a_ok, b_ok, 4, pack_bytes, pk);
  const lasg::SgemmPlan plan =
      lasg::plan_sgemm(M, N, K, cus, ft, fs, ws_floats, pack || (a_ok && b_ok));
  if (plan_padding(M, N, K, plan.tile, a16 && b_ok, pack_bytes, pk)) pack = true;
  last.valid = true;
  last.key = key;
  last.plan = plan;
  last.pk = pk;
  last.pack = pack;
  return plan;
}

lasg::HalfPlan decide_half(int M, int N, int K, bool a_ok, bool b_ok, int cus, size_t ws_floats,
                           size_t pack_bytes, Packing& pk, bool& pack) {
  const int ft = g_force_hgemm_tile.load(), fs = g_force_half_splits.load();
  const DecisionKey key{M, N, K, cus, ft, fs, false, a_ok, b_ok, lasg::use_tuned(), ws_floats,
                        pack_bytes};
  Decision<lasg::HalfPlan>& last = t_last_half;
  if (last.valid && last.key == key) {
    pk = last.pk;
    pack = last.pack;
    return last.plan;
  }
  pack = K > 0 && !(a_ok && b_ok) && plan_packing(M, N, K, a_ok, b_ok, 2, pack_bytes, pk);
  const lasg::HalfPlan plan =
      lasg::plan_half(M, N, K, cus, ft, fs, ws_floats, pack || (a_ok && b_ok));
  last.valid = true;
  last.key = key;
  last.plan = plan;
  last.pk = pk;
  last.pack = pack;
  return plan;
}

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
  {
    std::lock_guard<std::mutex> wl(g_ws.mu);
    void* ptr = nullptr;
    e = hipMalloc(&ptr, lasg::kWorkspaceBytes);
    if (e != hipSuccess) return hip_failure(e);
    void* pack = nullptr;
    e = hipMalloc(&pack, lasg::kPackBytes);
    if (e != hipSuccess) {
      (void)hipFree(ptr);
      return hip_failure(e);
    }
    hipEvent_t ev = nullptr;
    // The event orders workspace users on streams of this device only: no timing
    // and no system-scope fence (that fence writes back and invalidates the
    // caches at every record, about 5 us of GPU time per call).
    e = hipEventCreateWithFlags(&ev, hipEventDisableTiming | hipEventDisableSystemFence);
    if (e != hipSuccess) {
      (void)hipFree(ptr);
      (void)hipFree(pack);
      return hip_failure(e);
    }
    g_ws.ptr = static_cast<float*>(ptr);
    g_ws.floats = lasg::kWorkspaceBytes / sizeof(float);
    g_ws.pack = pack;
    g_ws.pack_bytes = lasg::kPackBytes;
    g_ws.done = ev;
    g_ws.last = nullptr;
    g_ws.used = false;
    g_ws.multi = false;
  }
  {
    float* sp = nullptr;
    const int st = scratch_on_current_device(&sp);
    if (st != GEMM_STATUS_SUCCESS) {
      std::lock_guard<std::mutex> wl(g_ws.mu);
      (void)hipEventDestroy(g_ws.done);
      (void)hipFree(g_ws.ptr);
      (void)hipFree(g_ws.pack);
      g_ws.ptr = nullptr;
      g_ws.pack = nullptr;
      g_ws.done = nullptr;
      return st;
    }
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
    std::lock_guard<std::mutex> wl(g_ws.mu);
    // Work still queued may use the workspace: let the device finish first.
    hipError_t e = hipDeviceSynchronize();
    if (g_ws.done) (void)hipEventDestroy(g_ws.done);
    if (g_ws.ptr) (void)hipFree(g_ws.ptr);
    if (g_ws.pack) (void)hipFree(g_ws.pack);
    g_ws.ptr = nullptr;
    g_ws.floats = 0;
    g_ws.pack = nullptr;
    g_ws.pack_bytes = 0;
    g_ws.done = nullptr;
    g_ws.used = false;
    g_ws.multi = false;
    if (e != hipSuccess) return hip_failure(e);
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
    Packing pk;
    bool pack = false;
    const bool a16 = sgemm_a_rows16(A, lda), a_ok = sgemm_a_ok(A, lda);
    const bool b_ok = sgemm_b_ok(B, ldb, N);
    lasg::SgemmPlan plan = decide_sgemm(M, N, K, a16, a_ok, b_ok, g_cus.load(), g_ws.floats,
                                        g_ws.pack_bytes, pk, pack);
    if (plan.splits > 1 || pack) {
      int st = GEMM_STATUS_SUCCESS;
      if (capturing(stream, &st)) {
        pk = Packing();
        plan = decide_sgemm(M, N, K, a16, a_ok, b_ok, g_cus.load(), 0, 0, pk, pack);
      }
      if (st != GEMM_STATUS_SUCCESS) return st;
    }
    if (plan.splits > 1 || pack) {
      return with_workspace(stream, [&](float* ws, void* pbuf) {
        lasg::SgemmCall cc = c;
        if (pack) {
          const void *a = A, *b = B;
          const hipError_t pe = pack_operands(pk, M, N, K, 4, pbuf, stream, a, cc.lda, b, cc.ldb);
          if (pe != hipSuccess) return pe;
          cc.A = static_cast<const float*>(a);
          cc.B = static_cast<const float*>(b);
          if (pk.b) cc.nb = pk.ldb;
          if (pk.padded) {
            cc.K = pk.k;
            cc.padded = true;
          }
        }
        return lasg::launch_sgemm(cc, plan, ws, stream);
      });
    } else {
      e = lasg::launch_sgemm(c, plan, nullptr, stream);
    }
  }
  return e == hipSuccess ? GEMM_STATUS_SUCCESS : hip_failure(e);
}

int sgemm_noalloc(int M, int N, int K, float alpha, const float* A, int lda, const float* B,
                  int ldb, float beta, float* C, int ldc, hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0) return GEMM_STATUS_INVALID_VALUE;
  if (!ld_ok(lda, K) || !ld_ok(ldb, N) || !ld_ok(ldc, N)) return GEMM_STATUS_INVALID_VALUE;
  const bool empty = (M == 0 || N == 0);
  const bool reads_ab = !empty && K > 0 && alpha != 0.0f;
  if (!empty && C == nullptr) return GEMM_STATUS_INVALID_VALUE;
  if (reads_ab && (A == nullptr || B == nullptr)) return GEMM_STATUS_INVALID_VALUE;
  if (!g_ready.load()) return GEMM_STATUS_NOT_INITIALIZED;
  if (empty) return GEMM_STATUS_SUCCESS;
  hipError_t e;
  if (!reads_ab) {
    e = lasg::launch_sgemm_scale(M, N, beta, C, ldc, stream);
  } else {
    float* ws = nullptr;
    const int st = scratch_on_current_device(&ws);
    if (st != GEMM_STATUS_SUCCESS) return st;
    // Planned with the static scratch as the split-K workspace and no pack
    // buffer: split counts are clamped so that splits * M * N fits, and
    // operands off 16-byte rows take the bounds-checked kernels.
    Packing pk;
    bool pack = false;
    const lasg::SgemmPlan plan =
        decide_sgemm(M, N, K, sgemm_a_rows16(A, lda), sgemm_a_ok(A, lda), sgemm_b_ok(B, ldb, N),
                     g_cus.load(), kScratchFloats, 0, pk, pack);
    if (pack || (plan.splits > 1 && (size_t)plan.splits * M * N > kScratchFloats))
      return GEMM_STATUS_INVALID_VALUE;   // beyond the scratch (the plan never asks for it)
    lasg::SgemmCall c{M, N, K, alpha, beta, A, lda, B, ldb, C, ldc};
    e = lasg::launch_sgemm(c, plan, ws, stream);
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
  const int cus = g_cus.load();
  Packing pk;
  bool pack = false;
  const bool a_ok = half_a_ok(A, lda), b_ok = half_b_ok(B, ldb, N);
  lasg::HalfPlan plan = decide_half(M, N, c.K, a_ok, b_ok, cus, g_ws.floats, g_ws.pack_bytes, pk,
                                    pack);
  if (plan.splits > 1 || pack) {
    int st = GEMM_STATUS_SUCCESS;
    if (capturing(stream, &st)) {
      pk = Packing();
      plan = decide_half(M, N, c.K, a_ok, b_ok, cus, 0, 0, pk, pack);
    }
    if (st != GEMM_STATUS_SUCCESS) return st;
  }
  auto launch = [&](float* ws, void* pbuf) {
    lasg::HgemmCall cc = c;
    if (pack) {
      const void *a = A, *b = B;
      const hipError_t pe = pack_operands(pk, M, N, K, 2, pbuf, stream, a, cc.lda, b, cc.ldb);
      if (pe != hipSuccess) return pe;
      cc.A = static_cast<const uint16_t*>(a);
      cc.B = static_cast<const uint16_t*>(b);
      if (pk.b) cc.nb = pk.ldb;
    }
    return bf16 ? lasg::launch_bgemm(cc, plan, cus, ws, stream)
                : lasg::launch_hgemm(cc, plan, cus, ws, stream);
  };
  if (plan.splits > 1 || pack) return with_workspace(stream, launch);
  const hipError_t e = launch(nullptr, nullptr);
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
  if (op != 0 && op != 1) return GEMM_STATUS_INVALID_VALUE;
  const int count = op == 0 ? lasg::kSgemmTileCount : lasg::kHgemmTileCount;
  if (tile < -1 || tile >= count) return GEMM_STATUS_INVALID_VALUE;
  (op == 0 ? g_force_sgemm_tile : g_force_hgemm_tile).store(tile);
  return GEMM_STATUS_SUCCESS;
}

int gemm_debug_force_splits(int op, int splits) {
  if (op != 0 && op != 1) return GEMM_STATUS_INVALID_VALUE;
  if (splits != -1 && (splits < 1 || splits > lasg::kMaxSplits)) return GEMM_STATUS_INVALID_VALUE;
  (op == 0 ? g_force_sgemm_splits : g_force_half_splits).store(splits);
  return GEMM_STATUS_SUCCESS;
}

int gemm_debug_use_tuned_table(int on) {
  if (on != 0 && on != 1) return GEMM_STATUS_INVALID_VALUE;
  lasg::set_use_tuned(on == 1);
  return GEMM_STATUS_SUCCESS;
}

int gemm_debug_force_swizzle(int group_m, int xcd_remap) {
  if (group_m < 0 || group_m > 64 || (xcd_remap != 0 && xcd_remap != 1))
    return GEMM_STATUS_INVALID_VALUE;
  lasg::set_swizzle(group_m, xcd_remap == 1);
  return GEMM_STATUS_SUCCESS;
}

int gemm_debug_tile_map(int tiles_m, int tiles_n, int group_m, int xcd_remap, int* tile_m,
                        int* tile_n) {
  if (tiles_m <= 0 || tiles_n <= 0 || group_m <= 0 || (xcd_remap != 0 && xcd_remap != 1) ||
      tile_m == nullptr || tile_n == nullptr || (int64_t)tiles_m * tiles_n > (1 << 24))
    return GEMM_STATUS_INVALID_VALUE;
  const int g = xcd_remap ? group_m : -group_m;
  for (int wg = 0; wg < tiles_m * tiles_n; ++wg)
    lasg::tile_of_workgroup(wg, tiles_m, tiles_n, g, tile_m[wg], tile_n[wg]);
  return GEMM_STATUS_SUCCESS;
}

int gemm_debug_pick_config(int op, int M, int N, int K, int cus, int* tile, int* splits) {
  if (M < 0 || N < 0 || K < 0 || cus <= 0 || tile == nullptr || splits == nullptr)
    return GEMM_STATUS_INVALID_VALUE;
  if (op == 0) {
    // Packed operands (lda = K, ldb = N) on 16-byte-aligned bases.
    Packing pk;
    bool pack = false;
    const lasg::SgemmPlan p =
        decide_sgemm(M, N, K, K % 4 == 0, (int64_t)K * 256 * 4 < (int64_t(1) << 31), N % 4 == 0,
                     cus, lasg::kWorkspaceBytes / sizeof(float), lasg::kPackBytes, pk, pack);
    *tile = p.tile;
    *splits = p.splits;
    return GEMM_STATUS_SUCCESS;
  }
  if (op == 1) {
    Packing pk;
    bool pack = false;
    const lasg::HalfPlan p =
        decide_half(M, N, K, K % 8 == 0, N % 8 == 0, cus, lasg::kWorkspaceBytes / sizeof(float),
                    lasg::kPackBytes, pk, pack);
    *tile = p.tile;
    *splits = p.splits;
    return GEMM_STATUS_SUCCESS;
  }
  return GEMM_STATUS_INVALID_VALUE;
}

}  // extern "C"
