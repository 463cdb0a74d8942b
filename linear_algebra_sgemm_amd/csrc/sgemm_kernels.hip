// FP32 GEMM kernels for gfx950: C = alpha * A x B + beta * C, row-major.
//
// The problem is the one of "SGEMM优化，从naive到warptiling" (section 问题与估算).
// The hierarchy follows the same pages' tiling ideas, mapped onto CDNA4:
//  * a workgroup owns a BM x BN output tile (shared-memory block tiling,
//    SGEMM page section k3, Tiled-GEMM chapter 11.2);
//  * each of its waves owns a WTM x WTN sub-tile made of 32x32 blocks computed
//    by v_mfma_f32_32x32x2_f32 into accumulator registers that never leave the
//    register file during the K loop (the warptiling station k10 of the SGEMM
//    page; the register-resident accumulators of the DeepGEMM page, 4.3);
//  * A and B tiles are staged global -> registers -> LDS with 16-byte loads and
//    double-buffered LDS, one barrier per K tile (lecture 24, sections 4.1 and
//    4.3; Tiled-GEMM 11.4);
//  * LDS rows are padded so the 16-byte fragment reads and the B row reads are
//    free of bank conflicts (Tiled-GEMM 11.5; lecture 24, 4.2);
//  * ragged M, N, K and unaligned leading dimensions are handled by zero-filling
//    out-of-range loads and predicating stores (Tiled-GEMM 11.3);
//  * shapes with too few output tiles to occupy the GPU split K over several
//    workgroups per tile (the split-K of lecture 24, section 8.3, exercise 2,
//    and of the DeepGEMM page, section 5.3).  Those pages merge the partials
//    with atomic adds; here each workgroup writes its FP32 partial to a
//    workspace and a second kernel adds the partials in a fixed order and
//    applies alpha and beta, so results do not change from run to run.
//
// The MFMA consumes, per lane, one A value (row l % 32, k-slot l / 32) and one
// B value (column l % 32, k-slot l / 32).  Which physical k feeds which k-slot
// is our choice as long as A and B agree, because the sum over k is the same
// set of products.  Within each group of 8 k values of a tile, MFMA step s
// (0..3) gives k-slot h the index 4h + s; a lane then finds its four A values
// for steps 0..3 side by side in an LDS row and reads them with one 16-byte
// load.
#include "gemm_common.h"
#include "gemm_launch.h"

namespace lasg {

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int WAVES_PER_SIMD_ = 1>
struct SgemmTile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  // Waves of this kernel that must fit on one SIMD at once (register budget:
  // 512 / WAVES_PER_SIMD registers per lane, accumulators included).
  static constexpr int WAVES_PER_SIMD = WAVES_PER_SIMD_;
  static constexpr int THREADS = WAVES_M * WAVES_N * kWave;
  static constexpr int WTM = BM / WAVES_M;     // wave sub-tile rows
  static constexpr int WTN = BN / WAVES_N;     // wave sub-tile columns
  static constexpr int FM = WTM / 32;          // 32x32 MFMA blocks per wave, along M
  static constexpr int FN = WTN / 32;          // ... along N
  static constexpr int A_STRIDE = BK + 4;      // floats per LDS row of the A tile (one row = one m)
  static constexpr int B_STRIDE = BN + 8;      // floats per LDS row of the B tile (one row = one k)
  static constexpr int A_STAGE = BM * A_STRIDE;
  static constexpr int B_STAGE = BK * B_STRIDE;
  static constexpr int LDS_FLOATS = 2 * (A_STAGE + B_STAGE);
  static constexpr int A_VECS = BM * BK / 4 / THREADS;   // float4 loads per thread per K tile
  static constexpr int B_VECS = BK * BN / 4 / THREADS;

  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 MFMA blocks");
  static_assert(BK % 8 == 0, "K tile is consumed in groups of 8");
  static_assert((BM * BK / 4) % THREADS == 0, "A tile must split evenly into float4 loads");
  static_assert((BK * BN / 4) % THREADS == 0, "B tile must split evenly into float4 loads");
  static_assert(THREADS % (BK / 4) == 0 && THREADS % (BN / 4) == 0, "load rows must not wrap");
  static_assert(LDS_FLOATS * 4 <= 160 * 1024, "two stages must fit gfx950's 160 KiB of LDS");
  static_assert(FM * FN * 16 <= 256 / WAVES_PER_SIMD, "accumulators must leave room for operands");
};

struct SgemmArgs {
  int M, N, K;
  float alpha, beta;
  const float* A;
  int lda;
  const float* B;
  int ldb;
  float* C;
  int ldc;
  int tiles_m, tiles_n, group_m;
  // Split-K: workgroup row blockIdx.y covers K range [y * k_chunk, min(K, (y + 1) * k_chunk))
  // and writes its raw partial to ws + y * M * N (M x N, row stride N).
  int k_chunk;
  float* ws;
};

// Global -> register staging of one K tile.  EDGE selects bounds-checked scalar
// loads (zero outside the matrix, any alignment); otherwise 16-byte loads with
// no checks, valid when the tile lies inside the matrix and rows are 16-byte aligned.
template <class T, bool EDGE>
struct Stage {
  f32x4 a[T::A_VECS];
  f32x4 b[T::B_VECS];

  __device__ __forceinline__ void load(const SgemmArgs& p, int m0, int n0, int k0, int tid) {
#pragma unroll
    for (int v = 0; v < T::A_VECS; ++v) {
      const int c = tid + v * T::THREADS;
      const int row = c / (T::BK / 4);
      const int kc = (c % (T::BK / 4)) * 4;
      const int gm = m0 + row;
      const int gk = k0 + kc;
      if constexpr (!EDGE) {
        a[v] = *reinterpret_cast<const f32x4*>(p.A + (size_t)gm * p.lda + gk);
      } else {
        const float* src = p.A + (size_t)gm * p.lda;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          a[v][e] = (gm < p.M && gk + e < p.K) ? src[gk + e] : 0.0f;
      }
    }
#pragma unroll
    for (int v = 0; v < T::B_VECS; ++v) {
      const int c = tid + v * T::THREADS;
      const int row = c / (T::BN / 4);
      const int nc = (c % (T::BN / 4)) * 4;
      const int gk = k0 + row;
      const int gn = n0 + nc;
      if constexpr (!EDGE) {
        b[v] = *reinterpret_cast<const f32x4*>(p.B + (size_t)gk * p.ldb + gn);
      } else {
        const float* src = p.B + (size_t)gk * p.ldb;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          b[v][e] = (gk < p.K && gn + e < p.N) ? src[gn + e] : 0.0f;
      }
    }
  }

  __device__ __forceinline__ void store(float* As, float* Bs, int tid) const {
#pragma unroll
    for (int v = 0; v < T::A_VECS; ++v) {
      const int c = tid + v * T::THREADS;
      const int row = c / (T::BK / 4);
      const int kc = (c % (T::BK / 4)) * 4;
      *reinterpret_cast<f32x4*>(As + row * T::A_STRIDE + kc) = a[v];
    }
#pragma unroll
    for (int v = 0; v < T::B_VECS; ++v) {
      const int c = tid + v * T::THREADS;
      const int row = c / (T::BN / 4);
      const int nc = (c % (T::BN / 4)) * 4;
      *reinterpret_cast<f32x4*>(Bs + row * T::B_STRIDE + nc) = b[v];
    }
  }
};

template <class T, bool EDGE, bool SPLIT>
__global__ void __launch_bounds__(T::THREADS) __attribute__((amdgpu_waves_per_eu(T::WAVES_PER_SIMD)))
sgemm_mfma_kernel(SgemmArgs p) {
  if constexpr (SPLIT) {
    // This workgroup's K chunk: shift A and B to its start and shorten K.  The
    // chunk length is a multiple of BK, so the fast path's alignment holds.
    const int kbeg = blockIdx.y * p.k_chunk;
    const int klen = p.K - kbeg < p.k_chunk ? p.K - kbeg : p.k_chunk;
    p.A += kbeg;
    p.B += (size_t)kbeg * p.ldb;
    p.K = klen;
  }
  __shared__ __attribute__((aligned(16))) float lds[T::LDS_FLOATS];
  float* const As0 = lds;
  float* const Bs0 = lds + T::A_STAGE;
  float* const As1 = lds + T::A_STAGE + T::B_STAGE;
  float* const Bs1 = As1 + T::A_STAGE;

  int tile_m, tile_n;
  tile_of_workgroup(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tile_m, tile_n);
  const int m0 = tile_m * T::BM;
  const int n0 = tile_n * T::BN;

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int wm = wave / T::WAVES_N;
  const int wn = wave % T::WAVES_N;
  const int l32 = lane % 32;
  const int half = lane / 32;

  f32x16 acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int ktiles = (p.K + T::BK - 1) / T::BK;
  Stage<T, EDGE> st;
  if (ktiles > 0) {
    st.load(p, m0, n0, 0, tid);
    st.store(As0, Bs0, tid);
  }
  __syncthreads();

  // Per-lane fragment origins inside one LDS stage.
  const int a_off = (wm * T::WTM + l32) * T::A_STRIDE + 4 * half;
  const int b_off = (4 * half) * T::B_STRIDE + wn * T::WTN + l32;

  for (int kt = 0; kt < ktiles; ++kt) {
    const bool odd = kt & 1;
    const float* As = odd ? As1 : As0;
    const float* Bs = odd ? Bs1 : Bs0;
    const bool more = kt + 1 < ktiles;
    if (more) st.load(p, m0, n0, (kt + 1) * T::BK, tid);

#pragma unroll
    for (int g = 0; g < T::BK / 8; ++g) {
      f32x4 af[T::FM];
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
        af[i] = *reinterpret_cast<const f32x4*>(As + a_off + i * 32 * T::A_STRIDE + 8 * g);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float bf[T::FN];
#pragma unroll
        for (int j = 0; j < T::FN; ++j) bf[j] = Bs[b_off + (8 * g + s) * T::B_STRIDE + j * 32];
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
#pragma unroll
          for (int j = 0; j < T::FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][s], bf[j], acc[i][j], 0, 0, 0);
      }
    }

    if (more) st.store(odd ? As0 : As1, odd ? Bs0 : Bs1, tid);
    __syncthreads();
  }

  if constexpr (SPLIT) {
    // Raw partial sums into this K chunk's slice of the workspace.
    float* W = p.ws + (size_t)blockIdx.y * p.M * p.N;
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
        const int col = n0 + wn * T::WTN + j * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * T::WTM + i * 32 + mfma32_row(r, lane);
          if (EDGE && (row >= p.M || col >= p.N)) continue;
          W[(size_t)row * p.N + col] = acc[i][j][r];
        }
      }
    return;
  }

  // Epilogue: C = alpha * acc + beta * C, C read only when beta != 0.  For each
  // row of blocks, all C loads are issued before the first one is consumed, so
  // their latencies overlap instead of adding up.
  const float alpha = p.alpha, beta = p.beta;
  const bool read_c = beta != 0.0f;
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
    float cv[T::FN][16];
    if (read_c) {
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
        const int col = n0 + wn * T::WTN + j * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * T::WTM + i * 32 + mfma32_row(r, lane);
          const bool ok = !EDGE || (row < p.M && col < p.N);
          cv[j][r] = ok ? p.C[(size_t)row * p.ldc + col] : 0.0f;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
      const int col = n0 + wn * T::WTN + j * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * T::WTM + i * 32 + mfma32_row(r, lane);
        if (EDGE && (row >= p.M || col >= p.N)) continue;
        const float v = alpha * acc[i][j][r];
        p.C[(size_t)row * p.ldc + col] = read_c ? __builtin_fmaf(beta, cv[j][r], v) : v;
      }
    }
  }
}

// C = beta * C (C = 0 when beta == 0, without reading C): the alpha == 0 / K == 0 case.
__global__ void __launch_bounds__(256) sgemm_scale_kernel(int M, int N, float beta, float* C,
                                                           int ldc) {
  const int64_t total = (int64_t)M * N;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = t / N, j = t % N;
    float* dst = C + i * ldc + j;
    *dst = (beta != 0.0f) ? beta * *dst : 0.0f;
  }
}

// Second half of split-K: C = alpha * (sum of the `splits` partials, added in
// order 0, 1, ...) + beta * C, C read only when beta != 0.
__global__ void __launch_bounds__(256) sgemm_splitk_reduce_kernel(int M, int N, int splits,
                                                                  const float* ws, float alpha,
                                                                  float beta, float* C, int ldc) {
  const int64_t total = (int64_t)M * N;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    float sum = ws[t];
    for (int q = 1; q < splits; ++q) sum += ws[q * total + t];
    const int64_t i = t / N, j = t % N;
    float* dst = C + i * ldc + j;
    const float v = alpha * sum;
    *dst = (beta != 0.0f) ? __builtin_fmaf(beta, *dst, v) : v;
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers.
// ---------------------------------------------------------------------------
using TileLarge = SgemmTile<256, 256, 16, 2, 2>;     // 4 waves, 128 x 128 each, 1 wave/SIMD
using TileMedium = SgemmTile<128, 128, 16, 2, 2>;    // 4 waves, 64 x 64 each
using TileSmall = SgemmTile<64, 64, 16, 2, 2>;       // 4 waves, 32 x 32 each
using TileLargeK32 = SgemmTile<256, 256, 32, 2, 2>;  // as TileLarge, half the barriers
using TileTall = SgemmTile<128, 256, 16, 2, 2, 2>;   // 4 waves, 64 x 128 each, 2 workgroups/CU

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static_assert(TileLarge::BK == sgemm_tile_bk(0) && TileMedium::BK == sgemm_tile_bk(1) &&
                  TileSmall::BK == sgemm_tile_bk(2) && TileLargeK32::BK == sgemm_tile_bk(3) &&
                  TileTall::BK == sgemm_tile_bk(4),
              "the host-side planner's K steps must match the tiles");

static hipError_t launch_reduce(const SgemmCall& c, int splits, const float* ws, hipStream_t s) {
  const int64_t total = (int64_t)c.M * c.N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(sgemm_splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, c.M,
                     c.N, splits, ws, c.alpha, c.beta, c.C, c.ldc);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_tile(const SgemmCall& c, const SgemmPlan& plan, int group_m, float* ws,
                              hipStream_t s) {
  SgemmArgs p;
  p.M = c.M; p.N = c.N; p.K = c.K;
  p.alpha = c.alpha; p.beta = c.beta;
  p.A = c.A; p.lda = c.lda; p.B = c.B; p.ldb = c.ldb; p.C = c.C; p.ldc = c.ldc;
  p.tiles_m = (c.M + T::BM - 1) / T::BM;
  p.tiles_n = (c.N + T::BN - 1) / T::BN;
  p.group_m = group_m;
  p.k_chunk = plan.k_chunk;
  p.ws = ws;
  const bool edge = !(c.M % T::BM == 0 && c.N % T::BN == 0 && c.K % T::BK == 0 &&
                      c.lda % 4 == 0 && c.ldb % 4 == 0 && aligned16(c.A) && aligned16(c.B));
  const bool split = plan.splits > 1;
  const dim3 grid(p.tiles_m * p.tiles_n, split ? plan.splits : 1), block(T::THREADS);
  if (split) {
    if (edge)
      hipLaunchKernelGGL((sgemm_mfma_kernel<T, true, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((sgemm_mfma_kernel<T, false, true>), grid, block, 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_reduce(c, plan.splits, ws, s);
  }
  if (edge)
    hipLaunchKernelGGL((sgemm_mfma_kernel<T, true, false>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((sgemm_mfma_kernel<T, false, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_sgemm(const SgemmCall& c, const SgemmPlan& plan, float* ws, hipStream_t s) {
  if (plan.splits > 1 && ws == nullptr) return hipErrorInvalidValue;
  switch (plan.tile) {
    case 0: return launch_tile<TileLarge>(c, plan, 4, ws, s);
    case 1: return launch_tile<TileMedium>(c, plan, 8, ws, s);
    case 2: return launch_tile<TileSmall>(c, plan, 8, ws, s);
    case 3: return launch_tile<TileLargeK32>(c, plan, 4, ws, s);
    case 4: return launch_tile<TileTall>(c, plan, 8, ws, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_sgemm_scale(int M, int N, float beta, float* C, int ldc, hipStream_t s) {
  const int64_t total = (int64_t)M * N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(sgemm_scale_kernel, dim3((unsigned)blocks), dim3(256), 0, s, M, N, beta, C,
                     ldc);
  return hipGetLastError();
}

}  // namespace lasg
