// FP16-input / FP32-accumulate GEMM with bias and activation fused into the
// single write-back, for gfx950:
//     C = act(alpha * A x B + bias),  A: M x K fp16, B: K x N fp16, bias: N fp32,
//     C: M x N fp16 (round to nearest even).
//
// This is the half-precision product of the DeepGEMM page: bias, scale and
// GELU applied to the accumulators in registers and stored once (sections 1.1
// and 3.2), accumulators kept in registers for the whole K loop (4.3), L2-aware
// tile order (3.4).  The tiling is the same block / wave hierarchy as the FP32
// kernels (SGEMM page, station k10), with v_mfma_f32_32x32x16_f16 as the wave's
// unit of work.
//
// Operand feed.  The MFMA takes, per lane, eight A values along k for row
// l % 32 and eight B values along k for column l % 32, lanes 0-31 and 32-63
// covering the two halves of the 16-wide k step.  A is row-major (k-contiguous)
// and is staged into LDS as As[m][k].  B is row-major in N, so its k values for
// one column are a full row apart; the staging transposes each 8 x 8 block of
// B in registers and stores it as Bt[n][k], after which both operands are read
// with one 16-byte LDS load per lane per MFMA.  LDS rows carry 8 halves of
// padding so these reads and the staging writes do not collide in the banks
// (Tiled-GEMM chapter 11.5).
#include "gemm_common.h"
#include "gemm_launch.h"

namespace lasg {

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_>
struct HgemmTile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int THREADS = WAVES_M * WAVES_N * kWave;
  static constexpr int WTM = BM / WAVES_M;
  static constexpr int WTN = BN / WAVES_N;
  static constexpr int FM = WTM / 32;
  static constexpr int FN = WTN / 32;
  static constexpr int STRIDE = BK + 8;                 // halves per LDS row (As and Bt)
  static constexpr int A_STAGE = BM * STRIDE;           // halves
  static constexpr int B_STAGE = BN * STRIDE;
  static constexpr int LDS_HALVES = 2 * (A_STAGE + B_STAGE);
  static constexpr int A_CHUNKS = BM * BK / 8 / THREADS;        // 16-byte A loads per thread
  static constexpr int B_BLOCK_TOTAL = (BK / 8) * (BN / 8);     // 8x8 blocks of the B tile
  static constexpr int B_BLOCKS = (B_BLOCK_TOTAL + THREADS - 1) / THREADS;  // per thread

  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 MFMA blocks");
  static_assert(BK % 16 == 0, "K tile is consumed in MFMA steps of 16");
  static_assert((BM * BK / 8) % THREADS == 0, "A tile must split evenly into 16-byte loads");
  static_assert(B_BLOCK_TOTAL % THREADS == 0 || B_BLOCK_TOTAL < THREADS,
                "B tile must split evenly into 8x8 blocks (or use fewer threads than blocks)");
  static_assert(LDS_HALVES * 2 <= 160 * 1024, "two stages must fit gfx950's 160 KiB of LDS");
  static_assert(FM * FN * 16 <= 256, "accumulators must fit in 256 registers per lane");
};

struct HgemmArgs {
  int M, N, K;
  float alpha;
  const uint16_t* A;
  int lda;
  const uint16_t* B;
  int ldb;
  const float* bias;
  int act;
  uint16_t* C;
  int ldc;
  int tiles_m, tiles_n, group_m;
};

template <class T, bool EDGE>
struct HStage {
  u32x4 a[T::A_CHUNKS];
  u32x4 b[T::B_BLOCKS][8];   // 8 rows (k) x 8 halves (n) per block

  // The thread's 8x8 block of B: k-block kb (8 rows) and n-block nb (8 columns).
  // Consecutive lanes take consecutive k-blocks so that their transposed 16-byte
  // LDS writes land on consecutive addresses.
  static __device__ __forceinline__ void b_block(int q, int& kb, int& nb) {
    kb = q % (T::BK / 8);
    nb = q / (T::BK / 8);
  }

  static __device__ __forceinline__ u32x4 load8(const uint16_t* base, int row, int col, int rows,
                                                int cols, int ld) {
    if constexpr (!EDGE) {
      return *reinterpret_cast<const u32x4*>(base + (size_t)row * ld + col);
    } else {
      uint16_t h[8];
      const uint16_t* src = base + (size_t)row * ld;
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = (row < rows && col + e < cols) ? src[col + e] : 0;
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (uint32_t)h[2 * e] | ((uint32_t)h[2 * e + 1] << 16);
      return v;
    }
  }

  __device__ __forceinline__ void load(const HgemmArgs& p, int m0, int n0, int k0, int tid) {
#pragma unroll
    for (int v = 0; v < T::A_CHUNKS; ++v) {
      const int c = tid + v * T::THREADS;
      const int row = c / (T::BK / 8);
      const int kc = (c % (T::BK / 8)) * 8;
      a[v] = load8(p.A, m0 + row, k0 + kc, p.M, p.K, p.lda);
    }
#pragma unroll
    for (int v = 0; v < T::B_BLOCKS; ++v) {
      const int q = tid + v * T::THREADS;
      if (T::B_BLOCK_TOTAL < T::THREADS && q >= T::B_BLOCK_TOTAL) break;
      int kb, nb;
      b_block(q, kb, nb);
#pragma unroll
      for (int r = 0; r < 8; ++r) b[v][r] = load8(p.B, k0 + 8 * kb + r, n0 + 8 * nb, p.K, p.N, p.ldb);
    }
  }

  __device__ __forceinline__ void store(uint16_t* As, uint16_t* Bt, int tid) const {
#pragma unroll
    for (int v = 0; v < T::A_CHUNKS; ++v) {
      const int c = tid + v * T::THREADS;
      const int row = c / (T::BK / 8);
      const int kc = (c % (T::BK / 8)) * 8;
      *reinterpret_cast<u32x4*>(As + row * T::STRIDE + kc) = a[v];
    }
#pragma unroll
    for (int v = 0; v < T::B_BLOCKS; ++v) {
      const int q = tid + v * T::THREADS;
      if (T::B_BLOCK_TOTAL < T::THREADS && q >= T::B_BLOCK_TOTAL) break;
      int kb, nb;
      b_block(q, kb, nb);
      // b[v][r][c] holds B(k = 8kb + r, n = 8nb + 2c) in its low half and n + 1 in
      // its high half.  Column n of the block, as 8 consecutive k, is the low (even
      // n) or high (odd n) halves of the 8 rows, paired two rows per dword.
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        u32x4 lo, hi;
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) {
          const uint32_t x = b[v][2 * pr][c];
          const uint32_t y = b[v][2 * pr + 1][c];
          lo[pr] = (x & 0xffffu) | (y << 16);
          hi[pr] = (x >> 16) | (y & 0xffff0000u);
        }
        *reinterpret_cast<u32x4*>(Bt + (8 * nb + 2 * c) * T::STRIDE + 8 * kb) = lo;
        *reinterpret_cast<u32x4*>(Bt + (8 * nb + 2 * c + 1) * T::STRIDE + 8 * kb) = hi;
      }
    }
  }
};

// GELU, tanh form: 0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3).
// Since 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)), this is x / (1 + exp(-2u));
// it tends to x for large positive x and to -0 for large negative x.
__device__ __forceinline__ float gelu_tanh(float x) {
  const float k0 = 0.7978845608028654f;   // sqrt(2 / pi)
  const float k1 = 0.044715f;
  const float u = k0 * __builtin_fmaf(k1 * x, x * x, x);
  return x / (1.0f + __expf(-2.0f * u));
}

template <class T, bool EDGE>
__global__ void __launch_bounds__(T::THREADS) hgemm_mfma_kernel(HgemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[T::LDS_HALVES];
  uint16_t* const As0 = lds;
  uint16_t* const Bt0 = lds + T::A_STAGE;
  uint16_t* const As1 = lds + T::A_STAGE + T::B_STAGE;
  uint16_t* const Bt1 = As1 + T::A_STAGE;

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
  HStage<T, EDGE> st;
  if (ktiles > 0) {
    st.load(p, m0, n0, 0, tid);
    st.store(As0, Bt0, tid);
  }
  __syncthreads();

  const int a_off = (wm * T::WTM + l32) * T::STRIDE + 8 * half;
  const int b_off = (wn * T::WTN + l32) * T::STRIDE + 8 * half;

  for (int kt = 0; kt < ktiles; ++kt) {
    const bool odd = kt & 1;
    const uint16_t* As = odd ? As1 : As0;
    const uint16_t* Bt = odd ? Bt1 : Bt0;
    const bool more = kt + 1 < ktiles;
    if (more) st.load(p, m0, n0, (kt + 1) * T::BK, tid);

#pragma unroll
    for (int s = 0; s < T::BK / 16; ++s) {
      f16x8 af[T::FM], bf[T::FN];
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
        af[i] = *reinterpret_cast<const f16x8*>(As + a_off + i * 32 * T::STRIDE + 16 * s);
#pragma unroll
      for (int j = 0; j < T::FN; ++j)
        bf[j] = *reinterpret_cast<const f16x8*>(Bt + b_off + j * 32 * T::STRIDE + 16 * s);
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }

    if (more) st.store(odd ? As0 : As1, odd ? Bt0 : Bt1, tid);
    __syncthreads();
  }

  // Epilogue: x = alpha * acc + bias[col]; y = act(x); C = fp16(y).
  const float alpha = p.alpha;
  const bool gelu = p.act == 1;
#pragma unroll
  for (int j = 0; j < T::FN; ++j) {
    const int col = n0 + wn * T::WTN + j * 32 + l32;
    const bool col_ok = !EDGE || col < p.N;
    const float bj = (p.bias != nullptr && col_ok) ? p.bias[col] : 0.0f;
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * T::WTM + i * 32 + mfma32_row(r, lane);
        if (EDGE && (row >= p.M || !col_ok)) continue;
        float x = __builtin_fmaf(alpha, acc[i][j][r], bj);
        if (gelu) x = gelu_tanh(x);
        const _Float16 h = (_Float16)x;
        p.C[(size_t)row * p.ldc + col] = __builtin_bit_cast(uint16_t, h);
      }
    }
  }
}

using HTileLarge = HgemmTile<256, 256, 64, 2, 2>;
using HTileMedium = HgemmTile<128, 128, 64, 2, 2>;
using HTileSmall = HgemmTile<64, 64, 64, 2, 2>;

template <class T>
static hipError_t launch_htile(const HgemmCall& c, int group_m, hipStream_t s) {
  HgemmArgs p;
  p.M = c.M; p.N = c.N; p.K = c.K;
  p.alpha = c.alpha;
  p.A = c.A; p.lda = c.lda; p.B = c.B; p.ldb = c.ldb;
  p.bias = c.bias; p.act = c.act;
  p.C = c.C; p.ldc = c.ldc;
  p.tiles_m = (c.M + T::BM - 1) / T::BM;
  p.tiles_n = (c.N + T::BN - 1) / T::BN;
  p.group_m = group_m;
  const bool fast = c.M % T::BM == 0 && c.N % T::BN == 0 && c.K % T::BK == 0 &&
                    c.lda % 8 == 0 && c.ldb % 8 == 0 &&
                    (reinterpret_cast<uintptr_t>(c.A) & 15u) == 0 &&
                    (reinterpret_cast<uintptr_t>(c.B) & 15u) == 0;
  const dim3 grid(p.tiles_m * p.tiles_n), block(T::THREADS);
  if (fast)
    hipLaunchKernelGGL((hgemm_mfma_kernel<T, false>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((hgemm_mfma_kernel<T, true>), grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_hgemm(const HgemmCall& c, int cus, int force_tile, hipStream_t s) {
  int tile = force_tile;
  if (tile < 0) tile = sgemm_pick_tile(c.M, c.N, cus);
  switch (tile) {
    case 0: return launch_htile<HTileLarge>(c, 4, s);
    case 1: return launch_htile<HTileMedium>(c, 8, s);
    default: return launch_htile<HTileSmall>(c, 8, s);
  }
}

}  // namespace lasg
