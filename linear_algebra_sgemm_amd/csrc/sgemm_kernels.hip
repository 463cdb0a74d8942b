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
#include "dma_common.h"
#include "gemm_common.h"
#include "gemm_launch.h"

namespace lasg {

// The FP32 MFMA block shapes.  BLK x BLK outputs per instruction, KSLOTS k-slots
// (lane / BLK selects the slot) of one k each; ACC accumulator registers per lane.
// A group of 4 * KSLOTS consecutive k is consumed by four MFMA steps; step s and
// slot h take k = 4 h + s of the group, so a lane's four A values of one group
// are contiguous.
struct MfmaF32x32 {   // v_mfma_f32_32x32x2_f32: 64 cycles, 16 accumulators per lane
  static constexpr int BLK = 32, KSLOTS = 2, ACC = 16;
  typedef f32x16 acc_t;
  static __device__ __forceinline__ acc_t mfma(float a, float b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  // Row (within the block) of accumulator register r of lane `lane`; the column is lane % 32.
  static __device__ __forceinline__ int row(int r, int lane) { return mfma32_row(r, lane); }
};
struct MfmaF16x16 {   // v_mfma_f32_16x16x4_f32: 32 cycles, 4 accumulators per lane
  static constexpr int BLK = 16, KSLOTS = 4, ACC = 4;
  typedef f32x4 acc_t;
  static __device__ __forceinline__ acc_t mfma(float a, float b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ int row(int r, int lane) { return 4 * (lane >> 4) + r; }
};

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int WAVES_PER_SIMD_ = 1,
          class MF_ = MfmaF32x32>
struct SgemmTile {
  using MF = MF_;
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  // Waves of this kernel that must fit on one SIMD at once (register budget:
  // 512 / WAVES_PER_SIMD registers per lane, accumulators included).
  static constexpr int WAVES_PER_SIMD = WAVES_PER_SIMD_;
  static constexpr int THREADS = WAVES_M * WAVES_N * kWave;
  static constexpr int WTM = BM / WAVES_M;     // wave sub-tile rows
  static constexpr int WTN = BN / WAVES_N;     // wave sub-tile columns
  static constexpr int BLK = MF::BLK;
  static constexpr int G = 4 * MF::KSLOTS;     // k per group of four MFMA steps
  static constexpr int FM = WTM / BLK;         // MFMA blocks per wave, along M
  static constexpr int FN = WTN / BLK;         // ... along N
  static constexpr int A_STRIDE = BK + 4;      // floats per LDS row of the A tile (one row = one m)
  // floats per LDS row of the B tile (one row = one k): the k-slots of one B read
  // are 4 rows apart, so 4 B_STRIDE must spread them over the 64 banks.
  static constexpr int B_STRIDE = BN + (MF::KSLOTS == 4 ? 4 : 8);
  static constexpr int A_STAGE = BM * A_STRIDE;
  static constexpr int B_STAGE = BK * B_STRIDE;
  static constexpr int LDS_FLOATS = 2 * (A_STAGE + B_STAGE);
  static constexpr int A_VECS = BM * BK / 4 / THREADS;   // float4 loads per thread per K tile
  static constexpr int B_VECS = BK * BN / 4 / THREADS;

  static_assert(WTM % BLK == 0 && WTN % BLK == 0, "wave tile must be whole MFMA blocks");
  static_assert(BK % G == 0, "K tile is consumed in whole groups");
  static_assert((BM * BK / 4) % THREADS == 0, "A tile must split evenly into float4 loads");
  static_assert((BK * BN / 4) % THREADS == 0, "B tile must split evenly into float4 loads");
  static_assert(THREADS % (BK / 4) == 0 && THREADS % (BN / 4) == 0, "load rows must not wrap");
  static_assert(LDS_FLOATS * 4 <= 160 * 1024, "two stages must fit gfx950's 160 KiB of LDS");
  static_assert(FM * FN * MF::ACC <= 256 / WAVES_PER_SIMD,
                "accumulators must leave room for operands");
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
  // Bounds-checked path: rows of A (B) are 16-byte aligned, so a 4-float chunk that
  // lies wholly inside the matrix may be read with one 16-byte load.
  int a_vec, b_vec;
  // Direct-to-LDS kernels: columns of each row of B that may be read (a multiple
  // of 4, at least N).
  int nb;
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
        if (p.a_vec && gm < p.M && gk + 3 < p.K) {
          a[v] = *reinterpret_cast<const f32x4*>(src + gk);   // whole chunk inside, 16-byte aligned
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            a[v][e] = (gm < p.M && gk + e < p.K) ? src[gk + e] : 0.0f;
        }
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
        if (p.b_vec && gk < p.K && gn + 3 < p.N) {
          b[v] = *reinterpret_cast<const f32x4*>(src + gn);   // whole chunk inside, 16-byte aligned
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            b[v][e] = (gk < p.K && gn + e < p.N) ? src[gn + e] : 0.0f;
        }
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

// Epilogue of one wave: C = alpha * acc + beta * C over the wave's WTM x WTN
// sub-tile at (r0, c0), C read only when beta != 0.  The C loads of a batch of
// JB blocks of one block row are all issued before the first one is consumed,
// so their latencies overlap instead of adding up: a whole block row on whole
// tiles, one block at a time in the bounds-checked form (EDGE), whose row and
// column checks hold registers of their own.
// `pre` (when given): this lane's values of C, loaded earlier, in the order of
// the accumulators (block i, j, element r at ((i FN + j) ACC + r)).
template <class T, bool EDGE, class ACC>
__device__ __forceinline__ void sgemm_store(const SgemmArgs& p, const ACC& acc, int r0, int c0,
                                            int lane, const float* pre = nullptr) {
  using MF = typename T::MF;
  constexpr int JB = EDGE ? 1 : T::FN;
  const int lb = lane % T::BLK;
  const float alpha = p.alpha, beta = p.beta;
  const bool read_c = beta != 0.0f;
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
#pragma unroll
    for (int j0 = 0; j0 < T::FN; j0 += JB) {
      float cv[JB][MF::ACC];
      if (read_c) {
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
          const int col = c0 + (j0 + jj) * T::BLK + lb;
#pragma unroll
          for (int r = 0; r < MF::ACC; ++r) {
            const int row = r0 + i * T::BLK + MF::row(r, lane);
            const bool ok = !EDGE || (row < p.M && col < p.N);
            if (pre != nullptr)
              cv[jj][r] = pre[(i * T::FN + j0 + jj) * MF::ACC + r];
            else
              cv[jj][r] = ok ? p.C[(size_t)row * p.ldc + col] : 0.0f;
          }
        }
      }
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        const int col = c0 + (j0 + jj) * T::BLK + lb;
#pragma unroll
        for (int r = 0; r < MF::ACC; ++r) {
          const int row = r0 + i * T::BLK + MF::row(r, lane);
          if (EDGE && (row >= p.M || col >= p.N)) continue;
          const float v = alpha * acc[i][j0 + jj][r];
          p.C[(size_t)row * p.ldc + col] = read_c ? __builtin_fmaf(beta, cv[jj][r], v) : v;
        }
      }
    }
  }
}

// EDGE: bounds-checked loads and stores; STORE_EDGE alone: operands padded to
// whole tiles (SgemmCall::padded), loads unchecked, stores of C checked.
template <class T, bool EDGE, bool SPLIT, bool STORE_EDGE = EDGE>
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
  using MF = typename T::MF;
  const int lb = lane % T::BLK;       // row of A / column of B within a block
  const int slot = lane / T::BLK;     // k-slot

  typename MF::acc_t acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int r = 0; r < MF::ACC; ++r) acc[i][j][r] = 0.0f;

  const int ktiles = (p.K + T::BK - 1) / T::BK;
  Stage<T, EDGE> st;
  if (ktiles > 0) {
    st.load(p, m0, n0, 0, tid);
    st.store(As0, Bs0, tid);
  }
  __syncthreads();

  // Per-lane fragment origins inside one LDS stage.
  const int a_off = (wm * T::WTM + lb) * T::A_STRIDE + 4 * slot;
  const int b_off = (4 * slot) * T::B_STRIDE + wn * T::WTN + lb;

  for (int kt = 0; kt < ktiles; ++kt) {
    const bool odd = kt & 1;
    const float* As = odd ? As1 : As0;
    const float* Bs = odd ? Bs1 : Bs0;
    const bool more = kt + 1 < ktiles;
    if (more) st.load(p, m0, n0, (kt + 1) * T::BK, tid);

#pragma unroll
    for (int g = 0; g < T::BK / T::G; ++g) {
      f32x4 af[T::FM];
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
        af[i] = *reinterpret_cast<const f32x4*>(As + a_off + i * T::BLK * T::A_STRIDE + T::G * g);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float bf[T::FN];
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
          bf[j] = Bs[b_off + (T::G * g + s) * T::B_STRIDE + j * T::BLK];
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
#pragma unroll
          for (int j = 0; j < T::FN; ++j) acc[i][j] = MF::mfma(af[i][s], bf[j], acc[i][j]);
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
        const int col = n0 + wn * T::WTN + j * T::BLK + lb;
#pragma unroll
        for (int r = 0; r < MF::ACC; ++r) {
          const int row = m0 + wm * T::WTM + i * T::BLK + MF::row(r, lane);
          if (STORE_EDGE && (row >= p.M || col >= p.N)) continue;
          W[(size_t)row * p.N + col] = acc[i][j][r];
        }
      }
    return;
  }

  sgemm_store<T, STORE_EDGE>(p, acc, m0 + wm * T::WTM, n0 + wn * T::WTN, lane);
}

// ---------------------------------------------------------------------------
// Small outputs: one 16 x 16 output tile per workgroup, its K range split over
// the workgroup's waves (the split-K of lecture 24, section 8.3, inside one
// workgroup).  A 256^3 product gives 256 such workgroups, one per CU; each wave
// takes every WAVES-th chunk of 256 / WAVES values of k, and its operands go
// straight from global memory into registers (no LDS staging).  The partial
// tiles meet in LDS, where they are added in wave order (0 + 1 + 2 + ..., so
// results do not change from run to run) before alpha and beta are applied.
//
// k mapping: for a chunk of 4 T values of k starting at kb, MFMA step s (0 ..
// T - 1) gives k-slot h (lane / 16) the index kb + T h + s, so a lane's T A
// values of a chunk are contiguous in its row (T / 4 16-byte loads) and A and B
// agree on which k each product uses.  Any M, N, K and leading dimension: loads
// outside the matrices are replaced by zero, stores are predicated.  WHOLE (M
// and N multiples of 16, K of 32, rows of A 16-byte aligned): every value read
// lies inside the matrices, so no value needs replacing.  Either way every load
// is unconditional (addresses clamped into the matrices) and all of a chunk's
// loads go out before its first MFMA -- one memory round trip per chunk, where
// loads each in its own branch made the first MFMA wait for all of them
// (256^3: 3.08 us against 3.44).
// ---------------------------------------------------------------------------
constexpr int kWksTile = 16;      // output tile edge
constexpr int kWksSpan = 256;     // k covered by one chunk of every wave

template <bool WHOLE, int WAVES>
__global__ void __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(WAVES / 4)))
sgemm_wave_ksplit_kernel(SgemmArgs p) {
  constexpr int CHUNK = kWksSpan / WAVES;   // k per wave per step
  constexpr int T = CHUNK / 4;              // MFMA steps per chunk
  static_assert(T % 4 == 0 && T % 2 == 0, "whole 16-byte loads of A, pairs of MFMAs");
  __shared__ float part[WAVES][kWksTile * kWksTile];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int m0 = (blockIdx.x / p.tiles_n) * kWksTile;
  const int n0 = (blockIdx.x % p.tiles_n) * kWksTile;
  const int l16 = lane % 16, h = lane / 16;
  const int row = m0 + l16, col = n0 + l16;
  const bool row_ok = row < p.M, col_ok = col < p.N;
  const float* arow = p.A + (size_t)(row_ok ? row : 0) * p.lda;
  f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int kb = wave * CHUNK; kb < p.K; kb += kWksSpan) {
    const int ka = kb + T * h;
    float a[T], b[T];
    if constexpr (WHOLE) {
#pragma unroll
      for (int v = 0; v < T / 4; ++v) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(arow + ka + 4 * v);
#pragma unroll
        for (int e = 0; e < 4; ++e) a[4 * v + e] = x[e];
      }
      const float* bk = p.B + (size_t)ka * p.ldb + col;
#pragma unroll
      for (int t = 0; t < T; ++t) b[t] = bk[(size_t)t * p.ldb];
      __builtin_amdgcn_sched_barrier(0);   // every load before the first MFMA
    } else {
      // Clamped loads: row, column and k are clamped into the matrices, so every
      // load is unconditional and in bounds, and values outside are replaced by
      // zero afterwards.  Whether A's row segments take 16-byte loads is decided
      // per wave (the whole chunk inside K), so the branch does not diverge.
      const float* bcol = p.B + (col_ok ? col : 0);
      if (p.a_vec && kb + CHUNK <= p.K) {
#pragma unroll
        for (int v = 0; v < T / 4; ++v) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(arow + ka + 4 * v);
#pragma unroll
          for (int e = 0; e < 4; ++e) a[4 * v + e] = x[e];
        }
#pragma unroll
        for (int t = 0; t < T; ++t) b[t] = bcol[(size_t)(ka + t) * p.ldb];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          a[t] = row_ok ? a[t] : 0.0f;
          b[t] = col_ok ? b[t] : 0.0f;
        }
      } else {
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const int k = ka + t < p.K ? ka + t : p.K - 1;
          a[t] = arow[k];
          b[t] = bcol[(size_t)k * p.ldb];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const bool in_k = ka + t < p.K;
          a[t] = row_ok && in_k ? a[t] : 0.0f;
          b[t] = col_ok && in_k ? b[t] : 0.0f;
        }
      }
    }
    // two accumulators, so consecutive MFMAs do not wait for each other
#pragma unroll
    for (int t = 0; t < T; t += 2) {
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t], b[t], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t + 1], b[t + 1], acc1, 0, 0, 0);
    }
  }
  // lane l holds column l % 16, rows 4 (l / 16) + r of this wave's partial tile
#pragma unroll
  for (int r = 0; r < 4; ++r) part[wave][(4 * h + r) * kWksTile + l16] = acc0[r] + acc1[r];
  __syncthreads();
  const int t = threadIdx.x;
  const int i = m0 + t / kWksTile, j = n0 + t % kWksTile;
  if (t < kWksTile * kWksTile && i < p.M && j < p.N) {
    float sum = part[0][t];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) sum += part[w][t];
    float* dst = p.C + (size_t)i * p.ldc + j;
    const float v = p.alpha * sum;
    *dst = p.beta != 0.0f ? __builtin_fmaf(p.beta, *dst, v) : v;
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

// ---------------------------------------------------------------------------
// Direct-to-LDS variant for whole tiles (M % BM == N % BN == 0, K % 32 == 0,
// lda and ldb multiples of 4, A and B 16-byte aligned).
//
// Loads go straight from global memory into a ring of STAGES LDS stages with
// global_load_lds_dwordx4 (lane l of one instruction writes its 16 bytes at
// base + 16 l): no staging registers, no LDS stores, STAGES - 1 K tiles in
// flight, and each wave reads the fragments of the next K tile while its MFMAs
// work on the current one, with one barrier per K tile (the pipelined main loop
// of the DeepGEMM page, 3.3; the double buffer of the Tiled-GEMM chapter, 11.4,
// made deeper).  Each copy instruction chooses the global chunk of every LDS
// slot, which sets the layout:
//  * A: 64-byte rows (one row of a 16-wide K tile), the four 16-byte chunks of
//    row r permuted by row64_swizzle(r); one instruction copies 16 whole rows
//    (A_DW: rows of A only 4-byte aligned, lda not a multiple of 4: 4-byte
//    copies, one instruction per 4 rows, the same LDS layout).
//    A fragment read (chunk 2 g + l / 32 of 32 consecutive rows) is then free
//    of bank conflicts.
//  * B: one instruction per 1 KiB of rows of the tile (one row of BN = 256
//    floats, or two of BN = 128), each copy's 1 KiB padded (to 1056 or 1088
//    bytes) so that the two k-slots of a B read (rows 4 apart) fall on
//    different halves of the 64 banks.
// ---------------------------------------------------------------------------
template <int BM_, int BN_, int STAGES_, int WAVES_PER_SIMD_ = 1, int WAVES_M_ = 2,
          int WAVES_N_ = 2, bool A_DW_ = false, bool LEAN_ = false, bool PAIR_ = false>
struct SDmaTile {
  using MF = MfmaF32x32;
  static constexpr int BM = BM_, BN = BN_, BK = 16, STAGES = STAGES_;
  static constexpr bool A_DW = A_DW_;
  // LEAN: two fragment sets instead of four (sdma_tile2): the second group of
  // a K tile is read under the MFMAs of its first group, and the next tile's
  // first group under those of the second; for the tile whose accumulators
  // leave no room for four sets.
  static constexpr bool LEAN = LEAN_;
  // The same tile copying A with 4-byte copies.
  using WithADw =
      SDmaTile<BM_, BN_, STAGES_, WAVES_PER_SIMD_, WAVES_M_, WAVES_N_, true, LEAN_, PAIR_>;
  static constexpr int WAVES_PER_SIMD = WAVES_PER_SIMD_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, WAVES = WAVES_M * WAVES_N;
  static constexpr int WG_PER_CU = WAVES_PER_SIMD * 4 / WAVES;
  static constexpr int THREADS = WAVES * kWave;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int BLK = 32;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int A_BYTES = BM * BK * 4;          // 64-byte rows
  static constexpr int B_RPC = 1024 / (BN * 4);        // rows of B per copy
  // Bytes per copy slot of B: rows r and r + 4 lie 4 / B_RPC slots apart, and
  // (4 / B_RPC) * B_SLOT = 128 (mod 256) puts them on opposite halves of the banks.
  static constexpr int B_SLOT = 1024 + 32 * B_RPC;
  static constexpr int B_BYTES = (BK / B_RPC) * B_SLOT;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int A_COPY = A_DW ? 256 : 1024;      // bytes of A per copy instruction
  static constexpr int A_INSTR = A_BYTES / A_COPY;       // 4 or 16 rows per copy
  static constexpr int B_INSTR = BK / B_RPC;
  static constexpr int A_PER_WAVE = A_INSTR / WAVES;
  static constexpr int B_PER_WAVE = B_INSTR / WAVES;
  static constexpr int LOADS_PER_TILE = A_PER_WAVE + B_PER_WAVE;
  // PAIR: one barrier per two K tiles (sdma_tile_pair): at the barrier before an
  // even tile kt, tiles kt + 1 and kt + 2 have landed and the copies of kt + 3
  // and kt + 4 go out; the odd tile runs without wait or barrier.  Taken where
  // the doubled copies still fit one per MFMA in a group, or on the 64 x 64
  // tile (its copies go out in one burst either way); the 128 x 128 tile copying
  // A 4 bytes at a time (20 copies, 16 MFMAs per group) measured 10 % slower with it.
  static constexpr bool PAIR = PAIR_ && (2 * LOADS_PER_TILE <= 4 * FM * FN || BM * BN <= 64 * 64);
  // Byte offset of row r (0 .. BK - 1) of B inside the stage's B region.
  static __device__ __forceinline__ int b_row(int r) {
    return (r / B_RPC) * B_SLOT + (r % B_RPC) * (BN * 4);
  }

  static_assert(BN * 4 == 1024 || BN * 4 == 512 || BN * 4 == 256,
                "one, two or four rows of B per copy instruction");
  static_assert(((4 / B_RPC) * B_SLOT) % 256 == 128, "k-slots of a B read on opposite bank halves");
  static_assert(A_INSTR % WAVES == 0 && B_INSTR % WAVES == 0, "copies split evenly over waves");
  static_assert(STAGE_BYTES % 16 == 0, "stages start on 16-byte boundaries");
  static_assert(STAGES >= 3 && STAGES * STAGE_BYTES * WG_PER_CU <= 160 * 1024,
                "the stages of every resident workgroup must fit in LDS");
  static_assert((STAGES - 2) * LOADS_PER_TILE <= 63, "in-flight copies must fit vmcnt");
  static_assert(FM * FN * 16 <= 256 / WAVES_PER_SIMD, "accumulators must leave room for operands");
  static_assert(!PAIR || (STAGES == 4 && !LEAN), "two tiles in use and two in flight");
  // A ragged K's last values go through the pipeline before the main loop on the
  // tiles narrower than 256 x 256 (measured faster there); the 256 x 256 tiles
  // take them after the loop.
  static constexpr bool TAIL_FIRST = BM * BN < 256 * 256;
  // PRE_C: a wave of one 32 x 32 block (the 64 x 64 tile) loads its 16 values
  // of C per lane at the start, ahead of the first copies, and keeps them in
  // registers for the epilogue: all workgroups of a round reach the epilogue
  // together, where the reads of C would wait a full memory round trip
  // (1000 x 3000 x 777: 1.3 us of a 46 us call).  The larger tiles have no
  // registers to spare for it.
  static constexpr bool PRE_C = FM * FN == 1;
};

// Per-lane byte offsets of a wave's copies relative to the K tile's A or B base
// (a_base(kt) = A + m0 lda + 16 kt, b_base(kt) = B + 16 kt ldb + n0, floats),
// and the LDS slot of copy v inside one stage.  On a tile that crosses the
// bottom or right edge, rows of A past M - 1 copy row M - 1 and 4-column chunks
// of B at or past nb (the readable width, a multiple of 4) copy the chunk at
// nb - 4, so every copy reads inside the matrices; the values land in rows and
// columns of the tile that the epilogue does not store.
template <class T>
struct SDmaPlan {
  uint32_t off[T::LOADS_PER_TILE];
  __device__ __forceinline__ SDmaPlan(const SgemmArgs& p, int wave, int lane, int m0, int n0) {
#pragma unroll
    for (int v = 0; v < T::LOADS_PER_TILE; ++v) {
      if (v < T::A_PER_WAVE) {
        if constexpr (T::A_DW) {
          // lane l fills byte 4 (l % 16) of row l / 16 of the copy: position
          // (l % 16) / 4, element l % 4, so it reads that element of the chunk
          // the permutation puts there.
          const int r = (wave * T::A_PER_WAVE + v) * 4 + lane / 16;
          const int chunk = ((lane % 16) / 4) ^ row64_swizzle(r);
          const int rc = m0 + r < p.M ? r : p.M - 1 - m0;
          off[v] = (uint32_t)(((size_t)rc * p.lda + 4 * chunk + lane % 4) * 4);
        } else {
          const int r = (wave * T::A_PER_WAVE + v) * 16 + lane / 4;
          const int chunk = (lane % 4) ^ row64_swizzle(r);
          const int rc = m0 + r < p.M ? r : p.M - 1 - m0;
          off[v] = (uint32_t)(((size_t)rc * p.lda + 4 * chunk) * 4);
        }
      } else {
        const int copy = wave * T::B_PER_WAVE + (v - T::A_PER_WAVE);
        const int kr = copy * T::B_RPC + lane / (T::BN / 4);
        const int c4 = 4 * (lane % (T::BN / 4));
        const int cc = n0 + c4 < p.nb ? c4 : p.nb - 4 - n0;
        off[v] = (uint32_t)(((size_t)kr * p.ldb + cc) * 4);
      }
    }
  }
  static __device__ __forceinline__ uint32_t slot(int v, int wave) {
    if (v < T::A_PER_WAVE) return (wave * T::A_PER_WAVE + v) * T::A_COPY;
    return T::A_BYTES + (wave * T::B_PER_WAVE + (v - T::A_PER_WAVE)) * T::B_SLOT;
  }
};

template <class T>
__device__ __forceinline__ void sdma_issue(const SgemmArgs& p, const SDmaPlan<T>& plan,
                                           const float* a_tile, const float* b_tile, int kt,
                                           uint32_t stage, int wave, int x) {
  const float* base = x < T::A_PER_WAVE ? a_tile + kt * T::BK
                                        : b_tile + (size_t)kt * T::BK * p.ldb;
  if (T::A_DW && x < T::A_PER_WAVE)
    dma4_sbase(base, plan.off[x], stage + SDmaPlan<T>::slot(x, wave));
  else
    dma16_sbase(base, plan.off[x], stage + SDmaPlan<T>::slot(x, wave));
}

// Fragments of one group of 8 k (four MFMA steps): a[i] holds A[row][8 g + 4 h
// .. + 3] for the wave's m-block i (h = lane / 32 is the lane's k-slot), b[s][j]
// holds B[8 g + 4 h + s][col] for n-block j.
template <class T>
struct SFrags {
  f32x4 a[T::FM];
  float b[4][T::FN];
};

template <class T>
__device__ __forceinline__ void sload_frags(SFrags<T>& f, const uint8_t* stage, int g, int wm,
                                            int wn, int lane) {
  const int l32 = lane % 32, h = lane / 32;
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
    const int r = wm * T::WTM + i * 32 + l32;
    f.a[i] = *reinterpret_cast<const f32x4*>(stage + r * 64 + 16 * ((2 * g + h) ^ row64_swizzle(r)));
  }
  const uint8_t* bs = stage + T::A_BYTES;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
      f.b[s][j] = *reinterpret_cast<const float*>(bs + T::b_row(8 * g + 4 * h + s) +
                                                  4 * (wn * T::WTN + j * 32 + l32));
}

// MFMA number idx (0 .. 4 FM FN - 1) of one group: step s, m-block i, n-block j.
template <class T>
__device__ __forceinline__ void smfma(f32x16 (&acc)[T::FM][T::FN], const SFrags<T>& f, int idx) {
  const int s = idx / (T::FM * T::FN), i = (idx / T::FN) % T::FM, j = idx % T::FN;
  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[i][s], f.b[s][j], acc[i][j], 0, 0, 0);
}

template <class T>
__device__ __forceinline__ void swait_tiles(int ahead) {
  static_assert(T::STAGES <= 5, "extend the cases below for deeper pipelines");
  if (ahead >= 3 && T::STAGES >= 5) {
    wait_vmcnt<(T::STAGES >= 5 ? 3 * T::LOADS_PER_TILE : 0)>();
  } else if (ahead >= 2 && T::STAGES >= 4) {
    wait_vmcnt<(T::STAGES >= 4 ? 2 * T::LOADS_PER_TILE : 0)>();
  } else if (ahead >= 1) {
    wait_vmcnt<T::LOADS_PER_TILE>();
  } else {
    wait_vmcnt<0>();
  }
}

// One K tile: MFMAs on the fragments of tile kt (x0: group 0, x1: group 1, read
// during the previous tile), reads of tile kt + 1's fragments into y0 / y1, the
// wait for tile kt + 1 and the barrier, and the copies of tile kt + STAGES - 1
// (unconditional when STEADY: the caller guarantees that tile exists).  After
// the last tile the reads hit a stage that is no longer used; their values are
// dropped.
template <class T, bool STEADY>
__device__ __forceinline__ void sdma_tile(const SgemmArgs& p, f32x16 (&acc)[T::FM][T::FN], int kt,
                                          int ktiles, SFrags<T>& x0, SFrags<T>& x1,
                                          SFrags<T>& y0, SFrags<T>& y1, const uint8_t* lds,
                                          uint32_t lds_base, const SDmaPlan<T>& plan,
                                          const float* a_tile, const float* b_tile, int wave,
                                          int wm, int wn, int lane) {
  constexpr int NM = 4 * T::FM * T::FN;            // MFMAs per group
  constexpr int NR = T::FM + 4 * T::FN;            // LDS reads per group
  constexpr int PRE = 2;
  constexpr int R0 = (NR + NM - PRE - 1) / (NM - PRE);
  // The copies go out one per MFMA at the end of group 1 -- or, where a wave
  // has too many of them for that (the 64x64 tile copying A 4 bytes at a
  // time), all together after group 1's MFMAs (BURST).
  constexpr bool BURST = !(NM - T::LOADS_PER_TILE >= NR / 2 && NM - T::LOADS_PER_TILE >= 1);
  constexpr int TAIL = BURST ? NM : NM - T::LOADS_PER_TILE;
  constexpr int R1 = (NR + TAIL - 1) / TAIL;
  static_assert(TAIL >= NR / 2 && TAIL >= 1, "enough MFMAs to spread the reads over");
  smfma<T>(acc, x0, 0);
  smfma<T>(acc, x0, 1);
  if constexpr (STEADY) {
    wait_vmcnt<(T::STAGES - 3) * T::LOADS_PER_TILE>();
  } else {
    const int left = ktiles - 2 - kt;
    swait_tiles<T>(left < 0 ? 0 : (left < T::STAGES - 3 ? left : T::STAGES - 3));
  }
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  const uint8_t* next = lds + ((kt + 1) % T::STAGES) * T::STAGE_BYTES;
  sload_frags<T>(y0, next, 0, wm, wn, lane);
#pragma unroll
  for (int x = PRE; x < NM; ++x) smfma<T>(acc, x0, x);
#pragma unroll
  for (int x = 0; x < NM - PRE; ++x) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, R0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int kt_issue = kt + T::STAGES - 1;
  const bool issue = STEADY || kt_issue < ktiles;
  const uint32_t st_issue = lds_base + (kt_issue % T::STAGES) * T::STAGE_BYTES;
  sload_frags<T>(y1, next, 1, wm, wn, lane);
#pragma unroll
  for (int x = 0; x < TAIL; ++x) smfma<T>(acc, x1, x);
#pragma unroll
  for (int x = 0; x < TAIL; ++x) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, R1, 1);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (BURST) {
#pragma unroll
    for (int x = 0; x < T::LOADS_PER_TILE; ++x)
      if (issue) sdma_issue<T>(p, plan, a_tile, b_tile, kt_issue, st_issue, wave, x);
  } else {
#pragma unroll
    for (int x = 0; x < T::LOADS_PER_TILE; ++x) {
      smfma<T>(acc, x1, TAIL + x);
      if (issue) sdma_issue<T>(p, plan, a_tile, b_tile, kt_issue, st_issue, wave, x);
      __builtin_amdgcn_sched_barrier(0);   // one copy between two MFMAs
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// One K tile of a PAIR tile (four fragment sets, as sdma_tile).  BAR (even kt):
// wait until this wave's copies (tiles kt + 1 and kt + 2) have landed and its
// LDS reads are done, then the barrier: past it tiles kt + 1 and kt + 2 are
// visible and every wave has read stages (kt - 1) % 4 (during tile kt - 2) and
// kt % 4 (during tile kt - 1), which the copies of tiles kt + 3 and kt + 4
// refill among the last MFMAs.  !BAR (odd kt): no wait, barrier or copy; the
// fragments of tile kt + 1 it reads landed before the previous barrier.  Each
// copy thus has two K tiles to land, as with one barrier per tile.
template <class T, bool STEADY, bool BAR>
__device__ __forceinline__ void sdma_tile_pair(const SgemmArgs& p, f32x16 (&acc)[T::FM][T::FN],
                                               int kt, int ktiles, SFrags<T>& x0, SFrags<T>& x1,
                                               SFrags<T>& y0, SFrags<T>& y1, const uint8_t* lds,
                                               uint32_t lds_base, const SDmaPlan<T>& plan,
                                               const float* a_tile, const float* b_tile, int wave,
                                               int wm, int wn, int lane) {
  constexpr int NM = 4 * T::FM * T::FN;            // MFMAs per group
  constexpr int NR = T::FM + 4 * T::FN;            // LDS reads per group
  constexpr int PRE = 2;
  constexpr int R0 = (NR + NM - PRE - 1) / (NM - PRE);
  constexpr int NCOPY = BAR ? 2 * T::LOADS_PER_TILE : 0;
  // Where a wave has more copies than MFMAs to spread them over (the 64 x 64
  // tile), they go out together after the group's MFMAs (BURST).
  constexpr bool BURST = !(NM - NCOPY >= NR / 2 && NM - NCOPY >= 1);
  constexpr int TAIL = BURST ? NM : NM - NCOPY;
  constexpr int R1 = (NR + TAIL - 1) / TAIL;
  static_assert(TAIL >= NR / 2 && TAIL >= 1, "enough MFMAs to spread the reads over");
  smfma<T>(acc, x0, 0);
  smfma<T>(acc, x0, 1);
  if constexpr (BAR) {
    wait_vmcnt<0>();
    lds_barrier();
  }
  const uint8_t* next = lds + ((kt + 1) % T::STAGES) * T::STAGE_BYTES;
  sload_frags<T>(y0, next, 0, wm, wn, lane);
#pragma unroll
  for (int x = PRE; x < NM; ++x) smfma<T>(acc, x0, x);
#pragma unroll
  for (int x = 0; x < NM - PRE; ++x) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, R0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  sload_frags<T>(y1, next, 1, wm, wn, lane);
#pragma unroll
  for (int x = 0; x < TAIL; ++x) smfma<T>(acc, x1, x);
#pragma unroll
  for (int x = 0; x < TAIL; ++x) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, R1, 1);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (BAR) {
#pragma unroll
    for (int x = 0; x < NCOPY; ++x) {
      if constexpr (!BURST) smfma<T>(acc, x1, TAIL + x);
      const int kt_issue = kt + 3 + x / T::LOADS_PER_TILE;
      if (STEADY || kt_issue < ktiles)
        sdma_issue<T>(p, plan, a_tile, b_tile, kt_issue,
                      lds_base + (kt_issue % T::STAGES) * T::STAGE_BYTES, wave,
                      x % T::LOADS_PER_TILE);
      if constexpr (!BURST) __builtin_amdgcn_sched_barrier(0);   // one copy between two MFMAs
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// One K tile with two fragment sets (LEAN tiles).  On entry x0 holds group 0
// of tile kt.  The MFMAs of group 0 run while group 1 of the same tile is read
// into x1; then the MFMAs of group 1 run while group 0 of tile kt + 1 is read
// back into x0, and the copies of tile kt + STAGES - 1 go out among the last of
// them.  The wait and barrier for tile kt + 1 come first, as in sdma_tile; past
// the barrier every wave has also read all of stage (kt - 1) % STAGES (its
// second group during tile kt - 1), which those copies refill.
template <class T, bool STEADY>
__device__ __forceinline__ void sdma_tile2(const SgemmArgs& p, f32x16 (&acc)[T::FM][T::FN],
                                           int kt, int ktiles, SFrags<T>& x0, SFrags<T>& x1,
                                           const uint8_t* lds, uint32_t lds_base,
                                           const SDmaPlan<T>& plan, const float* a_tile,
                                           const float* b_tile, int wave, int wm, int wn,
                                           int lane) {
  constexpr int NM = 4 * T::FM * T::FN;            // MFMAs per group
  constexpr int NR = T::FM + 4 * T::FN;            // LDS reads per group
  constexpr int PRE = 2;
  constexpr int R0 = (NR + NM - PRE - 1) / (NM - PRE);
  constexpr int TAIL = NM - T::LOADS_PER_TILE;
  constexpr int R1 = (NR + TAIL - 1) / TAIL;
  static_assert(TAIL >= NR / 2 && TAIL >= 1, "enough MFMAs to spread the reads over");
  smfma<T>(acc, x0, 0);
  smfma<T>(acc, x0, 1);
  if constexpr (STEADY) {
    wait_vmcnt<(T::STAGES - 3) * T::LOADS_PER_TILE>();
  } else {
    const int left = ktiles - 2 - kt;
    swait_tiles<T>(left < 0 ? 0 : (left < T::STAGES - 3 ? left : T::STAGES - 3));
  }
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  const uint8_t* cur = lds + (kt % T::STAGES) * T::STAGE_BYTES;
  const uint8_t* next = lds + ((kt + 1) % T::STAGES) * T::STAGE_BYTES;
  sload_frags<T>(x1, cur, 1, wm, wn, lane);
#pragma unroll
  for (int x = PRE; x < NM; ++x) smfma<T>(acc, x0, x);
#pragma unroll
  for (int x = 0; x < NM - PRE; ++x) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, R0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int kt_issue = kt + T::STAGES - 1;
  const bool issue = STEADY || kt_issue < ktiles;
  const uint32_t st_issue = lds_base + (kt_issue % T::STAGES) * T::STAGE_BYTES;
  sload_frags<T>(x0, next, 0, wm, wn, lane);
#pragma unroll
  for (int x = 0; x < TAIL; ++x) smfma<T>(acc, x1, x);
#pragma unroll
  for (int x = 0; x < TAIL; ++x) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, R1, 1);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int x = 0; x < T::LOADS_PER_TILE; ++x) {
    smfma<T>(acc, x1, TAIL + x);
    if (issue) sdma_issue<T>(p, plan, a_tile, b_tile, kt_issue, st_issue, wave, x);
    __builtin_amdgcn_sched_barrier(0);   // one copy between two MFMAs
  }
  __builtin_amdgcn_sched_barrier(0);
}

// The last K - k0 < 32 values of k on a ragged K: one 16-wide K tile at a time
// through stage STAGES - 1, filled with bounds-checked loads and plain LDS
// stores in the layout the copies produce (zeros for k >= K, clamped rows and
// columns as in SDmaPlan), then the MFMAs of that tile.  TAIL_FIRST tiles call
// it before the main loop, right after the prologue's copies are issued (that
// stage is then free), so the latency of these loads overlaps theirs; at the
// end of the K loop it was exposed (1000x3000x777 took longer than the same
// product with K = 800).  The main loop's first copy into that stage goes out
// after the first K tile's barrier, which a wave reaches only after its MFMAs
// here have consumed their fragments.  The other tiles call it after the main
// loop, behind a barrier.
template <class T>
__device__ __forceinline__ void sdma_k_tail(const SgemmArgs& p,
                                                  f32x16 (&acc)[T::FM][T::FN], uint8_t* lds,
                                                  int k0, int m0, int n0, int wm, int wn,
                                                  int lane) {
  uint8_t* const st = lds + (T::STAGES - 1) * T::STAGE_BYTES;
  const int tid = threadIdx.x;
  for (int kb = k0; kb < p.K; kb += T::BK) {
    if (kb > k0) lds_barrier();   // every wave is done reading the previous tail tile
    // A: BM rows x 4 chunks of 4 k.
    for (int c = tid; c < T::BM * 4; c += T::THREADS) {
      const int r = c / 4, chunk = c % 4;
      const int row = m0 + r < p.M ? m0 + r : p.M - 1;
      const int k = kb + 4 * chunk;
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = k + e < p.K ? p.A[(size_t)row * p.lda + k + e] : 0.0f;
      *reinterpret_cast<f32x4*>(st + r * 64 + 16 * (chunk ^ row64_swizzle(r))) = v;
    }
    // B: 16 rows of k x BN / 4 chunks of 4 columns.
    for (int c = tid; c < T::BK * (T::BN / 4); c += T::THREADS) {
      const int kr = c / (T::BN / 4), cc = 4 * (c % (T::BN / 4));
      const int k = kb + kr;
      const int col = n0 + cc < p.nb ? n0 + cc : p.nb - 4;
      f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
      if (k < p.K) v = *reinterpret_cast<const f32x4*>(p.B + (size_t)k * p.ldb + col);
      *reinterpret_cast<f32x4*>(st + T::A_BYTES + T::b_row(kr) + 4 * cc) = v;
    }
    lds_barrier();
    SFrags<T> f;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      sload_frags<T>(f, st, g, wm, wn, lane);
#pragma unroll
      for (int x = 0; x < 4 * T::FM * T::FN; ++x) smfma<T>(acc, f, x);
    }
  }
}

template <class T, bool SPLIT, bool EDGE>
__global__ void __launch_bounds__(T::THREADS) __attribute__((amdgpu_waves_per_eu(T::WAVES_PER_SIMD)))
sgemm_dma_kernel(SgemmArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[T::STAGES * T::STAGE_BYTES];
  if constexpr (SPLIT) {
    // This workgroup's K chunk (a multiple of 2 BK): shift A and B, shorten K.
    const int kbeg = blockIdx.y * p.k_chunk;
    const int klen = p.K - kbeg < p.k_chunk ? p.K - kbeg : p.k_chunk;
    p.A += kbeg;
    p.B += (size_t)kbeg * p.ldb;
    p.K = klen;
  }

  int tile_m, tile_n;
  tile_of_workgroup(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tile_m, tile_n);
  const int m0 = tile_m * T::BM;
  const int n0 = tile_n * T::BN;
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wm = wave / T::WAVES_N;
  const int wn = wave % T::WAVES_N;
  const uint32_t lds_base = lds_offset(lds);
  // Naming an accumulation register makes the compiler keep the accumulators in
  // that file (the MFMA form with AGPR sources and results), which leaves the
  // VGPR file to the fragments the LDS reads return: 0.4 % fewer main-loop
  // cycles at 4096^3 than accumulating in VGPRs.  (The 128-row tile would spill
  // with the register file split in two halves, so it keeps the VGPR form.)
  if constexpr (T::BM == 256) asm volatile("" ::: "a0");

  f32x16 acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Tile kt lives in stage kt % STAGES; its copies are issued during tile
  // kt - STAGES + 1 (the prologue issues the first STAGES - 1).  The loop covers
  // the largest multiple of 2 BK in K, two tiles per trip, so the fragment sets
  // alternate; on a ragged K (EDGE only) sdma_k_tail adds the rest.
  const int ktiles = EDGE ? (p.K / (2 * T::BK)) * 2 : p.K / T::BK;
  const float* a_tile = p.A + (size_t)m0 * p.lda;
  const float* b_tile = p.B + n0;
  const SDmaPlan<T> plan(p, wave, lane, m0, n0);
  // C ahead of the copies (PRE_C): row and column clamped into the matrix, so the
  // loads are unconditional; values outside are never stored.  Being the oldest
  // loads, they are complete by the first copy wait (loads finish in issue order).
  float cpre[T::PRE_C ? 16 * T::FM * T::FN : 1];
  if constexpr (T::PRE_C && !SPLIT) {
    if (p.beta != 0.0f) {
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
          const int col = n0 + wn * T::WTN + j * 32 + lane % 32;
          const int cc = col < p.N ? col : p.N - 1;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm * T::WTM + i * 32 + mfma32_row(r, lane);
            cpre[(i * T::FN + j) * 16 + r] = p.C[(size_t)(row < p.M ? row : p.M - 1) * p.ldc + cc];
          }
        }
    }
  }
  SFrags<T> f0, f1, f2, f3;
#pragma unroll
  for (int st = 0; st < T::STAGES - 1; ++st)
    if (st < ktiles) {
#pragma unroll
      for (int x = 0; x < T::LOADS_PER_TILE; ++x)
        sdma_issue<T>(p, plan, a_tile, b_tile, st, lds_base + st * T::STAGE_BYTES, wave, x);
    }
  if constexpr (EDGE && T::TAIL_FIRST) {
    if (ktiles * T::BK < p.K)
      sdma_k_tail<T>(p, acc, lds, ktiles * T::BK, m0, n0, wm, wn, lane);
  }
  if (ktiles > 0) {
    swait_tiles<T>(ktiles - 1 < T::STAGES - 2 ? ktiles - 1 : T::STAGES - 2);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    sload_frags<T>(f0, lds, 0, wm, wn, lane);
    if constexpr (!T::LEAN) sload_frags<T>(f1, lds, 1, wm, wn, lane);
  }
  int kt = 0;
  if constexpr (T::LEAN) {
    // One tile per trip: each tile leaves the next tile's first group in f0.
    for (; kt + T::STAGES - 1 < ktiles; ++kt)
      sdma_tile2<T, true>(p, acc, kt, ktiles, f0, f1, lds, lds_base, plan, a_tile, b_tile, wave,
                          wm, wn, lane);
    for (; kt < ktiles; ++kt)
      sdma_tile2<T, false>(p, acc, kt, ktiles, f0, f1, lds, lds_base, plan, a_tile, b_tile, wave,
                           wm, wn, lane);
  } else if constexpr (T::PAIR) {
    // Two tiles per trip, the barrier in the first; steady while tile kt + 4 exists.
    for (; kt + T::STAGES < ktiles; kt += 2) {
      sdma_tile_pair<T, true, true>(p, acc, kt, ktiles, f0, f1, f2, f3, lds, lds_base, plan,
                                    a_tile, b_tile, wave, wm, wn, lane);
      sdma_tile_pair<T, true, false>(p, acc, kt + 1, ktiles, f2, f3, f0, f1, lds, lds_base, plan,
                                     a_tile, b_tile, wave, wm, wn, lane);
    }
    for (; kt < ktiles; kt += 2) {
      sdma_tile_pair<T, false, true>(p, acc, kt, ktiles, f0, f1, f2, f3, lds, lds_base, plan,
                                     a_tile, b_tile, wave, wm, wn, lane);
      sdma_tile_pair<T, false, false>(p, acc, kt + 1, ktiles, f2, f3, f0, f1, lds, lds_base,
                                      plan, a_tile, b_tile, wave, wm, wn, lane);
    }
  } else {
    for (; kt + T::STAGES < ktiles; kt += 2) {
      sdma_tile<T, true>(p, acc, kt, ktiles, f0, f1, f2, f3, lds, lds_base, plan, a_tile, b_tile,
                         wave, wm, wn, lane);
      sdma_tile<T, true>(p, acc, kt + 1, ktiles, f2, f3, f0, f1, lds, lds_base, plan, a_tile,
                         b_tile, wave, wm, wn, lane);
    }
    for (; kt < ktiles; kt += 2) {
      sdma_tile<T, false>(p, acc, kt, ktiles, f0, f1, f2, f3, lds, lds_base, plan, a_tile, b_tile,
                          wave, wm, wn, lane);
      sdma_tile<T, false>(p, acc, kt + 1, ktiles, f2, f3, f0, f1, lds, lds_base, plan, a_tile,
                          b_tile, wave, wm, wn, lane);
    }
  }
  if constexpr (EDGE && !T::TAIL_FIRST) {
    if (ktiles * T::BK < p.K) {
      lds_barrier();   // every wave is done reading the stages
      sdma_k_tail<T>(p, acc, lds, ktiles * T::BK, m0, n0, wm, wn, lane);
    }
  }
  if constexpr (SPLIT) {
    // Raw partial sums into this K chunk's slice of the workspace.
    float* W = p.ws + (size_t)blockIdx.y * p.M * p.N;
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
        const int col = n0 + wn * T::WTN + j * 32 + lane % 32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * T::WTM + i * 32 + mfma32_row(r, lane);
          if (!EDGE || (row < p.M && col < p.N)) W[(size_t)row * p.N + col] = acc[i][j][r];
        }
      }
    return;
  }
  const float* pre = T::PRE_C ? cpre : nullptr;
  if (EDGE && (m0 + T::BM > p.M || n0 + T::BN > p.N))
    sgemm_store<T, true>(p, acc, m0 + wm * T::WTM, n0 + wn * T::WTN, lane, pre);
  else
    sgemm_store<T, false>(p, acc, m0 + wm * T::WTM, n0 + wn * T::WTN, lane, pre);
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
// 32 x 32 from 16x16x4 MFMA blocks, 4 waves of 16 x 16, K step 32: small outputs,
// where the per-wave MFMA chain (K / 4 blocks) sets the time.
using TileTiny = SgemmTile<32, 32, 32, 2, 2, 2, MfmaF16x16>;
using TileLargeK32 = SgemmTile<256, 256, 32, 2, 2>;  // as TileLarge, half the barriers
using TileTall = SgemmTile<128, 256, 16, 2, 2, 2>;   // 4 waves, 64 x 128 each, 2 workgroups/CU
// The same two shapes built from 16x16x4 MFMA blocks.
using TileLarge16 = SgemmTile<256, 256, 16, 2, 2, 1, MfmaF16x16>;
using TileTall16 = SgemmTile<128, 256, 16, 2, 2, 2, MfmaF16x16>;
// Direct-to-LDS: 256 x 256, 4 stages of 32.5 KiB, one workgroup per CU / 128 x 256,
// 3 stages of 24.5 KiB, two workgroups per CU.
using SDmaLarge = SDmaTile<256, 256, 4, 1>;
using SDmaTall = SDmaTile<128, 256, 3, 2, 2, 2, false, true>;
// 256 x 256 with eight waves (2 x 4, each 128 x 64), two per SIMD, one barrier per
// two K tiles (0.2 - 0.4 % faster than one per tile at 4096^3 and 8192^3).
using SDmaEight = SDmaTile<256, 256, 4, 2, 2, 4, false, false, true>;
// 128 x 128 with four waves of 64 x 64, 4 stages of 16.5 KiB, two workgroups per CU:
// outputs with too few 256 x 256 tiles to fill the CUs.
using SDmaSmall = SDmaTile<128, 128, 4, 2, 2, 2, false, false, true>;
// 64 x 64 with four waves of 32 x 32, 4 stages of 8.5 KiB, up to four workgroups
// per CU: small and mid-size outputs (about 100 to 1000 tiles), spread evenly.
using SDmaMini = SDmaTile<64, 64, 4, 4, 2, 2, false, false, true>;

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static_assert(TileLarge::BK == sgemm_tile_bk(0) && TileMedium::BK == sgemm_tile_bk(1) &&
                  TileSmall::BK == sgemm_tile_bk(2) && TileLargeK32::BK == sgemm_tile_bk(3) &&
                  TileTiny::BK == sgemm_tile_bk(12) && TileTiny::BM == sgemm_tile_bm(12) &&
                  TileTiny::BN == sgemm_tile_bn(12) &&
                  TileTall::BK == sgemm_tile_bk(4) && TileLarge16::BK == sgemm_tile_bk(5) &&
                  TileTall16::BK == sgemm_tile_bk(6) && TileLarge16::BM == sgemm_tile_bm(5) &&
                  TileLarge16::BN == sgemm_tile_bn(5) && TileTall16::BM == sgemm_tile_bm(6) &&
                  TileTall16::BN == sgemm_tile_bn(6) && TileTall::BM == sgemm_tile_bm(4) &&
                  2 * SDmaLarge::BK == sgemm_tile_bk(7) && 2 * SDmaTall::BK == sgemm_tile_bk(8) &&
                  SDmaLarge::BM == sgemm_tile_bm(7) && SDmaLarge::BN == sgemm_tile_bn(7) &&
                  SDmaTall::BM == sgemm_tile_bm(8) && SDmaTall::BN == sgemm_tile_bn(8) &&
                  SDmaEight::BM == sgemm_tile_bm(9) && SDmaEight::BN == sgemm_tile_bn(9) &&
                  2 * SDmaEight::BK == sgemm_tile_bk(9) && SDmaSmall::BM == sgemm_tile_bm(10) &&
                  SDmaSmall::BN == sgemm_tile_bn(10) && 2 * SDmaSmall::BK == sgemm_tile_bk(10) &&
                  SDmaMini::BM == sgemm_tile_bm(11) && SDmaMini::BN == sgemm_tile_bn(11) &&
                  2 * SDmaMini::BK == sgemm_tile_bk(11),
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
  p.group_m = swizzle_group(group_m);
  p.k_chunk = plan.k_chunk;
  p.ws = ws;
  p.a_vec = c.lda % 4 == 0 && aligned16(c.A);
  p.b_vec = c.ldb % 4 == 0 && aligned16(c.B);
  p.nb = c.N;
  const bool split = plan.splits > 1;
  const dim3 grid(p.tiles_m * p.tiles_n, split ? plan.splits : 1), block(T::THREADS);
  if (c.padded) {
    // Copies padded to whole tiles: every load is in range, only C is checked.
    if (c.K % T::BK != 0 || c.lda % 4 != 0 || c.ldb % 4 != 0 || !aligned16(c.A) ||
        !aligned16(c.B) || c.ldb < p.tiles_n * T::BN || c.lda < c.K)
      return hipErrorInvalidValue;
    if (split) {
      hipLaunchKernelGGL((sgemm_mfma_kernel<T, false, true, true>), grid, block, 0, s, p);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      return launch_reduce(c, plan.splits, ws, s);
    }
    hipLaunchKernelGGL((sgemm_mfma_kernel<T, false, false, true>), grid, block, 0, s, p);
    return hipGetLastError();
  }
  const bool edge = !(c.M % T::BM == 0 && c.N % T::BN == 0 && c.K % T::BK == 0 &&
                      c.lda % 4 == 0 && c.ldb % 4 == 0 && aligned16(c.A) && aligned16(c.B));
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

// The direct-to-LDS kernels copy 16-byte chunks of B, so rows of B must start
// on 16-byte boundaries and each row of B must be readable in whole chunks up
// to N (nb a multiple of 4); A is copied in 16-byte chunks where its rows start
// on 16-byte boundaries, else 4 bytes at a time (rows of A on 4-byte
// boundaries).  The per-lane copy offsets are 32-bit.  Whole tiles with K a
// multiple of 32 run the unchecked instantiation.
static bool a_rows16(const SgemmCall& c) { return c.lda % 4 == 0 && aligned16(c.A); }
static bool direct_operands_ok(const SgemmCall& c) {
  const int nb = readable_cols(c.nb, c.N);
  return (reinterpret_cast<uintptr_t>(c.A) & 3u) == 0 && c.ldb % 4 == 0 && nb % 4 == 0 &&
         nb >= c.N && nb <= c.ldb && aligned16(c.B) &&
         (int64_t)c.lda * 256 * 4 < (int64_t(1) << 31) &&
         (int64_t)c.ldb * 16 * 4 < (int64_t(1) << 31);
}

template <class T>
static bool sdma_fits(const SgemmCall& c) {
  static_assert(T::BM <= 256 && T::BK == 16, "direct_operands_ok's offset bounds");
  return direct_operands_ok(c);
}

template <class T>
static bool sdma_whole(const SgemmCall& c) {
  return c.M % T::BM == 0 && c.N % T::BN == 0 && c.K % (2 * T::BK) == 0;
}

template <class T, bool EDGE>
static hipError_t launch_sdma_kernel(const SgemmCall& c, const SgemmPlan& plan, const SgemmArgs& p,
                                     float* ws, hipStream_t s) {
  if (plan.splits > 1) {
    hipLaunchKernelGGL((sgemm_dma_kernel<T, true, EDGE>), dim3(p.tiles_m * p.tiles_n, plan.splits),
                       dim3(T::THREADS), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_reduce(c, plan.splits, ws, s);
  }
  hipLaunchKernelGGL((sgemm_dma_kernel<T, false, EDGE>), dim3(p.tiles_m * p.tiles_n),
                     dim3(T::THREADS), 0, s, p);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_sdma_as(const SgemmCall& c, const SgemmPlan& plan, int group_m,
                                 float* ws, hipStream_t s) {
  if (!sdma_fits<T>(c)) return hipErrorInvalidValue;
  if (plan.splits > 1 && (ws == nullptr || plan.k_chunk % (2 * T::BK) != 0))
    return hipErrorInvalidValue;
  SgemmArgs p;
  p.M = c.M; p.N = c.N; p.K = c.K;
  p.alpha = c.alpha; p.beta = c.beta;
  p.A = c.A; p.lda = c.lda; p.B = c.B; p.ldb = c.ldb; p.C = c.C; p.ldc = c.ldc;
  p.tiles_m = (c.M + T::BM - 1) / T::BM;
  p.tiles_n = (c.N + T::BN - 1) / T::BN;
  p.group_m = swizzle_group(group_m);
  p.k_chunk = plan.splits > 1 ? plan.k_chunk : c.K;
  p.ws = ws;
  p.a_vec = p.b_vec = 1;
  p.nb = readable_cols(c.nb, c.N);
  if (sdma_whole<T>(c)) return launch_sdma_kernel<T, false>(c, plan, p, ws, s);
  return launch_sdma_kernel<T, true>(c, plan, p, ws, s);
}

// Tile T, copying A 4 bytes at a time where its rows are not 16-byte aligned.
template <class T>
static hipError_t launch_sdma(const SgemmCall& c, const SgemmPlan& plan, int group_m, float* ws,
                              hipStream_t s) {
  if (a_rows16(c)) return launch_sdma_as<T>(c, plan, group_m, ws, s);
  return launch_sdma_as<typename T::WithADw>(c, plan, group_m, ws, s);
}

int sgemm_resolve_tile(int tile, int M, int N, int K, int splits, bool operands_ok) {
  // The direct-to-LDS kernels need rows of B on 16-byte boundaries (A on 4-byte
  // ones) and B readable in whole 4-float chunks (any M, N and K otherwise: ragged edges and
  // a ragged K run a bounds-checked instantiation); otherwise the
  // register-staged 128 x 256 kernel (the best of those for large outputs) runs,
  // or for the 64 x 64 tile its register-staged twin.
  (void)M; (void)N; (void)K; (void)splits;
  if (tile >= 7 && tile <= 11 && !operands_ok) return tile == 11 ? 2 : 4;
  return tile;
}

static hipError_t launch_wave_ksplit(const SgemmCall& c, hipStream_t s) {
  SgemmArgs p;
  p.M = c.M; p.N = c.N; p.K = c.K;
  p.alpha = c.alpha; p.beta = c.beta;
  p.A = c.A; p.lda = c.lda; p.B = c.B; p.ldb = c.ldb; p.C = c.C; p.ldc = c.ldc;
  p.tiles_m = (c.M + kWksTile - 1) / kWksTile;
  p.tiles_n = (c.N + kWksTile - 1) / kWksTile;
  p.group_m = 1;
  p.k_chunk = c.K;
  p.ws = nullptr;
  p.a_vec = c.lda % 4 == 0 && aligned16(c.A);
  p.b_vec = 0;
  p.nb = c.N;
  // Eight waves: at 256^3 as fast as four (3.1 us) and up to 17 % faster on
  // longer K or ragged shapes (64 x 512 x 1024: 4.9 vs 5.2 us; 200 x 120 x 2000:
  // 8.3 vs 10.0), each wave's MFMA chain and load round trip being shorter.
  constexpr int kWaves = 8;
  const bool whole = c.M % kWksTile == 0 && c.N % kWksTile == 0 &&
                     c.K % (kWksSpan / kWaves) == 0 && p.a_vec;
  if (whole)
    hipLaunchKernelGGL((sgemm_wave_ksplit_kernel<true, kWaves>), dim3(p.tiles_m * p.tiles_n),
                       dim3(kWaves * kWave), 0, s, p);
  else
    hipLaunchKernelGGL((sgemm_wave_ksplit_kernel<false, kWaves>), dim3(p.tiles_m * p.tiles_n),
                       dim3(kWaves * kWave), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_sgemm(const SgemmCall& c, const SgemmPlan& plan, float* ws, hipStream_t s) {
  if (plan.splits > 1 && ws == nullptr) return hipErrorInvalidValue;
  switch (sgemm_resolve_tile(plan.tile, c.M, c.N, c.K, plan.splits, direct_operands_ok(c))) {
    case 0: return launch_tile<TileLarge>(c, plan, 4, ws, s);
    case 1: return launch_tile<TileMedium>(c, plan, 8, ws, s);
    case 2: return launch_tile<TileSmall>(c, plan, 8, ws, s);
    case 3: return launch_tile<TileLargeK32>(c, plan, 4, ws, s);
    case 4: return launch_tile<TileTall>(c, plan, 8, ws, s);
    case 5: return launch_tile<TileLarge16>(c, plan, 4, ws, s);
    case 6: return launch_tile<TileTall16>(c, plan, 8, ws, s);
    case 7: return launch_sdma<SDmaLarge>(c, plan, 4, ws, s);
    case 8: return launch_sdma<SDmaTall>(c, plan, 8, ws, s);
    case 9: return launch_sdma<SDmaEight>(c, plan, 4, ws, s);
    case 10: return launch_sdma<SDmaSmall>(c, plan, 8, ws, s);
    case 11: return launch_sdma<SDmaMini>(c, plan, 8, ws, s);
    case 12: return launch_tile<TileTiny>(c, plan, 8, ws, s);
    case 13: return launch_wave_ksplit(c, s);
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
