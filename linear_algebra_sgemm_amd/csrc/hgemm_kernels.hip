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
#include "dma_common.h"
#include "gemm_common.h"
#include "gemm_launch.h"

namespace lasg {

// The 16-bit input formats: IEEE binary16 and bfloat16 share every load, LDS
// layout and transposing read; they differ in the MFMA and the output rounding.
struct EltF16 {
  typedef _Float16 vec8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  // fp32 -> binary16, round to nearest even (v_cvt_f16_f32)
  static __device__ __forceinline__ uint16_t bits(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
};

struct EltBF16 {
  typedef __bf16 vec8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // fp32 -> bfloat16, round to nearest even (v_cvt_pk_bf16_f32)
  static __device__ __forceinline__ uint16_t bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
  }
};

template <class E_, int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_>
struct HgemmTile {
  using E = E_;
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
  // Direct-to-LDS kernels: columns of each row of B that may be read (a multiple
  // of 8, at least N).
  int nb;
  // Split-K (register-staged kernel): workgroup row blockIdx.y covers K range
  // [y * k_chunk, min(K, (y + 1) * k_chunk)) and writes its raw FP32 partial to
  // ws + y * M * N (M x N, row stride N).
  int k_chunk;
  float* ws;
  // K-split kernel: rows of A 16-byte aligned (lda a multiple of 8, A aligned).
  int a_vec;
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
// Since 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)), this is x / (1 + exp(-2u)),
// computed as x * rcp(1 + 2^t) with t = -2 u log2(e): the hardware base-2
// exponential and reciprocal (about 1 ulp each, far inside the 16-bit output's
// rounding) instead of a full-precision division, which costs about ten
// instructions per element in the epilogue.  It tends to x for large positive x
// and to -0 for large negative x.
__device__ __forceinline__ float gelu_factor(float x) {
  const float k1 = 0.044715f;
  const float c = -2.302208198f;   // -2 sqrt(2 / pi) log2(e)
  const float t = c * __builtin_fmaf(k1 * x, x * x, x);
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
}
__device__ __forceinline__ float gelu_tanh(float x) { return x * gelu_factor(x); }

// The activation of a call, chosen without a branch per element: x times
// gs * factor + (1 - gs), with gs = 1 (GELU: exactly x * factor) or gs = 0
// (identity: exactly x * 1; the factor is finite).  A branch on the activation
// inside the element loops would be taken once per element.
struct Activation {
  float gs, g0;
  __device__ __forceinline__ explicit Activation(int act)
      : gs(act == 1 ? 1.0f : 0.0f), g0(act == 1 ? 0.0f : 1.0f) {}
  __device__ __forceinline__ float operator()(float x) const {
    return x * __builtin_fmaf(gs, gelu_factor(x), g0);
  }
};

template <class T, bool EDGE, bool SPLIT>
__global__ void __launch_bounds__(T::THREADS) hgemm_mfma_kernel(HgemmArgs p) {
  if constexpr (SPLIT) {
    // This workgroup's K chunk (a multiple of BK): shift A and B, shorten K.
    const int kbeg = blockIdx.y * p.k_chunk;
    const int klen = p.K - kbeg < p.k_chunk ? p.K - kbeg : p.k_chunk;
    p.A += kbeg;
    p.B += (size_t)kbeg * p.ldb;
    p.K = klen;
  }
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
      typedef typename T::E::vec8 vec8;
      vec8 af[T::FM], bf[T::FN];
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
        af[i] = *reinterpret_cast<const vec8*>(As + a_off + i * 32 * T::STRIDE + 16 * s);
#pragma unroll
      for (int j = 0; j < T::FN; ++j)
        bf[j] = *reinterpret_cast<const vec8*>(Bt + b_off + j * 32 * T::STRIDE + 16 * s);
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
          acc[i][j] = T::E::mfma(af[i], bf[j], acc[i][j]);
    }

    if (more) st.store(odd ? As0 : As1, odd ? Bt0 : Bt1, tid);
    __syncthreads();
  }

  if constexpr (SPLIT) {
    // Raw partial sums into this K chunk's slice of the workspace.
    float* W = p.ws + (size_t)blockIdx.y * p.M * p.N;
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
      const int col = n0 + wn * T::WTN + j * 32 + l32;
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * T::WTM + i * 32 + mfma32_row(r, lane);
          if (EDGE && (row >= p.M || col >= p.N)) continue;
          W[(size_t)row * p.N + col] = acc[i][j][r];
        }
    }
    return;
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
        p.C[(size_t)row * p.ldc + col] = T::E::bits(x);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Direct-to-LDS variant for whole tiles (M % BM == N % BN == K % BK == 0, A and
// B rows 16-byte aligned).
//
// Loads go straight from global memory into LDS with global_load_lds_dwordx4
// (lane l of one instruction writes its 16 bytes at base + 16 l), so no staging
// registers are needed and STAGES - 1 K tiles can be in flight at once.  Each
// instruction chooses the global chunk of every LDS slot, which sets the layout:
//  * A is stored row-major (64-byte rows of one K tile) with the four 16-byte
//    chunks of each row permuted by a_swizzle so that the fragment reads (one
//    chunk from each of 32 rows) do not collide in the banks.  One load moves 16
//    whole rows: the memory path serves about one cache line every two clocks
//    per CU, so loads must use the lines they touch in full.
//  * B, block (k-step s, half t, n-block jb) = 512 B: 32 chunks of 8 columns of
//    one row, in the order (h, cg, q, c2) so that lane l reads bytes [8l, 8l+8)
//    with ds_read_b64_tr_b16.  That instruction transposes inside groups of 16
//    lanes (lane 4a + b of a group receives element b of the rows loaded by
//    lanes a, a + 4, a + 8, a + 12), so lane l ends up with B[16 s + 8 h + 4 t +
//    e][32 jb + l % 32], e = 0..3: four consecutive k of its own column, the
//    operand layout the MFMA wants, without any transposition in registers.
// The MFMA is issued with the B fragment as its first operand and the A fragment
// as its second, which yields C^T blocks: lane l then holds four consecutive
// columns of one row of C and stores them with one 8-byte write.
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

template <class E_, int BM_, int BN_, int BK_, int STAGES_, int WAVES_PER_SIMD_ = 1,
          int WAVES_M_ = 2, int WAVES_N_ = 2>
struct HDmaTile {
  using E = E_;
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_;
  static constexpr int WAVES_PER_SIMD = WAVES_PER_SIMD_;   // waves sharing one SIMD
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, WAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = WAVES * kWave;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int KSTEPS = BK / 16;
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int B_BYTES = BK * BN * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int A_INSTR = A_BYTES / 1024;   // 1 KiB direct loads per stage
  static constexpr int B_INSTR = B_BYTES / 1024;
  static constexpr int A_PER_WAVE = A_INSTR / WAVES;
  static constexpr int B_PER_WAVE = B_INSTR / WAVES;
  static constexpr int LOADS_PER_TILE = A_PER_WAVE + B_PER_WAVE;   // per lane, counted by vmcnt
  static constexpr int A_CHUNKS_PER_ROW = BK / 8;                   // 16-byte chunks per A row

  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
  static_assert(BK % 16 == 0 && BN % 64 == 0, "k steps of 16; B loads cover 64 columns");
  static_assert(BK == 32, "the A chunk swizzle is laid out for rows of four 16-byte chunks");
  static_assert(A_INSTR % WAVES == 0 && B_INSTR % WAVES == 0, "loads split evenly over waves");
  static_assert(STAGES >= 2 && STAGES * STAGE_BYTES <= 160 * 1024, "stages must fit in LDS");
  static_assert((STAGES - 2) * LOADS_PER_TILE <= 63, "in-flight loads must fit vmcnt");
  static_assert(FM * FN * 16 <= 256 / WAVES_PER_SIMD, "accumulators must leave room for operands");
};

// Chunk permutation of A row r in LDS (64-byte rows: see row64_swizzle).
template <class T>
__device__ __forceinline__ int a_swizzle(int r) {
  static_assert(T::A_CHUNKS_PER_ROW == 4, "rows of four 16-byte chunks");
  return row64_swizzle(r);
}


// Global address of the 16-byte chunk that lane `lane` of direct load `v` (0 ..
// LOADS_PER_TILE - 1) of wave `wave` copies, and the offset of its LDS slot
// inside one stage.  Rows of A past M - 1 read row M - 1 and 8-column chunks of
// B at or past nb (the readable width, a multiple of 8) read the chunk at
// nb - 8, so on a tile that crosses the bottom or right edge every copy stays
// inside the matrices; those rows and columns of the tile are never stored.  `k_first` / `k_step` give the
// k of element e of the chunk: k_first + k_step e (8 consecutive k of one A row,
// or one k for the 8 columns of a B row).
template <class T>
__device__ __forceinline__ const uint16_t* hdma_source(const HgemmArgs& p, int m0, int n0, int k0,
                                                       int v, int wave, int lane,
                                                       uint32_t& stage_offset, int& k_first,
                                                       int& k_step) {
  if (v < T::A_PER_WAVE) {
    // A stage: row-major rows of BK halves with the 16-byte chunks of row r
    // permuted by a_swizzle(r); one load = 1 KiB = whole rows, so every cache
    // line it touches is read over its full width of the tile.
    const int ia = wave * T::A_PER_WAVE + v;
    const int r = ia * (1024 / (2 * T::BK)) + lane / T::A_CHUNKS_PER_ROW;
    const int slot = lane % T::A_CHUNKS_PER_ROW;
    stage_offset = ia * 1024;
    const int chunk = slot ^ a_swizzle<T>(r);
    const int row = m0 + r < p.M ? m0 + r : p.M - 1;
    k_first = k0 + 8 * chunk;
    k_step = 1;
    return p.A + (size_t)row * p.lda + k0 + 8 * chunk;
  }
  const int ibb = wave * T::B_PER_WAVE + (v - T::A_PER_WAVE);   // = (s * 2 + t) * (BN / 64) + jp
  const int jp = ibb % (T::BN / 64);
  const int st = ibb / (T::BN / 64);
  const int s = st / 2, t = st % 2;
  const int jb = 2 * jp + lane / 32;
  const int pidx = lane % 32;                     // ((h * 2 + cg) * 4 + q) * 2 + c2
  const int c2 = pidx & 1, q = (pidx >> 1) & 3, cg = (pidx >> 3) & 1, h = pidx >> 4;
  stage_offset = T::A_BYTES + ibb * 1024;
  const int row = k0 + 16 * s + 8 * h + 4 * t + q;
  const int col0 = n0 + 32 * jb + 16 * cg + 8 * c2;
  const int col = col0 < p.nb ? col0 : p.nb - 8;
  k_first = row;
  k_step = 0;
  return p.B + (size_t)row * p.ldb + col;
}

// The direct loads of one K tile as (wave-uniform base, per-lane offset) pairs:
// load v reads A at a_base(k0) + off[v] (v < A_PER_WAVE) or B at b_base(k0) +
// off[v], with a_base(k0) = A + m0 lda + k0 and b_base(k0) = B + k0 ldb + n0
// (elements).  The offsets do not depend on k0; they are the addresses of
// hdma_source minus the base, in bytes.
template <class T>
struct HDmaOffsets {
  uint32_t off[T::LOADS_PER_TILE];
  __device__ __forceinline__ HDmaOffsets(const HgemmArgs& p, int wave, int lane, int m0, int n0) {
#pragma unroll
    for (int v = 0; v < T::LOADS_PER_TILE; ++v) {
      uint32_t unused_slot;
      int unused_k, unused_step;
      const uint16_t* src = hdma_source<T>(p, m0, n0, 0, v, wave, lane, unused_slot, unused_k,
                                           unused_step);
      const uint16_t* base = v < T::A_PER_WAVE ? p.A + (size_t)m0 * p.lda : p.B + n0;
      off[v] = (uint32_t)((src - base) * sizeof(uint16_t));
    }
  }
};

template <class T>
__device__ __forceinline__ uint32_t hdma_lds_slot(int v, int wave) {
  if (v < T::A_PER_WAVE) return (wave * T::A_PER_WAVE + v) * 1024;
  return T::A_BYTES + (wave * T::B_PER_WAVE + (v - T::A_PER_WAVE)) * 1024;
}

// Issue the direct loads of K tile `kt` into the stage at LDS byte address `stage`.
template <class T>
__device__ __forceinline__ void hdma_issue_tile(const HgemmArgs& p, const HDmaOffsets<T>& o,
                                                const uint16_t* a_tile, const uint16_t* b_tile,
                                                int kt, uint32_t stage, int wave) {
  const uint16_t* a = a_tile + kt * T::BK;
  const uint16_t* b = b_tile + (size_t)kt * T::BK * p.ldb;
#pragma unroll
  for (int v = 0; v < T::LOADS_PER_TILE; ++v)
    dma16_sbase_u(v < T::A_PER_WAVE ? a : b, o.off[v], stage + hdma_lds_slot<T>(v, wave));
}

// MFMA operand fragments of one k step of one wave.
template <class T>
struct HFrags {
  typename T::E::vec8 a[T::FM];
  typename T::E::vec8 b[T::FN];
};

template <class T>
__device__ __forceinline__ void hload_frags(HFrags<T>& f, const uint8_t* stage, int s, int wm,
                                            int wn, int lane) {
  const uint8_t* As = stage;
  const uint8_t* Bs = stage + T::A_BYTES;
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
    const int r = (wm * T::FM + i) * 32 + lane % 32;
    const int chunk = 2 * s + lane / 32;
    f.a[i] = *reinterpret_cast<const typename T::E::vec8*>(As + r * (2 * T::BK) +
                                             16 * (chunk ^ a_swizzle<T>(r)));
  }
#pragma unroll
  for (int j = 0; j < T::FN; ++j) {
    const int jb = wn * T::FN + j;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t*)(Bs + ((s * 2 + 0) * (T::BN / 32) + jb) * 512 + 8 * lane));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t*)(Bs + ((s * 2 + 1) * (T::BN / 32) + jb) * 512 + 8 * lane));
    const s16x4 both[2] = {lo, hi};
    f.b[j] = __builtin_bit_cast(typename T::E::vec8, both);
  }
}

template <class T>
__device__ __forceinline__ void hmfma(f32x16 (&acc)[T::FN][T::FM], const HFrags<T>& f, int idx) {
  const int j = idx / T::FM, i = idx % T::FM;
  acc[j][i] = T::E::mfma(f.b[j], f.a[i], acc[j][i]);
}

// Wait until at most `ahead` tiles of direct loads are still in flight.
template <class T>
__device__ __forceinline__ void wait_tiles_in_flight(int ahead) {
  static_assert(T::STAGES <= 5, "extend the cases below for deeper pipelines");
  if (ahead >= 3 && T::STAGES >= 5) {
    wait_vmcnt<(T::STAGES >= 5 ? 3 * T::LOADS_PER_TILE : 0)>();
  } else if (ahead >= 2 && T::STAGES >= 4) {
    wait_vmcnt<(T::STAGES >= 4 ? 2 * T::LOADS_PER_TILE : 0)>();
  } else if (ahead >= 1 && T::STAGES >= 3) {
    wait_vmcnt<(T::STAGES >= 3 ? T::LOADS_PER_TILE : 0)>();
  } else {
    wait_vmcnt<0>();
  }
}

// One K tile of the direct-to-LDS kernel: MFMAs on the fragments of tile kt (x0:
// k step 0, x1: k step 1, read during the previous tile), reads of tile kt + 1's
// fragments into y0 / y1, the wait for tile kt + 1 and the barrier, and the direct
// loads of tile kt + STAGES - 1.  After the last tile the wait is for nothing, and
// the reads hit a stage that is no longer used; their values are dropped.
// STEADY: the caller guarantees kt + STAGES - 1 < ktiles (the look-ahead tile
// exists), so the wait depth is fixed and the loads are issued unconditionally.
// Wait until at most N + extra vector-memory operations of this wave are
// outstanding: extra counts stores issued after the awaited copies (a previous
// tile's epilogue in the persistent kernel) and is one of 0, 8 or 16 there;
// any other value waits for everything, which is always safe.
template <int N>
__device__ __forceinline__ void wait_vmcnt_plus(int extra) {
  if (extra == 16)
    wait_vmcnt<N + 16>();
  else if (extra == 8)
    wait_vmcnt<N + 8>();
  else if (extra == 0)
    wait_vmcnt<N>();
  else
    wait_vmcnt<0>();
}

// `extra`: stores issued after this tile's awaited copies (see wait_vmcnt_plus;
// a literal 0 everywhere but the first two tiles of a persistent kernel's tile).
template <class T, bool STEADY>
__device__ __forceinline__ void hdma_tile(const HgemmArgs& p, f32x16 (&acc)[T::FN][T::FM], int kt,
                                          int ktiles, HFrags<T>& x0, HFrags<T>& x1,
                                          HFrags<T>& y0, HFrags<T>& y1, const uint8_t* lds,
                                          uint32_t lds_base, const HDmaOffsets<T>& dma,
                                          const uint16_t* a_tile, const uint16_t* b_tile,
                                          int wave, int wm, int wn, int lane, int extra = 0) {
  static_assert(T::KSTEPS == 2, "two k steps per tile");
  constexpr int NM = T::FM * T::FN;                  // MFMAs per k step
  constexpr int NR = T::FM + 2 * T::FN;              // LDS reads per k step
  constexpr int PRE = 2;                             // MFMAs issued before the barrier
  constexpr int R0 = (NR + NM - PRE - 1) / (NM - PRE);          // reads per MFMA, step 0
  // Direct loads issued at the end of step 0 (L0) and among step 1's MFMAs (L1):
  // all in step 1 unless a wave has as many loads as MFMAs per k step (a
  // 128x128 tile), then half in each.
  constexpr int L0 = NM - T::LOADS_PER_TILE >= 1 ? 0 : T::LOADS_PER_TILE / 2;
  constexpr int L1 = T::LOADS_PER_TILE - L0;
  constexpr int TAIL = NM - L1;                                 // MFMAs before the direct loads
  static_assert(NM > PRE && TAIL >= 1 && L1 <= NM, "enough MFMAs to hide behind");
  constexpr int R1 = (NR + TAIL - 1) / TAIL;                    // reads per MFMA, step 1
  // Two MFMAs first, so the matrix unit has work queued while the waves meet.
  hmfma<T>(acc, x0, 0);
  hmfma<T>(acc, x0, 1);
  if constexpr (STEADY) {
    if (extra != 0)
      wait_vmcnt_plus<(T::STAGES - 3) * T::LOADS_PER_TILE>(extra);
    else
      wait_vmcnt<(T::STAGES - 3) * T::LOADS_PER_TILE>();
  } else {
    const int left = ktiles - 2 - kt;    // tiles after kt + 1 that may stay in flight
    if (extra != 0)
      wait_vmcnt<0>();
    else
      wait_tiles_in_flight<T>(left < 0 ? 0 : (left < T::STAGES - 3 ? left : T::STAGES - 3));
  }
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  const uint8_t* next = lds + ((kt + 1) % T::STAGES) * T::STAGE_BYTES;
  // Step 0: the remaining MFMAs with the reads of the next tile's first k step.
  hload_frags<T>(y0, next, 0, wm, wn, lane);
#pragma unroll
  for (int x = PRE; x < NM; ++x) hmfma<T>(acc, x0, x);
#pragma unroll
  for (int x = 0; x < NM - PRE; ++x) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, R0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int kt_issue = kt + T::STAGES - 1;
  const bool issue = STEADY || kt_issue < ktiles;
  const uint32_t st_issue = lds_base + (kt_issue % T::STAGES) * T::STAGE_BYTES;
  const uint16_t* a_issue = a_tile + kt_issue * T::BK;
  const uint16_t* b_issue = b_tile + (size_t)kt_issue * T::BK * p.ldb;
  if constexpr (L0 > 0) {
#pragma unroll
    for (int x = 0; x < L0; ++x)
      if (issue)
        dma16_sbase_u(x < T::A_PER_WAVE ? a_issue : b_issue, dma.off[x],
                    st_issue + hdma_lds_slot<T>(x, wave));
    __builtin_amdgcn_sched_barrier(0);
  }
  // Step 1: the reads of the next tile's second k step with the first MFMAs, then
  // the direct loads of tile kt + STAGES - 1 with the rest.  Reading first leaves
  // the last LDS reads of the tile several MFMAs before its end, so they have
  // landed when the next tile waits for its fragments (the compiler's wait at the
  // top of the K loop is for all of them).
  if constexpr (2 * TAIL >= NR) {
    hload_frags<T>(y1, next, 1, wm, wn, lane);
#pragma unroll
    for (int x = 0; x < TAIL; ++x) hmfma<T>(acc, x1, x);
#pragma unroll
    for (int x = 0; x < TAIL; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, R1, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int x = L0; x < T::LOADS_PER_TILE; ++x) {
      hmfma<T>(acc, x1, TAIL + x - L0);
      if (issue)
        dma16_sbase_u(x < T::A_PER_WAVE ? a_issue : b_issue, dma.off[x],
                    st_issue + hdma_lds_slot<T>(x, wave));
      __builtin_amdgcn_sched_barrier(0);   // one copy between two MFMAs
    }
  } else {
    // Few MFMAs per k step (the 128 x 256 tile): loads first, so the reads are
    // not crowded into the last MFMAs' registers.
#pragma unroll
    for (int x = L0; x < T::LOADS_PER_TILE; ++x) {
      hmfma<T>(acc, x1, x - L0);
      if (issue)
        dma16_sbase_u(x < T::A_PER_WAVE ? a_issue : b_issue, dma.off[x],
                    st_issue + hdma_lds_slot<T>(x, wave));
      __builtin_amdgcn_sched_barrier(0);   // one copy between two MFMAs
    }
    hload_frags<T>(y1, next, 1, wm, wn, lane);
#pragma unroll
    for (int x = L1; x < NM; ++x) hmfma<T>(acc, x1, x);
#pragma unroll
    for (int x = 0; x < TAIL; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, R1, 1);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// The last K - k0 < 2 BK values of k on a ragged K, taken before the main loop:
// one BK-wide K tile at a time through stage STAGES - 1, which the prologue's
// copies leave free, filled chunk for chunk where the copies would put them --
// a 16-byte load where the chunk lies wholly below K, 2-byte loads and zeros
// for k >= K where it does not -- then the MFMAs of that tile.  Called by every
// wave right after the prologue's copies are issued, so the latency of these
// loads overlaps theirs (after the main loop it was exposed, with a 2-byte load
// per element and always two K tiles: 2048 x 2048 x 2040 took 23 % longer than
// 2048^3).  The main loop's first copy into that stage goes out after the first
// K tile's barrier, which a wave reaches only after its MFMAs here have
// consumed their fragments.
template <class T>
__device__ __forceinline__ void hdma_k_tail(const HgemmArgs& p, f32x16 (&acc)[T::FN][T::FM],
                                            uint8_t* lds, int k0, int m0, int n0, int wave,
                                            int wm, int wn, int lane) {
  uint8_t* const st = lds + (T::STAGES - 1) * T::STAGE_BYTES;
  for (int kb = k0; kb < p.K; kb += T::BK) {
    if (kb > k0) lds_barrier();   // every wave is done reading the previous tail tile
#pragma unroll
    for (int v = 0; v < T::LOADS_PER_TILE; ++v) {
      uint32_t slot;
      int k_first, k_step;
      const uint16_t* src = hdma_source<T>(p, m0, n0, kb, v, wave, lane, slot, k_first, k_step);
      u32x4 val;
      if (k_first + 7 * k_step < p.K) {
        val = *reinterpret_cast<const u32x4*>(src);
      } else {
        uint16_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = k_first + k_step * e < p.K ? src[e] : (uint16_t)0;
        val = __builtin_bit_cast(u32x4, h);
      }
      *reinterpret_cast<u32x4*>(st + slot + 16 * lane) = val;
    }
    lds_barrier();
    HFrags<T> f;
#pragma unroll
    for (int ks = 0; ks < T::KSTEPS; ++ks) {
      hload_frags<T>(f, st, ks, wm, wn, lane);
#pragma unroll
      for (int x = 0; x < T::FM * T::FN; ++x) hmfma<T>(acc, f, x);
    }
  }
}

// Bias of the wave's output columns, n-blocks j0 .. j0 + JB - 1: lane l needs,
// for n-block j and q = 0..3, columns 32 j + 8 q + 4 (l / 32) + 0..3 of the
// wave's tile (zero without a bias, and past N on a ragged tile).  All loads of
// a batch are issued before any value is used.
template <class T, bool EDGE, int JB>
__device__ __forceinline__ void hdma_load_bias(const HgemmArgs& p, float (&bias)[JB][4][4], int j0,
                                               int n0, int wn, int lane) {
#pragma unroll
  for (int jj = 0; jj < JB; ++jj)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = n0 + wn * T::WTN + 32 * (j0 + jj) + 8 * q + 4 * (lane / 32);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        bias[jj][q][e] = (p.bias != nullptr && (!EDGE || col + e < p.N)) ? p.bias[col + e] : 0.0f;
    }
}

// n-blocks whose bias values a wave holds at once: two (32 values per lane) for
// the tiles of at most two n-blocks per wave, one for the wider wave tiles,
// whose accumulators and epilogue leave less room.
template <class T>
constexpr int bias_batch() { return T::FN == 2 ? 2 : 1; }

// Epilogue of the direct-to-LDS kernel: x = alpha acc + bias, the activation,
// rounded to the 16-bit format and stored.  Lane l holds, for n-block j, m-block
// i and q = 0..3, the four columns n = 8 q + 4 (l / 32) + 0..3 of row m = l % 32.
template <class T, bool EDGE>
__device__ __forceinline__ void hdma_epilogue(const HgemmArgs& p, const f32x16 (&acc)[T::FN][T::FM],
                                              uint8_t* lds, int m0, int n0, int wave, int wm,
                                              int wn, int lane) {
  constexpr int JB = bias_batch<T>();
  static_assert(T::FN % JB == 0, "n-blocks split into whole batches");
  // The eight-wave tiles load the first batch of bias values before the
  // barrier, so their latency overlaps the wait for the other waves; the
  // four-wave tiles, whose accumulators fill their registers up to the last
  // K tile, load it after.
  constexpr bool EARLY = T::WAVES_PER_SIMD == 2;
  float bias0[JB][4][4];
  if constexpr (EARLY) hdma_load_bias<T, EDGE, JB>(p, bias0, 0, n0, wn, lane);
  const float alpha = p.alpha;
  const Activation act(p.act);
  if (p.ldc % 8 == 0 && (reinterpret_cast<uintptr_t>(p.C) & 15u) == 0 && (!EDGE || p.N % 8 == 0)) {
    // Through LDS, so that every store instruction writes whole rows: the wave
    // puts its finished WTM x WTN tile into its own region of the (now idle)
    // stages, then reads it back 16 bytes per lane along rows.  16-byte chunks
    // of row r are permuted by (r / rows-per-256-bytes) % chunks-per-row, so
    // the writes of one column over 32 rows spread over the banks.
    static_assert(T::BM * T::BN * 2 <= T::STAGES * T::STAGE_BYTES, "output tile must fit the stages");
    constexpr int RB = T::WTN * 2;          // bytes per row of a wave's tile
    constexpr int CPR = RB / 16;            // 16-byte chunks per row
    constexpr int RPL = RB >= 256 ? 1 : 256 / RB;
    static_assert(RB % 128 == 0 && 1024 % RB == 0, "rows of 128 or 256 bytes");
    lds_barrier();   // every wave is done with the stages
    if constexpr (!EARLY) hdma_load_bias<T, EDGE, JB>(p, bias0, 0, n0, wn, lane);
    uint8_t* region = lds + wave * (T::WTM * RB);
#pragma unroll
    for (int j0 = 0; j0 < T::FN; j0 += JB) {
      float bias_next[JB][4][4];
      if (j0 > 0) hdma_load_bias<T, EDGE, JB>(p, bias_next, j0, n0, wn, lane);
      float (&bias)[JB][4][4] = j0 > 0 ? bias_next : bias0;
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        const int j = j0 + jj;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
          for (int i = 0; i < T::FM; ++i) {
            const int r = 32 * i + lane % 32;
            uint16_t h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              h[e] = T::E::bits(act(__builtin_fmaf(alpha, acc[j][i][4 * q + e], bias[jj][q][e])));
            }
            const int chunk = 4 * j + q;
            *reinterpret_cast<uint2*>(region + r * RB + 16 * (chunk ^ ((r / RPL) % CPR)) +
                                      8 * (lane / 32)) = __builtin_bit_cast(uint2, h);
          }
        }
      }
    }
#pragma unroll
    for (int it = 0; it < T::WTM * RB / 1024; ++it) {
      const int r = it * (1024 / RB) + lane / CPR;
      const int chunk = lane % CPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(region + r * RB +
                                                      16 * (chunk ^ ((r / RPL) % CPR)));
      // (N is a multiple of 8 here: a chunk is wholly in or out)
      if (EDGE && (m0 + wm * T::WTM + r >= p.M || n0 + wn * T::WTN + 8 * chunk >= p.N)) continue;
      *reinterpret_cast<u32x4*>(p.C + (size_t)(m0 + wm * T::WTM + r) * p.ldc + n0 +
                                wn * T::WTN + 8 * chunk) = v;
    }
    return;
  }
  if constexpr (!EARLY) hdma_load_bias<T, EDGE, JB>(p, bias0, 0, n0, wn, lane);
  const bool vec_store = (p.ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(p.C) & 7u) == 0);
#pragma unroll
  for (int j0 = 0; j0 < T::FN; j0 += JB) {
    float bias_next[JB][4][4];
    if (j0 > 0) hdma_load_bias<T, EDGE, JB>(p, bias_next, j0, n0, wn, lane);
    float (&bias)[JB][4][4] = j0 > 0 ? bias_next : bias0;
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
      const int j = j0 + jj;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n0 + wn * T::WTN + 32 * j + 8 * q + 4 * (lane / 32);
#pragma unroll
        for (int i = 0; i < T::FM; ++i) {
          const int row = m0 + wm * T::WTM + 32 * i + lane % 32;
          uint16_t h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            h[e] = T::E::bits(act(__builtin_fmaf(alpha, acc[j][i][4 * q + e], bias[jj][q][e])));
          }
          uint16_t* dst = p.C + (size_t)row * p.ldc + col;
          if (EDGE && (row >= p.M || col >= p.N)) continue;
          if (vec_store && (!EDGE || col + 3 < p.N)) {
            *reinterpret_cast<uint2*>(dst) = __builtin_bit_cast(uint2, h);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (!EDGE || col + e < p.N) dst[e] = h[e];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Persistent form of the column split (the FFN shape): one workgroup per CU
// walks a list of output tiles, head tiles (shape H) then tail tiles (shape
// T2), items g, g + G, g + 2G, ... for workgroup g of G.  After the K loop of a
// tile, once every wave is done reading the stages, the workgroup issues the
// direct loads of the next tile's first STAGES - 1 K tiles (and a copy of that
// tile's bias into LDS) before it runs this tile's epilogue, so those loads are
// in flight while the bias, GELU and stores of this tile run, and the next K
// loop starts on landed data (the pipelined main loop of the DeepGEMM page,
// 3.3, carried across tiles).  LDS: the K-tile ring at [0, STAGES x stage),
// the epilogue's staging area right after the largest ring's first three
// stages, two 1 KiB bias slots after the largest ring.
//
// The epilogue's stores are issued after the next tile's first loads, so the
// first two waits of the next K loop also allow them (vmcnt counts loads and
// stores in issue order): 16 stores per lane after a 256 x 256 tile, 8 after a
// 128 x 256 one.
// ---------------------------------------------------------------------------
template <class H, class T2>
struct HPersist {
  static constexpr int RING = H::STAGES * H::STAGE_BYTES > T2::STAGES * T2::STAGE_BYTES
                                  ? H::STAGES * H::STAGE_BYTES
                                  : T2::STAGES * T2::STAGE_BYTES;
  // staging: after the first three stages of either ring, 4 KiB per wave
  static constexpr int STAGING = 3 * H::STAGE_BYTES > 3 * T2::STAGE_BYTES ? 3 * H::STAGE_BYTES
                                                                          : 3 * T2::STAGE_BYTES;
  static constexpr int STAGING_BYTES = 4096 * (H::THREADS / kWave);
  static constexpr int BIAS = RING > STAGING + STAGING_BYTES ? RING : STAGING + STAGING_BYTES;
  static constexpr int LDS_BYTES = BIAS + 2 * 1024;
  static constexpr int STORES_H = H::WTM * H::WTN * 2 / 1024;    // 16-byte stores per lane
  static constexpr int STORES_T2 = T2::WTM * T2::WTN * 2 / 1024;
  static_assert(H::THREADS == T2::THREADS && H::WAVES_PER_SIMD == T2::WAVES_PER_SIMD,
                "both shapes run the same workgroup");
  static_assert(H::BN == 256 && T2::BN == 256, "a 1 KiB bias slot holds a tile's columns");
  static_assert(H::WTN == 64 && T2::WTN == 64, "staging rows of 128 bytes");
  static_assert(H::STAGES >= 4 && T2::STAGES >= 4, "three K tiles prefetched, one more in the ring");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(STORES_H == 16 && STORES_T2 == 8, "wait_vmcnt_plus knows 8 and 16");
};

// Issue the bias copy (every wave the same 1 KiB, at `bias_slot`) and the direct
// loads of K tiles 0 .. STAGES - 2 of tile `t` of the launch `p`.
template <class T>
__device__ __forceinline__ void hpersist_issue_first(const HgemmArgs& p, int t, uint32_t lds_base,
                                                     uint32_t bias_slot, int wave, int lane) {
  int tile_m, tile_n;
  tile_of_workgroup(t, p.tiles_m, p.tiles_n, p.group_m, tile_m, tile_n);
  const int m0 = tile_m * T::BM, n0 = tile_n * T::BN;
  if (p.bias != nullptr)
    dma16_sbase_u(p.bias + n0, 16u * (uint32_t)lane, bias_slot);
  const HDmaOffsets<T> dma(p, wave, lane, m0, n0);
  const uint16_t* a_tile = p.A + (size_t)m0 * p.lda;
  const uint16_t* b_tile = p.B + n0;
#pragma unroll
  for (int st = 0; st < T::STAGES - 1; ++st)
    hdma_issue_tile<T>(p, dma, a_tile, b_tile, st, lds_base + st * T::STAGE_BYTES, wave);
}

// K loop of tile `t` of `p`, whose first STAGES - 1 K tiles are in flight;
// `extra` stores were issued after them.  Whole tiles only, K a multiple of 2 BK
// with at least STAGES K tiles.
template <class T>
__device__ __forceinline__ void hpersist_k_loop(const HgemmArgs& p, int t,
                                                f32x16 (&acc)[T::FN][T::FM], uint8_t* lds,
                                                uint32_t lds_base, int wave, int lane,
                                                int extra) {
  int tile_m, tile_n;
  tile_of_workgroup(t, p.tiles_m, p.tiles_n, p.group_m, tile_m, tile_n);
  const int m0 = tile_m * T::BM, n0 = tile_n * T::BN;
  const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;
#pragma unroll
  for (int j = 0; j < T::FN; ++j)
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;
  const int ktiles = p.K / T::BK;
  const uint16_t* a_tile = p.A + (size_t)m0 * p.lda;
  const uint16_t* b_tile = p.B + n0;
  const HDmaOffsets<T> dma(p, wave, lane, m0, n0);
  HFrags<T> f0, f1, f2, f3;
  wait_vmcnt_plus<(T::STAGES - 2) * T::LOADS_PER_TILE>(extra);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  hload_frags<T>(f0, lds, 0, wm, wn, lane);
  hload_frags<T>(f1, lds, 1, wm, wn, lane);
  // The first two tiles allow the extra stores in their waits.
  hdma_tile<T, true>(p, acc, 0, ktiles, f0, f1, f2, f3, lds, lds_base, dma, a_tile, b_tile, wave,
                     wm, wn, lane, extra);
  hdma_tile<T, true>(p, acc, 1, ktiles, f2, f3, f0, f1, lds, lds_base, dma, a_tile, b_tile, wave,
                     wm, wn, lane, extra);
  int kt = 2;
  for (; kt + T::STAGES < ktiles; kt += 2) {
    hdma_tile<T, true>(p, acc, kt, ktiles, f0, f1, f2, f3, lds, lds_base, dma, a_tile, b_tile,
                       wave, wm, wn, lane);
    hdma_tile<T, true>(p, acc, kt + 1, ktiles, f2, f3, f0, f1, lds, lds_base, dma, a_tile, b_tile,
                       wave, wm, wn, lane);
  }
  for (; kt < ktiles; kt += 2) {
    hdma_tile<T, false>(p, acc, kt, ktiles, f0, f1, f2, f3, lds, lds_base, dma, a_tile, b_tile,
                        wave, wm, wn, lane);
    hdma_tile<T, false>(p, acc, kt + 1, ktiles, f2, f3, f0, f1, lds, lds_base, dma, a_tile,
                        b_tile, wave, wm, wn, lane);
  }
}

// Epilogue of tile `t` of `p` with its bias in LDS at `bias`: x = alpha acc +
// bias, the activation, 16-bit rounding; each wave stages 32 rows (4 KiB) at a
// time in its part of the staging area and stores them as whole rows.  Issues
// exactly WTM * WTN * 2 / 1024 stores per lane.
template <class T>
__device__ __forceinline__ void hpersist_epilogue(const HgemmArgs& p, int t,
                                                  const f32x16 (&acc)[T::FN][T::FM],
                                                  const float* bias, uint8_t* staging, int wave,
                                                  int lane) {
  int tile_m, tile_n;
  tile_of_workgroup(t, p.tiles_m, p.tiles_n, p.group_m, tile_m, tile_n);
  const int m0 = tile_m * T::BM, n0 = tile_n * T::BN;
  const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;
  const float alpha = p.alpha;
  const Activation act(p.act);
  const bool has_bias = p.bias != nullptr;
  constexpr int RB = T::WTN * 2;    // 128 bytes per row of a wave's tile
  constexpr int CPR = RB / 16;      // 8 chunks per row
  constexpr int RPL = 256 / RB;     // 2 rows per 256 bytes
  uint8_t* region = staging + wave * 4096;
  float bv[T::FN][4][4];
#pragma unroll
  for (int j = 0; j < T::FN; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int cl = wn * T::WTN + 32 * j + 8 * q + 4 * (lane / 32);
      const f32x4 b4 = has_bias ? *reinterpret_cast<const f32x4*>(bias + cl)
                                : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int e = 0; e < 4; ++e) bv[j][q][e] = b4[e];
    }
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {   // block row i = rows 32 i .. 32 i + 31 of the wave's tile
    const int r = lane % 32;
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint16_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          h[e] = T::E::bits(act(__builtin_fmaf(alpha, acc[j][i][4 * q + e], bv[j][q][e])));
        const int chunk = 4 * j + q;
        *reinterpret_cast<uint2*>(region + r * RB + 16 * (chunk ^ ((r / RPL) % CPR)) +
                                  8 * (lane / 32)) = __builtin_bit_cast(uint2, h);
      }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int rr = it * (1024 / RB) + lane / CPR;
      const int chunk = lane % CPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(region + rr * RB +
                                                      16 * (chunk ^ ((rr / RPL) % CPR)));
      *reinterpret_cast<u32x4*>(p.C + (size_t)(m0 + wm * T::WTM + 32 * i + rr) * p.ldc + n0 +
                                wn * T::WTN + 8 * chunk) = v;
    }
  }
}

// The launch arguments of the tail tiles: the columns from n1 on.
template <class T2>
__device__ __forceinline__ HgemmArgs hpersist_tail_args(const HgemmArgs& p, int n1) {
  HgemmArgs t = p;
  t.N = p.N - n1;
  t.B = p.B + n1;
  t.C = p.C + n1;
  t.bias = p.bias != nullptr ? p.bias + n1 : nullptr;
  t.nb = p.nb - n1;
  t.tiles_m = p.M / T2::BM;
  t.tiles_n = t.N / T2::BN;
  t.group_m = p.k_chunk;   // the tail's tile order (k_chunk is unused by these tiles)
  return t;
}

// `p`: the head launch (columns [0, n1), tiles_m x tiles_n tiles of H); the
// tail tiles (shape T2) cover columns [n1, N).
template <class H, class T2>
__global__ void __launch_bounds__(H::THREADS) __attribute__((amdgpu_waves_per_eu(H::WAVES_PER_SIMD)))
hgemm_dma_persistent_kernel(HgemmArgs p, int n1) {
  using L = HPersist<H, T2>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[L::LDS_BYTES];
  const int lane0 = threadIdx.x % kWave;
  const int lane = lane0;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t lds_base = lds_offset(lds);
  const int G = gridDim.x;
  const int head_items = p.tiles_m * p.tiles_n;
  const int total_items = head_items + (p.M / T2::BM) * ((p.N - n1) / T2::BN);
  int item = blockIdx.x;
  if (item >= total_items) return;
  uint8_t* staging = lds + L::STAGING;
  int n = 0, extra = 0;
  if (item < head_items) {
    hpersist_issue_first<H>(p, item, lds_base, lds_base + L::BIAS, wave, lane);
    for (; item < head_items; item += G, ++n) {
      // Per-lane addresses are recomputed in every iteration rather than held
      // across the loop: opaque copies of the lane and the LDS base keep the
      // compiler from hoisting them (they would not fit beside the accumulators).
      int lane = lane0;
      asm volatile("" : "+v"(lane));
      const int next = item + G;
      const uint32_t next_bias =
          __builtin_amdgcn_readfirstlane(lds_base + L::BIAS + ((n + 1) & 1) * 1024);
      f32x16 acc[H::FN][H::FM];
      hpersist_k_loop<H>(p, item, acc, lds, lds_base, wave, lane, extra);
      lds_barrier();   // every wave is done reading the ring
      if (next < head_items)
        hpersist_issue_first<H>(p, next, lds_base, next_bias, wave, lane);
      else if (next < total_items)
        hpersist_issue_first<T2>(hpersist_tail_args<T2>(p, n1), next - head_items, lds_base,
                                 next_bias, wave, lane);
      hpersist_epilogue<H>(p, item, acc,
                           reinterpret_cast<const float*>(lds + L::BIAS + (n & 1) * 1024), staging,
                           wave, lane);
      extra = L::STORES_H;
    }
  } else {
    hpersist_issue_first<T2>(hpersist_tail_args<T2>(p, n1), item - head_items, lds_base,
                             lds_base + L::BIAS, wave, lane);
  }
  const HgemmArgs t = hpersist_tail_args<T2>(p, n1);
  for (; item < total_items; item += G, ++n) {
    int lane = lane0;
    asm volatile("" : "+v"(lane));
    const int next = item + G;
    const uint32_t next_bias =
        __builtin_amdgcn_readfirstlane(lds_base + L::BIAS + ((n + 1) & 1) * 1024);
    f32x16 acc[T2::FN][T2::FM];
    hpersist_k_loop<T2>(t, item - head_items, acc, lds, lds_base, wave, lane, extra);
    lds_barrier();
    if (next < total_items)
      hpersist_issue_first<T2>(t, next - head_items, lds_base, next_bias, wave, lane);
    hpersist_epilogue<T2>(t, item - head_items, acc,
                          reinterpret_cast<const float*>(lds + L::BIAS + (n & 1) * 1024), staging,
                          wave, lane);
    extra = L::STORES_T2;
  }
}

// SPLIT: workgroup row blockIdx.y runs K chunk y (a multiple of 2 BK) and
// writes its raw FP32 partial sums to the workspace (the split-K scheme of the
// register-staged kernel, whose reduction kernel applies the epilogue).
// The work of one workgroup: output tile number `wg` of the launch (in the
// tile order of tile_of_workgroup) and K chunk `chunk` (SPLIT), in the LDS
// array `lds` of at least STAGES * STAGE_BYTES bytes.
template <class T, bool EDGE, bool SPLIT>
__device__ __forceinline__ void hdma_workgroup(HgemmArgs p, int wg, int chunk, uint8_t* lds) {
  static_assert(T::KSTEPS % 2 == 0, "fragments ping-pong between two register sets");
  static_assert(T::LOADS_PER_TILE <= T::FM * T::FN, "one direct load per MFMA at most");
  if constexpr (SPLIT) {
    const int kbeg = chunk * p.k_chunk;
    const int klen = p.K - kbeg < p.k_chunk ? p.K - kbeg : p.k_chunk;
    p.A += kbeg;
    p.B += (size_t)kbeg * p.ldb;
    p.K = klen;
  }

  int tile_m, tile_n;
  tile_of_workgroup(wg, p.tiles_m, p.tiles_n, p.group_m, tile_m, tile_n);
  const int m0 = tile_m * T::BM;
  const int n0 = tile_n * T::BN;
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wm = wave / T::WAVES_N;
  const int wn = wave % T::WAVES_N;
  const uint32_t lds_base = lds_offset(lds);

  // acc[j][i]: C^T block of n-block j and m-block i of this wave.
  f32x16 acc[T::FN][T::FM];
#pragma unroll
  for (int j = 0; j < T::FN; ++j)
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

  // Pipeline.  Tile kt lives in stage kt % STAGES; its direct loads are issued
  // during tile kt - STAGES + 1.  While the MFMAs of tile kt run, the waves read
  // every fragment of tile kt + 1 (two register sets per tile, four in all, so a
  // fragment is read a whole tile, about 1000 cycles, before its MFMA: LDS
  // latency under this load is several hundred cycles).  Early in tile kt the
  // waves wait for tile kt + 1 to land and meet at one barrier; past it, every
  // wave has also finished with stage (kt - 1) % STAGES (its fragments were
  // consumed in tile kt - 1), which the direct loads of tile kt + STAGES - 1
  // then refill.  K is a multiple of 2 BK, so the loop body covers two tiles.
  // On a ragged K (EDGE only) the loop covers the largest multiple of 2 BK in K
  // and hdma_k_tail adds the rest first.
  const int ktiles = EDGE ? (p.K / (2 * T::BK)) * 2 : p.K / T::BK;
  // Wave-uniform tile bases (k = 0) and the per-lane offsets of the direct loads.
  const uint16_t* a_tile = p.A + (size_t)m0 * p.lda;
  const uint16_t* b_tile = p.B + n0;
  const HDmaOffsets<T> dma(p, wave, lane, m0, n0);
  HFrags<T> f0, f1, f2, f3;
#pragma unroll
  for (int st = 0; st < T::STAGES - 1; ++st)
    if (st < ktiles) hdma_issue_tile<T>(p, dma, a_tile, b_tile, st, lds_base + st * T::STAGE_BYTES,
                                        wave);
  if constexpr (EDGE) {
    if (ktiles * T::BK < p.K) hdma_k_tail<T>(p, acc, lds, ktiles * T::BK, m0, n0, wave, wm, wn, lane);
  }
  if (ktiles > 0) {
    wait_tiles_in_flight<T>(ktiles - 1 < T::STAGES - 2 ? ktiles - 1 : T::STAGES - 2);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    hload_frags<T>(f0, lds, 0, wm, wn, lane);
    hload_frags<T>(f1, lds, 1, wm, wn, lane);
  }
  int kt = 0;
  // Steady state: both tiles of the pair have their look-ahead tile to load.
  for (; kt + T::STAGES < ktiles; kt += 2) {
    hdma_tile<T, true>(p, acc, kt, ktiles, f0, f1, f2, f3, lds, lds_base, dma, a_tile, b_tile,
                       wave, wm, wn, lane);
    hdma_tile<T, true>(p, acc, kt + 1, ktiles, f2, f3, f0, f1, lds, lds_base, dma, a_tile, b_tile,
                       wave, wm, wn, lane);
  }
  // Drain: the last STAGES (or fewer) tiles, loads and waits decided per tile.
  for (; kt < ktiles; kt += 2) {
    hdma_tile<T, false>(p, acc, kt, ktiles, f0, f1, f2, f3, lds, lds_base, dma, a_tile, b_tile,
                        wave, wm, wn, lane);
    hdma_tile<T, false>(p, acc, kt + 1, ktiles, f2, f3, f0, f1, lds, lds_base, dma, a_tile,
                        b_tile, wave, wm, wn, lane);
  }
  if constexpr (SPLIT) {
    // Lane l holds, for n-block j, m-block i and q = 0..3, columns 8 q + 4 (l / 32)
    // + 0..3 of row l % 32 (as in the epilogue below).
    float* W = p.ws + (size_t)chunk * p.M * p.N;
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < T::FM; ++i) {
          const int row = m0 + wm * T::WTM + 32 * i + lane % 32;
          const int col = n0 + wn * T::WTN + 32 * j + 8 * q + 4 * (lane / 32);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (!EDGE || (row < p.M && col + e < p.N))
              W[(size_t)row * p.N + col + e] = acc[j][i][4 * q + e];
        }
    return;
  }

  hdma_epilogue<T, EDGE>(p, acc, lds, m0, n0, wave, wm, wn, lane);
}

template <class T, bool EDGE, bool SPLIT = false>
__global__ void __launch_bounds__(T::THREADS) __attribute__((amdgpu_waves_per_eu(T::WAVES_PER_SIMD)))
hgemm_dma_kernel(HgemmArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[T::STAGES * T::STAGE_BYTES];
  hdma_workgroup<T, EDGE, SPLIT>(p, blockIdx.x, blockIdx.y, lds);
}

// Two tile shapes in one launch: workgroups 0 .. head_wgs - 1 take the tiles of
// `head` (tile shape H), the rest those of `tail` (shape T2), so the tail's
// tiles start on each compute unit as soon as it has finished its last head
// tile instead of after the whole head has drained.  Both shapes have the same
// number of waves; the LDS array is the larger of the two.
template <class H, class T2>
__global__ void __launch_bounds__(H::THREADS) __attribute__((amdgpu_waves_per_eu(H::WAVES_PER_SIMD)))
hgemm_dma_head_tail_kernel(HgemmArgs head, HgemmArgs tail, int head_wgs) {
  static_assert(H::THREADS == T2::THREADS && H::WAVES_PER_SIMD == T2::WAVES_PER_SIMD,
                "both shapes run the same workgroup");
  constexpr int HB = H::STAGES * H::STAGE_BYTES, TB = T2::STAGES * T2::STAGE_BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[HB > TB ? HB : TB];
  if ((int)blockIdx.x < head_wgs)
    hdma_workgroup<H, false, false>(head, blockIdx.x, 0, lds);
  else
    hdma_workgroup<T2, false, false>(tail, blockIdx.x - head_wgs, 0, lds);
}

template <class E> using HTileLarge = HgemmTile<E, 256, 256, 64, 2, 2>;
template <class E> using HTileMedium = HgemmTile<E, 128, 128, 64, 2, 2>;
template <class E> using HTileSmall = HgemmTile<E, 64, 64, 64, 2, 2>;
// direct-to-LDS: 4 stages x 32 KiB, one workgroup per CU / 3 stages x 24 KiB, two per CU /
// 5 stages x 32 KiB (all 160 KiB of LDS, three K tiles in flight while one is consumed)
template <class E> using HDmaLarge = HDmaTile<E, 256, 256, 32, 4>;
template <class E> using HDmaTall = HDmaTile<E, 128, 256, 32, 3, 2>;
template <class E> using HDmaDeep = HDmaTile<E, 256, 256, 32, 5>;
// 256 x 256 with eight waves (2 x 4, each 128 x 64), two per SIMD: while one
// wave waits on its LDS reads or the barrier, the other can issue MFMAs.
template <class E> using HDmaEight = HDmaTile<E, 256, 256, 32, 4, 2, 2, 4>;
// 128 x 256 with eight waves of 64 x 64 and four stages: 96 KiB of LDS, so each
// CU holds one workgroup and a round of them spreads over every CU.
template <class E> using HDmaHalfEight = HDmaTile<E, 128, 256, 32, 4, 2, 2, 4>;
// 128 x 128 with four waves of 64 x 64, four stages of 16 KiB, two workgroups per
// CU: outputs of a quarter to twice as many such tiles as CUs.  A wave has as
// many direct loads as MFMAs per k step, so half go out in each step.
template <class E> using HDmaSquare = HDmaTile<E, 128, 128, 32, 4, 2, 2, 2>;

// Second half of split-K: C = act(alpha * (sum of the `splits` partials, added
// in order 0, 1, ...) + bias[col]), rounded to the 16-bit format.
template <class E>
__global__ void __launch_bounds__(256) half_splitk_reduce_kernel(int M, int N, int splits,
                                                                 const float* ws, float alpha,
                                                                 const float* bias, int act,
                                                                 uint16_t* C, int ldc) {
  const int64_t total = (int64_t)M * N;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    float sum = ws[t];
    for (int q = 1; q < splits; ++q) sum += ws[q * total + t];
    const int64_t i = t / N, j = t % N;
    float x = __builtin_fmaf(alpha, sum, bias != nullptr ? bias[j] : 0.0f);
    if (act == 1) x = gelu_tanh(x);
    C[i * ldc + j] = E::bits(x);
  }
}

// The second kernel of a split call: the fixed-order sum of the partials and
// the epilogue.
template <class E>
static hipError_t launch_half_reduce(const HgemmCall& c, int splits, const float* ws,
                                     hipStream_t s) {
  const int64_t total = (int64_t)c.M * c.N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(half_splitk_reduce_kernel<E>, dim3((unsigned)blocks), dim3(256), 0, s, c.M,
                     c.N, splits, ws, c.alpha, c.bias, c.act, c.C, c.ldc);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_htile(const HgemmCall& c, int group_m, hipStream_t s, int splits = 1,
                               int k_chunk = 0, float* ws = nullptr) {
  HgemmArgs p;
  p.M = c.M; p.N = c.N; p.K = c.K;
  p.alpha = c.alpha;
  p.A = c.A; p.lda = c.lda; p.B = c.B; p.ldb = c.ldb;
  p.bias = c.bias; p.act = c.act;
  p.C = c.C; p.ldc = c.ldc;
  p.tiles_m = (c.M + T::BM - 1) / T::BM;
  p.tiles_n = (c.N + T::BN - 1) / T::BN;
  p.group_m = swizzle_group(group_m);
  p.k_chunk = k_chunk;
  p.nb = c.N;
  p.ws = ws;
  const bool fast = c.M % T::BM == 0 && c.N % T::BN == 0 && c.K % T::BK == 0 &&
                    c.lda % 8 == 0 && c.ldb % 8 == 0 &&
                    (reinterpret_cast<uintptr_t>(c.A) & 15u) == 0 &&
                    (reinterpret_cast<uintptr_t>(c.B) & 15u) == 0;
  if (splits > 1) {
    if (ws == nullptr || k_chunk % T::BK != 0) return hipErrorInvalidValue;
    const dim3 grid(p.tiles_m * p.tiles_n, splits), block(T::THREADS);
    if (fast)
      hipLaunchKernelGGL((hgemm_mfma_kernel<T, false, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((hgemm_mfma_kernel<T, true, true>), grid, block, 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_half_reduce<typename T::E>(c, splits, ws, s);
  }
  const dim3 grid(p.tiles_m * p.tiles_n), block(T::THREADS);
  if (fast)
    hipLaunchKernelGGL((hgemm_mfma_kernel<T, false, false>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((hgemm_mfma_kernel<T, true, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

// The direct-to-LDS kernels copy 16-byte chunks: rows of A and B on 16-byte
// boundaries, each row of B readable in whole chunks up to N (nb a multiple of
// 8), 32-bit per-lane copy offsets (at most 256 rows of A or 32 of B).  Whole
// tiles with K a multiple of 2 BK run the unchecked instantiation.
static bool half_operands_ok(const HgemmCall& c) {
  const int nb = readable_cols(c.nb, c.N);
  return c.lda % 8 == 0 && c.ldb % 8 == 0 && nb % 8 == 0 && nb >= c.N && nb <= c.ldb &&
         (reinterpret_cast<uintptr_t>(c.A) & 15u) == 0 &&
         (reinterpret_cast<uintptr_t>(c.B) & 15u) == 0 &&
         (int64_t)c.lda * 256 * 2 < (int64_t(1) << 31) &&
         (int64_t)c.ldb * 32 * 2 < (int64_t(1) << 31);
}

template <class T>
static bool dma_fits(const HgemmCall& c) {
  static_assert(T::BM <= 256 && T::BK == 32, "half_operands_ok's offset bounds");
  return half_operands_ok(c);
}

template <class T>
static bool dma_whole(const HgemmCall& c) {
  return c.M % T::BM == 0 && c.N % T::BN == 0 && c.K % (2 * T::BK) == 0;
}

template <class T>
static HgemmArgs hdma_args(const HgemmCall& c, int group_m, int k_chunk, float* ws) {
  HgemmArgs p;
  p.M = c.M; p.N = c.N; p.K = c.K;
  p.alpha = c.alpha;
  p.A = c.A; p.lda = c.lda; p.B = c.B; p.ldb = c.ldb;
  p.bias = c.bias; p.act = c.act;
  p.C = c.C; p.ldc = c.ldc;
  p.tiles_m = (c.M + T::BM - 1) / T::BM;
  p.tiles_n = (c.N + T::BN - 1) / T::BN;
  p.group_m = swizzle_group(group_m);
  p.nb = readable_cols(c.nb, c.N);
  p.k_chunk = k_chunk;
  p.ws = ws;
  return p;
}

template <class T>
static hipError_t launch_hdma(const HgemmCall& c, int group_m, hipStream_t s, int splits = 1,
                              int k_chunk = 0, float* ws = nullptr) {
  const HgemmArgs p = hdma_args<T>(c, group_m, k_chunk, ws);
  if (splits > 1) {
    if (ws == nullptr || k_chunk % (2 * T::BK) != 0) return hipErrorInvalidValue;
    const dim3 grid(p.tiles_m * p.tiles_n, splits);
    if (dma_whole<T>(c))
      hipLaunchKernelGGL((hgemm_dma_kernel<T, false, true>), grid, dim3(T::THREADS), 0, s, p);
    else
      hipLaunchKernelGGL((hgemm_dma_kernel<T, true, true>), grid, dim3(T::THREADS), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_half_reduce<typename T::E>(c, splits, ws, s);
  }
  if (dma_whole<T>(c))
    hipLaunchKernelGGL((hgemm_dma_kernel<T, false>), dim3(p.tiles_m * p.tiles_n),
                       dim3(T::THREADS), 0, s, p);
  else
    hipLaunchKernelGGL((hgemm_dma_kernel<T, true>), dim3(p.tiles_m * p.tiles_n),
                       dim3(T::THREADS), 0, s, p);
  return hipGetLastError();
}

static_assert(HDmaLarge<EltF16>::BM == 256 && HDmaLarge<EltF16>::BN == 256 &&
                  HDmaTall<EltF16>::BM == 128 && HDmaTall<EltF16>::BN == 256 &&
                  HDmaDeep<EltF16>::BM == 256 && HDmaDeep<EltF16>::BN == 256 &&
                  HDmaEight<EltF16>::BM == 256 && HDmaEight<EltF16>::BN == 256 &&
                  2 * HDmaEight<EltF16>::BK == 64 &&
                  2 * HDmaLarge<EltF16>::BK == 64 && 2 * HDmaTall<EltF16>::BK == 64 &&
                  2 * HDmaDeep<EltF16>::BK == 64 && HDmaSquare<EltF16>::BM == half_tile_rows(8) &&
                  HDmaSquare<EltF16>::BN == half_tile_cols(8) && 2 * HDmaSquare<EltF16>::BK == 64 &&
                  HDmaTall<EltF16>::BM == half_tile_rows(4) &&
                  HDmaTall<EltF16>::BN == half_tile_cols(4),
              "hgemm_resolve_tile's shape conditions must match the direct-to-LDS tiles");

int hgemm_tail_split(int M, int N, int cus) {
  // Columns [0, n1) in 256 x 256 tiles fill whole rounds of `cus` workgroups;
  // the rest, in 128 x 256 tiles, must fit one round.
  if (M % 256 != 0 || N % 256 != 0 || cus <= 0) return 0;
  const long tm = M / 256, tn = N / 256;
  if ((tm * tn) % cus == 0) return 0;   // no partial round to fix
  for (long n1 = tn - 1; n1 >= 1; --n1) {
    if ((tm * n1) % cus != 0) continue;
    const long tail = (M / 128) * (tn - n1);
    return tail <= cus ? (int)(n1 * 256) : 0;
  }
  return 0;
}

int hgemm_resolve_tile(int tile, int M, int N, int K, bool operands_ok, int cus) {
  // The direct-to-LDS kernels need rows of A and B on 16-byte boundaries and B
  // readable in whole 8-half chunks (ragged M, N and K run their bounds-checked
  // instantiation); otherwise the register-staged 256x256 kernel, which handles
  // every shape, runs.  The head/tail column split needs whole 256x256 tiles, K
  // a multiple of 64 and a split that fills the last round; else the eight-wave
  // tile runs alone.  The 128x128 direct-to-LDS tile falls back to its
  // register-staged twin.  The 16x16 K-split tile (9) takes any operands.
  if (tile >= 3 && tile != 9 && !operands_ok) return tile == 8 ? 1 : 0;
  if (tile == 7 && !(M % 256 == 0 && N % 256 == 0 && K % 64 == 0 && hgemm_tail_split(M, N, cus) > 0))
    return 6;
  return tile;
}

// ---------------------------------------------------------------------------
// Small outputs: one 16 x 16 output tile per workgroup, its K range split over
// eight waves and added in wave order through LDS (the split-K of lecture 24,
// section 8.3, inside one workgroup; the FP32 library's 16 x 16 tile in 16-bit
// form).  Operands go straight from global memory into registers; each wave
// takes every eighth chunk of 128 values of k and runs one
// v_mfma_f32_16x16x32 per 32 of them.  In MFMA step s lane l supplies row
// (or column) l % 16 at k = kb + 32 (l / 16) + 8 s + j, j = 0 .. 7, so a lane's
// 32 values of A in a chunk are contiguous in its row (four 16-byte loads) and
// A and B agree on which k each product uses; B's values are 2-byte loads down
// the column.  Every load is unconditional: row, column and k are clamped into
// the matrices and values outside are replaced by zero, and all of a chunk's
// loads go out before its first MFMA.  The epilogue (alpha, bias, activation,
// rounding) runs once per output element after the partial sums are added.
// ---------------------------------------------------------------------------
constexpr int kHksTile = 16;
constexpr int kHksWaves = 8;
constexpr int kHksSteps = 4;                      // MFMAs per wave per chunk
constexpr int kHksChunk = 32 * kHksSteps;         // k per wave per chunk
constexpr int kHksSpan = kHksWaves * kHksChunk;   // k of one chunk of every wave

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

template <class E>
__global__ void __launch_bounds__(kHksWaves * kWave)
    __attribute__((amdgpu_waves_per_eu(kHksWaves / 4))) hgemm_wave_ksplit_kernel(HgemmArgs p) {
  typedef typename E::vec8 vec8;
  __shared__ float part[kHksWaves][kHksTile * kHksTile];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int m0 = (blockIdx.x / p.tiles_n) * kHksTile;
  const int n0 = (blockIdx.x % p.tiles_n) * kHksTile;
  const int l16 = lane % 16, g = lane / 16;
  const int row = m0 + l16, col = n0 + l16;
  const bool row_ok = row < p.M, col_ok = col < p.N;
  const uint16_t* arow = p.A + (size_t)(row_ok ? row : 0) * p.lda;
  // B's values by 32-bit byte offsets from its base (the launcher checks that
  // 2 K ldb fits), so that each load takes the base from scalar registers and
  // needs one offset register, not a 64-bit address per value of k.
  const char* const bbase = reinterpret_cast<const char*>(p.B);
  const uint32_t bcol = 2u * (uint32_t)(col_ok ? col : 0);
  const uint32_t bstride = 2u * (uint32_t)p.ldb;
  auto bload = [&](int k) -> uint16_t {
    return *reinterpret_cast<const uint16_t*>(bbase + ((uint32_t)k * bstride + bcol));
  };
  f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int kb = wave * kHksChunk; kb < p.K; kb += kHksSpan) {
    const int ka = kb + 32 * g;
    if (p.a_vec && kb + kHksChunk <= p.K) {
      u16x8 a[kHksSteps], b[kHksSteps];
#pragma unroll
      for (int st = 0; st < kHksSteps; ++st)
        a[st] = *reinterpret_cast<const u16x8*>(arow + ka + 8 * st);
#pragma unroll
      for (int st = 0; st < kHksSteps; ++st)
#pragma unroll
        for (int j = 0; j < 8; ++j) b[st][j] = bload(ka + 8 * st + j);
      __builtin_amdgcn_sched_barrier(0);   // every load before the first MFMA
#pragma unroll
      for (int st = 0; st < kHksSteps; ++st) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          a[st][j] = row_ok ? a[st][j] : (uint16_t)0;
          b[st][j] = col_ok ? b[st][j] : (uint16_t)0;
        }
        // two accumulators, so consecutive MFMAs do not wait for each other
        f32x4& acc = st % 2 ? acc1 : acc0;
        acc = E::mfma16(__builtin_bit_cast(vec8, a[st]), __builtin_bit_cast(vec8, b[st]), acc);
      }
    } else {
      // The chunk that reaches past K, or rows of A off 16-byte boundaries:
      // 2-byte loads with k clamped, one MFMA step at a time.
#pragma unroll
      for (int st = 0; st < kHksSteps; ++st) {
        u16x8 a, b;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int k0 = ka + 8 * st + j;
          const int k = k0 < p.K ? k0 : p.K - 1;
          a[j] = arow[k];
          b[j] = bload(k);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bool in_k = ka + 8 * st + j < p.K;
          a[j] = row_ok && in_k ? a[j] : (uint16_t)0;
          b[j] = col_ok && in_k ? b[j] : (uint16_t)0;
        }
        f32x4& acc = st % 2 ? acc1 : acc0;
        acc = E::mfma16(__builtin_bit_cast(vec8, a), __builtin_bit_cast(vec8, b), acc);
      }
    }
  }
  // lane l holds column l % 16, rows 4 (l / 16) + r of this wave's partial tile
#pragma unroll
  for (int r = 0; r < 4; ++r) part[wave][(4 * g + r) * kHksTile + l16] = acc0[r] + acc1[r];
  __syncthreads();
  const int t = threadIdx.x;
  const int i = m0 + t / kHksTile, j = n0 + t % kHksTile;
  if (t < kHksTile * kHksTile && i < p.M && j < p.N) {
    float sum = part[0][t];
#pragma unroll
    for (int w = 1; w < kHksWaves; ++w) sum += part[w][t];
    // x = alpha * sum + bias[col]; y = act(x); C = 16-bit(y)
    float x = __builtin_fmaf(p.alpha, sum, p.bias != nullptr ? p.bias[j] : 0.0f);
    if (p.act == 1) x = gelu_tanh(x);
    p.C[(size_t)i * p.ldc + j] = E::bits(x);
  }
}

template <class E>
static hipError_t launch_hksplit(const HgemmCall& c, hipStream_t s) {
  HgemmArgs p{};
  p.M = c.M; p.N = c.N; p.K = c.K;
  p.alpha = c.alpha;
  p.A = c.A; p.lda = c.lda; p.B = c.B; p.ldb = c.ldb;
  p.bias = c.bias; p.act = c.act;
  p.C = c.C; p.ldc = c.ldc;
  p.tiles_m = (c.M + kHksTile - 1) / kHksTile;
  p.tiles_n = (c.N + kHksTile - 1) / kHksTile;
  p.group_m = 1;
  p.nb = c.N;
  p.k_chunk = c.K;
  p.ws = nullptr;
  p.a_vec = c.lda % 8 == 0 && (reinterpret_cast<uintptr_t>(c.A) & 15u) == 0;
  // B's byte offsets must fit 32 bits; past that the register-staged 64x64 tile,
  // which takes any shape, runs instead.
  if (2 * (int64_t)c.K * c.ldb >= (int64_t(1) << 32)) return launch_htile<HTileSmall<E>>(c, 8, s);
  hipLaunchKernelGGL(hgemm_wave_ksplit_kernel<E>, dim3(p.tiles_m * p.tiles_n),
                     dim3(kHksWaves * kWave), 0, s, p);
  return hipGetLastError();
}

HalfPlan plan_half_call(const HgemmCall& c, int cus, int force_tile, int force_splits,
                        size_t ws_floats) {
  return plan_half(c.M, c.N, c.K, cus, force_tile, force_splits, ws_floats, half_operands_ok(c));
}

template <class E>
static hipError_t launch_half(const HgemmCall& c, const HalfPlan& plan, int cus, float* ws,
                              hipStream_t s) {
  if (plan.splits > 1) {
    if ((plan.tile > 2 && plan.tile != 8) || ws == nullptr) return hipErrorInvalidValue;
    switch (plan.tile) {
      case 8:
        if (!dma_fits<HDmaSquare<E>>(c)) return hipErrorInvalidValue;
        return launch_hdma<HDmaSquare<E>>(c, 8, s, plan.splits, plan.k_chunk, ws);
      case 0: return launch_htile<HTileLarge<E>>(c, 4, s, plan.splits, plan.k_chunk, ws);
      case 1: return launch_htile<HTileMedium<E>>(c, 8, s, plan.splits, plan.k_chunk, ws);
      default: return launch_htile<HTileSmall<E>>(c, 8, s, plan.splits, plan.k_chunk, ws);
    }
  }
  switch (plan.tile) {
    case 9: return launch_hksplit<E>(c, s);
    case 0: return launch_htile<HTileLarge<E>>(c, 4, s);
    case 1: return launch_htile<HTileMedium<E>>(c, 8, s);
    case 2: return launch_htile<HTileSmall<E>>(c, 8, s);
    case 3:
      if (!dma_fits<HDmaLarge<E>>(c)) return hipErrorInvalidValue;
      return launch_hdma<HDmaLarge<E>>(c, 4, s);
    case 4:
      if (!dma_fits<HDmaTall<E>>(c)) return hipErrorInvalidValue;
      return launch_hdma<HDmaTall<E>>(c, 8, s);
    case 5:
      if (!dma_fits<HDmaDeep<E>>(c)) return hipErrorInvalidValue;
      return launch_hdma<HDmaDeep<E>>(c, 4, s);
    case 6:
      if (!dma_fits<HDmaEight<E>>(c)) return hipErrorInvalidValue;
      return launch_hdma<HDmaEight<E>>(c, 4, s);
    case 8:
      if (!dma_fits<HDmaSquare<E>>(c)) return hipErrorInvalidValue;
      return launch_hdma<HDmaSquare<E>>(c, 8, s);
    case 7: {
      // Columns [0, n1): eight-wave 256 x 256 tiles in whole rounds; the rest:
      // 128 x 256 tiles, twice as many half-size tiles in the last round.
      const int n1 = hgemm_tail_split(c.M, c.N, cus);
      HgemmCall head = c, tail = c;
      head.N = n1;
      tail.N = c.N - n1;
      tail.B = c.B + n1;
      if (c.nb > 0) tail.nb = c.nb - n1;
      tail.C = c.C + n1;
      tail.bias = c.bias ? c.bias + n1 : nullptr;
      if (n1 == 0 || !dma_fits<HDmaEight<E>>(head) || !dma_fits<HDmaHalfEight<E>>(tail) ||
          !dma_whole<HDmaEight<E>>(head) || !dma_whole<HDmaHalfEight<E>>(tail))
        return hipErrorInvalidValue;
      using H = HDmaEight<E>;
      using T2 = HDmaHalfEight<E>;
      const HgemmArgs ph = hdma_args<H>(head, 4, 0, nullptr);
      const HgemmArgs pt = hdma_args<T2>(tail, 8, 0, nullptr);
      const int head_wgs = ph.tiles_m * ph.tiles_n;
      const int total = head_wgs + pt.tiles_m * pt.tiles_n;
      if (c.K / H::BK >= H::STAGES + 2) {
        // One workgroup per CU walks its tiles, loading the next tile's first K
        // tiles under the current tile's epilogue.  The tail's arguments are
        // derived in the kernel from the head's (k_chunk carries its tile order).
        HgemmArgs pp = ph;
        pp.k_chunk = pt.group_m;
        pp.N = c.N;
        pp.nb = readable_cols(c.nb, c.N);
        const int grid = total < cus ? total : cus;
        hipLaunchKernelGGL((hgemm_dma_persistent_kernel<H, T2>), dim3(grid), dim3(H::THREADS), 0,
                           s, pp, n1);
        return hipGetLastError();
      }
      hipLaunchKernelGGL((hgemm_dma_head_tail_kernel<H, T2>), dim3(total), dim3(H::THREADS), 0, s,
                         ph, pt, head_wgs);
      return hipGetLastError();
    }
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_hgemm(const HgemmCall& c, const HalfPlan& plan, int cus, float* ws,
                        hipStream_t s) {
  return launch_half<EltF16>(c, plan, cus, ws, s);
}

hipError_t launch_bgemm(const HgemmCall& c, const HalfPlan& plan, int cus, float* ws,
                        hipStream_t s) {
  return launch_half<EltBF16>(c, plan, cus, ws, s);
}

}  // namespace lasg
