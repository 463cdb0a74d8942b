// Internal interface between the C ABI (gemm_capi.cpp) and the kernel files.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lasg {

struct SgemmCall {
  int M, N, K;
  float alpha, beta;
  const float* A;
  int lda;
  const float* B;
  int ldb;
  float* C;
  int ldc;
  // Columns of each row of B that may be read (at least N; more when B is a
  // padded copy); 0 means N.
  int nb = 0;
  // A and B are copies zero-padded to whole tiles of the configuration that
  // runs (register-staged tiles): A has ceil(M / BM) BM rows, B ceil(N / BN) BN
  // columns, and K is a multiple of the tile's K step; only the stores of C are
  // bounds-checked.
  bool padded = false;
};

struct HgemmCall {
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
  // Columns of each row of B that may be read (at least N; more when B is a
  // padded copy); 0 means N.
  int nb = 0;
};

inline int readable_cols(int nb, int N) { return nb > 0 ? nb : N; }

// Tile configurations.  SGEMM: 0 = 256x256 (K step 16), 1 = 128x128, 2 = 64x64,
// 3 = 256x256 with K step 32, 4 = 128x256 at two workgroups per CU (all with
// 32x32x2 MFMA blocks); 5 = 256x256 and 6 = 128x256 at two
// workgroups per CU, both with 16x16x4 MFMA blocks; 7 = 256x256 and 8 = 128x256
// at two workgroups per CU with direct-to-LDS copies into a multi-stage ring
// (rows of B 16-byte aligned and B readable in whole 4-float chunks, rows of A
// 4-byte aligned, else tile 4); 9 = tile 7 with eight waves, two per SIMD; 10 = 128x128 with
// direct-to-LDS copies at two workgroups per CU; 11 = 64x64 with direct-to-LDS
// copies at up to four workgroups per CU (else tile 2); 9, 10 and 11 meet at one
// barrier per two K tiles where their copies allow it; 12 = 32x32
// register-staged from 16x16x4 MFMA blocks, K step 32 (small outputs); 13 =
// 16x16 output tiles with K split over the workgroup's eight waves, operands
// loaded straight into registers (small outputs; any shape, never split-K).
// HGEMM: 0 = 256x256, 1 = 128x128, 2 = 64x64 (register-staged, K step 64),
// 3 = 256x256 direct-to-LDS, 4 stages of K step 32, 4 = 128x256 direct-to-LDS,
// 3 stages, two workgroups per CU, 5 = 256x256 direct-to-LDS, 5 stages, 6 = 256x256
// direct-to-LDS with eight waves, 7 = tile 6 on the columns that fill whole
// rounds of workgroups and 128 x 256 direct-to-LDS tiles on the rest, in one
// persistent launch of one workgroup per CU where K spans at least six 32-wide K
// tiles (3 to 7 need
// rows of A and B 16-byte aligned and B readable in whole 8-half chunks, 7 also
// whole tiles; other operands fall back to 0); 8 = 128x128 direct-to-LDS, 4
// stages, two workgroups per CU (other operands fall back to 1); 9 = 16x16
// output tiles with K split over the workgroup's eight waves, operands loaded
// straight into registers (small outputs; any shape, never split-K).
constexpr int kSgemmTileCount = 14;
constexpr int kHgemmTileCount = 10;

// K granularity of each SGEMM tile configuration: the K step (32 for tiles 3
// and 12), or for the direct-to-LDS tiles (7-11) their two-tile loop body
// (checked against the kernels).
constexpr int sgemm_tile_bk(int tile) { return tile == 13 ? 64 : tile == 3 || tile >= 7 ? 32 : 16; }
// Output tile of each SGEMM configuration.
constexpr int sgemm_tile_bm(int tile) {
  return tile == 0 || tile == 3 || tile == 5 || tile == 7 || tile == 9 ? 256
         : tile == 2 || tile == 11                                      ? 64
         : tile == 12                                                   ? 32
         : tile == 13                                                   ? 16
                                                                        : 128;
}
constexpr int sgemm_tile_bn(int tile) {
  return tile == 1 || tile == 10 ? 128
         : tile == 2 || tile == 11 ? 64
         : tile == 12              ? 32
         : tile == 13              ? 16
                                   : 256;
}

// Split-K: at most this many K chunks per output tile.
constexpr int kMaxSplits = 32;
// Library-owned FP32 workspace for split-K partials (per device, allocated by
// gemm_create): splits * M * N floats must fit.
constexpr size_t kWorkspaceBytes = size_t(64) << 20;
// Library-owned buffer for packed copies of operands whose rows are not 16-byte
// aligned (allocated by gemm_create beside the workspace).
constexpr size_t kPackBytes = size_t(256) << 20;

// How one SGEMM call runs: tile configuration, number of K chunks (1 = no
// split) and the chunk length in elements (a multiple of the tile's K step).
struct SgemmPlan {
  int tile;
  int splits;
  int k_chunk;
};

// The plan for an M x N x K product on `cus` compute units (`operands_ok`: the
// direct-to-LDS copies are legal: lda and ldb multiples of 4, A and B 16-byte
// aligned, B readable in whole 4-float chunks).  force_tile / force_splits
// < 0 let the shape decide (offline-tuned table, else the built-in rule); the
// split count is then clamped to the K tiles there are and to `ws_floats` of
// workspace.
SgemmPlan plan_sgemm(int M, int N, int K, int cus, int force_tile, int force_splits,
                     size_t ws_floats, bool operands_ok);
// The FP32 configuration that actually runs for `tile` with `splits` K chunks:
// the direct-to-LDS ones (7-10) become 4 when the operands (`operands_ok` as
// above) do not suit them.
int sgemm_resolve_tile(int tile, int M, int N, int K, int splits, bool operands_ok);

// Offline-tuned choice for (op, M, N, K) if the table has one for the shape's
// size class: op 0 = sgemm, op 1 = the half products.
bool tuned_config(int op, int M, int N, int K, int* tile, int* splits);

// How one half-product call runs: tile configuration, number of K chunks (1 =
// no split; only the register-staged tiles 0-2 split) and the chunk length.
struct HalfPlan {
  int tile;
  int splits;
  int k_chunk;
};
// Output tile of the register-staged half configurations 0-2 (K step 64).
constexpr int half_tile_bm(int tile) { return tile == 0 ? 256 : tile == 1 ? 128 : 64; }
constexpr int kHalfBK = 64;
// Output tile of every half configuration (rows, columns).
constexpr int half_tile_rows(int tile) {
  return tile <= 2 ? half_tile_bm(tile) : tile == 4 || tile == 8 ? 128 : tile == 9 ? 16 : 256;
}
constexpr int half_tile_cols(int tile) {
  return tile <= 2 ? half_tile_bm(tile) : tile == 8 ? 128 : tile == 9 ? 16 : 256;
}

// The plan for an M x N x K half product on `cus` compute units (`operands_ok`:
// lda and ldb are multiples of 8, A, B 16-byte aligned and B readable in whole
// 8-half chunks, as the direct-to-LDS kernels need).  force_tile / force_splits < 0 let the shape decide (tuned
// table, else the built-in rule); the result is resolved to what runs and the
// split count is clamped to the K tiles and to `ws_floats` of workspace.
HalfPlan plan_half(int M, int N, int K, int cus, int force_tile, int force_splits,
                   size_t ws_floats, bool operands_ok);
// plan_half with the operand conditions read from the call.
HalfPlan plan_half_call(const HgemmCall& c, int cus, int force_tile, int force_splits,
                        size_t ws_floats);
// The configuration that actually runs for `tile`: the direct-to-LDS ones (3
// to 7) become the register-staged 256x256 one (0), and 8 the register-staged
// 128x128 one (1), when the operands do not suit them; 9 runs anywhere.
// 7 (eight-wave 256 x 256 tiles with a 128 x 256 tail) becomes 6 when no split
// of the columns fills whole rounds of `cus` workgroups with the head and one
// round with the tail.
int hgemm_resolve_tile(int tile, int M, int N, int K, bool operands_ok, int cus);
// Column where that split falls (0: none).
int hgemm_tail_split(int M, int N, int cus);

// Whether the offline-tuned table is consulted (default on; a test hook turns
// it off to see the built-in rule).
void set_use_tuned(bool on);
bool use_tuned();

// Tile order of the launches (tile_of_workgroup): by default each launch's own
// group size with the XCD renumbering.  A test hook forces another group size
// (group_m > 0) or none (0) and turns the renumbering off or on.
void set_swizzle(int group_m, bool xcd_remap);
// The group_m value a launch passes to its kernel: the forced or the launch's
// own group size, negated when the XCD renumbering is off.
int swizzle_group(int launch_group_m);

// `ws` holds at least plan.splits * M * N floats when plan.splits > 1.
hipError_t launch_sgemm(const SgemmCall& c, const SgemmPlan& plan, float* ws, hipStream_t s);
hipError_t launch_sgemm_scale(int M, int N, float beta, float* C, int ldc, hipStream_t s);

// One operand copy (counts in elements): dst (dst_rows x ldd) = src (rows x
// cols, leading dimension lds) with columns [cols, ldd) and rows [rows,
// dst_rows) zero.  dst 16-byte aligned, ldd a multiple of 16 bytes.
struct PackJob {
  const void* src = nullptr;
  void* dst = nullptr;
  int rows = 0, cols = 0, lds = 0, dst_rows = 0, ldd = 0;
};
// One or two copies of 4-byte or 2-byte elements in one launch.
hipError_t launch_pack(const PackJob* jobs, int count, int elem_bytes, hipStream_t s);

// The half-precision product: binary16 (hgemm) or bfloat16 (bgemm) inputs and
// output, FP32 accumulation; same kernels, tiles and tile choice.
// `ws` holds at least plan.splits * M * N floats when plan.splits > 1.
hipError_t launch_hgemm(const HgemmCall& c, const HalfPlan& plan, int cus, float* ws,
                        hipStream_t s);
hipError_t launch_bgemm(const HgemmCall& c, const HalfPlan& plan, int cus, float* ws,
                        hipStream_t s);

}  // namespace lasg
