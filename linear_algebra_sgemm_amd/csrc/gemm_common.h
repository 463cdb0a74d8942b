// Shared device-side pieces of the GEMM kernels: vector types, the MFMA
// accumulator layout and the workgroup -> output-tile schedule.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lasg {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;     // CDNA wavefront width
constexpr int kXcds = 8;      // MI355X: 8 accelerator complex dies, 32 CUs each

// 32x32 MFMA result layout (all v_mfma_f32_32x32x* single-block forms): lane l
// holds column l % 32; its accumulator register r holds row
//   8 * (r / 4) + 4 * (l / 32) + r % 4.
__device__ __forceinline__ int mfma32_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Workgroup id -> (tile_m, tile_n).
//
// Step 1, XCD-aware: the dispatcher hands consecutive workgroup ids to the
// eight XCDs in turn, and each XCD has its own L2.  Renumber so that every XCD
// receives one contiguous run of the tile order.
// Step 2, grouped order: walk `group_m` tile rows column by column, so the
// tiles that run together on one XCD share a few A row panels and B column
// panels (the L2-reuse block swizzle of the DeepGEMM page, section 3.4).
// A negative `group_m` skips step 1 (a test hook compares both orders) and
// groups -group_m rows.  Both steps are bijections of [0, tiles_m * tiles_n),
// which a host test checks over all grids up to 64 x 64.
__host__ __device__ __forceinline__ void tile_of_workgroup(int wg, int tiles_m, int tiles_n,
                                                           int group_m, int& tile_m,
                                                           int& tile_n) {
  const int total = tiles_m * tiles_n;
  int t = wg;
  if (group_m > 0) {
    const int xcd = wg % kXcds;
    const int slot = wg / kXcds;
    const int per = total / kXcds;
    const int rem = total % kXcds;
    t = xcd * per + (xcd < rem ? xcd : rem) + slot;
  } else {
    group_m = -group_m;
  }
  const int group = group_m * tiles_n;
  const int gid = t / group;
  const int first = gid * group_m;
  const int rows = (tiles_m - first) < group_m ? (tiles_m - first) : group_m;
  const int r = t - gid * group;
  tile_m = first + r % rows;
  tile_n = r / rows;
}

}  // namespace lasg
