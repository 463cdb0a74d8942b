// Internal interface between the C ABI (gemm_capi.cpp) and the kernel files.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
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
};

// Tile configurations.  SGEMM: 0 = 256x256 (K step 16), 1 = 128x128, 2 = 64x64,
// 3 = 256x256 with K step 32, 4 = 128x256 at two workgroups per CU.
// HGEMM: 0 = 256x256, 1 = 128x128, 2 = 64x64 (register-staged, K step 64),
// 3 = 256x256 direct-to-LDS, 4 stages of K step 32, 4 = 128x256 direct-to-LDS,
// 3 stages, two workgroups per CU (3 and 4 need whole tiles and K a multiple of
// 64; other shapes fall back to 0).
constexpr int kSgemmTileCount = 5;
constexpr int kHgemmTileCount = 5;

// Tile configuration the shape selects on a device with `cus` compute units
// (for the half product, `dma_ok` says whether operand alignment and leading
// dimensions allow the direct-to-LDS kernel).
int sgemm_pick_tile(int M, int N, int cus);
int hgemm_pick_tile(int M, int N, int K, int cus, bool dma_ok);

// force_tile < 0 lets the shape decide; otherwise it names the tile configuration.
hipError_t launch_sgemm(const SgemmCall& c, int cus, int force_tile, hipStream_t s);
hipError_t launch_sgemm_scale(int M, int N, float beta, float* C, int ldc, hipStream_t s);

// The half-precision product: binary16 (hgemm) or bfloat16 (bgemm) inputs and
// output, FP32 accumulation; same kernels, tiles and tile choice.
hipError_t launch_hgemm(const HgemmCall& c, int cus, int force_tile, hipStream_t s);
hipError_t launch_bgemm(const HgemmCall& c, int cus, int force_tile, hipStream_t s);

}  // namespace lasg
