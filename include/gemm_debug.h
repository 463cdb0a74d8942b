/*
 * gemm_debug.h -- test hooks of the GEMM library (not needed by applications).
 *
 * The library picks a tile configuration from the problem shape.  Tests use
 * these hooks to run every configuration, fast path and bounds-checked path,
 * on the same inputs and to check the host-side choice without a GPU.
 */
#ifndef LINEAR_ALGEBRA_SGEMM_AMD_GEMM_DEBUG_H
#define LINEAR_ALGEBRA_SGEMM_AMD_GEMM_DEBUG_H

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Force the tile configuration of later calls in this process: op 0 = sgemm,
 * op 1 = the half-precision products (hgemm_bias_act and bgemm_bias_act); tile -1 = choose by shape (the default), 0 = the
 * largest tile, 1 = medium, 2 = small; sgemm also has 3 = largest tile with a
 * K step of 32 and 4 = 128 x 256 tiles at two workgroups per compute unit; the
 * half products also have 3 = 256 x 256 and 4 = 128 x 256 direct-to-LDS kernels
 * (whole tiles only, else the 256 x 256 register-staged kernel).
 * Whether the aligned fast path or the
 * bounds-checked path runs still follows the shape and alignment.  Returns
 * GEMM_STATUS_INVALID_VALUE for an unknown op or tile.  Pure host state: no
 * HIP call.  Not synchronised with calls in flight on other threads.
 */
int gemm_debug_force_tile(int op, int tile);

/* The tile configuration the library would choose for an M x N output on a
 * device with `cus` compute units (op 0 = sgemm; op 1 = hgemm_bias_act with
 * 16-byte-aligned operands and K a multiple of 64).  Returns -1 for an unknown
 * op.  Pure host computation. */
int gemm_debug_pick_tile(int op, int M, int N, int cus);

#ifdef __cplusplus
}
#endif

#endif /* LINEAR_ALGEBRA_SGEMM_AMD_GEMM_DEBUG_H */
