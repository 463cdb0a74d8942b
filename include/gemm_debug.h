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
 * K step of 32, 4 = 128 x 256 tiles at two workgroups per compute unit, 5
 * and 6 = tiles 0 and 4 built from 16 x 16 x 4 MFMA blocks, and 7 and 8 = tiles
 * 0 and 4 with direct-to-LDS copies (rows of B on 16-byte boundaries and N a
 * multiple of 4, else B is packed when the copy is small next to the product,
 * else tile 4 runs; rows of A off 16-byte boundaries are copied 4 bytes at a
 * time; ragged M, N or K run their bounds-checked instantiation), 9 = tile 7 with eight waves, 10 = 128 x 128 direct-to-LDS
 * tiles at two workgroups per compute unit, 11 = 64 x 64 direct-to-LDS tiles
 * at up to four workgroups per compute unit (tile 2 where the operands do not
 * allow direct copies), 12 = 32 x 32 tiles built from 16 x 16 x 4 MFMA blocks
 * with a K step of 32 (small outputs), 13 = 16 x 16 tiles whose eight waves
 * split K between them (small outputs; never split across workgroups); the
 * half products also have 3 = 256 x 256 and 4 = 128 x 256 direct-to-LDS kernels
 * 5 = the 256 x 256 one with a five-stage pipeline, 6 = the 256 x 256 one
 * with eight waves and 7 = tile 6 on the columns that fill whole rounds of
 * workgroups plus 128 x 256 tiles on the rest, one persistent workgroup per
 * compute unit walking both lists (whole tiles only, else the
 * 256 x 256 register-staged kernel; 7 becomes 6 where no such split exists),
 * 8 = 128 x 128 direct-to-LDS tiles at two workgroups per compute unit (tile 1
 * where the operands do not allow direct copies) and 9 = 16 x 16 tiles whose
 * eight waves split K between them (any operands; small outputs; never split
 * across workgroups).
 * Whether the aligned fast path or the
 * bounds-checked path runs still follows the shape and alignment.  Returns
 * GEMM_STATUS_INVALID_VALUE for an unknown op or tile.  Pure host state: no
 * HIP call.  Not synchronised with calls in flight on other threads.
 */
int gemm_debug_force_tile(int op, int tile);

/*
 * Force the number of K chunks (split-K) of later calls: op 0 = sgemm, op 1 =
 * the half products; splits -1 = choose by shape (the default), 1 = never
 * split, 2 .. 32 = that many chunks (still reduced to what K and the workspace
 * allow; the half products split only on their register-staged tiles 0-2 and
 * the 128 x 128 direct-to-LDS tile 8).
 * Returns GEMM_STATUS_INVALID_VALUE for another op or count.  Pure host state,
 * not synchronised with calls in flight on other threads.
 */
int gemm_debug_force_splits(int op, int splits);

/*
 * Whether the shape -> configuration choice consults the offline-tuned table
 * (on = 1, the default) or only the built-in rule (on = 0).  Forced tiles and
 * split counts win either way.  Returns GEMM_STATUS_INVALID_VALUE for another
 * value.  Pure host state.
 */
int gemm_debug_use_tuned_table(int on);

/*
 * The configuration the library would run for an M x N x K product on a device
 * with `cus` compute units, forced values included: *tile receives the tile
 * configuration, *splits the number of K chunks (1 = no split).  op 0 = sgemm,
 * op 1 = the half products, both with packed operands (lda = K, ldb = N) on
 * 16-byte-aligned bases; where those rows do not suit the direct-to-LDS
 * kernels (N not a multiple of 4 for sgemm; K or N not a multiple of 8 for the
 * half products), the call would pack them into the library's buffer when the
 * copy is small next to the product, and the result says what then runs (the
 * FP32 direct-to-LDS kernels copy rows of A with K not a multiple of 4 4 bytes
 * at a time).  Returns GEMM_STATUS_INVALID_VALUE for an unknown op,
 * negative sizes, cus <= 0 or a null output pointer.  Pure host computation:
 * no HIP call, no library state needed.
 */
int gemm_debug_pick_config(int op, int M, int N, int K, int cus, int* tile, int* splits);

/*
 * Tile order of later launches (both products): group_m 0 = each launch's own
 * group size (the default), 1..64 = walk that many tile rows per group;
 * xcd_remap 1 = renumber workgroups so that each of the eight XCDs takes one
 * contiguous run of the order (the default), 0 = keep the dispatcher's order.
 * Only the order of the output tiles changes, never a result.  Returns
 * GEMM_STATUS_INVALID_VALUE for other values.  Pure host state.
 */
int gemm_debug_force_swizzle(int group_m, int xcd_remap);

/*
 * The output tile (tile_m[wg], tile_n[wg]) that workgroup wg of a launch over
 * tiles_m x tiles_n tiles computes, for every wg < tiles_m * tiles_n, with
 * group size group_m and the XCD renumbering on (xcd_remap 1) or off (0): the
 * same function the kernels run.  tile_m and tile_n are host arrays of
 * tiles_m * tiles_n ints.  Returns GEMM_STATUS_INVALID_VALUE for non-positive
 * sizes, more than 2^24 tiles or null arrays.  Pure host computation.
 */
int gemm_debug_tile_map(int tiles_m, int tiles_n, int group_m, int xcd_remap, int* tile_m,
                        int* tile_n);

#ifdef __cplusplus
}
#endif

#endif /* LINEAR_ALGEBRA_SGEMM_AMD_GEMM_DEBUG_H */
