/*
 * gemm.h -- C ABI of the MI355X (gfx950) dense matrix-multiply library.
 *
 * The operation is the one stated in "SGEMM优化，从naive到warptiling",
 * section 问题与估算: C = alpha * A x B + beta * C, with A of M x K, B of K x N
 * and C of M x N, all row-major single-precision matrices.  The page's naive
 * kernel (section k1) takes (M, N, K, alpha, A, B, beta, C); this interface adds
 * leading dimensions and a HIP stream.  The half-precision entry point is the
 * FP16-input / FP32-accumulate product with bias and activation fused into the
 * single write-back, as described on the DeepGEMM page (sections 1.1 and 3.2).
 *
 * Conventions shared by every call:
 *  - Layout: row-major.  Element (i, j) of A is A[i*lda + j]; lda >= max(1, K),
 *    ldb >= max(1, N), ldc >= max(1, N).  No transpose options.
 *  - Memory: A, B, C and bias are DEVICE pointers owned by the caller; the
 *    library keeps no pointer after the enqueued work completes and allocates
 *    no device memory on the call path.  C must not overlap A, B or bias.
 *  - Alignment: element alignment only (4 bytes for float, 2 for half).
 *    Aligned shapes take a faster internal path; results do not depend on it.
 *  - Asynchrony: each call only enqueues work on `stream` (NULL = the default
 *    stream) and returns.  GEMM_STATUS_SUCCESS means "launched"; a device fault
 *    surfaces at the caller's next synchronisation.
 *  - Errors: invalid arguments return GEMM_STATUS_INVALID_VALUE and enqueue
 *    nothing (they are checked before anything else, with no HIP call).  A call
 *    before gemm_create returns GEMM_STATUS_NOT_INITIALIZED.  A failed launch
 *    returns GEMM_STATUS_HIP_ERROR; gemm_status_string then names the HIP error.
 *  - Threads: after gemm_create the compute calls may be made concurrently from
 *    several host threads and on several streams.  gemm_create/gemm_destroy must
 *    not race with compute calls.  Calls that use the library's workspace or pack
 *    buffer (split-K, operand copies) are ordered by the library: on one stream by
 *    stream order; the first such call on a second stream waits on the host for
 *    the device to finish its queued work (once), and from then on such calls
 *    order themselves with an event.  A call made while its stream is being
 *    captured into a HIP graph uses neither: it runs without split-K, and
 *    operands whose rows are off 16-byte boundaries are read in place by the
 *    bounds-checked kernels, so its replays need no ordering with other calls.
 */
#ifndef LINEAR_ALGEBRA_SGEMM_AMD_GEMM_H
#define LINEAR_ALGEBRA_SGEMM_AMD_GEMM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GEMM_STATUS_SUCCESS = 0,
  GEMM_STATUS_NOT_INITIALIZED = 1,
  GEMM_STATUS_INVALID_VALUE = 2,
  GEMM_STATUS_ARCH_MISMATCH = 3,
  GEMM_STATUS_HIP_ERROR = 4,
  GEMM_STATUS_INTERNAL = 5
} gemm_status_t;

typedef enum {
  GEMM_ACT_NONE = 0,      /* identity */
  GEMM_ACT_GELU_TANH = 1  /* 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) */
} gemm_act_t;

/*
 * Initialise the library for the current HIP device.  Checks that the device
 * is gfx950 (else GEMM_STATUS_ARCH_MISMATCH) and records its compute-unit count.
 * Allocates the library's device memory: a 64 MiB workspace for split-K
 * partial sums and a 256 MiB buffer for packed copies of operands whose rows
 * do not start on 16-byte boundaries (a call may copy such an operand there,
 * with padded rows, so that its fastest kernels can read it).
 * Reference counted: each successful gemm_create needs one gemm_destroy.
 */
int gemm_create(void);

/* Drop one reference; the last one releases the library state.  The caller
 * synchronises its streams first.  Returns NOT_INITIALIZED if there is none. */
int gemm_destroy(void);

/*
 * C = alpha * A x B + beta * C in FP32 (section 问题与估算 of the SGEMM page),
 * computed with FP32 multiply-accumulate (MFMA, round to nearest even).
 *   M, N, K >= 0; A: M x K (lda), B: K x N (ldb), C: M x N (ldc), device pointers.
 *   beta == 0: C is write-only (NaN or Inf already in C does not propagate).
 *   alpha == 0 or K == 0: A and B are not read; C = beta * C.
 *   M == 0 or N == 0: nothing is done.
 * A null pointer is accepted only for an operand that is not read.
 */
int sgemm(int M, int N, int K, float alpha,
          const float* A, int lda, const float* B, int ldb,
          float beta, float* C, int ldc, hipStream_t stream);

/*
 * sgemm for callers that cannot allocate device memory on the call path: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, layout, conventions and errors as sgemm, and the
 * same kernels; it calls no hipMalloc, hipFree or allocating library routine.
 * Its split-K partial sums live in a static device array of 16 MiB (4 Mi
 * floats; one copy per GPU, held until the process ends) instead of the
 * workspace gemm_create allocates: split counts are limited to
 * splits * M * N <= 4 Mi, and operands whose rows are off 16-byte boundaries
 * are read by the bounds-checked kernels instead of being copied.  A plan that
 * would need more scratch returns GEMM_STATUS_INVALID_VALUE.  Needs
 * gemm_create, which looks the array up on its device (another device's is
 * looked up by the first call there).  Every sgemm_noalloc call on one GPU
 * shares that GPU's array, which keeps the last call's contents; calls that
 * overlap on one GPU (different streams, or a graph replayed while another
 * call runs) race.
 */
int sgemm_noalloc(int M, int N, int K, float alpha,
                  const float* A, int lda, const float* B, int ldb,
                  float beta, float* C, int ldc, hipStream_t stream);

/*
 * C = act(alpha * A x B + bias) with A (M x K) and B (K x N) in IEEE binary16
 * (passed as uint16_t bit patterns), FP32 accumulation, an FP32 bias of length
 * N added to every row (NULL = no bias), the activation `act` (gemm_act_t) and
 * C written as binary16, rounded to nearest even.  This is the fused epilogue
 * of the DeepGEMM page: bias, scale and activation applied in registers before
 * one store.  alpha == 0 or K == 0: A and B are not read.
 */
int hgemm_bias_act(int M, int N, int K, float alpha,
                   const uint16_t* A, int lda, const uint16_t* B, int ldb,
                   const float* bias, int act,
                   uint16_t* C, int ldc, hipStream_t stream);

/*
 * The same product with bfloat16 inputs and output (the upper 16 bits of an
 * IEEE binary32, passed as uint16_t bit patterns): C = act(alpha * A x B +
 * bias), FP32 accumulation, C rounded to nearest even.  Arguments, layout,
 * conventions and errors are those of hgemm_bias_act.
 */
int bgemm_bias_act(int M, int N, int K, float alpha,
                   const uint16_t* A, int lda, const uint16_t* B, int ldb,
                   const float* bias, int act,
                   uint16_t* C, int ldc, hipStream_t stream);

/* Static text for a status code; for GEMM_STATUS_HIP_ERROR it also names the
 * last HIP error seen by the library on this host thread. */
const char* gemm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* LINEAR_ALGEBRA_SGEMM_AMD_GEMM_H */
