// Operand copies into the library's pack buffer: rows re-laid on 16-byte
// boundaries, zero-filled past the matrix (extra columns, and for the padded
// FP32 copies extra rows), so the product kernels can read them in whole
// 16-byte chunks.  Plain copies, bound by HBM bandwidth: each thread writes one
// 16-byte chunk (consecutive threads take consecutive chunks of the row-major
// copy, so a wave covers 1 KiB), reads the source with one 16-byte load when the
// source row allows it and element by element otherwise.  Up to two operands go
// in one launch (grid y).

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gemm_launch.h"

namespace lasg {

namespace {

constexpr int kPackMaxBlocks = 16384;

struct PackJobs {
  PackJob job[2];
};

template <class E>
__global__ void __launch_bounds__(256) pack_rows_kernel(PackJobs jobs) {
  constexpr int V = 16 / (int)sizeof(E);
  const PackJob j = jobs.job[blockIdx.y];
  const E* src = static_cast<const E*>(j.src);
  E* dst = static_cast<E*>(j.dst);
  const bool src_vec = reinterpret_cast<uintptr_t>(src) % 16 == 0 && j.lds % V == 0;
  const uint32_t chunks = (uint32_t)(j.ldd / V);   // per destination row
  const uint32_t total = chunks * (uint32_t)j.dst_rows;
  for (uint32_t t = blockIdx.x * 256u + threadIdx.x; t < total; t += gridDim.x * 256u) {
    const int r = (int)(t / chunks);
    const int c = (int)(t - (uint32_t)r * chunks) * V;   // first destination column
    union {
      uint4 u;
      E e[V];
    } v;
    const E* row = src + (size_t)r * j.lds;
    if (r < j.rows && src_vec && c + V <= j.cols) {
      v.u = *reinterpret_cast<const uint4*>(row + c);
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) v.e[i] = (r < j.rows && c + i < j.cols) ? row[c + i] : E(0);
    }
    *reinterpret_cast<uint4*>(dst + (size_t)r * j.ldd + c) = v.u;
  }
}

}  // namespace

hipError_t launch_pack(const PackJob* jobs, int count, int elem_bytes, hipStream_t s) {
  if (count < 1 || count > 2 || (elem_bytes != 4 && elem_bytes != 2)) return hipErrorInvalidValue;
  const int V = 16 / elem_bytes;
  PackJobs pj;
  int64_t max_total = 0;
  for (int i = 0; i < count; ++i) {
    const PackJob& j = jobs[i];
    if (j.rows < 0 || j.cols < 0 || j.dst_rows < j.rows || j.ldd < j.cols || j.ldd % V != 0 ||
        reinterpret_cast<uintptr_t>(j.dst) % 16 != 0 || (j.rows > 0 && j.lds < j.cols) ||
        (j.rows > 0 && j.cols > 0 && j.src == nullptr) || (j.dst_rows > 0 && j.dst == nullptr))
      return hipErrorInvalidValue;
    const int64_t total = (int64_t)(j.ldd / V) * j.dst_rows;
    if (total >= (int64_t(1) << 32) - 256LL * kPackMaxBlocks) return hipErrorInvalidValue;
    pj.job[i] = j;
    if (total > max_total) max_total = total;
  }
  if (count == 1) {
    pj.job[1] = pj.job[0];
  }
  if (max_total == 0) return hipSuccess;
  int64_t blocks = (max_total + 255) / 256;
  if (blocks > kPackMaxBlocks) blocks = kPackMaxBlocks;
  const dim3 grid((unsigned)blocks, (unsigned)count);
  if (elem_bytes == 4)
    hipLaunchKernelGGL(pack_rows_kernel<float>, grid, dim3(256), 0, s, pj);
  else
    hipLaunchKernelGGL(pack_rows_kernel<uint16_t>, grid, dim3(256), 0, s, pj);
  return hipGetLastError();
}

}  // namespace lasg
