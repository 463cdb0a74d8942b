// Operand copies into the library's pack buffer: rows re-laid on 16-byte
// boundaries, zero-filled past the matrix (extra columns, and for the padded
// FP32 copies extra rows), so the product kernels can read them in whole
// 16-byte chunks.  Plain copies, bound by HBM bandwidth: each thread writes one
// 16-byte chunk per row it visits (a 64-lane wave covers 1 KiB of a row), reads
// the source with one 16-byte load when the source row allows it and element
// by element otherwise.  Up to two operands go in one launch (grid z).

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gemm_launch.h"

namespace lasg {

namespace {

constexpr int kPackRowsPerBlock = 4;   // 256 threads: 64 chunks of 4 rows
constexpr int kPackMaxGridY = 16384;

struct PackJobs {
  PackJob job[2];
};

template <class E>
__global__ void __launch_bounds__(256) pack_rows_kernel(PackJobs jobs) {
  constexpr int V = 16 / (int)sizeof(E);
  const PackJob j = jobs.job[blockIdx.z];
  const int c = (int)(blockIdx.x * 64 + threadIdx.x % 64) * V;   // first destination column
  if (c >= j.ldd) return;
  const E* src = static_cast<const E*>(j.src);
  E* dst = static_cast<E*>(j.dst);
  const bool vec = reinterpret_cast<uintptr_t>(src) % 16 == 0 && j.lds % V == 0 && c + V <= j.cols;
  for (int r = (int)(blockIdx.y * kPackRowsPerBlock + threadIdx.x / 64); r < j.dst_rows;
       r += (int)gridDim.y * kPackRowsPerBlock) {
    union {
      uint4 u;
      E e[V];
    } v;
    const E* row = src + (size_t)r * j.lds;
    if (r < j.rows && vec) {
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
  int64_t max_chunks = 0, max_rows = 0;
  for (int i = 0; i < count; ++i) {
    const PackJob& j = jobs[i];
    if (j.rows < 0 || j.cols < 0 || j.dst_rows < j.rows || j.ldd < j.cols || j.ldd % V != 0 ||
        reinterpret_cast<uintptr_t>(j.dst) % 16 != 0 || (j.rows > 0 && j.lds < j.cols) ||
        (j.rows > 0 && j.cols > 0 && j.src == nullptr) || (j.dst_rows > 0 && j.dst == nullptr))
      return hipErrorInvalidValue;
    pj.job[i] = j;
    const int64_t chunks = j.ldd / V;
    if (chunks > max_chunks) max_chunks = chunks;
    if (j.dst_rows > max_rows) max_rows = j.dst_rows;
  }
  if (count == 1) {
    pj.job[1] = pj.job[0];
  }
  if (max_chunks == 0 || max_rows == 0) return hipSuccess;
  int64_t gy = (max_rows + kPackRowsPerBlock - 1) / kPackRowsPerBlock;
  if (gy > kPackMaxGridY) gy = kPackMaxGridY;
  const dim3 grid((unsigned)((max_chunks + 63) / 64), (unsigned)gy, (unsigned)count);
  if (elem_bytes == 4)
    hipLaunchKernelGGL(pack_rows_kernel<float>, grid, dim3(256), 0, s, pj);
  else
    hipLaunchKernelGGL(pack_rows_kernel<uint16_t>, grid, dim3(256), 0, s, pj);
  return hipGetLastError();
}

}  // namespace lasg
