// Small memory-bound kernels of the stage path: strided zero fill (the Q and
// K columns of dQKV when attention is the identity), the non-finite check of
// the gradient buffers at the step boundary, and flag clearing.  Fills are
// kernels rather than hipMemsetAsync so that the path can be graph-captured.
#include <hip/hip_runtime.h>

#include "zb_internal.h"

namespace zb {
namespace {

// rows x cols elements of elem_bytes (2 or 4) each, row stride ld elements.
// 16-byte stores where the row segment allows, scalar stores otherwise.
__global__ void zero2d_kernel(char* p, int64_t rows, int64_t row_bytes, int64_t ld_bytes) {
  const int64_t vec_per_row = row_bytes / 16;
  const int64_t tail = row_bytes - vec_per_row * 16;
  const int64_t total = rows * (vec_per_row + tail / 2);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t per = vec_per_row + tail / 2;
    const int64_t r = i / per, c = i % per;
    char* row = p + r * ld_bytes;
    if (c < vec_per_row)
      *reinterpret_cast<uint4*>(row + c * 16) = make_uint4(0u, 0u, 0u, 0u);
    else
      *reinterpret_cast<uint16_t*>(row + vec_per_row * 16 + (c - vec_per_row) * 2) = 0;
  }
}

__global__ void nonfinite_kernel(const float* __restrict__ p, int64_t n, int* flag) {
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t u = __float_as_uint(p[i]);
    bad |= (u & 0x7f800000u) == 0x7f800000u;
  }
  if (__any(bad) && (threadIdx.x & 63) == 0) *flag = 1;
}

__global__ void zero_int_kernel(int* p) { *p = 0; }

}  // namespace

zb_status launch_zero2d(void* p, int64_t rows, int64_t cols, int64_t ld, int elem_bytes, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return ZB_OK;
  const int64_t row_bytes = cols * elem_bytes, ld_bytes = ld * elem_bytes;
  if ((reinterpret_cast<uintptr_t>(p) & 15u) || (ld_bytes & 15) || (row_bytes & 1))
    return set_error(ZB_E_UNSUPPORTED, "zero2d: rows must be 16-byte aligned");
  const int64_t per = row_bytes / 16 + (row_bytes % 16) / 2;
  const int64_t total = rows * per;
  const int threads = 256;
  const int64_t blocks = std::min<int64_t>((total + threads - 1) / threads, 4096);
  ProfScope ps("zero2d", 0.0, (double)rows * row_bytes, s);
  hipLaunchKernelGGL(zero2d_kernel, dim3((unsigned)blocks), dim3(threads), 0, s, static_cast<char*>(p), rows,
                     row_bytes, ld_bytes);
  ZB_HIP_CHECK(hipGetLastError());
  return ZB_OK;
}

zb_status launch_nonfinite(const float* p, int64_t n, int* flag, hipStream_t s) {
  if (n <= 0) return ZB_OK;
  const int threads = 256;
  const int64_t blocks = std::min<int64_t>((n + threads - 1) / threads, 2048);
  hipLaunchKernelGGL(nonfinite_kernel, dim3((unsigned)blocks), dim3(threads), 0, s, p, n, flag);
  ZB_HIP_CHECK(hipGetLastError());
  return ZB_OK;
}

zb_status launch_zero_int(int* flag, hipStream_t s) {
  hipLaunchKernelGGL(zero_int_kernel, dim3(1), dim3(1), 0, s, flag);
  ZB_HIP_CHECK(hipGetLastError());
  return ZB_OK;
}

}  // namespace zb
