// Small memory-bound kernels of the stage path: strided zero fill (the Q and
// K columns of dQKV when attention is the identity), the non-finite check of
// the gradient buffers at the step boundary, flag clearing, and the GeLU that
// rebuilds the MLP activation A = gelu(Z) from the saved pre-activation for W.  Fills are
// kernels rather than hipMemsetAsync so that the path can be graph-captured.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.h"
#include "zb_internal.h"

namespace zb {
namespace {

// rows x cols elements of elem_bytes (2 or 4) each, row stride ld elements.
// 16-byte stores where the row segment allows, 2-byte stores for its tail.
// Rows go over blockIdx.y and chunks of a row over x, so no thread divides.
__global__ void zero2d_kernel(char* p, int64_t rows, int64_t row_bytes, int64_t ld_bytes) {
  const int64_t vec = row_bytes / 16;
  const int64_t per = vec + (row_bytes - vec * 16) / 2;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    char* row = p + r * ld_bytes;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < per; c += (int64_t)gridDim.x * blockDim.x) {
      if (c < vec)
        *reinterpret_cast<uint4*>(row + c * 16) = make_uint4(0u, 0u, 0u, 0u);
      else
        *reinterpret_cast<uint16_t*>(row + vec * 16 + (c - vec) * 2) = 0;
    }
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

// A = gelu(Z), bf16: 8 elements per thread (n % 8 == 0, 16-byte aligned), with
// the GeLU of the forward epilogue.  The forward took GeLU of the fp32
// pre-activation, this takes it of the stored bf16 Z: the two activations
// agree to within one bf16 rounding, and every schedule order rebuilds the
// same bits.
__global__ void gelu_bf16_kernel(const uint4* __restrict__ z, uint4* __restrict__ a, int64_t n8, int kind) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    const uint4 v = z[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = dev::pack_bf16x2(dev::gelu_f(__uint_as_float(w[e] << 16), kind),
                              dev::gelu_f(__uint_as_float(w[e] & 0xffff0000u), kind));
    a[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

__global__ void gelu_f32_kernel(const float* __restrict__ z, float* __restrict__ a, int64_t n, int kind) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    a[i] = dev::gelu_f(z[i], kind);
}

}  // namespace

zb_status launch_gelu(const void* z, void* a, int64_t n, int dtype, int kind, hipStream_t s) {
  if (n <= 0) return ZB_OK;
  const int64_t units = dtype == ZB_DTYPE_BF16 ? n / 8 : n;
  if (dtype == ZB_DTYPE_BF16 && (n % 8 || (reinterpret_cast<uintptr_t>(z) | reinterpret_cast<uintptr_t>(a)) & 15))
    return set_error(ZB_E_UNSUPPORTED, "gelu: bf16 needs a multiple of 8 elements, 16-byte aligned");
  const int64_t blocks = std::min<int64_t>((units + 255) / 256, 4096);
  ProfScope ps("gelu_recompute", 0.0, (dtype == ZB_DTYPE_BF16 ? 4.0 : 8.0) * n, s);
  if (dtype == ZB_DTYPE_BF16)
    hipLaunchKernelGGL(gelu_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const uint4*>(z),
                       static_cast<uint4*>(a), units, kind);
  else
    hipLaunchKernelGGL(gelu_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const float*>(z),
                       static_cast<float*>(a), units, kind);
  ZB_HIP_CHECK(hipGetLastError());
  return ZB_OK;
}

zb_status launch_zero2d(void* p, int64_t rows, int64_t cols, int64_t ld, int elem_bytes, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return ZB_OK;
  const int64_t row_bytes = cols * elem_bytes, ld_bytes = ld * elem_bytes;
  if ((reinterpret_cast<uintptr_t>(p) & 15u) || (ld_bytes & 15) || (row_bytes & 1))
    return set_error(ZB_E_UNSUPPORTED, "zero2d: rows must be 16-byte aligned");
  const int64_t per = row_bytes / 16 + (row_bytes % 16) / 2;
  const int threads = 256;
  const dim3 grid((unsigned)std::min<int64_t>((per + threads - 1) / threads, 64),
                  (unsigned)std::min<int64_t>(rows, 4096));
  ProfScope ps("zero2d", 0.0, (double)rows * row_bytes, s);
  hipLaunchKernelGGL(zero2d_kernel, grid, dim3(threads), 0, s, static_cast<char*>(p), rows, row_bytes, ld_bytes);
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
