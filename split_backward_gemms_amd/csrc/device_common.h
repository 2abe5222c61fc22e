// Device helpers shared by the GEMM and attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/zb.h"

namespace zb {
namespace dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Out-of-range byte offset for buffer accesses: every operand extent is below
// 2 GiB (checked on the host), so kOOB plus any in-range step stays out of
// range without wrapping; loads there return zero and stores are dropped.
constexpr uint32_t kOOB = 0x80000000u;
constexpr uint32_t kRsrcWord3 = 0x00020000u;

// Buffer descriptor (gfx9): 48-bit base, stride 0, extent in bytes, raw
// addressing with range checking against the extent.
__device__ __forceinline__ u32x4 make_rsrc4(const void* base, uint32_t extent_bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r[0] = (uint32_t)b;
  r[1] = (uint32_t)(b >> 32) & 0xffffu;
  r[2] = extent_bytes;
  r[3] = kRsrcWord3;
  return r;
}

// 16 bytes per lane from rsrc at byte offset off (zero when out of range)
// into LDS at lds + 16 * lane; lds must be wave-uniform.  Issued with inline
// assembly, so the compiler does not track these copies: every wait for them
// is explicit (wait_vm_barrier).
__device__ __forceinline__ void dma16(const u32x4& rsrc, uint32_t lds, uint32_t off) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(rsrc), "{m0}"(lds) : "memory");
}

// Lets at most N of this wave's vector-memory operations stay in flight,
// drains its LDS operations, and meets the other waves at the barrier: after
// it, the copies each wave issued before its last N are visible to all.  The
// memory clobber keeps the compiler from moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

// Round to nearest even, two at a time (v_cvt_pk_bf16_f32); NaN stays NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Standard normal CDF Phi(z) and exp(-z^2/2) without branches: erf(x) for
// x >= 0 by Abramowitz & Stegun, Handbook of Mathematical Functions, formula
// 7.1.26 (absolute error <= 1.5e-7),
//   erf(x) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-x^2),  t = 1 / (1 + p x),
// with erf(-x) = -erf(x); the reciprocal and exp2 run on the hardware
// transcendental unit.  At x = |z| / sqrt(2), exp(-x^2) is exp(-z^2 / 2).
struct NormalParts {
  float cdf;  // Phi(z)
  float e;    // exp(-z^2 / 2)
};
__device__ __forceinline__ NormalParts normal_parts(float z) {
  const float x = fabsf(z) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
  float poly = fmaf(1.061405429f, t, -1.453152027f);
  poly = fmaf(poly, t, 1.421413741f);
  poly = fmaf(poly, t, -0.284496736f);
  poly = fmaf(poly, t, 0.254829592f);
  poly *= t;
  const float e = __builtin_amdgcn_exp2f(-(x * x) * 1.4426950408889634f);
  const float erf_z = copysignf(1.0f - poly * e, z);
  return {fmaf(0.5f, erf_z, 0.5f), e};
}

// gelu(z) = z Phi(z); the tanh form is kept for callers that ask for it.
__device__ __forceinline__ float gelu_f(float z, int kind) {
  if (kind == ZB_GELU_TANH) {
    const float c = 0.7978845608028654f;  // sqrt(2/pi)
    float u = c * (z + 0.044715f * z * z * z);
    return 0.5f * z * (1.0f + tanhf(u));
  }
  return z * normal_parts(z).cdf;
}

// gelu'(z) = Phi(z) + z phi(z), phi(z) = exp(-z^2 / 2) / sqrt(2 pi).
__device__ __forceinline__ float gelu_grad_f(float z, int kind) {
  if (kind == ZB_GELU_TANH) {
    const float c = 0.7978845608028654f;
    float u = c * (z + 0.044715f * z * z * z);
    float t = tanhf(u);
    return 0.5f * (1.0f + t) + 0.5f * z * (1.0f - t * t) * c * (1.0f + 3.0f * 0.044715f * z * z);
  }
  const NormalParts n = normal_parts(z);
  return fmaf(z * n.e, 0.3989422804014327f, n.cdf);
}

}  // namespace dev
}  // namespace zb
