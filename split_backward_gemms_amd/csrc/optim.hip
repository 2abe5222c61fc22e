// Optimizer step of one stage with post-update validation ("Zero Bubble
// Pipeline Parallelism", section 4, and its Appendix C in-place rollback).
//
// The gradient state of a stage is {sum of squared dW, non-finite flag}, kept
// as two doubles.  sumsq_kernel writes one fp64 partial per workgroup in a
// fixed grid, state_combine_kernel folds every partial of the stage in a fixed
// order and adds the upstream stage's state: the same gradients always give
// the same bits.  adamw_kernel is the elementwise update (and its inverse);
// every thread derives the clip coefficient and the skip / rollback decision
// from the same device-resident doubles, so no host round trip is needed.
// All three are bound by HBM traffic.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "zb_internal.h"

namespace zb {
namespace {

constexpr int kThreads = 256;

__device__ inline bool finite_f(float x) { return (__float_as_uint(x) & 0x7f800000u) != 0x7f800000u; }

__device__ inline void block_sum2(double& a, double& b, double* sa, double* sb) {
  const int t = threadIdx.x;
  sa[t] = a;
  sb[t] = b;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (t < w) {
      sa[t] += sa[t + w];
      sb[t] += sb[t + w];
    }
    __syncthreads();
  }
  a = sa[0];
  b = sb[0];
}

__global__ void __launch_bounds__(kThreads) sumsq_kernel(const float* __restrict__ g, int64_t n,
                                                          double* __restrict__ part) {
  __shared__ double sa[kThreads], sb[kThreads];
  double acc = 0.0, bad = 0.0;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int64_t n4 = n >> 2;
  const float4* g4 = reinterpret_cast<const float4*>(g);
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride) {
    const float4 x = g4[i];
    acc += (double)x.x * x.x + (double)x.y * x.y + (double)x.z * x.z + (double)x.w * x.w;
    bad += (finite_f(x.x) && finite_f(x.y) && finite_f(x.z) && finite_f(x.w)) ? 0.0 : 1.0;
  }
  for (int64_t i = (n4 << 2) + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
    const float x = g[i];
    acc += (double)x * x;
    bad += finite_f(x) ? 0.0 : 1.0;
  }
  block_sum2(acc, bad, sa, sb);
  if (threadIdx.x == 0) {
    part[2 * blockIdx.x] = acc;
    part[2 * blockIdx.x + 1] = bad;
  }
}

// out = upstream (may be null) + sum of `count` (sumsq, bad) partials.
__global__ void __launch_bounds__(kThreads) state_combine_kernel(const double* __restrict__ part, int count,
                                                                  const double* __restrict__ up,
                                                                  double* __restrict__ out) {
  __shared__ double sa[kThreads], sb[kThreads];
  double acc = 0.0, bad = 0.0;
  for (int i = threadIdx.x; i < count; i += kThreads) {
    acc += part[2 * i];
    bad += part[2 * i + 1];
  }
  block_sum2(acc, bad, sa, sb);
  if (threadIdx.x == 0) {
    double s = acc, f = bad != 0.0 ? 1.0 : 0.0;
    if (up) {
      s += up[0];
      f = (f != 0.0 || up[1] != 0.0) ? 1.0 : 0.0;
    }
    out[0] = s;
    out[1] = f;
  }
}

struct AdamArgs {
  float lr, b1, b2, eps, wd, max_norm, bc1, bc2;
};

// Clip coefficient of a step taken with `st`; false = no update (NaN/Inf seen).
__device__ inline bool coef_of(const double* st, float max_norm, float& c) {
  const double s = st[0];
  if (st[1] != 0.0 || !(s <= 1.7976931348623157e308)) return false;
  c = 1.0f;
  if (max_norm > 0.0f) c = (float)fmin(1.0, (double)max_norm / (sqrt(s) + 1e-6));
  return true;
}

__device__ inline void adam_fwd(float& th, float& m, float& v, float g, const AdamArgs& a) {
  m = a.b1 * m + (1.0f - a.b1) * g;
  v = a.b2 * v + (1.0f - a.b2) * g * g;
  const float denom = sqrtf(v / a.bc2) + a.eps;
  th = th - a.lr * a.wd * th - a.lr * (m / a.bc1) / denom;
}

__device__ inline void adam_inv(float& th, float& m, float& v, float g, const AdamArgs& a) {
  const float denom = sqrtf(v / a.bc2) + a.eps;
  th = (th + a.lr * (m / a.bc1) / denom) / (1.0f - a.lr * a.wd);
  m = (m - (1.0f - a.b1) * g) / a.b1;
  v = fmaxf((v - (1.0f - a.b2) * g * g) / a.b2, 0.0f);
}

enum { MODE_STEP = 0, MODE_VALIDATE = 1, MODE_ROLLBACK = 2 };

// One tensor of the stage: master params, moments, gradient, and the working
// copy the GEMMs read (bf16 rounded to nearest even, or fp32).
__global__ void __launch_bounds__(kThreads) adamw_kernel(float* __restrict__ th, float* __restrict__ mm,
                                                          float* __restrict__ vv, const float* __restrict__ gr,
                                                          void* __restrict__ w, int w_bf16, int64_t n, AdamArgs a,
                                                          const double* __restrict__ used,
                                                          const double* __restrict__ glob, int mode,
                                                          int* __restrict__ rolled) {
  float cu = 0.0f, cg = 0.0f, ci = 0.0f, cf = 0.0f;
  const bool su = coef_of(used, a.max_norm, cu);
  bool inv = false, fwd = false;
  if (mode == MODE_STEP) {
    fwd = su;
    cf = cu;
  } else if (mode == MODE_ROLLBACK) {
    inv = su;
    ci = cu;
  } else {
    const bool sg = coef_of(glob, a.max_norm, cg);
    const bool same = su == sg && (!su || cu == cg);
    if (!same) {
      inv = su;
      ci = cu;
      fwd = sg;
      cf = cg;
    }
    if (rolled && blockIdx.x == 0 && threadIdx.x == 0) *rolled = same ? 0 : 1;
  }
  if (!inv && !fwd) return;
  auto one = [&](float& t, float& m, float& v, float g) {
    if (inv) adam_inv(t, m, v, ci * g, a);
    if (fwd) adam_fwd(t, m, v, cf * g, a);
  };
  auto bf16 = [](float t) -> uint32_t {
    const uint32_t u = __float_as_uint(t);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  };
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  // Four elements per thread with 16-byte accesses (every buffer is 16-byte
  // aligned); the n % 4 tail one by one.
  const int64_t n4 = n >> 2;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride) {
    float4 t = reinterpret_cast<const float4*>(th)[i];
    float4 m = reinterpret_cast<const float4*>(mm)[i];
    float4 v = reinterpret_cast<const float4*>(vv)[i];
    const float4 g = reinterpret_cast<const float4*>(gr)[i];
    one(t.x, m.x, v.x, g.x);
    one(t.y, m.y, v.y, g.y);
    one(t.z, m.z, v.z, g.z);
    one(t.w, m.w, v.w, g.w);
    reinterpret_cast<float4*>(th)[i] = t;
    reinterpret_cast<float4*>(mm)[i] = m;
    reinterpret_cast<float4*>(vv)[i] = v;
    if (w_bf16)
      reinterpret_cast<uint2*>(w)[i] = make_uint2(bf16(t.x) | (bf16(t.y) << 16), bf16(t.z) | (bf16(t.w) << 16));
    else
      reinterpret_cast<float4*>(w)[i] = t;
  }
  for (int64_t i = (n4 << 2) + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
    float t = th[i], m = mm[i], v = vv[i];
    one(t, m, v, gr[i]);
    th[i] = t;
    mm[i] = m;
    vv[i] = v;
    if (w_bf16)
      reinterpret_cast<uint16_t*>(w)[i] = (uint16_t)bf16(t);
    else
      reinterpret_cast<float*>(w)[i] = t;
  }
}

int grid_for(int64_t n) {
  const int64_t want = (n + 4LL * kThreads - 1) / (4LL * kThreads);
  return (int)std::max<int64_t>(1, std::min<int64_t>(want, kSumsqBlocks));
}

}  // namespace

int grad_sumsq_blocks(int64_t n) { return grid_for(n); }

zb_status launch_grad_sumsq(const float* g, int64_t n, double* part, int* blocks_out, hipStream_t s) {
  const int grid = grid_for(n);
  ProfScope ps("grad_sumsq", 0.0, 4.0 * (double)n, s);
  hipLaunchKernelGGL(sumsq_kernel, dim3(grid), dim3(kThreads), 0, s, g, n, part);
  ZB_HIP_CHECK(hipGetLastError());
  *blocks_out = grid;
  return ZB_OK;
}

zb_status launch_state_combine(const double* part, int count, const double* up, double* out, hipStream_t s) {
  hipLaunchKernelGGL(state_combine_kernel, dim3(1), dim3(kThreads), 0, s, part, count, up, out);
  ZB_HIP_CHECK(hipGetLastError());
  return ZB_OK;
}

zb_status launch_adamw(const AdamwLaunch& L, hipStream_t s) {
  if (L.n <= 0) return ZB_OK;
  AdamArgs a;
  a.lr = L.hp.lr;
  a.b1 = L.hp.beta1;
  a.b2 = L.hp.beta2;
  a.eps = L.hp.eps;
  a.wd = L.hp.weight_decay;
  a.max_norm = L.hp.max_grad_norm;
  a.bc1 = (float)L.bc1;
  a.bc2 = (float)L.bc2;
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>((L.n / 4 + kThreads - 1) / kThreads, 8192));
  static const char* names[3] = {"adamw_step", "adamw_validate", "adamw_rollback"};
  // Bytes of an update (validation moves them only when it rolls back).
  const double bytes = L.mode == 1 ? 0.0 : (28.0 + (L.w_bf16 ? 2.0 : 4.0)) * (double)L.n;
  ProfScope ps(names[L.mode], 0.0, bytes, s);
  hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, L.theta, L.m, L.v, L.g, L.w,
                     L.w_bf16, L.n, a, L.used, L.glob, L.mode, L.rolled);
  ZB_HIP_CHECK(hipGetLastError());
  return ZB_OK;
}

}  // namespace zb
