// Causal softmax attention of the FULL layer (head dim 128), bf16 in, fp32 math.
//
// Per head and sequence: S = Q K^T / sqrt(128), S_ij = -inf for j > i,
// P = softmax over each row, O = P V.  Backward: dV = P^T dO, dP = dO V^T,
// dS = P * (dP - D) with D_i = sum_d dO_id O_id, dQ = dS K / sqrt(128),
// dK = dS^T Q / sqrt(128).  (Attention is the 4s / 8s term of the forward and
// input-gradient FLOP counts in "Zero Bubble Pipeline Parallelism", section 2,
// Table 1; it has no parameters, so all of its backward belongs to B.)
//
// Layouts: QKV [T, 3h] (Q | K | V column blocks, head hd at columns hd*128..),
// O, dO [T, h], LSE2 and D [heads, T] fp32.  T = micro_batch * seq rows;
// sequence b owns rows b*seq .. b*seq+seq-1.  LSE2 is the row's log-sum-exp of
// S * log2(e) (base-2 domain), which the backward reuses to rebuild P.
//
// Every product is a v_mfma_f32_32x32x16_bf16 written as D[p][c] = sum_k
// X[p][k] Y[k][c]: lane l supplies row p = l%32 of X and column c = l%32 of Y
// for its half h = l/32 of k, and receives D[p][c = l%32] for the 16 rows
// p = 8g + 4h + t.  Operands contracted over the head dimension use the k set
// {8h..8h+7}; operands contracted over sequence positions use {4h..4h+3,
// 8+4h..8+4h+3}, which is exactly the row set a lane receives, so a product's
// output (rows = sequence positions) feeds the next product's Y operand from
// registers.  Forward and dQ keep one query row per lane column; dK/dV keep
// one key row per lane column.
//
// Determinism: dQ and dK/dV are separate passes (query-block and key-block
// parallel); no atomics, fixed summation order.
#include <hip/hip_runtime.h>

#include "zb_internal.h"

namespace zb {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int HD = 128;        // head dim
constexpr int NT = 256;        // 4 waves
constexpr uint32_t kOOB = 0x80000000u;
constexpr int kRsrcWord3 = 0x00020000;
constexpr float kLog2e = 1.4426950408889634f;

struct AttnParams {
  const uint16_t* qkv;  // [T, 3h]
  uint16_t* o;          // [T, h]   (forward output / backward input)
  float* lse2;          // [a, T]
  const uint16_t* dout; // [T, h]
  float* dsum;          // [a, T]   D = rowsum(dO * O)
  uint16_t* dqkv;       // [T, 3h]
  int T, h, heads, seq, nseq;
  float scale;          // 1/sqrt(128)
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t extent) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)extent, kRsrcWord3);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ void bstore8(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, 0);
}

__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ uint32_t pack2(float a, float b) { return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 8 fp32 -> bf16x8 fragment
__device__ __forceinline__ bf16x8 to_frag(const float* v) {
  u32x4 u = {pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7])};
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 x, bf16x8 y, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.0f;
  return z;
}

// ---- LDS tiles -------------------------------------------------------------
// "Row" tile [R][128] bf16: 256 bytes per row, 16-byte chunk c at (c ^ (row % 8)).
__device__ __forceinline__ uint32_t row_off(int row, int chunk) { return row * 256 + ((chunk ^ (row & 7)) << 4); }
// "Transposed" tile [128][64] bf16 (rows = head dim, 64 sequence positions):
// 128 bytes per row; chunk c (8 positions) at c ^ (row % 8), its two 8-byte
// halves swapped when (row / 8) is odd.
__device__ __forceinline__ uint32_t tr_off(int row, int chunk, int half) {
  return row * 128 + ((chunk ^ (row & 7)) << 4) + ((half ^ ((row >> 3) & 1)) << 3);
}

// X fragment, contracted over the head dim, from a row tile: row p, k = 16 kk + 8h .. +7.
__device__ __forceinline__ bf16x8 frag_row(const char* base, int row, int kk, int h) {
  return *reinterpret_cast<const bf16x8*>(base + row_off(row, 2 * kk + h));
}
// X fragment, contracted over positions, from a transposed tile: row p (head dim),
// positions 16 s + {4h..4h+3, 8+4h..8+4h+3}.
__device__ __forceinline__ bf16x8 frag_tr(const char* base, int row, int s, int h) {
  const u32x2 a = *reinterpret_cast<const u32x2*>(base + tr_off(row, 2 * s, h));
  const u32x2 b = *reinterpret_cast<const u32x2*>(base + tr_off(row, 2 * s + 1, h));
  u32x4 u = {a[0], a[1], b[0], b[1]};
  return __builtin_bit_cast(bf16x8, u);
}

// Cooperative loads of 64 sequence rows x 128 head dims (one head's block).
// Rows at or past `valid` (end of the sequence) read as zero.
// Row tile: 64 rows x 16 chunks = 1024 chunks, 4 per thread.
__device__ __forceinline__ void load_row_tile(char* lds, __amdgpu_buffer_rsrc_t r, int64_t row0, int valid,
                                              int64_t ld, int col0, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (tid >> 4) + 16 * i, c = tid & 15;
    const uint32_t off = row < valid ? (uint32_t)(((row0 + row) * ld + col0 + 8 * c) * 2) : kOOB;
    *reinterpret_cast<u32x4*>(lds + row_off(row, c)) = bload16(r, off);
  }
}
// Transposed tile: thread takes 4 rows x 8 head dims, writes 8 head-dim rows x 4 positions.
__device__ __forceinline__ void load_tr_tile(char* lds, __amdgpu_buffer_rsrc_t r, int64_t row0, int valid, int64_t ld,
                                             int col0, int tid) {
  const int dc = tid & 15, kg = tid >> 4;  // head dims 8dc..8dc+7, positions 4kg..4kg+3
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * kg + i;
    const uint32_t off = row < valid ? (uint32_t)(((row0 + row) * ld + col0 + 8 * dc) * 2) : kOOB;
    v[i] = bload16(r, off);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t w = e >> 1;
    uint32_t x0 = v[0][w], x1 = v[1][w], x2 = v[2][w], x3 = v[3][w];
    if (e & 1) {
      x0 >>= 16; x1 >>= 16; x2 >>= 16; x3 >>= 16;
    }
    const u32x2 out = {(x0 & 0xffffu) | (x1 << 16), (x2 & 0xffffu) | (x3 << 16)};
    const int drow = 8 * dc + e;
    *reinterpret_cast<u32x2*>(lds + tr_off(drow, kg >> 1, kg & 1)) = out;
  }
}

// ============================================================== forward
// Workgroup: 128 query rows (32 per wave) of one (sequence, head); keys in blocks of 64.
__global__ void __launch_bounds__(NT) attn_fwd(AttnParams p) {
  __shared__ __attribute__((aligned(16))) char lds[64 * 256 + 128 * 128];
  char* sK = lds;             // [64][128] row tile
  char* sVt = lds + 64 * 256; // [128][64] transposed
  const int nqb = (p.seq + 127) / 128;
  const int qb = nqb - 1 - (int)blockIdx.x;  // heaviest blocks first
  const int hd = blockIdx.y % p.heads, sq = blockIdx.y / p.heads;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, lc = lane & 31;
  const int64_t ld3 = 3LL * p.h, base_row = (int64_t)sq * p.seq;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.qkv, (uint32_t)((int64_t)p.T * ld3 * 2));
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.o, (uint32_t)((int64_t)p.T * p.h * 2));
  const float c = p.scale * kLog2e;

  const int q = qb * 128 + 32 * w + lc;  // this lane's query row
  const bool qv = q < p.seq;
  bf16x8 qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const uint32_t off = qv ? (uint32_t)(((base_row + q) * ld3 + hd * HD + 16 * kk + 8 * h) * 2) : kOOB;
    qf[kk] = __builtin_bit_cast(bf16x8, bload16(rq, off));
  }
  f32x16 o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) o[d] = zero16();
  float m = -INFINITY, l = 0.0f;
  const int q_wave_max = qb * 128 + 32 * w + 31;
  const int nkb = min((qb * 128 + 127) / 64, (p.seq - 1) / 64) + 1;

  for (int kb = 0; kb < nkb; ++kb) {
    const int k0 = kb * 64;
    __syncthreads();
    load_row_tile(sK, rq, base_row + k0, p.seq - k0, ld3, p.h + hd * HD, tid);
    load_tr_tile(sVt, rq, base_row + k0, p.seq - k0, ld3, 2 * p.h + hd * HD, tid);
    __syncthreads();
    if (k0 > q_wave_max) continue;
    f32x16 s[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s[b] = zero16();
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) s[b] = mfma(frag_row(sK, 32 * b + lc, kk, h), qf[kk], s[b]);
    }
    // scale, causal mask, running max
    float mb = -INFINITY;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kv = k0 + 32 * b + 8 * (r >> 2) + 4 * h + (r & 3);
        const float v = (kv <= q && kv < p.seq) ? s[b][r] * c : -INFINITY;
        s[b][r] = v;
        mb = fmaxf(mb, v);
      }
    mb = fmaxf(mb, __shfl_xor(mb, 32));
    const float mn = fmaxf(m, mb);
    const float alpha = exp2f(m - mn);
    m = mn;
    l *= alpha;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = exp2f(s[b][r] - mn);
        s[b][r] = e;
        l += e;
      }
    // O^T[d][q] += sum_kv V[kv][d] P[q][kv]
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = s[b][8 * st + e];
        const bf16x8 pf = to_frag(pv);
#pragma unroll
        for (int d = 0; d < 4; ++d) o[d] = mfma(frag_tr(sVt, 32 * d + lc, 2 * b + st, h), pf, o[d]);
      }
  }
  l += __shfl_xor(l, 32);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dd = 32 * d + 8 * g + 4 * h;
      const uint32_t off = qv ? (uint32_t)(((base_row + q) * p.h + hd * HD + dd) * 2) : kOOB;
      const u32x2 v = {pack2(o[d][4 * g] * inv, o[d][4 * g + 1] * inv), pack2(o[d][4 * g + 2] * inv, o[d][4 * g + 3] * inv)};
      bstore8(ro, off, v);
    }
  if (qv && h == 0) p.lse2[(int64_t)hd * p.T + base_row + q] = m + log2f(l);
}

// ================================================================ dQ (+ D)
__global__ void __launch_bounds__(NT) attn_bwd_dq(AttnParams p) {
  __shared__ __attribute__((aligned(16))) char lds[64 * 256 * 2 + 128 * 128];
  char* sK = lds;                  // [64][128]
  char* sV = lds + 64 * 256;       // [64][128]
  char* sKt = lds + 2 * 64 * 256;  // [128][64]
  const int nqb = (p.seq + 127) / 128;
  const int qb = nqb - 1 - (int)blockIdx.x;
  const int hd = blockIdx.y % p.heads, sq = blockIdx.y / p.heads;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, lc = lane & 31;
  const int64_t ld3 = 3LL * p.h, base_row = (int64_t)sq * p.seq;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.qkv, (uint32_t)((int64_t)p.T * ld3 * 2));
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.o, (uint32_t)((int64_t)p.T * p.h * 2));
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(p.dout, (uint32_t)((int64_t)p.T * p.h * 2));
  const __amdgpu_buffer_rsrc_t rdq = make_rsrc(p.dqkv, (uint32_t)((int64_t)p.T * ld3 * 2));
  const float c = p.scale * kLog2e;

  const int q = qb * 128 + 32 * w + lc;
  const bool qv = q < p.seq;
  bf16x8 qf[8], dof[8];
  float dsum = 0.0f;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const int dd = hd * HD + 16 * kk + 8 * h;
    const uint32_t offq = qv ? (uint32_t)(((base_row + q) * ld3 + dd) * 2) : kOOB;
    const uint32_t offo = qv ? (uint32_t)(((base_row + q) * p.h + dd) * 2) : kOOB;
    qf[kk] = __builtin_bit_cast(bf16x8, bload16(rq, offq));
    const u32x4 gv = bload16(rdo, offo);
    const u32x4 ov = bload16(ro, offo);
    dof[kk] = __builtin_bit_cast(bf16x8, gv);
#pragma unroll
    for (int t = 0; t < 4; ++t) dsum += bf_lo(gv[t]) * bf_lo(ov[t]) + bf_hi(gv[t]) * bf_hi(ov[t]);
  }
  dsum += __shfl_xor(dsum, 32);
  const float lse = qv ? p.lse2[(int64_t)hd * p.T + base_row + q] : 0.0f;
  if (qv && h == 0) p.dsum[(int64_t)hd * p.T + base_row + q] = dsum;

  f32x16 dq[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) dq[d] = zero16();
  const int q_wave_max = qb * 128 + 32 * w + 31;
  const int nkb = min((qb * 128 + 127) / 64, (p.seq - 1) / 64) + 1;
  for (int kb = 0; kb < nkb; ++kb) {
    const int k0 = kb * 64;
    __syncthreads();
    load_row_tile(sK, rq, base_row + k0, p.seq - k0, ld3, p.h + hd * HD, tid);
    load_row_tile(sV, rq, base_row + k0, p.seq - k0, ld3, 2 * p.h + hd * HD, tid);
    load_tr_tile(sKt, rq, base_row + k0, p.seq - k0, ld3, p.h + hd * HD, tid);
    __syncthreads();
    if (k0 > q_wave_max) continue;
    f32x16 s[2], dp[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s[b] = zero16();
      dp[b] = zero16();
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        s[b] = mfma(frag_row(sK, 32 * b + lc, kk, h), qf[kk], s[b]);
        dp[b] = mfma(frag_row(sV, 32 * b + lc, kk, h), dof[kk], dp[b]);
      }
    }
    // dS^T = P^T * (dP^T - D)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kv = k0 + 32 * b + 8 * (r >> 2) + 4 * h + (r & 3);
        const float pr = (kv <= q && kv < p.seq) ? exp2f(s[b][r] * c - lse) : 0.0f;
        s[b][r] = pr * (dp[b][r] - dsum);
      }
    // dQ^T[d][q] += sum_kv K[kv][d] dS[q][kv]
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = s[b][8 * st + e];
        const bf16x8 f = to_frag(v);
#pragma unroll
        for (int d = 0; d < 4; ++d) dq[d] = mfma(frag_tr(sKt, 32 * d + lc, 2 * b + st, h), f, dq[d]);
      }
  }
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dd = 32 * d + 8 * g + 4 * h;
      const uint32_t off = qv ? (uint32_t)(((base_row + q) * ld3 + hd * HD + dd) * 2) : kOOB;
      const float sc = p.scale;
      const u32x2 v = {pack2(dq[d][4 * g] * sc, dq[d][4 * g + 1] * sc), pack2(dq[d][4 * g + 2] * sc, dq[d][4 * g + 3] * sc)};
      bstore8(rdq, off, v);
    }
}

// =============================================================== dK, dV
// Workgroup: 128 key rows (32 per wave) of one (sequence, head); queries in blocks of 64.
__global__ void __launch_bounds__(NT) attn_bwd_dkdv(AttnParams p) {
  __shared__ __attribute__((aligned(16))) char lds[2 * 64 * 256 + 2 * 128 * 128 + 2 * 64 * 4];
  char* sQ = lds;                          // [64][128]
  char* sG = lds + 64 * 256;               // dO [64][128]
  char* sQt = lds + 2 * 64 * 256;          // [128][64]
  char* sGt = sQt + 128 * 128;             // dO^T [128][64]
  float* sL = reinterpret_cast<float*>(sGt + 128 * 128);  // LSE2 [64]
  float* sD = sL + 64;                                    // D [64]
  const int nkb = (p.seq + 127) / 128;
  const int kb = (int)blockIdx.x;  // lightest first is fine: heavy blocks are the early keys
  const int hd = blockIdx.y % p.heads, sq = blockIdx.y / p.heads;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, lc = lane & 31;
  const int64_t ld3 = 3LL * p.h, base_row = (int64_t)sq * p.seq;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.qkv, (uint32_t)((int64_t)p.T * ld3 * 2));
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(p.dout, (uint32_t)((int64_t)p.T * p.h * 2));
  const __amdgpu_buffer_rsrc_t rdq = make_rsrc(p.dqkv, (uint32_t)((int64_t)p.T * ld3 * 2));
  const float c = p.scale * kLog2e;
  (void)nkb;

  const int kv = kb * 128 + 32 * w + lc;  // this lane's key row
  const bool kvv = kv < p.seq;
  bf16x8 kf[8], vf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const int dd = hd * HD + 16 * kk + 8 * h;
    const uint32_t offk = kvv ? (uint32_t)(((base_row + kv) * ld3 + p.h + dd) * 2) : kOOB;
    const uint32_t offv = kvv ? (uint32_t)(((base_row + kv) * ld3 + 2 * p.h + dd) * 2) : kOOB;
    kf[kk] = __builtin_bit_cast(bf16x8, bload16(rq, offk));
    vf[kk] = __builtin_bit_cast(bf16x8, bload16(rq, offv));
  }
  f32x16 dk[4], dv[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    dk[d] = zero16();
    dv[d] = zero16();
  }
  const int kv_wave_min = kb * 128 + 32 * w;
  for (int q0 = kb * 128; q0 < p.seq; q0 += 64) {
    __syncthreads();
    load_row_tile(sQ, rq, base_row + q0, p.seq - q0, ld3, hd * HD, tid);
    load_row_tile(sG, rdo, base_row + q0, p.seq - q0, p.h, hd * HD, tid);
    load_tr_tile(sQt, rq, base_row + q0, p.seq - q0, ld3, hd * HD, tid);
    load_tr_tile(sGt, rdo, base_row + q0, p.seq - q0, p.h, hd * HD, tid);
    if (tid < 64) {
      const bool ok = q0 + tid < p.seq;
      sL[tid] = ok ? p.lse2[(int64_t)hd * p.T + base_row + q0 + tid] : 0.0f;
      sD[tid] = ok ? p.dsum[(int64_t)hd * p.T + base_row + q0 + tid] : 0.0f;
    }
    __syncthreads();
    if (q0 + 63 < kv_wave_min) continue;  // every query of the block precedes this wave's keys
    for (int b = 0; b < 2; ++b) {  // two 32-query halves, one at a time
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        s = mfma(frag_row(sQ, 32 * b + lc, kk, h), kf[kk], s);   // S[q][kv]
        dp = mfma(frag_row(sG, 32 * b + lc, kk, h), vf[kk], dp); // dP[q][kv]
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ql = 32 * b + 8 * g + 4 * h;  // local query row of register 4g
        const f32x4 lv = *reinterpret_cast<const f32x4*>(sL + ql);
        const f32x4 dv4 = *reinterpret_cast<const f32x4*>(sD + ql);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int qq = q0 + ql + t;
          const int r = 4 * g + t;
          const float pr = (kv <= qq && qq < p.seq) ? exp2f(s[r] * c - lv[t]) : 0.0f;
          s[r] = pr;                       // P
          dp[r] = pr * (dp[r] - dv4[t]);   // dS
        }
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float pv[8], sv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = s[8 * st + e];
          sv[e] = dp[8 * st + e];
        }
        const bf16x8 pf = to_frag(pv), sf = to_frag(sv);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          dv[d] = mfma(frag_tr(sGt, 32 * d + lc, 2 * b + st, h), pf, dv[d]);  // dV^T[d][kv]
          dk[d] = mfma(frag_tr(sQt, 32 * d + lc, 2 * b + st, h), sf, dk[d]);  // dK^T[d][kv]
        }
      }
    }
  }
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dd = hd * HD + 32 * d + 8 * g + 4 * h;
      const int64_t row = base_row + kv;
      const uint32_t offk = kvv ? (uint32_t)((row * ld3 + p.h + dd) * 2) : kOOB;
      const uint32_t offv = kvv ? (uint32_t)((row * ld3 + 2 * p.h + dd) * 2) : kOOB;
      const float sc = p.scale;
      const u32x2 kv2 = {pack2(dk[d][4 * g] * sc, dk[d][4 * g + 1] * sc), pack2(dk[d][4 * g + 2] * sc, dk[d][4 * g + 3] * sc)};
      const u32x2 vv2 = {pack2(dv[d][4 * g], dv[d][4 * g + 1]), pack2(dv[d][4 * g + 2], dv[d][4 * g + 3])};
      bstore8(rdq, offk, kv2);
      bstore8(rdq, offv, vv2);
    }
}

}  // namespace

zb_status launch_attention_fwd(const AttnArgs& a, hipStream_t s) {
  AttnParams p{};
  p.qkv = static_cast<const uint16_t*>(a.qkv);
  p.o = static_cast<uint16_t*>(a.o);
  p.lse2 = a.lse2;
  p.T = a.seq * a.nseq; p.h = a.heads * HD; p.heads = a.heads; p.seq = a.seq; p.nseq = a.nseq;
  p.scale = 0.08838834764831845f;
  if (3.0 * p.T * p.h * 2 >= 2147483648.0) return set_error(ZB_E_UNSUPPORTED, "attention: QKV spans 2 GiB or more");
  const dim3 grid((a.seq + 127) / 128, a.heads * a.nseq);
  const double flops = 2.0 * a.nseq * (double)a.seq * a.seq * p.h;  // causal half of 4 s^2 h
  ProfScope ps("attn_fwd", flops, 2.0 * p.T * 4.0 * p.h, s);
  hipLaunchKernelGGL(attn_fwd, grid, dim3(NT), 0, s, p);
  ZB_HIP_CHECK(hipGetLastError());
  return ZB_OK;
}

zb_status launch_attention_bwd(const AttnArgs& a, hipStream_t s) {
  AttnParams p{};
  p.qkv = static_cast<const uint16_t*>(a.qkv);
  p.o = static_cast<uint16_t*>(a.o);
  p.lse2 = a.lse2;
  p.dout = static_cast<const uint16_t*>(a.dout);
  p.dsum = a.dsum;
  p.dqkv = static_cast<uint16_t*>(a.dqkv);
  p.T = a.seq * a.nseq; p.h = a.heads * HD; p.heads = a.heads; p.seq = a.seq; p.nseq = a.nseq;
  p.scale = 0.08838834764831845f;
  if (3.0 * p.T * p.h * 2 >= 2147483648.0) return set_error(ZB_E_UNSUPPORTED, "attention: QKV spans 2 GiB or more");
  const dim3 grid((a.seq + 127) / 128, a.heads * a.nseq);
  // Algorithmic backward = causal half of 8 s^2 h = four s x s x d products; the
  // two passes execute seven (three in dQ, four in dK/dV) and share them out 3:4.
  const double alg = 4.0 * a.nseq * (double)a.seq * a.seq * p.h;
  {
    ProfScope ps("attn_bwd_dq", alg * 3.0 / 7.0, 2.0 * p.T * 6.0 * p.h, s);
    hipLaunchKernelGGL(attn_bwd_dq, grid, dim3(NT), 0, s, p);
    ZB_HIP_CHECK(hipGetLastError());
  }
  {
    ProfScope ps("attn_bwd_dkdv", alg * 4.0 / 7.0, 2.0 * p.T * 6.0 * p.h, s);
    hipLaunchKernelGGL(attn_bwd_dkdv, grid, dim3(NT), 0, s, p);
    ZB_HIP_CHECK(hipGetLastError());
  }
  return ZB_OK;
}

}  // namespace zb
