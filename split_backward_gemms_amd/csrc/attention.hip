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
// Blocks of 64 sequence rows x 128 head dims go from global memory straight
// into LDS (buffer loads with the LDS bit) through a two-stage ring, one
// barrier per block.  In LDS a block is row-major, 256 bytes per row, with
// the 16-byte chunk c of row r at position c ^ f(r), f(r) = 4 (r % 4) +
// (r / 4) % 4: 16-byte reads of 16 consecutive rows (operands contracted over
// the head dimension) and transposing 8-byte reads of 4 rows x 4 chunks
// (ds_read_b64_tr_b16, operands contracted over positions) are both free of
// bank conflicts, so no block is ever transposed in registers.
//
// Determinism: dQ and dK/dV are separate passes (query-block and key-block
// parallel); no atomics, fixed summation order.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "zb_internal.h"

namespace zb {
namespace {

using dev::dma16;
using dev::kOOB;
using dev::lds_addr;
using dev::make_rsrc4;
using dev::pack_bf16x2;
using dev::wait_vm_barrier;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int HD = 128;           // head dim
constexpr int NT = 256;           // 4 waves
constexpr int BLK = 64 * 256;     // one 64 x 128 bf16 block in LDS
constexpr float kLog2e = 1.4426950408889634f;
// Forward: exponentials may reach 2^8 before the running maximum is moved
// (the fp32 sums and the bf16 operands of P V keep their relative precision).
constexpr float kRescaleSlack = 8.0f;

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
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)extent, (int)dev::kRsrcWord3);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ void bstore8(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, 0);
}
// 4 bytes per lane from rsrc at byte offset off (zero when out of range) into
// LDS at lds + 4 * lane, lds wave-uniform: each lane's range check covers
// exactly its own value.  Untracked by the compiler, like dev::dma16.
__device__ __forceinline__ void dma4(const dev::u32x4& rsrc, uint32_t lds, uint32_t off) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(off), "s"(rsrc), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 8 fp32 -> bf16x8 fragment
__device__ __forceinline__ bf16x8 to_frag(const float* v) {
  u32x4 u = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
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

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt vmcnt(0) as an instruction the compiler tracks (gfx9 encoding:
// expcnt 7 and lgkmcnt 15 mean no wait on those).  The block copies and the
// ring's waits are inline assembly, which the compiler's wait insertion does
// not see; without this, operands loaded into registers before a block loop
// stay pending in its model, and it waits for them again inside the loop, where
// the hardware counter also holds the next block's copies, so every block would
// wait out its own prefetch.
__device__ __forceinline__ void wait_vm_known() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---- LDS blocks ------------------------------------------------------------
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// A buffer descriptor the copies can take from scalar registers: the value is
// the same in every lane, but after inlining into divergent-looking control
// flow the compiler may hold it in vector registers.
__device__ __forceinline__ dev::u32x4 uniform4(const dev::u32x4& v) {
  return {(uint32_t)__builtin_amdgcn_readfirstlane((int)v[0]), (uint32_t)__builtin_amdgcn_readfirstlane((int)v[1]),
          (uint32_t)__builtin_amdgcn_readfirstlane((int)v[2]), (uint32_t)__builtin_amdgcn_readfirstlane((int)v[3])};
}

// Copies of one block: rows row0 .. row0+63 (those at or past `valid` read as
// zero), columns col0 .. col0+127 of a row-major bf16 matrix with leading
// dimension ld.  The NW waves of the workgroup each issue 16 / NW copies;
// copy q of wave w covers LDS bytes 1024 (w 16 / NW + q) .. +1023, i.e. four
// rows, with lane l at LDS chunk l of them.
template <int NW>
struct BlockDma {
  static constexpr int NI = 16 / NW;  // copies per wave per block (16 KiB / NW waves / 1 KiB)
  dev::u32x4 rsrc;
  uint32_t boff[NI];  // lane's byte offset at row0 = 0
  uint32_t rowstep;   // bytes per row
  int row0;           // the lane's row within the block for copy 0 (copy q adds 4 q)
  uint32_t lds0;      // this wave's first KiB within the block

  __device__ __forceinline__ BlockDma(const uint16_t* base, uint32_t extent, int64_t ld, int col0, int wave,
                                      int lane) {
    rsrc = make_rsrc4(base, extent);
    rowstep = (uint32_t)(ld * 2);
    lds0 = (uint32_t)(wave * NI * 1024);
    row0 = wave * NI * 4 + (lane >> 4);
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int r = row0 + 4 * q;
      const int c = (lane & 15) ^ swz(r);
      boff[q] = (uint32_t)(((int64_t)r * ld + col0 + 8 * c) * 2);
    }
  }
  __device__ __forceinline__ void load(uint32_t dst, int64_t first_row, int valid) const {
    const uint32_t step = (uint32_t)(first_row * rowstep);
    const dev::u32x4 r = uniform4(rsrc);
#pragma unroll
    for (int q = 0; q < NI; ++q)
      dma16(r, dst + lds0 + q * 1024, row0 + 4 * q < valid ? boff[q] + step : kOOB);
  }
};

// Operand contracted over the head dim (16-byte reads): rows 32 b + lc of a
// block, k = 16 kk + 8 h .. +7.  rb[kk] = lane's offset for kk (rows 32 b
// differ by 8192 bytes and keep the swizzle).
struct RowFrag {
  uint32_t rb[8];
  __device__ __forceinline__ RowFrag(int lane) {
    const int lc = lane & 31, h = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) rb[kk] = lc * 256 + (((2 * kk + h) ^ swz(lc)) << 4);
  }
  __device__ __forceinline__ bf16x8 get(const char* blk, int b, int kk) const {
    return *reinterpret_cast<const bf16x8*>(blk + rb[kk] + b * 32 * 256);
  }
};

// Operand contracted over positions (transposing reads): X[p = head dim
// 32 db + lc][k = positions 16 ks + {4h..4h+3, 8+4h..8+4h+3}] from a block
// holding rows = positions.  Lane l = 16 g + i reads rows 16 ks + 4 (g / 2) +
// i / 4 (+ 8) at columns 32 db + 16 (g % 2) + 4 (i % 4).  tb[half][db] is the
// lane's offset for ks = 0.
struct TrFrag {
  uint32_t tb[2][4];
  __device__ __forceinline__ TrFrag(int lane) {
    const int g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int r = 4 * (g >> 1) + (i >> 2) + 8 * half;
        const int c = 4 * db + 2 * (g & 1) + ((i & 3) >> 1);
        tb[half][db] = r * 256 + ((c ^ swz(r)) << 4) + 8 * (i & 1);
      }
  }
  __device__ __forceinline__ bf16x8 get(const char* blk, int db, int ks) const {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(blk + tb[0][db] + ks * 16 * 256));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(blk + tb[1][db] + ks * 16 * 256));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

// ============================================================== forward
// Workgroup: 128 query rows (32 per wave) of one (sequence, head); keys in
// blocks of 64 through a two-stage ring of (K, V) blocks.
__global__ void __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(2, 2))) attn_fwd(AttnParams p) {
  __shared__ __attribute__((aligned(1024))) char sK0[BLK];
  __shared__ __attribute__((aligned(1024))) char sV0[BLK];
  __shared__ __attribute__((aligned(1024))) char sK1[BLK];
  __shared__ __attribute__((aligned(1024))) char sV1[BLK];
  // Grid (heads x sequences, query blocks).  Workgroups are handed out with x
  // varying fastest, so every head's heaviest block (the last one, which sees
  // all keys) goes out first and the light ones fill in behind them.
  const int nqb = (p.seq + 127) / 128;
  const int qb = nqb - 1 - (int)blockIdx.y;
  const int hd = blockIdx.x % p.heads, sq = blockIdx.x / p.heads;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, lc = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t ld3 = 3LL * p.h, base_row = (int64_t)sq * p.seq;
  const uint32_t ext3 = (uint32_t)((int64_t)p.T * ld3 * 2);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.qkv, ext3);
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
  const BlockDma<4> dk(p.qkv, ext3, ld3, p.h + hd * HD, w, lane);
  const BlockDma<4> dv(p.qkv, ext3, ld3, 2 * p.h + hd * HD, w, lane);
  const RowFrag rf(lane);
  const TrFrag tf(lane);

  f32x16 o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) o[d] = zero16();
  float m = -INFINITY, l = 0.0f;
  const int q_wave_min = qb * 128 + 32 * w, q_wave_max = q_wave_min + 31;
  const int nkb = min(qb * 128 + 127, p.seq - 1) / 64 + 1;

  auto fetch = [&](char* sk, char* sv, int kb) {
    const int k0 = kb * 64;
    dk.load(__builtin_amdgcn_readfirstlane(lds_addr(sk)), base_row + k0, p.seq - k0);
    dv.load(__builtin_amdgcn_readfirstlane(lds_addr(sv)), base_row + k0, p.seq - k0);
  };
  fetch(sK0, sV0, 0);
  wait_vm_known();  // the register loads above, and block 0, which is needed first anyway
  if (nkb > 1) fetch(sK1, sV1, 1);
  if (nkb > 1) wait_vm_barrier<2 * BlockDma<4>::NI>();
  else wait_vm_barrier<0>();

  // Block kb from (sk, sv); at the end every wave has its copies of block
  // kb+1 and is done with block kb, whose stage then takes block kb+2.
  auto body = [&](char* sk, char* sv, int kb) {
    const int k0 = kb * 64;
    if (k0 <= q_wave_max) {
      f32x16 s[2] = {zero16(), zero16()};
      // Two independent chains, interleaved; each step's K fragments are
      // requested one step ahead of their MFMAs.
      bf16x8 kf[2][2];
      kf[0][0] = rf.get(sk, 0, 0);
      kf[0][1] = rf.get(sk, 1, 0);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        if (kk + 1 < 8) {
          kf[(kk + 1) & 1][0] = rf.get(sk, 0, kk + 1);
          kf[(kk + 1) & 1][1] = rf.get(sk, 1, kk + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < 2; ++b) s[b] = mfma(kf[kk & 1][b], qf[kk], s[b]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (k0 + 63 > q_wave_min || k0 + 64 > p.seq) {  // diagonal or last block: mask
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kv = k0 + 32 * b + 8 * (r >> 2) + 4 * h + (r & 3);
            if (kv > q || kv >= p.seq) s[b][r] = -INFINITY;
          }
      }
      float mb = -INFINITY;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) mb = fmaxf(mb, s[b][r]);
      mb = fmaxf(mb, __shfl_xor(mb, 32));
      // The running maximum m (base 2) moves only when a row's block maximum
      // exceeds it by more than kRescaleSlack; until then the exponentials of
      // later blocks stay below 2^kRescaleSlack and the sums need no rescale.
      // Block 0 always has key 0 <= q, so the first maximum is finite.
      const float mc = mb * c;
      const bool grow = mc > m + kRescaleSlack;  // always true on the first block (m = -inf)
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float mn = grow ? mc : m;
        const float alpha = exp2_hw(m - mn);
        m = mn;
        l *= alpha;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
      }
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = exp2_hw(fmaf(s[b][r], c, -m));
          s[b][r] = e;
          l += e;
        }
      // O^T[d][q] += sum_kv V^T[d][kv] P^T[kv][q]
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = s[ks >> 1][8 * (ks & 1) + e];
        const bf16x8 pf = to_frag(pv);
#pragma unroll
        for (int d = 0; d < 4; ++d) o[d] = mfma(tf.get(sv, d, ks), pf, o[d]);
      }
    }
    wait_vm_barrier<0>();
    if (kb + 2 < nkb) fetch(sk, sv, kb + 2);
  };
  int kb = 0;
  for (; kb + 1 < nkb; kb += 2) {
    body(sK0, sV0, kb);
    body(sK1, sV1, kb + 1);
  }
  if (kb < nkb) body(sK0, sV0, kb);

  l += __shfl_xor(l, 32);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dd = 32 * d + 8 * g + 4 * h;
      const uint32_t off = qv ? (uint32_t)(((base_row + q) * p.h + hd * HD + dd) * 2) : kOOB;
      const u32x2 v = {pack_bf16x2(o[d][4 * g] * inv, o[d][4 * g + 1] * inv),
                       pack_bf16x2(o[d][4 * g + 2] * inv, o[d][4 * g + 3] * inv)};
      bstore8(ro, off, v);
    }
  if (qv && h == 0) p.lse2[(int64_t)hd * p.T + base_row + q] = m + log2f(l);
}

// ================================================================ dQ (+ D)
// Workgroup: 128 query rows of one (sequence, head); (K, V) blocks of 64 keys.
__global__ void __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(2, 2))) attn_bwd_dq(AttnParams p) {
  __shared__ __attribute__((aligned(1024))) char sK0[BLK];
  __shared__ __attribute__((aligned(1024))) char sV0[BLK];
  __shared__ __attribute__((aligned(1024))) char sK1[BLK];
  __shared__ __attribute__((aligned(1024))) char sV1[BLK];
  const int nqb = (p.seq + 127) / 128;
  const int qb = nqb - 1 - (int)blockIdx.y;  // grid and order as in the forward
  const int hd = blockIdx.x % p.heads, sq = blockIdx.x / p.heads;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, lc = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t ld3 = 3LL * p.h, base_row = (int64_t)sq * p.seq;
  const uint32_t ext3 = (uint32_t)((int64_t)p.T * ld3 * 2);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.qkv, ext3);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.o, (uint32_t)((int64_t)p.T * p.h * 2));
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(p.dout, (uint32_t)((int64_t)p.T * p.h * 2));
  const __amdgpu_buffer_rsrc_t rdq = make_rsrc(p.dqkv, ext3);
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
  const BlockDma<4> dk(p.qkv, ext3, ld3, p.h + hd * HD, w, lane);
  const BlockDma<4> dv(p.qkv, ext3, ld3, 2 * p.h + hd * HD, w, lane);
  const RowFrag rf(lane);
  const TrFrag tf(lane);

  f32x16 dq[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) dq[d] = zero16();
  const int q_wave_min = qb * 128 + 32 * w, q_wave_max = q_wave_min + 31;
  const int nkb = min(qb * 128 + 127, p.seq - 1) / 64 + 1;

  auto fetch = [&](char* sk, char* sv, int kb) {
    const int k0 = kb * 64;
    dk.load(__builtin_amdgcn_readfirstlane(lds_addr(sk)), base_row + k0, p.seq - k0);
    dv.load(__builtin_amdgcn_readfirstlane(lds_addr(sv)), base_row + k0, p.seq - k0);
  };
  fetch(sK0, sV0, 0);
  wait_vm_known();  // the register loads above, and block 0, which is needed first anyway
  if (nkb > 1) fetch(sK1, sV1, 1);
  if (nkb > 1) wait_vm_barrier<2 * BlockDma<4>::NI>();
  else wait_vm_barrier<0>();

  auto body = [&](char* sk, char* sv, int kb) {
    const int k0 = kb * 64;
    if (k0 <= q_wave_max) {
      const bool masked = k0 + 63 > q_wave_min || k0 + 64 > p.seq;
#pragma unroll
      for (int b = 0; b < 2; ++b) {  // two 32-key halves, one at a time
        f32x16 s = zero16(), dp = zero16();
        // K and V fragments requested one step ahead of their MFMAs.
        bf16x8 kf[2], vf[2];
        kf[0] = rf.get(sk, b, 0);
        vf[0] = rf.get(sv, b, 0);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          if (kk + 1 < 8) {
            kf[(kk + 1) & 1] = rf.get(sk, b, kk + 1);
            vf[(kk + 1) & 1] = rf.get(sv, b, kk + 1);
          }
          __builtin_amdgcn_sched_barrier(0);
          s = mfma(kf[kk & 1], qf[kk], s);     // S^T[kv][q]
          dp = mfma(vf[kk & 1], dof[kk], dp);  // dP^T[kv][q]
          __builtin_amdgcn_sched_barrier(0);
        }
        if (masked) {  // diagonal or last block (uniform branch: most blocks skip the index math)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kv = k0 + 32 * b + 8 * (r >> 2) + 4 * h + (r & 3);
            float pr = exp2_hw(fmaf(s[r], c, -lse));
            if (kv > q || kv >= p.seq) pr = 0.0f;
            s[r] = pr * (dp[r] - dsum);  // dS^T
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) s[r] = exp2_hw(fmaf(s[r], c, -lse)) * (dp[r] - dsum);
        }
        // dQ^T[d][q] += sum_kv K^T[d][kv] dS^T[kv][q]; the second step's K^T
        // fragments are requested ahead of the first step's MFMAs.
        bf16x8 ktf[2][4];
#pragma unroll
        for (int d = 0; d < 4; ++d) ktf[0][d] = tf.get(sk, d, 2 * b);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          if (st == 0) {
#pragma unroll
            for (int d = 0; d < 4; ++d) ktf[1][d] = tf.get(sk, d, 2 * b + 1);
          }
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = s[8 * st + e];
          const bf16x8 f = to_frag(v);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int d = 0; d < 4; ++d) dq[d] = mfma(ktf[st][d], f, dq[d]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    wait_vm_barrier<0>();
    if (kb + 2 < nkb) fetch(sk, sv, kb + 2);
  };
  int kb = 0;
  for (; kb + 1 < nkb; kb += 2) {
    body(sK0, sV0, kb);
    body(sK1, sV1, kb + 1);
  }
  if (kb < nkb) body(sK0, sV0, kb);

#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dd = 32 * d + 8 * g + 4 * h;
      const uint32_t off = qv ? (uint32_t)(((base_row + q) * ld3 + hd * HD + dd) * 2) : kOOB;
      const float sc = p.scale;
      const u32x2 v = {pack_bf16x2(dq[d][4 * g] * sc, dq[d][4 * g + 1] * sc),
                       pack_bf16x2(dq[d][4 * g + 2] * sc, dq[d][4 * g + 3] * sc)};
      bstore8(rdq, off, v);
    }
}

// =============================================================== dK, dV
// Workgroup: 128 key rows of one (sequence, head), four 32-key blocks;
// (Q, dO) blocks of 64 queries, from the first query that can see the keys to
// the end.  LSE2 and D of a block ride along: two more copies of 4 bytes per
// lane, one row each (rows past the sequence read as zero).
// Grid (heads x sequences, key blocks), heaviest first: key block 0 sees every
// query block, and workgroups are handed out with x varying fastest.
//
// Each key block is worked by a pair of waves on one SIMD, one query block
// apart.  In step j wave k (k < 4) takes query block j: S = Q K^T, P, and
// dV += P^T dO; it leaves P's four bf16 operand fragments in LDS.  Wave k + 4
// takes query block j - 1: dP = dO V^T, dS = P (dP - D) with P read back from
// those fragments, and dK += dS^T Q.  The two waves' instruction streams are
// independent within a step, so one's exponentials and element-wise work run
// under the other's MFMAs, and one barrier per step (which also retires the
// ring's oldest block) is all the pair needs.  (Q, dO, LSE2/D) blocks go
// through a three-block ring: j - 1 and j in use, j + 1 in flight.
constexpr int NTP = 512;                  // 8 waves
__global__ void __attribute__((amdgpu_flat_work_group_size(NTP, NTP), amdgpu_waves_per_eu(2, 2))) attn_bwd_dkdv_skew(AttnParams p) {
  // Three-block rings of Q, dO and (LSE2, D); the step loop is unrolled six
  // ways so that every ring slot and P buffer is a compile-time offset.
  __shared__ __attribute__((aligned(1024))) char sQr[3 * BLK];
  __shared__ __attribute__((aligned(1024))) char sGr[3 * BLK];
  __shared__ __attribute__((aligned(1024))) char sLDr[3 * 1024];
  __shared__ __attribute__((aligned(1024))) char sPf[2 * 4 * 4 * 1024];  // [step parity][key block][fragment][lane] 16 B
  const int kb = (int)blockIdx.y;
  const int hd = blockIdx.x % p.heads, sq = blockIdx.x / p.heads;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, lc = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kbw = w & 3;          // key block of the wave
  const bool role_p = w < 4;      // S, P, dV (else dP, dS, dK)
  const int64_t ld3 = 3LL * p.h, base_row = (int64_t)sq * p.seq;
  const uint32_t ext3 = (uint32_t)((int64_t)p.T * ld3 * 2);
  const uint32_t exth = (uint32_t)((int64_t)p.T * p.h * 2);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.qkv, ext3);
  const __amdgpu_buffer_rsrc_t rdq = make_rsrc(p.dqkv, ext3);
  const float c = p.scale * kLog2e;
  const int kv = kb * 128 + 32 * kbw + lc;  // this lane's key row
  const bool kvv = kv < p.seq;
  bf16x8 xf[8];  // K rows (role P) or V rows (role dS)
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const int dd = hd * HD + 16 * kk + 8 * h;
    const uint32_t off = kvv ? (uint32_t)(((base_row + kv) * ld3 + (role_p ? p.h : 2 * p.h) + dd) * 2) : kOOB;
    xf[kk] = __builtin_bit_cast(bf16x8, bload16(rq, off));
  }
  const BlockDma<8> dmq(p.qkv, ext3, ld3, hd * HD, w, lane);
  const BlockDma<8> dmg(p.dout, exth, p.h, hd * HD, w, lane);
  const dev::u32x4 rl = make_rsrc4(p.lse2 + (int64_t)hd * p.T + base_row, (uint32_t)(p.seq * 4));
  const dev::u32x4 rd = make_rsrc4(p.dsum + (int64_t)hd * p.T + base_row, (uint32_t)(p.seq * 4));
  const RowFrag rf(lane);
  const TrFrag tf(lane);

  f32x16 acc[4];  // dV^T (role P) or dK^T (role dS) of the wave's keys
#pragma unroll
  for (int d = 0; d < 4; ++d) acc[d] = zero16();
  const int kv_wave_min = kb * 128 + 32 * kbw, kv_wave_max = kv_wave_min + 31;
  const int qb0 = kb * 2;
  const int nqb = (p.seq + 63) / 64 - qb0;

  auto pfrag = [&](auto pb, int f) -> char* {
    return sPf + (((decltype(pb)::value) * 4 + kbw) * 4 + f) * 1024 + lane * 16;
  };
  auto fetch = [&](auto sl, int j) {
    constexpr int S = decltype(sl)::value;
    const int q0 = (qb0 + j) * 64;
    dmq.load(__builtin_amdgcn_readfirstlane(lds_addr(sQr + S * BLK)), base_row + q0, p.seq - q0);
    dmg.load(__builtin_amdgcn_readfirstlane(lds_addr(sGr + S * BLK)), base_row + q0, p.seq - q0);
    if (w == 0) {  // one value per lane and row: a sequence of any length ends exactly
      const uint32_t off = q0 + lane < p.seq ? (uint32_t)((q0 + lane) * 4) : kOOB;
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(sLDr + S * 1024));
      dma4(uniform4(rl), dst, off);
      dma4(uniform4(rd), dst + 256, off);
    }
  };
  // some query of block j sees some key of the wave's block
  auto active = [&](int j) { return (qb0 + j) * 64 + 63 >= kv_wave_min; };

  // Role P, query block j: S, P (masked), P's fragments to LDS, dV.
  auto p_step = [&](auto sl, auto pb, int j) {
    constexpr int S = decltype(sl)::value;
    const char* s = sQr + S * BLK;
    const char* sg = sGr + S * BLK;
    const int q0 = (qb0 + j) * 64;
    const float* sL = reinterpret_cast<const float*>(sLDr + S * 1024);
    f32x16 x[2] = {zero16(), zero16()};
    // The two halves are independent chains, interleaved; each step's Q
    // fragments are requested one step ahead of their MFMAs.
    bf16x8 qfr[2][2];
    qfr[0][0] = rf.get(s, 0, 0);
    qfr[0][1] = rf.get(s, 1, 0);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      if (kk + 1 < 8) {
        qfr[(kk + 1) & 1][0] = rf.get(s, 0, kk + 1);
        qfr[(kk + 1) & 1][1] = rf.get(s, 1, kk + 1);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < 2; ++b) x[b] = mfma(qfr[kk & 1][b], xf[kk], x[b]);  // S[q][kv]
      __builtin_amdgcn_sched_barrier(0);
    }
    const bool masked = q0 < kv_wave_max || q0 + 64 > p.seq;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ql = 32 * b + 8 * g + 4 * h;
        const f32x4 lv = *reinterpret_cast<const f32x4*>(sL + ql);
        if (masked) {  // uniform branch: only diagonal and last blocks pay for the index math
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int qq = q0 + ql + t;
            float pr = exp2_hw(fmaf(x[b][4 * g + t], c, -lv[t]));
            if (kv > qq || qq >= p.seq) pr = 0.0f;
            x[b][4 * g + t] = pr;
          }
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) x[b][4 * g + t] = exp2_hw(fmaf(x[b][4 * g + t], c, -lv[t]));
        }
      }
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = x[b][8 * st + e];
        const bf16x8 pf = to_frag(pv);
        *reinterpret_cast<bf16x8*>(pfrag(pb, 2 * b + st)) = pf;
#pragma unroll
        for (int d = 0; d < 4; ++d) acc[d] = mfma(tf.get(sg, d, 2 * b + st), pf, acc[d]);  // dV^T[d][kv]
      }
  };

  // Role dS, query block j: dP, dS from P's fragments, dK.
  auto ds_step = [&](auto sl, auto pb) {
    constexpr int S = decltype(sl)::value;
    const char* s = sQr + S * BLK;
    const char* sg = sGr + S * BLK;
    const float* sD = reinterpret_cast<const float*>(sLDr + S * 1024 + 256);
    f32x16 x[2] = {zero16(), zero16()};
    bf16x8 gfr[2][2];  // dO fragments, one step ahead as in the S chain
    gfr[0][0] = rf.get(sg, 0, 0);
    gfr[0][1] = rf.get(sg, 1, 0);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      if (kk + 1 < 8) {
        gfr[(kk + 1) & 1][0] = rf.get(sg, 0, kk + 1);
        gfr[(kk + 1) & 1][1] = rf.get(sg, 1, kk + 1);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < 2; ++b) x[b] = mfma(gfr[kk & 1][b], xf[kk], x[b]);  // dP[q][kv]
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const u32x4 pw = *reinterpret_cast<const u32x4*>(pfrag(pb, 2 * b + st));
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(sD + 32 * b + 16 * st + 4 * h);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(sD + 32 * b + 16 * st + 8 + 4 * h);
        float sv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pr = (e & 1) ? bf_hi(pw[e >> 1]) : bf_lo(pw[e >> 1]);
          const float dv = e < 4 ? d0[e] : d1[e - 4];
          sv[e] = pr * (x[b][8 * st + e] - dv);  // dS
        }
        const bf16x8 sf = to_frag(sv);
#pragma unroll
        for (int d = 0; d < 4; ++d) acc[d] = mfma(tf.get(s, d, 2 * b + st), sf, acc[d]);  // dK^T[d][kv]
      }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  fetch(I0{}, 0);
  if (nqb > 1) fetch(I1{}, 1);
  wait_vm_barrier<0>();
  wait_vm_known();  // nothing is in flight here; the compiler learns that the K / V rows have landed
  // Step j (j % 6 == R): role P takes block j (slot j % 3, P buffer j % 2), role
  // dS block j - 1; then block j+1 has landed, P of block j is visible and
  // block j-1's slot, (j + 2) % 3, takes block j + 2.
  auto step = [&](auto r, int j) {
    constexpr int R = decltype(r)::value;
    using SP = std::integral_constant<int, R % 3>;
    using PP = std::integral_constant<int, R % 2>;
    using SD = std::integral_constant<int, (R + 2) % 3>;
    using PD = std::integral_constant<int, (R + 1) % 2>;
    if (role_p) {
      if (j < nqb && active(j)) p_step(SP{}, PP{}, j);
    } else {
      if (j >= 1 && active(j - 1)) ds_step(SD{}, PD{});
    }
    wait_vm_barrier<0>();
    if (j + 2 < nqb) fetch(SD{}, j + 2);
  };
  // The roles run separate loops (wave-uniform branch) so that each keeps only
  // its own values live; both meet the same barriers, one per step.
  auto run = [&]() __attribute__((always_inline)) {
    for (int j = 0; j <= nqb; j += 6) {
      step(I0{}, j);
      if (j + 1 <= nqb) step(I1{}, j + 1);
      if (j + 2 <= nqb) step(I2{}, j + 2);
      if (j + 3 <= nqb) step(std::integral_constant<int, 3>{}, j + 3);
      if (j + 4 <= nqb) step(std::integral_constant<int, 4>{}, j + 4);
      if (j + 5 <= nqb) step(std::integral_constant<int, 5>{}, j + 5);
    }
  };
  if (role_p) run();
  else run();

  const float sc = role_p ? 1.0f : p.scale;
  const int col = role_p ? 2 * p.h : p.h;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dd = hd * HD + 32 * d + 8 * g + 4 * h;
      const uint32_t off = kvv ? (uint32_t)(((base_row + kv) * ld3 + col + dd) * 2) : kOOB;
      const u32x2 v2 = {pack_bf16x2(acc[d][4 * g] * sc, acc[d][4 * g + 1] * sc),
                        pack_bf16x2(acc[d][4 * g + 2] * sc, acc[d][4 * g + 3] * sc)};
      bstore8(rdq, off, v2);
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
  if (a.seq <= 0 || a.heads <= 0 || a.nseq <= 0) return ZB_OK;
  const dim3 grid(a.heads * a.nseq, (a.seq + 127) / 128);
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
  if (a.seq <= 0 || a.heads <= 0 || a.nseq <= 0) return ZB_OK;
  const dim3 grid(a.heads * a.nseq, (a.seq + 127) / 128);  // 128-row query (dQ) or key (dK/dV) blocks
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
    hipLaunchKernelGGL(attn_bwd_dkdv_skew, grid, dim3(NTP), 0, s, p);
    ZB_HIP_CHECK(hipGetLastError());
  }
  return ZB_OK;
}

}  // namespace zb
