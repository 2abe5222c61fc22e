// Dense contractions of a stage: the F, B and W GEMMs with fused epilogues.
//
//   F  Y[T,N]  = X[T,K] . W[K,N]            A k-contiguous, B n-contiguous
//   B  dX[T,K] = dY[T,N] . W[K,N]^T         A and B k-contiguous
//   W  dW[K,N] += X[T,K]^T . dY[T,N]        A m-contiguous, B n-contiguous (reduce over T)
//
// (B/W split of the backward pass: "Zero Bubble Pipeline Parallelism",
// section 3, "The Backward Pass Decomposition"; the three products as the
// tutorial "Pipeline Schedules: GPipe, 1F1B and Zero Bubble" writes them in
// "Zero bubble: split the backward pass".)
//
// bf16 path: 8 waves of 64 in a 2x4 grid, two per SIMD, for tiles of at least
// 128x128 (4 waves in a 2x2 grid for 128x64); each wave owns a (BM/2)x(BN/4)
// (or (BM/2)x(BN/2)) block of 32x32 MFMA tiles (v_mfma_f32_32x32x16_bf16,
// fp32 accumulators).  With two waves on a SIMD one wave's LDS reads, waits
// and barrier overlap the other's MFMAs: measured 5-20% faster than one wave
// per SIMD on every 256x256 F and B product of the seq-4096 workload and
// 3-9% on the 256x128 and 128x128 tiles of the seq-1024 one, bit-identical.  K advances 64 at a time (32 in the grouped W launch) through
// a ring of 2 to 4 LDS stages that global->LDS copies (buffer_load ... lds, 16
// bytes per lane, hardware range checks in place of bounds branches) keep
// filled ahead of the MFMAs; every wait for them is an explicit vmcnt wait
// plus a barrier.  k-contiguous operands sit in LDS as [rows][64] with 16-byte
// chunks XOR-ed by (row ^ row/8) & 7 and are read 16 bytes at a time;
// m/n-contiguous operands (F's weight, W's X and dY) stay untransposed as
// [k][rows] with chunks XOR-ed by 4 (k % 4) and are read with the transposing
// ds_read_b64_tr_b16.  Launches with more tiles than CUs run one persistent
// workgroup per CU looping over its tiles.
//
// Epilogues: bf16 store, residual add, GeLU (pre-activation stored beside),
// GeLU' of a saved pre-activation, with lanes l and l+32 swapping halves so
// every store is 16 bytes; W: dW = (first W of the step ? 0 : dW) + acc in
// fp32 after the k loop, so W of microbatches j, j+1, ... give the same bits in
// any slots as long as they run in the same order.  F and B may split K in
// two or four: the splits write fp32 partials and a second kernel adds them in
// split order (deterministic).  No atomics.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <type_traits>

#include "device_common.h"
#include "zb_internal.h"

namespace zb {
namespace {

using dev::dma16;
using dev::gelu_f;
using dev::gelu_grad_f;
using dev::kOOB;
using dev::kRsrcWord3;
using dev::lds_addr;
using dev::make_rsrc4;
using dev::pack_bf16x2;
using dev::wait_vm_barrier;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BKT = 64;   // K per LDS tile
constexpr int kWavesWide = 8;    // waves per workgroup for tiles of at least 128x128
constexpr int kWavesNarrow = 4;  // for 128x64
constexpr int XCDS = 8;   // MI355X: 8 accelerator complex dies, workgroups dealt round-robin

struct Params {
  int M, N, K;
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  void* C;
  int64_t ldc;
  const void* R;
  int64_t ldr;
  void* Z;
  int64_t ldz;
  int beta;
  int gelu;
  int nbm, nbn;
  int xcd_remap;
  // Split-K: `splits` workgroups share an output tile, each reducing over
  // `kts` 64-deep k tiles; with EPI_PART split s writes its fp32 sum to
  // C + s * M * ldc, and a second kernel adds the splits in order.
  int splits, kts;
};

// ------------------------------------------------------------- elementwise math

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return (uint16_t)pack_bf16x2(f, 0.0f); }

template <typename T>
__device__ __forceinline__ float ld_elem(const void* p, int64_t i);
template <>
__device__ __forceinline__ float ld_elem<uint16_t>(const void* p, int64_t i) {
  return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}
template <>
__device__ __forceinline__ float ld_elem<float>(const void* p, int64_t i) {
  return static_cast<const float*>(p)[i];
}
template <typename T>
__device__ __forceinline__ void st_elem(void* p, int64_t i, float v);
template <>
__device__ __forceinline__ void st_elem<uint16_t>(void* p, int64_t i, float v) {
  static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
}
template <>
__device__ __forceinline__ void st_elem<float>(void* p, int64_t i, float v) {
  static_cast<float*>(p)[i] = v;
}

// Output element (m, n) of the product with value v: the fused epilogue.
template <typename T, int EPI>
__device__ __forceinline__ void epi_store(const Params& p, int m, int n, float v) {
  if constexpr (EPI == EPI_ACC) {
    static_cast<float*>(p.C)[(int64_t)m * p.ldc + n] = v;
  } else {
    if constexpr (EPI == EPI_RESID) v += ld_elem<T>(p.R, (int64_t)m * p.ldr + n);
    if constexpr (EPI == EPI_GELU) {
      st_elem<T>(p.Z, (int64_t)m * p.ldz + n, v);
      v = gelu_f(v, p.gelu);
    }
    if constexpr (EPI == EPI_DGELU) v *= gelu_grad_f(ld_elem<T>(p.R, (int64_t)m * p.ldr + n), p.gelu);
    st_elem<T>(p.C, (int64_t)m * p.ldc + n, v);
  }
}

// Workgroups are dealt to the 8 XCDs round-robin; renumber them so that
// consecutive logical indices run on one XCD (its own L2).
__device__ __forceinline__ int xcd_remap(int b, int total) {
  return total % XCDS == 0 ? (b % XCDS) * (total / XCDS) + b / XCDS : b;
}

// Logical tile index -> output tile.  Tiles go in groups of 4 tile-rows, down
// each column of the group and then across, so neighbours reuse A rows and B
// columns; the 32 tiles an XCD works on at once then cover 4 tile-rows by 8
// tile-columns, whose output rows are written in longer contiguous runs than
// with 8 by 4 (measured 3-3.5% faster whole steps at T = 1024 and 2048; groups
// of 2 lose at T = 4096, of 1 everywhere).
__device__ __forceinline__ void tile_raster(const Params& p, int& tm, int& tn, int b) {
  const int G = 4;
  const int per_group = G * p.nbn;
  const int group = b / per_group;
  const int first_m = group * G;
  const int gsz = min(p.nbm - first_m, G);
  const int r = b - group * per_group;
  tm = first_m + r % gsz;
  tn = r / gsz;
}

__device__ __forceinline__ void tile_coords(const Params& p, int& tm, int& tn, int b) {
  if (p.xcd_remap) b = xcd_remap(b, p.nbm * p.nbn);
  tile_raster(p, tm, tn, b);
}

// ------------------------------------------------------------- bf16 MFMA GEMM

// Global memory is read and written through buffer resources: an access whose
// byte offset is at or past the operand's extent returns zero (loads) or is
// dropped (stores).  Lanes outside the matrix get an offset of kOOB, so edge
// tiles need no branches.

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t extent_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)extent_bytes, (int)kRsrcWord3);
}

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Global -> LDS copies (dev::dma16) are issued with inline assembly, so the
// compiler does not track them: every wait for them is explicit
// (dev::wait_vm_barrier), and its memory clobber keeps LDS reads from moving
// across it.

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// One operand tile (ROWS m/n rows by BK k) copied global -> LDS by the
// buffer unit, without passing through registers.  One instruction moves 64
// lanes x 16 bytes into 1 KiB of consecutive LDS (lane l at byte 16 l); the
// swizzle is applied by choosing which global chunk each lane fetches.
//   KCONTIG:   LDS [ROWS][64] bf16 (BK = 64 only); chunk c (8 k values) of row
//              r sits at position c ^ swz(r) of its 128-byte row.
//   otherwise: LDS [BK][ROWS] bf16; chunk c (8 m values) of k-row k sits at
//              position c ^ 4 (k % 4) of its 2 ROWS-byte row (c ^ 4 (k % 2) when
//              ROWS = 64).
// The WV waves of the workgroup each move an equal share of the tile.
template <int ROWS, bool KCONTIG, int BK, int WV>
struct DmaLoader {
  static_assert(BK == BKT || !KCONTIG, "k-contiguous operands use 64-deep tiles");
  static constexpr int NI = ROWS * BK / (512 * WV);  // instructions per wave per tile
  u32x4 rsrc;
  uint32_t voff[NI];                    // lane's byte offset at k0 = 0 (kOOB outside the matrix)
  int kofs[KCONTIG ? NI : 1];           // KCONTIG: lane's first k within the tile
  uint32_t kstep;                       // bytes per unit of k
  uint32_t lds0;                        // this wave's first KiB within the operand tile (uniform)

  __device__ __forceinline__ DmaLoader(const uint16_t* base, int64_t ld, int row0, int rows_lim, int K,
                                       int wave, int lane) {
    lds0 = (uint32_t)(wave * NI * 1024);
    if constexpr (KCONTIG) {
      rsrc = make_rsrc4(base, (uint32_t)(((int64_t)(rows_lim - 1) * ld + K) * 2));
      kstep = 2;
#pragma unroll
      for (int q = 0; q < NI; ++q) {
        const int row = (wave * NI + q) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz(row);
        const int gr = row0 + row;
        kofs[q] = 8 * c;
        voff[q] = gr < rows_lim ? (uint32_t)(((int64_t)gr * ld + 8 * c) * 2) : kOOB;
      }
    } else {
      constexpr int CH = ROWS / 8;  // 16-byte chunks per k-row
      constexpr int XM = ROWS >= 128 ? 3 : 1;  // 32-column blocks swapped by k % 4 (k % 2 at 64 rows)
      rsrc = make_rsrc4(base, (uint32_t)(((int64_t)(K - 1) * ld + rows_lim) * 2));
      kstep = (uint32_t)(ld * 2);
#pragma unroll
      for (int q = 0; q < NI; ++q) {
        const int L = (wave * NI + q) * 64 + lane;
        const int k = L / CH;
        const int c = (L % CH) ^ (4 * (k & XM));
        const int gm = row0 + 8 * c;
        voff[q] = gm < rows_lim ? (uint32_t)(((int64_t)k * ld + gm) * 2) : kOOB;
      }
      kofs[0] = 0;
    }
  }

  // The tile starting at k0 into the operand tile at LDS address dst.
  // CHECK_K: the tile straddles K (k-rows past K of an m/n-contiguous operand
  // fall outside the buffer by themselves).
  template <bool CHECK_K>
  __device__ __forceinline__ void load(uint32_t dst, int k0, int K) const {
    const uint32_t step = (uint32_t)k0 * kstep;
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      uint32_t off = voff[q] + step;
      if constexpr (CHECK_K && KCONTIG) off = (k0 + kofs[q] < K) ? off : kOOB;
      dma16(rsrc, dst + lds0 + q * 1024, off);
    }
  }
};

// Up to kMaxGroup independent GEMMs of one layout and epilogue in one launch;
// workgroup b works on GEMM g with tile_start[g] <= b < tile_start[g+1].
constexpr int kMaxGroup = 16;
struct GroupParams {
  Params p[kMaxGroup];
  int tile_start[kMaxGroup + 1];
  int n;
};

// LDS ring depth per tile shape: as many BK-deep stages (up to 4) as fit in a
// CU's 160 KiB shared by OCC workgroups (64 deep: a 256x256 stage is 64 KiB,
// 256x128 48 KiB, 128x128 32 KiB; 32 deep: half of that).
template <int BM, int BN, int OCC = 1, int BK = BKT>
struct Ring {
  static constexpr int STAGE = (BM + BN) * BK * 2;
  static constexpr int FIT = (160 * 1024 / OCC) / STAGE;  // OCC workgroups share a CU's 160 KiB
  static constexpr int NS = FIT < 4 ? FIT : 4;
  static_assert(NS >= 2, "the ring needs two stages");
  static constexpr int S2 = NS > 2 ? STAGE : 16;
  static constexpr int S3 = NS > 3 ? STAGE : 16;
};

template <int BM, int BN, bool AK, bool BKC, int EPI, int OCC, int BK, int WV>
__device__ __forceinline__ void gemm_tile(const Params& p, int tile, int split, char* s0, char* s1, char* s2,
                                          char* s3, bool pre, bool has_next, const Params& np, int ntile,
                                          int nsplit);

// The ring stages are separate LDS objects (so the code that addresses each
// one is fixed at compile time).
#define ZB_GEMM_LDS(BM, BN, OCC, BK)                                                  \
  __shared__ __attribute__((aligned(1024))) char s0[Ring<BM, BN, OCC, BK>::STAGE];  \
  __shared__ __attribute__((aligned(1024))) char s1[Ring<BM, BN, OCC, BK>::STAGE];  \
  __shared__ __attribute__((aligned(1024))) char s2[Ring<BM, BN, OCC, BK>::S2];     \
  __shared__ __attribute__((aligned(1024))) char s3[Ring<BM, BN, OCC, BK>::S3]

template <int BM, int BN, bool AK, bool BKC, int EPI, int WV>
__global__ void __attribute__((amdgpu_flat_work_group_size(64 * WV, 64 * WV), amdgpu_waves_per_eu(WV / 4, WV / 4)))
gemm_bf16_mfma(Params p) {
  ZB_GEMM_LDS(BM, BN, 1, BKT);
  const int total = p.nbm * p.nbn * p.splits;
  // Persistent when the grid is smaller: a tile's epilogue runs after the
  // first copies of the workgroup's next tile are issued.
  for (int b0 = blockIdx.x; b0 < total; b0 += gridDim.x) {
    const int nb0 = b0 + gridDim.x;
    int b = b0, nb = nb0 < total ? nb0 : b0;
    if (p.xcd_remap) {  // a tile's splits share an XCD
      b = xcd_remap(b, total);
      nb = xcd_remap(nb, total);
    }
    gemm_tile<BM, BN, AK, BKC, EPI, 1, BKT, WV>(p, b / p.splits, b % p.splits, s0, s1, s2, s3,
                                                 b0 != (int)blockIdx.x, nb0 < total, p, nb / p.splits,
                                                 nb % p.splits);
  }
}

template <int BM, int BN, bool AK, bool BKC, int EPI, int OCC, int BK, int WV>
__global__ void __attribute__((amdgpu_flat_work_group_size(64 * WV, 64 * WV),
                               amdgpu_waves_per_eu(OCC * WV / 4, OCC * WV / 4)))
gemm_bf16_mfma_group(GroupParams gp) {
  ZB_GEMM_LDS(BM, BN, OCC, BK);
  const int total = gp.tile_start[gp.n];
  // Persistent when the grid is smaller than the tile count: workgroup w takes
  // tiles w, w + grid, ..., and a tile's epilogue runs after the next tile's
  // first copies are issued.  The grid is a multiple of the XCD count, so a
  // workgroup's tiles stay on its XCD.
  auto locate = [&](int b0, int& g) {
    int b = b0;
    if (total % XCDS == 0) b = (b % XCDS) * (total / XCDS) + b / XCDS;  // one XCD works a GEMM's neighbours
    g = 0;
    while (g + 1 < gp.n && b >= gp.tile_start[g + 1]) ++g;
    return b - gp.tile_start[g];
  };
  for (int b0 = blockIdx.x; b0 < total; b0 += gridDim.x) {
    const int nb0 = b0 + gridDim.x;
    int g, ng;
    const int tile = locate(b0, g);
    const int ntile = locate(nb0 < total ? nb0 : b0, ng);
    gemm_tile<BM, BN, AK, BKC, EPI, OCC, BK, WV>(gp.p[g], tile, 0, s0, s1, s2, s3, b0 != (int)blockIdx.x,
                                                  nb0 < total, gp.p[ng], ntile, 0);
  }
}

// 32x16 bf16 MFMA operand (lane l: row l % 32, k = 8 (l / 32) .. +7) read
// from a k-contiguous LDS tile: one 16-byte read at a precomputed offset.
__device__ __forceinline__ bf16x8 frag_k(const char* tile, uint32_t off) {
  return *reinterpret_cast<const bf16x8*>(tile + off);
}
// The same operand from an m/n-contiguous tile: two transposing 8-byte reads
// (k 0..3 and 4..7 of the lane's eight), rows RB bytes apart.
template <int RB>
__device__ __forceinline__ bf16x8 frag_t(const char* tile, uint32_t off) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + off));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + off + 4 * RB));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Copies of the first min(NS, nk) k tiles of one output tile (split `split`
// of tile `tile`) into ring stages 0, 1, ..., A then B for each stage: the
// same copies, in the same order, as the k loop's own start.
template <int BM, int BN, bool AK, bool BKC, int OCC, int BK, int WV>
__device__ __forceinline__ void tile_prologue(const Params& p, int tile, int split, char* s0, char* s1, char* s2,
                                              char* s3) {
  constexpr int NS = Ring<BM, BN, OCC, BK>::NS;
  constexpr int AT = BM * BK * 2;
  char* const bufs[4] = {s0, s1, s2, s3};
  int tm, tn;
  tile_raster(p, tm, tn, tile);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  DmaLoader<BM, AK, BK, WV> la(static_cast<const uint16_t*>(p.A), p.lda, tm * BM, p.M, p.K, wave, lane);
  DmaLoader<BN, BKC, BK, WV> lb(static_cast<const uint16_t*>(p.B), p.ldb, tn * BN, p.N, p.K, wave, lane);
  const int nk_all = (p.K + BK - 1) / BK;
  const int kt0 = split * p.kts;
  const int nk = min(nk_all - kt0, p.kts);
  const bool k_ragged = (p.K % BK) != 0;
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    if (st < nk) {
      const uint32_t b = __builtin_amdgcn_readfirstlane(lds_addr(bufs[st]));
      const int k0 = (kt0 + st) * BK;
      if (k_ragged && kt0 + st == nk_all - 1) {
        la.template load<true>(b, k0, p.K);
        lb.template load<true>(b + AT, k0, p.K);
      } else {
        la.template load<false>(b, k0, p.K);
        lb.template load<false>(b + AT, k0, p.K);
      }
    }
  }
}

template <int BM, int BN, bool AK, bool BKC, int EPI, int OCC, int BK, int WV>
__device__ __forceinline__ void gemm_tile(const Params& p, int tile, int split, char* s0, char* s1, char* s2,
                                          char* s3, bool pre, bool has_next, const Params& np, int ntile,
                                          int nsplit) {
  constexpr int WTM = BM / 2, WTN = BN / (WV / 2);  // waves in a 2 x (WV / 2) grid
  // Fragments alternate between two register buffers over a tile's 16-deep k
  // steps; the last step's are in buffer 1 while the next tile's first go to
  // buffer 0, which needs an even number of steps per tile.
  static_assert(BK % 32 == 0, "k tiles of an even number of 16-deep steps");
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int NS = Ring<BM, BN, OCC, BK>::NS;
  constexpr int AT = BM * BK * 2;  // bytes of the A tile in a ring stage (the B tile follows)
  char* const bufs[4] = {s0, s1, s2, s3};

  int tm, tn;
  tile_raster(p, tm, tn, tile);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;

  // The MFMA takes the B fragment as its row operand and the A fragment as its
  // column operand, so lane l ends up with output row m = .. + l % 32 and the
  // four consecutive columns n = .. + 8 g + 4 (l / 32) + {0..3} in registers
  // 4g..4g+3 of each 32x32 block: vector stores in the epilogue.
  const int em = m0 + wm * WTM + (lane & 31);
  const int en = n0 + wn * WTN + 4 * (lane >> 5);

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  __amdgpu_buffer_rsrc_t crsrc = make_rsrc(p.C, (uint32_t)(((int64_t)(p.M - 1) * p.ldc + p.N) *
                                                           (EPI == EPI_ACC ? 4 : 2)));

  DmaLoader<BM, AK, BK, WV> la(static_cast<const uint16_t*>(p.A), p.lda, m0, p.M, p.K, wave, lane);
  DmaLoader<BN, BKC, BK, WV> lb(static_cast<const uint16_t*>(p.B), p.ldb, n0, p.N, p.K, wave, lane);
  constexpr int NI = DmaLoader<BM, AK, BK, WV>::NI + DmaLoader<BN, BKC, BK, WV>::NI;  // copies per wave per tile
  // 16-byte stores one wave's epilogue issues on every path.  With `pre` the
  // previous tile's epilogue (same kind) ran after this tile's first copies
  // were issued; loads and stores complete in issue order, so those copies are
  // done once no more than this many newer operations are outstanding.
  constexpr int EPN = (EPI == EPI_ACC || EPI == EPI_PART || EPI == EPI_GELU) ? TM * TN * 4 : TM * TN * 2;
  // This workgroup's k tiles: [kt0, kt0 + nk) of the product's ceil(K / BK).
  const int nk_all = (p.K + BK - 1) / BK;
  const int kt0 = split * p.kts;
  const int nk = min(nk_all - kt0, p.kts);
  const bool k_ragged = (p.K % BK) != 0;  // only the product's last tile straddles K

  // Fragment read offsets within an operand tile.
  //  k-contiguous: row = base + 32 i + lane % 32, chunk = 2 kk + lane / 32,
  //    stored at P ^ 2 (kk ^ 2 (i % 2)) with P fixed per lane: ra[kk ^ 2 (i % 2)] + 4096 i
  //    (P takes bit 5 of the wave's first row, set when a wave holds an odd number of
  //    32-row blocks, as in a 64-wide tile).
  //  m/n-contiguous (transposing reads): lane l = 16 g + ii reads k-row
  //    16 kk + 8 (g / 2) + 4 h + ii / 4 at column base + 32 i + 16 (g % 2) + 4 (ii % 4);
  //    with r = ii / 4 = k % 4 the chunk's position is ((base / 32 + i) ^ r) * 4 + s (r % 2 in a
  //    64-wide tile, which has two 32-column blocks).
  uint32_t ra[4], rb[4];
  {
    const int P = (lane >> 5) ^ (lane & 7) ^ ((lane >> 3) & 3);
    const int g = lane >> 4, ii = lane & 15, r = ii >> 2;
    const int s = 2 * (g & 1) + ((ii & 3) >> 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (AK) {
        ra[q] = (wm * WTM + (lane & 31)) * 128 + ((P ^ (2 * q) ^ (4 * ((wm * TM) & 1))) << 4);
      } else {
        const int blk = wm * WTM / 32 + q;
        ra[q] = (8 * (g >> 1) + r) * (BM * 2) + 64 * (blk ^ (r & (BM >= 128 ? 3 : 1))) + 16 * s + 8 * (ii & 1);
      }
      if constexpr (BKC) {
        rb[q] = (wn * WTN + (lane & 31)) * 128 + ((P ^ (2 * q) ^ (4 * ((wn * TN) & 1))) << 4);
      } else {
        const int blk = wn * WTN / 32 + q;
        rb[q] = (8 * (g >> 1) + r) * (BN * 2) + 64 * (blk ^ (r & (BN >= 128 ? 3 : 1))) + 16 * s + 8 * (ii & 1);
      }
    }
  }
  bf16x8 af[2][TM], bfr[2][TN];
  auto read_a = [&](const char* buf, int kk, int fb) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if constexpr (AK) af[fb][i] = frag_k(buf, ra[kk ^ (2 * (i & 1))] + i * 32 * 128);
      else af[fb][i] = frag_t<BM * 2>(buf, ra[i] + kk * 16 * (BM * 2));
    }
  };
  auto read_b = [&](const char* buf, int kk, int fb) {
    const char* bt = buf + AT;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if constexpr (BKC) bfr[fb][j] = frag_k(bt, rb[kk ^ (2 * (j & 1))] + j * 32 * 128);
      else bfr[fb][j] = frag_t<BN * 2>(bt, rb[j] + kk * 16 * (BN * 2));
    }
  };
  auto read_frags = [&](const char* buf, int kk, int fb) {
    read_a(buf, kk, fb);
    read_b(buf, kk, fb);
  };
  auto mfma_row = [&](int fb, int i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[fb][j], af[fb][i], acc[i][j], 0, 0, 0);
  };
  auto mfmas = [&](int fb) {
#pragma unroll
    for (int i = 0; i < TM; ++i) mfma_row(fb, i);
  };
  // Copies of tile t into ring stage BI: operand A (which = 0) or B (1).
  auto dma_op = [&](auto bi, int which, int t) {
    const uint32_t b = __builtin_amdgcn_readfirstlane(lds_addr(bufs[decltype(bi)::value]));
    const int k0 = (kt0 + t) * BK;
    const bool rag = k_ragged && kt0 + t == nk_all - 1;
    if (which == 0) {
      if (rag) la.template load<true>(b, k0, p.K);
      else la.template load<false>(b, k0, p.K);
    } else {
      if (rag) lb.template load<true>(b + AT, k0, p.K);
      else lb.template load<false>(b + AT, k0, p.K);
    }
  };

  // Ring: tiles t+1 .. t+NS-1 are in flight while tile t feeds the MFMAs;
  // tile t+NS goes into tile t's stage once every wave has read it.  The
  // first NS tiles' copies (none when K == 0) come from tile_prologue: here,
  // or before the previous tile's epilogue when `pre`.
  if (!pre) tile_prologue<BM, BN, AK, BKC, OCC, BK, WV>(p, tile, split, s0, s1, s2, s3);
  if (nk > 0) {  // K == 0: empty sum
    if (nk >= NS) {
      if (pre) wait_vm_barrier<(NS - 1) * NI + EPN>();
      else wait_vm_barrier<(NS - 1) * NI>();
    } else {
      wait_vm_barrier<0>();
    }
    read_frags(bufs[0], 0, 0);
  }

  // One tile from stage CUR: fragments double-buffered across its four
  // 16-deep k steps.  Before the last step every wave waits for its own copies
  // of tile t+1 and for its reads of tile t, then meets the others at the
  // barrier.  The last step's MFMA rows are interleaved with the first reads
  // of tile t+1 (issued even past the last tile, where they are discarded, so
  // the compiler sees one path) and with the refill of stage CUR.
  auto body = [&](auto bi, int t) {
    constexpr int CUR = decltype(bi)::value;
    constexpr int NXT = (CUR + 1) % NS;
    const char* cur = bufs[CUR];
#pragma unroll
    for (int kk = 0; kk < BK / 16 - 1; ++kk) {
      read_frags(cur, kk + 1, (kk + 1) & 1);  // all reads go out ahead of the step's MFMAs
      __builtin_amdgcn_sched_barrier(0);
      mfmas(kk & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (t + NS - 1 < nk) {
      // Tiles t + 1 .. NS - 1 came from the start before the previous epilogue.
      if (pre && t < NS - 1) wait_vm_barrier<(NS - 2) * NI + EPN>();
      else wait_vm_barrier<(NS - 2) * NI>();
    } else {
      wait_vm_barrier<0>();
    }
    const bool refill = t + NS < nk;
    read_a(bufs[NXT], 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfma_row(1, 0);
    __builtin_amdgcn_sched_barrier(0);
    read_b(bufs[NXT], 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfma_row(1, 1);
    __builtin_amdgcn_sched_barrier(0);
    if (refill) dma_op(bi, 0, t + NS);
    if constexpr (TM > 2) mfma_row(1, 2);
    __builtin_amdgcn_sched_barrier(0);
    if (refill) dma_op(bi, 1, t + NS);
    if constexpr (TM > 3) mfma_row(1, 3);
    __builtin_amdgcn_sched_barrier(0);
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, (NS > 2 ? 2 : 0)>;
  using B3 = std::integral_constant<int, (NS > 3 ? 3 : 0)>;

  int t = 0;
  for (; t + NS <= nk; t += NS) {
    body(B0{}, t);
    body(B1{}, t + 1);
    if constexpr (NS > 2) body(B2{}, t + 2);
    if constexpr (NS > 3) body(B3{}, t + 3);
  }
  // Fewer than NS tiles left; t is a multiple of NS, so tile t + b is in stage b.
  if (t < nk) body(B0{}, t);
  if constexpr (NS > 2) {
    if (t + 1 < nk) body(B1{}, t + 1);
  }
  if constexpr (NS > 3) {
    if (t + 2 < nk) body(B2{}, t + 2);
  }

  // The epilogue's residual / pre-activation values (every row of blocks,
  // 16 bytes per lane: 8 columns) are requested and waited for before the
  // next tile's first copies go out: vmcnt retires in order, so loads issued
  // after those copies would wait for the whole ring fill.
  const int sn = n0 + wn * WTN + 8 * (lane >> 5);  // this lane's stored column, before 32 j + 16 q
  __amdgpu_buffer_rsrc_t rrsrc = make_rsrc(EPI == EPI_RESID || EPI == EPI_DGELU ? p.R : p.C,
                                           (uint32_t)(((int64_t)(p.M - 1) * p.ldr + p.N) * 2));
  u32x4 wr[TM][TN][2];
  if constexpr (EPI == EPI_RESID || EPI == EPI_DGELU) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int m = em + i * 32, n = sn + j * 32 + 16 * q;
          const uint32_t roff = (m < p.M && n < p.N) ? (uint32_t)(((int64_t)m * p.ldr + n) * 2) : kOOB;
          wr[i][j][q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rrsrc, (int)roff, 0, 0));
        }
  }
  // s_waitcnt vmcnt(0) as an instruction the compiler tracks (gfx9 encoding; expcnt 7 and lgkmcnt 15
  // mean no wait on those), so it places no further waits for these loads.
  if constexpr (EPI == EPI_RESID || EPI == EPI_DGELU) __builtin_amdgcn_s_waitcnt(0x0F70);

  // Every wave is past its last read of the ring (and no copy is in flight):
  // the next tile's first copies go out before this tile's epilogue.
  if (has_next) {
    wait_vm_barrier<0>();
    tile_prologue<BM, BN, AK, BKC, OCC, BK, WV>(np, ntile, nsplit, s0, s1, s2, s3);
  }

  // Epilogue: lane (i, j, g) owns C[em + 32 i][en + 32 j + 8 g + 0..3].
  if constexpr (EPI == EPI_PART) {
    // This split's fp32 partial sum, to its own M x N slice.
    float* const cp = static_cast<float*>(p.C) + (int64_t)split * p.M * p.ldc;
    const __amdgpu_buffer_rsrc_t prsrc = make_rsrc(cp, (uint32_t)(((int64_t)(p.M - 1) * p.ldc + p.N) * 4));
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int m = em + i * 32, n = en + j * 32 + 8 * g;
          const uint32_t off = (m < p.M && n < p.N) ? (uint32_t)(((int64_t)m * p.ldc + n) * 4) : kOOB;
          f32x4 v;
#pragma unroll
          for (int t2 = 0; t2 < 4; ++t2) v[t2] = acc[i][j][4 * g + t2];
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), prsrc, (int)off, 0, 0);
        }
  } else if constexpr (EPI == EPI_ACC) {
    // dW (+)= this GEMM's sum over k, in fp32.  Rows of 32x32 blocks go
    // through a two-deep pipeline: the old values of row i + 1 (TN * 4
    // 16-byte loads per lane) are requested before row i is added and
    // stored, so one row's loads are in flight while the previous one is
    // written.
    auto offsets = [&](int i, uint32_t (&off)[TN][4]) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int m = em + i * 32, n = en + j * 32 + 8 * g;
          off[j][g] = (m < p.M && n < p.N) ? (uint32_t)(((int64_t)m * p.ldc + n) * 4) : kOOB;
        }
    };
    auto load_row = [&](const uint32_t (&off)[TN][4], f32x4 (&c)[TN][4]) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          c[j][g] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(crsrc, (int)off[j][g], 0, 0));
    };
    auto store_row = [&](int i, const uint32_t (&off)[TN][4], const f32x4 (*c)[4]) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v;
#pragma unroll
          for (int t2 = 0; t2 < 4; ++t2) v[t2] = acc[i][j][4 * g + t2];
          if (c) {
#pragma unroll
            for (int t2 = 0; t2 < 4; ++t2) v[t2] = c[j][g][t2] + v[t2];
          }
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), crsrc, (int)off[j][g], 0, 0);
        }
    };
    if (p.beta) {
      uint32_t off[2][TN][4];
      f32x4 c[2][TN][4];
      offsets(0, off[0]);
      load_row(off[0], c[0]);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if (i + 1 < TM) {
          offsets(i + 1, off[(i + 1) & 1]);
          load_row(off[(i + 1) & 1], c[(i + 1) & 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
        store_row(i, off[i & 1], c[i & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        uint32_t off[TN][4];
        offsets(i, off);
        store_row(i, off, nullptr);
      }
    }
  } else {
    __amdgpu_buffer_rsrc_t zrsrc = make_rsrc(EPI == EPI_GELU ? p.Z : p.C,
                                             (uint32_t)(((int64_t)(p.M - 1) * p.ldz + p.N) * 2));
    // The GeLU form is fixed per launch: one branch here, none per element.
    // Column groups g = 2q and 2q+1 of a 32x32 block are stored together: lane
    // l < 32 holds columns 8g..8g+3 of both, lane l+32 columns 8g+4..8g+7;
    // v_permlane32_swap gives lane l all eight columns of group 2q and lane
    // l+32 all eight of group 2q+1, so every store is 16 bytes per lane and 32
    // contiguous bytes per row.
    auto swap_store = [&](const __amdgpu_buffer_rsrc_t& rs, int64_t ld, int m, int n, u32x2 a, u32x2 b) {
      const auto s0 = __builtin_amdgcn_permlane32_swap(a[0], b[0], false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(a[1], b[1], false, false);
      const u32x4 w = {s0[0], s1[0], s0[1], s1[1]};
      const uint32_t off = (m < p.M && n < p.N) ? (uint32_t)(((int64_t)m * ld + n) * 2) : kOOB;
      __builtin_amdgcn_raw_buffer_store_b128(w, rs, (int)off, 0, 0);
    };
    auto store_all = [&](auto kind_c) {
      constexpr int KIND = decltype(kind_c)::value;
      // One row of 32x32 blocks at a time, its residual / pre-activation
      // values already in registers (loaded before the hand-over); the
      // barriers keep rows from interleaving (shorter live ranges).  With
      // GeLU the row's pre-activation Z is stored before its activation, so
      // each buffer's cache lines are completed by consecutive stores
      // (interleaving the two outputs wrote about 1.5x the bytes to memory).
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int m = em + i * 32;
        u32x2 rr[TN][4];
        if constexpr (EPI == EPI_RESID || EPI == EPI_DGELU) {
          // The inverse of swap_store: lanes l and l + 32 swap halves so that
          // lane l holds columns 8 g .. 8 g + 3 and lane l + 32 8 g + 4 .. + 7.
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const auto s = __builtin_amdgcn_permlane32_swap(wr[i][j][q][0], wr[i][j][q][2], false, false);
              const auto t = __builtin_amdgcn_permlane32_swap(wr[i][j][q][1], wr[i][j][q][3], false, false);
              rr[j][2 * q] = u32x2{s[0], t[0]};
              rr[j][2 * q + 1] = u32x2{s[1], t[1]};
            }
        }
        if constexpr (EPI == EPI_GELU) {
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              u32x2 zv[2];
#pragma unroll
              for (int gg = 0; gg < 2; ++gg) {
                const int g = 2 * q + gg;
                zv[gg] = u32x2{pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                               pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3])};
              }
              swap_store(zrsrc, p.ldz, m, sn + j * 32 + 16 * q, zv[0], zv[1]);
            }
        }
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            u32x2 cv[2];
#pragma unroll
            for (int gg = 0; gg < 2; ++gg) {
              const int g = 2 * q + gg;
              float v[4];
#pragma unroll
              for (int t2 = 0; t2 < 4; ++t2) v[t2] = acc[i][j][4 * g + t2];
              if constexpr (EPI == EPI_RESID || EPI == EPI_DGELU) {
                const u32x2 rv = rr[j][g];
                const float r[4] = {__uint_as_float(rv[0] << 16), __uint_as_float(rv[0] & 0xffff0000u),
                                    __uint_as_float(rv[1] << 16), __uint_as_float(rv[1] & 0xffff0000u)};
#pragma unroll
                for (int t2 = 0; t2 < 4; ++t2) {
                  if constexpr (EPI == EPI_RESID) v[t2] += r[t2];
                  else v[t2] *= gelu_grad_f(r[t2], KIND);
                }
              }
              if constexpr (EPI == EPI_GELU) {
#pragma unroll
                for (int t2 = 0; t2 < 4; ++t2) v[t2] = gelu_f(v[t2], KIND);
              }
              cv[gg] = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            }
            const int n = sn + j * 32 + 16 * q;
            swap_store(crsrc, p.ldc, m, n, cv[0], cv[1]);
          }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if ((EPI == EPI_GELU || EPI == EPI_DGELU) && p.gelu == ZB_GELU_TANH)
      store_all(std::integral_constant<int, ZB_GELU_TANH>{});
    else
      store_all(std::integral_constant<int, ZB_GELU_ERF>{});
  }
}

// Split-K second pass: C = epilogue(sum of the splits' fp32 partials, added in
// split order).  Partials are [splits][M][N] fp32; each thread takes 8
// consecutive outputs of a row (N and the leading dimensions of C, R and Z are
// multiples of 8, checked on the host).
template <int EPI>
__global__ void __launch_bounds__(256) splitk_reduce(Params p, const float* part) {
  const int groups = p.N / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)p.M * groups) return;
  const int m = (int)(idx / groups), n = (int)(idx % groups) * 8;
  const int64_t slice = (int64_t)p.M * p.N;
  const f32x4* q = reinterpret_cast<const f32x4*>(part + (int64_t)m * p.N + n);
  f32x4 a = q[0], b = q[1];
  for (int s = 1; s < p.splits; ++s) {
    const f32x4* r = reinterpret_cast<const f32x4*>(part + s * slice + (int64_t)m * p.N + n);
    a += r[0];
    b += r[1];
  }
  float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  if constexpr (EPI == EPI_RESID || EPI == EPI_DGELU) {
    const u32x4 rv = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.R) + (int64_t)m * p.ldr + n);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t w = rv[e >> 1];
      const float r = __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
      if constexpr (EPI == EPI_RESID) v[e] += r;
      else v[e] *= gelu_grad_f(r, p.gelu);
    }
  }
  if constexpr (EPI == EPI_GELU) {
    u32x4 zv;
#pragma unroll
    for (int e = 0; e < 4; ++e) zv[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.Z) + (int64_t)m * p.ldz + n) = zv;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = gelu_f(v[e], p.gelu);
  }
  u32x4 cv;
#pragma unroll
  for (int e = 0; e < 4; ++e) cv[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
  *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.C) + (int64_t)m * p.ldc + n) = cv;
}

// ------------------------------------------------- fp32 storage (plain FMA tiles)

template <typename T, int EPI>
__global__ void __launch_bounds__(256) gemm_simt(Params p, int ak, int bk) {
  constexpr int TB = 64, KB = 16;
  __shared__ float sA[KB][TB + 1], sB[KB][TB + 1];
  int tm, tn;
  tile_coords(p, tm, tn, blockIdx.x);
  const int m0 = tm * TB, n0 = tn * TB;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const T* A = static_cast<const T*>(p.A);
  const T* B = static_cast<const T*>(p.B);
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v = 0.0f;
      if constexpr (EPI == EPI_ACC) {
        const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
        if (p.beta && m < p.M && n < p.N) v = static_cast<const float*>(p.C)[(int64_t)m * p.ldc + n];
      }
      acc[i][j] = v;
    }
  for (int k0 = 0; k0 < p.K; k0 += KB) {
    for (int idx = tid; idx < KB * TB; idx += 256) {
      const int kk = idx / TB, mm = idx % TB;
      const int gk = k0 + kk, gm = m0 + mm, gn = n0 + mm;
      float a = 0.0f, b = 0.0f;
      if (gk < p.K && gm < p.M) a = ld_elem<T>(A, ak ? (int64_t)gm * p.lda + gk : (int64_t)gk * p.lda + gm);
      if (gk < p.K && gn < p.N) b = ld_elem<T>(B, bk ? (int64_t)gn * p.ldb + gk : (int64_t)gk * p.ldb + gn);
      sA[kk][mm] = a;
      sB[kk][mm] = b;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m < p.M && n < p.N) epi_store<T, EPI>(p, m, n, acc[i][j]);
    }
}

// ------------------------------------------------------------------- dispatch

struct TileCfg {
  int bm, bn;
  double rate;  // FLOP per microsecond of one workgroup with every CU busy (measured, MI355X)
};
// The 128x64 rate is the one seen with operands that start outside the caches,
// as in a pipeline whose other passes evict them: it moves 1.5x the bytes per
// FLOP of 128x128 into LDS and loses more than the wider tiles when it
// misses (1024x2048x8192: 3.4e6 warm, about 2.2e6 cold).  Its place is short
// k loops on few output tiles, where it fills the chip without a split-K pass.
constexpr TileCfg kTiles[] = {{256, 256, 5.4e6}, {256, 128, 4.75e6}, {128, 128, 4.1e6}, {128, 64, 2.4e6}};
constexpr int kNarrowTile = 3;  // 128x64: F and B layouts only
constexpr int kCUs = 256;
constexpr double kFixedUs = 2.0;        // per workgroup: first copies in, epilogue out
constexpr double kReduceFixedUs = 3.0;  // split-K: the second launch
constexpr double kReduceBytesPerUs = 4e6;   // its fp32 partial reads and bf16 traffic
constexpr double kPartWriteBytesPerUs = 8e6;  // the partial writes, beside the MFMA work

struct GemmPlan {
  int tile = 2, splits = 1, kts = 0;
  double cost = 1e300;
};

// Tile shape and split-K factor by a wave-quantised cost model: whole waves
// of workgroups over the CUs, each taking its k tiles at the shape's rate plus
// a fixed overhead; a split adds the pass that reads the fp32 partials back.
// Splitting is only considered while the tiles alone leave CUs idle, and only
// when the partials fit in `arena` bytes.  The narrow 128x64 tile fills the
// chip without a split where 128x128 tiles would leave CUs idle (T = 1024
// token products with N = 2048: 256 workgroups instead of 128).
GemmPlan plan_gemm(int M, int N, int K, bool can_split, size_t arena, bool narrow_ok) {
  const int nk = (K + BKT - 1) / BKT;
  GemmPlan best;
  best.kts = nk;
  for (int t = 0; t < (narrow_ok ? 4 : 3); ++t) {
    const TileCfg& c = kTiles[t];
    const int nb = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
    for (int S = 1; S <= 4; S *= 2) {
      if (S > 1 && (!can_split || S > nk || nb >= kCUs)) continue;
      const int kts = S > 1 ? (nk + S - 1) / S : nk;
      if (S > 1 && (S - 1) * kts >= nk) continue;
      if (S > 1 && (double)S * M * N * 4 > (double)arena) continue;
      const int waves = (nb * S + kCUs - 1) / kCUs;
      double cost = waves * (2.0 * c.bm * c.bn * (double)kts * BKT / c.rate + kFixedUs);
      if (S > 1)
        cost += kReduceFixedUs + (4.0 * S + 4.0) * M * (double)N / kReduceBytesPerUs +
                4.0 * S * M * (double)N / kPartWriteBytesPerUs;
      if (cost < best.cost - 1e-9) best = GemmPlan{t, S, kts, cost};
    }
  }
  return best;
}

// Compute units of the current device (queried once per device).
int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < XCDS) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

template <int BM, int BN, bool AK, bool BKC, int EPI>
void launch_mfma(Params p, hipStream_t s) {
  p.nbm = (p.M + BM - 1) / BM;
  p.nbn = (p.N + BN - 1) / BN;
  p.xcd_remap = 1;
  if (p.splits < 1) {
    p.splits = 1;
    p.kts = (p.K + BKT - 1) / BKT;
  }
  // One workgroup per CU looping over the tiles: the same kernel time, and
  // with the stages on separate streams a 2% shorter step (gpt_full_h4096).
  const int total = p.nbm * p.nbn * p.splits;
  const int grid = std::min(total, cu_count() / XCDS * XCDS);
  constexpr int WV = (BM >= 128 && BN >= 128) ? kWavesWide : kWavesNarrow;
  hipLaunchKernelGGL((gemm_bf16_mfma<BM, BN, AK, BKC, EPI, WV>), dim3(grid), dim3(64 * WV), 0, s, p);
}

template <int BM, int BN, int OCC = 1, int BK = BKT>
void launch_w_group(GroupParams gp, hipStream_t s) {
  int total = 0;
  for (int g = 0; g < gp.n; ++g) {
    gp.p[g].nbm = (gp.p[g].M + BM - 1) / BM;
    gp.p[g].nbn = (gp.p[g].N + BN - 1) / BN;
    gp.p[g].xcd_remap = 0;
    gp.p[g].splits = 1;
    gp.p[g].kts = (gp.p[g].K + BK - 1) / BK;
    gp.tile_start[g] = total;
    total += gp.p[g].nbm * gp.p[g].nbn;
  }
  gp.tile_start[gp.n] = total;
  // One workgroup per CU (OCC per CU), each looping over its tiles: measured
  // 3-4% faster than one workgroup per tile for the grouped W launch.
  const int grid = std::min(total, cu_count() / XCDS * XCDS * OCC);
  hipLaunchKernelGGL((gemm_bf16_mfma_group<BM, BN, false, false, EPI_ACC, OCC, BK, kWavesWide>), dim3(grid),
                     dim3(64 * kWavesWide), 0, s, gp);
}

template <bool AK, bool BKC, int EPI>
void launch_tile(int t, const Params& p, hipStream_t s) {
  switch (t) {
    case 0: launch_mfma<256, 256, AK, BKC, EPI>(p, s); break;
    case 1: launch_mfma<256, 128, AK, BKC, EPI>(p, s); break;
    case kNarrowTile:
      if constexpr (AK) {
        launch_mfma<128, 64, AK, BKC, EPI>(p, s);
        break;
      }
      [[fallthrough]];
    default: launch_mfma<128, 128, AK, BKC, EPI>(p, s); break;
  }
}

template <typename T, int EPI>
void launch_simt(Params p, bool ak, bool bk, hipStream_t s) {
  p.nbm = (p.M + 63) / 64;
  p.nbn = (p.N + 63) / 64;
  hipLaunchKernelGGL((gemm_simt<T, EPI>), dim3(p.nbm * p.nbn), dim3(256), 0, s, p, (int)ak, (int)bk);
}

template <typename T>
void launch_simt_epi(int epi, const Params& p, bool ak, bool bk, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: launch_simt<T, EPI_STORE>(p, ak, bk, s); break;
    case EPI_RESID: launch_simt<T, EPI_RESID>(p, ak, bk, s); break;
    case EPI_GELU: launch_simt<T, EPI_GELU>(p, ak, bk, s); break;
    case EPI_DGELU: launch_simt<T, EPI_DGELU>(p, ak, bk, s); break;
    default: launch_simt<T, EPI_ACC>(p, ak, bk, s); break;
  }
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

}  // namespace

// Several weight-gradient GEMMs (W layout, fp32 accumulate) in one launch.
zb_status launch_gemm_w_group(const GemmDesc* gs, int n, hipStream_t s) {
  if (n <= 0) return ZB_OK;
  for (int i = 0; i < n; i += kMaxGroup) {
    const int cnt = std::min(kMaxGroup, n - i);
    GroupParams gp{};
    gp.n = 0;
    double flops = 0.0, bytes = 0.0;
    for (int k = 0; k < cnt; ++k) {
      const GemmDesc& g = gs[i + k];
      if (g.a_kcontig || g.b_kcontig || g.epi != EPI_ACC || g.dtype != ZB_DTYPE_BF16)
        return set_error(ZB_E_ARG, "grouped W launch takes bf16 W-layout GEMMs only");
      if (g.M == 0 || g.N == 0) continue;
      if (g.M % 8 || g.N % 8 || g.lda % 8 || g.ldb % 8 || !aligned16(g.A) || !aligned16(g.B))
        return set_error(ZB_E_UNSUPPORTED, "gemm: contiguous extents and leading dims must be multiples of 8");
      const double lim = 2147483648.0 - 256.0;
      if (2.0 * ((double)(g.K - 1) * g.lda + g.M) >= lim || 2.0 * ((double)(g.K - 1) * g.ldb + g.N) >= lim ||
          4.0 * ((double)(g.M - 1) * g.ldc + g.N) >= lim)
        return set_error(ZB_E_UNSUPPORTED, "gemm: an operand spans 2 GiB or more");
      Params& p = gp.p[gp.n++];
      p.M = g.M; p.N = g.N; p.K = g.K;
      p.A = g.A; p.lda = g.lda; p.B = g.B; p.ldb = g.ldb; p.C = g.C; p.ldc = g.ldc;
      p.R = nullptr; p.ldr = 0; p.Z = nullptr; p.ldz = 0; p.beta = g.beta; p.gelu = g.gelu;
      flops += 2.0 * g.M * g.N * (double)g.K;
      bytes += 2.0 * ((double)g.M * g.K + (double)g.K * g.N) + (g.beta ? 8.0 : 4.0) * g.M * g.N;
    }
    if (gp.n == 0) continue;
    // 256x256 tiles, one workgroup of eight waves per CU, 32-deep k tiles in
    // a four-stage ring (three in flight).  Measured in one process against
    // 64-deep tiles in a two-stage ring: 3.6% faster at T = 1024 and 2048, 7.8%
    // at 4096; 128x128 and 256x128 tiles two to a CU, and 128x256 tiles one or
    // two to a CU, were slower at T >= 2048 and no faster at T = 1024.  Eight
    // waves instead of four: 3.5-5% shorter launches at T = 1024 and 4096.
    ProfScope ps("gemm_w_group_256x256", flops, bytes, s);
    launch_w_group<256, 256, 1, 32>(gp, s);
    ZB_HIP_CHECK(hipGetLastError());
  }
  return ZB_OK;
}

size_t gemm_split_arena(int M, int N, int K) {
  if (N % 8) return 0;
  const GemmPlan pl = plan_gemm(M, N, K, true, (size_t)-1, true);
  return pl.splits == 1 ? 0 : (size_t)pl.splits * M * N * 4;
}

zb_status launch_gemm(const GemmDesc& g, hipStream_t s) {
  if (g.M < 0 || g.N < 0 || g.K < 0) return set_error(ZB_E_ARG, "gemm: negative size");
  if (g.M == 0 || g.N == 0) return ZB_OK;
  if (!g.C || (g.K > 0 && (!g.A || !g.B))) return set_error(ZB_E_ARG, "gemm: null operand");  // K = 0: C = 0
  if ((g.epi == EPI_RESID || g.epi == EPI_DGELU) && !g.R) return set_error(ZB_E_ARG, "gemm: null R");
  if (g.epi == EPI_GELU && !g.Z) return set_error(ZB_E_ARG, "gemm: null Z");
  Params p{};
  p.M = g.M; p.N = g.N; p.K = g.K;
  p.A = g.A; p.lda = g.lda; p.B = g.B; p.ldb = g.ldb; p.C = g.C; p.ldc = g.ldc;
  p.R = g.R; p.ldr = g.ldr; p.Z = g.Z; p.ldz = g.ldz; p.beta = g.beta; p.gelu = g.gelu;

  const double flops = 2.0 * g.M * g.N * (double)g.K;
  const size_t es = g.dtype == ZB_DTYPE_BF16 ? 2 : 4;
  double bytes = es * ((double)g.M * g.K + (double)g.K * g.N);
  if (g.epi == EPI_ACC) bytes += (g.beta ? 8.0 : 4.0) * g.M * g.N;
  else bytes += es * (double)g.M * g.N * ((g.epi == EPI_STORE) ? 1 : 2);

  if (g.dtype == ZB_DTYPE_FP32) {
    char name[48];
    snprintf(name, sizeof name, "gemm_%s_simt64", g.tag);
    ProfScope ps(name, flops, bytes, s);
    launch_simt_epi<float>(g.epi, p, g.a_kcontig, g.b_kcontig, s);
    ZB_HIP_CHECK(hipGetLastError());
    return ZB_OK;
  }
  // bf16 MFMA path: 16-byte vectors along every contiguous dimension.
  const int a_contig = g.a_kcontig ? g.K : g.M;
  const int b_contig = g.b_kcontig ? g.K : g.N;
  if (a_contig % 8 || b_contig % 8 || g.lda % 8 || g.ldb % 8 || !aligned16(g.A) || !aligned16(g.B))
    return set_error(ZB_E_UNSUPPORTED, "gemm: contiguous extents and leading dims must be multiples of 8 "
                                       "(M=%d N=%d K=%d lda=%lld ldb=%lld)", g.M, g.N, g.K,
                     (long long)g.lda, (long long)g.ldb);
  if (g.epi != EPI_ACC && (g.N % 8 || g.ldc % 8 || reinterpret_cast<uintptr_t>(g.C) % 16 ||
                           ((g.epi == EPI_RESID || g.epi == EPI_DGELU) && (g.ldr % 8 || !aligned16(g.R))) ||
                           (g.epi == EPI_GELU && (g.ldz % 8 || !aligned16(g.Z)))))
    return set_error(ZB_E_UNSUPPORTED, "gemm: bf16 outputs need N and leading dims that are multiples of 8 "
                                       "and 16-byte aligned rows (N=%d ldc=%lld)", g.N, (long long)g.ldc);
  {
    // Buffer offsets are 32-bit with out-of-range lanes placed at 2 GiB.
    const double lim = 2147483648.0 - 256.0;
    const double ea = 2.0 * ((g.a_kcontig ? (double)(g.M - 1) * g.lda + g.K : (double)(g.K - 1) * g.lda + g.M));
    const double eb = 2.0 * ((g.b_kcontig ? (double)(g.N - 1) * g.ldb + g.K : (double)(g.K - 1) * g.ldb + g.N));
    const double ec = (g.epi == EPI_ACC ? 4.0 : 2.0) * ((double)(g.M - 1) * g.ldc + g.N);
    if (ea >= lim || eb >= lim || ec >= lim)
      return set_error(ZB_E_UNSUPPORTED, "gemm: an operand spans 2 GiB or more");
  }
  // Split-K needs an arena and 16-byte rows in the second pass.
  const bool rz8 = (g.epi != EPI_RESID && g.epi != EPI_DGELU) || (g.ldr % 8 == 0 && aligned16(g.R));
  const bool z8 = g.epi != EPI_GELU || (g.ldz % 8 == 0 && aligned16(g.Z));
  const bool can_split = g.epi != EPI_ACC && g.part && g.N % 8 == 0 && g.ldc % 8 == 0 && aligned16(g.C) &&
                         aligned16(g.part) && rz8 && z8;
  const GemmPlan pl = plan_gemm(g.M, g.N, g.K, can_split, g.part_bytes, g.a_kcontig != 0);
  const int t = pl.tile;
  p.splits = pl.splits;
  p.kts = pl.kts;
  char name[48];
  static const char* kEpi[] = {"store", "resid", "gelu", "dgelu", "acc"};
  if (pl.splits > 1)
    snprintf(name, sizeof name, "gemm_%s_%dx%dk%d_%s", g.tag, kTiles[t].bm, kTiles[t].bn, pl.splits, kEpi[g.epi]);
  else
    snprintf(name, sizeof name, "gemm_%s_%dx%d_%s", g.tag, kTiles[t].bm, kTiles[t].bn, kEpi[g.epi]);
  ProfScope ps(name, flops, bytes, s);
  const bool ak = g.a_kcontig, bk = g.b_kcontig;
  if (pl.splits > 1) {
    Params pp = p;
    pp.C = g.part;
    pp.ldc = g.N;
    if (ak && !bk) launch_tile<true, false, EPI_PART>(t, pp, s);
    else if (ak && bk) launch_tile<true, true, EPI_PART>(t, pp, s);
    else return set_error(ZB_E_UNSUPPORTED, "gemm: split-K of this layout not built");
    ZB_HIP_CHECK(hipGetLastError());
    const int64_t threads = (int64_t)g.M * (g.N / 8);
    const dim3 grid((unsigned)((threads + 255) / 256));
    switch (g.epi) {
      case EPI_STORE: hipLaunchKernelGGL(splitk_reduce<EPI_STORE>, grid, dim3(256), 0, s, p, g.part); break;
      case EPI_RESID: hipLaunchKernelGGL(splitk_reduce<EPI_RESID>, grid, dim3(256), 0, s, p, g.part); break;
      case EPI_GELU: hipLaunchKernelGGL(splitk_reduce<EPI_GELU>, grid, dim3(256), 0, s, p, g.part); break;
      case EPI_DGELU: hipLaunchKernelGGL(splitk_reduce<EPI_DGELU>, grid, dim3(256), 0, s, p, g.part); break;
      default: return set_error(ZB_E_UNSUPPORTED, "gemm: epilogue %d with split-K", g.epi);
    }
    ZB_HIP_CHECK(hipGetLastError());
    return ZB_OK;
  }
  if (ak && !bk) {  // F
    switch (g.epi) {
      case EPI_STORE: launch_tile<true, false, EPI_STORE>(t, p, s); break;
      case EPI_RESID: launch_tile<true, false, EPI_RESID>(t, p, s); break;
      case EPI_GELU: launch_tile<true, false, EPI_GELU>(t, p, s); break;
      default: return set_error(ZB_E_UNSUPPORTED, "gemm: epilogue %d with F layout", g.epi);
    }
  } else if (ak && bk) {  // B
    switch (g.epi) {
      case EPI_STORE: launch_tile<true, true, EPI_STORE>(t, p, s); break;
      case EPI_RESID: launch_tile<true, true, EPI_RESID>(t, p, s); break;
      case EPI_DGELU: launch_tile<true, true, EPI_DGELU>(t, p, s); break;
      default: return set_error(ZB_E_UNSUPPORTED, "gemm: epilogue %d with B layout", g.epi);
    }
  } else if (!ak && !bk) {  // W
    if (g.epi != EPI_ACC) return set_error(ZB_E_UNSUPPORTED, "gemm: W layout needs the fp32 accumulate epilogue");
    launch_tile<false, false, EPI_ACC>(t, p, s);
  } else {
    return set_error(ZB_E_UNSUPPORTED, "gemm: layout (A m-contiguous, B k-contiguous) not built");
  }
  ZB_HIP_CHECK(hipGetLastError());
  return ZB_OK;
}

}  // namespace zb
