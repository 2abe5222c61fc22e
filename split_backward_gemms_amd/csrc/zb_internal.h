// Internal declarations shared by the library's translation units.
#pragma once

#include <cstdint>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "../../include/zb.h"

namespace zb {

// ---------------------------------------------------------------- errors
zb_status set_error(zb_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

#define ZB_HIP_CHECK(expr)                                                           \
  do {                                                                               \
    hipError_t e_ = (expr);                                                          \
    if (e_ != hipSuccess)                                                            \
      return ::zb::set_error(ZB_E_HIP, "%s failed: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

// -------------------------------------------------------------- schedule
struct SimPass {
  int op;         // index into the input op list
  int stage;
  int64_t start;
  int64_t end;
};

zb_status schedule_stage_order(int order, int P, int m, int stage, std::vector<zb_op>& out);
zb_status schedule_simulate(int P, int m, const zb_op* ops, int n_ops, const int64_t* t,
                            int64_t t_comm, std::vector<SimPass>& passes, zb_sim_stats* stats);
void schedule_linearize(const std::vector<SimPass>& passes, std::vector<int>& order);
zb_status schedule_validate(int P, int m, const zb_op* ops, int n_ops, int* bad);

// ----------------------------------------------------------------- kernels
enum Epilogue {
  EPI_STORE = 0,   // C = acc
  EPI_RESID = 1,   // C = acc + R
  EPI_GELU = 2,    // Z = acc; C = gelu(acc)
  EPI_DGELU = 3,   // C = acc * gelu'(R)          (R = saved pre-activation)
  EPI_ACC = 4,     // C(fp32) = (beta ? C : 0) + acc
  EPI_PART = 5     // split-K partial: C(fp32) + split * M * ldc = acc (internal to the GEMM launcher)
};

// C[M,N] = sum_k A(m,k) B(k,n) with
//   A(m,k) = A[m*lda + k] if a_kcontig else A[k*lda + m]
//   B(k,n) = B[n*ldb + k] if b_kcontig else B[k*ldb + n]
struct GemmDesc {
  int M = 0, N = 0, K = 0;
  const void* A = nullptr;
  int64_t lda = 0;
  bool a_kcontig = true;
  const void* B = nullptr;
  int64_t ldb = 0;
  bool b_kcontig = true;
  void* C = nullptr;
  int64_t ldc = 0;
  const void* R = nullptr;   // residual (EPI_RESID) or pre-activation (EPI_DGELU)
  int64_t ldr = 0;
  void* Z = nullptr;         // pre-activation output (EPI_GELU)
  int64_t ldz = 0;
  int epi = EPI_STORE;
  int beta = 0;              // EPI_ACC: add into C
  int dtype = ZB_DTYPE_BF16; // storage type of A, B, R, Z and (non-ACC) C
  int gelu = ZB_GELU_ERF;
  const char* tag = "gemm";  // pass name for kernel timing ("f", "b", "w")
  // Split-K arena (optional, not for EPI_ACC): room for the fp32 partial sums
  // of the splits.  GEMMs that share an arena must run in stream order.
  float* part = nullptr;
  size_t part_bytes = 0;
};

zb_status launch_gemm(const GemmDesc& g, hipStream_t s);
// Arena bytes launch_gemm would use to split the K of an M x N x K product of
// the F or B layout; 0 when it would not split.
size_t gemm_split_arena(int M, int N, int K);
// Independent weight-gradient GEMMs (bf16, W layout, fp32 accumulate) in as few launches as possible.
zb_status launch_gemm_w_group(const GemmDesc* gs, int n, hipStream_t s);

// Causal attention of one FULL layer (head dim 128).  lse2/dsum: fp32 [heads, T].
struct AttnArgs {
  const void* qkv = nullptr;  // [T, 3h] bf16
  void* o = nullptr;          // [T, h] bf16
  float* lse2 = nullptr;
  const void* dout = nullptr; // [T, h] bf16 (backward)
  float* dsum = nullptr;      // scratch (backward)
  void* dqkv = nullptr;       // [T, 3h] bf16 (backward output)
  int heads = 0, seq = 0, nseq = 0;
};
zb_status launch_attention_fwd(const AttnArgs& a, hipStream_t s);
zb_status launch_attention_bwd(const AttnArgs& a, hipStream_t s);

// Fill rows x cols elements (row stride ld, 2 or 4 bytes each) with zero.
zb_status launch_zero2d(void* p, int64_t rows, int64_t cols, int64_t ld, int elem_bytes, hipStream_t s);
// Sets *flag (device int) to 1 if any of n fp32 values is NaN/Inf (flag must be pre-zeroed).
zb_status launch_nonfinite(const float* p, int64_t n, int* flag, hipStream_t s);
zb_status launch_zero_int(int* flag, hipStream_t s);
// a[i] = gelu(z[i]) for n elements of dtype (bf16: n % 8 == 0, 16-byte aligned):
// the MLP activation rebuilt from the stored pre-activation.
zb_status launch_gelu(const void* z, void* a, int64_t n, int dtype, int kind, hipStream_t s);

// ------------------------------------------------ optimizer (section 4)
// Workgroups of the sum-of-squares pass per gradient tensor (one fp64 pair each).
constexpr int kSumsqBlocks = 1024;
// part[2i], part[2i+1] = sum of squares, count of NaN/Inf over workgroup i's
// share of g[0..n); *blocks_out = the number of pairs written.
zb_status launch_grad_sumsq(const float* g, int64_t n, double* part, int* blocks_out, hipStream_t s);
// Pairs launch_grad_sumsq writes for n values (its grid).
int grad_sumsq_blocks(int64_t n);
// out[0..1] = up[0..1] (may be null) + the sum of `count` pairs (flag as 0/1).
zb_status launch_state_combine(const double* part, int count, const double* up, double* out, hipStream_t s);
struct AdamwLaunch {
  float* theta = nullptr;
  float* m = nullptr;
  float* v = nullptr;
  const float* g = nullptr;
  void* w = nullptr;          // working copy of the parameters the GEMMs read
  int w_bf16 = 1;
  int64_t n = 0;
  zb_adamw hp{};
  double bc1 = 1.0, bc2 = 1.0;  // 1 - beta^step
  const double* used = nullptr;  // device state the step is (was) taken with
  const double* glob = nullptr;  // device global state (validation)
  int mode = 0;                  // 0 step, 1 validate, 2 rollback
  int* rolled = nullptr;         // validation: device int, 1 if rolled back
};
zb_status launch_adamw(const AdamwLaunch& L, hipStream_t s);

// --------------------------------------------------------- kernel timing
bool prof_on();
struct ProfScope {
  // Brackets one kernel launch with a hipEvent pair when timing is enabled.
  ProfScope(const char* name, double flops, double bytes, hipStream_t s);
  ~ProfScope();
  int slot = -1;
  hipStream_t stream;
};

}  // namespace zb
