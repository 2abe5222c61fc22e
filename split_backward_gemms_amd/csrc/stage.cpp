// Stage object, saved-tensor lifetime manager and schedule executor.
//
// A stage keeps, per live microbatch, three classes of tensors in slots of a
// caller-provided workspace (the pages' activation memory M_B / M_W, "Zero
// Bubble Pipeline Parallelism", section 3, "The Memory Model"):
//   FW  from F to W:  each layer's input and what its W passes read
//   FB  from F to B:  what only B reads (pre-activations, attention inputs, LSE)
//   BW  from B to W:  every linear's output gradient
// The F -> B -> W order per microbatch and the optimizer dependency at the
// step boundary follow section 3's dependency rules and the audit's "Draw the
// event graph before the Gantt".
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "zb_internal.h"

// ================================================================ errors
namespace zb {
namespace {
thread_local std::string g_err;
}

zb_status set_error(zb_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

void clear_error() { g_err.clear(); }

// ========================================================== kernel timing
namespace {
struct ProfEvent {
  std::string name;
  double flops, bytes;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof = false;
std::vector<ProfEvent> g_prof_ev;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t pool_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

bool prof_on() { return g_prof; }

ProfScope::ProfScope(const char* name, double flops, double bytes, hipStream_t s) : stream(s) {
  if (!g_prof) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  hipEvent_t a = pool_event(), b = pool_event();
  if (!a || !b) return;
  g_prof_ev.push_back(ProfEvent{name, flops, bytes, a, b});
  slot = (int)g_prof_ev.size() - 1;
  (void)hipEventRecord(a, s);
}

ProfScope::~ProfScope() {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  (void)hipEventRecord(g_prof_ev[slot].b, stream);
}

}  // namespace zb

using namespace zb;

extern "C" const char* zb_last_error(void) { return g_err.c_str(); }

// ============================================================ debug sync
namespace zb {
namespace {
bool env_debug_sync() {
  const char* v = getenv("ZB_DEBUG_SYNC");
  return v && *v && strcmp(v, "0") != 0;
}
bool g_debug_sync = env_debug_sync();

// In debug mode: wait for the stream and report any device error, naming the pass.
zb_status debug_check(hipStream_t s, const char* what, int stage, int mb) {
  if (!g_debug_sync) return ZB_OK;
  const hipError_t e1 = hipStreamSynchronize(s);
  const hipError_t e2 = hipGetLastError();
  const hipError_t e = e1 != hipSuccess ? e1 : e2;
  if (e != hipSuccess)
    return set_error(ZB_E_HIP, "debug sync after %s of stage %d mb %d: %s", what, stage, mb, hipGetErrorString(e));
  return ZB_OK;
}
}  // namespace
}  // namespace zb

extern "C" void zb_set_debug_sync(int on) { zb::g_debug_sync = on != 0; }
extern "C" int zb_get_debug_sync(void) { return zb::g_debug_sync ? 1 : 0; }

extern "C" const char* zb_version(void) { return "zb-stage gfx950 0.1"; }

extern "C" void zb_prof_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof = on != 0;
}

extern "C" void zb_prof_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& e : g_prof_ev) {
    (void)hipEventSynchronize(e.b);
    g_event_pool.push_back(e.a);
    g_event_pool.push_back(e.b);
  }
  g_prof_ev.clear();
}

extern "C" zb_status zb_prof_read(zb_prof_rec* out, int cap, int* n) {
  clear_error();
  if (!n || (cap > 0 && !out)) return set_error(ZB_E_ARG, "null output");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  std::map<std::string, zb_prof_rec> agg;
  for (auto& e : g_prof_ev) {
    ZB_HIP_CHECK(hipEventSynchronize(e.b));
    float ms = 0.f;
    ZB_HIP_CHECK(hipEventElapsedTime(&ms, e.a, e.b));
    zb_prof_rec& r = agg[e.name];
    if (r.launches == 0) {
      memset(&r, 0, sizeof r);
      snprintf(r.name, sizeof r.name, "%s", e.name.c_str());
    }
    r.launches += 1;
    r.total_ms += ms;
    r.flops += e.flops;
    r.bytes += e.bytes;
  }
  int i = 0;
  for (auto& kv : agg) {
    if (i < cap) out[i] = kv.second;
    ++i;
  }
  *n = i;
  return ZB_OK;
}

// ============================================================ stage object
namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Slots of one tensor class.  When stages run on different streams, a slot
// released on one stream and claimed from another is ordered by an event
// recorded at the release.
struct Pool {
  size_t bytes = 0;  // per slot
  int n = 0;
  char* base = nullptr;
  std::vector<int> free_list;
  std::vector<hipEvent_t> ev;          // per slot, created on first cross-stream use
  std::vector<hipStream_t> ev_stream;  // stream of the last recorded release (null: none)
  void reset(char* b, int count) {
    base = b;
    n = count;
    free_list.clear();
    for (int i = count - 1; i >= 0; --i) free_list.push_back(i);
    for (hipEvent_t e : ev)
      if (e) (void)hipEventDestroy(e);
    ev.assign(count, nullptr);
    ev_stream.assign(count, nullptr);
  }
  ~Pool() {
    for (hipEvent_t e : ev)
      if (e) (void)hipEventDestroy(e);
  }
  int acquire() {
    if (free_list.empty()) return -1;
    int s = free_list.back();
    free_list.pop_back();
    return s;
  }
  // Orders work on `s` after the slot's last release when that was on another stream.
  zb_status order_after_release(int slot, hipStream_t s) {
    if (slot < 0 || !ev_stream[slot] || ev_stream[slot] == s) return ZB_OK;
    ZB_HIP_CHECK(hipStreamWaitEvent(s, ev[slot], 0));
    return ZB_OK;
  }
  zb_status release(int slot, hipStream_t s, bool multi) {
    if (slot < 0) return ZB_OK;
    if (multi) {
      if (!ev[slot]) ZB_HIP_CHECK(hipEventCreateWithFlags(&ev[slot], hipEventDisableTiming));
      ZB_HIP_CHECK(hipEventRecord(ev[slot], s));
      ev_stream[slot] = s;
    } else {
      ev_stream[slot] = nullptr;
    }
    free_list.push_back(slot);
    return ZB_OK;
  }
  char* at(int s) const { return base + (size_t)s * bytes; }
};

struct LayerOff {
  // FW (a: the MLP activation, stashed unless it is rebuilt from z for W)
  size_t x = 0, qkv_fw = 0, o = 0, xup = 0, a = 0;
  // FB, or FW when A is rebuilt (z: the MLP pre-activation)
  size_t z = 0, qkv_fb = 0, lse = 0;
  // BW
  size_t dy = 0, dz = 0, dp = 0, dqkv = 0;
};

enum MbState { MB_IDLE = 0, MB_F = 1, MB_B = 2, MB_DONE = 3 };

int linears_per_layer(int kind) { return kind == ZB_KIND_TINY_MLP ? 2 : 4; }

}  // namespace

struct zb_stage {
  zb_stage_desc d{};
  int index = 0;
  int T = 0, h = 0, f = 0, L = 0, nlin = 0;
  size_t es = 2;
  std::vector<const void*> w;
  std::vector<float*> dw;
  std::vector<int64_t> wK, wN;  // per linear
  hipStream_t stream = nullptr;
  std::vector<LayerOff> off;
  size_t fw_bytes = 0, fb_bytes = 0, bw_bytes = 0, scratch_bytes = 0;
  size_t scratch_do = 0, scratch_flag = 0, scratch_dsum = 0;
  size_t scratch_act = 0, act_bytes = 0;  // A = gelu(Z) per layer: forward hand-off, W operand
  size_t scratch_part = 0, part_bytes = 0;  // split-K arena of the F/B GEMMs
  size_t scratch_opt = 0;                   // per-workgroup partial gradient states
  // plan
  bool planned = false;
  int plan_fw = 0, plan_fb = 0, plan_bw = 0;
  // workspace
  char* ws = nullptr;
  size_t ws_bytes = 0;
  char* scratch = nullptr;
  Pool fw, fb, bw;
  bool bound = false;
  // per microbatch
  std::vector<int> st, s_fw, s_fb, s_bw;
  int w_count = 0;
  bool grads_ready = false;  // a flushed step's dW, not yet overwritten by the next step's first W
  // optimizer state (zb_stage_optim_bind)
  bool opt_bound = false;
  zb_adamw opt{};
  std::vector<float*> opt_p, opt_m, opt_v;
  // stage-boundary taps (zb_stage_set_taps): per microbatch, or empty
  std::vector<void*> tap_y, tap_dx;
  // multi-stream schedules: stages on different streams
  bool multi = false;
  std::vector<hipEvent_t> f_done, b_done;  // per microbatch, created on first use
  ~zb_stage() {
    for (hipEvent_t e : f_done)
      if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : b_done)
      if (e) (void)hipEventDestroy(e);
  }
};

namespace {

enum { LIN_QKV = 0, LIN_PROJ = 1, LIN_UP = 2, LIN_DOWN = 3 };

int lin_index(const zb_stage* S, int layer, int which) {
  if (S->d.kind == ZB_KIND_TINY_MLP) return layer * 2 + (which == LIN_UP ? 0 : 1);
  return layer * 4 + which;
}

void compute_layout(zb_stage* S) {
  const size_t T = S->T, h = S->h, f = S->f, es = S->es;
  const size_t a = S->d.n_heads;
  size_t fw = 0, fb = 0, bw = 0;
  S->off.assign(S->L, LayerOff{});
  for (int l = 0; l < S->L; ++l) {
    LayerOff& o = S->off[l];
    o.x = fw; fw += align_up(T * h * es);
    if (S->d.kind == ZB_KIND_MLP_LINEARS) {
      o.qkv_fw = fw; fw += align_up(T * 3 * h * es);
      o.xup = fw; fw += align_up(T * h * es);
    } else if (S->d.kind == ZB_KIND_FULL) {
      o.o = fw; fw += align_up(T * h * es);
      o.xup = fw; fw += align_up(T * h * es);
    }
    if (S->d.recompute_act) {
      o.z = fw; fw += align_up(T * f * es);
    } else {
      o.a = fw; fw += align_up(T * f * es);
      o.z = fb; fb += align_up(T * f * es);
    }
    if (S->d.kind == ZB_KIND_FULL) {
      o.qkv_fb = fb; fb += align_up(T * 3 * h * es);
      o.lse = fb; fb += align_up(a * T * 4);
    }

    o.dy = bw; bw += align_up(T * h * es);
    o.dz = bw; bw += align_up(T * f * es);
    if (S->d.kind != ZB_KIND_TINY_MLP) {
      o.dp = bw; bw += align_up(T * h * es);
      o.dqkv = bw; bw += align_up(T * 3 * h * es);
    }
  }
  S->fw_bytes = fw;
  S->fb_bytes = fb;
  S->bw_bytes = bw;
  size_t sc = 0;
  S->scratch_flag = sc; sc += kAlign;
  S->scratch_do = sc;
  if (S->d.kind == ZB_KIND_FULL) sc += align_up(T * h * es);
  S->scratch_dsum = sc;
  if (S->d.kind == ZB_KIND_FULL) sc += align_up(a * T * 4);
  S->act_bytes = align_up(T * f * es);
  S->scratch_act = sc;
  if (S->d.recompute_act) sc += (size_t)S->L * S->act_bytes;
  // Split-K arena: the largest any F or B GEMM of the stage asks for (bf16 only).
  size_t part = 0;
  if (S->d.dtype == ZB_DTYPE_BF16) {
    for (int i = 0; i < S->nlin; ++i) {
      part = std::max(part, gemm_split_arena(S->T, (int)S->wN[i], (int)S->wK[i]));  // F
      part = std::max(part, gemm_split_arena(S->T, (int)S->wK[i], (int)S->wN[i]));  // B
    }
  }
  S->scratch_part = sc;
  S->part_bytes = part;
  sc += align_up(part);
  S->scratch_opt = sc;
  sc += align_up((size_t)S->L * S->nlin * kSumsqBlocks * 2 * sizeof(double));
  S->scratch_bytes = sc;
  S->fw.bytes = fw;
  S->fb.bytes = fb;
  S->bw.bytes = bw;
}

// Replays slot claims and releases of stage `idx` over a one-device order.
void plan_counts(int idx, int m, const zb_op* ops, int n, int& nfw, int& nfb, int& nbw) {
  if (!ops) {
    nfw = nfb = nbw = m;
    return;
  }
  std::vector<char> hfw(m, 0), hfb(m, 0), hbw(m, 0);
  int cfw = 0, cfb = 0, cbw = 0;
  nfw = nfb = nbw = 0;
  auto take = [&](std::vector<char>& held, int j, int& c, int& mx) {
    if (j < 0 || j >= m || held[j]) return;
    held[j] = 1;
    mx = std::max(mx, ++c);
  };
  auto drop = [&](std::vector<char>& held, int j, int& c) {
    if (j < 0 || j >= m || !held[j]) return;
    held[j] = 0;
    --c;
  };
  for (int i = 0; i < n; ++i) {
    const zb_op& o = ops[i];
    const int j = o.mb;
    if (o.stage == idx - 1 && o.kind == 'F') take(hfw, j, cfw, nfw);
    if (o.stage == idx + 1 && (o.kind == 'B' || o.kind == 'U')) take(hbw, j, cbw, nbw);
    if (o.stage != idx) continue;
    switch (o.kind) {
      case 'F':
        take(hfw, j, cfw, nfw);
        take(hfb, j, cfb, nfb);
        break;
      case 'B':
        take(hbw, j, cbw, nbw);
        drop(hfb, j, cfb);
        break;
      case 'W':
        drop(hfw, j, cfw);
        drop(hbw, j, cbw);
        break;
      case 'U':
        take(hbw, j, cbw, nbw);
        drop(hfb, j, cfb);
        drop(hfw, j, cfw);
        drop(hbw, j, cbw);
        break;
      default:
        break;
    }
  }
}

size_t ws_size(const zb_stage* S, int nfw, int nfb, int nbw) {
  return S->scratch_bytes + (size_t)nfw * S->fw_bytes + (size_t)nfb * S->fb_bytes + (size_t)nbw * S->bw_bytes;
}

// ------------------------------------------------------------- GEMM calls

// The stage's split-K arena: its passes run in stream order, so its GEMMs
// share one arena.
void set_arena(zb_stage* S, GemmDesc& g) {
  if (S->part_bytes == 0 || !S->scratch) return;
  g.part = reinterpret_cast<float*>(S->scratch + S->scratch_part);
  g.part_bytes = S->part_bytes;
}

zb_status gemm_f(zb_stage* S, const void* X, int64_t ldx, int lin, void* Y, int64_t ldy, int epi,
                 const void* R = nullptr, int64_t ldr = 0, void* Z = nullptr, int64_t ldz = 0) {
  GemmDesc g;
  g.M = S->T; g.N = (int)S->wN[lin]; g.K = (int)S->wK[lin];
  g.A = X; g.lda = ldx; g.a_kcontig = true;
  g.B = S->w[lin]; g.ldb = S->wN[lin]; g.b_kcontig = false;
  g.C = Y; g.ldc = ldy; g.R = R; g.ldr = ldr; g.Z = Z; g.ldz = ldz;
  g.epi = epi; g.dtype = S->d.dtype; g.gelu = S->d.gelu; g.tag = "f";
  set_arena(S, g);
  return launch_gemm(g, S->stream);
}

// dX[T, K_in] = dY[T, N_out] . W^T
zb_status gemm_b(zb_stage* S, const void* dY, int64_t lddy, int lin, void* dX, int64_t lddx, int epi,
                 const void* R = nullptr, int64_t ldr = 0) {
  GemmDesc g;
  g.M = S->T; g.N = (int)S->wK[lin]; g.K = (int)S->wN[lin];
  g.A = dY; g.lda = lddy; g.a_kcontig = true;
  g.B = S->w[lin]; g.ldb = S->wN[lin]; g.b_kcontig = true;
  g.C = dX; g.ldc = lddx; g.R = R; g.ldr = ldr;
  g.epi = epi; g.dtype = S->d.dtype; g.gelu = S->d.gelu; g.tag = "b";
  set_arena(S, g);
  return launch_gemm(g, S->stream);
}

// dW[K_in, N_out] (+)= X^T . dY
GemmDesc w_desc(const zb_stage* S, const void* X, int64_t ldx, const void* dY, int64_t lddy, int lin, int beta) {
  GemmDesc g;
  g.M = (int)S->wK[lin]; g.N = (int)S->wN[lin]; g.K = S->T;
  g.A = X; g.lda = ldx; g.a_kcontig = false;
  g.B = dY; g.ldb = lddy; g.b_kcontig = false;
  g.C = S->dw[lin]; g.ldc = S->wN[lin];
  g.epi = EPI_ACC; g.beta = beta; g.dtype = S->d.dtype; g.tag = "w";
  return g;
}

// The W pass's kernel for a list of weight gradients: bf16 goes through the
// grouped W launch, all of them at once or (per_linear) one launch each.
zb_status issue_w(zb_stage* S, const std::vector<GemmDesc>& gs, bool per_linear) {
  if (S->d.dtype != ZB_DTYPE_BF16) {
    for (const GemmDesc& g : gs) {
      zb_status st = launch_gemm(g, S->stream);
      if (st != ZB_OK) return st;
    }
    return ZB_OK;
  }
  if (!per_linear) return launch_gemm_w_group(gs.data(), (int)gs.size(), S->stream);
  for (const GemmDesc& g : gs) {
    zb_status st = launch_gemm_w_group(&g, 1, S->stream);
    if (st != ZB_OK) return st;
  }
  return ZB_OK;
}

// One linear's weight gradient inside the unsplit backward: the W pass's kernel.
zb_status gemm_w(zb_stage* S, const void* X, int64_t ldx, const void* dY, int64_t lddy, int lin, int beta) {
  return issue_w(S, {w_desc(S, X, ldx, dY, lddy, lin, beta)}, true);
}

#define ZB_TRY(expr)                   \
  do {                                 \
    zb_status s_ = (expr);             \
    if (s_ != ZB_OK) return s_;        \
  } while (0)

char* elem(char* base, size_t off, int64_t col, size_t es) { return base + off + (size_t)col * es; }

// ---------------------------------------------------------------- passes

// Where layer l's MLP activation A = gelu(Z) and pre-activation Z live for
// microbatch slots (fwb, fbb).  With recompute_act, A is not stashed: the
// forward writes it to stage scratch for the down projection, and W (or the
// unsplit backward) rebuilds it there from the stashed bf16 Z, which B needs
// anyway for GeLU'.  That keeps 8 T f bytes per layer out of every microbatch
// between F and B.
char* act(zb_stage* S, char* fwb, int l) {
  return S->d.recompute_act ? S->scratch + S->scratch_act + (size_t)l * S->act_bytes : fwb + S->off[l].a;
}
char* pre(zb_stage* S, char* fwb, char* fbb, int l) {
  return (S->d.recompute_act ? fwb : fbb) + S->off[l].z;
}
// A for W: rebuilt from Z when it was not stashed.
zb_status act_for_w(zb_stage* S, char* fwb, int l, char** A) {
  *A = act(S, fwb, l);
  if (!S->d.recompute_act) return ZB_OK;
  return launch_gelu(fwb + S->off[l].z, *A, (int64_t)S->T * S->f, S->d.dtype, S->d.gelu, S->stream);
}

zb_status run_forward(zb_stage* S, int mb, void* y) {
  char* fwb = S->fw.at(S->s_fw[mb]);
  char* fbb = S->fb.at(S->s_fb[mb]);
  const int64_t h = S->h, f = S->f;
  const size_t es = S->es;
  for (int l = 0; l < S->L; ++l) {
    const LayerOff& o = S->off[l];
    char* A = act(S, fwb, l);
    char* Z = pre(S, fwb, fbb, l);
    void* out = (l + 1 < S->L) ? (void*)(fwb + S->off[l + 1].x) : y;
    char* X = fwb + o.x;
    switch (S->d.kind) {
      case ZB_KIND_TINY_MLP:
        ZB_TRY(gemm_f(S, X, h, lin_index(S, l, LIN_UP), A, f, EPI_GELU, nullptr, 0, Z, f));
        ZB_TRY(gemm_f(S, A, f, lin_index(S, l, LIN_DOWN), out, h, EPI_STORE));
        break;
      case ZB_KIND_MLP_LINEARS: {
        char* qkv = fwb + o.qkv_fw;
        ZB_TRY(gemm_f(S, X, h, lin_index(S, l, LIN_QKV), qkv, 3 * h, EPI_STORE));
        // identity attention: proj reads the V columns of qkv in place
        ZB_TRY(gemm_f(S, elem(fwb, o.qkv_fw, 2 * h, es), 3 * h, lin_index(S, l, LIN_PROJ), fwb + o.xup, h,
                      EPI_STORE));
        ZB_TRY(gemm_f(S, fwb + o.xup, h, lin_index(S, l, LIN_UP), A, f, EPI_GELU, nullptr, 0, Z, f));
        ZB_TRY(gemm_f(S, A, f, lin_index(S, l, LIN_DOWN), out, h, EPI_STORE));
        break;
      }
      default: {  // FULL
        char* qkv = fbb + o.qkv_fb;
        ZB_TRY(gemm_f(S, X, h, lin_index(S, l, LIN_QKV), qkv, 3 * h, EPI_STORE));
        AttnArgs at;
        at.qkv = qkv; at.o = fwb + o.o; at.lse2 = reinterpret_cast<float*>(fbb + o.lse);
        at.heads = S->d.n_heads; at.seq = S->d.seq; at.nseq = S->d.micro_batch;
        ZB_TRY(launch_attention_fwd(at, S->stream));
        ZB_TRY(gemm_f(S, fwb + o.o, h, lin_index(S, l, LIN_PROJ), fwb + o.xup, h, EPI_RESID, X, h));
        ZB_TRY(gemm_f(S, fwb + o.xup, h, lin_index(S, l, LIN_UP), A, f, EPI_GELU, nullptr, 0, Z, f));
        ZB_TRY(gemm_f(S, A, f, lin_index(S, l, LIN_DOWN), out, h, EPI_RESID, fwb + o.xup, h));
        break;
      }
    }
  }
  return ZB_OK;
}

// Input-gradient pass; with `unsplit`, each linear's weight gradient follows its B GEMM.
zb_status run_backward(zb_stage* S, int mb, void* dx, bool unsplit, int beta) {
  char* fwb = S->fw.at(S->s_fw[mb]);
  char* fbb = S->fb.at(S->s_fb[mb]);
  char* bwb = S->bw.at(S->s_bw[mb]);
  const int64_t h = S->h, f = S->f;
  const size_t es = S->es;
  for (int l = S->L - 1; l >= 0; --l) {
    const LayerOff& o = S->off[l];
    void* out = (l > 0) ? (void*)(bwb + S->off[l - 1].dy) : dx;
    char* dY = bwb + o.dy;
    switch (S->d.kind) {
      case ZB_KIND_TINY_MLP: {
        const int up = lin_index(S, l, LIN_UP), down = lin_index(S, l, LIN_DOWN);
        ZB_TRY(gemm_b(S, dY, h, down, bwb + o.dz, f, EPI_DGELU, pre(S, fwb, fbb, l), f));
        if (unsplit) {
          char* A;
          ZB_TRY(act_for_w(S, fwb, l, &A));
          ZB_TRY(gemm_w(S, A, f, dY, h, down, beta));
        }
        ZB_TRY(gemm_b(S, bwb + o.dz, f, up, out, h, EPI_STORE));
        if (unsplit) ZB_TRY(gemm_w(S, fwb + o.x, h, bwb + o.dz, f, up, beta));
        break;
      }
      case ZB_KIND_MLP_LINEARS: {
        const int qkv = lin_index(S, l, LIN_QKV), proj = lin_index(S, l, LIN_PROJ);
        const int up = lin_index(S, l, LIN_UP), down = lin_index(S, l, LIN_DOWN);
        ZB_TRY(gemm_b(S, dY, h, down, bwb + o.dz, f, EPI_DGELU, pre(S, fwb, fbb, l), f));
        if (unsplit) {
          char* A;
          ZB_TRY(act_for_w(S, fwb, l, &A));
          ZB_TRY(gemm_w(S, A, f, dY, h, down, beta));
        }
        ZB_TRY(gemm_b(S, bwb + o.dz, f, up, bwb + o.dp, h, EPI_STORE));
        if (unsplit) ZB_TRY(gemm_w(S, fwb + o.xup, h, bwb + o.dz, f, up, beta));
        // identity attention backward: dV = dO; dQ = dK = 0 stay in the slot from
        // zb_stage_bind_workspace
        ZB_TRY(gemm_b(S, bwb + o.dp, h, proj, elem(bwb, o.dqkv, 2 * h, es), 3 * h, EPI_STORE));
        if (unsplit) ZB_TRY(gemm_w(S, elem(fwb, o.qkv_fw, 2 * h, es), 3 * h, bwb + o.dp, h, proj, beta));
        ZB_TRY(gemm_b(S, bwb + o.dqkv, 3 * h, qkv, out, h, EPI_STORE));
        if (unsplit) ZB_TRY(gemm_w(S, fwb + o.x, h, bwb + o.dqkv, 3 * h, qkv, beta));
        break;
      }
      default: {  // FULL
        const int qkv = lin_index(S, l, LIN_QKV), proj = lin_index(S, l, LIN_PROJ);
        const int up = lin_index(S, l, LIN_UP), down = lin_index(S, l, LIN_DOWN);
        char* dO = S->scratch + S->scratch_do;
        ZB_TRY(gemm_b(S, dY, h, down, bwb + o.dz, f, EPI_DGELU, pre(S, fwb, fbb, l), f));
        if (unsplit) {
          char* A;
          ZB_TRY(act_for_w(S, fwb, l, &A));
          ZB_TRY(gemm_w(S, A, f, dY, h, down, beta));
        }
        ZB_TRY(gemm_b(S, bwb + o.dz, f, up, bwb + o.dp, h, EPI_RESID, dY, h));
        if (unsplit) ZB_TRY(gemm_w(S, fwb + o.xup, h, bwb + o.dz, f, up, beta));
        ZB_TRY(gemm_b(S, bwb + o.dp, h, proj, dO, h, EPI_STORE));
        if (unsplit) ZB_TRY(gemm_w(S, fwb + o.o, h, bwb + o.dp, h, proj, beta));
        AttnArgs at;
        at.qkv = fbb + o.qkv_fb; at.o = fwb + o.o; at.lse2 = reinterpret_cast<float*>(fbb + o.lse);
        at.dout = dO; at.dsum = reinterpret_cast<float*>(S->scratch + S->scratch_dsum); at.dqkv = bwb + o.dqkv;
        at.heads = S->d.n_heads; at.seq = S->d.seq; at.nseq = S->d.micro_batch;
        ZB_TRY(launch_attention_bwd(at, S->stream));
        ZB_TRY(gemm_b(S, bwb + o.dqkv, 3 * h, qkv, out, h, EPI_RESID, bwb + o.dp, h));
        if (unsplit) ZB_TRY(gemm_w(S, fwb + o.x, h, bwb + o.dqkv, 3 * h, qkv, beta));
        break;
      }
    }
  }
  return ZB_OK;
}

// W pass: every linear's weight gradient.  They are independent of each other,
// so in bf16 they go out as one grouped launch.
zb_status run_weight(zb_stage* S, int mb, int beta) {
  char* fwb = S->fw.at(S->s_fw[mb]);
  char* bwb = S->bw.at(S->s_bw[mb]);
  const int64_t h = S->h, f = S->f;
  const size_t es = S->es;
  std::vector<GemmDesc> gs;
  for (int l = 0; l < S->L; ++l) {
    const LayerOff& o = S->off[l];
    char* A;
    ZB_TRY(act_for_w(S, fwb, l, &A));
    switch (S->d.kind) {
      case ZB_KIND_TINY_MLP:
        gs.push_back(w_desc(S, fwb + o.x, h, bwb + o.dz, f, lin_index(S, l, LIN_UP), beta));
        gs.push_back(w_desc(S, A, f, bwb + o.dy, h, lin_index(S, l, LIN_DOWN), beta));
        break;
      case ZB_KIND_MLP_LINEARS:
        gs.push_back(w_desc(S, fwb + o.x, h, bwb + o.dqkv, 3 * h, lin_index(S, l, LIN_QKV), beta));
        gs.push_back(w_desc(S, elem(fwb, o.qkv_fw, 2 * h, es), 3 * h, bwb + o.dp, h, lin_index(S, l, LIN_PROJ), beta));
        gs.push_back(w_desc(S, fwb + o.xup, h, bwb + o.dz, f, lin_index(S, l, LIN_UP), beta));
        gs.push_back(w_desc(S, A, f, bwb + o.dy, h, lin_index(S, l, LIN_DOWN), beta));
        break;
      default:  // FULL
        gs.push_back(w_desc(S, fwb + o.x, h, bwb + o.dqkv, 3 * h, lin_index(S, l, LIN_QKV), beta));
        gs.push_back(w_desc(S, fwb + o.o, h, bwb + o.dp, h, lin_index(S, l, LIN_PROJ), beta));
        gs.push_back(w_desc(S, fwb + o.xup, h, bwb + o.dz, f, lin_index(S, l, LIN_UP), beta));
        gs.push_back(w_desc(S, A, f, bwb + o.dy, h, lin_index(S, l, LIN_DOWN), beta));
        break;
    }
  }
  return issue_w(S, gs, S->d.w_per_linear != 0);
}

zb_status copy_in(zb_stage* S, void* dst, const void* src) {
  if (dst == src) return ZB_OK;
  const size_t bytes = (size_t)S->T * S->h * S->es;
  ZB_HIP_CHECK(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, S->stream));
  return ZB_OK;
}

// Stage-boundary tap: a copy of a [T, h] boundary tensor of mb, if tapped.
zb_status tap(zb_stage* S, const std::vector<void*>& taps, int mb, const void* src) {
  if (taps.empty() || !taps[mb]) return ZB_OK;
  return copy_in(S, taps[mb], src);
}

zb_status check_mb(const zb_stage* S, int mb) {
  if (!S) return set_error(ZB_E_ARG, "null stage");
  if (!S->bound) return set_error(ZB_E_STATE, "stage %d has no workspace bound", S->index);
  if (mb < 0 || mb >= S->d.n_micro) return set_error(ZB_E_INVALID_MB, "mb %d outside [0, %d)", mb, S->d.n_micro);
  return ZB_OK;
}

// Claims (if not yet held) the input slot of mb for work enqueued on `by`.
zb_status claim_fw(zb_stage* S, int mb, hipStream_t by) {
  if (S->s_fw[mb] >= 0) return ZB_OK;
  int s = S->fw.acquire();
  if (s < 0) return set_error(ZB_E_BUDGET, "stage %d: no free F->W slot for mb %d (workspace planned for %d)",
                              S->index, mb, S->fw.n);
  S->s_fw[mb] = s;
  return S->fw.order_after_release(s, by);
}

zb_status claim_bw(zb_stage* S, int mb, hipStream_t by) {
  if (S->s_bw[mb] >= 0) return ZB_OK;
  int s = S->bw.acquire();
  if (s < 0) return set_error(ZB_E_BUDGET, "stage %d: no free B->W slot for mb %d (workspace planned for %d)",
                              S->index, mb, S->bw.n);
  S->s_bw[mb] = s;
  return S->bw.order_after_release(s, by);
}

zb_status release_all(zb_stage* S, int mb) {
  ZB_TRY(S->fw.release(S->s_fw[mb], S->stream, S->multi));
  ZB_TRY(S->fb.release(S->s_fb[mb], S->stream, S->multi));
  ZB_TRY(S->bw.release(S->s_bw[mb], S->stream, S->multi));
  S->s_fw[mb] = S->s_fb[mb] = S->s_bw[mb] = -1;
  return ZB_OK;
}

zb_status do_forward(zb_stage* S, int mb, const void* x, void* y) {
  ZB_TRY(check_mb(S, mb));
  if (!x || !y) return set_error(ZB_E_ARG, "null x or y");
  if (S->st[mb] != MB_IDLE) return set_error(ZB_E_STATE, "stage %d mb %d already forwarded this step", S->index, mb);
  const bool had_fw = S->s_fw[mb] >= 0;
  if (!had_fw && S->fb.free_list.empty())
    return set_error(ZB_E_BUDGET, "stage %d: no free F->B slot for mb %d", S->index, mb);
  ZB_TRY(claim_fw(S, mb, S->stream));
  int sfb = S->fb.acquire();
  if (sfb < 0) return set_error(ZB_E_BUDGET, "stage %d: no free F->B slot for mb %d", S->index, mb);
  S->s_fb[mb] = sfb;
  ZB_TRY(S->fb.order_after_release(sfb, S->stream));
  ZB_TRY(copy_in(S, S->fw.at(S->s_fw[mb]) + S->off[0].x, x));
  ZB_TRY(run_forward(S, mb, y));
  ZB_TRY(tap(S, S->tap_y, mb, y));
  S->st[mb] = MB_F;
  return debug_check(S->stream, "F", S->index, mb);
}

zb_status do_backward(zb_stage* S, int mb, const void* dy, void* dx, bool unsplit) {
  ZB_TRY(check_mb(S, mb));
  if (!dy || !dx) return set_error(ZB_E_ARG, "null dy or dx");
  if (S->st[mb] != MB_F)
    return set_error(ZB_E_STATE, "stage %d mb %d: backward needs a finished forward and no earlier backward",
                     S->index, mb);
  ZB_TRY(claim_bw(S, mb, S->stream));
  const int beta = S->w_count > 0 ? 1 : 0;
  ZB_TRY(copy_in(S, S->bw.at(S->s_bw[mb]) + S->off[S->L - 1].dy, dy));
  ZB_TRY(run_backward(S, mb, dx, unsplit, beta));
  ZB_TRY(tap(S, S->tap_dx, mb, dx));
  ZB_TRY(S->fb.release(S->s_fb[mb], S->stream, S->multi));
  S->s_fb[mb] = -1;
  if (unsplit) {
    ZB_TRY(release_all(S, mb));
    S->st[mb] = MB_DONE;
    S->w_count += 1;
    S->grads_ready = false;
  } else {
    S->st[mb] = MB_B;
  }
  return debug_check(S->stream, unsplit ? "U" : "B", S->index, mb);
}

zb_status do_weight(zb_stage* S, int mb) {
  ZB_TRY(check_mb(S, mb));
  if (S->st[mb] != MB_B)
    return set_error(ZB_E_STATE, "stage %d mb %d: W needs its B first (and runs once)", S->index, mb);
  ZB_TRY(run_weight(S, mb, S->w_count > 0 ? 1 : 0));
  ZB_TRY(release_all(S, mb));
  S->st[mb] = MB_DONE;
  S->w_count += 1;
  S->grads_ready = false;
  return debug_check(S->stream, "W", S->index, mb);
}

}  // namespace

// ================================================================== ABI

extern "C" zb_status zb_stage_create(const zb_stage_desc* d, int stage_index, const void* const* weights,
                                     float* const* dw, void* stream, zb_stage** out) {
  clear_error();
  if (!d || !weights || !dw || !out) return set_error(ZB_E_ARG, "null argument");
  *out = nullptr;
  if (d->kind < ZB_KIND_TINY_MLP || d->kind > ZB_KIND_FULL) return set_error(ZB_E_ARG, "kind");
  if (d->dtype != ZB_DTYPE_BF16 && d->dtype != ZB_DTYPE_FP32) return set_error(ZB_E_ARG, "dtype");
  if (d->gelu != ZB_GELU_ERF && d->gelu != ZB_GELU_TANH) return set_error(ZB_E_ARG, "gelu");
  if (d->recompute_act != 0 && d->recompute_act != 1) return set_error(ZB_E_ARG, "recompute_act must be 0 or 1");
  if (d->w_per_linear != 0 && d->w_per_linear != 1) return set_error(ZB_E_ARG, "w_per_linear must be 0 or 1");
  if (d->n_layers < 1 || d->hidden < 1 || d->ffn < 1 || d->seq < 1 || d->micro_batch < 1 || d->n_micro < 1)
    return set_error(ZB_E_ARG, "sizes must be >= 1");
  if (stage_index < 0) return set_error(ZB_E_ARG, "stage_index must be >= 0");
  const int64_t T = (int64_t)d->seq * d->micro_batch;
  if (T > (1 << 30) || (int64_t)d->hidden * 3 > (1 << 30) || d->ffn > (1 << 30)) return set_error(ZB_E_ARG, "too large");
  if (d->hidden % 8 || d->ffn % 8 || T % 8)
    return set_error(ZB_E_UNSUPPORTED, "hidden, ffn and seq*micro_batch must be multiples of 8");
  if (d->kind == ZB_KIND_FULL) {
    if (d->n_heads < 1 || d->hidden % d->n_heads || d->hidden / d->n_heads != 128)
      return set_error(ZB_E_UNSUPPORTED, "FULL needs hidden / n_heads == 128");
    if (d->dtype != ZB_DTYPE_BF16) return set_error(ZB_E_UNSUPPORTED, "FULL is bf16 only");
  }
  zb_stage* S = new zb_stage();
  S->d = *d;
  S->index = stage_index;
  S->T = (int)T;
  S->h = d->hidden;
  S->f = d->ffn;
  S->L = d->n_layers;
  S->nlin = linears_per_layer(d->kind);
  S->es = d->dtype == ZB_DTYPE_BF16 ? 2 : 4;
  S->stream = static_cast<hipStream_t>(stream);
  const int nw = S->L * S->nlin;
  for (int i = 0; i < nw; ++i) {
    if (!weights[i] || !dw[i]) {
      delete S;
      return set_error(ZB_E_ARG, "null weight or gradient pointer %d", i);
    }
    if ((reinterpret_cast<uintptr_t>(weights[i]) & 15) || (reinterpret_cast<uintptr_t>(dw[i]) & 15)) {
      delete S;
      return set_error(ZB_E_ARG, "weight / gradient %d not 16-byte aligned", i);
    }
    S->w.push_back(weights[i]);
    S->dw.push_back(dw[i]);
    const int which = S->d.kind == ZB_KIND_TINY_MLP ? (i % 2 == 0 ? LIN_UP : LIN_DOWN) : i % 4;
    int64_t K = 0, N = 0;
    switch (which) {
      case LIN_QKV: K = S->h; N = 3LL * S->h; break;
      case LIN_PROJ: K = S->h; N = S->h; break;
      case LIN_UP: K = S->h; N = S->f; break;
      default: K = S->f; N = S->h; break;
    }
    S->wK.push_back(K);
    S->wN.push_back(N);
  }
  compute_layout(S);
  const int m = d->n_micro;
  S->st.assign(m, MB_IDLE);
  S->s_fw.assign(m, -1);
  S->s_fb.assign(m, -1);
  S->s_bw.assign(m, -1);
  *out = S;
  return ZB_OK;
}

extern "C" zb_status zb_stage_class_bytes(const zb_stage* S, size_t* fw, size_t* fb, size_t* bw) {
  clear_error();
  if (!S || !fw || !fb || !bw) return set_error(ZB_E_ARG, "null argument");
  *fw = S->fw_bytes;
  *fb = S->fb_bytes;
  *bw = S->bw_bytes;
  return ZB_OK;
}

extern "C" zb_status zb_stage_workspace_bytes(zb_stage* S, const zb_op* ops, int n_ops, size_t* bytes) {
  clear_error();
  if (!S || !bytes || n_ops < 0 || (n_ops > 0 && !ops)) return set_error(ZB_E_ARG, "bad arguments");
  int a, b, c;
  plan_counts(S->index, S->d.n_micro, ops, n_ops, a, b, c);
  S->plan_fw = a;
  S->plan_fb = b;
  S->plan_bw = c;
  S->planned = true;
  *bytes = ws_size(S, a, b, c);
  return ZB_OK;
}

extern "C" zb_status zb_stage_bind_workspace(zb_stage* S, void* p, size_t bytes) {
  clear_error();
  if (!S || !p) return set_error(ZB_E_ARG, "null argument");
  if (reinterpret_cast<uintptr_t>(p) % kAlign) return set_error(ZB_E_ARG, "workspace must be 256-byte aligned");
  for (int j = 0; j < S->d.n_micro; ++j)
    if (S->st[j] != MB_IDLE && S->st[j] != MB_DONE)
      return set_error(ZB_E_STATE, "stage %d: microbatch %d is live", S->index, j);
  if (!S->planned) {
    S->plan_fw = S->plan_fb = S->plan_bw = S->d.n_micro;
    S->planned = true;
  }
  const size_t need = ws_size(S, S->plan_fw, S->plan_fb, S->plan_bw);
  if (bytes < need) return set_error(ZB_E_BUDGET, "workspace %zu bytes < planned %zu", bytes, need);
  char* base = static_cast<char*>(p);
  char* const q_fw = base + S->scratch_bytes;
  char* const q_fb = q_fw + (size_t)S->plan_fw * S->fw_bytes;
  char* const q_bw = q_fb + (size_t)S->plan_fb * S->fb_bytes;
  // Identity attention (MLP linears): the dQ and dK columns of every layer's
  // dQKV in every B slot are zero for good and nothing else writes them, so
  // they are cleared once here instead of in every backward.  Enqueued before
  // the stage takes the buffer, so a failed launch leaves the old binding.
  if (S->d.kind == ZB_KIND_MLP_LINEARS)
    for (int s = 0; s < S->plan_bw; ++s)
      for (int l = 0; l < S->L; ++l)
        ZB_TRY(launch_zero2d(q_bw + (size_t)s * S->bw_bytes + S->off[l].dqkv, S->T, 2 * S->h, 3 * S->h,
                             (int)S->es, S->stream));
  S->ws = base;
  S->ws_bytes = bytes;
  S->scratch = base;
  S->fw.reset(q_fw, S->plan_fw);
  S->fb.reset(q_fb, S->plan_fb);
  S->bw.reset(q_bw, S->plan_bw);
  std::fill(S->s_fw.begin(), S->s_fw.end(), -1);
  std::fill(S->s_fb.begin(), S->s_fb.end(), -1);
  std::fill(S->s_bw.begin(), S->s_bw.end(), -1);
  S->bound = true;
  return ZB_OK;
}

extern "C" zb_status zb_stage_input_slot(zb_stage* S, int mb, void** p) {
  clear_error();
  if (!p) return set_error(ZB_E_ARG, "null output");
  ZB_TRY(check_mb(S, mb));
  if (S->st[mb] != MB_IDLE) return set_error(ZB_E_STATE, "stage %d mb %d already forwarded", S->index, mb);
  ZB_TRY(claim_fw(S, mb, S->stream));
  *p = S->fw.at(S->s_fw[mb]) + S->off[0].x;
  return ZB_OK;
}

extern "C" zb_status zb_stage_grad_slot(zb_stage* S, int mb, void** p) {
  clear_error();
  if (!p) return set_error(ZB_E_ARG, "null output");
  ZB_TRY(check_mb(S, mb));
  if (S->st[mb] != MB_IDLE && S->st[mb] != MB_F)
    return set_error(ZB_E_STATE, "stage %d mb %d already past its B", S->index, mb);
  ZB_TRY(claim_bw(S, mb, S->stream));
  *p = S->bw.at(S->s_bw[mb]) + S->off[S->L - 1].dy;
  return ZB_OK;
}

extern "C" zb_status zb_stage_set_taps(zb_stage* S, void* const* y_tap, void* const* dx_tap) {
  clear_error();
  if (!S) return set_error(ZB_E_ARG, "null stage");
  const int m = S->d.n_micro;
  for (int j = 0; j < m; ++j)
    if ((y_tap && !y_tap[j]) || (dx_tap && !dx_tap[j])) return set_error(ZB_E_ARG, "null tap for mb %d", j);
  S->tap_y.clear();
  S->tap_dx.clear();
  if (y_tap) S->tap_y.assign(y_tap, y_tap + m);
  if (dx_tap) S->tap_dx.assign(dx_tap, dx_tap + m);
  return ZB_OK;
}

extern "C" zb_status zb_forward(zb_stage* S, int mb, const void* x, void* y) {
  clear_error();
  return do_forward(S, mb, x, y);
}

extern "C" zb_status zb_backward_input(zb_stage* S, int mb, const void* dy, void* dx) {
  clear_error();
  return do_backward(S, mb, dy, dx, false);
}

extern "C" zb_status zb_backward_unsplit(zb_stage* S, int mb, const void* dy, void* dx) {
  clear_error();
  return do_backward(S, mb, dy, dx, true);
}

extern "C" zb_status zb_backward_weight(zb_stage* S, int mb) {
  clear_error();
  return do_weight(S, mb);
}

extern "C" zb_status zb_grad_flush(zb_stage* S, int* nonfinite_out) {
  clear_error();
  if (!S) return set_error(ZB_E_ARG, "null stage");
  for (int j = 0; j < S->d.n_micro; ++j)
    if (S->st[j] != MB_DONE)
      return set_error(ZB_E_MISSING, "stage %d: microbatch %d has no W yet; the optimizer step needs all of them",
                       S->index, j);
  if (nonfinite_out) {
    if (!S->bound) return set_error(ZB_E_STATE, "no workspace");
    int* flag = reinterpret_cast<int*>(S->scratch + S->scratch_flag);
    ZB_TRY(launch_zero_int(flag, S->stream));
    for (size_t i = 0; i < S->dw.size(); ++i)
      ZB_TRY(launch_nonfinite(S->dw[i], S->wK[i] * S->wN[i], flag, S->stream));
    int host = 0;
    ZB_HIP_CHECK(hipMemcpyAsync(&host, flag, sizeof(int), hipMemcpyDeviceToHost, S->stream));
    ZB_HIP_CHECK(hipStreamSynchronize(S->stream));
    *nonfinite_out = host;
  }
  std::fill(S->st.begin(), S->st.end(), (int)MB_IDLE);
  S->w_count = 0;
  S->grads_ready = true;
  return ZB_OK;
}

// ------------------------------------------------------------ optimizer

extern "C" zb_status zb_stage_optim_bind(zb_stage* S, const zb_adamw* hp, float* const* master,
                                         float* const* exp_avg, float* const* exp_avg_sq,
                                         void* const* weights_rw) {
  clear_error();
  if (!S || !hp || !master || !exp_avg || !exp_avg_sq || !weights_rw) return set_error(ZB_E_ARG, "null argument");
  if (!(hp->lr >= 0.0f) || !(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) || !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f) ||
      !(hp->eps >= 0.0f) || !(hp->weight_decay >= 0.0f) || !(hp->lr * hp->weight_decay < 1.0f))
    return set_error(ZB_E_ARG, "AdamW hyperparameters outside lr >= 0, 0 <= beta < 1, eps >= 0, 0 <= lr*wd < 1");
  if (hp->beta1 == 0.0f || hp->beta2 == 0.0f)
    return set_error(ZB_E_ARG, "beta1 and beta2 must be > 0 for the step to be invertible");
  const int nw = (int)S->w.size();
  for (int i = 0; i < nw; ++i) {
    const void* bufs[4] = {master[i], exp_avg[i], exp_avg_sq[i], weights_rw[i]};
    for (const void* b : bufs)
      if (!b || (reinterpret_cast<uintptr_t>(b) & 15))
        return set_error(ZB_E_ARG, "linear %d: optimizer buffers must be non-null and 16-byte aligned", i);
    if (weights_rw[i] != S->w[i])
      return set_error(ZB_E_ARG, "linear %d: weights_rw must be the stage's own weight buffer", i);
  }
  S->opt = *hp;
  S->opt_p.assign(master, master + nw);
  S->opt_m.assign(exp_avg, exp_avg + nw);
  S->opt_v.assign(exp_avg_sq, exp_avg_sq + nw);
  S->opt_bound = true;
  return ZB_OK;
}

namespace {
zb_status optim_ready(const zb_stage* S, bool need_opt) {
  if (!S) return set_error(ZB_E_ARG, "null stage");
  if (!S->bound) return set_error(ZB_E_STATE, "stage %d: no workspace", S->index);
  if (need_opt && !S->opt_bound) return set_error(ZB_E_STATE, "stage %d: no optimizer state bound", S->index);
  if (!S->grads_ready)
    return set_error(ZB_E_STATE, "stage %d: no flushed step gradients (flush first; a W of the next step "
                     "overwrites them)", S->index);
  return ZB_OK;
}

zb_status optim_launch(zb_stage* S, int mode, int step, const double* used, const double* glob, int* rolled) {
  if (step < 1) return set_error(ZB_E_ARG, "step must be >= 1");
  if (!used || (mode == 1 && !glob)) return set_error(ZB_E_ARG, "null state");
  ZB_TRY(optim_ready(S, true));
  for (size_t i = 0; i < S->w.size(); ++i) {
    AdamwLaunch L;
    L.theta = S->opt_p[i];
    L.m = S->opt_m[i];
    L.v = S->opt_v[i];
    L.g = S->dw[i];
    L.w = const_cast<void*>(S->w[i]);
    L.w_bf16 = S->d.dtype == ZB_DTYPE_BF16;
    L.n = S->wK[i] * S->wN[i];
    L.hp = S->opt;
    L.bc1 = 1.0 - std::pow((double)S->opt.beta1, step);
    L.bc2 = 1.0 - std::pow((double)S->opt.beta2, step);
    L.used = used;
    L.glob = glob;
    L.mode = mode;
    L.rolled = rolled;
    ZB_TRY(launch_adamw(L, S->stream));
  }
  return ZB_OK;
}
}  // namespace

extern "C" zb_status zb_stage_grad_state(zb_stage* S, const double* upstream, double* partial_out) {
  clear_error();
  if (!partial_out) return set_error(ZB_E_ARG, "null partial_out");
  ZB_TRY(optim_ready(S, false));
  double* part = reinterpret_cast<double*>(S->scratch + S->scratch_opt);
  int count = 0;
  for (size_t i = 0; i < S->w.size(); ++i) {
    int blocks = 0;
    ZB_TRY(launch_grad_sumsq(S->dw[i], S->wK[i] * S->wN[i], part + 2 * count, &blocks, S->stream));
    count += blocks;
  }
  return launch_state_combine(part, count, upstream, partial_out, S->stream);
}

// ------------------------------------ gradient state without allocating

namespace {
// Per-workgroup partial gradient states of zb_stage_grad_state_noalloc: the
// library's own device array instead of the stage workspace, so the call
// allocates nothing.  Every GPU the library runs on holds its own copy, at its
// own address, until the process ends.  In host code `scratch` only names the
// symbol: its device address comes from hipGetSymbolAddress, once per device.
constexpr int kNoAllocPairs = 65536;  // (sum of squares, non-finite count) pairs: 1 MiB
static __device__ __align__(256) double scratch[2 * kNoAllocPairs];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
double* g_scratch_ptr[kMaxDevices] = {};

// Address of the current device's copy of `scratch`, looked up on first use.
zb_status noalloc_scratch(double** out) {
  int dev = -1;
  ZB_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return set_error(ZB_E_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    ZB_HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return set_error(ZB_E_HIP, "hipGetSymbolAddress gave a null address");
    g_scratch_ptr[dev] = static_cast<double*>(p);
  }
  *out = g_scratch_ptr[dev];
  return ZB_OK;
}
}  // namespace

extern "C" zb_status zb_stage_grad_state_noalloc(zb_stage* S, const double* upstream, double* partial_out) {
  clear_error();
  if (!S) return set_error(ZB_E_ARG, "null stage");
  if (!partial_out) return set_error(ZB_E_ARG, "null partial_out");
  int64_t pairs = 0;
  for (size_t i = 0; i < S->w.size(); ++i) pairs += grad_sumsq_blocks(S->wK[i] * S->wN[i]);
  if (pairs > kNoAllocPairs)
    return set_error(ZB_E_UNSUPPORTED, "stage %d: %lld partial states exceed the %d of the library's scratch",
                     S->index, (long long)pairs, kNoAllocPairs);
  if (!S->grads_ready)
    return set_error(ZB_E_STATE, "stage %d: no flushed step gradients (flush first; a W of the next step "
                     "overwrites them)", S->index);
  double* part = nullptr;
  ZB_TRY(noalloc_scratch(&part));
  int count = 0;
  for (size_t i = 0; i < S->w.size(); ++i) {
    int blocks = 0;
    ZB_TRY(launch_grad_sumsq(S->dw[i], S->wK[i] * S->wN[i], part + 2 * count, &blocks, S->stream));
    count += blocks;
  }
  return launch_state_combine(part, count, upstream, partial_out, S->stream);
}

extern "C" zb_status zb_stage_optim_step(zb_stage* S, int step, const double* used) {
  clear_error();
  return optim_launch(S, 0, step, used, nullptr, nullptr);
}

extern "C" zb_status zb_stage_optim_validate(zb_stage* S, int step, const double* used, const double* global,
                                             int* rolled_back) {
  clear_error();
  return optim_launch(S, 1, step, used, global, rolled_back);
}

extern "C" zb_status zb_stage_optim_rollback(zb_stage* S, int step, const double* used) {
  clear_error();
  return optim_launch(S, 2, step, used, nullptr, nullptr);
}

namespace {
zb_status ensure_done_events(zb_stage* S) {
  const int m = S->d.n_micro;
  if ((int)S->f_done.size() == m) return ZB_OK;
  S->f_done.assign(m, nullptr);
  S->b_done.assign(m, nullptr);
  for (int j = 0; j < m; ++j) {
    ZB_HIP_CHECK(hipEventCreateWithFlags(&S->f_done[j], hipEventDisableTiming));
    ZB_HIP_CHECK(hipEventCreateWithFlags(&S->b_done[j], hipEventDisableTiming));
  }
  return ZB_OK;
}
}  // namespace

extern "C" zb_status zb_run_schedule(zb_stage* const* stages, int P, const zb_op* ops, int n_ops,
                                     const void* const* x0, const void* const* dy_last, void* const* y_last,
                                     void* const* dx0, zb_trace_rec* trace) {
  clear_error();
  if (!stages || P < 1 || !ops || n_ops < 1 || !x0 || !dy_last || !y_last || !dx0)
    return set_error(ZB_E_ARG, "null argument");
  bool multi = false;
  for (int p = 0; p < P; ++p) {
    const zb_stage* S = stages[p];
    if (!S) return set_error(ZB_E_ARG, "stages[%d] is null", p);
    if (S->index != p) return set_error(ZB_E_ARG, "stages[%d] was created as stage %d", p, S->index);
    if (S->stream != stages[0]->stream) multi = true;
    if (S->d.n_micro != stages[0]->d.n_micro || S->T != stages[0]->T || S->h != stages[0]->h ||
        S->d.dtype != stages[0]->d.dtype)
      return set_error(ZB_E_ARG, "stage %d: microbatch count, tokens, hidden or dtype differ", p);
    if (!S->bound) return set_error(ZB_E_STATE, "stage %d has no workspace bound", p);
    for (int j = 0; j < S->d.n_micro; ++j)
      if (S->st[j] != MB_IDLE || S->s_fw[j] >= 0 || S->s_bw[j] >= 0)
        return set_error(ZB_E_STATE, "stage %d mb %d is live (flush the previous step first)", p, j);
  }
  const int m = stages[0]->d.n_micro;
  for (int j = 0; j < m; ++j)
    if (!x0[j] || !dy_last[j] || !y_last[j] || !dx0[j]) return set_error(ZB_E_ARG, "null buffer for mb %d", j);
  int bad = -1;
  ZB_TRY(schedule_validate(P, m, ops, n_ops, &bad));
  for (int p = 0; p < P; ++p) {
    int a, b, c;
    plan_counts(p, m, ops, n_ops, a, b, c);
    const zb_stage* S = stages[p];
    if (a > S->fw.n || b > S->fb.n || c > S->bw.n)
      return set_error(ZB_E_BUDGET, "stage %d: order needs %d/%d/%d slots (F->W, F->B, B->W), workspace has %d/%d/%d",
                       p, a, b, c, S->fw.n, S->fb.n, S->bw.n);
  }
  if (multi)
    for (int p = 0; p < P; ++p) ZB_TRY(ensure_done_events(stages[p]));
  for (int p = 0; p < P; ++p) stages[p]->multi = multi;
  std::vector<hipEvent_t> ev;
  if (trace) {
    ev.resize(2 * (size_t)n_ops, nullptr);
    for (auto& e : ev) ZB_HIP_CHECK(hipEventCreate(&e));
  }
  // With one stream per stage, stage s+1's forward waits for stage s's forward
  // of the same microbatch and stage s's backward for stage s+1's backward;
  // everything else is ordered by the stage's own stream.
  zb_status rc = ZB_OK;
  for (int i = 0; i < n_ops && rc == ZB_OK; ++i) {
    const zb_op& o = ops[i];
    zb_stage* S = stages[o.stage];
    hipStream_t st = S->stream;
    const int j = o.mb;
    // The cross-stage hand-off first, so a traced pass's start is when its
    // stream could begin it (its time then excludes the wait for a producer).
    if (multi) {
      hipEvent_t dep = nullptr;
      if (o.kind == 'F' && o.stage > 0) dep = stages[o.stage - 1]->f_done[j];
      if ((o.kind == 'B' || o.kind == 'U') && o.stage + 1 < P) dep = stages[o.stage + 1]->b_done[j];
      if (dep && hipStreamWaitEvent(st, dep, 0) != hipSuccess) {
        rc = set_error(ZB_E_HIP, "hipStreamWaitEvent failed");
        break;
      }
    }
    if (trace) (void)hipEventRecord(ev[2 * i], st);
    switch (o.kind) {
      case 'F': {
        void* y = y_last[j];
        if (o.stage + 1 < P) {
          zb_stage* N = stages[o.stage + 1];
          if (N->st[j] != MB_IDLE) {
            rc = set_error(ZB_E_STATE, "stage %d mb %d already forwarded", N->index, j);
            break;
          }
          rc = claim_fw(N, j, st);
          if (rc != ZB_OK) break;
          y = N->fw.at(N->s_fw[j]) + N->off[0].x;
        }
        const void* x = x0[j];
        if (o.stage > 0) x = S->fw.at(S->s_fw[j]) + S->off[0].x;
        rc = do_forward(S, j, x, y);
        if (rc == ZB_OK && multi && hipEventRecord(S->f_done[j], st) != hipSuccess)
          rc = set_error(ZB_E_HIP, "hipEventRecord failed");
        break;
      }
      case 'B':
      case 'U': {
        void* dx = dx0[j];
        if (o.stage > 0) {
          zb_stage* U = stages[o.stage - 1];
          rc = claim_bw(U, j, st);
          if (rc != ZB_OK) break;
          dx = U->bw.at(U->s_bw[j]) + U->off[U->L - 1].dy;
        }
        const void* dy = dy_last[j];
        if (o.stage + 1 < P) dy = S->bw.at(S->s_bw[j]) + S->off[S->L - 1].dy;
        rc = do_backward(S, j, dy, dx, o.kind == 'U');
        if (rc == ZB_OK && multi && hipEventRecord(S->b_done[j], st) != hipSuccess)
          rc = set_error(ZB_E_HIP, "hipEventRecord failed");
        break;
      }
      case 'W':
        rc = do_weight(S, j);
        break;
      default:
        rc = set_error(ZB_E_ARG, "op %d kind", i);
    }
    if (trace) (void)hipEventRecord(ev[2 * i + 1], st);
  }
  if (rc != ZB_OK) {
    for (auto& e : ev) (void)hipEventDestroy(e);
    return rc;
  }
  if (trace) {
    for (auto& e : ev) ZB_HIP_CHECK(hipEventSynchronize(e));
    for (int i = 0; i < n_ops; ++i) {
      trace[i].op = ops[i];
      float ms = 0.f, t0 = 0.f;
      (void)hipEventElapsedTime(&ms, ev[2 * i], ev[2 * i + 1]);
      (void)hipEventElapsedTime(&t0, ev[0], ev[2 * i]);
      trace[i].ms = ms;
      trace[i].t0_ms = t0;
    }
    for (auto& e : ev) (void)hipEventDestroy(e);
  }
  return ZB_OK;
}

extern "C" void zb_stage_destroy(zb_stage* S) { delete S; }

// ========================================================== single linears

namespace {
zb_status linear_args(int dtype, int T, int K, int N, const void* a, const void* b, const void* c) {
  if (dtype != ZB_DTYPE_BF16 && dtype != ZB_DTYPE_FP32) return set_error(ZB_E_ARG, "dtype");
  if (T < 0 || K < 0 || N < 0) return set_error(ZB_E_ARG, "negative size");
  if ((T > 0 && K > 0 && N > 0) && (!a || !b || !c)) return set_error(ZB_E_ARG, "null pointer");
  return ZB_OK;
}
}  // namespace

extern "C" zb_status zb_linear_forward(int dtype, int T, int K, int N, const void* x, const void* w, void* y,
                                       void* stream) {
  clear_error();
  ZB_TRY(linear_args(dtype, T, K, N, x, w, y));
  GemmDesc g;
  g.M = T; g.N = N; g.K = K;
  g.A = x; g.lda = K; g.a_kcontig = true;
  g.B = w; g.ldb = N; g.b_kcontig = false;
  g.C = y; g.ldc = N; g.epi = EPI_STORE; g.dtype = dtype; g.tag = "f";
  return launch_gemm(g, static_cast<hipStream_t>(stream));
}

extern "C" zb_status zb_linear_backward_input(int dtype, int T, int K, int N, const void* dy, const void* w,
                                              void* dx, void* stream) {
  clear_error();
  ZB_TRY(linear_args(dtype, T, K, N, dy, w, dx));
  GemmDesc g;
  g.M = T; g.N = K; g.K = N;
  g.A = dy; g.lda = N; g.a_kcontig = true;
  g.B = w; g.ldb = N; g.b_kcontig = true;
  g.C = dx; g.ldc = K; g.epi = EPI_STORE; g.dtype = dtype; g.tag = "b";
  return launch_gemm(g, static_cast<hipStream_t>(stream));
}

extern "C" zb_status zb_linear_backward_weight(int dtype, int T, int K, int N, const void* x, const void* dy,
                                               float* dw, int accumulate, void* stream) {
  clear_error();
  ZB_TRY(linear_args(dtype, T, K, N, x, dy, dw));
  GemmDesc g;
  g.M = K; g.N = N; g.K = T;
  g.A = x; g.lda = K; g.a_kcontig = false;
  g.B = dy; g.ldb = N; g.b_kcontig = false;
  g.C = dw; g.ldc = N; g.epi = EPI_ACC; g.beta = accumulate ? 1 : 0; g.dtype = dtype; g.tag = "w";
  return launch_gemm(g, static_cast<hipStream_t>(stream));
}
