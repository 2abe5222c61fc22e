/*
 * zb.h -- C ABI of one zero-bubble pipeline stage on an MI355X (gfx950).
 *
 * One pipeline stage holds n_layers layers.  Its three passes follow the split
 * of the backward pass in "Zero Bubble Pipeline Parallelism" (structured summary
 * of arXiv 2401.10241), section 3, "The Backward Pass Decomposition: B and W",
 * and the tutorial "Pipeline Schedules: GPipe, 1F1B and Zero Bubble", section
 * "Zero bubble: split the backward pass":
 *
 *   F  forward:          Y  = X . W        per linear (+ GeLU, attention, residual)
 *   B  input gradient:   dX = dY . W^T     per linear, layers in reverse
 *   W  weight gradient:  dW += X^T . dY    per linear, fp32, summed over microbatches
 *
 * B of stage s for microbatch j needs F(s,j) and B(s+1,j); W(s,j) needs only
 * B(s,j); the optimizer step needs every W of the step ("Zero-Bubble Pipeline
 * Parallelism, Proven", section "Draw the event graph before the Gantt").
 *
 * Conventions
 *  - Every tensor is row-major.  Activations are [T, width] with T = seq *
 *    micro_batch tokens; weight W of a linear K -> N is [K, N] (Y = X . W).
 *    Its gradient buffer dW is fp32 [K, N].
 *  - bf16 mode stores weights and activations as bfloat16 and accumulates in
 *    fp32; fp32 mode stores fp32.  Weight gradients are always fp32.
 *  - Linears of one layer, in order: TINY_MLP {up, down}; MLP_LINEARS and
 *    FULL {qkv, proj, up, down} with qkv: h -> 3h (Q | K | V column blocks,
 *    head-major inside each), proj: h -> h, up: h -> ffn, down: ffn -> h.
 *  - Device pointers are plain device addresses (hipMalloc'd or torch
 *    tensors); host pointers are marked "host".  The caller owns every
 *    buffer it passes: weights, gradient buffers, inputs, outputs and the
 *    workspace.  The library never allocates device memory.
 *  - Work is enqueued asynchronously on the stream given at creation, in call
 *    order.  Inputs must stay valid until the work that reads them has run on
 *    that stream.
 *  - On any error the call changes no state and enqueues no work; the text of
 *    the last error of the calling thread is returned by zb_last_error().
 *    Device faults surface as ZB_E_HIP at the next call that synchronises.
 *  - Shapes: hidden, ffn and seq*micro_batch must be multiples of 8 (seq itself
 *    may be any length from 1); FULL needs hidden / n_heads == 128.
 */
#ifndef ZB_H
#define ZB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ZB_OK = 0,
  ZB_E_ARG = 1,            /* bad argument (null pointer, bad size, bad kind)      */
  ZB_E_STATE = 2,          /* pass called out of F -> B -> W order for (stage, mb) */
  ZB_E_DUPLICATE = 3,      /* a pass repeated in a schedule / duplicate event id   */
  ZB_E_INVALID_STAGE = 4,  /* stage index outside [0, P)                           */
  ZB_E_INVALID_MB = 5,     /* microbatch index outside [0, m)                      */
  ZB_E_MISSING = 6,        /* flush before every W ran / pass or dependency absent */
  ZB_E_DEPENDENCY = 7,     /* a pass placed before one it depends on               */
  ZB_E_BUDGET = 8,         /* workspace too small for the planned live tensors     */
  ZB_E_HIP = 9,            /* HIP runtime error                                    */
  ZB_E_UNSUPPORTED = 10,   /* shape or mode this build does not implement          */
  ZB_E_DEADLOCK = 11,      /* per-stage orders that can never all complete        */
  ZB_E_INTERVAL = 12,      /* timed event with end <= start or start < 0           */
  ZB_E_OVERLAP = 13        /* two timed events of one stage overlap                */
} zb_status;

enum { ZB_KIND_TINY_MLP = 0, ZB_KIND_MLP_LINEARS = 1, ZB_KIND_FULL = 2 };
enum { ZB_DTYPE_BF16 = 0, ZB_DTYPE_FP32 = 1 };
enum { ZB_GELU_ERF = 0, ZB_GELU_TANH = 1 };
enum { ZB_ORDER_GPIPE = 0, ZB_ORDER_1F1B = 1, ZB_ORDER_ZBH1 = 2, ZB_ORDER_ZBH2 = 3,
       ZB_ORDER_WLAST = 4 };

/* Shape of one stage.  MLP_LINEARS routes the V columns of qkv straight to
 * proj (attention replaced by the identity); FULL uses causal softmax attention
 * and residual adds around the attention and MLP blocks. */
typedef struct {
  int kind;         /* ZB_KIND_*                                   */
  int dtype;        /* ZB_DTYPE_*                                  */
  int n_layers;
  int hidden;       /* h                                           */
  int ffn;          /* f (4h in the GPT shapes)                    */
  int n_heads;      /* FULL only                                   */
  int seq;          /* tokens per sequence                         */
  int micro_batch;  /* sequences per microbatch                    */
  int n_micro;      /* m, microbatches per step                    */
  int gelu;         /* ZB_GELU_*                                   */
  int recompute_act; /* 0: stash the MLP activation A = GeLU(Z) from F to W
                      *    and Z from F to B;
                      * 1: stash only Z (F to W) and rebuild A from it
                      *    before W: 8 T ffn bytes less per layer for every
                      *    microbatch between F and B, one elementwise pass
                      *    more per W (A then comes from the bf16 Z).      */
  int w_per_linear; /* 0: a W pass issues the weight gradients of all its
                     *    linears as one grouped launch (they are independent);
                     * 1: one launch of the same kernel per linear, as the
                     *    unsplit backward issues them.  Same bits either way. */
} zb_stage_desc;

/* One pass of a schedule.  kind: 'F', 'B', 'W', or 'U' = unsplit backward
 * (B and W of (stage, mb) as one pass, the conventional backward). */
typedef struct {
  int32_t stage;
  int32_t mb;
  char kind;
  char pad_[3];
} zb_op;

/* ------------------------------------------------------------------------
 * Schedule layer (host only, no GPU needed).
 * Zero Bubble Pipeline Parallelism, section 3: handcrafted ZB-H1 / ZB-H2,
 * "The Memory Model", ILP appendix Eq. 3-7; tutorial sections "1F1B" and
 * "Interleaved stages"; audit section "Validate the schedule as data".
 * ---------------------------------------------------------------------- */

/* Statistics of a simulated schedule (integer time units). */
typedef struct {
  int64_t makespan;  /* max over stages of (end of last pass - start of first pass), Eq. 3 */
  int64_t span;      /* latest end over all passes (all stages start at t = 0)            */
  int64_t busy;      /* sum of pass durations                                             */
  int64_t ideal;     /* m * (T_F + T_B + T_W) per stage                                   */
  int64_t bubble;    /* makespan - ideal                                                  */
} zb_sim_stats;

/* Pass order of stage `stage` (0-indexed) of P under ZB_ORDER_*.  Writes at most
 * `cap` ops to out (host) and their count to *n_out (host).  GPIPE and 1F1B emit
 * unsplit 'U' backwards; ZBH1, ZBH2 and WLAST emit split 'B' and 'W' with the W's
 * of a stage in ascending microbatch order.  ZBH2 needs m >= 2P - 1.
 * Errors: ZB_E_ARG (P < 1, m < 1, bad order, cap too small), ZB_E_INVALID_STAGE. */
zb_status zb_schedule_stage_order(int order, int P, int m, int stage,
                                  zb_op* out, int cap, int* n_out);

/* As-soon-as-possible simulation of per-stage orders.  `ops` (host, n_ops) holds
 * the passes of every stage; the passes of one stage run in the order they
 * appear.  times[3] (host) = {T_F, T_B, T_W} >= 1; an unsplit pass lasts
 * T_B + T_W.  A pass starts once its stage is free and its producers have
 * ended (+ t_comm across stages).  Outputs (host, may be NULL): linear_out[n_ops]
 * the one-device order (by simulated start, ties to the lower stage, then the
 * stage's own order), start_out/end_out[n_ops] aligned with linear_out, stats.
 * Errors: ZB_E_ARG, ZB_E_INVALID_STAGE, ZB_E_INVALID_MB, ZB_E_DEADLOCK. */
zb_status zb_schedule_simulate(int P, int m, const zb_op* ops, int n_ops,
                               const int64_t* times, int64_t t_comm,
                               zb_op* linear_out, int64_t* start_out, int64_t* end_out,
                               zb_sim_stats* stats);

/* Generate every stage's order, simulate it and linearize it in one call.
 * linear_out (host) needs cap >= 3*P*m (2*P*m for GPIPE / 1F1B). */
zb_status zb_schedule_build(int order, int P, int m, const int64_t* times, int64_t t_comm,
                            zb_op* linear_out, int cap, int* n_out, zb_sim_stats* stats);

/* Automatic schedule (Zero Bubble Pipeline Parallelism, section 3.1, the
 * heuristic): builds every stage's order from profiled times[3] = {T_F, T_B,
 * T_W} (>= 1) and t_comm, keeping each stage's activation memory within
 * m_limit when F adds m_b, B adds m_w - m_b and W adds -m_w (charged at the
 * start of a pass).  ZB-1p takes 1F1B's peak, P * m_b + max(0, m_w - m_b)
 * (the microbatch in its backward also holds its gradients when a B adds
 * memory), ZB-2p twice the P * m_b term.  Two binary choices (warm-up fill, warm-up balance) are searched and
 * the order with the smallest simulated makespan kept; *choice_out (host, may
 * be NULL) receives 2 * fill + balance.  Emits split B and W passes with each
 * stage's W in ascending microbatch order, linearized like zb_schedule_build
 * into linear_out (host, cap >= 3*P*m); stats (host, may be NULL).
 * Errors: ZB_E_ARG (sizes, times < 1, m_limit < max(m_b, m_w), cap),
 * ZB_E_DEADLOCK. */
zb_status zb_schedule_heuristic(int P, int m, const int64_t* times, int64_t t_comm, int64_t m_b,
                                int64_t m_w, int64_t m_limit, zb_op* linear_out, int cap, int* n_out,
                                zb_sim_stats* stats, int* choice_out);

/* ZB-V (Zero Bubble Pipeline Parallelism, section 6): 2P chunks, device d
 * holding chunks d and 2P-1-d (a V: forwards run down the devices and back
 * up).  times[3] = {T_F, T_B, T_W} per chunk pass (>= 1); t_comm per hand-off
 * between chunks on different devices; m_b, m_w the stash of one chunk and
 * microbatch; m_limit the budget per device (P M_B of a whole stage = 2P *
 * m_b).  The order is list-scheduled within the budget (a forward of a
 * device's earlier chunk keeps room for one later-chunk forward).  When
 * T_F = T_B = T_W a second candidate is searched: an order at unit slots with
 * no idle slot inside any device's span, at most m_limit / max(m_b, m_w) live
 * chunk stashes per device (the section reports zero bubble within P M_B);
 * the search gives up after a fixed number of steps (it finds one for
 * m >= 2P - 1 up to P = 9 at least).  The candidate with the smaller makespan
 * at times and t_comm is emitted, ties to the searched one.  Emits the
 * 6*P*m chunk passes (zb_op.stage = chunk index 0..2P-1, split B and W, each
 * chunk's W ascending) into linear_out (host, cap >= 6*P*m) by start time,
 * ties to the lower chunk: a one-device order for 2P chained stages.  stats
 * (host, may be NULL): makespan = the largest per-device time (Eq. 3), ideal =
 * 2m(T_F+T_B+T_W), bubble = makespan - ideal.  Errors: ZB_E_ARG (sizes, times,
 * m_limit < 2 m_b + max(0, m_w - m_b) or < m_w, cap), ZB_E_DEADLOCK. */
zb_status zb_schedule_zbv(int P, int m, const int64_t* times, int64_t t_comm, int64_t m_b, int64_t m_w,
                          int64_t m_limit, zb_op* linear_out, int cap, int* n_out, zb_sim_stats* stats);

/* Interleaved pipeline with v chunks per device (simulation only): forwards
 * group by group of P microbatches over chunks 0..v-1, unsplit backwards over
 * chunks v-1..0.  times are per chunk.  Needs m % P == 0. */
zb_status zb_schedule_simulate_interleaved(int P, int m, int v, const int64_t* times,
                                           zb_sim_stats* stats);

/* Validate a one-device execution order (host ops).  Pass by pass, first
 * failure wins: kind not F/B/W/U -> ZB_E_ARG; stage outside [0,P) ->
 * ZB_E_INVALID_STAGE; mb outside [0,m) -> ZB_E_INVALID_MB; repeated pass, or
 * U mixed with B/W of the same (stage, mb) -> ZB_E_DUPLICATE; F(s,j) before
 * F(s-1,j), B|U(s,j) before F(s,j) or before B|U(s+1,j), W(s,j) before B(s,j)
 * -> ZB_E_DEPENDENCY.  Then every (s,j) must have F and B+W or U, else
 * ZB_E_MISSING with *bad_index = n_ops.  *bad_index (host) = -1 on success. */
zb_status zb_schedule_validate(int P, int m, const zb_op* ops, int n_ops, int* bad_index);

/* Running activation memory of stage `stage` in `ops` (host): F adds m_b, B adds
 * m_w - m_b, W adds -m_w, U adds -m_b, each at the start of its pass ("The
 * Memory Model").  *peak (host) = the maximum level (>= 0). */
zb_status zb_schedule_peak_memory(const zb_op* ops, int n_ops, int stage,
                                  int64_t m_b, int64_t m_w, int64_t* peak);

/* Timed event of a schedule, for zb_events_inspect. */
typedef struct {
  int32_t id;
  int32_t stage;
  int32_t micro;
  char kind;            /* 'F', 'B', 'W', 'U' (others allowed, ignored by the ledger) */
  char pad_[3];
  double start;
  double end;
  int32_t n_deps;
  const int32_t* deps;  /* host array of n_deps event ids */
} zb_event;

typedef struct {
  double span;               /* latest end (the schedule's time starts at 0)   */
  double busy;               /* sum of (end - start)                           */
  double bubble_ratio;       /* 1 - busy / (stage_count * span)                */
  int64_t unfinished_activations;  /* (stage, micro) activations whose F ran and
                                    * whose stash no W (or U) has released      */
  int64_t peak_live_activations;   /* most activations one stage held at once,
                                    * each from its F to the W that frees its stash */
} zb_event_report;

/* Checks a schedule given as timed events (host), as the audit "Zero-Bubble
 * Pipeline Parallelism, Proven" asks in "Validate the schedule as data" and
 * "Budget activation lifetime".  Phases, first failure wins:
 *   n < 1, a null array or stage_count < 1 -> ZB_E_ARG;
 *   an id used twice -> ZB_E_DUPLICATE (*bad_index = its second use);
 *   stage outside [0, stage_count) -> ZB_E_INVALID_STAGE (first in list order);
 *   start < 0 or end <= start -> ZB_E_INTERVAL (first in list order);
 *   a dependency id naming no event -> ZB_E_MISSING (first in list order);
 *   an event starting before one of its producers ends -> ZB_E_DEPENDENCY
 *     (the violating event with the earliest start, ties to list order);
 *   two events of one stage overlapping in time -> ZB_E_OVERLAP (over every
 *     overlapping pair, the later-starting event, ties to the later in the
 *     list; the earliest such start, ties to list order).
 * *bad_index (host, may be NULL) names the offending event (-1 if none). */
zb_status zb_events_inspect(const zb_event* events, int n, int stage_count,
                            zb_event_report* report, int* bad_index);

/* ------------------------------------------------------------------------
 * Stage objects (GPU).
 * ---------------------------------------------------------------------- */

typedef struct zb_stage zb_stage;

/* Create stage number `stage_index` (0-indexed; used to match schedule ops).
 * weights (host array of n_layers * n_linears device pointers, [layer][linear])
 * point at bf16 or fp32 [K, N] weights; dw (host array, same count) at fp32
 * [K, N] gradient buffers.  Both stay owned by the caller and must outlive the
 * stage.  stream: a hipStream_t (NULL = default stream).
 * Errors: ZB_E_ARG, ZB_E_UNSUPPORTED (shape not a multiple of 8, FULL with
 * head_dim != 128, fp32 with FULL). */
zb_status zb_stage_create(const zb_stage_desc* desc, int stage_index,
                          const void* const* weights, float* const* dw,
                          void* stream, zb_stage** out);

/* Bytes of the per-microbatch tensor classes of a stage (host outputs):
 * fw = live from F to W (layer inputs and what W reads), fb = live from F to B
 * (what only B reads), bw = live from B to W (every linear's output gradient).
 * fw + fb is this build's M_B, fw + bw its M_W. */
zb_status zb_stage_class_bytes(const zb_stage* st, size_t* fw, size_t* fb, size_t* bw);

/* Workspace the stage needs to run `ops` (host, the whole one-device order of
 * all stages; NULL = every microbatch live at once).  Slots of each class are
 * counted by replaying allocations: the input of F(s,j) is claimed when
 * F(s-1,j) runs (or F(s,j) itself on the first stage), freed by W|U(s,j); the
 * F->B tensors live from F(s,j) to B|U(s,j); the gradient entering B(s,j) is
 * claimed when B(s+1,j) runs (or B|U(s,j) on the last stage), freed by
 * W|U(s,j).  The plan is remembered by the stage for zb_stage_bind_workspace.
 * *bytes (host) receives the size. */
zb_status zb_stage_workspace_bytes(zb_stage* st, const zb_op* ops, int n_ops, size_t* bytes);

/* Hand the stage a device buffer of at least the planned size (256-byte
 * aligned).  The stage sub-allocates its stash and the scratch of its kernels
 * (including the split-K partial sums of its GEMMs) from it; the caller keeps
 * ownership and must not write to it while it is bound.  Only allowed while no
 * microbatch is live.  For MLP-linears stages it enqueues, on the stage's
 * stream, the clearing of the dQ and dK columns that identity attention keeps
 * at zero in every B slot.
 * Errors: ZB_E_ARG (null, misaligned), ZB_E_BUDGET (too small), ZB_E_STATE,
 * ZB_E_HIP (that clearing failed to launch: the stage keeps its previous
 * binding, and the new buffer may have been partly cleared). */
zb_status zb_stage_bind_workspace(zb_stage* st, void* dev_ptr, size_t bytes);

/* Device address of the stage's input slot for microbatch mb (claimed on
 * first use): writing stage input there makes zb_forward's copy a no-op. */
zb_status zb_stage_input_slot(zb_stage* st, int mb, void** dev_ptr);
/* Device address of the slot holding the gradient that enters B(mb). */
zb_status zb_stage_grad_slot(zb_stage* st, int mb, void** dev_ptr);

/* F of microbatch mb: x (device, [T, h]) is copied into the input slot (unless
 * it is that slot), the layers run, y (device, [T, h]) receives the stage
 * output.  Needs mb not yet forwarded this step.  Errors: ZB_E_INVALID_MB,
 * ZB_E_STATE, ZB_E_BUDGET (no free slot), ZB_E_HIP. */
zb_status zb_forward(zb_stage* st, int mb, const void* x, void* y);

/* B of microbatch mb: dy (device, [T, h]) is the gradient of the stage output
 * (copied into the gradient slot unless it is that slot); dx (device, [T, h])
 * receives the gradient of the stage input -- the value handed upstream.
 * Frees the F->B tensors and keeps every linear's output gradient for W.
 * Needs F(mb) done and B(mb) not.  Errors as zb_forward. */
zb_status zb_backward_input(zb_stage* st, int mb, const void* dy, void* dx);

/* W of microbatch mb: dW += X^T . dY for every linear, accumulated in fp32 in
 * the caller's gradient buffers.  The first W of a step overwrites dW instead
 * of adding (the buffers need no zeroing).  Frees the microbatch's tensors.
 * Needs B(mb) done.  Errors: ZB_E_INVALID_MB, ZB_E_STATE, ZB_E_HIP. */
zb_status zb_backward_weight(zb_stage* st, int mb);

/* Unsplit backward (B and W of mb as one pass, each linear's input gradient
 * and weight gradient back to back): the fused baseline.  Every weight
 * gradient goes out as its own launch of the kernel the W pass uses (the W
 * pass groups them unless w_per_linear is set), so a comparison with B + W
 * measures the deferral and not a kernel difference; same bits as B then W. */
zb_status zb_backward_unsplit(zb_stage* st, int mb, const void* dy, void* dx);

/* Stage-boundary taps, for stage-by-stage checks ("Zero-Bubble Pipeline
 * Parallelism, Proven", section "Split backward without changing the update":
 * keep per-stage results so the first divergent one can be found).  y_tap and
 * dx_tap are host arrays of n_micro device pointers ([T, h] each, either
 * array may be NULL): after F(mb) the stage output is copied to y_tap[mb],
 * after B(mb) (or U) the stage input gradient to dx_tap[mb], on the stage's
 * stream before any hand-off event is recorded.  Passing NULL for both removes
 * the taps.  The pointers are copied; the buffers stay caller-owned and must
 * outlive the passes that write them.  Errors: ZB_E_ARG (a null entry in a
 * non-null array). */
zb_status zb_stage_set_taps(zb_stage* st, void* const* y_tap, void* const* dx_tap);

/* ------------------------------------------------------------------------
 * Optimizer step with post-update validation (Zero Bubble Pipeline
 * Parallelism, section 4 "the optimizer synchronization bypass", and its
 * Appendix C in-place AdamW rollback).  A stage's gradient state is two
 * doubles in device memory: {sum of the squares of every dW element, 1.0 if any
 * dW element is NaN/Inf else 0.0}.  The clip coefficient of a state is
 * min(1, max_grad_norm / (sqrt(sum) + 1e-6)) (1 when max_grad_norm <= 0); a
 * state with the flag set means "no update".  AdamW step t (1-based), with
 * g = coefficient * dW:
 *   m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
 *   p = p - lr wd p - lr (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps),
 * and the working copy the GEMMs read is refreshed from p (bf16: rounded to
 * nearest even). */
typedef struct {
  float lr, beta1, beta2, eps, weight_decay;
  float max_grad_norm; /* <= 0: no clipping */
} zb_adamw;

/* Give the stage its optimizer state: per linear (the zb_stage_create order)
 * fp32 device buffers of K*N elements — master parameters, first and second
 * moments — all caller-owned, 16-byte aligned, plus weights_rw: the same
 * pointers as the stage's weights, which the step rewrites.  ZB_E_ARG on null
 * or misaligned buffers, weights_rw[i] differing from the stage's weights, or
 * hyperparameters outside lr >= 0, 0 <= beta < 1, eps >= 0, 0 <= lr*wd < 1. */
zb_status zb_stage_optim_bind(zb_stage* st, const zb_adamw* hp, float* const* master, float* const* exp_avg,
                              float* const* exp_avg_sq, void* const* weights_rw);

/* Staged reduce: partial_out (device, 2 doubles) = upstream (device, the
 * previous stage's partial; NULL on the first stage) + this stage's gradient
 * state, on the stage's stream.  Needs a flushed step (zb_grad_flush) whose
 * gradients have not been overwritten yet, else ZB_E_STATE.  Deterministic:
 * fixed reduction order. */
zb_status zb_stage_grad_state(zb_stage* st, const double* upstream, double* partial_out);

/* zb_stage_grad_state for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid it):
 * same result bits, but the per-workgroup partial states live in the
 * library's own device array of 65536 (sum of squares, non-finite count)
 * pairs (1 MiB, one copy per GPU, held until the process ends) instead of the
 * stage's workspace, so neither this call nor the stage needs a bound
 * workspace for it, and nothing is allocated.  Needs the stage's device to be
 * current.  Every call on one GPU shares that array: calls that overlap on one
 * GPU (other streams, other threads) race and must be ordered by the caller.
 * The array needs no clearing: every partial is written before it is read.
 * Errors: ZB_E_ARG (null), ZB_E_UNSUPPORTED (the stage's gradients need more
 * than 65536 partial states: about 64 linears of 1 M elements or more),
 * ZB_E_STATE (no flushed step gradients), ZB_E_HIP. */
zb_status zb_stage_grad_state_noalloc(zb_stage* st, const double* upstream, double* partial_out);

/* Optimistic step number `step` (>= 1) with the state `used` (device, 2
 * doubles; normally this stage's partial).  Same preconditions. */
zb_status zb_stage_optim_step(zb_stage* st, int step, const double* used);

/* Post-update validation of step `step`: when the step taken with `used`
 * differs from the one `global` (device, the last stage's partial) calls for —
 * another clip coefficient or another skip decision — roll it back in place
 * and step again with `global`.  *rolled_back (device int, may be NULL) = 1 if
 * it did, else 0.  The decision is taken on the device; nothing synchronises.
 * Must run before this stage's first W of the next step overwrites dW, else
 * ZB_E_STATE. */
zb_status zb_stage_optim_validate(zb_stage* st, int step, const double* used, const double* global,
                                  int* rolled_back);

/* Undo step `step` taken with `used` (the inverse update alone). */
zb_status zb_stage_optim_rollback(zb_stage* st, int step, const double* used);

/* Step boundary (the optimizer dependency): requires W (or U) of every
 * microbatch of the step, else ZB_E_MISSING.  If nonfinite_out (host) is not
 * NULL, synchronises the stream and stores 1 if any dW holds a NaN or Inf, else
 * 0.  Afterwards the gradient buffers hold the step's full sum until the first
 * W of the next step overwrites them, and every microbatch may be forwarded
 * again. */
zb_status zb_grad_flush(zb_stage* st, int* nonfinite_out);

/* Per-pass record filled by zb_run_schedule when trace != NULL. */
typedef struct {
  zb_op op;
  float ms;      /* device time of the pass (hipEvent pair)          */
  float t0_ms;   /* start, relative to the first pass's start event  */
} zb_trace_rec;

/* Run a one-device order over P stages (host array stages[P], stage_index p at
 * stages[p]).  If all stages share one stream the passes run in list order on
 * it.  If they have different streams, each pass goes to its stage's stream and
 * the cross-stage dependencies become event waits (F(s,j) after F(s-1,j),
 * B|U(s,j) after B|U(s+1,j)), so independent stages run concurrently like
 * pipeline stages on separate devices; the caller must make x0 and dy_last
 * visible to every stage stream beforehand and synchronise every stage stream
 * afterwards.  The whole list is validated
 * (zb_schedule_validate rules) and every stage's workspace plan checked before
 * anything is launched.  x0[mb], dy_last[mb], y_last[mb], dx0[mb] (host arrays
 * of m device pointers, [T, h] each) are the first stage's inputs, the last
 * stage's output gradients, the last stage's outputs and the first stage's
 * input gradients.  Stage s's output is written straight into stage s+1's
 * input slot and stage s+1's dx into stage s's gradient slot.  trace (host,
 * n_ops records, may be NULL) receives per-pass device times, which
 * synchronises the stream at the end.  Does not flush. */
zb_status zb_run_schedule(zb_stage* const* stages, int P, const zb_op* ops, int n_ops,
                          const void* const* x0, const void* const* dy_last,
                          void* const* y_last, void* const* dx0, zb_trace_rec* trace);

/* Text of the calling thread's last error ("" if none); names the first
 * violating op index for schedule errors. */
const char* zb_last_error(void);

/* Debug mode: when on (or when the environment variable ZB_DEBUG_SYNC is set
 * to a non-zero value at library load), every pass (zb_forward,
 * zb_backward_input, zb_backward_weight, zb_backward_unsplit and each op of
 * zb_run_schedule) synchronises its stream and checks for a device error
 * afterwards, returning ZB_E_HIP that names the pass.  Off by default: it
 * serialises the host with the device. */
void zb_set_debug_sync(int on);
int zb_get_debug_sync(void);

/* Release the stage object (not the caller's buffers).  Enqueued work must have
 * finished. */
void zb_stage_destroy(zb_stage* st);

/* ------------------------------------------------------------------------
 * One linear layer's three passes, the per-linear definitions of the tutorial
 * "Pipeline Schedules: GPipe, 1F1B and Zero Bubble", section "Zero bubble:
 * split the backward pass", run by the same kernels the stage uses.
 * x, dy, y, dx, w (device) are row-major bf16 (dtype ZB_DTYPE_BF16) or fp32;
 * dw (device) is fp32 [K, N].  Asynchronous on stream (hipStream_t or NULL).
 * Errors: ZB_E_ARG (null pointer, negative size), ZB_E_UNSUPPORTED (bf16
 * with K, N or T not a multiple of 8, or a pointer not 16-byte aligned).
 * Zero sizes are legal: an empty output is left alone, and an empty
 * contraction (K = 0 in F, N = 0 in B, T = 0 in W) gives zeros (W with
 * accumulate != 0 leaves dw unchanged); the operands of an empty contraction
 * may be NULL.
 * ---------------------------------------------------------------------- */

/* F: y[T, N] = x[T, K] . w[K, N] */
zb_status zb_linear_forward(int dtype, int T, int K, int N, const void* x, const void* w, void* y,
                            void* stream);
/* B: dx[T, K] = dy[T, N] . w[K, N]^T */
zb_status zb_linear_backward_input(int dtype, int T, int K, int N, const void* dy, const void* w, void* dx,
                                   void* stream);
/* W: dw[K, N] = (accumulate ? dw : 0) + x[T, K]^T . dy[T, N], the fp32 sum
 * continuing from the buffer's value inside the same accumulation chain. */
zb_status zb_linear_backward_weight(int dtype, int T, int K, int N, const void* x, const void* dy, float* dw,
                                    int accumulate, void* stream);

/* ------------------------------------------------------------------------
 * Kernel-level timing (measurement).  When enabled, every kernel the library
 * launches is bracketed by a hipEvent pair on its stream; zb_prof_read
 * synchronises and returns per-kernel totals.
 * ---------------------------------------------------------------------- */
typedef struct {
  char name[48];      /* kernel family and tile, e.g. "gemm_w_256x256"   */
  int64_t launches;
  double total_ms;
  double flops;       /* algorithmic FLOPs summed over launches          */
  double bytes;       /* algorithmic HBM bytes summed over launches      */
} zb_prof_rec;

void zb_prof_enable(int on);
void zb_prof_reset(void);
/* Writes up to cap records (host) and the number of distinct kernels to *n. */
zb_status zb_prof_read(zb_prof_rec* out, int cap, int* n);

/* Version string of the library build. */
const char* zb_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ZB_H */
