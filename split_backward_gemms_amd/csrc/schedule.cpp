// Schedule layer: per-stage pass orders, ASAP simulation, one-device
// linearization, order validation, the activation-memory ledger, the
// timed-event inspector, the automatic (ZB-1p / ZB-2p) scheduler and the
// V-placement order (ZB-V).  Host code only.
//
// Sources: "Zero Bubble Pipeline Parallelism" section 3 (ZB-H1, ZB-H2, the
// memory model, ILP appendix Eq. 3-7) and section 5 (bubble rate); the
// tutorial "Pipeline Schedules: GPipe, 1F1B and Zero Bubble" (1F1B warm-up
// P-1-p, interleaved stages); the audit "Zero-Bubble Pipeline Parallelism,
// Proven", section "Validate the schedule as data".  The automatic scheduler
// follows section 3.1 of the first page, ZB-V its section 6.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <map>
#include <string>
#include <unordered_map>
#include <vector>

#include "zb_internal.h"

namespace zb {

namespace {

// Pass kinds packed as small integers for table lookups.
enum { KF = 0, KB = 1, KW = 2, KU = 3, KBAD = 4 };

int kind_index(char k) {
  switch (k) {
    case 'F': return KF;
    case 'B': return KB;
    case 'W': return KW;
    case 'U': return KU;
    default: return KBAD;
  }
}

zb_op mk(int s, int j, char k) {
  zb_op o;
  o.stage = s;
  o.mb = j;
  o.kind = k;
  o.pad_[0] = o.pad_[1] = o.pad_[2] = 0;
  return o;
}

// Builds the op sequence of one stage.  The three split orders share one
// shape: a warm-up of forwards, then one steady-state round per B, then the
// W's still held back.  They differ in the warm-up length, in where a round
// puts its forward, and in how many W's a stage holds back.
std::vector<zb_op> stage_order(int order, int P, int m, int s) {
  std::vector<zb_op> v;
  if (order == ZB_ORDER_GPIPE) {
    for (int j = 0; j < m; ++j) v.push_back(mk(s, j, 'F'));
    for (int j = 0; j < m; ++j) v.push_back(mk(s, j, 'U'));
    return v;
  }
  int warm, held;
  bool f_first;  // round = F,B(,W) if true; B(,W),F if false
  switch (order) {
    case ZB_ORDER_1F1B:
    case ZB_ORDER_ZBH1:
    case ZB_ORDER_WLAST:
      warm = P - 1 - s;       // tutorial: stage p warms up with P-1-p forwards
      held = s;               // ZB-H1: stage s keeps s W's back
      f_first = true;
      break;
    case ZB_ORDER_ZBH2:
      warm = 2 * (P - s) - 1; // 2P-1 forwards on the first stage
      held = 2 * s;
      f_first = false;
      break;
    default:
      return v;
  }
  warm = std::min(warm, m);
  int nf = 0, nw = 0;
  for (; nf < warm; ++nf) v.push_back(mk(s, nf, 'F'));
  for (int b = 0; b < m; ++b) {
    if (f_first && nf < m) v.push_back(mk(s, nf++, 'F'));
    if (order == ZB_ORDER_1F1B) {
      v.push_back(mk(s, b, 'U'));
    } else {
      v.push_back(mk(s, b, 'B'));
      if (order != ZB_ORDER_WLAST && b >= held) v.push_back(mk(s, nw++, 'W'));
    }
    if (!f_first && nf < m) v.push_back(mk(s, nf++, 'F'));
  }
  if (order != ZB_ORDER_1F1B)
    for (; nw < m; ++nw) v.push_back(mk(s, nw, 'W'));
  return v;
}

int64_t duration(int k, const int64_t* t) { return k == KU ? t[1] + t[2] : t[k]; }

}  // namespace

zb_status schedule_stage_order(int order, int P, int m, int stage, std::vector<zb_op>& out) {
  if (P < 1 || m < 1) return set_error(ZB_E_ARG, "P and m must be >= 1");
  if (order < ZB_ORDER_GPIPE || order > ZB_ORDER_WLAST) return set_error(ZB_E_ARG, "unknown order");
  if (stage < 0 || stage >= P) return set_error(ZB_E_INVALID_STAGE, "stage outside [0, P)");
  if (order == ZB_ORDER_ZBH2 && m < 2 * P - 1)
    return set_error(ZB_E_ARG, "ZB-H2 needs m >= 2P-1");
  out = stage_order(order, P, m, stage);
  return ZB_OK;
}

zb_status schedule_simulate(int P, int m, const zb_op* ops, int n_ops, const int64_t* t,
                            int64_t t_comm, std::vector<SimPass>& passes, zb_sim_stats* stats) {
  if (P < 1 || m < 1 || n_ops < 0 || (n_ops > 0 && !ops) || !t)
    return set_error(ZB_E_ARG, "bad simulate arguments");
  for (int i = 0; i < 3; ++i)
    if (t[i] < 1) return set_error(ZB_E_ARG, "pass times must be >= 1");
  if (t_comm < 0) return set_error(ZB_E_ARG, "t_comm must be >= 0");
  std::vector<std::vector<int>> per(P);
  for (int i = 0; i < n_ops; ++i) {
    const zb_op& o = ops[i];
    if (o.stage < 0 || o.stage >= P) return set_error(ZB_E_INVALID_STAGE, "op %d: stage %d", i, o.stage);
    if (o.mb < 0 || o.mb >= m) return set_error(ZB_E_INVALID_MB, "op %d: mb %d", i, o.mb);
    if (kind_index(o.kind) == KBAD) return set_error(ZB_E_ARG, "op %d: kind", i);
    per[o.stage].push_back(i);
  }
  // end time per (stage, mb, kind); -1 = not yet run
  const int64_t NONE = -1;
  std::vector<int64_t> endt((size_t)P * m * 4, NONE), backend((size_t)P * m, NONE);
  auto E = [&](int s, int j, int k) -> int64_t& { return endt[((size_t)s * m + j) * 4 + k]; };
  std::vector<size_t> pos(P, 0);
  std::vector<int64_t> freet(P, 0);
  passes.assign(n_ops, SimPass{});
  int remaining = n_ops;
  while (remaining > 0) {
    bool progressed = false;
    for (int s = 0; s < P; ++s) {
      while (pos[s] < per[s].size()) {
        int idx = per[s][pos[s]];
        const zb_op& o = ops[idx];
        int k = kind_index(o.kind), j = o.mb;
        int64_t ready = freet[s];
        bool ok = true;
        if (k == KF) {
          if (s > 0) {
            if (E(s - 1, j, KF) == NONE) ok = false;
            else ready = std::max(ready, E(s - 1, j, KF) + t_comm);
          }
        } else if (k == KB || k == KU) {
          if (E(s, j, KF) == NONE) ok = false;
          else ready = std::max(ready, E(s, j, KF));
          if (ok && s < P - 1) {
            int64_t be = backend[(size_t)(s + 1) * m + j];
            if (be == NONE) ok = false;
            else ready = std::max(ready, be + t_comm);
          }
        } else {  // W
          if (E(s, j, KB) == NONE) ok = false;
          else ready = std::max(ready, E(s, j, KB));
        }
        if (!ok) break;
        int64_t d = duration(k, t);
        passes[idx] = SimPass{idx, s, ready, ready + d};
        E(s, j, k) = ready + d;
        if (k == KB || k == KU) backend[(size_t)s * m + j] = ready + d;
        freet[s] = ready + d;
        ++pos[s];
        --remaining;
        progressed = true;
      }
    }
    if (!progressed) {
      for (int s = 0; s < P; ++s)
        if (pos[s] < per[s].size())
          return set_error(ZB_E_DEADLOCK, "deadlock: op %d (stage %d) can never start",
                           per[s][pos[s]], s);
    }
  }
  if (stats) {
    int64_t makespan = 0, span = 0, busy = 0;
    for (int s = 0; s < P; ++s) {
      if (per[s].empty()) continue;
      int64_t c = passes[per[s].back()].end - passes[per[s].front()].start;
      makespan = std::max(makespan, c);
    }
    for (const SimPass& p : passes) {
      span = std::max(span, p.end);
      busy += p.end - p.start;
    }
    stats->makespan = makespan;
    stats->span = span;
    stats->busy = busy;
    stats->ideal = (int64_t)m * (t[0] + t[1] + t[2]);
    stats->bubble = makespan - stats->ideal;
  }
  return ZB_OK;
}

void schedule_linearize(const std::vector<SimPass>& passes, std::vector<int>& order) {
  order.resize(passes.size());
  for (size_t i = 0; i < passes.size(); ++i) order[i] = (int)i;
  // Ties: lower stage first, then the stage's own order (which is the input index order).
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
    if (passes[a].start != passes[b].start) return passes[a].start < passes[b].start;
    if (passes[a].stage != passes[b].stage) return passes[a].stage < passes[b].stage;
    return a < b;
  });
}

zb_status schedule_validate(int P, int m, const zb_op* ops, int n_ops, int* bad) {
  if (bad) *bad = -1;
  if (P < 1 || m < 1 || n_ops < 0 || (n_ops > 0 && !ops)) return set_error(ZB_E_ARG, "bad validate arguments");
  std::vector<uint8_t> done((size_t)P * m * 4, 0);
  auto D = [&](int s, int j, int k) -> uint8_t& { return done[((size_t)s * m + j) * 4 + k]; };
  for (int i = 0; i < n_ops; ++i) {
    const zb_op& o = ops[i];
    int k = kind_index(o.kind), s = o.stage, j = o.mb;
    auto fail = [&](zb_status st, const char* why) {
      if (bad) *bad = i;
      return set_error(st, "op %d (stage %d, mb %d, kind %c): %s", i, s, j,
                       (o.kind >= 32 && o.kind < 127) ? o.kind : '?', why);
    };
    if (k == KBAD) return fail(ZB_E_ARG, "kind must be F, B, W or U");
    if (s < 0 || s >= P) return fail(ZB_E_INVALID_STAGE, "stage outside [0, P)");
    if (j < 0 || j >= m) return fail(ZB_E_INVALID_MB, "microbatch outside [0, m)");
    if (D(s, j, k)) return fail(ZB_E_DUPLICATE, "pass repeated");
    if (k == KU && (D(s, j, KB) || D(s, j, KW))) return fail(ZB_E_DUPLICATE, "unsplit pass after split B/W");
    if ((k == KB || k == KW) && D(s, j, KU)) return fail(ZB_E_DUPLICATE, "split pass after unsplit backward");
    if (k == KF) {
      if (s > 0 && !D(s - 1, j, KF)) return fail(ZB_E_DEPENDENCY, "forward before the previous stage's forward");
    } else if (k == KB || k == KU) {
      if (!D(s, j, KF)) return fail(ZB_E_DEPENDENCY, "backward before its own forward");
      if (s < P - 1 && !D(s + 1, j, KB) && !D(s + 1, j, KU))
        return fail(ZB_E_DEPENDENCY, "backward before the next stage's backward");
    } else {
      if (!D(s, j, KB)) return fail(ZB_E_DEPENDENCY, "weight gradient before its B");
    }
    D(s, j, k) = 1;
  }
  for (int s = 0; s < P; ++s)
    for (int j = 0; j < m; ++j) {
      bool f = D(s, j, KF), split = D(s, j, KB) && D(s, j, KW), un = D(s, j, KU);
      if (!f || !(split || un)) {
        if (bad) *bad = n_ops;
        return set_error(ZB_E_MISSING, "stage %d mb %d: %s missing before the step boundary", s, j,
                         !f ? "F" : (D(s, j, KB) ? "W" : "backward"));
      }
    }
  return ZB_OK;
}

}  // namespace zb

using namespace zb;

extern "C" zb_status zb_schedule_stage_order(int order, int P, int m, int stage, zb_op* out, int cap,
                                             int* n_out) {
  clear_error();
  if (!out || !n_out) return set_error(ZB_E_ARG, "null output");
  std::vector<zb_op> v;
  zb_status st = schedule_stage_order(order, P, m, stage, v);
  if (st != ZB_OK) return st;
  if ((int)v.size() > cap) return set_error(ZB_E_ARG, "cap %d < %zu ops", cap, v.size());
  std::copy(v.begin(), v.end(), out);
  *n_out = (int)v.size();
  return ZB_OK;
}

extern "C" zb_status zb_schedule_simulate(int P, int m, const zb_op* ops, int n_ops, const int64_t* times,
                                          int64_t t_comm, zb_op* linear_out, int64_t* start_out,
                                          int64_t* end_out, zb_sim_stats* stats) {
  clear_error();
  std::vector<SimPass> passes;
  zb_status st = schedule_simulate(P, m, ops, n_ops, times, t_comm, passes, stats);
  if (st != ZB_OK) return st;
  std::vector<int> lin;
  schedule_linearize(passes, lin);
  for (int i = 0; i < n_ops; ++i) {
    const SimPass& p = passes[lin[i]];
    if (linear_out) linear_out[i] = ops[lin[i]];
    if (start_out) start_out[i] = p.start;
    if (end_out) end_out[i] = p.end;
  }
  return ZB_OK;
}

extern "C" zb_status zb_schedule_build(int order, int P, int m, const int64_t* times, int64_t t_comm,
                                       zb_op* linear_out, int cap, int* n_out, zb_sim_stats* stats) {
  clear_error();
  if (!linear_out || !n_out) return set_error(ZB_E_ARG, "null output");
  if (P < 1 || m < 1) return set_error(ZB_E_ARG, "P and m must be >= 1");
  std::vector<zb_op> all;
  for (int s = 0; s < P; ++s) {
    std::vector<zb_op> v;
    zb_status st = schedule_stage_order(order, P, m, s, v);
    if (st != ZB_OK) return st;
    all.insert(all.end(), v.begin(), v.end());
  }
  if ((int)all.size() > cap) return set_error(ZB_E_ARG, "cap %d < %zu ops", cap, all.size());
  std::vector<SimPass> passes;
  zb_status st = schedule_simulate(P, m, all.data(), (int)all.size(), times, t_comm, passes, stats);
  if (st != ZB_OK) return st;
  std::vector<int> lin;
  schedule_linearize(passes, lin);
  for (size_t i = 0; i < lin.size(); ++i) linear_out[i] = all[lin[i]];
  *n_out = (int)all.size();
  return ZB_OK;
}

// ------------------------------------------------------ automatic scheduler
//
// The heuristic of "Zero Bubble Pipeline Parallelism", section 3.1 (the
// structured summary's "The Heuristic Scheduling Algorithm"): warm-up forwards
// within the activation-memory budget, a steady state that alternates F and B
// and fills gaps with W, a forward-count balance between neighbouring stages,
// a cool-down that drains the remaining W, and a search over two binary
// choices.  Readings where the description is open:
//  - list scheduling in time: the stage that is free first (ties: lower stage)
//    picks among passes whose producers are placed; stages free at the same
//    moment re-decide until none places another pass;
//  - primary pass: F while warming up (no B yet), then B and F alternate, B
//    first (a W does not break the alternation);
//  - memory is charged at the start of a pass: F +M_B, B +(M_W - M_B), W -M_W;
//    a forward also leaves room for its own B; an F over the budget yields
//    to a pending W (memory-triggered W), else to B; a B over it yields to W;
//    else the stage waits;
//  - fill: during warm-up, a forward that would end after the first B could
//    start is placed anyway (1) or the stage switches to B (0);
//  - balance: during warm-up a forward on stage s > 0 needs stage s-1 to stay
//    at least one forward ahead (unless s-1 has placed all forwards); the
//    first forward of a stage is exempt, so a small budget cannot deadlock;
//  - a pending W (ascending microbatch) fills the wait for the primary pass if
//    the wait is at least T_W, if the primary pass cannot run at all, or if
//    waiting would make this stage's accumulated idle time the largest;
//  - the four (fill, balance) choices are tried in the order (0,0), (0,1),
//    (1,0), (1,1), scored by the simulator's makespan; the first best wins.
namespace {

constexpr int64_t kInf = INT64_MAX / 4;

zb_status heuristic_build(int P, int m, const int64_t* t, int64_t t_comm, int64_t m_b, int64_t m_w,
                          int64_t m_limit, int fill, int balance, std::vector<std::vector<zb_op>>& orders) {
  const int64_t dF = m_b, dB = m_w - m_b, dW = -m_w;
  const int64_t reserve = std::max<int64_t>(0, m_w - m_b);
  orders.assign(P, {});
  std::vector<int> nf(P, 0), nb(P, 0), wq_head(P, 0);
  std::vector<std::vector<int>> wq(P);
  std::vector<int64_t> mem(P, 0), freet(P, 0), idle(P, 0);
  std::vector<char> last(P, 0);
  std::vector<int64_t> end_f((size_t)P * m, -1), end_b((size_t)P * m, -1);
  const int64_t total = 3LL * P * m;
  int64_t placed = 0;
  auto active = [&](int s) { return (int)orders[s].size() < 3 * m; };
  auto ready_f = [&](int s) -> int64_t {
    if (s == 0) return 0;
    const int64_t e = end_f[(size_t)(s - 1) * m + nf[s]];
    return e < 0 ? kInf : e + t_comm;
  };
  auto ready_b = [&](int s) -> int64_t {
    const int j = nb[s];
    int64_t r = end_f[(size_t)s * m + j];
    if (r < 0) return kInf;
    if (s < P - 1) {
      const int64_t e = end_b[(size_t)(s + 1) * m + j];
      if (e < 0) return kInf;
      r = std::max(r, e + t_comm);
    }
    return r;
  };
  auto primary = [&](int s) -> char {
    const bool f_left = nf[s] < m, b_avail = nb[s] < nf[s];
    if (nb[s] == 0) return f_left ? 'F' : (b_avail ? 'B' : 0);
    if (!f_left) return nb[s] < m ? 'B' : 0;
    if (last[s] == 'B' || !b_avail) return 'F';
    return 'B';
  };
  auto place = [&](int s, char kind, int64_t now) {
    int j;
    int64_t start = now;
    if (kind == 'F') {
      j = nf[s];
      start = std::max(now, ready_f(s));
      ++nf[s];
      end_f[(size_t)s * m + j] = start + t[0];
    } else if (kind == 'B') {
      j = nb[s];
      start = std::max(now, ready_b(s));
      ++nb[s];
      end_b[(size_t)s * m + j] = start + t[1];
      wq[s].push_back(j);
    } else {
      j = wq[s][wq_head[s]++];
    }
    if (!orders[s].empty()) idle[s] += start - now;
    mem[s] += kind == 'F' ? dF : (kind == 'B' ? dB : dW);
    freet[s] = start + t[kind == 'F' ? 0 : (kind == 'B' ? 1 : 2)];
    zb_op o{};
    o.stage = s;
    o.mb = j;
    o.kind = kind;
    orders[s].push_back(o);
    if (kind != 'W') last[s] = kind;
    ++placed;
  };
  // 0: place `kind`; 1: wait until `until`; 2: defer to the next event.
  auto decide = [&](int s, int64_t now, char& kind, int64_t& until) -> int {
    char p = primary(s);
    if (p == 'F') {
      const bool full = mem[s] + dF + reserve > m_limit;
      if (full && wq_head[s] < (int)wq[s].size()) {  // memory-triggered W frees a stash first
        kind = 'W';
        return 0;
      }
      bool blocked = full;
      if (balance && nb[s] == 0 && nf[s] > 0 && s > 0 && nf[s - 1] < m && nf[s - 1] < nf[s] + 2) blocked = true;
      if (blocked) {
        p = nb[s] < nf[s] ? 'B' : 0;
      } else if (nb[s] == 0 && nb[s] < nf[s] && !fill) {
        const int64_t rb = ready_b(s);
        if (rb < kInf && std::max(now, ready_f(s)) + t[0] > rb) p = 'B';
      }
    }
    if (p == 'B' && mem[s] + dB > m_limit) p = 0;
    const int64_t r = p == 'F' ? ready_f(s) : (p == 'B' ? ready_b(s) : kInf);
    if (p && r <= now) {
      kind = p;
      return 0;
    }
    if (wq_head[s] < (int)wq[s].size()) {
      const int64_t gap = r >= kInf ? kInf : r - now;
      const int64_t worst = *std::max_element(idle.begin(), idle.end());
      if (!p || gap >= t[2] || (!orders[s].empty() && gap < kInf && idle[s] + gap > worst)) {
        kind = 'W';
        return 0;
      }
    }
    if (p && r < kInf) {
      until = r;
      return 1;
    }
    return 2;
  };

  while (placed < total) {
    int64_t now = kInf;
    for (int s = 0; s < P; ++s)
      if (active(s)) now = std::min(now, freet[s]);
    bool progress = true;
    while (progress) {
      progress = false;
      for (int s = 0; s < P; ++s) {
        if (!active(s) || freet[s] != now) continue;
        char kind = 0;
        int64_t until = 0;
        const int what = decide(s, now, kind, until);
        if (what == 0) {
          place(s, kind, now);
          progress = true;
        } else if (what == 1) {
          if (!orders[s].empty()) idle[s] += until - now;
          freet[s] = until;
        }
      }
    }
    int64_t nxt = kInf;
    bool stuck = false;
    for (int q = 0; q < P; ++q) {
      if (!active(q)) continue;
      if (freet[q] > now) nxt = std::min(nxt, freet[q]);
      else stuck = true;
    }
    if (stuck) {
      if (nxt >= kInf) return set_error(ZB_E_DEADLOCK, "heuristic: no stage can progress");
      for (int s = 0; s < P; ++s)
        if (active(s) && freet[s] == now) {
          if (!orders[s].empty()) idle[s] += nxt - now;
          freet[s] = nxt;
        }
    }
  }
  return ZB_OK;
}

}  // namespace

extern "C" zb_status zb_schedule_heuristic(int P, int m, const int64_t* times, int64_t t_comm, int64_t m_b,
                                           int64_t m_w, int64_t m_limit, zb_op* linear_out, int cap,
                                           int* n_out, zb_sim_stats* stats, int* choice_out) {
  clear_error();
  if (!times || !linear_out || !n_out) return set_error(ZB_E_ARG, "null argument");
  if (P < 1 || m < 1) return set_error(ZB_E_ARG, "P and m must be >= 1");
  if ((int64_t)P * m > (1 << 24)) return set_error(ZB_E_ARG, "P * m too large");
  if (times[0] < 1 || times[1] < 1 || times[2] < 1 || t_comm < 0)
    return set_error(ZB_E_ARG, "times must be >= 1 and t_comm >= 0");
  if (m_b < 0 || m_w < 0 || m_limit < std::max(m_b, m_w))
    return set_error(ZB_E_ARG, "M_limit %lld holds no microbatch (M_B %lld, M_W %lld)", (long long)m_limit,
                     (long long)m_b, (long long)m_w);
  if (cap < 3 * P * m) return set_error(ZB_E_ARG, "cap %d < %d ops", cap, 3 * P * m);
  std::vector<zb_op> best_all;
  std::vector<SimPass> best_passes;
  zb_sim_stats best{};
  int best_choice = -1;
  for (int c = 0; c < 4; ++c) {
    std::vector<std::vector<zb_op>> orders;
    zb_status st = heuristic_build(P, m, times, t_comm, m_b, m_w, m_limit, c >> 1, c & 1, orders);
    if (st != ZB_OK) return st;
    std::vector<zb_op> all;
    for (auto& o : orders) all.insert(all.end(), o.begin(), o.end());
    std::vector<SimPass> passes;
    zb_sim_stats ss{};
    st = schedule_simulate(P, m, all.data(), (int)all.size(), times, t_comm, passes, &ss);
    if (st != ZB_OK) return st;
    if (best_choice < 0 || ss.makespan < best.makespan) {
      best = ss;
      best_choice = c;
      best_all = std::move(all);
      best_passes = std::move(passes);
    }
  }
  std::vector<int> lin;
  schedule_linearize(best_passes, lin);
  for (size_t i = 0; i < lin.size(); ++i) linear_out[i] = best_all[lin[i]];
  *n_out = (int)best_all.size();
  if (stats) *stats = best;
  if (choice_out) *choice_out = best_choice;
  return ZB_OK;
}

// ---------------------------------------------------------------- ZB-V
//
// "Zero Bubble Pipeline Parallelism", section 6: 2P chunks, device d holding
// chunks d and 2P-1-d, so every microbatch's forward runs down the devices and
// back up and its backward retraces that path.  The pages fix the placement
// and its properties, not the order; the order is built by list scheduling:
//  - the device free first (ties: lower device) takes the candidate pass that
//    can start earliest, ties in the order B of its earlier chunk, F of its
//    later chunk, F of its earlier chunk, B of its later chunk;
//  - its oldest pending W runs when nothing else can start at once, or when
//    the next forward would pass the budget;
//  - memory per chunk pass F +M_B, B +(M_W-M_B), W -M_W at the start; a
//    forward of the earlier chunk keeps room for a later-chunk forward and a
//    B's growth, a forward of the later chunk room for its B's growth;
//  - hand-offs between chunks on different devices cost t_comm.
// At equal pass times the section reports zero bubble within P M_B, which
// that list order does not reach.  A second candidate comes from a search
// over unit slots (zbv_search below); the candidate with the smaller makespan
// simulated at the given times and t_comm wins, ties to the searched one.
namespace {

zb_status zbv_build(int P, int m, const int64_t* t, int64_t t_comm, int64_t m_b, int64_t m_w, int64_t m_limit,
                    std::vector<zb_op>& ops, std::vector<int64_t>& start) {
  const int C = 2 * P;
  const int64_t reserve = std::max<int64_t>(0, m_w - m_b);
  auto dev = [P](int c) { return c < P ? c : 2 * P - 1 - c; };
  auto hop = [&](int a, int b) { return dev(a) == dev(b) ? int64_t(0) : t_comm; };
  std::vector<int> nf(C, 0), nb(C, 0), count(P, 0), wq_head(P, 0);
  std::vector<std::vector<std::pair<int, int>>> wq(P);
  std::vector<int64_t> end_f((size_t)C * m, -1), end_b((size_t)C * m, -1), mem(P, 0), freet(P, 0);
  auto ready_f = [&](int c) -> int64_t {
    const int j = nf[c];
    if (j >= m) return -1;
    if (c == 0) return 0;
    const int64_t e = end_f[(size_t)(c - 1) * m + j];
    return e < 0 ? -1 : e + hop(c - 1, c);
  };
  auto ready_b = [&](int c) -> int64_t {
    const int j = nb[c];
    if (j >= nf[c]) return -1;
    int64_t r = end_f[(size_t)c * m + j];
    if (c < C - 1) {
      const int64_t e = end_b[(size_t)(c + 1) * m + j];
      if (e < 0) return -1;
      r = std::max(r, e + hop(c + 1, c));
    }
    return r;
  };
  struct Cand { int64_t st; int rank; char kind; int chunk; };
  ops.clear();
  start.clear();
  const int64_t total = 6LL * P * m;
  for (int64_t placed = 0; placed < total; ++placed) {
    bool have = false;
    Cand best{};
    int best_d = -1;
    for (int d = 0; d < P; ++d) {
      if (count[d] == 6 * m) continue;
      const int lo = d, hi = C - 1 - d;
      const int64_t now = freet[d];
      Cand c[5];
      int n = 0;
      int64_t r;
      if ((r = ready_b(lo)) >= 0 && mem[d] + m_w - m_b <= m_limit) c[n++] = {std::max(now, r), 0, 'B', lo};
      if ((r = ready_f(hi)) >= 0 && mem[d] + m_b + reserve <= m_limit) c[n++] = {std::max(now, r), 1, 'F', hi};
      if ((r = ready_f(lo)) >= 0 && mem[d] + 2 * m_b + reserve <= m_limit) c[n++] = {std::max(now, r), 2, 'F', lo};
      if ((r = ready_b(hi)) >= 0 && mem[d] + m_w - m_b <= m_limit) c[n++] = {std::max(now, r), 3, 'B', hi};
      if (wq_head[d] < (int)wq[d].size()) {
        int64_t first = -1;
        for (int i = 0; i < n; ++i) first = first < 0 ? c[i].st : std::min(first, c[i].st);
        const bool full = n == 0 || mem[d] + m_b + reserve > m_limit;
        if (full || first > now) c[n++] = {now, 4, 'W', wq[d][wq_head[d]].first};
      }
      for (int i = 0; i < n; ++i) {
        const bool better = !have || c[i].st < best.st || (c[i].st == best.st && d < best_d) ||
                            (c[i].st == best.st && d == best_d && c[i].rank < best.rank);
        if (better) {
          best = c[i];
          best_d = d;
          have = true;
        }
      }
    }
    if (!have) return set_error(ZB_E_DEADLOCK, "zb-v: no device can progress");
    const int d = best_d;
    int ch = best.chunk, j;
    if (best.kind == 'F') {
      j = nf[ch]++;
      end_f[(size_t)ch * m + j] = best.st + t[0];
      mem[d] += m_b;
      freet[d] = best.st + t[0];
    } else if (best.kind == 'B') {
      j = nb[ch]++;
      end_b[(size_t)ch * m + j] = best.st + t[1];
      wq[d].push_back({ch, j});
      mem[d] += m_w - m_b;
      freet[d] = best.st + t[1];
    } else {
      ch = wq[d][wq_head[d]].first;
      j = wq[d][wq_head[d]].second;
      ++wq_head[d];
      mem[d] -= m_w;
      freet[d] = best.st + t[2];
    }
    ++count[d];
    zb_op o;
    o.stage = ch;
    o.mb = j;
    o.kind = best.kind;
    ops.push_back(o);
    start.push_back(best.st);
  }
  return ZB_OK;
}

constexpr int64_t kZbvSearchBudget = 1000000;  // search steps before the searched candidate is given up

// Latest slot of every chunk pass when device d works in slots d .. d+6m-1:
// each successor (F(c+1,j) and B(c,j) after F(c,j); B(c-1,j) and W(c,j) after
// B(c,j); the same pass of microbatch j+1 after j) starts at least one slot
// later, and no pass ends after its device's last slot.  Index
// (kind*C + c)*m + j, kind 0 = F, 1 = B, 2 = W.
std::vector<int> zbv_latest_starts(int P, int m) {
  const int C = 2 * P;
  auto dev = [P](int c) { return c < P ? c : 2 * P - 1 - c; };
  std::vector<int> L((size_t)3 * C * m);
  auto at = [&](int k, int c, int j) -> int& { return L[((size_t)k * C + c) * m + j]; };
  for (int j = m - 1; j >= 0; --j) {
    for (int c = 0; c < C; ++c) {
      int cap = dev(c) + 6 * m - 1;
      if (j + 1 < m) cap = std::min(cap, at(2, c, j + 1) - 1);
      at(2, c, j) = cap;
    }
    for (int c = 0; c < C; ++c) {
      int cap = std::min(dev(c) + 6 * m - 1, at(2, c, j) - 1);
      if (c > 0) cap = std::min(cap, at(1, c - 1, j) - 1);
      if (j + 1 < m) cap = std::min(cap, at(1, c, j + 1) - 1);
      at(1, c, j) = cap;
    }
    for (int c = C - 1; c >= 0; --c) {
      int cap = std::min(dev(c) + 6 * m - 1, at(1, c, j) - 1);
      if (c + 1 < C) cap = std::min(cap, at(0, c + 1, j) - 1);
      if (j + 1 < m) cap = std::min(cap, at(0, c, j + 1) - 1);
      at(0, c, j) = cap;
    }
  }
  return L;
}

struct VPass { char kind; int chunk, mb; };

// A V order with no idle slot inside any device's span at unit pass times,
// within m_limit per device.  Slots are filled in time order, devices 0..P-1
// within a slot; a device picks among the passes whose producers finished
// before the slot began.  Choices go by urgency: the pass's latest start (for
// microbatches more than P+1 before the last, that of microbatch m-P-1 less six
// slots per microbatch, so early microbatches are as urgent as in a short
// pipeline), then W before F before B, then the earlier chunk.  After each slot
// a branch is cut when a pending pass is past its latest start, or when some
// device cannot have work in every coming slot even if every chain ran as early
// as it allows.  Returns false when none is found within the budget.
bool zbv_search(int P, int m, int64_t m_b, int64_t m_w, int64_t m_limit,
                std::vector<std::vector<VPass>>& orders) {
  const int C = 2 * P, h = P + 1;
  const std::vector<int> lst = zbv_latest_starts(P, m);
  auto L = [&](int k, int c, int j) { return lst[((size_t)k * C + c) * m + j]; };
  auto urgency = [&](int k, int c, int j) {
    if (m > h && j < m - h) return L(k, c, m - h) - 6 * (m - h - j);
    return L(k, c, j);
  };
  std::vector<int> cnt((size_t)3 * C, 0), done(P, 0);
  auto N = [&](int k, int c) -> int& { return cnt[(size_t)k * C + c]; };
  orders.assign(P, {});
  static const int rank[3] = {1, 2, 0};  // F, B, W -> W first, then F, then B
  static const char kname[3] = {'F', 'B', 'W'};

  struct Choice { int k, c; };  // k = -1: nothing this slot
  struct Level { int t, d; bool finished; std::vector<Choice> opts; int i; };
  std::vector<std::vector<int>> snaps;  // counts at the start of each slot
  std::vector<int> est((size_t)3 * C * m), mine;

  auto hopeless = [&](int t) {
    for (int k = 0; k < 3; ++k)
      for (int c = 0; c < C; ++c) {
        const int j = N(k, c);
        if (j < m && L(k, c, j) < t) return true;
      }
    auto E = [&](int k, int c, int j) -> int& { return est[((size_t)k * C + c) * m + j]; };
    std::fill(est.begin(), est.end(), -1);
    for (int j = 0; j < m; ++j) {
      for (int c = 0; c < C; ++c) {
        if (N(0, c) > j) continue;
        int e = t;
        if (c > 0 && E(0, c - 1, j) >= 0) e = std::max(e, E(0, c - 1, j) + 1);
        if (j > 0 && E(0, c, j - 1) >= 0) e = std::max(e, E(0, c, j - 1) + 1);
        E(0, c, j) = e;
      }
      for (int c = C - 1; c >= 0; --c) {
        if (N(1, c) <= j) {
          int e = t;
          if (E(0, c, j) >= 0) e = std::max(e, E(0, c, j) + 1);
          if (c < C - 1 && E(1, c + 1, j) >= 0) e = std::max(e, E(1, c + 1, j) + 1);
          if (j > 0 && E(1, c, j - 1) >= 0) e = std::max(e, E(1, c, j - 1) + 1);
          E(1, c, j) = e;
        }
        if (N(2, c) <= j) {
          int e = t;
          if (E(1, c, j) >= 0) e = std::max(e, E(1, c, j) + 1);
          if (j > 0 && E(2, c, j - 1) >= 0) e = std::max(e, E(2, c, j - 1) + 1);
          E(2, c, j) = e;
        }
      }
    }
    for (int d = 0; d < P; ++d) {
      if (done[d] == 6 * m) continue;
      mine.clear();
      for (int c : {d, C - 1 - d})
        for (int k = 0; k < 3; ++k)
          for (int j = N(k, c); j < m; ++j) mine.push_back(E(k, c, j));
      std::sort(mine.begin(), mine.end());
      const int first = std::max(t, d);
      for (size_t i = 0; i < mine.size(); ++i)
        if (mine[i] > first + (int)i) return true;
    }
    return false;
  };

  // Stashes live per device (forward started, W not yet): at most `room`, so
  // that the ledger level, at most max(M_B, M_W) per live stash, stays within
  // m_limit whatever the ratio of M_B to M_W.
  const int64_t big = std::max(m_b, m_w);
  const int64_t room = big > 0 ? m_limit / big : 2LL * m;
  auto choices = [&](int d, const std::vector<int>& s, std::vector<Choice>& out) {
    out.clear();
    auto S = [&](int k, int c) { return s[(size_t)k * C + c]; };
    int64_t live = 0;
    for (int c : {d, C - 1 - d}) live += S(0, c) - S(2, c);
    for (int c : {d, C - 1 - d}) {
      if (S(0, c) < m && live < room && (c == 0 || S(0, c - 1) > S(0, c))) out.push_back({0, c});
      if (S(1, c) < S(0, c) && (c == C - 1 || S(1, c + 1) > S(1, c))) out.push_back({1, c});
      if (S(2, c) < S(1, c)) out.push_back({2, c});
    }
    std::stable_sort(out.begin(), out.end(), [&](const Choice& a, const Choice& b) {
      const int ua = urgency(a.k, a.c, N(a.k, a.c)), ub = urgency(b.k, b.c, N(b.k, b.c));
      if (ua != ub) return ua < ub;
      return rank[a.k] < rank[b.k];
    });
  };

  int64_t steps = 0;
  auto enter = [&](int t, int d, Level& lv) -> bool {  // false: budget spent
    if (++steps > kZbvSearchBudget) return false;
    lv.t = t;
    lv.d = d;
    lv.finished = false;
    lv.i = -1;
    lv.opts.clear();
    if (d == P) {
      bool all = true;
      for (int x : done) all = all && x == 6 * m;
      if (all) {
        lv.finished = true;
        return true;
      }
      if (hopeless(t + 1)) return true;
      if ((int)snaps.size() < t + 2) snaps.resize(t + 2);
      snaps[t + 1] = cnt;
      lv.opts.push_back({-1, -1});
      return true;
    }
    if (done[d] == 6 * m || t < d) {
      lv.opts.push_back({-1, -1});
      return true;
    }
    choices(d, snaps[t], lv.opts);
    return true;
  };

  snaps.assign(1, cnt);
  std::vector<Level> stack(1);
  if (!enter(0, 0, stack[0])) return false;
  size_t depth = 1;
  while (depth) {
    Level& lv = stack[depth - 1];
    if (lv.finished) return true;
    if (lv.i >= 0 && lv.opts[lv.i].k >= 0) {
      const Choice& ch = lv.opts[lv.i];
      --N(ch.k, ch.c);
      --done[lv.d];
      orders[lv.d].pop_back();
    }
    ++lv.i;
    if (lv.i >= (int)lv.opts.size()) {
      --depth;
      continue;
    }
    const Choice ch = lv.opts[lv.i];
    if (ch.k >= 0) {
      orders[lv.d].push_back({kname[ch.k], ch.c, N(ch.k, ch.c)});
      ++N(ch.k, ch.c);
      ++done[lv.d];
    }
    const int nt = lv.d == P ? lv.t + 1 : lv.t, nd = lv.d == P ? 0 : lv.d + 1;
    if (stack.size() <= depth) stack.resize(depth + 1);
    if (!enter(nt, nd, stack[depth])) return false;
    ++depth;
  }
  return false;
}

// As-soon-as-possible start of every pass of fixed per-device V orders; false
// when the orders deadlock.  ops/start are filled device by device.
bool zbv_simulate(int P, int m, const std::vector<std::vector<VPass>>& orders, const int64_t* t,
                  int64_t t_comm, std::vector<zb_op>& ops, std::vector<int64_t>& start) {
  const int C = 2 * P;
  auto dev = [P](int c) { return c < P ? c : 2 * P - 1 - c; };
  auto hop = [&](int a, int b) { return dev(a) == dev(b) ? int64_t(0) : t_comm; };
  std::vector<int64_t> end_f((size_t)C * m, -1), end_b((size_t)C * m, -1), freet(P, 0);
  std::vector<size_t> pos(P, 0);
  ops.clear();
  start.clear();
  size_t remaining = 0;
  for (const auto& o : orders) remaining += o.size();
  while (remaining) {
    bool progressed = false;
    for (int d = 0; d < P; ++d) {
      while (pos[d] < orders[d].size()) {
        const VPass& p = orders[d][pos[d]];
        const int c = p.chunk, j = p.mb;
        int64_t r = freet[d];
        bool ok = true;
        auto need = [&](int64_t e, int64_t extra) {
          if (e < 0) ok = false;
          else r = std::max(r, e + extra);
        };
        if (p.kind == 'F') {
          if (c > 0) need(end_f[(size_t)(c - 1) * m + j], hop(c - 1, c));
        } else if (p.kind == 'B') {
          need(end_f[(size_t)c * m + j], 0);
          if (c < C - 1) need(end_b[(size_t)(c + 1) * m + j], hop(c + 1, c));
        } else {
          need(end_b[(size_t)c * m + j], 0);
        }
        if (!ok) break;
        const int64_t e = r + (p.kind == 'F' ? t[0] : (p.kind == 'B' ? t[1] : t[2]));
        if (p.kind == 'F') end_f[(size_t)c * m + j] = e;
        if (p.kind == 'B') end_b[(size_t)c * m + j] = e;
        freet[d] = e;
        zb_op o;
        o.stage = c;
        o.mb = j;
        o.kind = p.kind;
        ops.push_back(o);
        start.push_back(r);
        ++pos[d];
        --remaining;
        progressed = true;
      }
    }
    if (!progressed) return false;
  }
  return true;
}

// Eq. 3 makespan of passes with start times: the largest per-device span.
int64_t zbv_makespan(int P, const std::vector<zb_op>& ops, const std::vector<int64_t>& start, const int64_t* t) {
  std::vector<int64_t> first(P, -1), last(P, 0);
  for (size_t i = 0; i < ops.size(); ++i) {
    const int c = ops[i].stage, d = c < P ? c : 2 * P - 1 - c;
    const int64_t e = start[i] + (ops[i].kind == 'F' ? t[0] : (ops[i].kind == 'B' ? t[1] : t[2]));
    if (first[d] < 0 || start[i] < first[d]) first[d] = start[i];
    last[d] = std::max(last[d], e);
  }
  int64_t mk = 0;
  for (int d = 0; d < P; ++d) mk = std::max(mk, last[d] - first[d]);
  return mk;
}

}  // namespace

extern "C" zb_status zb_schedule_zbv(int P, int m, const int64_t* times, int64_t t_comm, int64_t m_b, int64_t m_w,
                                     int64_t m_limit, zb_op* linear_out, int cap, int* n_out,
                                     zb_sim_stats* stats) {
  clear_error();
  if (!times || !linear_out || !n_out) return set_error(ZB_E_ARG, "null argument");
  if (P < 1 || m < 1) return set_error(ZB_E_ARG, "P and m must be >= 1");
  if ((int64_t)P * m > (1 << 23)) return set_error(ZB_E_ARG, "P * m too large");
  if (times[0] < 1 || times[1] < 1 || times[2] < 1 || t_comm < 0)
    return set_error(ZB_E_ARG, "times must be >= 1 and t_comm >= 0");
  const int64_t reserve = std::max<int64_t>(0, m_w - m_b);
  if (m_b < 0 || m_w < 0 || m_limit < 2 * m_b + reserve || m_limit < m_w)
    return set_error(ZB_E_ARG, "M_limit %lld holds no microbatch through both chunks (M_B %lld, M_W %lld)",
                     (long long)m_limit, (long long)m_b, (long long)m_w);
  if (cap < 6 * P * m) return set_error(ZB_E_ARG, "cap %d < %d ops", cap, 6 * P * m);
  std::vector<zb_op> ops;
  std::vector<int64_t> start;
  zb_status st = zbv_build(P, m, times, t_comm, m_b, m_w, m_limit, ops, start);
  if (st != ZB_OK) return st;
  if (times[0] == times[1] && times[1] == times[2]) {
    std::vector<std::vector<VPass>> found;
    std::vector<zb_op> s_ops;
    std::vector<int64_t> s_start;
    if (zbv_search(P, m, m_b, m_w, m_limit, found) && zbv_simulate(P, m, found, times, t_comm, s_ops, s_start) &&
        zbv_makespan(P, s_ops, s_start, times) <= zbv_makespan(P, ops, start, times)) {
      ops.swap(s_ops);
      start.swap(s_start);
    }
  }
  // Linearize over the 2P chunk stages by start time, ties to the lower chunk.
  std::vector<int> idx(ops.size());
  for (size_t i = 0; i < idx.size(); ++i) idx[i] = (int)i;
  std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) {
    if (start[a] != start[b]) return start[a] < start[b];
    return ops[a].stage < ops[b].stage;
  });
  for (size_t i = 0; i < idx.size(); ++i) linear_out[i] = ops[idx[i]];
  *n_out = (int)ops.size();
  if (stats) {
    auto dur = [&](char k) { return k == 'F' ? times[0] : (k == 'B' ? times[1] : times[2]); };
    std::vector<int64_t> first(P, -1), last(P, 0);
    int64_t span = 0, busy = 0;
    for (size_t i = 0; i < ops.size(); ++i) {
      const int c = ops[i].stage, d = c < P ? c : 2 * P - 1 - c;
      const int64_t e = start[i] + dur(ops[i].kind);
      if (first[d] < 0 || start[i] < first[d]) first[d] = start[i];
      last[d] = std::max(last[d], e);
      span = std::max(span, e);
      busy += dur(ops[i].kind);
    }
    int64_t mk = 0;
    for (int d = 0; d < P; ++d) mk = std::max(mk, last[d] - first[d]);
    stats->makespan = mk;
    stats->span = span;
    stats->busy = busy;
    stats->ideal = 2LL * m * (times[0] + times[1] + times[2]);
    stats->bubble = mk - stats->ideal;
  }
  return ZB_OK;
}

extern "C" zb_status zb_schedule_simulate_interleaved(int P, int m, int v, const int64_t* t,
                                                      zb_sim_stats* stats) {
  clear_error();
  if (P < 1 || m < 1 || v < 1 || !t || !stats) return set_error(ZB_E_ARG, "bad arguments");
  if (m % P) return set_error(ZB_E_ARG, "interleaved order needs m %% P == 0");
  for (int i = 0; i < 3; ++i)
    if (t[i] < 1) return set_error(ZB_E_ARG, "pass times must be >= 1");
  // Virtual stage k = c*P + d lives on device d; dependencies run along k.
  const int V = v * P;
  struct VOp { int k, kind, j; };
  std::vector<std::vector<VOp>> dev(P);
  for (int d = 0; d < P; ++d) {
    for (int g = 0; g < m; g += P)
      for (int c = 0; c < v; ++c)
        for (int j = g; j < g + P; ++j) dev[d].push_back({c * P + d, KF, j});
    for (int g = 0; g < m; g += P)
      for (int c = v - 1; c >= 0; --c)
        for (int j = g; j < g + P; ++j) dev[d].push_back({c * P + d, KU, j});
  }
  const int64_t NONE = -1;
  std::vector<int64_t> fend((size_t)V * m, NONE), uend((size_t)V * m, NONE);
  std::vector<int64_t> first_start(P, NONE), last_end(P, 0), freet(P, 0);
  std::vector<size_t> pos(P, 0);
  size_t remaining = 0;
  for (auto& q : dev) remaining += q.size();
  int64_t busy = 0, span = 0;
  while (remaining) {
    bool progressed = false;
    for (int d = 0; d < P; ++d) {
      while (pos[d] < dev[d].size()) {
        const VOp& o = dev[d][pos[d]];
        int64_t ready = freet[d];
        if (o.kind == KF) {
          if (o.k > 0) {
            int64_t e = fend[(size_t)(o.k - 1) * m + o.j];
            if (e == NONE) break;
            ready = std::max(ready, e);
          }
        } else {
          int64_t fe = fend[(size_t)o.k * m + o.j];
          if (fe == NONE) break;
          ready = std::max(ready, fe);
          if (o.k < V - 1) {
            int64_t e = uend[(size_t)(o.k + 1) * m + o.j];
            if (e == NONE) break;
            ready = std::max(ready, e);
          }
        }
        int64_t dur = duration(o.kind, t);
        if (o.kind == KF) fend[(size_t)o.k * m + o.j] = ready + dur;
        else uend[(size_t)o.k * m + o.j] = ready + dur;
        if (first_start[d] == NONE) first_start[d] = ready;
        last_end[d] = ready + dur;
        freet[d] = ready + dur;
        busy += dur;
        span = std::max(span, ready + dur);
        ++pos[d];
        --remaining;
        progressed = true;
      }
    }
    if (!progressed) return set_error(ZB_E_DEADLOCK, "interleaved order deadlocked");
  }
  int64_t makespan = 0;
  for (int d = 0; d < P; ++d) makespan = std::max(makespan, last_end[d] - first_start[d]);
  stats->makespan = makespan;
  stats->span = span;
  stats->busy = busy;
  stats->ideal = (int64_t)m * v * (t[0] + t[1] + t[2]);
  stats->bubble = makespan - stats->ideal;
  return ZB_OK;
}

extern "C" zb_status zb_schedule_validate(int P, int m, const zb_op* ops, int n_ops, int* bad_index) {
  clear_error();
  return schedule_validate(P, m, ops, n_ops, bad_index);
}

extern "C" zb_status zb_schedule_peak_memory(const zb_op* ops, int n_ops, int stage, int64_t m_b,
                                             int64_t m_w, int64_t* peak) {
  clear_error();
  if (!peak || n_ops < 0 || (n_ops > 0 && !ops)) return set_error(ZB_E_ARG, "bad arguments");
  int64_t level = 0, best = 0;
  for (int i = 0; i < n_ops; ++i) {
    if (ops[i].stage != stage) continue;
    switch (kind_index(ops[i].kind)) {
      case KF: level += m_b; break;
      case KB: level += m_w - m_b; break;
      case KW: level -= m_w; break;
      case KU: level -= m_b; break;
      default: return set_error(ZB_E_ARG, "op %d: kind", i);
    }
    best = std::max(best, level);
  }
  *peak = best;
  return ZB_OK;
}

namespace {
// One boundary of an event's interval for the per-stage sweep.
struct SweepPoint {
  double t;
  int is_start;  // ends sort before starts at one instant: touching intervals do not overlap
  int idx;
};
}  // namespace

extern "C" zb_status zb_events_inspect(const zb_event* ev, int n, int stage_count, zb_event_report* rep,
                                       int* bad_index) {
  clear_error();
  if (bad_index) *bad_index = -1;
  if (n < 1 || !ev || !rep) return set_error(ZB_E_ARG, "need at least one event and a report");
  if (stage_count < 1) return set_error(ZB_E_ARG, "invalid_stage_count %d", stage_count);
  auto fail = [&](zb_status st, int i, const char* why) {
    if (bad_index) *bad_index = i;
    return set_error(st, "event %d (id %d): %s", i, ev[i].id, why);
  };
  // Ids -> positions; the second use of an id is the duplicate.
  std::unordered_map<int32_t, int> pos;
  pos.reserve((size_t)n * 2);
  for (int i = 0; i < n; ++i)
    if (!pos.emplace(ev[i].id, i).second) return fail(ZB_E_DUPLICATE, i, "duplicate_task");
  for (int i = 0; i < n; ++i)
    if (ev[i].stage < 0 || ev[i].stage >= stage_count) return fail(ZB_E_INVALID_STAGE, i, "invalid_stage");
  for (int i = 0; i < n; ++i)
    if (!(ev[i].start >= 0.0 && ev[i].end > ev[i].start)) return fail(ZB_E_INTERVAL, i, "invalid_interval");
  // Resolve the dependency edges once; a name with no event is a missing producer.
  std::vector<int> prod_first(n + 1, 0), prod;
  for (int i = 0; i < n; ++i) {
    if (ev[i].n_deps > 0 && !ev[i].deps) return fail(ZB_E_ARG, i, "null dependency array");
    for (int d = 0; d < ev[i].n_deps; ++d) {
      auto it = pos.find(ev[i].deps[d]);
      if (it == pos.end()) return fail(ZB_E_MISSING, i, "missing_dependency");
      prod.push_back(it->second);
    }
    prod_first[i + 1] = (int)prod.size();
  }
  // A consumer that begins before a producer ends: report the earliest such start.
  int early = -1;
  for (int i = 0; i < n; ++i) {
    double ready = 0.0;
    for (int q = prod_first[i]; q < prod_first[i + 1]; ++q) ready = std::max(ready, ev[prod[q]].end);
    if (ready > ev[i].start && (early < 0 || ev[i].start < ev[early].start)) early = i;
  }
  if (early >= 0) return fail(ZB_E_DEPENDENCY, early, "dependency_violation");
  // Exclusive work per stage: sweep every interval boundary in time order and
  // count what is running on each stage; a start on a busy stage overlaps.
  std::vector<SweepPoint> pts;
  pts.reserve(2 * (size_t)n);
  for (int i = 0; i < n; ++i) {
    pts.push_back({ev[i].start, 1, i});
    pts.push_back({ev[i].end, 0, i});
  }
  std::sort(pts.begin(), pts.end(), [](const SweepPoint& a, const SweepPoint& b) {
    if (a.t != b.t) return a.t < b.t;
    if (a.is_start != b.is_start) return a.is_start < b.is_start;
    return a.idx < b.idx;
  });
  std::vector<int> running(stage_count, 0);
  for (const SweepPoint& p : pts) {
    int& r = running[ev[p.idx].stage];
    if (!p.is_start) {
      --r;
      continue;
    }
    if (r > 0) return fail(ZB_E_OVERLAP, p.idx, "stage_overlap");
    ++r;
  }
  // Totals and the activation ledger: an activation of (stage, micro) is held
  // from its F until the W (or unsplit U) that frees the stash its B left.
  double span = 0.0, busy = 0.0;
  for (int i = 0; i < n; ++i) {
    span = std::max(span, ev[i].end);
    busy += ev[i].end - ev[i].start;
  }
  std::vector<int> by_start(n);
  for (int i = 0; i < n; ++i) by_start[i] = i;
  std::stable_sort(by_start.begin(), by_start.end(), [&](int a, int b) { return ev[a].start < ev[b].start; });
  std::map<std::pair<int32_t, int32_t>, int64_t> held;
  std::vector<int64_t> held_by_stage(stage_count, 0);
  int64_t peak = 0;
  for (int i : by_start) {
    const std::pair<int32_t, int32_t> key(ev[i].stage, ev[i].micro);
    if (ev[i].kind == 'F') {
      held[key] += 1;
      held_by_stage[ev[i].stage] += 1;
    } else if (ev[i].kind == 'W' || ev[i].kind == 'U') {
      auto it = held.find(key);
      if (it != held.end() && it->second > 0) {
        it->second -= 1;
        held_by_stage[ev[i].stage] -= 1;
      }
    }
    peak = std::max(peak, held_by_stage[ev[i].stage]);
  }
  int64_t unfinished = 0;
  for (const auto& kv : held) unfinished += kv.second;
  rep->span = span;
  rep->busy = busy;
  rep->bubble_ratio = 1.0 - busy / (stage_count * span);
  rep->unfinished_activations = unfinished;
  rep->peak_live_activations = peak;
  return ZB_OK;
}
