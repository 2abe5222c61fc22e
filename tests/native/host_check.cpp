// Host-side checks of libzb's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (device code is not
// instrumented) and run without a GPU.
//
// It walks the host paths a pipeline takes before anything reaches the
// device: the schedule layer (generation, simulation, validation, memory
// peaks, the automatic and V schedulers, the timed-event inspector), and for
// every workload shape the stage set-up a pipeline performs -- create,
// per-class sizes, the workspace plan for the real one-device order, binding,
// slot claims, taps -- with device addresses that are only stored, never
// dereferenced on the host.  Any invalid access or undefined behaviour aborts
// the run with the sanitizer's report; a wrong status is counted as a failure.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "../../include/zb.h"

static int g_fail = 0;
#define CHECK(c)                                                                          \
  do {                                                                                    \
    if (!(c)) {                                                                           \
      std::fprintf(stderr, "FAIL %s:%d %s (%s)\n", __FILE__, __LINE__, #c, zb_last_error()); \
      ++g_fail;                                                                           \
    }                                                                                     \
  } while (0)

static std::vector<zb_op> build(int order, int P, int m, const int64_t* t) {
  std::vector<zb_op> ops(3 * (size_t)P * m + 1);
  int n = 0;
  zb_sim_stats st;
  zb_status rc = zb_schedule_build(order, P, m, t, 0, ops.data(), (int)ops.size(), &n, &st);
  if (rc != ZB_OK) return {};
  ops.resize(n);
  return ops;
}

static void schedule_layer(std::mt19937& rng) {
  const int64_t unit[3] = {1, 1, 1};
  for (int P = 1; P <= 8; ++P)
    for (int m = 1; m <= 24; m += (m < 8 ? 1 : 5))
      for (int order = ZB_ORDER_GPIPE; order <= ZB_ORDER_WLAST; ++order) {
        if (order == ZB_ORDER_ZBH2 && m < 2 * P - 1) continue;
        std::vector<zb_op> ops = build(order, P, m, unit);
        CHECK(!ops.empty());
        int bad = 0;
        CHECK(zb_schedule_validate(P, m, ops.data(), (int)ops.size(), &bad) == ZB_OK && bad == -1);
        std::vector<zb_op> lin(ops.size());
        std::vector<int64_t> s(ops.size()), e(ops.size());
        zb_sim_stats st;
        const int64_t t[3] = {2, 3, 1};
        CHECK(zb_schedule_simulate(P, m, ops.data(), (int)ops.size(), t, 1, lin.data(), s.data(), e.data(), &st) ==
              ZB_OK);
        for (int stage = 0; stage < P; ++stage) {
          int64_t peak = -1;
          CHECK(zb_schedule_peak_memory(ops.data(), (int)ops.size(), stage, 7, 5, &peak) == ZB_OK && peak >= 0);
        }
        // perturbations must be rejected or accepted, never crash
        for (int k = 0; k < 8 && !ops.empty(); ++k) {
          std::vector<zb_op> bad_ops = ops;
          const size_t i = rng() % bad_ops.size(), j = rng() % bad_ops.size();
          std::swap(bad_ops[i], bad_ops[j]);
          if (k % 3 == 0) bad_ops[i].mb = (int32_t)(rng() % (m + 2)) - 1;
          if (k % 4 == 1) bad_ops.pop_back();
          (void)zb_schedule_validate(P, m, bad_ops.data(), (int)bad_ops.size(), &bad);
        }
        if (order != ZB_ORDER_GPIPE && order != ZB_ORDER_1F1B) {
          std::vector<zb_op> h(3 * (size_t)P * m);
          int n = 0, choice = -1;
          zb_sim_stats hs;
          CHECK(zb_schedule_heuristic(P, m, t, 0, 10, 12, 2 * (int64_t)P * 10 + 2, h.data(), (int)h.size(), &n,
                                      &hs, &choice) == ZB_OK);
          std::vector<zb_op> v(6 * (size_t)P * m);
          CHECK(zb_schedule_zbv(P, m, unit, 0, 10, 12, 2 * (int64_t)P * 10 + 2, v.data(), (int)v.size(), &n, &hs) ==
                ZB_OK);
          // equal stashes and 2P of them per device: the zero-bubble search runs and succeeds when m >= 2P - 1
          CHECK(zb_schedule_zbv(P, m, unit, 0, 1, 1, 2 * (int64_t)P, v.data(), (int)v.size(), &n, &hs) == ZB_OK);
          CHECK(m < 2 * P - 1 || P > 8 || hs.bubble == 0);
        }
        if (m % P == 0) {
          zb_sim_stats is;
          CHECK(zb_schedule_simulate_interleaved(P, m, 2, unit, &is) == ZB_OK);
        }
      }
  // timed-event inspector on random events with random dependencies
  for (int trial = 0; trial < 2000; ++trial) {
    const int n = 1 + (int)(rng() % 40);
    std::vector<zb_event> ev(n);
    std::vector<std::vector<int32_t>> deps(n);
    for (int i = 0; i < n; ++i) {
      ev[i].id = (int32_t)(rng() % (2 * n));
      ev[i].stage = (int32_t)(rng() % 5) - 1;
      ev[i].micro = (int32_t)(rng() % 4);
      ev[i].kind = "FBWU?"[rng() % 5];
      ev[i].start = (double)(rng() % 20) - 1.0;
      ev[i].end = ev[i].start + (double)(rng() % 4) - 0.5;
      const int nd = (int)(rng() % 3);
      for (int d = 0; d < nd; ++d) deps[i].push_back((int32_t)(rng() % (2 * n + 2)));
      ev[i].n_deps = (int32_t)deps[i].size();
      ev[i].deps = deps[i].empty() ? nullptr : deps[i].data();
    }
    zb_event_report rep;
    int bad = 0;
    (void)zb_events_inspect(ev.data(), n, (int)(rng() % 4), &rep, &bad);
    CHECK(bad >= -1 && bad < n);
  }
}

struct Shape {
  const char* name;
  zb_stage_desc d;
  int P, order;
};

static void stage_layer() {
  // The workloads' stage shapes with their pipeline depth and handcrafted order.
  const Shape shapes[] = {
      {"tiny", {ZB_KIND_TINY_MLP, ZB_DTYPE_FP32, 1, 256, 1024, 0, 512, 1, 4, ZB_GELU_ERF, 0, 0}, 2, ZB_ORDER_ZBH1},
      {"gpt_mlp_h2048", {ZB_KIND_MLP_LINEARS, ZB_DTYPE_BF16, 4, 2048, 8192, 16, 1024, 1, 8, ZB_GELU_ERF, 0, 0}, 4,
       ZB_ORDER_ZBH1},
      {"gpt_full_h4096", {ZB_KIND_FULL, ZB_DTYPE_BF16, 4, 4096, 16384, 32, 2048, 1, 16, ZB_GELU_ERF, 0, 0}, 4,
       ZB_ORDER_ZBH1},
      {"gpt_full_h6144", {ZB_KIND_FULL, ZB_DTYPE_BF16, 2, 6144, 24576, 48, 1024, 2, 24, ZB_GELU_ERF, 0, 0}, 8,
       ZB_ORDER_ZBH2},
      {"gpt_full_s4096", {ZB_KIND_FULL, ZB_DTYPE_BF16, 4, 4096, 16384, 32, 4096, 1, 32, ZB_GELU_ERF, 0, 0}, 8,
       ZB_ORDER_ZBH2},
  };
  for (const Shape& sh : shapes) {
    for (int recompute = 0; recompute <= 1; ++recompute)
      for (int per_linear = 0; per_linear <= 1; ++per_linear) {
        zb_stage_desc d = sh.d;
        d.recompute_act = recompute;
        d.w_per_linear = per_linear;
        const int nlin = d.n_layers * (d.kind == ZB_KIND_TINY_MLP ? 2 : 4);
        // Device addresses that are stored, never dereferenced on the host.
        std::vector<const void*> w(nlin);
        std::vector<float*> dw(nlin);
        for (int i = 0; i < nlin; ++i) {
          w[i] = reinterpret_cast<const void*>((uintptr_t)(1ull << 40) + (uintptr_t)i * (1ull << 32));
          dw[i] = reinterpret_cast<float*>((uintptr_t)(1ull << 41) + (uintptr_t)i * (1ull << 32));
        }
        const int64_t unit[3] = {1, 1, 1};
        std::vector<zb_op> ops = build(sh.order, sh.P, d.n_micro, unit);
        CHECK(!ops.empty());
        std::vector<zb_stage*> st(sh.P, nullptr);
        for (int s = 0; s < sh.P; ++s) CHECK(zb_stage_create(&d, s, w.data(), dw.data(), nullptr, &st[s]) == ZB_OK);
        for (int s = 0; s < sh.P; ++s) {
          size_t fw = 0, fb = 0, bw = 0, bytes = 0;
          CHECK(zb_stage_class_bytes(st[s], &fw, &fb, &bw) == ZB_OK && fw > 0 && bw > 0);
          CHECK(zb_stage_workspace_bytes(st[s], ops.data(), (int)ops.size(), &bytes) == ZB_OK && bytes > 0);
          size_t all = 0;
          CHECK(zb_stage_workspace_bytes(st[s], nullptr, 0, &all) == ZB_OK && all >= bytes);
          CHECK(zb_stage_workspace_bytes(st[s], ops.data(), (int)ops.size(), &bytes) == ZB_OK);
          if (d.kind == ZB_KIND_FULL || d.kind == ZB_KIND_TINY_MLP) {
            // binding launches nothing for these kinds
            void* ws = reinterpret_cast<void*>((uintptr_t)(1ull << 45) + (uintptr_t)s * (1ull << 40));
            CHECK(zb_stage_bind_workspace(st[s], ws, bytes - 256) == ZB_E_BUDGET);
            CHECK(zb_stage_bind_workspace(st[s], reinterpret_cast<char*>(ws) + 8, bytes) == ZB_E_ARG);
            CHECK(zb_stage_bind_workspace(st[s], ws, bytes) == ZB_OK);
            void* slot = nullptr;
            for (int j = 0; j < d.n_micro; ++j) {
              zb_status rc = zb_stage_input_slot(st[s], j, &slot);
              CHECK(rc == ZB_OK || rc == ZB_E_BUDGET);
              rc = zb_stage_grad_slot(st[s], j, &slot);
              CHECK(rc == ZB_OK || rc == ZB_E_BUDGET);
            }
          }
          std::vector<void*> taps(d.n_micro, reinterpret_cast<void*>((uintptr_t)(1ull << 44)));
          CHECK(zb_stage_set_taps(st[s], taps.data(), nullptr) == ZB_OK);
          CHECK(zb_stage_set_taps(st[s], nullptr, nullptr) == ZB_OK);
          int nf = -1;
          CHECK(zb_grad_flush(st[s], &nf) == ZB_E_MISSING);
        }
        // a schedule with a pass moved before its producer is refused before any launch
        if (d.kind == ZB_KIND_FULL) {
          std::vector<zb_op> bad = ops;
          for (size_t i = 0; i < bad.size(); ++i)
            if (bad[i].kind == 'B') {
              zb_op b = bad[i];
              bad.erase(bad.begin() + (long)i);
              bad.insert(bad.begin(), b);
              break;
            }
          std::vector<void*> io(d.n_micro, reinterpret_cast<void*>((uintptr_t)(1ull << 43)));
          CHECK(zb_run_schedule(st.data(), sh.P, bad.data(), (int)bad.size(), io.data(), io.data(), io.data(),
                                io.data(), nullptr) != ZB_OK);
        }
        for (zb_stage* s : st) zb_stage_destroy(s);
      }
  }
}

int main() {
  std::mt19937 rng(20261202u);
  schedule_layer(rng);
  stage_layer();
  std::printf("host checks: %d failure(s)\n", g_fail);
  return g_fail == 0 ? 0 : 1;
}
