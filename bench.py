#!/usr/bin/env python3
"""Throughput of one zero-bubble pipeline stage's hot path on one MI355X.

A step is one whole schedule: every emulated stage's F, B and W passes for
every microbatch (the workload's handcrafted order by default), run through
zb_run_schedule with the emulated stages spread over two HIP streams (stages
2k and 2k+1 on stream k mod 2; --streams), then the step boundary
(zb_grad_flush) of every stage.  Inputs, weights and gradient buffers are
resident in HBM before timing starts.  The default workload is the largest
single-GPU one: 8 emulated stages of 4 full layers (h = 4096, 32 heads,
seq 4096), 32 microbatches, ZB-H2.  --order zb1p / zb2p runs the automatic
scheduler's order, built from pass times measured on this device and the
stages' own stash sizes, with 1F1B's activation budget or twice it; --order
zbv runs the model cut into 2P chunk stages in the V placement's order.

Reported value: stage F+B+W TFLOP/s = algorithmic GEMM (+ attention) FLOPs of
the step / wall time.  Also reported: % of the bf16 dense MFMA peak; the
split-backward overhead against the fused backward (1F1B order, unsplit
passes) with the same W kernel issued once per linear on both sides, and with
the split W pass grouped as it runs in the headline; the dominant kernel's
roofline; a planned-versus-observed join of one traced headline step; and the
fp64 CPU oracle's rate on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--order zbh1|zb1p|zb2p|zbv|...]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# Automatic orders: activation budget in units of P microbatches' stash (ZB-1p, ZB-2p).
HEURISTIC = {"zb1p": 1, "zb2p": 2}
# Secondary phases (one-stream passes, fused baseline, kernel timing) run a
# fixed number of steps whatever --steps is, so the whole run stays within a
# few minutes on the largest workload (about 5 s per step).
SHORT_STEP_MS = 500.0


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def gpu_step_flops(w) -> float:
    per_mb_stage = 3 * w.gemm_flops_per_pass() + w.attn_flops_fwd() + w.attn_flops_bwd()
    return float(per_mb_stage) * w.n_micro * w.n_stages


KERNEL_SOURCES = {
    # the files that define each kernel family's device code
    "gemm": ["split_backward_gemms_amd/csrc/gemm.hip", "split_backward_gemms_amd/csrc/device_common.h"],
    "attn": ["split_backward_gemms_amd/csrc/attention.hip", "split_backward_gemms_amd/csrc/device_common.h"],
    "other": ["split_backward_gemms_amd/csrc/elementwise.hip", "split_backward_gemms_amd/csrc/device_common.h"],
}


def sources_of(kernel: str):
    return KERNEL_SOURCES["gemm" if kernel.startswith("gemm") else "attn" if kernel.startswith("attn") else "other"]


def sources_sha16(srcs) -> str:
    import hashlib
    h = hashlib.sha256()
    for src in srcs:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    return h.hexdigest()[:16]


def pmc_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE / WRITE_SIZE, calibrated against a plain copy), or None
    when there is none or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"pmc_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    k = json.load(open(path))["kernels"].get(kernel)
    if k is None or k.get("source_sha256_16") != sources_sha16(k.get("source", [])):
        return None
    return k["hbm_bytes_per_launch"]


def cpu_baseline(w, budget_s: float = 12.0) -> dict:
    """The fp64 oracle (as it stands) on a bounded sample: F+B+W of whole
    layers of one stage and one microbatch at full size (one layer at a time
    for full layers, whose s x s attention probabilities the oracle keeps),
    repeated until budget_s elapses."""
    import numpy as np
    import synthetic_inputs as si
    from oracle import stage as ost
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    unit = w.replace(n_layers=1) if w.kind == si.FULL else w
    ws = ost.to64(si.stage_weights(unit, 0))
    x = si.stage_input(unit, 0).astype(np.float64)
    dy = si.last_stage_grad(unit, 0).astype(np.float64)
    units = 0
    t0 = time.perf_counter()
    while True:
        _, saved = ost.stage_forward(unit, ws, x)
        _, grads = ost.stage_backward_input(unit, ws, saved, dy)
        for sv in saved:
            sv.pop("probs", None)
        ost.stage_backward_weight(unit, saved, grads)
        units += 1
        el = time.perf_counter() - t0
        if el >= budget_s or units >= 8:
            break
    flops = units * (3 * unit.gemm_flops_per_pass() + unit.attn_flops_fwd() + unit.attn_flops_bwd())
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{units} x (F+B+W of {unit.n_layers} layer(s) of one stage, one microbatch) at full size "
                      f"(T={unit.tokens}, h={unit.hidden}), fp64 numpy, {el:.1f} s"}


def draw_inputs(w, threads: int = 8):
    import synthetic_inputs as si
    ws = [si.stage_weights(w, s) for s in range(w.n_stages)]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        xs = list(ex.map(lambda j: si.stage_input(w, j), range(w.n_micro)))
        dys = list(ex.map(lambda j: si.last_stage_grad(w, j), range(w.n_micro)))
    return ws, xs, dys


def roofline_of(kern, workload: str) -> dict:
    """The dominant kernel (largest total time) against the MFMA peak when its
    algorithmic intensity is above the ridge point, against HBM otherwise."""
    top = kern[0]
    avg_ms = top["total_ms"] / top["launches"]
    per_launch_flops = top["flops"] / top["launches"]
    per_launch_bytes = top["bytes"] / top["launches"]
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    intensity = per_launch_flops / per_launch_bytes if per_launch_bytes > 0 else float("inf")
    if intensity >= ridge:
        achieved = per_launch_flops / (avg_ms / 1e3) / 1e12
        r = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
             "frac": achieved / PEAK_BF16_TFLOPS}
    else:
        achieved = per_launch_bytes / (avg_ms / 1e3) / 1e9
        r = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": achieved / PEAK_HBM_GBS}
    r.update({"traffic": pmc_traffic(workload, top["name"]), "kernel": top["name"],
              "avg_launch_us": avg_ms * 1e3, "flops_per_launch": per_launch_flops,
              "bytes_per_launch": per_launch_bytes, "flop_per_byte": intensity, "ridge": ridge,
              "tflops": per_launch_flops / (avg_ms / 1e3) / 1e12,
              "measured_on": "one stream, hipEvent pair per launch on the launch's stream"})
    return r


class ClockSampler:
    """Samples the GPU's GFX clocks with `amd-smi metric -g 0 -c` (a child process, about three
    times a second) on a background thread while a timed region runs.  Reports the mean of the
    per-sample means over the eight XCDs, or None where the tool is missing or prints no clock."""

    def __init__(self):
        import threading

        self.means, self._stop = [], threading.Event()
        self._thread = threading.Thread(target=self._loop, daemon=True)

    @staticmethod
    def _sample():
        import re
        import subprocess

        try:
            out = subprocess.run(["amd-smi", "metric", "-g", "0", "-c"], capture_output=True, text=True,
                                 timeout=10).stdout
        except (OSError, subprocess.SubprocessError):
            return None
        clocks, in_gfx = [], False
        for line in out.splitlines():
            if re.match(r"\s+GFX_\d+:", line):
                in_gfx = True
                continue
            m = re.match(r"\s+CLK: (\d+) MHz", line)
            if m and in_gfx:
                clocks.append(int(m.group(1)))
                in_gfx = False
            elif re.match(r"\s+[A-Z]+_?\d*:$", line):
                in_gfx = False
        return sum(clocks) / len(clocks) if clocks else None

    def _loop(self):
        while not self._stop.is_set():
            v = self._sample()
            if v is None:
                return
            self.means.append(v)
            self._stop.wait(0.2)

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join(timeout=15)
        return False

    def report(self):
        if len(self.means) < 9:  # under ~2 s of samples: too few to stand for the timed region
            return None
        m = self.means[1:]  # the first sample can predate the load
        return {"mean": sum(m) / len(m), "min_sample": min(m), "max_sample": max(m), "samples": len(m),
                "source": "amd-smi metric -g 0 -c during the timed steps; mean of the eight XCDs' GFX clocks"}


def counter_run(w0, a) -> int:
    """One full-size stage of the workload, two microbatches, two steps, one stream."""
    import torch

    import split_backward_gemms_amd as zb
    import synthetic_inputs as si
    from split_backward_gemms_amd.pipeline import EmulatedPipeline, upload

    w = w0.replace(n_stages=1, n_micro=2)
    torch.cuda.set_device(0)
    ws = [si.stage_weights(w, 0)]
    X = [upload(si.stage_input(w, j), w.dtype, "cuda:0") for j in range(2)]
    DY = [upload(si.last_stage_grad(w, j), w.dtype, "cuda:0") for j in range(2)]
    ops = [(0, "F", 0), (0, "F", 1), (0, "B", 0), (0, "B", 1), (0, "W", 0), (0, "W", 1)]
    pipe = EmulatedPipeline(w, ws, ops=ops, device="cuda:0", recompute_act=a.recompute_act)
    y, dx = pipe.io_buffers()
    log(f"counter run {w.name}: one stage, 2 microbatches, recompute_act={pipe.recompute_act}")
    zb.zb_prof_reset()
    for step in range(2):
        zb.zb_prof_enable(step == 1)
        pipe.run(ops, X, DY, y, dx)
        torch.cuda.synchronize()
    zb.zb_prof_enable(False)
    kern = sorted(zb.zb_prof_read(), key=lambda r: -r["total_ms"])
    zb.zb_prof_reset()
    pipe.close()
    print(json.dumps({"mode": "counters", "workload": w0.name, "recompute_act": pipe.recompute_act,
                      "kernels": [{"name": r["name"], "launches": r["launches"],
                                   "avg_us": 1e3 * r["total_ms"] / r["launches"],
                                   "flops_per_launch": r["flops"] / r["launches"],
                                   "bytes_per_launch": r["bytes"] / r["launches"]} for r in kern]}), flush=True)
    return 0


def sustained_run(a) -> int:
    """One GEMM kind at n x n x n (bf16 operands) for a fixed wall time, back to back on one
    stream: the library's F (store epilogue), B or W (fp32 accumulate, one launch) through the
    C ABI, or torch.matmul (hipBLASLt) for reference.  Run beside a clock sampler (amd-smi) it
    shows the clock the chip sustains under each dense load, and so the peak at that clock."""
    import torch

    import split_backward_gemms_amd as zb

    n, kind = a.size, a.kind
    torch.cuda.set_device(0)
    g = torch.Generator(device="cuda:0").manual_seed(1)
    x = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16, generator=g)
    w = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16, generator=g)
    y = torch.empty(n, n, device="cuda:0", dtype=torch.bfloat16)
    dw = torch.zeros(n, n, device="cuda:0", dtype=torch.float32) if kind == "W" else None

    def one():
        if kind == "F":
            zb.zb_linear_forward(x, w, y)
        elif kind == "B":
            zb.zb_linear_backward_input(x, w, y)
        elif kind == "W":
            zb.zb_linear_backward_weight(x, w, dw, True)
        else:
            torch.matmul(x, w, out=y)

    one()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    calls, t0 = 0, time.perf_counter()
    e0.record()
    while time.perf_counter() - t0 < a.seconds:
        for _ in range(20):
            one()
        calls += 20
        torch.cuda.synchronize()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / calls
    print(json.dumps({"mode": "sustained", "kind": kind, "size": n, "calls": calls, "ms_per_call": ms,
                      "tflops": 2.0 * n ** 3 / (ms * 1e-3) / 1e12}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=12)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gpt_full_s4096")
    ap.add_argument("--order", default=None)
    ap.add_argument("--streams", type=int, default=2,
                    help="HIP streams the emulated stages are spread over (stages 2k, 2k+1 on stream k mod n; "
                         "2 measured fastest on every workload, P gives one per stage)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-fused", action="store_true")
    ap.add_argument("--no-optim", action="store_true",
                    help="skip timing the optimizer step with post-update validation")
    ap.add_argument("--mode", choices=["full", "kernels", "counters", "sustained"], default="full",
                    help="kernels: only the one-stream kernel-timing phase (the phase a kernel profile covers); "
                         "counters: one full-size stage of the workload with two microbatches (F, F, B, B, W, W), "
                         "two steps: the same kernels at the same shapes for counter passes, in a few GiB; "
                         "sustained: one GEMM kind (--kind) back to back for --seconds")
    ap.add_argument("--kind", choices=["F", "B", "W", "matmul"], default="F",
                    help="sustained mode: the library's F, B or W GEMM, or torch.matmul (hipBLASLt)")
    ap.add_argument("--size", type=int, default=8192, help="sustained mode: n of the n x n x n product")
    ap.add_argument("--seconds", type=float, default=15.0, help="sustained mode: wall time of the loop")
    ap.add_argument("--recompute-act", type=int, choices=[0, 1], default=None,
                    help="stash layout (zb_stage_desc.recompute_act); default: stash A when it fits")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run one plain device-to-device copy kernel of BYTES bytes (counter calibration)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py: this build measures one GPU's share of the pipeline only; --gpus {a.gpus} is not "
              f"supported (the pipeline stages are emulated on one device, and no run here uses a second GPU).",
              file=sys.stderr)
        return 2
    if a.mode == "sustained":
        if a.size < 8 or a.size % 8 or 4.0 * a.size * a.size >= 2147483648.0:
            print("bench.py: --size must be a multiple of 8 with a dW below 2 GiB", file=sys.stderr)
            return 2
        return sustained_run(a)
    if a.calibrate_copy:
        import torch
        n = a.calibrate_copy // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": 4 * n}))
        return 0

    import torch

    import split_backward_gemms_amd as zb
    import synthetic_inputs as si
    from split_backward_gemms_amd import tracing
    from split_backward_gemms_amd.pipeline import (EmulatedPipeline, heuristic_ops, pass_times_us,
                                                   stash_per_microbatch, upload, zbv_ops)

    w0 = si.WORKLOADS[a.workload]
    if a.mode == "counters":
        return counter_run(w0, a)
    order = a.order or w0.order
    # ZB-V runs the same model cut into 2P chunk stages of half the layers.
    w = si.v_chunks(w0) if order == "zbv" else w0
    n_dev = w0.n_stages
    dev = "cuda:0"
    torch.cuda.set_device(0)
    log(f"workload {w.name}: P={w.n_stages} m={w.n_micro} layers={w.n_layers} h={w.hidden} T={w.tokens} {order}")
    t0 = time.perf_counter()
    ws, xs, dys = draw_inputs(w)
    log(f"inputs drawn in {time.perf_counter() - t0:.1f} s")

    P, m = w.n_stages, w.n_micro
    hand = w0.order if order in HEURISTIC else ("zbh1" if order == "zbv" else order)
    ops, sim = zb.zb_schedule_build(hand, P, m)
    ops_fused, _ = zb.zb_schedule_build("1f1b", P, m)
    X = [upload(x, w.dtype, dev) for x in xs]
    DY = [upload(d, w.dtype, dev) for d in dys]
    del xs, dys
    flops = gpu_step_flops(w)
    torch.cuda.synchronize()

    step_ev_ms = []

    def timed(pipe, o, steps, warmup):
        # Wall time over `steps` back-to-back steps, synchronised only at both
        # ends.  Each step also closes with a hipEvent on the caller's stream,
        # which every stage stream joins at the end of a step: per-step times
        # for the median and minimum, without a host wait between steps.
        for _ in range(warmup):
            pipe.run(o, X, DY, y, dx)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        t = time.perf_counter()
        ev[0].record()
        for i in range(steps):
            pipe.run(o, X, DY, y, dx)
            ev[i + 1].record()
        torch.cuda.synchronize()
        step_ev_ms[:] = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
        return 1000.0 * (time.perf_counter() - t) / max(1, steps)

    def traced(pipe, o):
        torch.cuda.synchronize()
        t = time.perf_counter()
        tr, _ = pipe.run(o, X, DY, y, dx, trace=True)
        torch.cuda.synchronize()
        return tr, 1000.0 * (time.perf_counter() - t)

    heur = {}
    if order in HEURISTIC or order == "zbv":
        # The automatic scheduler and ZB-V take the passes' measured times (one
        # stream, hipEvents) and the stages' own stash sizes.
        probe = EmulatedPipeline(w, ws, ops=ops, device=dev)
        y, dx = probe.io_buffers()
        probe.run(ops, X, DY, y, dx)
        tr, _ = probe.run(ops, X, DY, y, dx, trace=True)
        times = pass_times_us(tr)
        if order == "zbv":
            ops, hstats, m_limit = zbv_ops(probe.handles, m, times)
            choice = None
        else:
            ops, hstats, choice, m_limit = heuristic_ops(probe.handles, P, m, times, HEURISTIC[order] * P)
        sim = hstats
        heur = {"pass_us": times, "m_limit_bytes": m_limit, "fill_balance": choice,
                "sim_bubble_us": hstats["bubble"], "sim_makespan_us": hstats["makespan"]}
        log(f"{order}: pass times {times} us, M_limit {m_limit / 2**30:.2f} GiB per device, choice {choice}, "
            f"simulated bubble {hstats['bubble']} of {hstats['makespan']} us")
        probe.close()
        del probe, y, dx, tr
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    out_extra = {}
    ms_per_step = tflops = float("nan")
    if a.mode == "full":
        # Headline: the emulated stages spread over a few HIP streams, so independent
        # stages overlap the way pipeline stages on separate devices would.
        pipe = EmulatedPipeline(w, ws, ops=ops, device=dev, stage_streams=True, n_streams=a.streams)
    else:
        pipe = EmulatedPipeline(w, ws, ops=ops, device=dev)
    del ws
    y, dx = pipe.io_buffers()
    torch.cuda.synchronize()
    log(f"device ready: workspace {pipe.workspace_bytes() / 2**30:.2f} GiB, "
        f"{'A rebuilt for W' if pipe.recompute_act else 'A stashed'}")
    t_split = {}
    sim_measured = {}
    join = None
    if a.mode == "full":
        with ClockSampler() as clk:
            ms_per_step = timed(pipe, ops, a.steps, a.warmup)
        tflops = flops / (ms_per_step / 1000.0) / 1e12
        clock = clk.report()
        out_extra["gfx_clock_mhz"] = clock
        if clock is not None:
            # the published bf16 dense peak assumes the 2400 MHz maximum clock
            at_clock = PEAK_BF16_TFLOPS * clock["mean"] / 2400.0
            out_extra["bf16_peak_at_sampled_clock_tflops"] = at_clock
            out_extra["pct_of_bf16_peak_at_sampled_clock"] = 100.0 * tflops / at_clock
        ev_steps = sorted(step_ev_ms)
        out_extra["step_ms_median"] = ev_steps[len(ev_steps) // 2] if ev_steps else None
        out_extra["step_ms_min"] = ev_steps[0] if ev_steps else None
        log(f"{order}, {min(a.streams, P)} streams: {ms_per_step:.3f} ms/step, {tflops:.1f} TFLOP/s")
        short = ms_per_step < SHORT_STEP_MS
        tr_multi, _ = traced(pipe, ops)
        stream_of_stage = pipe.stream_index_of_stage()
        if short and not a.no_fused:
            pipe.plan(ops_fused)
            fms = timed(pipe, ops_fused, max(2, a.steps // 2), 1)
            out_extra["ms_per_step_1f1b_unsplit"] = fms
            out_extra["zb_vs_1f1b_speedup"] = fms / ms_per_step - 1.0
            log(f"1f1b unsplit, {min(a.streams, P)} streams: {fms:.3f} ms/step")

        # One shared stream: passes run in isolation, for per-pass times, the
        # split overhead and the plan's durations.
        pipe.rebuild(ops, stage_streams=False)
        reps = 2 if short else 1
        if short:
            timed(pipe, ops, 0, 1)
        tr_one, wall_one = traced(pipe, ops)
        t_split = {k: sum(ms for (op, ms, _) in tr_one if op[1] == k) for k in "FBW"}
        log(f"{order}, one stream: {wall_one:.1f} ms/step; passes {t_split}")
        join = tracing.join(ops, P, stream_of_stage, tr_multi, tracing.median_durations(tr_one))
        log(f"plan vs observed ({join['streams']} streams): span {join['planned_span_ms']:.1f} planned, "
            f"{join['observed_span_ms']:.1f} observed; dependency wait {join['dependency_wait_ms']}, "
            f"resource wait {join['resource_wait_ms']}")
        # Bubble rates the simulator gives across P devices at these measured
        # pass times (a ZB-V chunk counts as half a stage, in time and stash).
        if any(k in ("B", "W") for (_, k, _) in ops):
            times = pass_times_us(tr_one)
            cut = 2 if order == "zbv" else 1
            st_times = tuple(cut * x for x in times)
            ch_times = times if order == "zbv" else tuple(max(1, x // 2) for x in times)
            m_b, m_w = (cut * v for v in stash_per_microbatch(pipe.handles))
            for nm in ["1f1b", "zbh1"] + (["zbh2"] if m >= 2 * n_dev - 1 else []):
                st = zb.zb_schedule_build(nm, n_dev, m, st_times)[1]
                sim_measured[nm] = st["bubble"] / st["makespan"]
            for nm, k in HEURISTIC.items():
                st = zb.zb_schedule_heuristic(n_dev, m, st_times, m_b, m_w, k * n_dev * m_b + max(0, m_w - m_b))[1]
                sim_measured[nm] = st["bubble"] / st["makespan"]
            cb, cw = m_b // 2, m_w // 2
            st = zb.zb_schedule_zbv(n_dev, m, ch_times, cb, cw, 2 * n_dev * cb + max(0, cw - cb))[1]
            sim_measured["zbv"] = st["bubble"] / st["makespan"]
            log(f"simulated bubble rates at measured pass times {times} us: "
                + ", ".join(f"{k} {100 * v:.1f}%" for k, v in sim_measured.items()))

        if not a.no_fused and t_split.get("B", 0) > 0:
            # Split overhead, like for like: the W pass issues one launch per linear,
            # exactly as the fused backward does (same kernel, same launches).
            pipe.rebuild(ops, stage_streams=False, w_per_linear=1)
            if short:
                timed(pipe, ops, 0, 1)
            tr_pl, wall_pl = traced(pipe, ops)
            t_pl = {k: sum(ms for (op, ms, _) in tr_pl if op[1] == k) for k in "FBW"}
            pipe.rebuild(ops_fused, stage_streams=False, w_per_linear=0)
            timed(pipe, ops_fused, 0, 1)
            tr_fu, wall_fu = traced(pipe, ops_fused)
            t_fu = {k: sum(ms for (op, ms, _) in tr_fu if op[1] == k) for k in "FU"}
            out_extra.update({
                "split_overhead_pass": (t_pl["B"] + t_pl["W"]) / t_fu["U"] - 1.0,
                "split_overhead_pass_grouped_w": (t_split["B"] + t_split["W"]) / t_fu["U"] - 1.0,
                "split_overhead_wall_one_stream": wall_pl / wall_fu - 1.0,
                "split_overhead_wall_one_stream_grouped_w": wall_one / wall_fu - 1.0,
                "ms_per_step_one_stream": wall_one,
                "ms_per_step_one_stream_w_per_linear": wall_pl,
                "ms_per_step_1f1b_unsplit_one_stream": wall_fu,
                "pass_ms_w_per_linear": t_pl,
                "pass_ms_1f1b": {"F": t_fu["F"], "U": t_fu["U"]},
                "split_overhead_definition": "sum(t_B + t_W) of the split order / sum(t_U) of 1F1B's fused "
                                             "backwards - 1, per-pass hipEvents on one stream; W issued with the "
                                             "same kernel, one launch per linear, on both sides "
                                             "(_grouped_w: the split W pass as one grouped launch)"})
            log(f"split overhead (B+W vs U, same W launches): {100 * out_extra['split_overhead_pass']:.2f}%, "
                f"grouped W {100 * out_extra['split_overhead_pass_grouped_w']:.2f}%; wall one stream "
                f"{wall_pl:.1f} / {wall_one:.1f} (grouped) vs {wall_fu:.1f} ms")
            pipe.rebuild(ops, stage_streams=False, w_per_linear=0)
    if a.mode != "full":
        pipe.run(ops, X, DY, y, dx)  # one untimed step before the kernel-timing phase

    # Kernel-level timing over one profiled step of the measured order (one stream).
    zb.zb_prof_reset()
    zb.zb_prof_enable(True)
    prof_steps = 1
    for _ in range(prof_steps):
        pipe.run(ops, X, DY, y, dx)
    torch.cuda.synchronize()
    zb.zb_prof_enable(False)
    kern = zb.zb_prof_read()
    zb.zb_prof_reset()
    kern.sort(key=lambda r: -r["total_ms"])
    for r in kern[:12]:
        log(f"  {r['name']:<28} {r['launches']:6d} launches {r['total_ms'] / prof_steps:8.3f} ms/step "
            f"{r['flops'] / r['total_ms'] / 1e9:8.1f} TFLOP/s")
    gemm_ms = sum(r["total_ms"] for r in kern if r["name"].startswith("gemm")) / prof_steps
    gemm_flops = sum(r["flops"] for r in kern if r["name"].startswith("gemm")) / prof_steps
    roofline = roofline_of(kern, w0.name)
    kernels = [{"name": r["name"], "launches_per_step": r["launches"] / prof_steps,
                "ms_per_step": r["total_ms"] / prof_steps,
                "tflops": r["flops"] / r["total_ms"] / 1e9} for r in kern]

    # Optimizer step with post-update validation (outside the step above), where
    # the moments fit beside the stash.
    optim = None
    n_params = sum(int(t.numel()) for ws_ in pipe.weights for t in ws_)
    if a.mode == "full" and not a.no_optim and 12 * n_params * 1.25 < torch.cuda.mem_get_info()[0]:
        def ev_ms(fn):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1)
        res = {}
        for name, max_norm in (("no_rollback", 1e30), ("rollback", 1e-30)):
            pipe.optim_init(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_grad_norm=max_norm)
            pipe.run(ops, X, DY, y, dx)
            torch.cuda.synchronize()
            step_ms = ev_ms(lambda: pipe.optim_step(1))
            val_ms = ev_ms(lambda: pipe.optim_validate(1))
            rolled = int(pipe.rolled.sum().item())
            res[name] = {"step_ms": step_ms, "validate_ms": val_ms, "stages_rolled_back": rolled}
        step_bytes = 30.0 * n_params if w.dtype == "bf16" else 32.0 * n_params
        optim = {"params": n_params, "bytes_per_update": step_bytes, **res,
                 "step_gbs": step_bytes / (res["no_rollback"]["step_ms"] / 1e3) / 1e9}
        log(f"optimizer: {n_params / 1e6:.0f} M params, step {res['no_rollback']['step_ms']:.2f} ms "
            f"({optim['step_gbs']:.0f} GB/s), validate {res['no_rollback']['validate_ms']:.3f} ms, "
            f"with rollback {res['rollback']['validate_ms']:.2f} ms ({res['rollback']['stages_rolled_back']} stages)")

    recompute_act = pipe.recompute_act
    pipe.close()
    out = {
        "metric": "stage F+B+W TFLOP/s",
        "value": tflops if a.mode == "full" else None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step if a.mode == "full" else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w0.name, "devices": n_dev, "stages_emulated": w.n_stages, "n_micro": w.n_micro,
                   "layers_per_stage": w.n_layers, "hidden": w.hidden, "ffn": w.ffn, "heads": w.n_heads,
                   "seq": w.seq, "micro_batch": w.micro_batch, "order": order,
                   "executor": (f"{P} HIP streams, one per stage" if a.streams >= P else
                                f"{a.streams} HIP streams, stages 2k, 2k+1 on stream k mod {a.streams}"),
                   "recompute_act": recompute_act, "flops_per_step": flops},
        "pct_of_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS if a.mode == "full" else None,
        "gemm_only_tflops": gemm_flops / (gemm_ms / 1e3) / 1e12 if gemm_ms > 0 else None,
        "gemm_only_pct_of_peak": 100.0 * gemm_flops / (gemm_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS if gemm_ms > 0 else None,
        "pass_ms": t_split,
        "sim_bubble_unit_times": {hand: zb.zb_schedule_build(hand, n_dev, m)[1]["bubble"],
                                  "1f1b": zb.zb_schedule_build("1f1b", n_dev, m)[1]["bubble"]},
        "sim_bubble_rate_measured_times": sim_measured,
        "roofline": roofline,
        "kernels": kernels,
    }
    out.update(out_extra)
    if join:
        out["plan_vs_observed"] = join
    if optim:
        out["optimizer"] = optim
    if heur:
        out["heuristic"] = heur
    if not a.no_cpu and a.mode == "full":
        log("timing the CPU oracle sample ...")
        out["cpu_baseline"] = cpu_baseline(w0)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
