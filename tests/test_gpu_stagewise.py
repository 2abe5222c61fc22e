"""GPU parity stage by stage: every emulated stage's output Y, input gradient
dX and flushed dW against the fp64 oracle run on that stage's own inputs.

The executor hands stage s's output straight to stage s+1 and stage s+1's input
gradient back to stage s.  With boundary taps (zb_stage_set_taps) the test
reads every stage's bf16 output and input gradient, then runs the oracle one
stage at a time: stage s forward on the GPU's output of stage s-1 (the seeded
input on stage 0), backward on the GPU's input gradient of stage s+1 (the
seeded upstream gradient on the last stage).  Each stage's tensors then meet
|gpu - ref| <= 2e-2 * max|ref| per tensor at any pipeline depth, as the
per-stage checksums of "Zero-Bubble Pipeline Parallelism, Proven" (section
"Split backward without changing the update") would locate the first
divergent stage and pass.

Cases: the structures of the P = 8 workloads (ZB-H2 with m = 24 and m = 32,
two layers of h = 6144 and four of h = 4096 in the full-size runs) at reduced
width with ragged sequence lengths, through the two-stream executor (stages
2k, 2k+1 on stream k mod 2); the 4-stage, 4-layer full-layer structure at
full depth in ZB-H1 with m = 16; one full-size layer of the h = 4096, seq 2048
workload with two microbatches against the oracle, and the whole full-size
4-layer stage with two microbatches against the fp32 sum of single-microbatch
runs (the fp32 accumulation of W across microbatches at full shapes); and at
P = 8 devices, the orders searched at run time (the automatic scheduler at two
budgets, the V placement over 16 chunk stages), each bit-identical to 1F1B.
"""
import numpy as np
import pytest
import torch

import split_backward_gemms_amd as zb
import synthetic_inputs as si
from oracle import stage as ost
from split_backward_gemms_amd.pipeline import EmulatedPipeline, heuristic_ops, upload, zbv_ops

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    scale = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(gpu.astype(np.float64) - ref))) / (scale if scale > 0 else 1.0)


def _host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def _run_tapped(w, order, n_streams):
    """Runs one step of `order` with every stage tapped; returns the host copies
    of each stage's output and input gradient, the flushed dW, the last stage's
    outputs and the first stage's input gradients, and the inputs."""
    ws = [si.stage_weights(w, s) for s in range(w.n_stages)]
    xs = [si.stage_input(w, j) for j in range(w.n_micro)]
    dys = [si.last_stage_grad(w, j) for j in range(w.n_micro)]
    ops = zb.zb_schedule_build(order, w.n_stages, w.n_micro)[0] if isinstance(order, str) else order
    pipe = EmulatedPipeline(w, ws, ops=ops, stage_streams=n_streams is not None, n_streams=n_streams,
                            recompute_act=0)
    shape, dt = (w.tokens, w.hidden), torch.bfloat16
    ytap = [[torch.empty(shape, dtype=dt, device="cuda") for _ in range(w.n_micro)] for _ in range(w.n_stages)]
    dxtap = [[torch.empty(shape, dtype=dt, device="cuda") for _ in range(w.n_micro)] for _ in range(w.n_stages)]
    pipe.set_taps(ytap, dxtap)
    X = [upload(x, w.dtype, "cuda") for x in xs]
    DY = [upload(d, w.dtype, "cuda") for d in dys]
    y, dx = pipe.io_buffers()
    torch.cuda.synchronize()
    pipe.run(ops, X, DY, y, dx)
    torch.cuda.synchronize()
    out = {"y": [[_host(t) for t in row] for row in ytap], "dx": [[_host(t) for t in row] for row in dxtap],
           "dw": pipe.grads_host(), "y_last": [_host(t) for t in y], "dx0": [_host(t) for t in dx]}
    pipe.set_taps(None, None)
    pipe.close()
    del pipe, ytap, dxtap, X, DY, y, dx
    torch.cuda.empty_cache()
    return out, ws, xs, dys


def _stagewise_errors(w, got, ws, xs, dys):
    """Oracle of every stage on the GPU's own stage inputs; per-tensor errors."""
    P, m = w.n_stages, w.n_micro
    errs = {}
    for s in range(P):
        w64 = ost.to64(ws[s])
        dw_ref = None
        for j in range(m):
            x_in = (xs[j] if s == 0 else got["y"][s - 1][j]).astype(np.float64)
            dy_in = (dys[j] if s == P - 1 else got["dx"][s + 1][j]).astype(np.float64)
            y_ref, saved = ost.stage_forward(w, w64, x_in)
            dx_ref, grads = ost.stage_backward_input(w, w64, saved, dy_in)
            for sv in saved:
                sv.pop("probs", None)
            dw_j = ost.stage_backward_weight(w, saved, grads)
            dw_ref = dw_j if dw_ref is None else ost.add_grads(dw_ref, dw_j)
            errs[f"Y[{s},{j}]"] = _rel_err(got["y"][s][j], y_ref)
            errs[f"dX[{s},{j}]"] = _rel_err(got["dx"][s][j], dx_ref)
        for l in range(w.n_layers):
            for nm in dw_ref[l]:
                errs[f"dW[{s}].{l}.{nm}"] = _rel_err(got["dw"][s][l][nm], dw_ref[l][nm])
    return errs


def _check_stagewise(w, order, n_streams, got=None):
    print(f"stagewise {w.name}: P={w.n_stages} m={w.n_micro} L={w.n_layers} h={w.hidden} T={w.tokens} "
          f"{order if isinstance(order, str) else 'searched order'} streams={n_streams}", flush=True)
    if got is None:
        got, ws, xs, dys = _run_tapped(w, order, n_streams)
    else:
        got, ws, xs, dys = got
    # The taps hold exactly what the executor handed on: the last stage's
    # outputs and the first stage's input gradients are the same bits.
    for j in range(w.n_micro):
        assert np.array_equal(got["y"][w.n_stages - 1][j], got["y_last"][j])
        assert np.array_equal(got["dx"][0][j], got["dx0"][j])
    errs = _stagewise_errors(w, got, ws, xs, dys)
    worst = max(errs, key=errs.get)
    print(f"worst {worst} {errs[worst]:.3e} over {len(errs)} tensors", flush=True)
    assert errs[worst] <= TOL, (worst, errs[worst])


# Reduced-width structures of the P = 8 workloads, ragged against the 128-row
# attention blocks and the GEMM tiles.
STAGEWISE = {
    # h=6144 workload's structure: 2 layers, 2 sequences per microbatch, m = 24, ZB-H2
    "p8_m24_two_layers_two_seqs": (si.reduced(si.WORKLOADS["gpt_full_h6144"], hidden=256, heads=2, seq=136,
                                              n_micro=24, n_stages=8, n_layers=2), "zbh2"),
    # seq-4096 workload's structure: 4 layers, m = 32, ZB-H2
    "p8_m32_four_layers": (si.reduced(si.WORKLOADS["gpt_full_s4096"], hidden=256, heads=2, seq=264,
                                      n_micro=32, n_stages=8, n_layers=4), "zbh2"),
    # the h=4096, seq 2048 workload's structure at full depth: 4 stages x 4 layers, m = 16, ZB-H1
    "p4_m16_full_depth": (si.reduced(si.WORKLOADS["gpt_full_h4096"], hidden=256, heads=2, seq=200,
                                     n_micro=16, n_stages=4, n_layers=4), "zbh1"),
    # MLP-linears structure at P = 8 in ZB-H2 (identity attention)
    "p8_m16_mlp_linears": (si.reduced(si.WORKLOADS["gpt_mlp_h2048"], hidden=200, seq=104, n_micro=16,
                                      n_stages=8, n_layers=2).replace(ffn=328), "zbh2"),
}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(STAGEWISE))
def test_stagewise_two_streams_matches_oracle(name):
    w, order = STAGEWISE[name]
    _check_stagewise(w, order, 2)


@pytest.mark.timeout(900)
def test_stagewise_one_stream_per_stage_p8():
    """One HIP stream per stage at P = 8 (eight concurrent stage streams)."""
    w, order = STAGEWISE["p8_m24_two_layers_two_seqs"]
    _check_stagewise(w, order, 8)


@pytest.mark.timeout(900)
def test_p8_zbh2_streams_bitwise_equal_one_stream():
    """At P = 8, ZB-H2, m = 24: the two-stream executor (stages 0,1,4,5 and
    2,3,6,7 sharing streams) and one stream per stage give the bits of one
    shared stream, for the taps, the outputs and every flushed dW."""
    w, order = STAGEWISE["p8_m24_two_layers_two_seqs"]
    base, _, _, _ = _run_tapped(w, order, None)
    for n_streams in (2, 8):
        got, _, _, _ = _run_tapped(w, order, n_streams)
        for key in ("y", "dx"):
            for s in range(w.n_stages):
                for j in range(w.n_micro):
                    assert np.array_equal(got[key][s][j], base[key][s][j]), (n_streams, key, s, j)
        for s in range(w.n_stages):
            for l in range(w.n_layers):
                for nm in got["dw"][s][l]:
                    assert np.array_equal(got["dw"][s][l][nm].view(np.uint32),
                                          base["dw"][s][l][nm].view(np.uint32)), (n_streams, s, l, nm)


def _full_size_run(w, xs, dys, ws):
    ops = [(0, "F", j) for j in range(w.n_micro)] + [(0, "B", j) for j in range(w.n_micro)] + \
          [(0, "W", j) for j in range(w.n_micro)]
    pipe = EmulatedPipeline(w, ws, ops=ops, recompute_act=0)
    X = [upload(x, "bf16", "cuda") for x in xs]
    DY = [upload(d, "bf16", "cuda") for d in dys]
    y, dx = pipe.io_buffers()
    pipe.run(ops, X, DY, y, dx)
    torch.cuda.synchronize()
    got = {"y": [[_host(t) for t in y]], "dx": [[_host(t) for t in dx]], "dw": pipe.grads_host()}
    pipe.close()
    del pipe, X, DY, y, dx
    torch.cuda.empty_cache()
    return got


@pytest.mark.timeout(900)
def test_full_size_layer_two_microbatches_matches_oracle():
    """One full-size layer of the h = 4096, 32-head, seq 2048 workload with two
    microbatches (F, F, B, B, W, W): every GEMM and attention launch at its full
    shape, and the flushed dW is the fp32 sum of both microbatches' W, against
    the oracle's fp64 sum."""
    w = si.WORKLOADS["gpt_full_h4096"].replace(n_micro=2, n_stages=1, n_layers=1)
    print(f"full-size layer {w.name}: h={w.hidden} T={w.tokens} m={w.n_micro}", flush=True)
    ws = [si.stage_weights(w, 0)]
    xs = [si.stage_input(w, j) for j in range(w.n_micro)]
    dys = [si.last_stage_grad(w, j) for j in range(w.n_micro)]
    got = _full_size_run(w, xs, dys, ws)
    errs = _stagewise_errors(w, got, ws, xs, dys)
    worst = max(errs, key=errs.get)
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert errs[worst] <= TOL, (worst, errs[worst])


@pytest.mark.timeout(900)
def test_full_size_stage_accumulates_microbatches_exactly():
    """A whole full-size stage (4 layers, h = 4096, seq 2048) with two
    microbatches: each microbatch's Y and dX are the bits of a step holding that
    microbatch alone, and the flushed dW is exactly the fp32 sum of the two
    single-microbatch dW (the first W of a step stores its sum, the second adds
    its own sum to it once).  This holds at any depth, where a comparison with
    the fp64 oracle does not: without normalisation the residual stream of this
    workload grows about fivefold per layer, and by the fourth layer the
    attention logits are so large that rounding Q and K to bf16 alone moves
    softmax probabilities by up to 0.99."""
    w2 = si.WORKLOADS["gpt_full_h4096"].replace(n_micro=2, n_stages=1)
    w1 = w2.replace(n_micro=1)
    print(f"full-size stage {w2.name}: L={w2.n_layers} h={w2.hidden} T={w2.tokens} m=2 vs 2 x m=1", flush=True)
    ws = [si.stage_weights(w2, 0)]
    xs = [si.stage_input(w2, j) for j in range(2)]
    dys = [si.last_stage_grad(w2, j) for j in range(2)]
    both = _full_size_run(w2, xs, dys, ws)
    alone = [_full_size_run(w1, [xs[j]], [dys[j]], ws) for j in range(2)]
    for j in range(2):
        assert np.array_equal(both["y"][0][j], alone[j]["y"][0][0]), j
        assert np.array_equal(both["dx"][0][j], alone[j]["dx"][0][0]), j
    for l in range(w2.n_layers):
        for nm in both["dw"][0][l]:
            want = alone[0]["dw"][0][l][nm].astype(np.float32) + alone[1]["dw"][0][l][nm].astype(np.float32)
            assert np.isfinite(want).all()
            assert np.array_equal(both["dw"][0][l][nm].view(np.uint32), want.view(np.uint32)), (l, nm)


def test_split_w_per_linear_and_grouped_give_the_same_bits():
    """The W pass as one grouped launch, the W pass with one launch per linear,
    and the unsplit backward (one launch per linear, interleaved with B) flush
    identical gradient bits."""
    w = si.reduced(si.WORKLOADS["gpt_full_h4096"], hidden=256, heads=2, seq=136, n_micro=4, n_stages=2,
                   n_layers=2)
    ws = [si.stage_weights(w, s) for s in range(w.n_stages)]
    xs = [si.stage_input(w, j) for j in range(w.n_micro)]
    dys = [si.last_stage_grad(w, j) for j in range(w.n_micro)]
    res = {}
    for per_linear in (0, 1):
        pipe = EmulatedPipeline(w, ws, ops=None, recompute_act=0, w_per_linear=per_linear)
        X = [upload(x, "bf16", "cuda") for x in xs]
        DY = [upload(d, "bf16", "cuda") for d in dys]
        for order in ("zbh1", "1f1b"):
            ops, _ = zb.zb_schedule_build(order, w.n_stages, w.n_micro)
            y, dx = pipe.io_buffers()
            pipe.run(ops, X, DY, y, dx)
            torch.cuda.synchronize()
            res[(per_linear, order)] = ([_host(t) for t in y], [_host(t) for t in dx], pipe.grads_host())
        pipe.close()
    base = res[(0, "zbh1")]
    for key, (y, dx, dw) in res.items():
        for j in range(w.n_micro):
            assert np.array_equal(y[j], base[0][j]) and np.array_equal(dx[j], base[1][j]), key
        for s in range(w.n_stages):
            for l in range(w.n_layers):
                for nm in dw[s][l]:
                    assert np.array_equal(dw[s][l][nm].view(np.uint32), base[2][s][l][nm].view(np.uint32)), key


def test_debug_sync_mode_runs_clean_and_keeps_bits():
    """With the debug mode on every pass synchronises and checks for device
    errors; a correct schedule runs through it with unchanged results."""
    w = si.reduced(si.WORKLOADS["gpt_mlp_h2048"], hidden=256, seq=128, n_micro=4, n_stages=2, n_layers=1)
    ws = [si.stage_weights(w, s) for s in range(w.n_stages)]
    xs = [si.stage_input(w, j) for j in range(w.n_micro)]
    dys = [si.last_stage_grad(w, j) for j in range(w.n_micro)]
    ops, _ = zb.zb_schedule_build("zbh1", w.n_stages, w.n_micro)
    pipe = EmulatedPipeline(w, ws, ops=ops, stage_streams=True)
    X = [upload(x, "bf16", "cuda") for x in xs]
    DY = [upload(d, "bf16", "cuda") for d in dys]
    outs = []
    prev = zb.zb_get_debug_sync()
    try:
        for on in (False, True):
            zb.zb_set_debug_sync(on)
            assert zb.zb_get_debug_sync() == on
            y, dx = pipe.io_buffers()
            pipe.run(ops, X, DY, y, dx)
            torch.cuda.synchronize()
            outs.append(([_host(t) for t in y], [_host(t) for t in dx], pipe.grads_host()))
    finally:
        zb.zb_set_debug_sync(prev)
    pipe.close()
    for j in range(w.n_micro):
        assert np.array_equal(outs[0][0][j], outs[1][0][j])
        assert np.array_equal(outs[0][1][j], outs[1][1][j])
    for s in range(w.n_stages):
        for nm in outs[0][2][s][0]:
            assert np.array_equal(outs[0][2][s][0][nm].view(np.uint32), outs[1][2][s][0][nm].view(np.uint32))


def _same_bits(a, b, w):
    for s in range(w.n_stages):
        for j in range(w.n_micro):
            assert np.array_equal(a["y"][s][j], b["y"][s][j]), ("Y", s, j)
            assert np.array_equal(a["dx"][s][j], b["dx"][s][j]), ("dX", s, j)
        for l in range(w.n_layers):
            for nm in a["dw"][s][l]:
                assert np.array_equal(a["dw"][s][l][nm].view(np.uint32), b["dw"][s][l][nm].view(np.uint32)), \
                    ("dW", s, l, nm)


def _stash_handles(w):
    """Stage objects of the workload, for the stash sizes the searched orders budget with."""
    ws = [si.stage_weights(w, s) for s in range(w.n_stages)]
    return EmulatedPipeline(w, ws, ops=None, recompute_act=0)


# The orders searched at run time at the depth of the P = 8 workloads, through
# the two-stream executor: the automatic scheduler with budgets of P and 2P
# stashes ("The Heuristic Scheduling Algorithm" of "Zero Bubble Pipeline
# Parallelism") and the V placement over 2P chunk stages ("Innovation 3: The
# V-Shaped Interleaving Pattern").  Every stage issues its W passes in
# ascending microbatch order, so each order gives 1F1B's bits on every stage
# boundary and in every dW; 1F1B itself is checked stage by stage.
def test_p8_searched_orders_stagewise_and_1f1b_bits():
    w = si.reduced(si.WORKLOADS["gpt_full_s4096"], hidden=256, heads=2, seq=136, n_micro=16, n_stages=8,
                   n_layers=2)
    ref, ws, xs, dys = _run_tapped(w, "1f1b", 2)
    _check_stagewise(w, "1f1b", 2, got=(ref, ws, xs, dys))
    probe = _stash_handles(w)
    cases = []
    for budget in (w.n_stages, 2 * w.n_stages):
        for times in ((1, 1, 1), (2, 3, 1)):
            ops, stats, choice, _ = heuristic_ops(probe.handles, w.n_stages, w.n_micro, times, budget)
            assert zb.zb_schedule_validate(w.n_stages, w.n_micro, ops) == (zb.ZB_OK, -1)
            cases.append((f"budget {budget} times {times} choice {choice} bubble {stats['bubble']}", ops))
    probe.close()
    for label, ops in cases:
        print(f"P=8 searched order: {label}", flush=True)
        got, _, _, _ = _run_tapped(w, ops, 2)
        _same_bits(got, ref, w)

    wv = si.v_chunks(w)  # 16 chunk stages of one layer
    ref_v, ws_v, xs_v, dys_v = _run_tapped(wv, "1f1b", 2)
    _check_stagewise(wv, "1f1b", 2, got=(ref_v, ws_v, xs_v, dys_v))
    probe = _stash_handles(wv)
    ops_v, stats_v, _ = zbv_ops(probe.handles, wv.n_micro, (1, 1, 1))
    probe.close()
    assert zb.zb_schedule_validate(wv.n_stages, wv.n_micro, ops_v) == (zb.ZB_OK, -1)
    print(f"P=8 ZB-V over {wv.n_stages} chunk stages: bubble {stats_v['bubble']}", flush=True)
    got, _, _, _ = _run_tapped(wv, ops_v, 2)
    _same_bits(got, ref_v, wv)
