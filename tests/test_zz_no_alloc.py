"""The allocation-free gradient state, zb_stage_grad_state_noalloc, against the
workspace-backed zb_stage_grad_state it varies: on two calls in a row, the
second on smaller stages, both give the same doubles bit for bit (same kernels,
same fixed reduction order), and both agree with the fp64 sum of squares of
the flushed gradients.  A stage whose gradients need more partial states than
the library's array holds is refused before anything is launched."""
import numpy as np
import pytest
import torch

import split_backward_gemms_amd as zb
import synthetic_inputs as si
from split_backward_gemms_amd.pipeline import EmulatedPipeline, desc_of, upload


pytestmark = pytest.mark.gpu


def _flushed_pipeline(w):
    ws = [si.stage_weights(w, s) for s in range(w.n_stages)]
    xs = [si.stage_input(w, j) for j in range(w.n_micro)]
    dys = [si.last_stage_grad(w, j) for j in range(w.n_micro)]
    ops, _ = zb.zb_schedule_build("zbh1", w.n_stages, w.n_micro)
    pipe = EmulatedPipeline(w, ws, ops=ops)
    X = [upload(x, w.dtype, "cuda") for x in xs]
    DY = [upload(d, w.dtype, "cuda") for d in dys]
    y, dx = pipe.io_buffers()
    pipe.run(ops, X, DY, y, dx)  # flushes every stage
    torch.cuda.synchronize()
    return pipe


def _states(pipe, fn):
    out = torch.full((pipe.P, 2), -1.0, dtype=torch.float64, device="cuda")
    for s, h in enumerate(pipe.handles):
        fn(h, None if s == 0 else out[s - 1], out[s])
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_noalloc_grad_state_matches_workspace_version_twice():
    big = si.reduced(si.WORKLOADS["gpt_mlp_h2048"], hidden=512, seq=256, n_micro=4, n_stages=3, n_layers=2)
    small = si.reduced(si.WORKLOADS["gpt_full_h4096"], hidden=128, heads=1, seq=64, n_micro=2, n_stages=2,
                       n_layers=1)
    for w in (big, small):
        print(f"noalloc grad state: {w.name} P={w.n_stages} L={w.n_layers} h={w.hidden}", flush=True)
        pipe = _flushed_pipeline(w)
        ref = _states(pipe, zb.zb_stage_grad_state)
        got = _states(pipe, zb.zb_stage_grad_state_noalloc)
        assert np.array_equal(ref.view(np.uint64), got.view(np.uint64)), (ref, got)
        sumsq = 0.0
        for s, grads in enumerate(pipe.grads_host()):
            sumsq += sum(float(np.sum(g.astype(np.float64) ** 2)) for layer in grads for g in layer.values())
            assert abs(got[s, 0] - sumsq) <= 1e-12 * sumsq
            assert got[s, 1] == 0.0
        pipe.close()


def test_noalloc_grad_state_refuses_oversized_stage_before_launch():
    # 40 layers of two 1024 x 1024 linears: 80 x 1024 partial states > 65536.
    w = si.WORKLOADS["tiny"].replace(hidden=1024, ffn=1024, n_layers=40, n_stages=1, n_micro=1)
    buf = torch.empty(64, dtype=torch.float32, device="cuda")  # only addresses; nothing is launched
    n = 2 * w.n_layers
    h = zb.zb_stage_create(desc_of(w), 0, [buf] * n, [buf] * n, torch.cuda.current_stream().cuda_stream)
    try:
        out = torch.zeros(2, dtype=torch.float64, device="cuda")
        with pytest.raises(zb.ZbError) as e:
            zb.zb_stage_grad_state_noalloc(h, None, out)
        assert e.value.status == zb.ZB_E_UNSUPPORTED
        torch.cuda.synchronize()
        assert torch.all(out == 0).item()
    finally:
        zb.zb_stage_destroy(h)
