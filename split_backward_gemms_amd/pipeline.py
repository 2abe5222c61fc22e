"""Device-memory plumbing for P emulated stages on one GPU.

Allocates, with torch, the weights, fp32 gradient buffers, per-stage
workspaces and microbatch I/O buffers, and calls the C ABI.  It performs no
arithmetic of the method itself.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

import split_backward_gemms_amd as zb

KIND_OF = {0: zb.ZB_KIND_TINY_MLP, 1: zb.ZB_KIND_MLP_LINEARS, 2: zb.ZB_KIND_FULL}


def torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def desc_of(w, recompute_act: int = 0, w_per_linear: int = 0) -> "zb.zb_stage_desc":
    """Stage descriptor of a synthetic_inputs.Workload."""
    return zb.make_desc(KIND_OF[w.kind], zb.ZB_DTYPE_BF16 if w.dtype == "bf16" else zb.ZB_DTYPE_FP32,
                        w.n_layers, w.hidden, w.ffn, max(w.n_heads, 0), w.seq, w.micro_batch, w.n_micro,
                        zb.ZB_GELU_TANH if w.gelu == "tanh" else zb.ZB_GELU_ERF, recompute_act, w_per_linear)


def upload(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """fp32 array holding bf16-exact values -> device tensor (exact conversion)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device).to(torch_dtype(dtype))


def pass_times_us(trace) -> Tuple[int, int, int]:
    """Median duration, in whole microseconds (at least 1), of the F, B and W
    passes of a traced run: the per-pass times the automatic scheduler takes."""
    out = []
    for kind in "FBW":
        ms = sorted(t for (op, t, _) in trace if op[1] == kind)
        if not ms:
            raise ValueError(f"trace holds no {kind} pass")
        out.append(max(1, int(round(1000.0 * ms[len(ms) // 2]))))
    return tuple(out)


def stash_per_microbatch(handles: Sequence[int]) -> Tuple[int, int]:
    """(M_B, M_W) in bytes: the stash one microbatch holds after its F and after
    its B, the largest over the stages (the three slot classes of a stage)."""
    m_b = m_w = 0
    for h in handles:
        fw, fb, bw = zb.zb_stage_class_bytes(h)
        m_b, m_w = max(m_b, fw + fb), max(m_w, fw + bw)
    return m_b, m_w


def heuristic_ops(handles: Sequence[int], n_stages: int, n_micro: int, times: Sequence[int],
                  budget_microbatches: int):
    """One-device order from the automatic scheduler for the stages behind
    `handles`.  The activation budget per stage is `budget_microbatches` times
    M_B (P for ZB-1p, 2P for ZB-2p) plus max(0, M_W - M_B): 1F1B's own peak in a
    ledger where a B adds memory, since the microbatch in its backward holds its
    output gradients too.  Returns (ops, stats, (fill, balance), M_limit)."""
    m_b, m_w = stash_per_microbatch(handles)
    m_limit = max(budget_microbatches * m_b + max(0, m_w - m_b), m_b, m_w)
    ops, stats, choice = zb.zb_schedule_heuristic(n_stages, n_micro, times, m_b, m_w, m_limit)
    return ops, stats, choice, m_limit


def zbv_ops(handles: Sequence[int], n_micro: int, times: Sequence[int], t_comm: int = 0):
    """ZB-V order for the 2P chunk stages behind `handles` (chunk c is stage c),
    with the budget of P whole-stage microbatches per device: 2P chunk M_B plus
    max(0, M_W - M_B) for the B in flight.  Returns (ops, stats, M_limit)."""
    if len(handles) % 2:
        raise ValueError("ZB-V needs an even number of chunk stages")
    P = len(handles) // 2
    m_b, m_w = stash_per_microbatch(handles)
    m_limit = max(2 * P * m_b + max(0, m_w - m_b), 2 * m_b + max(0, m_w - m_b), m_w)
    ops, stats = zb.zb_schedule_zbv(P, n_micro, times, m_b, m_w, m_limit, t_comm)
    return ops, stats, m_limit


class EmulatedPipeline:
    """P stages of one workload, each with its own weights, on one device."""

    # Free device memory kept out of the stash when the layout is picked.
    HEADROOM = 6 << 30

    def __init__(self, w, weights: Sequence[Sequence[Dict[str, np.ndarray]]], ops: Optional[Sequence] = None,
                 device: str = "cuda", stream: Optional[torch.cuda.Stream] = None,
                 stage_streams: bool = False, recompute_act: Optional[int] = None,
                 n_streams: Optional[int] = None, w_per_linear: int = 0):
        """stage_streams=True gives every emulated stage its own HIP stream (default
        priority), so independent stages' passes run concurrently; n_streams below P
        caps the number of streams, with neighbouring stages in pairs sharing one
        (stages 2k and 2k+1 on stream k % n_streams: passes issued in the
        linearized order stay valid on a shared stream).  recompute_act
        0 / 1 fixes the stash layout (see zb_stage_desc); None stashes the MLP
        activation when that plan fits in free device memory and rebuilds it for W
        otherwise.  w_per_linear=1 makes every W pass issue one launch per
        linear instead of one grouped launch (same kernel, same bits)."""
        self.w = w
        self.w_per_linear = int(w_per_linear)
        self.device = torch.device(device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        self.P = w.n_stages
        self.streams = self._make_streams(stage_streams, n_streams)
        self.handles: List[int] = []
        self.weights: List[List[torch.Tensor]] = []
        self.grads: List[List[torch.Tensor]] = []
        self.workspaces: List[torch.Tensor] = []
        names = [nm for nm, _, _ in w.linears()]
        shapes = {nm: (k, n) for nm, k, n in w.linears()}
        for s in range(self.P):
            self.weights.append([upload(weights[s][l][nm], w.dtype, self.device)
                                 for l in range(w.n_layers) for nm in names])
            self.grads.append([torch.empty(shapes[nm], dtype=torch.float32, device=self.device)
                               for _ in range(w.n_layers) for nm in names])
        if recompute_act is None:
            self._create(0)
            need = sum(zb.zb_stage_workspace_bytes(h, ops) for h in self.handles)
            free = torch.cuda.mem_get_info(self.device)[0]
            if need + self.HEADROOM > free:
                self.close()
                self._create(1)
        else:
            self._create(int(recompute_act))
        self.plan(ops)

    def rebuild(self, ops: Optional[Sequence], stage_streams: bool = False, n_streams: Optional[int] = None,
                w_per_linear: Optional[int] = None) -> None:
        """New stage objects over the same weights and gradient buffers: other
        streams (one shared stream when stage_streams is False) or another W
        launch mode, and workspaces planned for `ops`.  The stash layout stays."""
        for st in self._distinct_streams():
            st.synchronize()
        self.close()
        if w_per_linear is not None:
            self.w_per_linear = int(w_per_linear)
        self.streams = self._make_streams(stage_streams, n_streams)
        self._create(self.recompute_act)
        self.workspaces = []
        self.plan(ops)

    def _make_streams(self, stage_streams: bool, n_streams: Optional[int]):
        if not stage_streams:
            return [self.stream] * self.P
        n = self.P if n_streams is None else max(1, min(self.P, n_streams))
        pool = [torch.cuda.Stream(self.device) for _ in range(n)]
        # Pairs keep the hand-off between stages 2k and 2k+1 on one stream:
        # measured 0.7-0.9% faster than alternating stages at P = 4 (two
        # streams) and no different at P = 8.
        return pool if n == self.P else [pool[(s // 2) % n] for s in range(self.P)]

    def stream_index_of_stage(self) -> List[int]:
        """Index of the distinct stream each stage runs on."""
        ids: Dict[int, int] = {}
        return [ids.setdefault(id(st), len(ids)) for st in self.streams]

    def _create(self, recompute_act: int) -> None:
        self.recompute_act = recompute_act
        desc = desc_of(self.w, recompute_act, self.w_per_linear)
        self.handles = [zb.zb_stage_create(desc, s, self.weights[s], self.grads[s], self.streams[s].cuda_stream)
                        for s in range(self.P)]

    def _distinct_streams(self):
        return list({id(s): s for s in self.streams}.values())

    def plan(self, ops: Optional[Sequence]) -> None:
        """(Re)size and bind every stage's workspace for the given order (None = all m live).

        The old workspaces may still be read by work queued on the stage streams,
        so those streams are drained before the old buffers go back to torch's
        allocator; a new buffer comes from the caller's stream, and each stage
        stream waits for that stream before the bind enqueues anything on it."""
        cur = torch.cuda.current_stream(self.device)
        if self.workspaces:
            for st in self._distinct_streams():
                st.synchronize()
        self.workspaces = []
        for s, h in enumerate(self.handles):
            nbytes = zb.zb_stage_workspace_bytes(h, ops)
            buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
            off = (-buf.data_ptr()) % 256
            if self.streams[s] != cur:
                self.streams[s].wait_stream(cur)
            zb.zb_stage_bind_workspace(h, buf.data_ptr() + off, nbytes)
            self.workspaces.append(buf)
        for st in self._distinct_streams():
            if st != cur:
                cur.wait_stream(st)  # the binds' clearing work before anything the caller queues

    def set_taps(self, y_taps: Optional[Sequence[Sequence[torch.Tensor]]],
                 dx_taps: Optional[Sequence[Sequence[torch.Tensor]]]) -> None:
        """Per-stage boundary taps: y_taps[s][j] receives stage s's output of
        microbatch j after its F, dx_taps[s][j] its input gradient after its B."""
        for s, h in enumerate(self.handles):
            zb.zb_stage_set_taps(h, None if y_taps is None else y_taps[s],
                                 None if dx_taps is None else dx_taps[s])

    def workspace_bytes(self) -> int:
        return sum(int(b.numel()) for b in self.workspaces)

    def io_buffers(self):
        w = self.w
        shape = (w.tokens, w.hidden)
        dt = torch_dtype(w.dtype)
        y = [torch.empty(shape, dtype=dt, device=self.device) for _ in range(w.n_micro)]
        dx = [torch.empty(shape, dtype=dt, device=self.device) for _ in range(w.n_micro)]
        return y, dx

    def run(self, ops, xs: Sequence[torch.Tensor], dys: Sequence[torch.Tensor], y_last, dx0, trace: bool = False,
            flush: bool = True, check_finite: bool = False):
        cur = torch.cuda.current_stream(self.device)
        distinct = {id(s): s for s in self.streams}.values()
        for st in distinct:
            if st != cur:
                st.wait_stream(cur)  # inputs written on the caller's stream
        tr = zb.zb_run_schedule(self.handles, ops, xs, dys, y_last, dx0, trace=trace)
        flags = None
        if flush:
            flags = [zb.zb_grad_flush(h, check_finite) for h in self.handles]
        for st in distinct:
            if st != cur:
                cur.wait_stream(st)
        return tr, flags

    # ---------------------------------------------------------- optimizer

    def optim_init(self, **hp) -> None:
        """fp32 master parameters (an exact copy of the working weights), zero
        moments, bound to every stage.  hp: lr, beta1, beta2, eps, weight_decay,
        max_grad_norm."""
        self.hp = zb.zb_adamw(**hp)
        self.master = [[w.detach().to(torch.float32, copy=True) for w in ws] for ws in self.weights]
        self.exp_avg = [[torch.zeros_like(p) for p in ps] for ps in self.master]
        self.exp_avg_sq = [[torch.zeros_like(p) for p in ps] for ps in self.master]
        for s, h in enumerate(self.handles):
            zb.zb_stage_optim_bind(h, self.hp, self.master[s], self.exp_avg[s], self.exp_avg_sq[s], self.weights[s])
        self.opt_state = torch.zeros((self.P, 2), dtype=torch.float64, device=self.device)
        self.rolled = torch.zeros(self.P, dtype=torch.int32, device=self.device)

    def optim_step(self, step: int) -> None:
        """Staged reduce of the gradient state, stage 0 first, each stage stepping
        with its partial state as soon as it has it."""
        cur = torch.cuda.current_stream(self.device)
        for s, h in enumerate(self.handles):
            self.streams[s].wait_stream(cur if s == 0 else self.streams[s - 1])
            zb.zb_stage_grad_state(h, None if s == 0 else self.opt_state[s - 1], self.opt_state[s])
            zb.zb_stage_optim_step(h, step, self.opt_state[s])
        for st in {id(x): x for x in self.streams}.values():
            cur.wait_stream(st)

    def optim_validate(self, step: int) -> torch.Tensor:
        """Post-update validation: the global state (the last stage's) travels
        back stage by stage; returns the device flags of the stages that rolled
        back and stepped again."""
        cur = torch.cuda.current_stream(self.device)
        for s in reversed(range(self.P)):
            self.streams[s].wait_stream(cur if s == self.P - 1 else self.streams[s + 1])
            zb.zb_stage_optim_validate(self.handles[s], step, self.opt_state[s], self.opt_state[self.P - 1],
                                       self.rolled[s:s + 1])
        for st in {id(x): x for x in self.streams}.values():
            cur.wait_stream(st)
        return self.rolled

    def grads_host(self) -> List[List[Dict[str, np.ndarray]]]:
        names = [nm for nm, _, _ in self.w.linears()]
        out = []
        for s in range(self.P):
            per = []
            for l in range(self.w.n_layers):
                per.append({nm: self.grads[s][l * len(names) + i].cpu().numpy() for i, nm in enumerate(names)})
            out.append(per)
        return out

    def close(self) -> None:
        for h in self.handles:
            zb.zb_stage_destroy(h)
        self.handles = []

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
