"""Seeded synthetic inputs shared by the oracle, the tests and the benchmark.

This module holds no arithmetic of the method: it only names the workloads
(layer shapes, microbatch counts, pipeline depth, schedule order) and draws the
random tensors that feed one pipeline stage.  Both the fp64 CPU oracle and the
HIP path receive exactly the same values from here.

Value distributions: stage inputs X and the upstream gradient dY are N(0, 1),
weights are N(0, 0.02) (standard deviation).  Every tensor is drawn from its own
PCG64 stream keyed by SeedSequence([seed, workload_id, stage, layer, tensor, mb]),
then rounded to bfloat16 with round-to-nearest-even so that the bf16 device
copy and the fp64 oracle copy hold identical numbers.  An fp32 workload keeps
the fp32 draw as is.

Weight layout: W is row-major [K, N] so that a linear computes Y = X.W, the
input gradient is dX = dY.W^T and the weight gradient is dW = X^T.dY (the
zero-bubble section of the pipeline-schedules tutorial writes them that way).
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Tuple

import numpy as np

# Layer kinds of a stage.
TINY_MLP = 0      # Linear(K->F), GeLU, Linear(F->K); no attention, no residual
MLP_LINEARS = 1   # QKV, identity attention (V slice), proj, up, GeLU, down; no residual
FULL = 2          # QKV, causal softmax attention, proj (+residual), up, GeLU, down (+residual)

KIND_NAMES = {TINY_MLP: "tiny_mlp", MLP_LINEARS: "mlp_linears", FULL: "full"}

# Tensor ids used in the seed key.
T_QKV, T_PROJ, T_UP, T_DOWN = 0, 1, 2, 3
T_X0, T_DY = 10, 11

WEIGHT_STD = 0.02
BASE_SEED = 1234


@dataclasses.dataclass(frozen=True)
class Workload:
    """One stage shape plus the pipeline it runs in."""
    name: str
    wid: int            # workload id used in the seed key
    kind: int
    n_layers: int
    hidden: int
    ffn: int
    n_heads: int
    seq: int
    micro_batch: int
    n_micro: int        # m
    n_stages: int       # P (emulated on one GPU)
    order: str          # "1f1b", "zbh1", "zbh2"
    dtype: str = "bf16"  # "bf16" or "fp32"
    gelu: str = "erf"    # "erf" (exact) or "tanh" (the tanh approximation)

    @property
    def tokens(self) -> int:
        return self.seq * self.micro_batch

    @property
    def head_dim(self) -> int:
        return self.hidden // self.n_heads if self.n_heads else 0

    def linears(self) -> List[Tuple[str, int, int]]:
        """(name, K, N) of every linear of one layer, in forward order."""
        h, f = self.hidden, self.ffn
        if self.kind == TINY_MLP:
            return [("up", h, f), ("down", f, h)]
        return [("qkv", h, 3 * h), ("proj", h, h), ("up", h, f), ("down", f, h)]

    def gemm_flops_per_pass(self) -> int:
        """2*T*K*N summed over the linears of all layers of one stage (one microbatch)."""
        return self.n_layers * sum(2 * self.tokens * k * n for _, k, n in self.linears())

    def attn_flops_fwd(self) -> int:
        """Causal-only attention forward FLOPs per stage and microbatch: two
        s x s x d products per head, half of the square kept by the mask."""
        if self.kind != FULL:
            return 0
        s, b = self.seq, self.micro_batch
        return self.n_layers * 2 * s * s * self.hidden * b

    def attn_flops_bwd(self) -> int:
        return 2 * self.attn_flops_fwd()

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads.  P for the middle three is not fixed by the workload
# text; the values below are the readings recorded in the design notes.
WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 1, TINY_MLP, 1, 256, 1024, 0, 512, 1, 4, 2, "zbh1"),
    "gpt_mlp_h2048": Workload("gpt_mlp_h2048", 2, MLP_LINEARS, 4, 2048, 8192, 16, 1024, 1, 8, 4, "zbh1"),
    "gpt_full_h4096": Workload("gpt_full_h4096", 3, FULL, 4, 4096, 16384, 32, 2048, 1, 16, 4, "zbh1"),
    "gpt_full_h6144": Workload("gpt_full_h6144", 4, FULL, 2, 6144, 24576, 48, 1024, 2, 24, 8, "zbh2"),
    "gpt_full_s4096": Workload("gpt_full_s4096", 5, FULL, 4, 4096, 16384, 32, 4096, 1, 32, 8, "zbh2"),
}


def reduced(w: Workload, hidden: int = 256, heads: int = 2, seq: int = 128,
            n_micro: Optional[int] = None, n_stages: Optional[int] = None,
            n_layers: Optional[int] = None) -> Workload:
    """Same layer structure at a size the fp64 oracle finishes in seconds."""
    return w.replace(name=w.name + "_reduced", hidden=hidden, ffn=4 * hidden,
                     n_heads=heads if w.kind != TINY_MLP else 0, seq=seq,
                     n_micro=w.n_micro if n_micro is None else n_micro,
                     n_stages=w.n_stages if n_stages is None else n_stages,
                     n_layers=w.n_layers if n_layers is None else n_layers)


def v_chunks(w: Workload) -> Workload:
    """The same model cut for the V placement: 2P chunk stages of half a stage's
    layers each (chunk c is stage c of a 2P-stage chain)."""
    if w.n_layers % 2:
        raise ValueError(f"{w.name}: {w.n_layers} layers per stage do not split into two chunks")
    return w.replace(name=w.name + "_v", n_stages=2 * w.n_stages, n_layers=w.n_layers // 2)


# ---------------------------------------------------------------------------
# bf16 encoding (round to nearest even); pure data preparation.

def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> uint16 bf16 bit patterns, round-to-nearest-even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(to_bf16_bits(a))


# ---------------------------------------------------------------------------

def _rng(w: Workload, stage: int, layer: int, tensor: int, mb: int, seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [seed, w.wid, stage, layer, tensor, mb])))


def _draw(w: Workload, shape, std: float, key, seed: int) -> np.ndarray:
    a = _rng(w, *key, seed=seed).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if w.dtype == "bf16":
        a = round_bf16(a)
    return a


def weight(w: Workload, stage: int, layer: int, name: str, seed: int = BASE_SEED) -> np.ndarray:
    """Weight [K, N] as float32 holding bf16-exact values (or fp32 values)."""
    tid = {"qkv": T_QKV, "proj": T_PROJ, "up": T_UP, "down": T_DOWN}[name]
    k, n = {nm: (kk, nn) for nm, kk, nn in w.linears()}[name]
    return _draw(w, (k, n), WEIGHT_STD, (stage, layer, tid, 0), seed)


def stage_weights(w: Workload, stage: int, seed: int = BASE_SEED,
                  threads: int = 8) -> List[Dict[str, np.ndarray]]:
    jobs = [(l, nm) for l in range(w.n_layers) for nm, _, _ in w.linears()]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        arrs = list(ex.map(lambda j: weight(w, stage, j[0], j[1], seed), jobs))
    out: List[Dict[str, np.ndarray]] = [dict() for _ in range(w.n_layers)]
    for (l, nm), a in zip(jobs, arrs):
        out[l][nm] = a
    return out


def stage_input(w: Workload, mb: int, seed: int = BASE_SEED) -> np.ndarray:
    """Input X [T, h] of the first stage for microbatch mb, N(0, 1)."""
    return _draw(w, (w.tokens, w.hidden), 1.0, (0, 0, T_X0, mb), seed)


def last_stage_grad(w: Workload, mb: int, seed: int = BASE_SEED) -> np.ndarray:
    """Upstream gradient dY [T, h] entering the last stage for microbatch mb, N(0, 1)."""
    return _draw(w, (w.tokens, w.hidden), 1.0, (w.n_stages - 1, 0, T_DY, mb), seed)


def integer_valued(shape, lo: int, hi: int, seed: int) -> np.ndarray:
    """Small integers in [lo, hi] as float32 (exact in bf16 for |v| <= 256)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 77])))
    return g.integers(lo, hi + 1, size=shape).astype(np.float32)
