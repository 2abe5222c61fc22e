"""Python binding of libzb.so, the C ABI of one zero-bubble pipeline stage.

Argument marshalling only: every function here converts Python values (ints,
lists of (stage, kind, mb) tuples, torch tensors for device buffers) into the
C types of ``include/zb.h`` and calls the function of the same name.  All
computation happens in the HIP library; there is no Python or CPU fallback.
If the library has not been built, importing works but the first call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import List, Optional, Sequence, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzb.so")

# ------------------------------------------------------------------ constants
ZB_OK, ZB_E_ARG, ZB_E_STATE, ZB_E_DUPLICATE, ZB_E_INVALID_STAGE, ZB_E_INVALID_MB = 0, 1, 2, 3, 4, 5
ZB_E_MISSING, ZB_E_DEPENDENCY, ZB_E_BUDGET, ZB_E_HIP, ZB_E_UNSUPPORTED = 6, 7, 8, 9, 10
ZB_E_DEADLOCK, ZB_E_INTERVAL, ZB_E_OVERLAP = 11, 12, 13
STATUS_NAMES = {0: "ok", 1: "arg", 2: "state", 3: "duplicate", 4: "invalid_stage", 5: "invalid_mb",
                6: "missing", 7: "dependency", 8: "budget", 9: "hip", 10: "unsupported",
                11: "deadlock", 12: "interval", 13: "overlap"}

ZB_KIND_TINY_MLP, ZB_KIND_MLP_LINEARS, ZB_KIND_FULL = 0, 1, 2
ZB_DTYPE_BF16, ZB_DTYPE_FP32 = 0, 1
ZB_GELU_ERF, ZB_GELU_TANH = 0, 1
ZB_ORDER_GPIPE, ZB_ORDER_1F1B, ZB_ORDER_ZBH1, ZB_ORDER_ZBH2, ZB_ORDER_WLAST = 0, 1, 2, 3, 4
ORDER_IDS = {"gpipe": 0, "1f1b": 1, "zbh1": 2, "zbh2": 3, "wlast": 4}


class ZbError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))


# ---------------------------------------------------------------- C structs

class zb_adamw(C.Structure):
    _fields_ = [("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float), ("eps", C.c_float),
                ("weight_decay", C.c_float), ("max_grad_norm", C.c_float)]


class zb_stage_desc(C.Structure):
    _fields_ = [("kind", C.c_int), ("dtype", C.c_int), ("n_layers", C.c_int), ("hidden", C.c_int),
                ("ffn", C.c_int), ("n_heads", C.c_int), ("seq", C.c_int), ("micro_batch", C.c_int),
                ("n_micro", C.c_int), ("gelu", C.c_int), ("recompute_act", C.c_int), ("w_per_linear", C.c_int)]


class zb_op(C.Structure):
    _fields_ = [("stage", C.c_int32), ("mb", C.c_int32), ("kind", C.c_char), ("pad_", C.c_char * 3)]


class zb_sim_stats(C.Structure):
    _fields_ = [("makespan", C.c_int64), ("span", C.c_int64), ("busy", C.c_int64), ("ideal", C.c_int64),
                ("bubble", C.c_int64)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class zb_event(C.Structure):
    _fields_ = [("id", C.c_int32), ("stage", C.c_int32), ("micro", C.c_int32), ("kind", C.c_char),
                ("pad_", C.c_char * 3), ("start", C.c_double), ("end", C.c_double), ("n_deps", C.c_int32),
                ("deps", C.POINTER(C.c_int32))]


class zb_event_report(C.Structure):
    _fields_ = [("span", C.c_double), ("busy", C.c_double), ("bubble_ratio", C.c_double),
                ("unfinished_activations", C.c_int64), ("peak_live_activations", C.c_int64)]


class zb_trace_rec(C.Structure):
    _fields_ = [("op", zb_op), ("ms", C.c_float), ("t0_ms", C.c_float)]


class zb_prof_rec(C.Structure):
    _fields_ = [("name", C.c_char * 48), ("launches", C.c_int64), ("total_ms", C.c_double),
                ("flops", C.c_double), ("bytes", C.c_double)]


# ------------------------------------------------------------------ loading

_lib = None


def lib():
    """The loaded libzb.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m split_backward_gemms_amd.build` (hipcc, gfx950)")
        L = C.CDLL(LIB_PATH)
        P, I, I64, S = C.c_void_p, C.c_int, C.c_int64, C.c_size_t
        op_p = C.POINTER(zb_op)
        sig = {
            "zb_schedule_stage_order": (I, [I, I, I, I, op_p, I, C.POINTER(I)]),
            "zb_schedule_simulate": (I, [I, I, op_p, I, C.POINTER(I64), I64, op_p, C.POINTER(I64),
                                         C.POINTER(I64), C.POINTER(zb_sim_stats)]),
            "zb_schedule_build": (I, [I, I, I, C.POINTER(I64), I64, op_p, I, C.POINTER(I),
                                      C.POINTER(zb_sim_stats)]),
            "zb_schedule_heuristic": (I, [I, I, C.POINTER(C.c_int64), C.c_int64, C.c_int64, C.c_int64, C.c_int64,
                                               op_p, I, C.POINTER(I), C.POINTER(zb_sim_stats), C.POINTER(I)]),
            "zb_schedule_zbv": (I, [I, I, C.POINTER(I64), I64, I64, I64, I64, op_p, I, C.POINTER(I),
                                    C.POINTER(zb_sim_stats)]),
            "zb_schedule_simulate_interleaved": (I, [I, I, I, C.POINTER(I64), C.POINTER(zb_sim_stats)]),
            "zb_schedule_validate": (I, [I, I, op_p, I, C.POINTER(I)]),
            "zb_schedule_peak_memory": (I, [op_p, I, I, I64, I64, C.POINTER(I64)]),
            "zb_events_inspect": (I, [C.POINTER(zb_event), I, I, C.POINTER(zb_event_report), C.POINTER(I)]),
            "zb_stage_create": (I, [C.POINTER(zb_stage_desc), I, C.POINTER(P), C.POINTER(P), P,
                                    C.POINTER(P)]),
            "zb_stage_class_bytes": (I, [P, C.POINTER(S), C.POINTER(S), C.POINTER(S)]),
            "zb_stage_workspace_bytes": (I, [P, op_p, I, C.POINTER(S)]),
            "zb_stage_bind_workspace": (I, [P, P, S]),
            "zb_stage_input_slot": (I, [P, I, C.POINTER(P)]),
            "zb_stage_grad_slot": (I, [P, I, C.POINTER(P)]),
            "zb_forward": (I, [P, I, P, P]),
            "zb_backward_input": (I, [P, I, P, P]),
            "zb_backward_weight": (I, [P, I]),
            "zb_backward_unsplit": (I, [P, I, P, P]),
            "zb_stage_set_taps": (I, [P, C.POINTER(P), C.POINTER(P)]),
            "zb_set_debug_sync": (None, [I]),
            "zb_get_debug_sync": (I, []),
            "zb_grad_flush": (I, [P, C.POINTER(I)]),
            "zb_stage_optim_bind": (I, [P, C.POINTER(zb_adamw), C.POINTER(P), C.POINTER(P), C.POINTER(P),
                                        C.POINTER(P)]),
            "zb_stage_grad_state": (I, [P, P, P]),
            "zb_stage_grad_state_noalloc": (I, [P, P, P]),
            "zb_stage_optim_step": (I, [P, I, P]),
            "zb_stage_optim_validate": (I, [P, I, P, P, P]),
            "zb_stage_optim_rollback": (I, [P, I, P]),
            "zb_run_schedule": (I, [C.POINTER(P), I, op_p, I, C.POINTER(P), C.POINTER(P), C.POINTER(P),
                                    C.POINTER(P), C.POINTER(zb_trace_rec)]),
            "zb_last_error": (C.c_char_p, []),
            "zb_stage_destroy": (None, [P]),
            "zb_prof_enable": (None, [I]),
            "zb_prof_reset": (None, []),
            "zb_prof_read": (I, [C.POINTER(zb_prof_rec), I, C.POINTER(I)]),
            "zb_version": (C.c_char_p, []),
            "zb_linear_forward": (I, [I, I, I, I, P, P, P, P]),
            "zb_linear_backward_input": (I, [I, I, I, I, P, P, P, P]),
            "zb_linear_backward_weight": (I, [I, I, I, I, P, P, P, I, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def exported_symbols() -> List[str]:
    """Names of the C entry points this binding expects (all declared in zb.h)."""
    return ["zb_schedule_stage_order", "zb_schedule_simulate", "zb_schedule_build", "zb_schedule_heuristic",
            "zb_schedule_zbv", "zb_schedule_simulate_interleaved", "zb_schedule_validate", "zb_schedule_peak_memory",
            "zb_events_inspect", "zb_stage_create", "zb_stage_class_bytes", "zb_stage_workspace_bytes",
            "zb_stage_bind_workspace", "zb_stage_input_slot", "zb_stage_grad_slot", "zb_forward",
            "zb_backward_input", "zb_backward_weight", "zb_backward_unsplit", "zb_stage_set_taps",
            "zb_set_debug_sync", "zb_get_debug_sync", "zb_grad_flush",
            "zb_stage_optim_bind", "zb_stage_grad_state", "zb_stage_grad_state_noalloc", "zb_stage_optim_step",
            "zb_stage_optim_validate",
            "zb_stage_optim_rollback",
            "zb_run_schedule", "zb_last_error", "zb_stage_destroy", "zb_prof_enable", "zb_prof_reset",
            "zb_prof_read", "zb_version", "zb_linear_forward", "zb_linear_backward_input",
            "zb_linear_backward_weight"]


def _check(st: int) -> None:
    if st != ZB_OK:
        raise ZbError(st, lib().zb_last_error().decode())


def _ptr(x) -> Optional[int]:
    """Device address of a torch tensor, or an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


# --------------------------------------------------------------- op lists

Op = Tuple[int, str, int]  # (stage, kind, mb)


def ops_to_c(ops: Sequence[Op]):
    arr = (zb_op * max(1, len(ops)))()
    for i, (s, k, j) in enumerate(ops):
        arr[i].stage, arr[i].mb, arr[i].kind = s, j, k.encode()
    return arr


def ops_from_c(arr, n: int) -> List[Op]:
    return [(arr[i].stage, arr[i].kind.decode(), arr[i].mb) for i in range(n)]


def _times(t) -> C.Array:
    return (C.c_int64 * 3)(int(t[0]), int(t[1]), int(t[2]))


# ------------------------------------------------------------ schedule layer

def zb_schedule_stage_order(order, P: int, m: int, stage: int) -> List[Op]:
    o = ORDER_IDS[order] if isinstance(order, str) else int(order)
    cap = 3 * m + 1
    arr = (zb_op * cap)()
    n = C.c_int(0)
    _check(lib().zb_schedule_stage_order(o, P, m, stage, arr, cap, C.byref(n)))
    return ops_from_c(arr, n.value)


def zb_schedule_simulate(P: int, m: int, ops: Sequence[Op], times=(1, 1, 1), t_comm: int = 0):
    """Returns (linear order, start list, end list, stats dict)."""
    n = len(ops)
    src = ops_to_c(ops)
    lin = (zb_op * max(1, n))()
    start = (C.c_int64 * max(1, n))()
    end = (C.c_int64 * max(1, n))()
    st = zb_sim_stats()
    _check(lib().zb_schedule_simulate(P, m, src, n, _times(times), t_comm, lin, start, end, C.byref(st)))
    return ops_from_c(lin, n), list(start[:n]), list(end[:n]), st.as_dict()


def zb_schedule_build(order, P: int, m: int, times=(1, 1, 1), t_comm: int = 0):
    """Returns (one-device order, stats dict)."""
    o = ORDER_IDS[order] if isinstance(order, str) else int(order)
    cap = 3 * P * m
    arr = (zb_op * cap)()
    n = C.c_int(0)
    st = zb_sim_stats()
    _check(lib().zb_schedule_build(o, P, m, _times(times), t_comm, arr, cap, C.byref(n), C.byref(st)))
    return ops_from_c(arr, n.value), st.as_dict()


def zb_schedule_heuristic(P: int, m: int, times, m_b: int, m_w: int, m_limit: int, t_comm: int = 0):
    """Automatic schedule within an activation-memory budget.  Returns (one-device
    order, stats dict, (fill, balance) choice)."""
    cap = 3 * P * m
    arr = (zb_op * cap)()
    n = C.c_int(0)
    st = zb_sim_stats()
    ch = C.c_int(-1)
    _check(lib().zb_schedule_heuristic(P, m, _times(times), t_comm, m_b, m_w, m_limit, arr, cap, C.byref(n),
                                       C.byref(st), C.byref(ch)))
    return ops_from_c(arr, n.value), st.as_dict(), (ch.value >> 1, ch.value & 1)


def zb_schedule_zbv(P: int, m: int, times, m_b: int, m_w: int, m_limit: int, t_comm: int = 0):
    """V-shaped placement: one-device order over the 2P chunk stages (stage
    field = chunk index) and the per-device stats dict."""
    cap = 6 * P * m
    arr = (zb_op * cap)()
    n = C.c_int(0)
    st = zb_sim_stats()
    _check(lib().zb_schedule_zbv(P, m, _times(times), t_comm, m_b, m_w, m_limit, arr, cap, C.byref(n),
                                 C.byref(st)))
    return ops_from_c(arr, n.value), st.as_dict()


def zb_schedule_simulate_interleaved(P: int, m: int, v: int, times=(1, 1, 1)) -> dict:
    st = zb_sim_stats()
    _check(lib().zb_schedule_simulate_interleaved(P, m, v, _times(times), C.byref(st)))
    return st.as_dict()


def zb_schedule_validate(P: int, m: int, ops: Sequence[Op]) -> Tuple[int, int]:
    """Returns (status, first bad index); does not raise."""
    bad = C.c_int(-1)
    st = lib().zb_schedule_validate(P, m, ops_to_c(ops), len(ops), C.byref(bad))
    return st, bad.value


def zb_schedule_peak_memory(ops: Sequence[Op], stage: int, m_b: int, m_w: int) -> int:
    peak = C.c_int64(0)
    _check(lib().zb_schedule_peak_memory(ops_to_c(ops), len(ops), stage, m_b, m_w, C.byref(peak)))
    return peak.value


def zb_events_inspect(tasks: Sequence[dict], stage_count: int):
    """tasks: dicts with id (any hashable), stage, micro, kind, start, end, depends_on.
    Returns (status, report dict or None, bad index).  Ids are mapped to integers
    in list order; an unknown dependency id maps to -1."""
    ids = {}
    for t in tasks:
        ids.setdefault(t["id"], len(ids))
    n = len(tasks)
    arr = (zb_event * max(1, n))()
    keep = []
    for i, t in enumerate(tasks):
        deps = [ids.get(d, -1) for d in t.get("depends_on", [])]  # -1: names no task
        dep_arr = (C.c_int32 * max(1, len(deps)))(*deps)
        keep.append(dep_arr)
        e = arr[i]
        e.id = ids[t["id"]]
        e.stage, e.micro = int(t["stage"]), int(t["micro"])
        e.kind = str(t["kind"]).encode()[:1] or b"?"
        e.start, e.end = float(t["start"]), float(t["end"])
        e.n_deps = len(deps)
        e.deps = C.cast(dep_arr, C.POINTER(C.c_int32))
    rep = zb_event_report()
    bad = C.c_int(-1)
    st = lib().zb_events_inspect(arr, n, int(stage_count), C.byref(rep), C.byref(bad))
    if st != ZB_OK:
        return st, None, bad.value
    return st, {"span": rep.span, "busy": rep.busy, "bubble_ratio": rep.bubble_ratio,
                "unfinished_activations": rep.unfinished_activations,
                "peak_live_activations": rep.peak_live_activations}, -1


# -------------------------------------------------------------- stage layer

def make_desc(kind: int, dtype: int, n_layers: int, hidden: int, ffn: int, n_heads: int, seq: int,
              micro_batch: int, n_micro: int, gelu: int = ZB_GELU_ERF, recompute_act: int = 0,
              w_per_linear: int = 0) -> zb_stage_desc:
    return zb_stage_desc(kind, dtype, n_layers, hidden, ffn, n_heads, seq, micro_batch, n_micro, gelu,
                         recompute_act, w_per_linear)


def zb_stage_create(desc: zb_stage_desc, stage_index: int, weights: Sequence, dw: Sequence, stream=None) -> int:
    """weights / dw: device buffers ([layer][linear] order); stream: hipStream_t address or None."""
    nw = len(weights)
    wa = (C.c_void_p * nw)(*[_ptr(w) for w in weights])
    ga = (C.c_void_p * nw)(*[_ptr(g) for g in dw])
    out = C.c_void_p()
    _check(lib().zb_stage_create(C.byref(desc), stage_index, wa, ga, stream, C.byref(out)))
    return out.value


def zb_stage_class_bytes(stage: int) -> Tuple[int, int, int]:
    a, b, c = C.c_size_t(), C.c_size_t(), C.c_size_t()
    _check(lib().zb_stage_class_bytes(stage, C.byref(a), C.byref(b), C.byref(c)))
    return a.value, b.value, c.value


def zb_stage_workspace_bytes(stage: int, ops: Optional[Sequence[Op]]) -> int:
    b = C.c_size_t()
    if ops is None:
        _check(lib().zb_stage_workspace_bytes(stage, None, 0, C.byref(b)))
    else:
        _check(lib().zb_stage_workspace_bytes(stage, ops_to_c(ops), len(ops), C.byref(b)))
    return b.value


def zb_stage_bind_workspace(stage: int, buf, nbytes: int) -> None:
    _check(lib().zb_stage_bind_workspace(stage, _ptr(buf), nbytes))


def zb_stage_input_slot(stage: int, mb: int) -> int:
    p = C.c_void_p()
    _check(lib().zb_stage_input_slot(stage, mb, C.byref(p)))
    return p.value


def zb_stage_grad_slot(stage: int, mb: int) -> int:
    p = C.c_void_p()
    _check(lib().zb_stage_grad_slot(stage, mb, C.byref(p)))
    return p.value


def zb_forward(stage: int, mb: int, x, y) -> None:
    _check(lib().zb_forward(stage, mb, _ptr(x), _ptr(y)))


def zb_backward_input(stage: int, mb: int, dy, dx) -> None:
    _check(lib().zb_backward_input(stage, mb, _ptr(dy), _ptr(dx)))


def zb_backward_weight(stage: int, mb: int) -> None:
    _check(lib().zb_backward_weight(stage, mb))


def zb_backward_unsplit(stage: int, mb: int, dy, dx) -> None:
    _check(lib().zb_backward_unsplit(stage, mb, _ptr(dy), _ptr(dx)))


def zb_stage_set_taps(stage: int, y_tap: Optional[Sequence], dx_tap: Optional[Sequence]) -> None:
    """Device buffers ([T, h] per microbatch) that receive the stage output after
    each F and the stage input gradient after each B; None removes a tap."""
    def arr(xs):
        return None if xs is None else (C.c_void_p * len(xs))(*[_ptr(x) for x in xs])
    _check(lib().zb_stage_set_taps(stage, arr(y_tap), arr(dx_tap)))


def zb_set_debug_sync(on: bool) -> None:
    lib().zb_set_debug_sync(1 if on else 0)


def zb_get_debug_sync() -> bool:
    return bool(lib().zb_get_debug_sync())


def zb_grad_flush(stage: int, check_finite: bool = False) -> Optional[int]:
    if check_finite:
        flag = C.c_int(-1)
        _check(lib().zb_grad_flush(stage, C.byref(flag)))
        return flag.value
    _check(lib().zb_grad_flush(stage, None))
    return None


def zb_stage_optim_bind(stage: int, hp: "zb_adamw", master: Sequence, exp_avg: Sequence, exp_avg_sq: Sequence,
                        weights_rw: Sequence) -> None:
    def arr(xs):
        return (C.c_void_p * len(xs))(*[_ptr(x) for x in xs])
    _check(lib().zb_stage_optim_bind(stage, C.byref(hp), arr(master), arr(exp_avg), arr(exp_avg_sq),
                                     arr(weights_rw)))


def zb_stage_grad_state(stage: int, upstream, partial_out) -> None:
    _check(lib().zb_stage_grad_state(stage, _ptr(upstream), _ptr(partial_out)))


def zb_stage_grad_state_noalloc(stage: int, upstream, partial_out) -> None:
    """As zb_stage_grad_state, with the partial states in the library's own
    device array (allocates nothing; calls on one GPU must not overlap)."""
    _check(lib().zb_stage_grad_state_noalloc(stage, _ptr(upstream), _ptr(partial_out)))


def zb_stage_optim_step(stage: int, step: int, used) -> None:
    _check(lib().zb_stage_optim_step(stage, step, _ptr(used)))


def zb_stage_optim_validate(stage: int, step: int, used, glob, rolled_back=None) -> None:
    _check(lib().zb_stage_optim_validate(stage, step, _ptr(used), _ptr(glob), _ptr(rolled_back)))


def zb_stage_optim_rollback(stage: int, step: int, used) -> None:
    _check(lib().zb_stage_optim_rollback(stage, step, _ptr(used)))


def zb_run_schedule(stages: Sequence[int], ops: Sequence[Op], x0: Sequence, dy_last: Sequence,
                    y_last: Sequence, dx0: Sequence, trace: bool = False):
    """Runs a one-device order over len(stages) stages.  Returns the per-pass
    trace [(op, ms, t0_ms)] when trace is True, else None."""
    P = len(stages)
    sa = (C.c_void_p * P)(*stages)
    m = len(x0)

    def arr(xs):
        return (C.c_void_p * m)(*[_ptr(x) for x in xs])

    recs = (zb_trace_rec * len(ops))() if trace else None
    _check(lib().zb_run_schedule(sa, P, ops_to_c(ops), len(ops), arr(x0), arr(dy_last), arr(y_last), arr(dx0),
                                 recs))
    if not trace:
        return None
    return [((r.op.stage, r.op.kind.decode(), r.op.mb), r.ms, r.t0_ms) for r in recs]


def zb_stage_destroy(stage: int) -> None:
    if stage:
        lib().zb_stage_destroy(stage)


def zb_prof_enable(on: bool) -> None:
    lib().zb_prof_enable(1 if on else 0)


def zb_prof_reset() -> None:
    lib().zb_prof_reset()


def zb_prof_read() -> List[dict]:
    n = C.c_int(0)
    _check(lib().zb_prof_read(None, 0, C.byref(n)))
    cap = n.value
    recs = (zb_prof_rec * max(1, cap))()
    _check(lib().zb_prof_read(recs, cap, C.byref(n)))
    return [{"name": r.name.decode(), "launches": r.launches, "total_ms": r.total_ms, "flops": r.flops,
             "bytes": r.bytes} for r in recs[:min(cap, n.value)]]


def zb_version() -> str:
    return lib().zb_version().decode()


def zb_last_error() -> str:
    return lib().zb_last_error().decode()


# ------------------------------------------------------------ single linears

def _dt(t) -> int:
    import torch
    return ZB_DTYPE_BF16 if t.dtype == torch.bfloat16 else ZB_DTYPE_FP32


def zb_linear_forward(x, w, y, stream=None) -> None:
    T, K = x.shape
    N = w.shape[1]
    _check(lib().zb_linear_forward(_dt(x), T, K, N, _ptr(x), _ptr(w), _ptr(y), stream))


def zb_linear_backward_input(dy, w, dx, stream=None) -> None:
    T, N = dy.shape
    K = w.shape[0]
    _check(lib().zb_linear_backward_input(_dt(dy), T, K, N, _ptr(dy), _ptr(w), _ptr(dx), stream))


def zb_linear_backward_weight(x, dy, dw, accumulate: bool, stream=None) -> None:
    T, K = x.shape
    N = dy.shape[1]
    _check(lib().zb_linear_backward_weight(_dt(x), T, K, N, _ptr(x), _ptr(dy), _ptr(dw), 1 if accumulate else 0,
                                           stream))
