"""The C-ABI library loads and exports every function include/zb.h declares.
No compute call is made (no GPU needed)."""
import ctypes
import os
import re

import split_backward_gemms_amd as zb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "zb.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zb_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for required in ("zb_stage_create", "zb_forward", "zb_backward_input", "zb_backward_weight",
                     "zb_grad_flush", "zb_run_schedule"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(zb.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_every_declared_symbol():
    assert sorted(zb.exported_symbols()) == _declared()
    zb.lib()  # sets every signature


def test_stage_create_rejects_bad_descriptors_without_gpu():
    d = zb.make_desc(zb.ZB_KIND_MLP_LINEARS, zb.ZB_DTYPE_BF16, 1, 100, 400, 1, 64, 1, 2)
    try:
        zb.zb_stage_create(d, 0, [16] * 4, [16] * 4)
    except zb.ZbError as e:
        assert e.status == zb.ZB_E_UNSUPPORTED
    else:
        raise AssertionError("hidden 100 must be rejected")
    d = zb.make_desc(zb.ZB_KIND_FULL, zb.ZB_DTYPE_BF16, 1, 256, 1024, 4, 64, 1, 2)
    try:
        zb.zb_stage_create(d, 0, [16] * 4, [16] * 4)
    except zb.ZbError as e:
        assert e.status == zb.ZB_E_UNSUPPORTED  # head_dim 64
    else:
        raise AssertionError("head_dim 64 must be rejected")


def _status(fn, *args):
    st = fn(*args)
    return st, zb.lib().zb_last_error().decode()


def test_linear_entry_points_reject_bad_arguments_before_any_launch():
    """Host-side checks of the bf16 linear passes: each case below is refused
    before the library makes its first HIP call (the addresses are never
    dereferenced), so this runs without a GPU."""
    L = zb.lib()
    bf16, fp32 = zb.ZB_DTYPE_BF16, zb.ZB_DTYPE_FP32
    p = 1 << 20  # 16-byte aligned stand-in address
    # Buffer offsets are 32-bit: an operand whose extent reaches 2 GiB is refused.
    st, msg = _status(L.zb_linear_forward, bf16, 1 << 20, 1024, 8, p, p, p, None)
    assert st == zb.ZB_E_UNSUPPORTED and "2 GiB" in msg, msg           # x: 2^20 x 1024 bf16 = 2 GiB
    st, msg = _status(L.zb_linear_backward_input, bf16, 8, 8, 1 << 27, p, p, p, None)
    assert st == zb.ZB_E_UNSUPPORTED and "2 GiB" in msg, msg           # dy: 8 x 2^27 bf16 = 2 GiB
    st, msg = _status(L.zb_linear_backward_weight, bf16, 8, 1 << 14, 1 << 15, p, p, p, 1, None)
    assert st == zb.ZB_E_UNSUPPORTED and "2 GiB" in msg, msg           # dw: 2^14 x 2^15 fp32 = 2 GiB
    # 16-byte vectors along every contiguous dimension.
    st, msg = _status(L.zb_linear_forward, bf16, 64, 60, 64, p, p, p, None)
    assert st == zb.ZB_E_UNSUPPORTED and "multiples of 8" in msg, msg  # K = 60
    st, msg = _status(L.zb_linear_forward, bf16, 64, 64, 64, p + 8, p, p, None)
    assert st == zb.ZB_E_UNSUPPORTED, msg                              # x 8-byte aligned only
    st, msg = _status(L.zb_linear_backward_weight, bf16, 64, 64, 60, p, p, p, 0, None)
    assert st == zb.ZB_E_UNSUPPORTED, msg                              # N = 60
    # Argument errors.
    for fn in (L.zb_linear_forward, L.zb_linear_backward_input):
        assert _status(fn, bf16, -1, 64, 64, p, p, p, None)[0] == zb.ZB_E_ARG
        assert _status(fn, bf16, 64, 64, 64, None, p, p, None)[0] == zb.ZB_E_ARG
        assert _status(fn, bf16, 64, 64, 64, p, p, None, None)[0] == zb.ZB_E_ARG
        assert _status(fn, 7, 64, 64, 64, p, p, p, None)[0] == zb.ZB_E_ARG
    assert _status(L.zb_linear_backward_weight, bf16, 64, 64, -8, p, p, p, 0, None)[0] == zb.ZB_E_ARG
    assert _status(L.zb_linear_backward_weight, fp32, 64, 64, 64, p, None, p, 0, None)[0] == zb.ZB_E_ARG
    # Empty outputs are legal and launch nothing.
    assert _status(L.zb_linear_forward, bf16, 0, 64, 64, None, None, None, None)[0] == zb.ZB_OK
    assert _status(L.zb_linear_backward_weight, bf16, 64, 0, 64, None, None, None, 1, None)[0] == zb.ZB_OK
