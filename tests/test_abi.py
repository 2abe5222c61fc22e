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
