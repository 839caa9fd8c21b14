"""The C ABI without a GPU: the library loads, exports every declared entry
point, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

import sparse_moe_transformer_gemv_amd as fm
from sparse_moe_transformer_gemv_amd import flint_moe as b

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "flint_moe.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flint_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = fm.load_library()
    names = _declared()
    assert "flint_moe_forward" in names and len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    assert sorted(b.EXPORTED) == sorted(names)


def _cfg(**kw):
    c = dict(d_model=2048, n_experts=256, top_k=6, d_ff=512, d_ff_shared=512, act_dtype=1,
             weight_dtype=1, max_tokens=64, flags=0)
    c.update(kw)
    return fm.flint_moe_config(ctypes.sizeof(fm.flint_moe_config), c["d_model"], c["n_experts"],
                               c["top_k"], c["d_ff"], c["d_ff_shared"], c["act_dtype"],
                               c["weight_dtype"], c["max_tokens"], c["flags"])


@pytest.mark.parametrize("bad", [
    dict(d_model=100), dict(d_model=0), dict(n_experts=0), dict(n_experts=300),
    dict(top_k=0), dict(top_k=9), dict(n_experts=4, top_k=5), dict(d_ff=48),
    dict(d_ff_shared=-32), dict(act_dtype=2), dict(weight_dtype=7), dict(max_tokens=0),
    dict(max_tokens=70000), dict(flags=0x10), dict(flags=0x3),
])
def test_create_rejects_bad_config_before_device(bad):
    L = fm.load_library()
    h = ctypes.c_void_p()
    st = L.flint_moe_create(ctypes.byref(_cfg(**bad)), ctypes.byref(h))
    assert st == b.FLINT_ERR_INVALID_ARG, (bad, st, L.flint_last_error())
    assert h.value is None
    assert L.flint_last_error()


def test_create_rejects_wrong_struct_size_and_nulls():
    L = fm.load_library()
    c = _cfg()
    c.struct_size = 12
    h = ctypes.c_void_p()
    assert L.flint_moe_create(ctypes.byref(c), ctypes.byref(h)) == b.FLINT_ERR_INVALID_ARG
    assert L.flint_moe_create(None, ctypes.byref(h)) == b.FLINT_ERR_INVALID_ARG
    assert L.flint_moe_create(ctypes.byref(_cfg()), None) == b.FLINT_ERR_INVALID_ARG


def test_prefill_flag_needs_bf16():
    L = fm.load_library()
    h = ctypes.c_void_p()
    st = L.flint_moe_create(ctypes.byref(_cfg(flags=0x2, weight_dtype=2)), ctypes.byref(h))
    assert st == b.FLINT_ERR_UNSUPPORTED


def test_valid_config_without_gpu_reports_no_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    L = fm.load_library()
    h = ctypes.c_void_p()
    assert L.flint_moe_create(ctypes.byref(_cfg()), ctypes.byref(h)) == b.FLINT_ERR_NO_DEVICE
    assert b"no HIP device" in L.flint_last_error() or b"gfx950" in L.flint_last_error()


def test_null_handle_calls_are_rejected():
    L = fm.load_library()
    assert L.flint_moe_forward(None, 1, None, None, None, None, None, None, None,
                               None) == b.FLINT_ERR_INVALID_ARG
    assert L.flint_moe_destroy(None) == b.FLINT_ERR_INVALID_ARG
    assert L.flint_moe_get_routing(None, None, None, None, None, None, None,
                                   None) == b.FLINT_ERR_INVALID_ARG
    assert L.flint_moe_profile_begin(None, 0, 1) == b.FLINT_ERR_INVALID_ARG
    n = ctypes.c_int32(0)
    assert L.flint_moe_profile_end(None, None, 0, ctypes.byref(n)) == b.FLINT_ERR_INVALID_ARG


def test_rmsnorm_argument_checks():
    L = fm.load_library()
    assert L.flint_rmsnorm_forward(4, 100, None, 1e-6, None, None) == b.FLINT_ERR_INVALID_ARG
    assert L.flint_rmsnorm_forward(-1, 128, None, 1e-6, None, None) == b.FLINT_ERR_INVALID_ARG
    # T == 0 with valid-looking pointers is a no-op, no device needed
    buf = (ctypes.c_float * 64)()
    out = (ctypes.c_uint16 * 64)()
    assert L.flint_rmsnorm_forward(0, 64, ctypes.cast(buf, ctypes.c_void_p), 1e-6,
                                   ctypes.cast(out, ctypes.c_void_p), None) == b.FLINT_OK


def test_status_strings():
    L = fm.load_library()
    for s in range(6):
        assert L.flint_status_string(s).startswith(b"FLINT_")
    assert L.flint_status_string(42) == b"FLINT_ERR_UNKNOWN"
