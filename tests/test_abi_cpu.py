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


def test_prefill_flag_needs_bf16_activations_and_bf16_or_nvfp4_weights():
    L = fm.load_library()
    h = ctypes.c_void_p()
    for bad in (dict(weight_dtype=0), dict(act_dtype=0)):
        st = L.flint_moe_create(ctypes.byref(_cfg(flags=0x2, **bad)), ctypes.byref(h))
        assert st == b.FLINT_ERR_UNSUPPORTED, bad


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
    assert L.flint_moe_get_fault(None, None, None) == b.FLINT_ERR_INVALID_ARG
    assert L.flint_moe_forward_prenorm(None, 1, None, None, None, None, None, None, None, 1e-6, None,
                                       None) == b.FLINT_ERR_INVALID_ARG
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


# ------------------------------------------------ binding checks of forward tensors

def _tensors(wd=1, T=3, d=128, E=8, f=32, fs=32, residual=False, out=True):
    import torch
    act = torch.bfloat16
    wt = {0: torch.float32, 1: torch.bfloat16, 2: torch.uint8}[wd]

    def ws(n, F):
        if wd == 2:
            return fm.ExpertWeights(torch.zeros(n, 2 * F, d // 2, dtype=torch.uint8),
                                    torch.zeros(n, d, F // 2, dtype=torch.uint8),
                                    torch.zeros(n, 2 * F, d // 16, dtype=torch.uint8),
                                    torch.zeros(n, d, F // 16, dtype=torch.uint8),
                                    torch.ones(n, 3, dtype=torch.float32))
        return fm.ExpertWeights(torch.zeros(n, 2 * F, d, dtype=wt), torch.zeros(n, d, F, dtype=wt))

    a = dict(x=torch.zeros(T, d, dtype=act), router_w=torch.zeros(E, d), experts=ws(E, f),
             shared=ws(1, fs) if fs else None, router_bias=None,
             residual=torch.zeros(T, d) if residual else None)
    a["out"] = (torch.zeros(T, d) if residual else torch.zeros(T, d, dtype=act)) if out else None
    return a


def _check(a, wd=1, fs=32):
    import torch
    cfg = _cfg(d_model=128, n_experts=8, d_ff=32, d_ff_shared=fs, weight_dtype=wd)
    b.check_forward_args(cfg, torch.device("cpu"), a["x"], a["router_w"], a["experts"],
                         a["shared"], a["router_bias"], a["residual"], a["out"])


@pytest.mark.parametrize("wd", [0, 1, 2])
@pytest.mark.parametrize("residual", [False, True])
def test_binding_accepts_matching_tensors(wd, residual):
    _check(_tensors(wd, residual=residual), wd)
    _check(_tensors(wd, fs=0), wd, fs=0)


def _bad_cases():
    import torch
    cases = []

    def mk(label, fn, wd=1, fs=32, exc=(ValueError, TypeError)):
        cases.append(pytest.param(fn, wd, fs, exc, id=label))

    mk("bf16 out with fp32 residual",
       lambda a: a.update(residual=torch.zeros(3, 128), out=torch.zeros(3, 128, dtype=torch.bfloat16)))
    mk("out too short", lambda a: a.update(out=torch.zeros(2, 128, dtype=torch.bfloat16)))
    mk("out fp32 without residual", lambda a: a.update(out=torch.zeros(3, 128)))
    mk("residual wrong shape", lambda a: a.update(residual=torch.zeros(3, 64), out=torch.zeros(3, 128)))
    mk("x wrong width", lambda a: a.update(x=torch.zeros(3, 64, dtype=torch.bfloat16)))
    mk("x fp32 for a bf16 layer", lambda a: a.update(x=torch.zeros(3, 128)))
    mk("router rows short", lambda a: a.update(router_w=torch.zeros(7, 128)))
    mk("router bf16", lambda a: a.update(router_w=torch.zeros(8, 128, dtype=torch.bfloat16)))
    mk("bias length", lambda a: a.update(router_bias=torch.zeros(7)))
    mk("gate_up short",
       lambda a: a.update(experts=fm.ExpertWeights(torch.zeros(7, 64, 128, dtype=torch.bfloat16),
                                                   a["experts"].down)))
    mk("down short",
       lambda a: a.update(experts=fm.ExpertWeights(a["experts"].gate_up,
                                                   torch.zeros(8, 128, 16, dtype=torch.bfloat16))))
    mk("shared missing", lambda a: a.update(shared=None))
    mk("shared given without width", lambda a: None, fs=0)
    mk("scales on bf16 weights",
       lambda a: a.update(experts=fm.ExpertWeights(a["experts"].gate_up, a["experts"].down,
                                                   torch.zeros(8, 64, 8, dtype=torch.uint8))))
    mk("non-contiguous x", lambda a: a.update(x=torch.zeros(128, 3, dtype=torch.bfloat16).t()))
    mk("nvfp4 scales short",
       lambda a: a.update(experts=fm.ExpertWeights(a["experts"].gate_up, a["experts"].down,
                                                   a["experts"].gate_up_scales[:7],
                                                   a["experts"].down_scales,
                                                   a["experts"].tensor_scales)), wd=2)
    mk("nvfp4 tensor scales missing",
       lambda a: a.update(shared=fm.ExpertWeights(a["shared"].gate_up, a["shared"].down,
                                                  a["shared"].gate_up_scales,
                                                  a["shared"].down_scales, None)), wd=2)
    return cases


@pytest.mark.parametrize("mutate,wd,fs,exc", _bad_cases())
def test_binding_rejects_mismatched_tensors(mutate, wd, fs, exc):
    a = _tensors(wd)
    mutate(a)
    with pytest.raises(exc):
        _check(a, wd, fs=fs)


def test_binding_rejects_tensor_on_another_device():
    import torch
    a = _tensors(1)
    cfg = _cfg(d_model=128, n_experts=8, d_ff=32, d_ff_shared=32)
    with pytest.raises(ValueError, match="is on"):
        b.check_forward_args(cfg, torch.device("meta"), a["x"], a["router_w"], a["experts"],
                             a["shared"], None, None, a["out"])


def test_noalloc_entry_point_checks_before_device():
    L = fm.load_library()
    args = (None,) * 8
    # a bad configuration and a T out of range are argument errors
    assert L.flint_moe_forward_noalloc(ctypes.byref(_cfg(top_k=9)), 4, *args) == b.FLINT_ERR_INVALID_ARG
    assert L.flint_moe_forward_noalloc(None, 4, *args) == b.FLINT_ERR_INVALID_ARG
    assert L.flint_moe_forward_noalloc(ctypes.byref(_cfg()), -1, *args) == b.FLINT_ERR_INVALID_ARG
    # T = 0 is a no-op
    assert L.flint_moe_forward_noalloc(ctypes.byref(_cfg()), 0, *args) == b.FLINT_OK
    # a workspace larger than the static scratch is refused by size, before any device call
    assert L.flint_moe_forward_noalloc(ctypes.byref(_cfg()), 4096, *args) == b.FLINT_ERR_INVALID_ARG
    assert b"static scratch" in L.flint_last_error()
    import torch
    if not torch.cuda.is_available():
        # a size that fits gets as far as the device check
        assert L.flint_moe_forward_noalloc(ctypes.byref(_cfg()), 128, *args) == b.FLINT_ERR_NO_DEVICE
