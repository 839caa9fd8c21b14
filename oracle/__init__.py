"""Plain fp64 CPU oracle of the Flint routed-expert MoE layer.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are its only users.  The product library never imports,
loads or calls anything here, and this package imports nothing from the
product package.  The arithmetic lives in ``moe_oracle.c`` (fp64, index-order
sums); this module only compiles it with gcc, marshals numpy arrays in their
stored formats, and adds the per-row RMSNorm stack of the 47-layer
configuration.

Stored formats understood here: fp32 (``np.float32``), bf16 as raw bits
(``np.uint16``), NVFP4 as packed E2M1 codes (``np.uint8``, even element in the
low nibble) plus E4M3 block-scale codes (``np.uint8``, one per 16 elements
along K) and fp32 per-tensor scales ``[n][3] = {gate, up, down}``.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

__all__ = [
    "build", "lib", "F32", "BF16", "NVFP4",
    "moe_forward", "route", "expert_forward", "ffn_forward", "rmsnorm", "round_to_bf16",
    "bf16_value", "e2m1_value", "e4m3_value", "silu", "stack_forward",
]

F32, BF16, NVFP4 = 0, 1, 2

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "moe_oracle.c")
_SO = os.path.join(_DIR, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile moe_oracle.c with gcc (fp64, OpenMP, no FMA contraction)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-Wno-unknown-pragmas", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = load_library(_SO)
    return _lib


@contextlib.contextmanager
def using_library(path):
    """Run the wrappers against another build of moe_oracle.c (used by the
    test that plants mistakes in a copy of the oracle)."""
    global _lib
    saved = _lib
    _lib = load_library(path)
    try:
        yield _lib
    finally:
        _lib = saved


def load_library(path):
    """Load a build of moe_oracle.c and declare its signatures."""
    L = ctypes.CDLL(path)
    vp, ip, dp = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
    L.oracle_moe_forward.restype = ip
    L.oracle_moe_forward.argtypes = [ip] * 8 + [vp] * 17
    L.oracle_route.restype = ip
    L.oracle_route.argtypes = [ip] * 5 + [vp] * 6
    L.oracle_expert_forward.restype = ip
    L.oracle_expert_forward.argtypes = [ip, ip, ip, ctypes.c_long] + [vp] * 7
    L.oracle_rmsnorm.restype = None
    L.oracle_rmsnorm.argtypes = [ip, ip, vp, dp, vp]
    L.oracle_bf16_value.restype = dp
    L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    L.oracle_e2m1_value.restype = dp
    L.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
    L.oracle_e4m3_value.restype = dp
    L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    L.oracle_round_to_bf16.restype = ctypes.c_uint16
    L.oracle_round_to_bf16.argtypes = [dp]
    L.oracle_silu.restype = dp
    L.oracle_silu.argtypes = [dp]
    return L


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s, got %s" % (np.dtype(dtype), a.dtype))
    return a


def _act_dtype(x):
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:
        return BF16
    raise TypeError("activations must be float32 or bf16 bits (uint16)")


def _weights(ws, wdtype):
    """Return (gate_up, down, gu_scales, dn_scales, tscales) made contiguous."""
    if wdtype == F32:
        return _c(ws["gate_up"], np.float32), _c(ws["down"], np.float32), None, None, None
    if wdtype == BF16:
        return _c(ws["gate_up"], np.uint16), _c(ws["down"], np.uint16), None, None, None
    return (_c(ws["gate_up"], np.uint8), _c(ws["down"], np.uint8),
            _c(ws["gate_up_scales"], np.uint8), _c(ws["down_scales"], np.uint8),
            _c(ws["tensor_scales"], np.float32))


def moe_forward(x, router_w, experts, shared, *, top_k=6, router_bias=None, wdtype=BF16,
                f=None, fs=None, want_logits=True):
    """fp64 layer output for the tokens in ``x``.

    x        [T, d] float32, or bf16 bits as uint16
    router_w [E, d] float32;  router_bias [E] float32 or None
    experts / shared: dicts with "gate_up", "down" (and the NVFP4 scale arrays)
    Returns a dict: out [T, d] fp64, idx [T, k] int32, w [T, k] fp64,
    logits [T, E] fp64.
    """
    x = np.ascontiguousarray(x)
    act = _act_dtype(x)
    T, d = x.shape
    router_w = _c(router_w, np.float32)
    E = router_w.shape[0]
    router_bias = _c(router_bias, np.float32)
    gu, dn, gs, ds, ts = _weights(experts, wdtype)
    if f is None:
        f = (gu.shape[1] // 2)
    if shared is not None:
        sgu, sdn, sgs, sds, sts = _weights(shared, wdtype)
        if fs is None:
            fs = sgu.shape[1] // 2
    else:
        sgu = sdn = sgs = sds = sts = None
        fs = 0
    out = np.zeros((T, d), np.float64)
    idx = np.zeros((T, top_k), np.int32)
    w = np.zeros((T, top_k), np.float64)
    logits = np.zeros((T, E), np.float64) if want_logits else None
    rc = lib().oracle_moe_forward(T, d, E, top_k, f, fs, act, wdtype, _p(x), _p(router_w),
                                  _p(router_bias), _p(gu), _p(dn), _p(gs), _p(ds), _p(ts),
                                  _p(sgu), _p(sdn), _p(sgs), _p(sds), _p(sts), _p(out),
                                  _p(idx), _p(w), _p(logits))
    if rc != 0:
        raise ValueError("oracle_moe_forward rejected its arguments")
    return {"out": out, "idx": idx, "w": w, "logits": logits}


def route(x, router_w, *, top_k=6, router_bias=None):
    """The router alone for the tokens in ``x`` (the same steps as moe_forward):
    returns idx [T, k] int32, w [T, k] fp64 and logits [T, E] fp64."""
    x = np.ascontiguousarray(x)
    act = _act_dtype(x)
    T, d = x.shape
    router_w = _c(router_w, np.float32)
    E = router_w.shape[0]
    router_bias = _c(router_bias, np.float32)
    idx = np.zeros((T, top_k), np.int32)
    w = np.zeros((T, top_k), np.float64)
    logits = np.zeros((T, E), np.float64)
    rc = lib().oracle_route(T, d, E, top_k, act, _p(x), _p(router_w), _p(router_bias), _p(idx),
                            _p(w), _p(logits))
    if rc != 0:
        raise ValueError("oracle_route rejected its arguments")
    return {"idx": idx, "w": w, "logits": logits}


def expert_forward(x, ws, e, *, wdtype=BF16, f=None):
    """One expert e on one fp64 vector x [d]."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    gu, dn, gs, ds, ts = _weights(ws, wdtype)
    d = x.shape[0]
    if f is None:
        f = gu.shape[1] // 2
    y = np.zeros(d, np.float64)
    rc = lib().oracle_expert_forward(d, f, wdtype, e, _p(gu), _p(dn), _p(gs), _p(ds), _p(ts),
                                     _p(x), _p(y))
    if rc != 0:
        raise ValueError("oracle_expert_forward rejected its arguments")
    return y


def ffn_forward(x, ws, *, wdtype=BF16):
    """fp64 output of a dense SwiGLU feed-forward layer for the tokens in ``x``.

    The model's first layers are dense, the rest mixture-of-experts
    [evermx.com, "Recursive Flint: Open-Weight MoE Coding Model, 2.5B Active",
    Feature Overview, "Sparse architecture"].  A dense layer applies the one
    SwiGLU feed-forward map that every expert is (width a parameter) to every
    token, so this is ``expert_forward`` of expert 0 of the weight set ``ws``
    (gate_up [1][2F][d], down [1][d][F], NVFP4 scales of one expert) per token.
    x [T, d] float32, or bf16 bits as uint16.  Returns [T, d] fp64.
    """
    x = np.ascontiguousarray(x)
    xv = bf16_value(x) if x.dtype == np.uint16 else x.astype(np.float64)
    return np.stack([expert_forward(xv[t], ws, 0, wdtype=wdtype) for t in range(xv.shape[0])])


def rmsnorm(h, eps=1e-6):
    h = np.ascontiguousarray(h, dtype=np.float64)
    out = np.zeros_like(h)
    lib().oracle_rmsnorm(h.shape[0], h.shape[1], _p(h), eps, _p(out))
    return out


def round_to_bf16(v):
    """fp64 array -> bf16 bits (uint16), nearest, ties to even."""
    v = np.asarray(v, dtype=np.float64)
    f = lib().oracle_round_to_bf16
    return np.array([f(float(a)) for a in v.ravel()], dtype=np.uint16).reshape(v.shape)


def bf16_value(bits):
    f = lib().oracle_bf16_value
    b = np.asarray(bits, dtype=np.uint16)
    return np.array([f(int(a)) for a in b.ravel()], dtype=np.float64).reshape(b.shape)


def e2m1_value(code):
    return lib().oracle_e2m1_value(int(code))


def e4m3_value(code):
    return lib().oracle_e4m3_value(int(code))


def silu(z):
    return lib().oracle_silu(float(z))


def stack_forward(h0, layers, *, top_k=6, eps=1e-6, wdtype=BF16):
    """The stacked configuration: h <- h + MoE_l(bf16(RMSNorm(h))) per layer.

    The MoE layer's activations are bf16, so its input is the nearest bf16 of
    the fp64 RMSNorm output; the residual stream h stays fp64.  ``layers`` is
    a sequence of dicts with "router_w", "experts", "shared" (an iterator is
    fine, so layers can be produced one at a time).  Returns the final h and
    the per-layer selections, weights and logits.
    """
    h = np.asarray(h0, dtype=np.float64).copy()
    trace = []
    for L in layers:
        y = rmsnorm(h, eps)
        xb = round_to_bf16(y)
        r = moe_forward(xb, L["router_w"], L["experts"], L["shared"], top_k=top_k,
                        router_bias=L.get("router_bias"), wdtype=wdtype)
        h = h + r["out"]
        trace.append({"idx": r["idx"], "w": r["w"], "logits": r["logits"], "x": xb,
                      "out_rms": float(np.sqrt(np.mean(r["out"] ** 2)))})
    return h, trace
