"""ctypes binding of libflint_moe.so (argument marshalling only).

Every step of the layer runs in the library's HIP kernels; this module only
checks that tensors live on the GPU and are contiguous, passes their device
pointers and the current HIP stream, and turns status codes into exceptions.
PyTorch provides device memory and streams, nothing else.  If the library is
missing the import fails loudly: there is no CPU fallback.

Names follow the C ABI (include/flint_moe.h): flint_moe_create,
flint_moe_forward, flint_moe_get_routing, flint_moe_destroy,
flint_rmsnorm_forward, plus a small MoELayer wrapper around a handle.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libflint_moe.so")

FLINT_OK, FLINT_ERR_INVALID_ARG, FLINT_ERR_UNSUPPORTED = 0, 1, 2
FLINT_ERR_OUT_OF_MEMORY, FLINT_ERR_NO_DEVICE, FLINT_ERR_HIP = 3, 4, 5
FLINT_F32, FLINT_BF16, FLINT_NVFP4 = 0, 1, 2
FLINT_FORCE_DECODE_PATH, FLINT_FORCE_PREFILL_PATH = 0x1, 0x2
FLINT_DEBUG_POISON_WORKSPACE = 0x4
FLINT_UNFUSED_DECODE = 0x8
(KERNEL_ROUTE, KERNEL_SORT, KERNEL_EXPERT_UP, KERNEL_EXPERT_DOWN, KERNEL_COMBINE, KERNEL_FUSED,
 KERNEL_FORWARD) = range(7)

EXPORTED = [
    "flint_moe_create", "flint_moe_forward", "flint_moe_get_routing", "flint_moe_profile_begin",
    "flint_moe_profile_end", "flint_moe_destroy", "flint_status_string", "flint_last_error",
    "flint_rmsnorm_forward", "flint_moe_forward_noalloc", "flint_moe_get_fault",
    "flint_moe_forward_prenorm",
]


class FlintError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__("%s: %s" % (_status_name(status), detail))
        self.status = status


class flint_moe_config(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("d_model", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("d_ff_shared", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("weight_dtype", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class flint_expert_weights(ctypes.Structure):
    _fields_ = [("gate_up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("gate_up_scales", ctypes.c_void_p), ("down_scales", ctypes.c_void_p),
                ("tensor_scales", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libflint_moe.so and declare the C signatures (no device call)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libflint_moe.so is not built (%s); run "
                          "`python -m sparse_moe_transformer_gemv_amd.build`" % path)
    L = ctypes.CDLL(path)
    vp, i32, u32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_int
    L.flint_moe_create.argtypes = [ctypes.POINTER(flint_moe_config), ctypes.POINTER(vp)]
    L.flint_moe_create.restype = st
    L.flint_moe_forward.argtypes = [vp, i32, vp, vp, vp, ctypes.POINTER(flint_expert_weights),
                                    ctypes.POINTER(flint_expert_weights), vp, vp, vp]
    L.flint_moe_forward.restype = st
    L.flint_moe_forward_noalloc.argtypes = [ctypes.POINTER(flint_moe_config), i32, vp, vp, vp,
                                            ctypes.POINTER(flint_expert_weights),
                                            ctypes.POINTER(flint_expert_weights), vp, vp, vp]
    L.flint_moe_forward_noalloc.restype = st
    L.flint_moe_get_routing.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.POINTER(i32), vp]
    L.flint_moe_get_routing.restype = st
    L.flint_moe_get_fault.argtypes = [vp, vp, vp]
    L.flint_moe_forward_prenorm.argtypes = [vp, i32, vp, vp, vp, ctypes.POINTER(flint_expert_weights),
                                            ctypes.POINTER(flint_expert_weights), vp, vp, ctypes.c_float, vp, vp]
    L.flint_moe_forward_prenorm.restype = st
    L.flint_moe_get_fault.restype = st
    L.flint_moe_profile_begin.argtypes = [vp, i32, i32]
    L.flint_moe_profile_begin.restype = st
    L.flint_moe_profile_end.argtypes = [vp, ctypes.POINTER(ctypes.c_float), i32,
                                        ctypes.POINTER(i32)]
    L.flint_moe_profile_end.restype = st
    L.flint_moe_destroy.argtypes = [vp]
    L.flint_moe_destroy.restype = st
    L.flint_status_string.argtypes = [st]
    L.flint_status_string.restype = ctypes.c_char_p
    L.flint_last_error.argtypes = []
    L.flint_last_error.restype = ctypes.c_char_p
    L.flint_rmsnorm_forward.argtypes = [i32, i32, vp, ctypes.c_float, vp, vp]
    L.flint_rmsnorm_forward.restype = st
    _lib = L
    return L


def _status_name(s: int) -> str:
    try:
        return load_library().flint_status_string(s).decode()
    except Exception:  # noqa: BLE001 - only used to label an error
        return "status %d" % s


def _check(status: int):
    if status != FLINT_OK:
        raise FlintError(status, load_library().flint_last_error().decode())


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return t.data_ptr()


_TORCH_ACT = {FLINT_F32: torch.float32, FLINT_BF16: torch.bfloat16}
_TORCH_W = {FLINT_F32: torch.float32, FLINT_BF16: torch.bfloat16, FLINT_NVFP4: torch.uint8}


def _expect(t, name, numel, dtype, device):
    """t must be a contiguous tensor of `numel` elements of `dtype` on `device`."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.device != device:
        raise ValueError("%s is on %s, the layer runs on %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.numel() != numel:
        raise ValueError("%s holds %d elements, the configuration needs %d" % (name, t.numel(), numel))


def check_expert_weights(w, cfg, n: int, f: int, device, name: str) -> None:
    """Sizes, dtypes and device of one expert set of n experts of width f
    (layouts of include/flint_moe.h)."""
    d, wd = cfg.d_model, cfg.weight_dtype
    if not isinstance(w, ExpertWeights):
        raise TypeError("%s must be ExpertWeights" % name)
    if wd == FLINT_NVFP4:
        _expect(w.gate_up, name + ".gate_up", n * 2 * f * d // 2, torch.uint8, device)
        _expect(w.down, name + ".down", n * d * f // 2, torch.uint8, device)
        _expect(w.gate_up_scales, name + ".gate_up_scales", n * 2 * f * d // 16, torch.uint8, device)
        _expect(w.down_scales, name + ".down_scales", n * d * f // 16, torch.uint8, device)
        _expect(w.tensor_scales, name + ".tensor_scales", n * 3, torch.float32, device)
    else:
        _expect(w.gate_up, name + ".gate_up", n * 2 * f * d, _TORCH_W[wd], device)
        _expect(w.down, name + ".down", n * d * f, _TORCH_W[wd], device)
        for s in ("gate_up_scales", "down_scales", "tensor_scales"):
            if getattr(w, s) is not None:
                raise ValueError("%s.%s must be None unless the weights are NVFP4" % (name, s))


def check_forward_args(cfg, device, x, router_w, experts, shared, router_bias=None,
                       residual=None, out=None) -> None:
    """Every tensor of a forward against the layer configuration, before any
    pointer reaches the library: the C ABI sees raw device pointers and cannot
    tell an undersized or misplaced tensor from a good one.

    x [T, d] act dtype; router_w [E, d] fp32; router_bias None or [E] fp32;
    experts / shared: ExpertWeights of E experts of width f / one of width f_s
    (shared None exactly when f_s == 0); residual None or [T, d] fp32; out
    None or [T, d], fp32 when a residual is given, else the act dtype.  All on
    `device`."""
    d, E = cfg.d_model, cfg.n_experts
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.shape[1] != d:
        raise ValueError("x must be [T, %d]" % d)
    T = x.shape[0]
    _expect(x, "x", T * d, _TORCH_ACT[cfg.act_dtype], device)
    _expect(router_w, "router_w", E * d, torch.float32, device)
    if router_bias is not None:
        _expect(router_bias, "router_bias", E, torch.float32, device)
    check_expert_weights(experts, cfg, E, cfg.d_ff, device, "experts")
    if cfg.d_ff_shared > 0:
        if shared is None:
            raise ValueError("the layer has a shared expert (d_ff_shared = %d): pass its weights"
                             % cfg.d_ff_shared)
        check_expert_weights(shared, cfg, 1, cfg.d_ff_shared, device, "shared")
    elif shared is not None:
        raise ValueError("shared weights given but d_ff_shared == 0")
    if residual is not None:
        _expect(residual, "residual", T * d, torch.float32, device)
        if residual.shape != (T, d):
            raise ValueError("residual must be [T, d] = [%d, %d]" % (T, d))
    if out is not None:
        odt = torch.float32 if residual is not None else _TORCH_ACT[cfg.act_dtype]
        _expect(out, "out", T * d, odt, device)
        if out.shape != (T, d):
            raise ValueError("out must be [T, d] = [%d, %d]" % (T, d))


@dataclass
class ExpertWeights:
    """Device tensors of one expert set (layouts as in include/flint_moe.h)."""
    gate_up: torch.Tensor
    down: torch.Tensor
    gate_up_scales: Optional[torch.Tensor] = None
    down_scales: Optional[torch.Tensor] = None
    tensor_scales: Optional[torch.Tensor] = None

    def as_c(self, wdtype: int) -> flint_expert_weights:
        wt = _TORCH_W[wdtype]
        return flint_expert_weights(
            _ptr(self.gate_up, "gate_up", wt), _ptr(self.down, "down", wt),
            _ptr(self.gate_up_scales, "gate_up_scales", torch.uint8),
            _ptr(self.down_scales, "down_scales", torch.uint8),
            _ptr(self.tensor_scales, "tensor_scales", torch.float32))


def flint_moe_create(cfg: flint_moe_config) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(load_library().flint_moe_create(ctypes.byref(cfg), ctypes.byref(h)))
    return h


def flint_moe_destroy(h) -> None:
    _check(load_library().flint_moe_destroy(h))


def flint_rmsnorm_forward(x: torch.Tensor, eps: float = 1e-6,
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16(x / sqrt(mean(x^2) + eps)) per row; x [T, d] fp32 on the GPU."""
    if x.dim() != 2:
        raise ValueError("x must be [T, d]")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    _check(load_library().flint_rmsnorm_forward(x.shape[0], x.shape[1],
                                                _ptr(x, "x", torch.float32), eps,
                                                _ptr(out, "out", torch.bfloat16), _stream()))
    return out


def flint_moe_forward_noalloc(cfg: flint_moe_config, x: torch.Tensor, router_w: torch.Tensor,
                              experts: ExpertWeights, shared: Optional[ExpertWeights],
                              out: torch.Tensor, router_bias: Optional[torch.Tensor] = None,
                              residual: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The layer through the allocation-free entry point (static device
    scratch; no handle).  `out` must be given: nothing is allocated here."""
    device = torch.device("cuda", torch.cuda.current_device())
    check_forward_args(cfg, device, x, router_w, experts, shared, router_bias, residual, out)
    ew = experts.as_c(cfg.weight_dtype)
    sw = shared.as_c(cfg.weight_dtype) if shared is not None else None
    _check(load_library().flint_moe_forward_noalloc(
        ctypes.byref(cfg), x.shape[0], _ptr(x, "x"), _ptr(router_w, "router_w"),
        _ptr(router_bias, "router_bias"), ctypes.byref(ew),
        ctypes.byref(sw) if sw is not None else None, _ptr(residual, "residual"),
        _ptr(out, "out"), _stream()))
    return out


class MoELayer:
    """One handle (workspace) of the MoE layer; serves any number of weight sets."""

    def __init__(self, d_model: int, n_experts: int = 256, top_k: int = 6, d_ff: int = 512,
                 d_ff_shared: int = 512, act_dtype: int = FLINT_BF16,
                 weight_dtype: int = FLINT_BF16, max_tokens: int = 64, flags: int = 0):
        load_library()
        self.cfg = flint_moe_config(ctypes.sizeof(flint_moe_config), d_model, n_experts, top_k,
                                    d_ff, d_ff_shared, act_dtype, weight_dtype, max_tokens, flags)
        self.device = torch.device("cuda", torch.cuda.current_device())
        self.handle = flint_moe_create(self.cfg)

    def close(self):
        if getattr(self, "handle", None):
            flint_moe_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass

    def forward(self, x: torch.Tensor, router_w: torch.Tensor, experts: ExpertWeights,
                shared: Optional[ExpertWeights], router_bias: Optional[torch.Tensor] = None,
                residual: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
        c = self.cfg
        check_forward_args(c, self.device, x, router_w, experts, shared, router_bias, residual,
                           out)
        T = x.shape[0]
        if out is None:
            odt = torch.float32 if residual is not None else _TORCH_ACT[c.act_dtype]
            out = torch.empty((T, c.d_model), dtype=odt, device=x.device)
        ew = experts.as_c(c.weight_dtype)
        sw = shared.as_c(c.weight_dtype) if shared is not None else None
        _check(load_library().flint_moe_forward(
            self.handle, T, _ptr(x, "x", _TORCH_ACT[c.act_dtype]),
            _ptr(router_w, "router_w", torch.float32),
            _ptr(router_bias, "router_bias", torch.float32), ctypes.byref(ew),
            ctypes.byref(sw) if sw is not None else None,
            _ptr(residual, "residual", torch.float32), _ptr(out, "out"), _stream()))
        return out

    __call__ = forward

    def forward_prenorm(self, x: torch.Tensor, router_w: torch.Tensor, experts: ExpertWeights,
                        shared: Optional[ExpertWeights], residual: torch.Tensor, eps: float = 1e-6,
                        router_bias: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                        norm_out: Optional[torch.Tensor] = None):
        """One pre-norm residual step: out = residual + MoE(x) (fp32) and
        norm_out = bf16(RMSNorm(out)), the next layer's input.  Returns (out, norm_out)."""
        c = self.cfg
        if residual is None:
            raise ValueError("forward_prenorm needs the fp32 residual")
        check_forward_args(c, self.device, x, router_w, experts, shared, router_bias, residual, out)
        T = x.shape[0]
        if out is None:
            out = torch.empty((T, c.d_model), dtype=torch.float32, device=x.device)
        if norm_out is None:
            norm_out = torch.empty((T, c.d_model), dtype=torch.bfloat16, device=x.device)
        _expect(norm_out, "norm_out", T * c.d_model, torch.bfloat16, self.device)
        ew = experts.as_c(c.weight_dtype)
        sw = shared.as_c(c.weight_dtype) if shared is not None else None
        _check(load_library().flint_moe_forward_prenorm(
            self.handle, T, _ptr(x, "x", _TORCH_ACT[c.act_dtype]),
            _ptr(router_w, "router_w", torch.float32),
            _ptr(router_bias, "router_bias", torch.float32), ctypes.byref(ew),
            ctypes.byref(sw) if sw is not None else None,
            _ptr(residual, "residual", torch.float32), _ptr(out, "out"), float(eps),
            _ptr(norm_out, "norm_out"), _stream()))
        return out, norm_out

    def routing(self) -> dict:
        """Routing of the last forward: idx, weights, sorted_pair, counts, logits."""
        c = self.cfg
        T = ctypes.c_int32(0)
        _check(load_library().flint_moe_get_routing(self.handle, None, None, None, None, None,
                                                    ctypes.byref(T), _stream()))
        T = T.value
        dev = torch.device("cuda", torch.cuda.current_device())
        r = {"idx": torch.empty((T, c.top_k), dtype=torch.int32, device=dev),
             "weights": torch.empty((T, c.top_k), dtype=torch.float32, device=dev),
             "sorted_pair": torch.empty((T * c.top_k,), dtype=torch.int32, device=dev),
             "counts": torch.empty((c.n_experts,), dtype=torch.int32, device=dev),
             "logits": torch.empty((T, c.n_experts), dtype=torch.float32, device=dev)}
        _check(load_library().flint_moe_get_routing(
            self.handle, r["idx"].data_ptr(), r["weights"].data_ptr(),
            r["sorted_pair"].data_ptr(), r["counts"].data_ptr(), r["logits"].data_ptr(), None,
            _stream()))
        return r

    def fault(self) -> int:
        """The single-launch decode kernel's sticky fault word (0: no wait gave up)."""
        dev = torch.device("cuda", torch.cuda.current_device())
        f = torch.full((1,), -1, dtype=torch.int32, device=dev)
        _check(load_library().flint_moe_get_fault(self.handle, f.data_ptr(), _stream()))
        return int(f.item())

    def profile_begin(self, kernel_id: int, n_launches: int) -> None:
        _check(load_library().flint_moe_profile_begin(self.handle, kernel_id, n_launches))

    def profile_end(self, cap: int = 100000) -> list:
        buf = (ctypes.c_float * cap)()
        n = ctypes.c_int32(0)
        _check(load_library().flint_moe_profile_end(self.handle, buf, cap, ctypes.byref(n)))
        return [buf[i] for i in range(n.value)]


class DenseFFN:
    """A dense SwiGLU feed-forward layer, out = [residual +] D (SiLU(G x) * (U x)).

    The first layers of the model are dense rather than mixture-of-experts
    [evermx.com, "Recursive Flint: Open-Weight MoE Coding Model, 2.5B Active",
    Feature Overview, "Sparse architecture"]; their width is a parameter.  The
    MoE engine runs it unchanged, configured with one routed expert, top-1 and no
    shared expert: the router is all zeros, the renormalised softmax over the one
    chosen logit is exactly 1, and the layer output is that expert's output.
    Weights use the layout of one expert: gate_up [1][2F][d] (gate rows first),
    down [1][d][F]; NVFP4 adds the scales of one expert.
    """

    def __init__(self, d_model: int, d_ff: int, act_dtype: int = FLINT_BF16,
                 weight_dtype: int = FLINT_BF16, max_tokens: int = 64, flags: int = 0):
        self.layer = MoELayer(d_model, 1, 1, d_ff, 0, act_dtype, weight_dtype, max_tokens, flags)
        self.router_w = torch.zeros((1, d_model), dtype=torch.float32,
                                    device=torch.device("cuda", torch.cuda.current_device()))

    def close(self):
        self.layer.close()

    def forward(self, x: torch.Tensor, weights: ExpertWeights,
                residual: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
        return self.layer.forward(x, self.router_w, weights, None, None, residual, out)

    __call__ = forward
