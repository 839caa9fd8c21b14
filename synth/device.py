"""Upload the seeded host tensors of ``synth`` to the GPU, and read outputs back.

Marshalling only (no arithmetic of the layer): bf16 tensors travel as their
raw bits, NVFP4 tensors as their packed bytes.  Used by the tests, the smoke
check and the benchmark.
"""
from __future__ import annotations

import numpy as np
import torch

from . import BF16, NVFP4


def dev_array(a: np.ndarray, bf16: bool = False) -> torch.Tensor:
    """A host array on the current GPU; ``bf16=True`` reinterprets uint16 bits."""
    if bf16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.cuda()


def dev_weights(ws: dict, wdtype: int):
    """One expert set (synth.expert_set) as device tensors."""
    from sparse_moe_transformer_gemv_amd import ExpertWeights
    if wdtype == NVFP4:
        return ExpertWeights(dev_array(ws["gate_up"]), dev_array(ws["down"]),
                             dev_array(ws["gate_up_scales"]), dev_array(ws["down_scales"]),
                             dev_array(ws["tensor_scales"]))
    bf = wdtype == BF16
    return ExpertWeights(dev_array(ws["gate_up"], bf), dev_array(ws["down"], bf))


def dev_layer(L: dict) -> dict:
    """A whole layer (synth.layer) as device tensors."""
    wd = L["cfg"]["wdtype"]
    return {"router_w": dev_array(L["router_w"]),
            "router_bias": None if L["router_bias"] is None else dev_array(L["router_bias"]),
            "experts": dev_weights(L["experts"], wd),
            "shared": None if L["shared"] is None else dev_weights(L["shared"], wd)}


def x_device(x: np.ndarray) -> torch.Tensor:
    """Token activations (fp32, or bf16 bits) on the GPU."""
    return dev_array(x, bf16=(x.dtype == np.uint16))


def out_host(out: torch.Tensor) -> np.ndarray:
    """A layer output (fp32 or bf16) as a float64 host array (exact)."""
    return out.float().cpu().numpy().astype(np.float64)


def make_layer_obj(cfg: dict, max_tokens: int, flags: int = 0):
    """A MoELayer handle for configuration dict ``cfg`` (synth.CONFIGS entry)."""
    from sparse_moe_transformer_gemv_amd import MoELayer
    return MoELayer(cfg["d"], cfg["E"], cfg["k"], cfg["f"], cfg["fs"], cfg["act"], cfg["wdtype"],
                    max_tokens, flags)
