"""The allocation-free entry point (flint_moe_forward_noalloc, static device
scratch) against the handle-based flint_moe_forward, through the C ABI.

Two calls in a row per path, the second with a smaller batch (a different
workspace layout over the same scratch, holding the first call's bytes): each
output must equal the handle-based forward's bit for bit (same kernels, same
inputs, fixed summation order), and the first call's fp32 output must meet
the plain bound against the oracle.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import TOL, compare, dev_layer, make_layer_obj, out_host, run_oracle, x_device
from sparse_moe_transformer_gemv_amd import (FLINT_FORCE_PREFILL_PATH, FlintError,
                                             flint_moe_forward_noalloc)

pytestmark = pytest.mark.gpu

CASES = [
    # (config, (T1, T2), flags, overrides)
    (1, (16, 4), 0, {}),                                              # full-size bf16 decode
    (1, (64, 1), 0, {}),
    (4, (16, 1), 0, {}),                                              # full-size NVFP4 decode
    (1, (300, 120), FLINT_FORCE_PREFILL_PATH, dict(d=256, E=64, f=128, fs=256)),  # prefill path
    (2, (128, 70), 0, dict(d=512, E=64, f=256, fs=128)),              # Zipf router, default path choice
]


@pytest.mark.parametrize("cfg_id,Ts,flags,over", CASES)
def test_noalloc_matches_handle_forward(cfg_id, Ts, flags, over):
    L = synth.layer(cfg_id, **over)
    c = L["cfg"]
    D = dev_layer(L)
    layer = make_layer_obj(c, max(Ts), flags)
    cfg = layer.cfg
    cfg.flags = flags
    print("noalloc cfg=%d T=%s flags=%d %s" % (cfg_id, Ts, flags, over), flush=True)
    for i, T in enumerate(Ts):
        x = x_device(synth.hidden(cfg_id, T, c["d"], c["act"], draw=10 + i))
        want = layer.forward(x, D["router_w"], D["experts"], D["shared"], D["router_bias"])
        got = torch.empty_like(want)
        flint_moe_forward_noalloc(cfg, x, D["router_w"], D["experts"], D["shared"], got,
                                  router_bias=D["router_bias"])
        torch.cuda.synchronize()
        assert torch.equal(got, want), "T=%d: the no-alloc output differs from the handle's" % T
        zero = torch.zeros((T, c["d"]), dtype=torch.float32, device="cuda")
        got32 = torch.empty_like(zero)
        flint_moe_forward_noalloc(cfg, x, D["router_w"], D["experts"], D["shared"], got32,
                                  router_bias=D["router_bias"], residual=zero)
        want32 = layer.forward(x, D["router_w"], D["experts"], D["shared"], D["router_bias"],
                               residual=zero)
        torch.cuda.synchronize()
        assert torch.equal(got32, want32), "T=%d: fp32 output differs" % T
        if i == 0:
            xh = synth.hidden(cfg_id, T, c["d"], c["act"], draw=10 + i)
            ref = run_oracle(L, xh)
            r = layer.routing()
            rout = {"idx": r["idx"].cpu().numpy(), "weights": r["weights"].cpu().numpy()}
            rep = compare(out_host(got32), rout, ref, c["k"], c["wdtype"])
            print("  T=%d vs oracle: %s" % (T, rep), flush=True)


def test_noalloc_rejects_oversized_batch():
    L = synth.layer(1, d=256, E=16, f=32, fs=32)
    c = L["cfg"]
    D = dev_layer(L)
    layer = make_layer_obj(c, 4)
    cfg = layer.cfg
    T = 20000  # the workspace for this many tokens exceeds the static scratch
    x = torch.zeros((T, c["d"]), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(x)
    with pytest.raises(FlintError, match="static scratch"):
        flint_moe_forward_noalloc(cfg, x, D["router_w"], D["experts"], D["shared"], out)
