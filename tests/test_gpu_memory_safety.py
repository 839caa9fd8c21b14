"""GPU memory-safety checks of the layer.

Poisoned workspace: with FLINT_DEBUG_POISON_WORKSPACE every forward starts
from a workspace whose floating-point part is NaN, so a kernel that read data
no kernel of the same forward wrote (a previous forward's rows, unwritten
padding) would make the output NaN.  Each case must still match the oracle and
equal, bit for bit, the same forward on a handle without the poison.

Guard regions: the output is a window of a larger buffer whose rows before and
after hold a canary pattern; no path may write outside [T, d].
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import check_layer, dev_layer, make_layer_obj, out_host, run_gpu, run_oracle, x_device
from sparse_moe_transformer_gemv_amd import (FLINT_DEBUG_POISON_WORKSPACE, FLINT_FORCE_DECODE_PATH,
                                             FLINT_FORCE_PREFILL_PATH)

pytestmark = pytest.mark.gpu

POISON_CASES = [
    # (config, T, flags, overrides) -- decode bf16 with and without the folded
    # combine, NVFP4, the prefill path, the VALU fallbacks, split-K down
    (1, 1, 0, dict(d=512, E=64, f=128, fs=256)),
    (1, 16, 0, dict(d=512, E=64, f=128, fs=256)),
    (1, 64, 0, dict(d=512, E=64, f=128, fs=256)),
    (1, 37, FLINT_FORCE_DECODE_PATH, dict(d=256, E=64, f=64, fs=96)),
    (1, 200, FLINT_FORCE_PREFILL_PATH, dict(d=256, E=64, f=128, fs=256)),
    (2, 700, 0, dict(d=512, E=64, f=256, fs=128)),
    (4, 1, 0, dict(d=512, E=32, k=4, f=512, fs=1024)),
    (4, 16, 0, dict(d=512, E=32, k=4, f=512, fs=1024)),
    (4, 40, 0, dict(d=256, E=32, k=4, f=64, fs=64)),
    (1, 40, 0, dict(d=256, E=64, f=128, fs=2048)),
    (0, 64, 0, dict()),
]


@pytest.mark.parametrize("cfg_id,T,flags,over", POISON_CASES)
def test_poisoned_workspace(cfg_id, T, flags, over):
    L = synth.layer(cfg_id, **over)
    c = L["cfg"]
    print("poison cfg=%d T=%d flags=%d %s" % (cfg_id, T, flags, over), flush=True)
    D = dev_layer(L)
    x = synth.hidden(cfg_id, T, c["d"], c["act"], draw=3)
    ref = run_oracle(L, x)
    poisoned = make_layer_obj(c, max(T, 64), flags | FLINT_DEBUG_POISON_WORKSPACE)
    rep, _ = check_layer(poisoned, D, x, ref, c)
    plain = make_layer_obj(c, max(T, 64), flags)
    a, _ = run_gpu(plain, D, x)
    b, _ = run_gpu(poisoned, D, x)
    assert np.array_equal(a, b), "the poisoned workspace changed the result"
    print("  -> %s" % rep, flush=True)


def test_poisoned_workspace_between_forward_sizes():
    # decode then prefill then decode on one poisoned handle (no shared expert:
    # the combine must not read the shared slots that a forward never writes)
    L = synth.layer(1, d=256, E=32, f=128, fs=128)
    L["shared"] = None
    c = dict(L["cfg"], fs=0)
    L["cfg"] = c
    layer = make_layer_obj(c, 256, FLINT_DEBUG_POISON_WORKSPACE)
    D = dev_layer(L)
    for T in (64, 100, 5):
        x = synth.hidden(1, T, 256, synth.BF16, draw=T)
        ref = oracle.moe_forward(x, L["router_w"], L["experts"], None, top_k=c["k"], wdtype=synth.BF16)
        check_layer(layer, D, x, ref, c)


CANARY_CASES = [
    (1, 4, 0, dict(d=512, E=64, f=128, fs=128)),       # decode, combine in down
    (1, 40, 0, dict(d=512, E=64, f=128, fs=128)),      # decode + combine kernel
    (1, 300, FLINT_FORCE_PREFILL_PATH, dict(d=256, E=64, f=128, fs=128)),
    (4, 3, 0, dict(d=512, E=32, k=4, f=512, fs=512)),  # NVFP4
    (4, 20, 0, dict(d=512, E=32, k=4, f=512, fs=512)),
]
CANARY_F32 = np.float32(-12345.678)


@pytest.mark.parametrize("cfg_id,T,flags,over", CANARY_CASES)
@pytest.mark.parametrize("residual", [False, True])
def test_output_guard_rows(cfg_id, T, flags, over, residual):
    L = synth.layer(cfg_id, **over)
    c = L["cfg"]
    d, G = c["d"], 3  # guard rows on each side
    D = dev_layer(L)
    x = synth.hidden(cfg_id, T, d, c["act"], draw=1)
    layer = make_layer_obj(c, T, flags)
    dt = torch.float32 if residual else torch.bfloat16
    full = torch.full((T + 2 * G, d), float(CANARY_F32), dtype=dt, device="cuda")
    out = full[G:G + T]
    res = None
    if residual:
        res = torch.zeros((T, d), dtype=torch.float32, device="cuda")
    layer.forward(x_device(x), D["router_w"], D["experts"], D["shared"], D["router_bias"],
                  residual=res, out=out)
    torch.cuda.synchronize()
    h = out_host(full)
    want = float(torch.tensor(float(CANARY_F32), dtype=dt).item())
    assert np.all(h[:G] == want) and np.all(h[G + T:] == want), "a guard row was written"
    assert np.all(np.isfinite(h[G:G + T]))
    if residual:  # the fp32 form is the one gated at the plain bound elsewhere
        ref = run_oracle(L, x)
        err = np.abs(h[G:G + T] - ref["out"]).max()
        assert err <= 2e-2 * np.sqrt(np.mean(ref["out"] ** 2))
