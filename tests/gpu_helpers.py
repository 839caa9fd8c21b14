"""Helpers shared by the GPU tests: upload seeded inputs, run the HIP layer,
compare with the oracle.

Tolerances: max|out_gpu - out_ref| <= 1e-4 * RMS(out_ref) with fp32 weights
and activations, <= 2e-2 * RMS(out_ref) with bf16 or NVFP4 weights; RMS over
all compared elements.  Expert selection must match as a set for every token
whose oracle gap between the k-th and (k+1)-th logit is >= 1e-4; tokens under
that gap are reported separately and, if their selection differs, left out of
the output comparison.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
from sparse_moe_transformer_gemv_amd import ExpertWeights, MoELayer

GAP = 1e-4
TOL = {synth.F32: 1e-4, synth.BF16: 2e-2, synth.NVFP4: 2e-2}


def dev_array(a: np.ndarray, bf16: bool = False) -> torch.Tensor:
    if bf16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.cuda()


def dev_weights(ws: dict, wdtype: int) -> ExpertWeights:
    if wdtype == synth.NVFP4:
        return ExpertWeights(dev_array(ws["gate_up"]), dev_array(ws["down"]),
                             dev_array(ws["gate_up_scales"]), dev_array(ws["down_scales"]),
                             dev_array(ws["tensor_scales"]))
    bf = wdtype == synth.BF16
    return ExpertWeights(dev_array(ws["gate_up"], bf), dev_array(ws["down"], bf))


def dev_layer(L: dict) -> dict:
    wd = L["cfg"]["wdtype"]
    return {"router_w": dev_array(L["router_w"]),
            "router_bias": None if L["router_bias"] is None else dev_array(L["router_bias"]),
            "experts": dev_weights(L["experts"], wd),
            "shared": None if L["shared"] is None else dev_weights(L["shared"], wd)}


def x_device(x: np.ndarray) -> torch.Tensor:
    return dev_array(x, bf16=(x.dtype == np.uint16))


def out_host(out: torch.Tensor) -> np.ndarray:
    return out.float().cpu().numpy().astype(np.float64)


def make_layer_obj(cfg: dict, max_tokens: int, flags: int = 0) -> MoELayer:
    return MoELayer(cfg["d"], cfg["E"], cfg["k"], cfg["f"], cfg["fs"], cfg["act"], cfg["wdtype"],
                    max_tokens, flags)


def run_gpu(layer: MoELayer, D: dict, x: np.ndarray, residual=None):
    xd = x_device(x)
    out = layer.forward(xd, D["router_w"], D["experts"], D["shared"], D["router_bias"],
                        residual=residual)
    r = layer.routing()
    torch.cuda.synchronize()
    return out_host(out), {k: v.cpu().numpy() for k, v in r.items()}


def run_oracle(L: dict, x: np.ndarray):
    c = L["cfg"]
    return oracle.moe_forward(x, L["router_w"], L["experts"], L["shared"], top_k=c["k"],
                              router_bias=L["router_bias"], wdtype=c["wdtype"])


def gaps(logits: np.ndarray, k: int) -> np.ndarray:
    s = -np.sort(-logits, axis=1)
    if k >= logits.shape[1]:
        return np.full(logits.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


def half_ulp_bf16(v):
    """Half a bf16 unit in the last place of |v| (what rounding to bf16 may cost)."""
    _, e = np.frexp(np.abs(v))
    return np.ldexp(1.0, e - 9)


def compare(out_gpu, rout, ref, k, wdtype, *, out_bf16, tokens=None):
    """Check selection and output; returns a report dict (asserts on failure).

    A bf16 output is itself a rounding of the result, which alone may cost
    half a bf16 ulp of each value; for bf16 outputs that format allowance is
    added per element to the tolerance (the fp32-output variant of each
    full-size test checks the plain bound).
    """
    idx_ref = ref["idx"]
    g = gaps(ref["logits"], k)
    T = idx_ref.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    near = g < GAP
    sel_ok = np.array([set(rout["idx"][i]) == set(idx_ref[i]) for i in range(T)])
    bad = np.where(~sel_ok & ~near)[0]
    assert bad.size == 0, "selection differs for tokens %s (gaps %s)" % (
        tokens[bad][:8], g[bad][:8])
    keep = sel_ok | ~near
    ref_out = ref["out"][keep]
    err = np.abs(out_gpu[keep] - ref_out)
    rms = float(np.sqrt(np.mean(ref_out ** 2))) if ref_out.size else 0.0
    maxerr = float(err.max()) if err.size else 0.0
    tol = TOL[wdtype] * rms
    allow = tol + (half_ulp_bf16(ref_out) if out_bf16 else 0.0)
    worst = np.unravel_index(np.argmax(err - allow), err.shape) if err.size else None
    assert np.all(err <= allow), "max|err| %.3e vs %.1e * RMS (%.3e)%s; worst at %s: ref %r gpu %r" % (
        maxerr, TOL[wdtype], rms, " + half bf16 ulp" if out_bf16 else "", worst,
        ref_out[worst], out_gpu[keep][worst])
    # combine weights of matching selections agree closely (fp32 softmax)
    for i in np.where(sel_ok)[0]:
        order = {e: j for j, e in enumerate(idx_ref[i])}
        wr = np.array([ref["w"][i][order[e]] for e in rout["idx"][i]])
        assert np.all(np.abs(rout["weights"][i] - wr) <= 1e-5), (i, rout["weights"][i], wr)
    return {"maxerr": maxerr, "rms": rms, "ratio": maxerr / rms if rms else 0.0,
            "near_ties": int(near.sum()), "near_tie_mismatch": int((near & ~sel_ok).sum())}


def check_permutation(rout, T, k, E):
    """sorted_pair is the stable argsort of the chosen expert ids."""
    keys = rout["idx"].reshape(-1).astype(np.int64)
    want = np.argsort(keys, kind="stable")
    assert np.array_equal(rout["sorted_pair"][:T * k], want)
    assert np.array_equal(rout["counts"], np.bincount(keys, minlength=E))


def stack_gpu(moe: MoELayer, h: torch.Tensor, layers, eps: float = 1e-6, record: bool = False):
    """The stacked workload on the GPU, in place on the fp32 residual h [T, d]:
    per layer, x = bf16(RMSNorm(h)) (rmsnorm kernel), then h += MoE(x) (the
    layer's combine adds the fp32 residual).  With record=True, returns each
    layer's routing (idx, logits) as host arrays."""
    from sparse_moe_transformer_gemv_amd import flint_rmsnorm_forward
    x = torch.empty(h.shape, dtype=torch.bfloat16, device=h.device)
    rec = []
    for D in layers:
        flint_rmsnorm_forward(h, eps, out=x)
        moe.forward(x, D["router_w"], D["experts"], D["shared"], D["router_bias"], residual=h,
                    out=h)
        if record:
            r = moe.routing()
            rec.append({"idx": r["idx"].cpu().numpy(), "logits": r["logits"].cpu().numpy()})
    return rec


def stack_compare(h_gpu: np.ndarray, h_ref: np.ndarray, trace, rec, k: int, tol: float = 2e-2):
    """Final residual of the stack against the fp64 oracle.

    Each layer requantises its input to bf16, so fp32-vs-fp64 differences that
    cross a bf16 rounding midpoint grow from layer to layer; a token's choice
    may then legitimately differ from the oracle's where the oracle's k-th /
    (k+1)-th logit gap is no larger than twice that token's largest
    GPU-vs-oracle logit difference.  Every such flip is checked to be of that kind; tokens that
    never flipped must match the final residual within tol * RMS."""
    T = h_ref.shape[0]
    flipped = np.zeros(T, bool)
    n_flips = 0
    for l, (tr, g) in enumerate(zip(trace, rec)):
        gp = gaps(tr["logits"], k)
        dl = np.abs(g["logits"] - tr["logits"]).max(1)
        for t in range(T):
            if set(g["idx"][t]) != set(tr["idx"][t]):
                n_flips += 1
                # the two logits at the boundary can move in opposite directions
                assert gp[t] <= max(2 * dl[t], GAP), (
                    "layer %d token %d: selection differs with oracle gap %.3g above the logit "
                    "difference %.3g" % (l, t, gp[t], dl[t]))
                flipped[t] = True
    keep = ~flipped
    ref = h_ref[keep]
    err = np.abs(h_gpu[keep] - ref)
    rms = float(np.sqrt(np.mean(h_ref ** 2)))
    maxerr = float(err.max()) if err.size else 0.0
    # a layer whose bf16 input differs by one rounding step in some elements
    # moves its output by up to about 2^-8 of that output's size; over the
    # stack these steps add up on top of the single-layer bound
    drift = sum(2.0 ** -8 * tr["out_rms"] for tr in trace)
    allow = tol * rms + drift
    assert maxerr <= allow, "stack: max|err| %.3e > %.0e * RMS %.3e + drift %.3e" % (
        maxerr, tol, rms, drift)
    return {"maxerr": maxerr, "rms": rms, "ratio": maxerr / rms, "drift_allowance": drift,
            "flipped_tokens": int(flipped.sum()), "flips": n_flips,
            "compared_tokens": int(keep.sum())}
