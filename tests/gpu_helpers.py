"""Helpers shared by the GPU tests: run the HIP layer through the C ABI and
compare it with the oracle.

Tolerances (the plain bound, with no per-element term): max|out_gpu -
out_ref| <= 1e-4 * RMS(out_ref) with fp32 weights and activations,
<= 2e-2 * RMS(out_ref) with bf16 or NVFP4 weights; RMS over all compared
elements.  Expert selection must match as a set for every token whose oracle
gap between the k-th and (k+1)-th logit is >= 1e-4; tokens under that gap are
reported separately and, if their selection differs, left out of the output
comparison.

A bf16-activation layer is run twice: once with its bf16 output and once
with an fp32 output (a zero fp32 residual, which the combine adds first, so
the fp32 sum is the same).  The fp32 leg must meet the plain bound; the bf16
leg must be the round-to-nearest-even of the fp32 leg, value for value; the
full-size workloads also gate the bf16 leg itself at the plain bound.  The
share of the bf16 leg's error that the output format alone accounts for (half
a bf16 ulp of the largest value, over RMS) is reported beside the gate.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
from synth.device import (dev_array, dev_layer, dev_weights, make_layer_obj,  # noqa: F401
                          out_host, x_device)

GAP = 1e-4
TOL = {synth.F32: 1e-4, synth.BF16: 2e-2, synth.NVFP4: 2e-2}


def run_gpu(layer, D: dict, x: np.ndarray, residual=None, out=None, routing=True):
    xd = x_device(x)
    o = layer.forward(xd, D["router_w"], D["experts"], D["shared"], D["router_bias"],
                      residual=residual, out=out)
    r = layer.routing() if routing else {}
    torch.cuda.synchronize()
    return out_host(o), {k: v.cpu().numpy() for k, v in r.items()}


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


def rne_bf16(v: np.ndarray) -> np.ndarray:
    """fp32 values (given as float64) rounded to the nearest bf16, ties to even."""
    return synth.bf16_to_f32(synth.bf16_bits(np.asarray(v, np.float32))).astype(np.float64)


def check_selection(gpu_idx, gpu_w, ref, k, tokens=None):
    """Selected sets equal the oracle's for every token with gap >= GAP, and
    the combine weights of equal selections agree to 1e-5.  Returns
    (sel_ok, near) boolean arrays over the tokens."""
    idx_ref = ref["idx"]
    g = gaps(ref["logits"], k)
    T = idx_ref.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    near = g < GAP
    sel_ok = np.array([set(gpu_idx[i]) == set(idx_ref[i]) for i in range(T)], bool)
    bad = np.where(~sel_ok & ~near)[0]
    assert bad.size == 0, "selection differs for tokens %s (gaps %s)" % (tokens[bad][:8], g[bad][:8])
    for i in np.where(sel_ok)[0]:
        order = {e: j for j, e in enumerate(idx_ref[i])}
        wr = np.array([ref["w"][i][order[e]] for e in gpu_idx[i]])
        assert np.all(np.abs(gpu_w[i] - wr) <= 1e-5), (tokens[i], gpu_w[i], wr)
    return sel_ok, near


def compare(out_gpu, rout, ref, k, wdtype, tokens=None, gate=True):
    """Check selection and output against the plain bound; returns a report
    (asserts on failure when gate is set)."""
    sel_ok, near = check_selection(rout["idx"], rout["weights"], ref, k, tokens)
    keep = sel_ok | ~near
    ref_out = ref["out"][keep]
    err = np.abs(out_gpu[keep] - ref_out)
    assert np.all(np.isfinite(out_gpu)), "non-finite output"
    rms = float(np.sqrt(np.mean(ref_out ** 2))) if ref_out.size else 0.0
    maxerr = float(err.max()) if err.size else 0.0
    tol = TOL[wdtype] * rms
    if gate:
        worst = np.unravel_index(np.argmax(err), err.shape) if err.size else None
        assert maxerr <= tol, "max|err| %.3e > %.1e * RMS (%.3e); worst at %s: ref %r gpu %r" % (
            maxerr, TOL[wdtype], rms, worst, ref_out[worst], out_gpu[keep][worst])
    return {"maxerr": maxerr, "rms": rms, "ratio": maxerr / rms if rms else 0.0,
            "near_ties": int(near.sum()), "near_tie_mismatch": int((near & ~sel_ok).sum())}


def check_layer(layer, D, x, ref, c, *, full=False, tokens=None, rows=None):
    """Both output legs of one forward (see the module docstring).

    rows: the token rows of the batch that ``ref`` covers (default all);
    tokens: their labels in reports.  Returns (report, routing)."""
    T = x.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    zero = torch.zeros((T, c["d"]), dtype=torch.float32, device="cuda")
    out32, rout = run_gpu(layer, D, x, residual=zero)
    sub = {"idx": rout["idx"][rows], "weights": rout["weights"][rows]}
    rep32 = compare(out32[rows], sub, ref, c["k"], c["wdtype"], tokens)
    rep = {"fp32_out": rep32}
    out16, rout16 = run_gpu(layer, D, x)
    assert np.array_equal(rout16["idx"], rout["idx"]), "routing differs between the two legs"
    if c["act"] != synth.BF16:
        # fp32 activations: the plain output is the same fp32 sum
        assert np.array_equal(out16, out32), "output without a residual differs from the fp32 leg"
    else:
        # the bf16 output is the rounding of the same fp32 sum
        mism = out16 != rne_bf16(out32)
        assert not mism.any(), "bf16 output is not RNE(fp32 output) at %d elements, first %s" % (
            int(mism.sum()), np.argwhere(mism)[0])
        rep16 = compare(out16[rows], sub, ref, c["k"], c["wdtype"], tokens, gate=full)
        rep16["format_share"] = float(half_ulp_bf16(np.abs(ref["out"]).max()) / rep16["rms"]) \
            if rep16["rms"] else 0.0
        rep["bf16_out"] = rep16
    return rep, rout


def check_permutation(rout, T, k, E):
    """sorted_pair is the stable argsort of the chosen expert ids."""
    keys = rout["idx"].reshape(-1).astype(np.int64)
    want = np.argsort(keys, kind="stable")
    assert np.array_equal(rout["sorted_pair"][:T * k], want)
    assert np.array_equal(rout["counts"], np.bincount(keys, minlength=E))


def stack_layer_gpu(moe, h: torch.Tensor, D: dict, x: torch.Tensor, x_next: torch.Tensor,
                    eps: float = 1e-6, record: bool = False):
    """One layer of the stacked workload on the GPU, in place on the fp32
    residual h [T, d]: x holds bf16(RMSNorm(h)) on entry; h += MoE(x) (the
    layer's combine adds the fp32 residual) and x_next = bf16(RMSNorm(h)),
    the next layer's input, from the same launch where the path allows.  With
    record, returns host copies of h before and after, x, and the routing."""
    rec = None
    if record:
        h_before = out_host(h)
    moe.forward_prenorm(x, D["router_w"], D["experts"], D["shared"], residual=h, eps=eps,
                        router_bias=D["router_bias"], out=h, norm_out=x_next)
    if record:
        r = moe.routing()
        torch.cuda.synchronize()
        rec = {"h_before": h_before, "h_after": out_host(h),
               "x": x.view(torch.int16).cpu().numpy().view(np.uint16).copy(),
               "idx": r["idx"].cpu().numpy(), "weights": r["weights"].cpu().numpy(),
               "logits": r["logits"].cpu().numpy()}
    return rec


def stack_gpu(moe, h: torch.Tensor, layers, eps: float = 1e-6):
    """The whole stacked pass on the GPU (no read-back): the first pre-norm by
    the RMSNorm kernel, every later one by the layer before it."""
    from sparse_moe_transformer_gemv_amd import flint_rmsnorm_forward
    x = torch.empty(h.shape, dtype=torch.bfloat16, device=h.device)
    xn = torch.empty_like(x)
    flint_rmsnorm_forward(h, eps, out=x)
    for D in layers:
        stack_layer_gpu(moe, h, D, x, xn, eps)
        x, xn = xn, x


def teacher_forced_layer(rec: dict, L: dict, k: int, eps: float = 1e-6):
    """Layer l of the stack checked on the GPU's own input.

    The pre-norm: the GPU's bf16 x equals the nearest bf16 of the oracle's
    RMSNorm of the GPU's fp32 residual h_l within one bf16 step, at fewer
    than 0.1% of the elements.  The layer: the oracle runs on that same x;
    the GPU's layer output (h_{l+1} - h_l, exact in fp64) must meet the plain
    2e-2 * RMS bound and its selection the set rule."""
    c = L["cfg"]
    want = oracle.round_to_bf16(oracle.rmsnorm(rec["h_before"], eps))
    diff = np.abs(rec["x"].astype(np.int32) - want.astype(np.int32))
    assert diff.max() <= 1 and (diff > 0).mean() < 1e-3, (
        "rmsnorm: %d elements differ, max %d bf16 steps" % (int((diff > 0).sum()), int(diff.max())))
    ref = oracle.moe_forward(rec["x"], L["router_w"], L["experts"], L["shared"], top_k=k,
                             router_bias=L["router_bias"], wdtype=c["wdtype"])
    out_gpu = rec["h_after"] - rec["h_before"]
    rep = compare(out_gpu, {"idx": rec["idx"], "weights": rec["weights"]}, ref, k, c["wdtype"])
    rep["rmsnorm_steps_differing"] = int((diff > 0).sum())
    return rep
