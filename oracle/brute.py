"""Brute-force reference of the MoE layer for tiny inputs: pure Python.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): a second, independent
statement of the layer used to pin the C oracle on dense random weights.  It
shares nothing with ``moe_oracle.c``: every sum is ``math.fsum`` (the exactly
rounded sum of its terms), the selection is a full stable sort, and the
inputs arrive as plain Python floats (the caller decodes any stored format).

What it computes, per token x (the readings the C oracle also takes):
  logits   l_e = sum_i x_i Wr[e][i] + b_e                     (all E experts)
  chosen   the first k experts ordered by (-l_e, e): the largest logits, ties
           to the lower expert index  [6 of 256 per token: evermx.com,
           "Recursive Flint: Open-Weight MoE Coding Model, 2.5B Active",
           Feature Overview, "Sparse architecture"]
  weights  softmax over all E logits, renormalised over the chosen k
  expert   h_j = SiLU(G_j . x) (U_j . x), y_n = D_n . h, SiLU(z) = z / (1 + e^-z)
  output   y_shared + sum_j w_j y_{chosen_j}   (shared weight exactly 1)
"""
from __future__ import annotations

import math
import struct


def bf16_to_float(bits: int) -> float:
    """bf16 bits -> float: the upper half of an IEEE binary32."""
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def f32_to_float(v) -> float:
    return float(v)


def dot(a, b) -> float:
    return math.fsum(p * q for p, q in zip(a, b))


def silu(z: float) -> float:
    return z / (1.0 + math.exp(-z))


def route(x, router, bias, k):
    """(logits, chosen experts, weights) of one token."""
    E = len(router)
    logits = [dot(x, router[e]) + (bias[e] if bias is not None else 0.0) for e in range(E)]
    order = sorted(range(E), key=lambda e: (-logits[e], e))
    chosen = order[:k]
    m = max(logits)
    p = [math.exp(l - m) for l in logits]
    z = math.fsum(p)
    p = [v / z for v in p]
    s = math.fsum(p[e] for e in chosen)
    return logits, chosen, [p[e] / s for e in chosen]


def expert(x, gate_up, down):
    """One SwiGLU expert: gate_up [2f][d] (gate rows first), down [d][f]."""
    f = len(gate_up) // 2
    h = [silu(dot(gate_up[j], x)) * dot(gate_up[f + j], x) for j in range(f)]
    return [dot(row, h) for row in down]


def layer(xs, router, bias, experts_gu, experts_dn, shared_gu, shared_dn, k):
    """The layer on tokens xs (lists of floats).  experts_gu[e] is [2f][d],
    experts_dn[e] is [d][f]; shared_* the same for one expert, or None.
    Returns (out [T][d], chosen [T][k], weights [T][k], logits [T][E])."""
    outs, sels, wts, lgs = [], [], [], []
    for x in xs:
        logits, chosen, w = route(x, router, bias, k)
        terms = []
        if shared_gu is not None:
            terms.append(expert(x, shared_gu, shared_dn))
        for j, e in enumerate(chosen):
            y = expert(x, experts_gu[e], experts_dn[e])
            terms.append([w[j] * v for v in y])
        d = len(x)
        outs.append([math.fsum(t[n] for t in terms) for n in range(d)])
        sels.append(chosen)
        wts.append(w)
        lgs.append(logits)
    return outs, sels, wts, lgs
