"""Pins of the fp64 oracle to facts fixed outside the oracle itself.

Each test ties one part of the oracle to something it cannot agree with by
construction: the OCP number-format tables (golden files), closed forms of
SiLU, RMSNorm and softmax, weight matrices built from scaled permutations
(whose layer output can be written down term by term), exhaustive subset
enumeration for the top-k choice, and invariants of the layer (weights sum
to one, the shared expert is always applied, batch invariance, the dense
limit k = E).  The cases are chosen so that a transposed operand, a swapped
gate/up, a wrong nibble or block-scale index, a wrong tie-break, a missing
renormalisation, a dropped bias or a dropped shared expert each fail at
least one of them.
"""
import itertools
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        a, b = line.split()
        rows.append((int(a, 0), float(b)))
    return rows


def sigmoid(z):
    return 1.0 / (1.0 + math.exp(-z))


# ---------------------------------------------------------------- formats

def test_e2m1_matches_ocp_table():
    rows = _read_table("e2m1_ocp_mx.txt")
    assert len(rows) == 16
    for code, val in rows:
        got = oracle.e2m1_value(code)
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code


def test_e4m3_matches_ocp_table():
    rows = _read_table("e4m3_ocp_fp8.txt")
    for code, val in rows:
        got = oracle.e4m3_value(code)
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)
    # the scale range of the 4-bit workload is exactly codes 0x28..0x40
    scale_codes = [c for c, _ in rows if 0x28 <= c <= 0x40]
    assert sorted(scale_codes) == list(range(0x28, 0x41))


def test_bf16_decode_closed_forms():
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x4049: 3.140625, 0x0000: 0.0, 0x3E80: 0.25,
             0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127}
    for b, v in cases.items():
        assert oracle.bf16_value([b])[0] == v, hex(b)
    assert math.isinf(oracle.bf16_value([0x7F80])[0])
    # bf16 is the upper half of binary32: agree with numpy's own float32 view
    bits = np.arange(0, 65536, 97, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]
    ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(oracle.bf16_value(bits), ref)


def test_round_to_bf16_nearest_even():
    # grid points stay put; midpoints go to the even neighbour; anything off
    # the midpoint goes to the nearer neighbour
    rng = np.random.default_rng(5)
    lo = rng.integers(0x0080, 0x7F00, size=200).astype(np.uint16)
    lo |= rng.integers(0, 2, size=200).astype(np.uint16) << 15
    a = (lo.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nxt = ((lo.astype(np.uint32) + 1) << 16).view(np.float32).astype(np.float64)
    mid = (a + nxt) / 2  # exact in fp64
    assert np.array_equal(oracle.round_to_bf16(a), lo)
    even = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint16)
    assert np.array_equal(oracle.round_to_bf16(mid), even)
    step = np.abs(nxt - a)
    assert np.array_equal(oracle.round_to_bf16(mid - np.sign(a) * step * 1e-3), lo)
    assert np.array_equal(oracle.round_to_bf16(mid + np.sign(a) * step * 1e-3),
                          (lo + 1).astype(np.uint16))


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(1.0) - 0.7310585786300049) < 1e-15
    assert abs(oracle.silu(-1.0) + 0.2689414213699951) < 1e-15
    for z in (0.3, 1.7, 4.0, 11.0):
        # silu(z) - silu(-z) = z for every z
        assert abs(oracle.silu(z) - oracle.silu(-z) - z) < 1e-14 * max(1, z)
    assert abs(oracle.silu(40.0) - 40.0) < 1e-12
    assert abs(oracle.silu(-40.0)) < 1e-15


def test_rmsnorm_closed_forms():
    c = np.full((1, 8), -3.0)
    out = oracle.rmsnorm(c, eps=1e-6)
    assert np.allclose(out, -3.0 / math.sqrt(9.0 + 1e-6), rtol=0, atol=1e-15)
    v = np.array([[3.0, 4.0]])
    assert np.allclose(oracle.rmsnorm(v, eps=0.0), v / math.sqrt(12.5), rtol=1e-15)
    r = np.random.default_rng(1).standard_normal((3, 16))
    assert np.allclose(oracle.rmsnorm(r * 7.5, eps=0.0), oracle.rmsnorm(r, eps=0.0),
                       rtol=1e-14, atol=0)
    # rows are normalised independently
    both = oracle.rmsnorm(np.vstack([r[:1], 100 * r[1:2]]), eps=0.0)
    assert np.allclose(both[0], oracle.rmsnorm(r[:1], eps=0.0)[0], rtol=1e-15)


# ---------------------------------------------------------------- router

def _route(x, wr, k, bias=None):
    E, d = wr.shape
    f = 16
    z = {"gate_up": np.zeros((E, 2 * f, d), np.float32), "down": np.zeros((E, d, f), np.float32)}
    s = {"gate_up": np.zeros((1, 2 * f, d), np.float32), "down": np.zeros((1, d, f), np.float32)}
    return oracle.moe_forward(np.asarray(x, np.float32), wr.astype(np.float32), z, s, top_k=k,
                              router_bias=bias, wdtype=oracle.F32)


def test_logits_read_router_rows():
    # one-hot tokens read one column of the router: l_e = Wr[e, i]
    rng = np.random.default_rng(2)
    E, d = 8, 5
    wr = rng.integers(-8, 9, size=(E, d)).astype(np.float32) / 4
    x = np.eye(d, dtype=np.float32)
    r = _route(x, wr, 3)
    assert np.array_equal(r["logits"], wr.T.astype(np.float64))


def test_selection_matches_subset_enumeration():
    rng = np.random.default_rng(3)
    E, d = 8, 4
    for trial in range(30):
        k = int(rng.integers(1, 6))
        # small integer logits make exact ties common
        wr = rng.integers(-2, 3, size=(E, d)).astype(np.float32)
        x = rng.integers(-1, 2, size=(1, d)).astype(np.float32)
        r = _route(x, wr, k)
        l = [float(np.dot(x[0].astype(np.float64), wr[e].astype(np.float64))) for e in range(E)]

        def beats(a, b):
            return l[a] > l[b] or (l[a] == l[b] and a < b)

        winners = [S for S in itertools.combinations(range(E), k)
                   if all(beats(a, b) for a in S for b in range(E) if b not in S)]
        assert len(winners) == 1
        got = list(r["idx"][0])
        assert sorted(got) == list(winners[0])
        # slots run in descending logit, ties by index
        for a, b in zip(got, got[1:]):
            assert beats(a, b)


def test_all_equal_logits_pick_lowest_indices():
    E, d, k = 16, 4, 6
    r = _route(np.ones((2, d), np.float32), np.zeros((E, d), np.float32), k)
    assert np.array_equal(r["idx"], np.tile(np.arange(k), (2, 1)))
    assert np.all(r["w"] == 1.0 / 6)


def test_duplicate_router_rows_lower_index_first():
    E, d = 10, 3
    wr = np.zeros((E, d), np.float32)
    wr[7] = wr[2] = [1, 2, 3]
    wr[4] = [1, 1, 1]
    r = _route(np.ones((1, d), np.float32), wr, 3)
    assert list(r["idx"][0]) == [2, 7, 4]


def test_zipf_bias_weights_closed_form():
    # with a zero router, the logits are the bias b_e = -1.65 ln(e+1): the
    # chosen set is {0..5} and w_j = (j+1)^-1.65 / sum_i (i+1)^-1.65
    E, d, k = 256, 4, 6
    bias = synth.zipf_bias(E)
    r = _route(np.ones((1, d), np.float32), np.zeros((E, d), np.float32), k, bias=bias)
    assert list(r["idx"][0]) == list(range(6))
    p = np.exp(bias[:6].astype(np.float64))
    assert np.allclose(r["w"][0], p / p.sum(), rtol=1e-14, atol=0)
    q = np.array([(j + 1) ** -1.65 for j in range(6)])
    assert np.allclose(r["w"][0], q / q.sum(), rtol=1e-6, atol=0)  # bias stored in fp32


def test_weights_are_renormalised_softmax():
    rng = np.random.default_rng(4)
    E, d, k = 32, 16, 6
    wr = rng.standard_normal((E, d)).astype(np.float32)
    x = rng.standard_normal((5, d)).astype(np.float32)
    r = _route(x, wr, k)
    for t in range(5):
        w = r["w"][t]
        l = r["logits"][t][r["idx"][t]]
        assert abs(w.sum() - 1.0) <= 1e-15
        assert np.all(w > 0)
        # ratios of weights are exponentials of logit differences
        for a in range(k):
            for b in range(k):
                assert abs(w[a] / w[b] - math.exp(l[a] - l[b])) <= 1e-12 * w[a] / w[b]
        assert np.all(np.diff(w) <= 0)
    r1 = _route(x, wr, 1)
    assert np.all(r1["w"] == 1.0)


# ---------------------------------------------------------------- experts

def _perm_expert(rng, d, f):
    """Scaled permutation matrices: gate row j reads x[pg[j]] times a[j], up
    row j reads x[pu[j]] times b[j], down row n reads h[pd[n]] times c[n]."""
    pg = rng.integers(0, d, size=f)
    pu = rng.integers(0, d, size=f)
    pd = rng.integers(0, f, size=d)
    a = rng.integers(1, 8, size=f) * rng.choice([-1, 1], size=f) / 4.0
    b = rng.integers(1, 8, size=f) * rng.choice([-1, 1], size=f) / 4.0
    c = rng.integers(1, 8, size=d) * rng.choice([-1, 1], size=d) / 4.0
    gu = np.zeros((2 * f, d), np.float32)
    dn = np.zeros((d, f), np.float32)
    for j in range(f):
        gu[j, pg[j]] = a[j]
        gu[f + j, pu[j]] = b[j]
    for n in range(d):
        dn[n, pd[n]] = c[n]

    def apply(x):
        h = [(a[j] * x[pg[j]]) * sigmoid(a[j] * x[pg[j]]) * (b[j] * x[pu[j]]) for j in range(f)]
        return np.array([c[n] * h[pd[n]] for n in range(d)])

    return gu, dn, apply


def test_expert_closed_form_permutation_weights():
    rng = np.random.default_rng(6)
    d, f = 7, 3
    gu, dn, apply = _perm_expert(rng, d, f)
    ws = {"gate_up": gu[None], "down": dn[None]}
    for _ in range(5):
        x = rng.integers(-6, 7, size=d) / 2.0
        y = oracle.expert_forward(x, ws, 0, wdtype=oracle.F32)
        assert np.allclose(y, apply(x), rtol=1e-14, atol=1e-15)


def test_bf16_weights_equal_fp32_weights():
    rng = np.random.default_rng(7)
    d, f = 32, 16
    gu32 = synth.bf16_to_f32(synth.bf16_bits(rng.standard_normal((2, 2 * f, d))))
    dn32 = synth.bf16_to_f32(synth.bf16_bits(rng.standard_normal((2, d, f))))
    x = rng.standard_normal(d)
    for e in range(2):
        a = oracle.expert_forward(x, {"gate_up": gu32, "down": dn32}, e, wdtype=oracle.F32)
        b = oracle.expert_forward(x, {"gate_up": synth.bf16_bits(gu32),
                                      "down": synth.bf16_bits(dn32)}, e, wdtype=oracle.BF16)
        assert np.array_equal(a, b)


def _nvfp4_pair(rng, n, rows, cols, tscale):
    """Random NVFP4 codes + scales and the fp32 matrix they stand for, built
    from the golden OCP tables (not from the oracle's decoders)."""
    e2m1 = dict(_read_table("e2m1_ocp_mx.txt"))
    e4m3 = dict(_read_table("e4m3_ocp_fp8.txt"))
    codes = rng.integers(0, 16, size=(n, rows, cols)).astype(np.uint8)
    sc = rng.integers(0x28, 0x41, size=(n, rows, cols // 16)).astype(np.uint8)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    val = np.vectorize(lambda c: e2m1[int(c)])(codes).astype(np.float64)
    sv = np.vectorize(lambda c: e4m3[int(c)])(sc).astype(np.float64)
    dense = val * np.repeat(sv, 16, axis=-1) * np.float64(np.float32(tscale))
    return packed, sc, dense


def test_nvfp4_expert_equals_dequantised_dense():
    rng = np.random.default_rng(8)
    n, d, f = 2, 32, 16
    tg, tu, td = 0.125, 0.25, 0.5
    gcode, gsc, gval = _nvfp4_pair(rng, n, f, d, 1.0)
    ucode, usc, uval = _nvfp4_pair(rng, n, f, d, 1.0)
    dcode, dsc, dval = _nvfp4_pair(rng, n, d, f, 1.0)
    ws4 = {"gate_up": np.concatenate([gcode, ucode], 1),
           "gate_up_scales": np.concatenate([gsc, usc], 1),
           "down": dcode, "down_scales": dsc,
           "tensor_scales": np.tile(np.array([[tg, tu, td]], np.float32), (n, 1))}
    dense = {"gate_up": np.concatenate([gval * tg, uval * tu], 1).astype(np.float32),
             "down": (dval * td).astype(np.float32)}
    # the dequantised values need at most 2+4+1 significant bits: exact in fp32
    assert np.array_equal(dense["down"].astype(np.float64), dval * td)
    x = rng.standard_normal(d)
    for e in range(n):
        a = oracle.expert_forward(x, ws4, e, wdtype=oracle.NVFP4)
        b = oracle.expert_forward(x, dense, e, wdtype=oracle.F32)
        assert np.allclose(a, b, rtol=1e-13, atol=1e-15)
    # swapping the nibble order changes the answer (the pin sees it)
    swapped = dict(ws4)
    swapped["gate_up"] = ((ws4["gate_up"] >> 4) | (ws4["gate_up"] << 4)).astype(np.uint8)
    assert not np.allclose(oracle.expert_forward(x, swapped, 0, wdtype=oracle.NVFP4),
                           oracle.expert_forward(x, dense, 0, wdtype=oracle.F32))


# ---------------------------------------------------------------- layer

def _perm_layer(rng, E, d, f, fs):
    gus, dns, fns = [], [], []
    for _ in range(E):
        gu, dn, fn = _perm_expert(rng, d, f)
        gus.append(gu), dns.append(dn), fns.append(fn)
    sgu, sdn, sfn = _perm_expert(rng, d, fs)
    # router: row e reads one coordinate, so l_e = r_e * x[ie]
    ie = rng.integers(0, d, size=E)
    re_ = rng.integers(1, 9, size=E) * rng.choice([-1, 1], size=E) / 8.0
    wr = np.zeros((E, d), np.float32)
    for e in range(E):
        wr[e, ie[e]] = re_[e]
    experts = {"gate_up": np.stack(gus), "down": np.stack(dns)}
    shared = {"gate_up": sgu[None], "down": sdn[None]}
    return wr, experts, shared, fns, sfn, ie, re_


def test_layer_closed_form_tiny():
    rng = np.random.default_rng(9)
    E, d, f, fs, k, T = 8, 6, 3, 4, 3, 5
    wr, experts, shared, fns, sfn, ie, re_ = _perm_layer(rng, E, d, f, fs)
    x = (rng.integers(-8, 9, size=(T, d)) / 4.0).astype(np.float32)
    r = oracle.moe_forward(x, wr, experts, shared, top_k=k, wdtype=oracle.F32)
    for t in range(T):
        xt = x[t].astype(np.float64)
        l = [re_[e] * xt[ie[e]] for e in range(E)]
        order = sorted(range(E), key=lambda e: (-l[e], e))[:k]
        assert list(r["idx"][t]) == order
        p = [math.exp(l[e] - max(l)) for e in order]
        w = [v / sum(p) for v in p]
        want = sfn(xt) + sum(w[j] * fns[order[j]](xt) for j in range(k))
        assert np.allclose(r["out"][t], want, rtol=1e-13, atol=1e-14)


def test_shared_expert_always_applied():
    rng = np.random.default_rng(10)
    E, d, f, fs, k, T = 8, 6, 3, 4, 2, 4
    wr, experts, shared, fns, sfn, ie, re_ = _perm_layer(rng, E, d, f, fs)
    x = rng.standard_normal((T, d)).astype(np.float32)
    no_routed = dict(experts, down=np.zeros_like(experts["down"]))
    r = oracle.moe_forward(x, wr, no_routed, shared, top_k=k, wdtype=oracle.F32)
    for t in range(T):
        assert np.allclose(r["out"][t], sfn(x[t].astype(np.float64)), rtol=1e-13, atol=1e-15)
    no_shared = dict(shared, down=np.zeros_like(shared["down"]))
    full = oracle.moe_forward(x, wr, experts, shared, top_k=k, wdtype=oracle.F32)
    part = oracle.moe_forward(x, wr, experts, no_shared, top_k=k, wdtype=oracle.F32)
    for t in range(T):
        assert np.allclose(full["out"][t] - part["out"][t], sfn(x[t].astype(np.float64)),
                           rtol=1e-12, atol=1e-14)


def test_identical_experts_make_routing_irrelevant():
    rng = np.random.default_rng(11)
    E, d, f, k, T = 12, 8, 4, 6, 6
    gu, dn, fn = _perm_expert(rng, d, f)
    experts = {"gate_up": np.repeat(gu[None], E, 0), "down": np.repeat(dn[None], E, 0)}
    shared = {"gate_up": np.zeros((1, 2 * f, d), np.float32), "down": np.zeros((1, d, f), np.float32)}
    wr = rng.standard_normal((E, d)).astype(np.float32)
    x = rng.standard_normal((T, d)).astype(np.float32)
    r = oracle.moe_forward(x, wr, experts, shared, top_k=k, wdtype=oracle.F32)
    for t in range(T):
        assert np.allclose(r["out"][t], fn(x[t].astype(np.float64)), rtol=1e-13, atol=1e-15)


def test_batch_invariance_and_distinct_experts():
    L = synth.layer(0)
    x = synth.hidden(0, 64, 128, synth.F32)
    full = oracle.moe_forward(x, L["router_w"], L["experts"], L["shared"], wdtype=oracle.F32)
    for t in (0, 17, 63):
        one = oracle.moe_forward(x[t:t + 1], L["router_w"], L["experts"], L["shared"],
                                 wdtype=oracle.F32)
        assert np.array_equal(one["out"][0], full["out"][t])
        assert np.array_equal(one["idx"][0], full["idx"][t])
    for t in range(64):
        assert len(set(full["idx"][t])) == 6
    assert np.all(np.abs(full["w"].sum(1) - 1.0) <= 1e-15)


def test_dense_limit_equals_full_softmax_mixture():
    rng = np.random.default_rng(12)
    E, d, f, fs, T = 16, 8, 4, 4, 3
    wr = rng.standard_normal((E, d)).astype(np.float32)
    experts = {"gate_up": rng.standard_normal((E, 2 * f, d)).astype(np.float32),
               "down": rng.standard_normal((E, d, f)).astype(np.float32)}
    shared = {"gate_up": rng.standard_normal((1, 2 * fs, d)).astype(np.float32),
              "down": rng.standard_normal((1, d, fs)).astype(np.float32)}
    x = rng.standard_normal((T, d)).astype(np.float32)
    r = oracle.moe_forward(x, wr, experts, shared, top_k=E, wdtype=oracle.F32)
    for t in range(T):
        xt = x[t].astype(np.float64)
        l = wr.astype(np.float64) @ xt
        p = np.exp(l - l.max())
        p /= p.sum()
        want = oracle.expert_forward(xt, shared, 0, wdtype=oracle.F32)
        for e in range(E):
            want = want + p[e] * oracle.expert_forward(xt, experts, e, wdtype=oracle.F32)
        assert np.allclose(r["out"][t], want, rtol=1e-12, atol=1e-13)
        assert sorted(r["idx"][t]) == list(range(E))


def test_expert_relabelling_is_invisible():
    rng = np.random.default_rng(13)
    E, d, f, k, T = 16, 8, 4, 6, 4
    wr = rng.standard_normal((E, d)).astype(np.float32)
    experts = {"gate_up": rng.standard_normal((E, 2 * f, d)).astype(np.float32),
               "down": rng.standard_normal((E, d, f)).astype(np.float32)}
    shared = {"gate_up": rng.standard_normal((1, 2 * f, d)).astype(np.float32),
              "down": rng.standard_normal((1, d, f)).astype(np.float32)}
    x = rng.standard_normal((T, d)).astype(np.float32)
    perm = rng.permutation(E)
    a = oracle.moe_forward(x, wr, experts, shared, top_k=k, wdtype=oracle.F32)
    b = oracle.moe_forward(x, wr[perm], {kk: v[perm] for kk, v in experts.items()}, shared,
                           top_k=k, wdtype=oracle.F32)
    assert np.allclose(a["out"], b["out"], rtol=1e-12, atol=1e-13)
    for t in range(T):
        assert sorted(perm[b["idx"][t]]) == sorted(a["idx"][t])


def test_stack_with_zero_layers_is_identity_and_rounds_input():
    d, E, f = 16, 8, 4
    zero = {"router_w": np.zeros((E, d), np.float32),
            "experts": {"gate_up": np.zeros((E, 2 * f, d), np.uint16),
                        "down": np.zeros((E, d, f), np.uint16)},
            "shared": {"gate_up": np.zeros((1, 2 * f, d), np.uint16),
                       "down": np.zeros((1, d, f), np.uint16)}}
    h0 = np.random.default_rng(14).standard_normal((3, d))
    h, trace = oracle.stack_forward(h0, [zero, zero], top_k=2)
    assert np.array_equal(h, h0)
    assert np.array_equal(trace[0]["x"], oracle.round_to_bf16(oracle.rmsnorm(h0)))


# ---------------------------------------------------------- dense FFN layer

def test_dense_ffn_closed_form_permutation_weights():
    # every token of a dense layer goes through the same SwiGLU map, written out
    # term by term for permutation weights; bf16 activations read as their values
    rng = np.random.default_rng(21)
    d, f, T = 7, 3, 4
    gu, dn, apply = _perm_expert(rng, d, f)
    ws = {"gate_up": gu[None], "down": dn[None]}
    x = (rng.integers(-6, 7, size=(T, d)) / 2.0).astype(np.float32)
    y = oracle.ffn_forward(x, ws, wdtype=oracle.F32)
    assert y.shape == (T, d)
    for t in range(T):
        assert np.allclose(y[t], apply(x[t].astype(np.float64)), rtol=1e-14, atol=1e-15)
    yb = oracle.ffn_forward(synth.bf16_bits(x), ws, wdtype=oracle.F32)  # these x are exact in bf16
    assert np.array_equal(yb, y)


def test_dense_ffn_is_the_top1_layer_of_one_expert():
    # one routed expert, top-1, no shared expert: the renormalised weight of the
    # single chosen logit is exactly 1, whatever the router, so the layer is the FFN
    rng = np.random.default_rng(22)
    d, f, T = 16, 8, 5
    gu = synth.bf16_bits(rng.standard_normal((1, 2 * f, d)) / math.sqrt(d))
    dn = synth.bf16_bits(rng.standard_normal((1, d, f)) / math.sqrt(f))
    ws = {"gate_up": gu, "down": dn}
    x = synth.bf16_bits(rng.standard_normal((T, d)))
    ref = oracle.ffn_forward(x, ws)
    for wr in (np.zeros((1, d), np.float32), rng.standard_normal((1, d)).astype(np.float32)):
        r = oracle.moe_forward(x, wr, ws, None, top_k=1)
        assert (r["idx"] == 0).all() and (r["w"] == 1.0).all()
        assert np.array_equal(r["out"], ref)


# ------------------------------------------------ dense brute force (pure Python)

def _dense_case(wdtype, k, bias, shared, seed):
    """Random dense tiny layer in stored formats, plus its fp64 decoding done
    here (bf16 bits through their binary32 bit layout, NVFP4 through the OCP
    golden tables and the documented packing: even element in the low nibble,
    one E4M3 scale per 16 elements, a tensor scale per matrix)."""
    from oracle import brute
    rng = np.random.default_rng(seed)
    T, d, E, f = 3, 32, 8, 16
    x = synth.bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    router = (rng.standard_normal((E, d)) / math.sqrt(d)).astype(np.float32)
    b = (rng.standard_normal(E) * 0.3).astype(np.float32) if bias else None
    e2m1 = dict(_read_table("e2m1_ocp_mx.txt"))
    e4m3 = dict(_read_table("e4m3_ocp_fp8.txt"))

    def mk(n):
        if wdtype == synth.NVFP4:
            gu = rng.integers(0, 256, (n, 2 * f, d // 2), dtype=np.uint8)
            dn = rng.integers(0, 256, (n, d, f // 2), dtype=np.uint8)
            gs = rng.integers(0x28, 0x41, (n, 2 * f, d // 16), dtype=np.uint8)
            ds = rng.integers(0x28, 0x41, (n, d, f // 16), dtype=np.uint8)
            ts = rng.uniform(0.05, 0.5, (n, 3)).astype(np.float32)
            ws = dict(gate_up=gu, down=dn, gate_up_scales=gs, down_scales=ds, tensor_scales=ts)

            def dq(codes, scales, tsc, K):
                out = []
                for r in range(codes.shape[0]):
                    row = []
                    for c in range(K):
                        byte = int(codes[r][c // 2])
                        code = byte & 0xF if c % 2 == 0 else byte >> 4
                        row.append(e2m1[code] * e4m3[int(scales[r][c // 16])] * float(tsc))
                    out.append(row)
                return out
            dense_gu = [dq(gu[e][:f], gs[e][:f], ts[e][0], d) + dq(gu[e][f:], gs[e][f:], ts[e][1], d)
                        for e in range(n)]
            dense_dn = [dq(dn[e], ds[e], ts[e][2], f) for e in range(n)]
            return ws, dense_gu, dense_dn
        gu = rng.standard_normal((n, 2 * f, d)).astype(np.float32) / np.float32(math.sqrt(d))
        dn = rng.standard_normal((n, d, f)).astype(np.float32) / np.float32(math.sqrt(f))
        if wdtype == synth.BF16:
            gu, dn = synth.bf16_bits(gu), synth.bf16_bits(dn)
            conv = brute.bf16_to_float
        else:
            conv = brute.f32_to_float
        dense_gu = [[[conv(v) for v in row] for row in gu[e]] for e in range(n)]
        dense_dn = [[[conv(v) for v in row] for row in dn[e]] for e in range(n)]
        return dict(gate_up=gu, down=dn), dense_gu, dense_dn

    ex, egu, edn = mk(E)
    sh, sgu, sdn = mk(1) if shared else (None, [None], [None])
    xs = [[brute.bf16_to_float(v) for v in row] for row in x]
    want = brute.layer(xs, [[float(v) for v in row] for row in router],
                       None if b is None else [float(v) for v in b], egu, edn, sgu[0], sdn[0], k)
    got = oracle.moe_forward(x, router, ex, sh, top_k=k, router_bias=b, wdtype=wdtype)
    return got, want


def test_dense_layer_matches_brute_force():
    # (not parametrized: the planted-mistake test calls every pin without arguments)
    for wdtype in (synth.F32, synth.BF16, synth.NVFP4):
        for k, bias, shared in ((1, False, True), (2, True, True), (6, False, False), (6, True, True)):
            got, (out, sel, w, logits) = _dense_case(wdtype, k, bias, shared, seed=17 + k)
            assert np.array_equal(got["idx"], np.array(sel, np.int32))
            assert np.allclose(got["logits"], np.array(logits), rtol=0, atol=1e-13)
            assert np.allclose(got["w"], np.array(w), rtol=0, atol=1e-14)
            out = np.array(out)
            scale = np.abs(out).max()
            assert scale > 0
            err = np.abs(got["out"] - out).max()
            assert err <= 1e-12 * scale, (wdtype, k, bias, shared, err / scale)


def test_dense_brute_force_with_ties():
    # duplicate router rows (equal logits): the brute force's stable sort and
    # the oracle's selection keep the lower index
    from oracle import brute
    rng = np.random.default_rng(3)
    d, E = 32, 8
    router = (rng.standard_normal((E, d)) / math.sqrt(d)).astype(np.float32)
    router[5] = router[2]
    router[7] = router[2]
    b = np.zeros(E, np.float32)
    b[[2, 5, 7]] = 20.0  # the three equal rows lead every token
    x = synth.bf16_bits(rng.standard_normal((4, d)).astype(np.float32))
    got = oracle.route(x, router, top_k=2, router_bias=b)
    for t in range(4):
        xs = [brute.bf16_to_float(v) for v in x[t]]
        _, chosen, w = brute.route(xs, [[float(v) for v in r] for r in router], [float(v) for v in b], 2)
        assert chosen == [2, 5]
        assert list(got["idx"][t]) == chosen
        assert np.allclose(got["w"][t], w, rtol=0, atol=1e-15)
