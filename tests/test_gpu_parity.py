"""GPU parity: the HIP layer (through the C ABI) against the fp64 oracle.

Reduced shapes span several work items with ragged tails; the full-size
cases are the workloads the benchmark times: decode and NVFP4 compared on
every token, prefill on every token's selection and on at least 512 tokens'
outputs that cover every non-empty expert group, and the 47-layer stack layer
by layer on the GPU's own inputs.  Every case runs a bf16-activation layer
with both output forms (see gpu_helpers): the fp32 output is gated at the
plain bound, the bf16 output must be its correct rounding, and the full-size
workloads gate the bf16 output at the plain bound too.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import (check_layer, check_permutation, check_selection, compare, dev_array,
                         dev_layer, make_layer_obj, out_host, run_gpu, run_oracle,
                         stack_layer_gpu, teacher_forced_layer, x_device)
from sparse_moe_transformer_gemv_amd import (FLINT_FORCE_DECODE_PATH, FLINT_FORCE_PREFILL_PATH,
                                             FlintError, flint_rmsnorm_forward)

pytestmark = pytest.mark.gpu


def _case(cfg_id, T, max_tokens=None, flags=0, draw=0, full=False, **override):
    L = synth.layer(cfg_id, **override)
    c = L["cfg"]
    x = synth.hidden(cfg_id, T, c["d"], c["act"], draw=draw)
    print("case cfg=%d T=%d flags=%d %s" % (cfg_id, T, flags, override), flush=True)
    layer = make_layer_obj(c, max_tokens or T, flags)
    D = dev_layer(L)
    ref = run_oracle(L, x)
    rep, rout = check_layer(layer, D, x, ref, c, full=full)
    check_permutation(rout, T, c["k"], c["E"])
    print("  -> %s" % rep, flush=True)
    return L, x, layer, D, rout, ref


def test_tiny_f32_workload():
    _case(0, 64)


@pytest.mark.parametrize("T", [1, 3, 17, 64])
def test_small_bf16_decode(T):
    _case(1, T, d=256, E=64, f=64, fs=96)


@pytest.mark.parametrize("T", [1, 5, 40])
def test_small_nvfp4_decode(T):
    _case(4, T, d=256, E=32, k=4, f=64, fs=64)


@pytest.mark.parametrize("T", [1, 9, 16, 23, 64])
def test_small_nvfp4_matrix_core_path(T):
    # d, f, fs multiples of 512 select the NVFP4 matrix-core expert kernels;
    # the shared expert has more features than a routed one
    _case(4, T, d=512, E=32, k=4, f=512, fs=1024)


def test_nvfp4_decode_path_above_64_tokens():
    # the expert-GEMV kernels at a prefill-sized batch (forced)
    _case(4, 150, flags=FLINT_FORCE_DECODE_PATH, d=512, E=32, k=4, f=512, fs=1024)


@pytest.mark.parametrize("T,flags", [(150, 0), (37, FLINT_FORCE_PREFILL_PATH), (1, FLINT_FORCE_PREFILL_PATH)])
def test_nvfp4_prefill_path(T, flags):
    # grouped GEMM with the NVFP4 weights dequantised in registers; above 64
    # tokens the host picks it by itself
    _case(4, T, flags=flags, d=512, E=32, k=4, f=512, fs=1024)


def test_nvfp4_prefill_zipf_ragged():
    # Zipf-skewed routing, a group spanning several tiles, ragged tails, and
    # widths that take half tiles (f = 384: three 128-wide halves per feature block)
    _case(4, 700, d=512, E=64, f=384, fs=128, bias=True)


@pytest.mark.parametrize("T", [5, 19])
def test_nvfp4_matrix_core_path_d1024_ragged_f(T):
    # f = 1536: three 128-groups per wave in the down kernel
    _case(4, T, d=1024, E=16, k=3, f=1536, fs=512)


@pytest.mark.parametrize("T", [1, 7, 40, 64])
def test_small_bf16_matrix_core_path(T):
    # d % 128 == 0 and f, fs % 128 == 0 select the MFMA router and expert kernels
    _case(1, T, d=256, E=64, f=128, fs=256)


@pytest.mark.parametrize("T,shared", [(17, True), (40, True), (64, False)])
def test_decode_down_through_lds(T, shared):
    # routed and shared experts 512 wide, more than 16 tokens: the down kernel
    # stages three waves' weights through LDS (the shared group spans several
    # 16-token tiles; the last case has no shared expert)
    if shared:
        _case(1, T, d=512, E=64, k=6, f=512, fs=512)
        return
    L = synth.layer(1, d=512, E=64, k=6, f=512, fs=512)
    L["shared"] = None
    c = dict(L["cfg"], fs=0)
    L["cfg"] = c
    x = synth.hidden(1, T, c["d"], c["act"])
    layer = make_layer_obj(c, T)
    ref = oracle.moe_forward(x, L["router_w"], L["experts"], None, top_k=c["k"], wdtype=synth.BF16)
    rep, rout = check_layer(layer, dev_layer(L), x, ref, c)
    check_permutation(rout, T, c["k"], c["E"])


@pytest.mark.parametrize("T", [16, 48])
def test_decode_gateup_d2048(T):
    # d = 2048: three gate/up waves stage weights through LDS and the fourth
    # loads into registers; ragged groups over few experts
    _case(1, T, d=2048, E=32, k=4, f=512, fs=512)


def test_matrix_core_path_d128_k2():
    _case(1, 33, d=128, E=32, k=2, f=128, fs=128)


def test_zipf_bias_many_tokens_decode_path():
    # skewed routing (one expert takes most tokens), forced onto the decode path
    _case(2, 300, flags=FLINT_FORCE_DECODE_PATH, d=256, E=64, f=128, fs=128)


@pytest.mark.parametrize("T", [1, 37, 200])
def test_small_prefill_path_forced(T):
    _case(1, T, flags=FLINT_FORCE_PREFILL_PATH, d=256, E=64, f=128, fs=256)


def test_prefill_path_zipf_default_choice():
    # T above the decode threshold picks the grouped-MFMA path by itself
    _case(2, 700, d=512, E=64, f=256, fs=128)


def test_prefill_path_k8_odd_experts():
    _case(2, 333, flags=FLINT_FORCE_PREFILL_PATH, d=256, E=100, k=8, f=128, fs=128)


def test_prefill_sort_beyond_4096_tokens():
    # more than 256 sixteen-token blocks of expert counts, so every sort block
    # reads them in more than one pass, with a ragged last block and the Zipf
    # bias; every token's output against the oracle
    _case(2, 5000, d=256, E=64, f=128, fs=128)


def test_f32_activations_bf16_weights():
    _case(1, 9, d=192, E=48, f=32, fs=64, act=synth.F32)


def test_no_shared_expert():
    L = synth.layer(1, d=128, E=16, f=32, fs=32)
    L["shared"] = None
    c = dict(L["cfg"], fs=0)
    L["cfg"] = c
    x = synth.hidden(1, 7, 128, synth.BF16)
    layer = make_layer_obj(c, 8)
    ref = oracle.moe_forward(x, L["router_w"], L["experts"], None, top_k=c["k"],
                             wdtype=synth.BF16)
    check_layer(layer, dev_layer(L), x, ref, c)


def test_no_shared_expert_decode_then_prefill_same_handle():
    # the prefill forward must not pick up rows an earlier decode forward left in
    # the shared slots' place (there is no shared expert to write them)
    L = synth.layer(1, d=256, E=32, f=128, fs=128)
    L["shared"] = None
    c = dict(L["cfg"], fs=0)
    L["cfg"] = c
    layer = make_layer_obj(c, 256)
    D = dev_layer(L)
    # decode at T=64 writes rows over the bytes where the T=100 prefill
    # forward's shared-slot rows would sit
    for T in (64, 100):
        x = synth.hidden(1, T, 256, synth.BF16, draw=T)
        ref = oracle.moe_forward(x, L["router_w"], L["experts"], None, top_k=c["k"], wdtype=synth.BF16)
        rep, _ = check_layer(layer, D, x, ref, c)
        print("no shared expert T=%d: %s" % (T, rep), flush=True)


@pytest.mark.parametrize("T,flags", [(48, 0), (700, FLINT_FORCE_PREFILL_PATH), (300, FLINT_FORCE_DECODE_PATH)])
def test_every_token_picks_the_same_experts(T, flags):
    # degenerate routing: a router bias makes every token choose the same k
    # experts (in a fixed order), so k groups hold all T tokens and every
    # other expert is empty; one prefill group spans several 256-row tiles
    L = synth.layer(1, d=256, E=64, f=128, fs=128)
    b = np.zeros(64, np.float32)
    chosen = [63, 3, 40, 9, 33, 17]
    b[chosen] = [60.0, 50.0, 40.0, 30.0, 20.0, 10.0]
    L["router_bias"] = b
    c = L["cfg"]
    x = synth.hidden(1, T, 256, synth.BF16, draw=5)
    layer = make_layer_obj(c, T, flags)
    ref = run_oracle(L, x)
    rep, rout = check_layer(layer, dev_layer(L), x, ref, c)
    assert np.array_equal(rout["idx"], np.tile(np.array(chosen), (T, 1)))
    check_permutation(rout, T, c["k"], c["E"])
    print("same experts T=%d flags=%d: %s" % (T, flags, rep), flush=True)


def test_odd_expert_count_and_k8():
    _case(1, 20, d=128, E=100, k=8, f=32, fs=32)


@pytest.mark.parametrize("flags", [0, FLINT_FORCE_PREFILL_PATH])
def test_every_expert_chosen(flags):
    # k = E: each token takes every expert (a dense softmax mixture)
    _case(1, 13, flags=flags, d=256, E=8, k=8, f=128, fs=128)


@pytest.mark.parametrize("flags", [0, FLINT_FORCE_PREFILL_PATH])
def test_single_expert(flags):
    # E = 1, k = 1: one routed expert (weight 1) plus the shared one
    _case(1, 21, flags=flags, d=256, E=1, k=1, f=128, fs=128)


def test_top1():
    _case(1, 11, d=128, E=64, k=1, f=32, fs=32)


def test_equal_logits_pick_lowest_indices():
    L = synth.layer(1, d=128, E=64, f=32, fs=32)
    L["router_w"] = np.zeros_like(L["router_w"])
    c = L["cfg"]
    x = synth.hidden(1, 5, 128, synth.BF16)
    layer = make_layer_obj(c, 5)
    out, rout = run_gpu(layer, dev_layer(L), x)
    assert np.array_equal(rout["idx"], np.tile(np.arange(6), (5, 1)))
    assert np.allclose(rout["weights"], 1.0 / 6, atol=1e-7)
    ref = run_oracle(L, x)
    # every gap is 0 here, so compare the outputs directly
    err = np.abs(out - ref["out"]).max()
    assert err <= 2e-2 * np.sqrt(np.mean(ref["out"] ** 2))


def test_zero_tokens_is_a_noop():
    L = synth.layer(1, d=128, E=16, f=32, fs=32)
    layer = make_layer_obj(L["cfg"], 4)
    D = dev_layer(L)
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    layer.forward(x, D["router_w"], D["experts"], D["shared"], out=out)
    torch.cuda.synchronize()


def test_too_many_tokens_rejected():
    L = synth.layer(1, d=128, E=16, f=32, fs=32)
    layer = make_layer_obj(L["cfg"], 4)
    D = dev_layer(L)
    x = x_device(synth.hidden(1, 5, 128, synth.BF16))
    with pytest.raises(FlintError):
        layer.forward(x, D["router_w"], D["experts"], D["shared"])


def test_residual_gives_fp32_sum():
    L = synth.layer(1, d=256, E=32, f=64, fs=64)
    c = L["cfg"]
    x = synth.hidden(1, 6, 256, synth.BF16)
    res = np.random.default_rng(3).standard_normal((6, 256)).astype(np.float32)
    layer = make_layer_obj(c, 6)
    D = dev_layer(L)
    rd = dev_array(res)
    out, rout = run_gpu(layer, D, x, residual=rd)
    ref = run_oracle(L, x)
    ref = dict(ref, out=ref["out"] + res.astype(np.float64))
    compare(out, rout, ref, c["k"], synth.BF16)
    # in place: out aliases the residual
    layer.forward(x_device(x), D["router_w"], D["experts"], D["shared"], residual=rd, out=rd)
    torch.cuda.synchronize()
    assert np.abs(out_host(rd) - out).max() <= 1e-6 * np.abs(out).max()


def test_rmsnorm_kernel():
    from sparse_moe_transformer_gemv_amd import flint_rmsnorm_forward
    h = np.random.default_rng(4).standard_normal((32, 2048)).astype(np.float32) * 3
    out = flint_rmsnorm_forward(dev_array(h), 1e-6)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    want = oracle.round_to_bf16(oracle.rmsnorm(h.astype(np.float64), 1e-6))
    # fp32 vs fp64 arithmetic may land on the other side of a bf16 midpoint
    diff = np.abs(got.astype(np.int32) - want.astype(np.int32))
    assert diff.max() <= 1 and (diff > 0).mean() < 1e-3


def test_deterministic_repeat():
    L = synth.layer(1, d=256, E=64, f=64, fs=64)
    c = L["cfg"]
    x = synth.hidden(1, 33, 256, synth.BF16)
    layer = make_layer_obj(c, 64)
    D = dev_layer(L)
    a, ra = run_gpu(layer, D, x)
    b, rb = run_gpu(layer, D, x)
    assert np.array_equal(a, b)
    assert np.array_equal(ra["sorted_pair"], rb["sorted_pair"])


# ----------------------------------------------------------- full-size workloads

@pytest.fixture(scope="module")
def decode_layer():
    L = synth.layer(1)
    return L, dev_layer(L)


@pytest.mark.parametrize("T", [1, 4, 16, 64])
def test_full_decode_bf16(decode_layer, T):
    L, D = decode_layer
    c = L["cfg"]
    x = synth.hidden(1, T, c["d"], c["act"])
    layer = make_layer_obj(c, 64)
    ref = run_oracle(L, x)
    rep, rout = check_layer(layer, D, x, ref, c, full=True)
    check_permutation(rout, T, c["k"], c["E"])
    assert layer.fault() == 0
    print("decode bf16 T=%d: %s" % (T, rep), flush=True)


@pytest.fixture(scope="module")
def fp4_layer():
    L = synth.layer(4)
    return L, dev_layer(L)


@pytest.mark.parametrize("T", [1, 16])
def test_full_decode_nvfp4(fp4_layer, T):
    L, D = fp4_layer
    c = L["cfg"]
    x = synth.hidden(4, T, c["d"], c["act"])
    layer = make_layer_obj(c, 16)
    ref = run_oracle(L, x)
    rep, rout = check_layer(layer, D, x, ref, c, full=True)
    check_permutation(rout, T, c["k"], c["E"])
    print("decode nvfp4 T=%d: %s" % (T, rep), flush=True)


@pytest.mark.parametrize("which,T,unfused", [("bf16", 4, True), ("bf16", 7, False), ("nvfp4", 3, True)])
def test_decode_combine_in_down_with_residual(decode_layer, fp4_layer, which, T, unfused):
    # small batches that run as separate launches fold the combine into the
    # down kernel (bf16 up to 8 tokens, NVFP4 up to 4; the smallest batches
    # take the single launch unless it is turned off); a nonzero residual is
    # added there, also when the output aliases it
    from sparse_moe_transformer_gemv_amd import FLINT_UNFUSED_DECODE
    L, D = decode_layer if which == "bf16" else fp4_layer
    c = L["cfg"]
    cfg_id = 1 if which == "bf16" else 4
    x = synth.hidden(cfg_id, T, c["d"], c["act"])
    res = np.random.default_rng(11).standard_normal((T, c["d"])).astype(np.float32)
    layer = make_layer_obj(c, 16, FLINT_UNFUSED_DECODE if unfused else 0)
    rd = dev_array(res)
    out, rout = run_gpu(layer, D, x, residual=rd)
    ref = run_oracle(L, x)
    ref = dict(ref, out=ref["out"] + res.astype(np.float64))
    rep = compare(out, rout, ref, c["k"], c["wdtype"])
    layer.forward(x_device(x), D["router_w"], D["experts"], D["shared"], residual=rd, out=rd)
    torch.cuda.synchronize()
    assert np.abs(out_host(rd) - out).max() <= 1e-6 * np.abs(out).max()
    print("combine in down %s T=%d: %s" % (which, T, rep), flush=True)


@pytest.mark.parametrize("which,T,flags", [("bf16", 4, 0), ("bf16", 64, 0), ("nvfp4", 1, 0),
                                           ("bf16", 700, FLINT_FORCE_PREFILL_PATH)])
def test_forward_replayed_from_hip_graph(decode_layer, fp4_layer, which, T, flags):
    # a forward captured in a HIP graph and replayed, with eager forwards and new
    # inputs between the replays, gives the eager result bit for bit every time
    # (the hand-off tickets reset themselves; nothing is allocated or cleared
    # with a memset inside the forward)
    L, D = decode_layer if which == "bf16" else fp4_layer
    c = L["cfg"]
    cfg_id = 1 if which == "bf16" else 4
    layer = make_layer_obj(c, max(T, 64), flags)
    xs = [x_device(synth.hidden(cfg_id, T, c["d"], c["act"], draw=i)) for i in range(2)]
    fwd = lambda x, out=None: layer.forward(x, D["router_w"], D["experts"], D["shared"], out=out)
    ref = []
    for x in xs:
        o = fwd(x)
        torch.cuda.synchronize()
        ref.append(out_host(o))
    x_static = xs[0].clone()
    out_static = torch.empty_like(fwd(x_static))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fwd(x_static, out_static)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd(x_static, out_static)
    for rep in range(4):
        i = rep % 2
        x_static.copy_(xs[i])
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out_host(out_static), ref[i]), "replay %d differs from the eager forward" % rep
        fwd(xs[1 - i])  # eager work between the replays
        torch.cuda.synchronize()


@pytest.fixture(scope="module")
def prefill_layer():
    L = synth.layer(2)
    return L, dev_layer(L)


def test_full_prefill_zipf(prefill_layer):
    # selection of all 4096 tokens against the router-only oracle; outputs of
    # at least 512 tokens that include the first and last token of every
    # non-empty expert group (so every group's tiles, ragged tails included,
    # are compared), both output forms at the plain bound
    L, D = prefill_layer
    c = L["cfg"]
    T, k, E = 4096, c["k"], c["E"]
    x = synth.hidden(2, T, c["d"], c["act"])
    layer = make_layer_obj(c, T)
    out, rout = run_gpu(layer, D, x)
    check_permutation(rout, T, k, E)
    rref = oracle.route(x, L["router_w"], top_k=k, router_bias=L["router_bias"])
    sel_ok, near = check_selection(rout["idx"], rout["weights"], rref, k)
    dl = np.abs(rout["logits"] - rref["logits"]).max()
    assert dl <= 2e-5, "router logits differ from the oracle's by %.3g" % dl
    counts = rout["counts"]
    pick = set()
    for e in np.where(counts > 0)[0]:
        toks = np.where((rout["idx"] == e).any(1))[0]
        pick.update((int(toks[0]), int(toks[-1])))
    n_group_tokens = len(pick)
    rng = np.random.default_rng(7)
    rest = np.setdiff1d(np.arange(T), np.array(sorted(pick)))
    pick.update(rng.choice(rest, max(0, 512 - len(pick)), replace=False).tolist())
    pick = np.array(sorted(pick))
    ref = run_oracle(L, x[pick])
    rep, _ = check_layer(layer, D, x, ref, c, full=True, rows=pick, tokens=pick)
    print("prefill T=4096: selection of all tokens (near ties %d, mismatched %d, max logit diff %.2e); "
          "outputs of %d tokens (%d from group ends), groups used %d, largest %d: %s" % (
              int(near.sum()), int((near & ~sel_ok).sum()), dl, len(pick), n_group_tokens,
              int((counts > 0).sum()), int(counts.max()), rep), flush=True)


@pytest.fixture(scope="module")
def fp4_prefill_layer():
    L = synth.layer(4, bias=True)  # NVFP4 weights, the Zipf router bias
    return L, dev_layer(L)


def test_full_prefill_nvfp4_zipf(fp4_prefill_layer):
    # the 4-bit layer at T = 4096: selection of every token, outputs of >= 512
    # tokens covering every non-empty group, both output forms at the plain bound
    L, D = fp4_prefill_layer
    c = L["cfg"]
    T, k, E = 4096, c["k"], c["E"]
    x = synth.hidden(4, T, c["d"], c["act"], draw=7)
    layer = make_layer_obj(c, T)
    out, rout = run_gpu(layer, D, x)
    check_permutation(rout, T, k, E)
    rref = oracle.route(x, L["router_w"], top_k=k, router_bias=L["router_bias"])
    sel_ok, near = check_selection(rout["idx"], rout["weights"], rref, k)
    counts = rout["counts"]
    pick = set()
    for e in np.where(counts > 0)[0]:
        toks = np.where((rout["idx"] == e).any(1))[0]
        pick.update((int(toks[0]), int(toks[-1])))
    rng = np.random.default_rng(11)
    rest = np.setdiff1d(np.arange(T), np.array(sorted(pick)))
    pick.update(rng.choice(rest, max(0, 512 - len(pick)), replace=False).tolist())
    pick = np.array(sorted(pick))
    ref = run_oracle(L, x[pick])
    rep, _ = check_layer(layer, D, x, ref, c, full=True, rows=pick, tokens=pick)
    print("nvfp4 prefill T=4096: near ties %d (mismatched %d); outputs of %d tokens, groups used %d: %s" % (
        int(near.sum()), int((near & ~sel_ok).sum()), len(pick), int((counts > 0).sum()), rep), flush=True)


def _stack_teacher_forced(n_layers, T, **override):
    """The stacked workload, one resident layer at a time: every layer's GPU
    step is checked against the oracle on the GPU's own input (pre-norm and
    layer, see teacher_forced_layer).  The free-running oracle stack alongside
    it gives the end-to-end drift and the selection flips, which are
    reported, not gated: requantising every layer's input to bf16 lets
    fp32-vs-fp64 differences grow through the layers."""
    cfg = 3
    c = dict(synth.CONFIGS[cfg], **override)
    moe = make_layer_obj(c, T)
    h0 = synth.hidden(cfg, T, c["d"], synth.F32)
    h = dev_array(h0.copy())
    x = torch.empty((T, c["d"]), dtype=torch.bfloat16, device="cuda")
    xn = torch.empty_like(x)
    flint_rmsnorm_forward(h, 1e-6, out=x)
    h_ref = h0.astype(np.float64)
    worst, flips, flipped = 0.0, 0, np.zeros(T, bool)
    for l in range(n_layers):
        L = synth.layer(cfg, l, **override)
        D = dev_layer(L)
        rec = stack_layer_gpu(moe, h, D, x, xn, record=True)
        x, xn = xn, x
        rep = teacher_forced_layer(rec, L, c["k"])
        worst = max(worst, rep["ratio"])
        if l % 8 == 0 or l == n_layers - 1:
            print("  layer %d on the GPU's input: %s" % (l, rep), flush=True)
        xb = oracle.round_to_bf16(oracle.rmsnorm(h_ref))
        r = oracle.moe_forward(xb, L["router_w"], L["experts"], L["shared"], top_k=c["k"],
                               wdtype=c["wdtype"])
        f = np.array([set(r["idx"][t]) != set(rec["idx"][t]) for t in range(T)])
        flips += int(f.sum())
        flipped |= f
        h_ref = h_ref + r["out"]
        del D, L
    torch.cuda.synchronize()
    hg = out_host(h)
    assert np.all(np.isfinite(hg))
    e2e = float(np.abs(hg - h_ref).max() / np.sqrt(np.mean(h_ref ** 2)))
    print("stack %d layers T=%d %s: worst teacher-forced layer ratio %.4f; end to end (reported): "
          "max|err|/RMS %.4f, %d selection flips in %d tokens" % (
              n_layers, T, override, worst, e2e, flips, int(flipped.sum())), flush=True)


@pytest.mark.parametrize("cfg_id,T,flags,over", [
    (1, 32, 0, dict(d=512, E=64, f=128, fs=128)),                          # combine kernel with the norm
    (1, 4, 0, dict(d=512, E=64, f=128, fs=128)),                           # single launch, then the norm
    (1, 12, 0, dict(d=512, E=64, f=128, fs=128)),                          # combine folded into down
    (1, 200, FLINT_FORCE_PREFILL_PATH, dict(d=256, E=64, f=128, fs=128)),  # prefill path
    (4, 2, 0, dict(d=512, E=32, k=4, f=512, fs=512)),                      # NVFP4
    (1, 32, 0, dict(d=8192, E=16, k=2, f=128, fs=128)),                    # d past the one-launch form
])
def test_forward_prenorm_matches_forward_then_rmsnorm(cfg_id, T, flags, over):
    # the pre-norm output of the stacked step equals, bit for bit, the layer's
    # forward followed by the RMSNorm kernel; out may be the residual itself
    L = synth.layer(cfg_id, **over)
    c = L["cfg"]
    D = dev_layer(L)
    x = x_device(synth.hidden(cfg_id, T, c["d"], c["act"], draw=5))
    h0 = dev_array(np.random.default_rng(8).standard_normal((T, c["d"])).astype(np.float32))
    layer = make_layer_obj(c, max(T, 64), flags)
    ref_out = layer.forward(x, D["router_w"], D["experts"], D["shared"], D["router_bias"], residual=h0)
    ref_norm = flint_rmsnorm_forward(ref_out, 1e-6)
    h = h0.clone()
    out, norm = layer.forward_prenorm(x, D["router_w"], D["experts"], D["shared"], residual=h, eps=1e-6,
                                      router_bias=D["router_bias"], out=h)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), "the layer output differs"
    assert torch.equal(norm.view(torch.int16), ref_norm.view(torch.int16)), "the pre-norm output differs"
    print("prenorm cfg=%d T=%d %s: equal to forward + rmsnorm" % (cfg_id, T, over), flush=True)


def test_stack_47_layers_small_shape():
    _stack_teacher_forced(47, 32, d=256, E=64, f=128, fs=128)


@pytest.mark.timeout(600)
def test_stack_47_layers_full_size():
    # every layer at full size, all 32 tokens
    _stack_teacher_forced(47, 32)


# ------------------------------------------------------------- dense FFN layer

@pytest.mark.parametrize("cfg_id,d,F,T,flags", [
    (1, 256, 512, 3, 0),                           # decode, matrix-core kernels
    (1, 256, 512, 300, FLINT_FORCE_PREFILL_PATH),  # grouped GEMM, one group
    (1, 2048, 16384, 4, 0),                        # full width decode: K split in 16 chunks, combine folded
    (1, 2048, 16384, 32, 0),                       # the same without the folded combine
    (1, 2048, 16384, 4096, 0),                     # full width prefill, sampled rows
    (4, 2048, 2048, 16, 0),                        # NVFP4 matrix-core decode
    (4, 2048, 16384, 2, 0),                        # NVFP4, K split in 8 chunks
    (4, 2048, 16384, 32, 0),                       # the same at a larger batch
])
def test_dense_ffn(cfg_id, d, F, T, flags):
    from sparse_moe_transformer_gemv_amd import DenseFFN
    from gpu_helpers import TOL, dev_weights, rne_bf16
    wd = synth.CONFIGS[cfg_id]["wdtype"]
    act = synth.CONFIGS[cfg_id]["act"]
    ws = synth.expert_set(cfg_id, 0, 1, d, F, wd)
    x = synth.hidden(cfg_id, T, d, act)
    ffn = DenseFFN(d, F, act, wd, max_tokens=max(T, 64), flags=flags)
    out = out_host(ffn.forward(x_device(x), dev_weights(ws, wd)))
    # the fp32-output form (zero residual) meets the plain bound
    zero = torch.zeros((T, d), dtype=torch.float32, device="cuda")
    out32 = out_host(ffn.forward(x_device(x), dev_weights(ws, wd), residual=zero))
    torch.cuda.synchronize()
    assert np.array_equal(out, rne_bf16(out32)), "bf16 output is not the rounding of the fp32 output"
    rows = np.arange(T) if T <= 64 else np.random.default_rng(5).choice(T, 24, replace=False)
    ref = oracle.ffn_forward(x[rows], ws, wdtype=wd)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err32 = np.abs(out32[rows] - ref)
    assert err32.max() <= TOL[wd] * rms, "fp32 out: max|err| %.3e vs %.1e * RMS %.3e" % (
        err32.max(), TOL[wd], rms)
    err = np.abs(out[rows] - ref)
    print("dense FFN cfg %d d=%d F=%d T=%d: max|err|/RMS %.4f (fp32 out, gated), %.4f (bf16 out)" % (
        cfg_id, d, F, T, err32.max() / rms, err.max() / rms), flush=True)


@pytest.mark.parametrize("T", [3, 40])
def test_wide_shared_expert_splits_k(T):
    # a shared expert wider than one K chunk of the decode down kernel: only its
    # group is split (two chunks), the routed groups are not
    _case(1, T, d=256, E=64, f=128, fs=2048)


@pytest.mark.parametrize("T", [3, 20])
def test_wide_nvfp4_shared_expert_splits_k(T):
    # an NVFP4 shared expert twice as wide as one K chunk of the NVFP4 down kernel
    _case(4, T, d=512, E=64, f=512, fs=4096)


# ------------------------------------------------------- single-launch decode

FUSED_SHAPES = [
    dict(d=256, E=64, f=128, fs=256),
    dict(d=512, E=100, k=8, f=256, fs=128),   # odd expert count, k = 8
    dict(d=256, E=32, f=128, fs=0),           # no shared expert
    dict(d=1024, E=128, f=256, fs=512),       # shared expert wider than a routed one
]


@pytest.mark.parametrize("T", [1, 2, 5, 8])
@pytest.mark.parametrize("over", FUSED_SHAPES, ids=["d256", "E100k8", "noshared", "d1024"])
def test_single_launch_decode(T, over, monkeypatch):
    # small bf16 batches run as one launch (the timing hook sees exactly one
    # launch of it); the result meets the oracle, and the routing equals that of
    # the separate route / gate-up / down launches.  The limit is raised to the
    # kernel's own 8 tokens so that every batch size it takes is covered.
    from sparse_moe_transformer_gemv_amd import FLINT_UNFUSED_DECODE, KERNEL_FUSED
    monkeypatch.setenv("FLINT_MOE_FUSED_MAX_T", "8")
    over = dict(over)
    no_shared = over.get("fs") == 0
    if no_shared:
        over["fs"] = 32
    L = synth.layer(1, **over)
    c = L["cfg"]
    if no_shared:
        L["shared"] = None
        c = dict(c, fs=0)
        L["cfg"] = c
    x = synth.hidden(1, T, c["d"], c["act"], draw=T)
    D = dev_layer(L)
    ref = oracle.moe_forward(x, L["router_w"], L["experts"], L["shared"], top_k=c["k"],
                             wdtype=synth.BF16)
    fused = make_layer_obj(c, 16)
    rep, rout = check_layer(fused, D, x, ref, c)
    check_permutation(rout, T, c["k"], c["E"])
    fused.profile_begin(KERNEL_FUSED, 4)
    run_gpu(fused, D, x, routing=False)
    assert len(fused.profile_end()) == 1, "the single-launch decode kernel did not run"
    assert fused.fault() == 0, "a grid-barrier wait gave up"
    sep = make_layer_obj(c, 16, FLINT_UNFUSED_DECODE)
    rep2, rout2 = check_layer(sep, D, x, ref, c)
    assert all(set(a) == set(b) for a, b in zip(rout["idx"], rout2["idx"]))
    print("single launch T=%d %s: %s | separate launches: %s" % (T, over, rep, rep2), flush=True)


FUSED_FP4_SHAPES = [
    dict(d=512, E=32, k=4, f=512, fs=512),
    dict(d=1024, E=100, k=8, f=512, fs=0),     # odd expert count, k = 8, no shared expert
    dict(d=2048, E=64, k=6, f=512, fs=1024),   # shared expert wider than a routed one
]


@pytest.mark.parametrize("T", [1, 3, 8])
@pytest.mark.parametrize("over", FUSED_FP4_SHAPES, ids=["d512", "E100k8noshared", "d2048fs1024"])
def test_single_launch_decode_nvfp4(T, over, monkeypatch):
    # NVFP4 weights take the single launch too: one launch of it, the oracle's
    # result, the separate launches' routing, a clear fault word (limit raised
    # to the kernel's own 8 tokens, as above)
    from sparse_moe_transformer_gemv_amd import FLINT_UNFUSED_DECODE, KERNEL_FUSED
    monkeypatch.setenv("FLINT_MOE_FUSED_MAX_T", "8")
    over = dict(over)
    no_shared = over.get("fs") == 0
    if no_shared:
        over["fs"] = 512
    L = synth.layer(4, **over)
    c = L["cfg"]
    if no_shared:
        L["shared"] = None
        c = dict(c, fs=0)
        L["cfg"] = c
    x = synth.hidden(4, T, c["d"], c["act"], draw=T)
    D = dev_layer(L)
    ref = oracle.moe_forward(x, L["router_w"], L["experts"], L["shared"], top_k=c["k"], wdtype=synth.NVFP4)
    fused = make_layer_obj(c, 16)
    rep, rout = check_layer(fused, D, x, ref, c)
    check_permutation(rout, T, c["k"], c["E"])
    fused.profile_begin(KERNEL_FUSED, 4)
    run_gpu(fused, D, x, routing=False)
    assert len(fused.profile_end()) == 1, "the single-launch decode kernel did not run"
    assert fused.fault() == 0, "a grid-barrier wait gave up"
    sep = make_layer_obj(c, 16, FLINT_UNFUSED_DECODE)
    rep2, rout2 = check_layer(sep, D, x, ref, c)
    assert all(set(a) == set(b) for a, b in zip(rout["idx"], rout2["idx"]))
    print("single launch nvfp4 T=%d %s: %s | separate launches: %s" % (T, over, rep, rep2), flush=True)


def test_single_launch_decode_back_to_back_and_graph(monkeypatch):
    # consecutive launches (barrier counters and work queues reset themselves),
    # changing batch sizes (T = 16 runs as separate launches on the same
    # handle), and replay from a HIP graph; the limit is raised to 8 tokens so
    # that T = 7 takes the single launch as well
    monkeypatch.setenv("FLINT_MOE_FUSED_MAX_T", "8")
    L = synth.layer(1, d=256, E=64, f=128, fs=256)
    c = L["cfg"]
    D = dev_layer(L)
    layer = make_layer_obj(c, 16)
    for i, T in enumerate([3, 16, 1, 16, 7, 7, 2]):
        x = synth.hidden(1, T, c["d"], c["act"], draw=40 + i)
        out, rout = run_gpu(layer, D, x, residual=torch.zeros((T, c["d"]), device="cuda"))
        compare(out, rout, run_oracle(L, x), c["k"], c["wdtype"])
    T = 5
    xs = [x_device(synth.hidden(1, T, c["d"], c["act"], draw=60 + i)) for i in range(2)]
    fwd = lambda x, out=None: layer.forward(x, D["router_w"], D["experts"], D["shared"], out=out)
    ref = [out_host(fwd(x)) for x in xs]
    torch.cuda.synchronize()
    x_static = xs[0].clone()
    out_static = torch.empty_like(fwd(x_static))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fwd(x_static, out_static)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd(x_static, out_static)
    for rep in range(6):
        i = rep % 2
        x_static.copy_(xs[i])
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out_host(out_static), ref[i]), "replay %d differs" % rep
        fwd(xs[1 - i])
        torch.cuda.synchronize()
    assert layer.fault() == 0, "a grid-barrier wait gave up"


@pytest.mark.parametrize("cfg_id,T,env,fused", [
    (1, 5, None, True), (1, 6, None, False),   # bf16 weights: single launch up to 5 tokens
    (4, 4, None, True), (4, 5, None, False),   # NVFP4 weights: up to 4
    (1, 1, "0", False), (4, 6, "6", True),     # the environment override
])
def test_single_launch_default_limits(cfg_id, T, env, fused, monkeypatch):
    # which batches take the single launch by default, and the override; the
    # result meets the oracle either way
    from sparse_moe_transformer_gemv_amd import KERNEL_FUSED
    if env is None:
        monkeypatch.delenv("FLINT_MOE_FUSED_MAX_T", raising=False)
    else:
        monkeypatch.setenv("FLINT_MOE_FUSED_MAX_T", env)
    over = dict(d=256, E=64, f=128, fs=256) if cfg_id == 1 else dict(d=512, E=32, k=4, f=512, fs=512)
    L = synth.layer(cfg_id, **over)
    c = L["cfg"]
    x = synth.hidden(cfg_id, T, c["d"], c["act"], draw=70 + T)
    D = dev_layer(L)
    layer = make_layer_obj(c, 16)
    check_layer(layer, D, x, run_oracle(L, x), c)
    layer.profile_begin(KERNEL_FUSED, 4)
    run_gpu(layer, D, x, routing=False)
    assert (len(layer.profile_end()) == 1) == fused
    assert layer.fault() == 0
