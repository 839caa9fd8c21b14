"""GPU parity: the HIP layer (through the C ABI) against the fp64 oracle.

Reduced shapes span several work items with ragged tails; the full-size
cases are the workloads the benchmark times, compared on every token (decode)
or on sampled tokens (prefill).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import (check_permutation, compare, dev_array, dev_layer, make_layer_obj,
                         out_host, run_gpu, run_oracle, x_device)
from sparse_moe_transformer_gemv_amd import (FLINT_FORCE_DECODE_PATH, FLINT_FORCE_PREFILL_PATH,
                                             FlintError)

pytestmark = pytest.mark.gpu


def _case(cfg_id, T, max_tokens=None, flags=0, draw=0, **override):
    L = synth.layer(cfg_id, **override)
    c = L["cfg"]
    x = synth.hidden(cfg_id, T, c["d"], c["act"], draw=draw)
    layer = make_layer_obj(c, max_tokens or T, flags)
    D = dev_layer(L)
    out, rout = run_gpu(layer, D, x)
    ref = run_oracle(L, x)
    rep = compare(out, rout, ref, c["k"], c["wdtype"], out_bf16=c["act"] == synth.BF16)
    check_permutation(rout, T, c["k"], c["E"])
    print("case cfg=%d T=%d %s -> %s" % (cfg_id, T, override, rep), flush=True)
    return L, x, layer, D, out, rout, ref


def test_tiny_f32_workload():
    _case(0, 64)


@pytest.mark.parametrize("T", [1, 3, 17, 64])
def test_small_bf16_decode(T):
    _case(1, T, d=256, E=64, f=64, fs=96)


@pytest.mark.parametrize("T", [1, 5, 40])
def test_small_nvfp4_decode(T):
    _case(4, T, d=256, E=32, k=4, f=64, fs=64)


@pytest.mark.parametrize("T", [1, 9, 16, 23, 64, 150])
def test_small_nvfp4_matrix_core_path(T):
    # d, f, fs multiples of 512 select the NVFP4 matrix-core expert kernels;
    # the shared expert has more features than a routed one; NVFP4 layers
    # always take the decode path, so T = 150 runs it above 64 tokens
    _case(4, T, d=512, E=32, k=4, f=512, fs=1024)


@pytest.mark.parametrize("T", [5, 19])
def test_nvfp4_matrix_core_path_d1024_ragged_f(T):
    # f = 1536: three 128-groups per wave in the down kernel
    _case(4, T, d=1024, E=16, k=3, f=1536, fs=512)


@pytest.mark.parametrize("T", [1, 7, 40, 64])
def test_small_bf16_matrix_core_path(T):
    # d % 128 == 0 and f, fs % 128 == 0 select the MFMA router and expert kernels
    _case(1, T, d=256, E=64, f=128, fs=256)


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


def test_f32_activations_bf16_weights():
    _case(1, 9, d=192, E=48, f=32, fs=64, act=synth.F32)


def test_no_shared_expert():
    L = synth.layer(1, d=128, E=16, f=32, fs=32)
    L["shared"] = None
    c = dict(L["cfg"], fs=0)
    L["cfg"] = c
    x = synth.hidden(1, 7, 128, synth.BF16)
    layer = make_layer_obj(c, 8)
    out, rout = run_gpu(layer, dev_layer(L), x)
    ref = oracle.moe_forward(x, L["router_w"], L["experts"], None, top_k=c["k"],
                             wdtype=synth.BF16)
    compare(out, rout, ref, c["k"], synth.BF16, out_bf16=True)


def test_no_shared_expert_decode_then_prefill_same_handle():
    # the prefill forward must not pick up rows an earlier decode forward left in
    # the shared slots' place (there is no shared expert to write them)
    L = synth.layer(1, d=256, E=32, f=128, fs=128)
    L["shared"] = None
    c = dict(L["cfg"], fs=0)
    L["cfg"] = c
    layer = make_layer_obj(c, 256)
    D = dev_layer(L)
    # decode at T=64 writes fp32 rows over the bytes where the T=100 prefill
    # forward's (bf16) shared-slot rows would sit
    for T in (64, 100):
        x = synth.hidden(1, T, 256, synth.BF16, draw=T)
        out, rout = run_gpu(layer, D, x)
        ref = oracle.moe_forward(x, L["router_w"], L["experts"], None, top_k=c["k"], wdtype=synth.BF16)
        rep = compare(out, rout, ref, c["k"], synth.BF16, out_bf16=True)
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
    out, rout = run_gpu(layer, dev_layer(L), x)
    assert np.array_equal(rout["idx"], np.tile(np.array(chosen), (T, 1)))
    ref = run_oracle(L, x)
    rep = compare(out, rout, ref, c["k"], c["wdtype"], out_bf16=True)
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
    compare(out, rout, ref, c["k"], synth.BF16, out_bf16=False)
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
    out, rout = run_gpu(layer, D, x)
    ref = run_oracle(L, x)
    rep = compare(out, rout, ref, c["k"], c["wdtype"], out_bf16=True)
    check_permutation(rout, T, c["k"], c["E"])
    # the same layer with an fp32 output (zero fp32 residual): the plain bound
    zero = torch.zeros((T, c["d"]), dtype=torch.float32, device="cuda")
    out32, rout32 = run_gpu(layer, D, x, residual=zero)
    rep32 = compare(out32, rout32, ref, c["k"], c["wdtype"], out_bf16=False)
    print("decode bf16 T=%d: %s | fp32 out: %s" % (T, rep, rep32), flush=True)


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
    out, rout = run_gpu(layer, D, x)
    ref = run_oracle(L, x)
    rep = compare(out, rout, ref, c["k"], c["wdtype"], out_bf16=True)
    zero = torch.zeros((T, c["d"]), dtype=torch.float32, device="cuda")
    out32, rout32 = run_gpu(layer, D, x, residual=zero)
    rep32 = compare(out32, rout32, ref, c["k"], c["wdtype"], out_bf16=False)
    print("decode nvfp4 T=%d: %s | fp32 out: %s" % (T, rep, rep32), flush=True)


@pytest.mark.parametrize("which,T", [("bf16", 4), ("nvfp4", 1)])
def test_decode_combine_in_down_with_residual(decode_layer, fp4_layer, which, T):
    # small batches fold the combine into the down kernel; a nonzero residual
    # is added there, also when the output aliases it
    L, D = decode_layer if which == "bf16" else fp4_layer
    c = L["cfg"]
    cfg_id = 1 if which == "bf16" else 4
    x = synth.hidden(cfg_id, T, c["d"], c["act"])
    res = np.random.default_rng(11).standard_normal((T, c["d"])).astype(np.float32)
    layer = make_layer_obj(c, 16)
    rd = dev_array(res)
    out, rout = run_gpu(layer, D, x, residual=rd)
    ref = run_oracle(L, x)
    ref = dict(ref, out=ref["out"] + res.astype(np.float64))
    rep = compare(out, rout, ref, c["k"], c["wdtype"], out_bf16=False)
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


def test_full_prefill_zipf_sampled(prefill_layer):
    L, D = prefill_layer
    c = L["cfg"]
    T = 4096
    x = synth.hidden(2, T, c["d"], c["act"])
    layer = make_layer_obj(c, T)
    out, rout = run_gpu(layer, D, x)
    check_permutation(rout, T, c["k"], c["E"])
    counts = rout["counts"]
    # sample tokens: spread over the batch, plus tokens of the largest and of
    # the smallest non-empty expert groups (ragged tiles)
    rng = np.random.default_rng(7)
    pick = set(rng.choice(T, 40, replace=False).tolist())
    big, small = int(np.argmax(counts)), int(np.argmin(np.where(counts > 0, counts, 1 << 30)))
    for e in (big, small):
        pick.update(np.where((rout["idx"] == e).any(1))[0][:4].tolist())
    pick = np.array(sorted(pick))
    ref = run_oracle(L, x[pick])
    sub = {"idx": rout["idx"][pick], "weights": rout["weights"][pick]}
    rep = compare(out[pick], sub, ref, c["k"], c["wdtype"], out_bf16=True)
    print("prefill T=4096 sampled %d tokens: %s, groups used %d, largest %d" % (
        len(pick), rep, int((counts > 0).sum()), int(counts.max())), flush=True)


def _stack_case(n_layers, T, tokens=None, min_compared=1, **override):
    cfg = 3
    Ls = [synth.layer(cfg, l, **override) for l in range(n_layers)]
    c = Ls[0]["cfg"]
    h0 = synth.hidden(cfg, T, c["d"], synth.F32)
    moe = make_layer_obj(c, T)
    from gpu_helpers import stack_compare, stack_gpu
    h = dev_array(h0.copy())
    rec = stack_gpu(moe, h, [dev_layer(L) for L in Ls], record=True)
    torch.cuda.synchronize()
    hg = out_host(h)
    pick = np.arange(T) if tokens is None else np.asarray(tokens)
    href, trace = oracle.stack_forward(h0[pick].astype(np.float64), Ls, top_k=c["k"])
    rec = [{"idx": r["idx"][pick], "logits": r["logits"][pick]} for r in rec]
    rep = stack_compare(hg[pick], href, trace, rec, c["k"])
    print("stack %d layers T=%d %s -> %s" % (n_layers, T, override, rep), flush=True)
    # every flip was checked above; enough tokens must stay flip-free to compare
    assert rep["compared_tokens"] >= min_compared


def test_stack_47_layers_small_shape():
    _stack_case(47, 32, min_compared=16, d=256, E=64, f=128, fs=128)


def test_stack_47_layers_full_size_sampled():
    # full-size layers (76 GB resident); the oracle follows 8 of the 32 tokens
    _stack_case(47, 32, tokens=[0, 5, 9, 14, 20, 23, 27, 31])


@pytest.mark.parametrize("layer_idx", [0, 23, 46])
def test_stack_layer_alone_full_size(layer_idx):
    # every resident layer of the stacked workload meets the single-layer bound
    # on its own seeded input (T = 32, fp32 output)
    L = synth.layer(3, layer_idx)
    c = L["cfg"]
    x = synth.hidden(3, 32, c["d"], c["act"], draw=100 + layer_idx)
    layer = make_layer_obj(c, 32)
    D = dev_layer(L)
    zero = torch.zeros((32, c["d"]), dtype=torch.float32, device="cuda")
    out, rout = run_gpu(layer, D, x, residual=zero)
    rep = compare(out, rout, run_oracle(L, x), c["k"], c["wdtype"], out_bf16=False)
    print("stack layer %d alone: %s" % (layer_idx, rep), flush=True)


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
    from gpu_helpers import TOL, dev_weights, half_ulp_bf16
    wd = synth.CONFIGS[cfg_id]["wdtype"]
    act = synth.CONFIGS[cfg_id]["act"]
    ws = synth.expert_set(cfg_id, 0, 1, d, F, wd)
    x = synth.hidden(cfg_id, T, d, act)
    ffn = DenseFFN(d, F, act, wd, max_tokens=max(T, 64), flags=flags)
    out = out_host(ffn.forward(x_device(x), dev_weights(ws, wd)))
    torch.cuda.synchronize()
    rows = np.arange(T) if T <= 64 else np.random.default_rng(5).choice(T, 24, replace=False)
    ref = oracle.ffn_forward(x[rows], ws, wdtype=wd)
    err = np.abs(out[rows] - ref)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    assert np.all(err <= TOL[wd] * rms + half_ulp_bf16(ref)), "max|err| %.3e vs %.1e * RMS %.3e" % (
        err.max(), TOL[wd], rms)
    # the fp32-output form (zero residual) meets the plain bound
    zero = torch.zeros((T, d), dtype=torch.float32, device="cuda")
    out32 = out_host(ffn.forward(x_device(x), dev_weights(ws, wd), residual=zero))
    torch.cuda.synchronize()
    err32 = np.abs(out32[rows] - ref)
    assert err32.max() <= TOL[wd] * rms, "fp32 out: max|err| %.3e vs %.1e * RMS %.3e" % (
        err32.max(), TOL[wd], rms)
    print("dense FFN cfg %d d=%d F=%d T=%d: max|err| %.2e (bf16 out), %.2e (fp32 out), RMS %.3e" % (
        cfg_id, d, F, T, err.max(), err32.max(), rms), flush=True)


@pytest.mark.parametrize("T", [3, 40])
def test_wide_shared_expert_splits_k(T):
    # a shared expert wider than one K chunk of the decode down kernel: only its
    # group is split (two chunks), the routed groups are not
    _case(1, T, d=256, E=64, f=128, fs=2048)


@pytest.mark.parametrize("T", [3, 20])
def test_wide_nvfp4_shared_expert_splits_k(T):
    # an NVFP4 shared expert twice as wide as one K chunk of the NVFP4 down kernel
    _case(4, T, d=512, E=64, f=512, fs=4096)
