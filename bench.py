#!/usr/bin/env python3
"""Benchmark of the Flint routed-expert MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all|decode|prefill|stack|nvfp4|tiny|dense]

Prints ONE JSON line.  A step is one forward of the whole layer (router, top-k,
permutation, experts, combine) over one batch of seeded synthetic tokens, with
every input already resident in HBM; for the 47-layer stack a step is the
whole pass.  The headline (`value`) is the bf16 decode layer at T = 64 tokens;
the line also carries every workload of the five configurations under
`workloads`:
  tiny     fp32 layer, d = 128, f = 32, T = 64 (correctness scale)
  decode   bf16 layer, d = 2048, 256 experts, top-6 + shared, f = 512, T = 1, 4, 16, 64
  prefill  the same layer at T = 4096 with the Zipf router bias
  stack    47 such layers (76 GB resident), pre-RMSNorm and fp32 residual, T = 32
  nvfp4    the layer with NVFP4 expert weights, T = 1, 16
  nvfp4_prefill  the NVFP4 layer at T = 4096 with the Zipf router bias
Decode steps rotate through several independently seeded layers and 16 token
batches, as consecutive layers of a model would, so weights come from HBM and
not from the 256 MB last-level cache.  The stack's pass is one HIP graph,
replayed once per step.

Per workload and token count:
  us          mean = the timed region (K eager steps between two HIP events) / K;
              median, min, p90 of the per-forward times (events the library
              records before a forward's first launch and after its last, on
              its stream) over K more steps; the stack: per replayed pass
  layer_frac  algorithmic bytes (decode) or bf16 flops (prefill) of the whole
              layer per step over the step time, against the HBM (8 TB/s) or
              dense bf16 MFMA (2.5 PFLOP/s) peak
  roofline    the dominant kernel: its algorithmic bytes (or flops) per launch
              over its mean launch time, timed with HIP events on the forward's
              stream over K eager steps after the timed region; `traffic` is
              its HBM bytes per
              launch from rocprofv3 counters (profiles/*_traffic.json) when
              they were taken on the current kernel source, else null
  cpu_baseline the fp64 CPU oracle on a bounded sample of the same workload,
              with the thread count and CPU model
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; % peak HBM BW (decode), % MFMA peak (prefill)"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, TFLOP/s
CSRC = "sparse_moe_transformer_gemv_amd/csrc/"
# dominant kernel -> the source it is built from (for the counter-traffic sha)
KERNEL_SRC = {"gateup_decode": CSRC + "expert_decode.hip", "decode_fused": CSRC + "expert_decode.hip",
              "gateup_prefill": CSRC + "expert_prefill.hip"}
DENSE_F = 16384  # width of the dense SwiGLU layer workload (about 0.1B parameters at d = 2048)
ALL = ("decode", "prefill", "stack", "nvfp4", "tiny", "nvfp4_prefill")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all", choices=("all",) + ALL + ("dense",))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU time of the headline oracle sample (the other workloads get half)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (reference for HBM counters)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def file_sha(path):
    with open(os.path.join(ROOT, path), "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def cpu_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    return model, threads


def expert_bytes(c, F, parts=("gate_up", "down")):
    d, per = c["d"], 0
    for part in parts:
        n = 2 * F * d if part == "gate_up" else d * F
        if c["wdtype"] == 2:   # NVFP4: codes + E4M3 scales (tensor scales: 12 B, ignored)
            per += n // 2 + n // 16
        else:
            per += n * (4 if c["wdtype"] == 0 else 2)
    return per


def layer_bytes(c, T, distinct, out_bytes=None):
    """Bytes the layer must move: active experts (+ shared), router, x, out."""
    act = 4 if c["act"] == 0 else 2
    return (distinct * expert_bytes(c, c["f"]) + expert_bytes(c, c["fs"]) + c["E"] * c["d"] * 4 +
            T * c["d"] * act + T * c["d"] * (out_bytes or act))


def gateup_bytes(c, T, distinct):
    """Dominant decode kernel: active gate/up weights, x, and h (fp32 values)."""
    act = 4 if c["act"] == 0 else 2
    return (distinct * expert_bytes(c, c["f"], ("gate_up",)) + expert_bytes(c, c["fs"], ("gate_up",)) +
            T * c["d"] * act + (c["k"] * T * c["f"] + T * c["fs"]) * 4)


def layer_flops(c, T):
    return 2.0 * (c["k"] * T * c["f"] + T * c["fs"]) * c["d"] * 3


def step_stats(per_ms, total_ms, steps):
    import numpy as np
    a = np.asarray(per_ms) * 1e3
    return {"mean": round(total_ms * 1e3 / steps, 2), "median": round(float(np.median(a)), 2),
            "min": round(float(a.min()), 2), "p90": round(float(np.percentile(a, 90)), 2)}


def timed_steps(fn, steps, warmup, stream, per_step=True):
    """W untimed steps, then K steps between two HIP events (and, with per_step,
    an event after each), synchronised before and after; returns (total ms,
    per-step ms or None)."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1 if per_step else 2)]
    ev[0].record(stream)
    for i in range(steps):
        fn(i)
        if per_step:
            ev[i + 1].record(stream)
    if not per_step:
        ev[1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)] if per_step else None
    return ev[0].elapsed_time(ev[-1]), per


def traffic_for(kname, workload, T):
    path = os.path.join(ROOT, "profiles", "%s_%s_T%d_traffic.json" % (kname, workload, T))
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        tr = json.load(fh)
    return tr.get("bytes_per_launch") if tr.get("source_sha") == file_sha(KERNEL_SRC[kname]) else None


def hbm_roofline(kname, nbytes, us, traffic):
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kname,
            "bytes_per_launch": int(nbytes), "us_per_launch": round(us, 2)}


def mfma_roofline(kname, flops, us, traffic):
    tf = flops / (us * 1e-6) / 1e12
    return {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / BF16_PEAK_TFLOPS, 4), "traffic": traffic, "kernel": kname,
            "flops_per_launch": flops, "us_per_launch": round(us, 2)}


def cpu_baseline(run_once, tokens_per_call, seconds, sample, scale=1.0):
    """The oracle (as it stands) on a bounded sample: repeated calls for about
    `seconds`; tokens/s, divided by `scale` (layers per pass for the stack)."""
    model, threads = cpu_info()
    n = 0
    t0 = time.time()
    while True:
        run_once()
        n += 1
        if time.time() - t0 >= seconds:
            break
    dt = time.time() - t0
    return {"value": round(n * tokens_per_call / dt / scale, 3), "unit": "tokens/s", "cores": threads,
            "cpu_model": model, "kind": "oracle", "sample": sample % n}


# ----------------------------------------------------------------- workloads

def run_layer_workload(name, cfg_id, Ts, n_layers, args, cpu_seconds, **override):
    """One forward of one layer per step (decode, nvfp4, tiny, prefill)."""
    import numpy as np
    import torch

    import synth
    from synth.device import dev_layer, make_layer_obj, x_device
    import sparse_moe_transformer_gemv_amd as fm

    c = dict(synth.CONFIGS[cfg_id], **override)
    t0 = time.time()
    layers, host0 = [], None
    for l in range(n_layers):
        L = synth.layer(cfg_id, l, **override)
        layers.append(dev_layer(L))
        if l == 0:
            host0 = L
    log("%s: generated %d layer(s) in %.1fs" % (name, n_layers, time.time() - t0))
    Tmax = max(Ts)
    n_x = 16 if Tmax <= 64 else 2
    moe = make_layer_obj(c, Tmax)
    stream = torch.cuda.current_stream()
    prefill = max(Ts) > 64
    sweep = {}
    for T in Ts:
        xs = [x_device(synth.hidden(cfg_id, T, c["d"], c["act"], draw=i)) for i in range(n_x)]

        def fwd(i, xs=xs):
            D = layers[i % n_layers]
            return moe.forward(xs[i % n_x], D["router_w"], D["experts"], D["shared"], D["router_bias"])

        # distinct experts each timed step selects (read back outside the timed region)
        nd = []
        for i in range(args.steps):
            fwd(i)
            nd.append(int((moe.routing()["counts"] > 0).sum().item()))
        # the dominant kernel: the single-launch decode where it runs, else gate/up
        moe.profile_begin(fm.KERNEL_FUSED, 1)
        fwd(0)
        fused = len(moe.profile_end()) == 1
        # timed region: K eager steps between two events (per-step events would
        # make the host's launch loop, not the GPU, the limit at small T)
        total, _ = timed_steps(fwd, args.steps, args.warmup, stream, per_step=False)
        ms = total / args.steps
        # per-forward times (first launch to last, events recorded by the library
        # on the forward's stream) and the dominant kernel's launches, each over
        # K more eager steps
        moe.profile_begin(fm.KERNEL_FORWARD, args.steps)
        for i in range(args.steps):
            fwd(i)
        torch.cuda.synchronize()
        per = moe.profile_end()
        moe.profile_begin(fm.KERNEL_FUSED if fused else fm.KERNEL_EXPERT_UP, args.steps)
        for i in range(args.steps):
            fwd(i)
        torch.cuda.synchronize()
        kus = float(np.mean(moe.profile_end())) * 1e3
        lb = float(np.mean([layer_bytes(c, T, n) for n in nd]))
        rec = {"tok_s": round(T / (ms * 1e-3), 1), "us": step_stats(per, total, args.steps),
               "distinct_experts": float(np.mean(nd))}
        if prefill:
            fl = layer_flops(c, T)
            rec["layer_frac"] = {"bound": "mfma", "frac": round(fl / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4),
                                 "flops": fl}
            upf = 2.0 * (c["k"] * T * c["f"] + T * c["fs"]) * c["d"] * 2
            rec["roofline"] = mfma_roofline("gateup_prefill", upf, kus, traffic_for("gateup_prefill", name, T))
        else:
            rec["layer_frac"] = {"bound": "hbm", "frac": round(lb / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                                 "bytes": int(lb)}
            if fused:
                rec["roofline"] = hbm_roofline("decode_fused", lb, kus, traffic_for("decode_fused", name, T))
            else:
                gb = float(np.mean([gateup_bytes(c, T, n) for n in nd]))
                rec["roofline"] = hbm_roofline("gateup_decode", gb, kus, traffic_for("gateup_decode", name, T))
        sweep[T] = rec
        log("%s T=%d: %.1f us/step (median %.1f, p90 %.1f), %.0f tok/s, layer %.1f%% of %s peak, %s %.1f us" % (
            name, T, ms * 1e3, rec["us"]["median"], rec["us"]["p90"], rec["tok_s"],
            100 * rec["layer_frac"]["frac"], rec["layer_frac"]["bound"], rec["roofline"]["kernel"], kus))
    out = {"config": "%s (d=%d, E=%d, top-%d + shared, f=%d, %s weights%s)" % (
        name, c["d"], c["E"], c["k"], c["f"], {0: "fp32", 1: "bf16", 2: "NVFP4"}[c["wdtype"]],
        ", Zipf router bias" if c["bias"] else ""), "layers_rotated": n_layers,
        "t_sweep": {str(T): r for T, r in sweep.items()}}
    if not args.no_cpu_baseline:
        import oracle
        tc = min(Tmax, 64)
        xh = synth.hidden(cfg_id, Tmax, c["d"], c["act"], draw=0)[:tc]
        out["cpu_baseline"] = cpu_baseline(
            lambda: oracle.moe_forward(xh, host0["router_w"], host0["experts"], host0["shared"],
                                       top_k=c["k"], router_bias=host0["router_bias"], wdtype=c["wdtype"]),
            tc, cpu_seconds, "%%d fp64 oracle forwards of the first %d tokens of the T=%d batch, layer 0" % (
                tc, Tmax))
    del layers, moe
    torch.cuda.empty_cache()
    return out, sweep


def run_stack(args, cpu_seconds):
    """47 resident layers, T = 32: h <- h + MoE_l(bf16(RMSNorm(h))) per layer; one
    step is the whole pass, captured once as a HIP graph and replayed."""
    import numpy as np
    import torch

    import synth
    from synth.device import dev_array, dev_layer, make_layer_obj
    import sparse_moe_transformer_gemv_amd as fm

    cfg_id, T = 3, 32
    c = dict(synth.CONFIGS[cfg_id])
    n_layers = c["layers"]
    t0 = time.time()
    layers, host0 = [], None
    for l in range(n_layers):
        L = synth.layer(cfg_id, l)
        layers.append(dev_layer(L))
        if l == 0:
            host0 = L
    log("stack: generated %d layers in %.1fs" % (n_layers, time.time() - t0))
    h0 = dev_array(synth.hidden(cfg_id, T, c["d"], synth.F32))
    h = h0.clone()
    moe = make_layer_obj(c, T)
    xbufs = [torch.empty((T, c["d"]), dtype=torch.bfloat16, device="cuda") for _ in range(2)]

    def one_pass(record=False):
        # the first pre-norm by the RMSNorm kernel; each layer's own launches
        # then produce the next layer's pre-norm with its output
        nd = []
        fm.flint_rmsnorm_forward(h, 1e-6, out=xbufs[0])
        for l, D in enumerate(layers):
            moe.forward_prenorm(xbufs[l & 1], D["router_w"], D["experts"], D["shared"], residual=h, eps=1e-6,
                                out=h, norm_out=xbufs[(l + 1) & 1])
            if record:
                nd.append(int((moe.routing()["counts"] > 0).sum().item()))
        return nd

    h.copy_(h0)
    nd = one_pass(record=True)  # distinct experts per layer (read back, untimed)
    # the gate/up kernel time from one eager pass with the event hook
    h.copy_(h0)
    torch.cuda.synchronize()
    moe.profile_begin(fm.KERNEL_EXPERT_UP, n_layers)
    one_pass()
    torch.cuda.synchronize()
    kus = float(np.mean(moe.profile_end())) * 1e3
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            h.copy_(h0)
            one_pass()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h.copy_(h0)
        one_pass()
    total, per = timed_steps(lambda i: g.replay(), args.steps, args.warmup, torch.cuda.current_stream())
    ms = total / args.steps
    pass_bytes = sum(layer_bytes(c, T, n, out_bytes=4) + T * c["d"] * (4 + 2) for n in nd)
    gb = float(np.mean([gateup_bytes(c, T, n) for n in nd]))
    rec = {"config": "%d x (RMSNorm + MoE layer + fp32 residual), graph-replayed pass (d=%d, E=%d, top-%d + "
                     "shared, f=%d, bf16)" % (n_layers, c["d"], c["E"], c["k"], c["f"]),
           "tokens": T, "tok_s": round(T / (ms * 1e-3), 1), "us": step_stats(per, total, args.steps),
           "distinct_experts_per_layer": float(np.mean(nd)),
           "layer_frac": {"bound": "hbm", "frac": round(pass_bytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                          "bytes": int(pass_bytes)},
           "roofline": hbm_roofline("gateup_decode", gb, kus, traffic_for("gateup_decode", "stack", T))}
    log("stack: %.3f ms/pass (median %.3f), %.0f tok/s, %.1f%% HBM per pass, gate/up %.1f us" % (
        ms, rec["us"]["median"] / 1e3, rec["tok_s"], 100 * rec["layer_frac"]["frac"], kus))
    if not args.no_cpu_baseline:
        import oracle
        xs = synth.hidden(cfg_id, T, c["d"], c["act"], draw=0)
        rec["cpu_baseline"] = cpu_baseline(
            lambda: oracle.moe_forward(xs, host0["router_w"], host0["experts"], host0["shared"], top_k=c["k"],
                                       wdtype=c["wdtype"]),
            T, cpu_seconds, "%%d fp64 oracle forwards of one layer at T=%d, scaled to %d layers" % (T, n_layers),
            scale=n_layers)
    del layers, g, moe
    torch.cuda.empty_cache()
    return rec


def run_dense(args, cpu_seconds):
    """Dense SwiGLU FFN of width DENSE_F (the model's dense layers), T = 32 and 4096."""
    import numpy as np
    import torch

    import synth
    from synth.device import dev_weights, x_device
    import sparse_moe_transformer_gemv_amd as fm

    cfg_id = 1
    c = dict(synth.CONFIGS[cfg_id])
    d, F, wd = c["d"], DENSE_F, c["wdtype"]
    hosts = [synth.expert_set(cfg_id, l, 1, d, F, wd) for l in range(2)]
    ws = [dev_weights(h_, wd) for h_ in hosts]
    Ts = (32, 4096)
    ffn = fm.DenseFFN(d, F, c["act"], wd, max_tokens=max(Ts))
    stream = torch.cuda.current_stream()
    sweep = {}
    for T in Ts:
        xs = [x_device(synth.hidden(cfg_id, T, d, c["act"], draw=i)) for i in range(4)]
        ffn.layer.profile_begin(fm.KERNEL_EXPERT_UP, args.steps)
        total, per = timed_steps(lambda i: ffn.forward(xs[i % 4], ws[i % 2]), args.steps, args.warmup, stream)
        kus = float(np.mean(ffn.layer.profile_end())) * 1e3
        ms = total / args.steps
        fl = 2.0 * T * 3 * F * d
        wb = 3.0 * F * d * 2 + 2 * T * d * 2
        rec = {"tok_s": round(T / (ms * 1e-3), 1), "us": step_stats(per, total, args.steps),
               "layer_frac": {"hbm": round(wb / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                              "mfma": round(fl / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4)}}
        if T > 64:
            rec["roofline"] = mfma_roofline("gateup_prefill", 2.0 * T * 2 * F * d, kus,
                                            traffic_for("gateup_prefill", "dense", T))
        else:
            rec["roofline"] = hbm_roofline("gateup_decode", 2.0 * F * d * 2 + T * d * 2 + T * F * 4, kus, None)
        sweep[str(T)] = rec
        log("dense T=%d: %.1f us/step, %.0f tok/s" % (T, ms * 1e3, rec["tok_s"]))
    out = {"config": "dense SwiGLU FFN (d=%d, f=%d, bf16)" % (d, F), "t_sweep": sweep}
    if not args.no_cpu_baseline:
        import oracle
        xh = synth.hidden(cfg_id, 2, d, c["act"], draw=0)
        out["cpu_baseline"] = cpu_baseline(lambda: oracle.ffn_forward(xh, hosts[0], wdtype=wd), 2,
                                           cpu_seconds, "%d fp64 oracle forwards of 2 tokens")
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus %d requested)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    half = args.cpu_seconds / 2
    todo = ALL if args.workload == "all" else (args.workload,)
    work, headline = {}, None
    t_start = time.time()
    for name in todo:
        if name == "stack":
            rec = run_stack(args, half)
            cand = ("stack", 32, rec, rec)
        elif name == "dense":
            rec = run_dense(args, half)
            cand = ("dense", 4096, rec["t_sweep"]["4096"], rec)
        else:
            cfg_id, Ts, n_layers = {"decode": (1, (1, 4, 16, 64), 8), "nvfp4": (4, (1, 16), 8),
                                    "tiny": (0, (64,), 1), "prefill": (2, (4096,), 2),
                                    "nvfp4_prefill": (4, (4096,), 2)}[name]
            over = {"bias": True} if name == "nvfp4_prefill" else {}
            rec, sweep = run_layer_workload(name, cfg_id, Ts, n_layers, args,
                                            args.cpu_seconds if name == "decode" else half, **over)
            cand = (name, max(Ts), sweep[max(Ts)], rec)
        work[name] = rec
        if headline is None or name == "decode":
            headline = cand
    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB device-to-device copy done")
    wname, T, H, R = headline
    line = {
        "metric": METRIC, "value": H["tok_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(H["us"]["mean"] / 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "nvfp4" if wname == "nvfp4" else "bf16",
        "data": "synthetic", "config": {"workload": "%s T=%d: %s" % (wname, T, R["config"]), "tokens": T},
        "roofline": H["roofline"], "cpu_baseline": R.get("cpu_baseline"),
        "layer_frac": H["layer_frac"], "step_us": H["us"], "workloads": work,
        "wall_s": round(time.time() - t_start, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
