#!/usr/bin/env python3
"""Benchmark of the Flint routed-expert MoE layer on one MI355X.

    python bench.py [--workload decode|fp4|prefill|stack|tiny|dense] [--steps K] [--warmup W]

Prints ONE JSON line.  A step is one forward of the whole layer (router +
top-k + permutation + experts + combine) over one batch of seeded synthetic
tokens, with inputs already resident in HBM.  Decode steps rotate through
several independently seeded layers (and a pool of token batches), as
consecutive layers of the model would, so no weight byte is served from the
256 MB last-level cache left warm by the previous step.

Besides the driver's fields the line carries:
  roofline      the dominant kernel's algorithmic bytes (or flops) per launch
                over its average duration, timed with HIP events on the
                forward's stream inside the timed region, against the MI355X
                peak; `traffic` is the HBM bytes per launch measured with
                rocprofv3 counters (profiles/*_traffic.json) when those were
                taken on the current kernel source, else null
  cpu_baseline  the fp64 CPU oracle on a bounded sample of the same workload
  t_sweep       every token count of the workload (decode/fp4)
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
# logical dominant kernel (gate/up + SwiGLU of the chosen path) -> its source
KERNEL_SRC = {
    "gateup_decode": "sparse_moe_transformer_gemv_amd/csrc/expert_decode.hip",
    "gateup_prefill": "sparse_moe_transformer_gemv_amd/csrc/expert_prefill.hip",
}

WORKLOADS = {
    # name: (config id, token counts (last = headline), distinct layers to rotate)
    "decode": (1, (1, 4, 16, 64), 8),
    "fp4": (4, (1, 16), 8),
    "prefill": (2, (4096,), 2),
    "stack": (3, (32,), 47),
    "tiny": (0, (64,), 1),
    # dense SwiGLU FFN (the model's first layers), width DENSE_F, on the same engine
    "dense": (1, (32, 4096), 2),
}
DENSE_F = 16384  # about 0.1B parameters per dense layer at d = 2048


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (reference for HBM counters)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def file_sha(path):
    with open(os.path.join(ROOT, path), "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def expert_bytes(c, F, parts=("gate_up", "down")):
    d = c["d"]
    per = 0
    for part in parts:
        n = 2 * F * d if part == "gate_up" else d * F
        if c["wdtype"] == 2:   # NVFP4: codes + E4M3 scales (+ 2 tensor scales, ignored)
            per += n // 2 + n // 16
        else:
            per += n * (4 if c["wdtype"] == 0 else 2)
    return per


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from synth.device import dev_layer, make_layer_obj, x_device
    import sparse_moe_transformer_gemv_amd as fm

    torch.cuda.set_device(0)
    cfg_id, Ts, n_layers = WORKLOADS[args.workload]
    c = dict(synth.CONFIGS[cfg_id])
    if args.workload == "stack":
        return bench_stack(args, c, cfg_id, Ts[0], n_layers)
    if args.workload == "dense":
        return bench_dense(args, c, cfg_id, Ts, n_layers)
    Tmax = max(Ts)

    t0 = time.time()
    layers = []
    host0 = None
    for l in range(n_layers):
        L = synth.layer(cfg_id, l)
        layers.append(dev_layer(L))
        if l == 0:
            host0 = L
        else:
            del L
    log("generated %d layer(s) in %.1fs" % (n_layers, time.time() - t0))
    n_x = 16
    xs = {T: [x_device(synth.hidden(cfg_id, T, c["d"], c["act"], draw=i)) for i in range(n_x)]
          for T in Ts}
    moe = make_layer_obj(c, Tmax)
    stream = torch.cuda.current_stream()

    def forward(T, i):
        D = layers[i % n_layers]
        return moe.forward(xs[T][i % n_x], D["router_w"], D["experts"], D["shared"],
                           D["router_bias"])

    def distinct_experts(T, i):
        forward(T, i)
        cnt = moe.routing()["counts"]
        return int((cnt > 0).sum().item())

    results = {}
    for T in Ts:
        steps, warm = args.steps, args.warmup
        nd = [distinct_experts(T, i) for i in range(steps)]
        for i in range(warm):
            forward(T, i)
        torch.cuda.synchronize()
        dominant = fm.KERNEL_EXPERT_UP
        moe.profile_begin(dominant, steps)
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(steps):
            forward(T, i)
        ev1.record(stream)
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / steps
        kms = moe.profile_end()
        f, fs, d, k = c["f"], c["fs"], c["d"], c["k"]
        act_b = 4 if c["act"] == 0 else 2
        up_flops = 2.0 * (k * T * f + T * fs) * d * 2
        # whole-layer algorithmic bytes: active expert weights + router + x + out
        layer_bytes = [(n * expert_bytes(c, f) + expert_bytes(c, fs)) + c["E"] * d * 4 +
                       2 * T * d * act_b for n in nd]
        # dominant kernel (gate/up + SwiGLU): active gate/up weights + x + h out (fp32)
        up_bytes = [n * expert_bytes(c, f, ("gate_up",)) + expert_bytes(c, fs, ("gate_up",)) +
                    T * d * act_b + (k * T * f + T * fs) * 4 for n in nd]
        results[T] = dict(
            ms=ms, tok_s=T / (ms * 1e-3),
            hbm_frac=float(np.mean(layer_bytes)) / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
            distinct=float(np.mean(nd)), layer_bytes=float(np.mean(layer_bytes)),
            up_us=float(np.mean(kms)) * 1e3, up_bytes=float(np.mean(up_bytes)),
            layer_flops=2.0 * (k * T * f + T * fs) * d * 3, up_flops=up_flops)
        results[T]["mfma_frac"] = results[T]["layer_flops"] / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12)
        log("T=%d: %.1f us/step, %.0f tok/s, %.1f%% HBM / %.1f%% MFMA (layer), dominant %.1f us" % (
            T, ms * 1e3, results[T]["tok_s"], 100 * results[T]["hbm_frac"],
            100 * results[T]["mfma_frac"], results[T]["up_us"]))

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB device-to-device copy done")

    H = results[Tmax]
    prefill = args.workload == "prefill"
    kname = "gateup_prefill" if prefill else "gateup_decode"
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "%s_%s_T%d_traffic.json" % (kname, args.workload, Tmax))
    if os.path.exists(tpath):
        with open(tpath) as fh:
            tr = json.load(fh)
        if tr.get("source_sha") == file_sha(KERNEL_SRC[kname]):
            traffic = tr.get("bytes_per_launch")
    if prefill:
        achieved = H["up_flops"] / (H["up_us"] * 1e-6) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                    "traffic": traffic, "kernel": kname, "flops_per_launch": H["up_flops"],
                    "us_per_launch": round(H["up_us"], 2)}
    else:
        achieved = H["up_bytes"] / (H["up_us"] * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "kernel": kname, "bytes_per_launch": int(H["up_bytes"]),
                    "us_per_launch": round(H["up_us"], 2)}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        x0 = synth.hidden(cfg_id, Tmax, c["d"], c["act"], draw=0)
        # bounded sample: batches of up to 64 tokens of the same workload
        sample = x0[:64]
        ntok = 0
        t1 = time.time()
        while True:
            oracle.moe_forward(sample, host0["router_w"], host0["experts"], host0["shared"],
                               top_k=c["k"], router_bias=host0["router_bias"],
                               wdtype=c["wdtype"])
            ntok += sample.shape[0]
            if time.time() - t1 >= args.cpu_seconds:
                break
        dt = time.time() - t1
        cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
        cpu = {"value": round(ntok / dt, 2), "unit": "tokens/s", "cores": cores,
               "kind": "oracle",
               "sample": "%d forwards of the first %d tokens of the same batch, layer 0, fp64" % (
                   ntok // sample.shape[0], sample.shape[0])}

    line = {
        "metric": "MoE-layer tokens/s",
        "value": round(H["tok_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(H["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {0: "f32", 1: "bf16", 2: "nvfp4"}[c["wdtype"]],
        "data": "synthetic",
        "config": {"workload": "%s T=%d (d=%d, E=%d, top-%d + shared, f=%d)" % (
            c["name"], Tmax, c["d"], c["E"], c["k"], c["f"]), "tokens": Tmax,
            "layers_rotated": n_layers, "hbm_frac_layer": round(H["hbm_frac"], 4),
            "mfma_frac_layer": round(H["mfma_frac"], 4), "distinct_experts": H["distinct"]},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "t_sweep": {str(T): {"tok_s": round(r["tok_s"], 1), "us": round(r["ms"] * 1e3, 2),
                             "hbm_frac_layer": round(r["hbm_frac"], 4),
                             "mfma_frac_layer": round(r["mfma_frac"], 4),
                             "dominant_us": round(r["up_us"], 2),
                             "distinct_experts": r["distinct"]} for T, r in results.items()},
    }
    print(json.dumps(line), flush=True)


def bench_dense(args, c, cfg_id, Ts, n_layers):
    """Dense SwiGLU FFN of width DENSE_F: out = D (SiLU(G x) * (U x)) for T tokens."""
    import numpy as np
    import torch

    import synth
    from synth.device import dev_weights, x_device
    import sparse_moe_transformer_gemv_amd as fm

    d, F, wd = c["d"], DENSE_F, c["wdtype"]
    t0 = time.time()
    hosts = [synth.expert_set(cfg_id, l, 1, d, F, wd) for l in range(n_layers)]
    ws = [dev_weights(h, wd) for h in hosts]
    log("generated %d dense layer(s) of width %d in %.1fs" % (n_layers, F, time.time() - t0))
    Tmax = max(Ts)
    ffn = fm.DenseFFN(d, F, c["act"], wd, max_tokens=Tmax)
    stream = torch.cuda.current_stream()
    n_x = 4
    results = {}
    for T in Ts:
        xs = [x_device(synth.hidden(cfg_id, T, d, c["act"], draw=i)) for i in range(n_x)]
        for i in range(args.warmup):
            ffn.forward(xs[i % n_x], ws[i % n_layers])
        torch.cuda.synchronize()
        ffn.layer.profile_begin(fm.KERNEL_EXPERT_UP, args.steps)
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for i in range(args.steps):
            ffn.forward(xs[i % n_x], ws[i % n_layers])
        ev1.record(stream)
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / args.steps
        up_us = float(np.mean(ffn.layer.profile_end())) * 1e3
        w_bytes = 3.0 * F * d * 2
        up_flops = 2.0 * T * 2 * F * d
        results[T] = dict(ms=ms, tok_s=T / (ms * 1e-3), up_us=up_us, up_flops=up_flops,
                          up_bytes=2.0 * F * d * 2 + T * d * 2 + T * F * 4,
                          hbm_frac=(w_bytes + 2 * T * d * 2) / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
                          mfma_frac=3 * up_flops / 2 / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12))
        log("T=%d: %.1f us/step, %.0f tok/s, %.1f%% HBM / %.1f%% MFMA (layer), gate/up %.1f us" % (
            T, ms * 1e3, results[T]["tok_s"], 100 * results[T]["hbm_frac"],
            100 * results[T]["mfma_frac"], up_us))
    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB device-to-device copy done")
    H = results[Tmax]
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "gateup_prefill_dense_T%d_traffic.json" % Tmax)
    if os.path.exists(tpath):
        with open(tpath) as fh:
            tr = json.load(fh)
        if tr.get("source_sha") == file_sha(KERNEL_SRC["gateup_prefill"]):
            traffic = tr.get("bytes_per_launch")
    achieved = H["up_flops"] / (H["up_us"] * 1e-6) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                "kernel": "gateup_prefill", "flops_per_launch": H["up_flops"],
                "us_per_launch": round(H["up_us"], 2)}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        sample = synth.hidden(cfg_id, 2, d, c["act"], draw=0)
        ntok = 0
        t1 = time.time()
        while True:
            oracle.ffn_forward(sample, hosts[0], wdtype=wd)
            ntok += sample.shape[0]
            if time.time() - t1 >= args.cpu_seconds:
                break
        dt = time.time() - t1
        cpu = {"value": round(ntok / dt, 2), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": "%d forwards of 2 tokens, layer 0, fp64" % (ntok // 2)}
    line = {
        "metric": "dense-FFN tokens/s", "value": round(H["tok_s"], 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(H["ms"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {0: "f32", 1: "bf16", 2: "nvfp4"}[wd], "data": "synthetic",
        "config": {"workload": "dense SwiGLU FFN T=%d (d=%d, f=%d)" % (Tmax, d, F), "tokens": Tmax,
                   "layers_rotated": n_layers, "hbm_frac_layer": round(H["hbm_frac"], 4),
                   "mfma_frac_layer": round(H["mfma_frac"], 4)},
        "roofline": roofline, "cpu_baseline": cpu,
        "t_sweep": {str(T): {"tok_s": round(r["tok_s"], 1), "us": round(r["ms"] * 1e3, 2),
                             "hbm_frac_layer": round(r["hbm_frac"], 4),
                             "mfma_frac_layer": round(r["mfma_frac"], 4),
                             "dominant_us": round(r["up_us"], 2)} for T, r in results.items()},
    }
    print(json.dumps(line), flush=True)


def bench_stack(args, c, cfg_id, T, n_layers):
    """47 resident layers, T tokens: h <- h + MoE_l(bf16(RMSNorm(h))) per layer.
    One step = the whole pass (rmsnorm + layer for every layer), captured once
    as a HIP graph and replayed."""
    import numpy as np
    import torch

    import synth
    from synth.device import dev_array, dev_layer, make_layer_obj
    import sparse_moe_transformer_gemv_amd as fm

    xbuf = torch.empty((T, c["d"]), dtype=torch.bfloat16, device="cuda")

    def stack_gpu(moe, h, layers):
        for D in layers:
            fm.flint_rmsnorm_forward(h, 1e-6, out=xbuf)
            moe.forward(xbuf, D["router_w"], D["experts"], D["shared"], None, residual=h, out=h)

    t0 = time.time()
    layers, nd = [], []
    host0 = None
    for l in range(n_layers):
        L = synth.layer(cfg_id, l)
        layers.append(dev_layer(L))
        if l == 0:
            host0 = L
        del L
    log("generated %d layer(s) in %.1fs" % (n_layers, time.time() - t0))
    h0 = dev_array(synth.hidden(cfg_id, T, c["d"], synth.F32))
    h = h0.clone()
    moe = make_layer_obj(c, T)
    # distinct experts per layer for this batch (eager pass with routing read-back)
    h.copy_(h0)
    from sparse_moe_transformer_gemv_amd import flint_rmsnorm_forward
    x = torch.empty((T, c["d"]), dtype=torch.bfloat16, device="cuda")
    for D in layers:
        flint_rmsnorm_forward(h, 1e-6, out=x)
        moe.forward(x, D["router_w"], D["experts"], D["shared"], None, residual=h, out=h)
        nd.append(int((moe.routing()["counts"] > 0).sum().item()))
    # dominant kernel timing: one eager pass with the event hook
    h.copy_(h0)
    torch.cuda.synchronize()
    moe.profile_begin(fm.KERNEL_EXPERT_UP, n_layers)
    stack_gpu(moe, h, layers)
    torch.cuda.synchronize()
    kms = moe.profile_end()
    # graph of one full pass
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for _ in range(2):
            h.copy_(h0)
            stack_gpu(moe, h, layers)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h.copy_(h0)
        stack_gpu(moe, h, layers)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    f, fs, d, k = c["f"], c["fs"], c["d"], c["k"]
    pass_bytes = sum(n * expert_bytes(c, f) + expert_bytes(c, fs) + c["E"] * d * 4 +
                     T * d * (2 + 4 + 4) for n in nd)
    up_bytes = float(np.mean([n * expert_bytes(c, f, ("gate_up",)) +
                              expert_bytes(c, fs, ("gate_up",)) + T * d * 2 +
                              (k * T * f + T * fs) * 4 for n in nd]))
    up_us = float(np.mean(kms)) * 1e3
    achieved = up_bytes / (up_us * 1e-6) / 1e9
    log("stack: %.3f ms/pass, %.0f tok/s, %.1f%% HBM, gate/up %.1f us" % (
        ms, T / (ms * 1e-3), 100 * pass_bytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), up_us))
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        # one layer's forward on the same T tokens stands for 1/47 of a pass
        xs = synth.hidden(cfg_id, T, d, c["act"], draw=0)
        t1 = time.time()
        n = 0
        while True:
            oracle.moe_forward(xs, host0["router_w"], host0["experts"], host0["shared"],
                               top_k=k, wdtype=c["wdtype"])
            n += 1
            if time.time() - t1 >= args.cpu_seconds:
                break
        per_layer = (time.time() - t1) / n
        cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
        cpu = {"value": round(T / (per_layer * n_layers), 3), "unit": "tokens/s", "cores": cores,
               "kind": "oracle",
               "sample": "%d single-layer forwards of T=%d (layer 0), scaled to %d layers" % (
                   n, T, n_layers)}
    line = {
        "metric": "MoE-layer tokens/s", "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s: %d layers x (RMSNorm + MoE + residual), T=%d" % (
            c["name"], n_layers, T), "tokens": T, "layers": n_layers,
            "hbm_frac_pass": round(pass_bytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
            "pass_bytes": int(pass_bytes), "graph": True},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "gateup_decode", "bytes_per_launch": int(up_bytes),
                     "us_per_launch": round(up_us, 2)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
