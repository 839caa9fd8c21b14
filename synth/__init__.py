"""Seeded synthetic inputs for the Flint MoE layer (shared by tests, smoke and bench).

This module draws random tensors and stores them in the formats the layer
consumes; it holds none of the layer's arithmetic.  Every tensor comes from
its own ``numpy`` PCG64 stream keyed by ``(SEED_BASE, config id, layer,
tensor id, expert or draw index)``, so any single expert of any layer can be
regenerated on its own, bit for bit.

Distributions (the five workloads, by configuration id):
  x ~ N(0, 1); router rows ~ N(0, 1/d); gate/up rows ~ N(0, 1/d);
  down rows ~ N(0, 1/f).  Values are drawn as float32 and, for bf16 tensors,
  rounded to the nearest bf16 (ties to even).  The prefill workload adds the
  router bias b_e = 1.5 * ln(1 / (e + 1)^1.1) (Zipf-skewed expert
  popularity).  NVFP4 weights are uniform E2M1 codes (all 16, -0 included),
  one E4M3 block scale per 16 elements along K drawn uniformly from the codes
  0x28..0x40 (0.25 to 2.0), and an fp32 per-tensor scale 1/sqrt(K).

Stored formats: fp32 as ``np.float32``; bf16 as raw bits ``np.uint16``;
NVFP4 as packed codes ``np.uint8`` [rows][K/2] (even k in the low nibble),
E4M3 scale codes ``np.uint8`` [rows][K/16], tensor scales ``np.float32``
[n][3] = {gate, up, down}.
Weight layouts: gate_up [n][2f][d] (gate rows 0..f-1, up rows f..2f-1);
down [n][d][f]; router [E][d].
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SEED_BASE = 20261021

F32, BF16, NVFP4 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", BF16: "bf16", NVFP4: "nvfp4"}

# tensor ids inside a layer's seed key
_T_X, _T_ROUTER, _T_GATE_UP, _T_DOWN, _T_SGATE_UP, _T_SDOWN = 0, 1, 2, 3, 4, 5
_T_GU_SCALE, _T_DN_SCALE, _T_SGU_SCALE, _T_SDN_SCALE = 6, 7, 8, 9

# The five workloads.
CONFIGS = {
    0: dict(name="tiny_f32", d=128, E=256, k=6, f=32, fs=32, act=F32, wdtype=F32,
            T=(64,), bias=False, layers=1),
    1: dict(name="decode_bf16", d=2048, E=256, k=6, f=512, fs=512, act=BF16, wdtype=BF16,
            T=(1, 4, 16, 64), bias=False, layers=1),
    2: dict(name="prefill_bf16_zipf", d=2048, E=256, k=6, f=512, fs=512, act=BF16,
            wdtype=BF16, T=(4096,), bias=True, layers=1),
    3: dict(name="stack47_decode_bf16", d=2048, E=256, k=6, f=512, fs=512, act=BF16,
            wdtype=BF16, T=(32,), bias=False, layers=47),
    4: dict(name="decode_nvfp4", d=2048, E=256, k=6, f=512, fs=512, act=BF16, wdtype=NVFP4,
            T=(1, 16), bias=False, layers=1),
}


def rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_BASE, *key])))


def bf16_bits(a) -> np.ndarray:
    """float32 array -> nearest bf16 (ties to even), as uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    # finite inputs only: the sum stays below 2^32
    u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return u.astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bits -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(g, shape, std):
    a = g.standard_normal(shape, dtype=np.float32)
    a *= np.float32(std)
    return a


def _workers(n):
    return max(1, min(n, int(os.environ.get("FLINT_SYNTH_THREADS", "0")) or
                      min(16, os.cpu_count() or 1)))


def hidden(cfg: int, T: int, d: int, act: int, draw: int = 0, layer: int = 0) -> np.ndarray:
    """Token activations x [T][d] ~ N(0, 1)."""
    a = _normal(rng(cfg, layer, _T_X, draw, T), (T, d), 1.0)
    return bf16_bits(a) if act == BF16 else a


def router(cfg: int, layer: int, E: int, d: int) -> np.ndarray:
    """Router weights [E][d] float32 ~ N(0, 1/d)."""
    return _normal(rng(cfg, layer, _T_ROUTER), (E, d), 1.0 / math.sqrt(d))


def zipf_bias(E: int) -> np.ndarray:
    """b_e = 1.5 * ln(1 / (e + 1)^1.1) for e = 0..E-1, as float32."""
    e = np.arange(E, dtype=np.float64)
    return (1.5 * np.log(1.0 / (e + 1.0) ** 1.1)).astype(np.float32)


def _one_expert(cfg, layer, tid_gu, tid_dn, tid_gs, tid_ds, e, d, f, wdtype):
    if wdtype == NVFP4:
        g = rng(cfg, layer, tid_gu, e)
        gu = g.integers(0, 256, size=(2 * f, d // 2), dtype=np.uint8)
        g = rng(cfg, layer, tid_dn, e)
        dn = g.integers(0, 256, size=(d, f // 2), dtype=np.uint8)
        g = rng(cfg, layer, tid_gs, e)
        gs = g.integers(0x28, 0x41, size=(2 * f, d // 16), dtype=np.uint8)
        g = rng(cfg, layer, tid_ds, e)
        ds = g.integers(0x28, 0x41, size=(d, f // 16), dtype=np.uint8)
        return gu, dn, gs, ds
    gu = _normal(rng(cfg, layer, tid_gu, e), (2 * f, d), 1.0 / math.sqrt(d))
    dn = _normal(rng(cfg, layer, tid_dn, e), (d, f), 1.0 / math.sqrt(f))
    if wdtype == BF16:
        gu, dn = bf16_bits(gu), bf16_bits(dn)
    return gu, dn, None, None


def expert_set(cfg: int, layer: int, n: int, d: int, f: int, wdtype: int, shared: bool = False,
               experts=None) -> dict:
    """Weights of n experts (or of the listed expert ids only, in that order).

    Returns {"gate_up", "down"} plus, for NVFP4, {"gate_up_scales",
    "down_scales", "tensor_scales"}.
    """
    if shared:
        tids = (_T_SGATE_UP, _T_SDOWN, _T_SGU_SCALE, _T_SDN_SCALE)
    else:
        tids = (_T_GATE_UP, _T_DOWN, _T_GU_SCALE, _T_DN_SCALE)
    ids = list(range(n)) if experts is None else [int(e) for e in experts]
    m = len(ids)
    if wdtype == NVFP4:
        gu = np.empty((m, 2 * f, d // 2), np.uint8)
        dn = np.empty((m, d, f // 2), np.uint8)
        gs = np.empty((m, 2 * f, d // 16), np.uint8)
        ds = np.empty((m, d, f // 16), np.uint8)
    else:
        dt = np.uint16 if wdtype == BF16 else np.float32
        gu = np.empty((m, 2 * f, d), dt)
        dn = np.empty((m, d, f), dt)
        gs = ds = None

    def fill(i):
        a, b, c, s = _one_expert(cfg, layer, *tids, ids[i], d, f, wdtype)
        gu[i], dn[i] = a, b
        if wdtype == NVFP4:
            gs[i], ds[i] = c, s

    if m > 4:
        with ThreadPoolExecutor(_workers(m)) as ex:
            list(ex.map(fill, range(m)))
    else:
        for i in range(m):
            fill(i)
    out = {"gate_up": gu, "down": dn}
    if wdtype == NVFP4:
        ts = np.empty((m, 3), np.float32)
        ts[:, 0] = ts[:, 1] = np.float32(1.0 / math.sqrt(d))
        ts[:, 2] = np.float32(1.0 / math.sqrt(f))
        out.update(gate_up_scales=gs, down_scales=ds, tensor_scales=ts)
    return out


def layer(cfg: int, layer_idx: int = 0, experts=None, **override) -> dict:
    """All inputs of one MoE layer of configuration ``cfg`` except x.

    ``experts`` limits the routed set to the listed expert ids (in that order;
    used to rebuild only the experts a sampled token needs).
    """
    c = dict(CONFIGS[cfg])
    c.update(override)
    d, E, f, fs, wd = c["d"], c["E"], c["f"], c["fs"], c["wdtype"]
    out = {
        "router_w": router(cfg, layer_idx, E, d),
        "router_bias": zipf_bias(E) if c["bias"] else None,
        "experts": expert_set(cfg, layer_idx, E, d, f, wd, experts=experts),
        "shared": expert_set(cfg, layer_idx, 1, d, fs, wd, shared=True),
        "cfg": c,
    }
    return out
