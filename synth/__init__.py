"""Seeded synthetic inputs for the MoE layer workloads.

This module draws random numbers and lays out input tensors; it holds none of the
layer's arithmetic, and both the library's tests/benchmark and the oracle consume
what it produces.  The workloads stand in for the pages' measurement set-ups ("Ai2
rebuilds Olmo's training stack ..." / "MXFP8 reduces compute and memory costs":
uniform routing across experts; "A 1.2-trillion-parameter systems test": random
routing; learned routers give uneven loads), at the layer shapes below.

Recipe (numpy PCG64, one independent stream per tensor, so draw order cannot matter):
  x             default_rng([seed, 0])          standard normal, bf16
  dy            default_rng([seed, 5])          standard normal, bf16
  router        default_rng([seed, E, 1])       router weight N(0, 0.02^2) fp32 [d, E],
                                                or logit noise N(0, 1) fp32 [T, E]
  expert e      default_rng([seed, E, 2|3|4, e]) W_gate | W_up | W_down, N(0, 0.02^2), bf16
Normals are drawn as float32 (`standard_normal(dtype=float32)`), scaled in float32 and
rounded to bf16 (round-to-nearest-even) by torch's CPU cast.  bf16 tensors are returned
as uint16 bit patterns.

Logit constructions:
  "router"     logits come from the layer's own router projection of x (w_r given)
  "roundrobin" L[t, (k*t + j) mod E] = k - j for j < k, 0 elsewhere: every expert gets
               exactly T*k/E rows when E divides T*k and k*T covers all experts evenly
  "normal"     N(0, 1) logits
  "zipf"       N(0, 1) + 3*ln(p_e), p_e = (e+1)^-1.2 / sum_i i^-1.2: a few experts take
               most rows, some take none
"""

import concurrent.futures
import os
from dataclasses import dataclass, replace

import numpy as np
import torch

W_STD = 0.02


@dataclass(frozen=True)
class LayerConfig:
    name: str
    seed: int
    T: int
    d: int
    E: int
    k: int
    f: int
    logits: str          # "router" | "roundrobin" | "normal" | "zipf"
    mxfp8: bool = False
    forward_only: bool = False

    @property
    def n(self):
        return self.T * self.k

    def with_(self, **kw):
        return replace(self, **kw)


CONFIGS = {
    "tiny": LayerConfig("tiny", 0, 256, 128, 8, 2, 256, "router", forward_only=True),
    "balanced": LayerConfig("balanced", 1, 8192, 2048, 64, 4, 1024, "roundrobin"),
    "sweep": LayerConfig("sweep", 2, 16384, 4096, 8, 4, 1536, "normal"),   # E in SWEEP_E
    "skewed": LayerConfig("skewed", 3, 16384, 4096, 128, 8, 768, "zipf"),
    "mxfp8": LayerConfig("mxfp8", 4, 32768, 7168, 64, 4, 2048, "router", mxfp8=True),
}
SWEEP_E = (8, 16, 32, 64, 128)


def to_bf16_bits(a):
    """float32 array -> bf16 bit patterns (uint16) via torch's RNE cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _normal(key, shape, std=1.0):
    g = np.random.default_rng(key)
    a = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def gen_x(cfg):
    return to_bf16_bits(_normal([cfg.seed, 0], (cfg.T, cfg.d)))


def gen_dy(cfg):
    return to_bf16_bits(_normal([cfg.seed, 5], (cfg.T, cfg.d)))


def gen_router_weight(cfg):
    return _normal([cfg.seed, cfg.E, 1], (cfg.d, cfg.E), W_STD)


def gen_logits(cfg):
    """Logits for the constructions that do not use a router projection."""
    T, E, k = cfg.T, cfg.E, cfg.k
    if cfg.logits == "roundrobin":
        L = np.zeros((T, E), dtype=np.float32)
        t = np.arange(T)
        for j in range(k):
            L[t, (k * t + j) % E] = np.float32(k - j)
        return L
    noise = _normal([cfg.seed, E, 1], (T, E))
    if cfg.logits == "normal":
        return noise
    if cfg.logits == "zipf":
        ranks = np.arange(1, E + 1, dtype=np.float64)
        p = ranks ** -1.2
        p /= p.sum()
        bias = (3.0 * np.log(p)).astype(np.float32)
        return noise + bias[None, :]
    raise ValueError(f"gen_logits: construction {cfg.logits!r} has no direct logits")


def gen_expert_weights(cfg, experts=None):
    """(w_gate [E,f,d], w_up [E,f,d], w_down [E,d,f]) as bf16 bits; `experts` limits the
    draw to a subset (the other experts' slices are left zero and must not be used).  Experts
    are drawn on a thread pool (each has its own streams, so the result does not depend on it)."""
    E, d, f = cfg.E, cfg.d, cfg.f
    wg = np.zeros((E, f, d), dtype=np.uint16)
    wu = np.zeros((E, f, d), dtype=np.uint16)
    wd = np.zeros((E, d, f), dtype=np.uint16)

    def one(e):
        wg[e] = to_bf16_bits(_normal([cfg.seed, E, 2, e], (f, d), W_STD))
        wu[e] = to_bf16_bits(_normal([cfg.seed, E, 3, e], (f, d), W_STD))
        wd[e] = to_bf16_bits(_normal([cfg.seed, E, 4, e], (d, f), W_STD))

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(one, range(E) if experts is None else experts))
    return wg, wu, wd


def make_inputs(cfg, with_dy=True):
    """All host inputs of one workload as numpy arrays (bf16 tensors as uint16 bits)."""
    out = dict(x=gen_x(cfg))
    if cfg.logits == "router":
        out["w_r"] = gen_router_weight(cfg)
    else:
        out["logits"] = gen_logits(cfg)
    out["w_gate"], out["w_up"], out["w_down"] = gen_expert_weights(cfg)
    if with_dy:
        out["dy"] = gen_dy(cfg)
    return out


def to_torch(inputs, device):
    """Moves a make_inputs() dict to `device`: bf16 bit arrays become torch.bfloat16 tensors,
    fp32 arrays torch.float32 (a layout change only)."""
    out = {}
    for key, a in inputs.items():
        if a.dtype == np.uint16:
            out[key] = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
        else:
            out[key] = torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return out
