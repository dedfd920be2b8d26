"""Seeded synthetic inputs for the MoE-LoRA expert layer.

This module only draws random tensors with the shapes and value distributions of the
workloads (layer shapes of Qwen3-30B-A3B, gpt-oss-20b and DeepSeek-V3, plus a tiny fp32
layer). It computes nothing of the layer itself: no routing, no products, no reductions.
The CPU oracle's tests, the GPU parity tests and the benchmark all draw their inputs here,
so both sides of every comparison see the same values.

Distributions (the second argument of N(0, .) is a standard deviation):
  X ~ N(0,1); W_gu, W_d ~ N(0, 0.02); A_* ~ N(0, 1/r); B_* ~ N(0, 0.01); dY ~ N(0,1).
  W_r ~ N(0, 0.02) for the tiny layer, N(0, 1/sqrt(m)) otherwise so that router logits are
  close to N(0,1) and expert load is near uniform.
  The skewed layer adds a router bias beta_e = -zipf * ln(rank_e), rank a seeded permutation
  of 1..E, so that the bias alone puts a Zipf(zipf) law on the experts.
Every tensor is drawn in fp32 from its own generator stream (seed, tensor id) and, for bf16
layers, rounded once to bf16 (round to nearest even).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch

__all__ = ["LayerConfig", "CONFIGS", "config", "make_inputs", "TENSOR_IDS", "WEIGHT_NAMES"]


@dataclass(frozen=True)
class LayerConfig:
    name: str
    s: int            # tokens
    m: int            # hidden size
    n: int            # expert intermediate size
    E: int            # experts
    k: int            # experts per token
    r: int            # LoRA rank
    alpha: float      # LoRA alpha (scale alpha / r)
    dtype: str        # "f32" or "bf16"
    score: str        # "softmax" or "sigmoid"
    backward: bool    # whether the workload runs the backward pass
    wr_std: float | None = None   # None: 1/sqrt(m)
    zipf: float | None = None     # router-bias exponent for the skewed layer
    renormalize: bool = True

    @property
    def P(self) -> int:
        return self.s * self.k

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


CONFIGS: dict[str, LayerConfig] = {
    # tiny fp32 layer, forward only
    "tiny_fp32": LayerConfig("tiny_fp32", s=256, m=128, n=64, E=8, k=2, r=4, alpha=8.0,
                             dtype="f32", score="softmax", backward=False, wr_std=0.02),
    # Qwen3-30B-A3B expert layer, near-uniform load
    "qwen3_30b_a3b": LayerConfig("qwen3_30b_a3b", s=4096, m=2048, n=768, E=128, k=8, r=16,
                                 alpha=32.0, dtype="bf16", score="softmax", backward=True),
    # same layer, Zipf(1.2)-skewed routing, 16K tokens
    "qwen3_30b_a3b_zipf": LayerConfig("qwen3_30b_a3b_zipf", s=16384, m=2048, n=768, E=128, k=8,
                                      r=16, alpha=32.0, dtype="bf16", score="softmax",
                                      backward=True, zipf=1.2),
    # gpt-oss-20b expert layer
    "gpt_oss_20b": LayerConfig("gpt_oss_20b", s=8192, m=2880, n=2880, E=32, k=4, r=32,
                               alpha=64.0, dtype="bf16", score="softmax", backward=True),
    # DeepSeek-V3 routed-expert layer, sigmoid router
    "deepseek_v3": LayerConfig("deepseek_v3", s=8192, m=7168, n=2048, E=256, k=8, r=16,
                               alpha=32.0, dtype="bf16", score="sigmoid", backward=True),
}


def config(name: str, **overrides) -> LayerConfig:
    """A named layer configuration, optionally with fields replaced (smaller test variants)."""
    cfg = CONFIGS[name]
    if overrides:
        cfg = replace(cfg, **overrides)
    return cfg


TENSOR_IDS = {"X": 1, "W_r": 2, "W_gu": 3, "W_d": 4, "A_g": 5, "B_g": 6, "A_u": 7, "B_u": 8,
              "A_d": 9, "B_d": 10, "dY": 11, "rank": 12}
WEIGHT_NAMES = ("W_gu", "W_d", "A_g", "B_g", "A_u", "B_u", "A_d", "B_d")


def _generator(seed: int, tid: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + tid)
    return g


def _normal(shape, std, seed, tid, device, dtype, chunk_dim0=False):
    """N(0, std) in fp32 from the (seed, tid) stream, rounded once to `dtype`.

    With chunk_dim0 the tensor is drawn one leading slice at a time (bounded fp32 transient
    for multi-GB expert weights); the values then depend only on the stream, not the device
    memory available.
    """
    g = _generator(seed, tid, device)
    if not chunk_dim0:
        t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
        t.mul_(std)
        return t.to(dtype)
    out = torch.empty(*shape, device=device, dtype=dtype)
    for i in range(shape[0]):
        t = torch.randn(*shape[1:], generator=g, device=device, dtype=torch.float32)
        t.mul_(std)
        out[i].copy_(t.to(dtype))
    return out


def make_inputs(cfg: LayerConfig, seed: int = 0, device="cpu", with_grad_output=None) -> dict:
    """Draw every input of the layer for `cfg`.

    Returns a dict of torch tensors on `device`: X [s,m], W_r [m,E], router_bias [E] (fp32,
    or None), W_gu [E,m,2n] (gate columns first, then up), W_d [E,n,m], A_g/A_u [E,m,r],
    B_g/B_u [E,r,n], A_d [E,n,r], B_d [E,r,m], and dY [s,m] when the workload has a backward.
    Values drawn on a CUDA device come from that device's generator and differ from CPU draws
    with the same seed; each set is self-consistent.
    """
    dev = torch.device(device)
    dt = cfg.torch_dtype
    s, m, n, E, r = cfg.s, cfg.m, cfg.n, cfg.E, cfg.r
    big = dev.type != "cpu"
    wr_std = cfg.wr_std if cfg.wr_std is not None else 1.0 / math.sqrt(m)
    out = {
        "X": _normal((s, m), 1.0, seed, TENSOR_IDS["X"], dev, dt),
        "W_r": _normal((m, E), wr_std, seed, TENSOR_IDS["W_r"], dev, dt),
        "W_gu": _normal((E, m, 2 * n), 0.02, seed, TENSOR_IDS["W_gu"], dev, dt, chunk_dim0=big),
        "W_d": _normal((E, n, m), 0.02, seed, TENSOR_IDS["W_d"], dev, dt, chunk_dim0=big),
        "A_g": _normal((E, m, r), 1.0 / r, seed, TENSOR_IDS["A_g"], dev, dt),
        "B_g": _normal((E, r, n), 0.01, seed, TENSOR_IDS["B_g"], dev, dt),
        "A_u": _normal((E, m, r), 1.0 / r, seed, TENSOR_IDS["A_u"], dev, dt),
        "B_u": _normal((E, r, n), 0.01, seed, TENSOR_IDS["B_u"], dev, dt),
        "A_d": _normal((E, n, r), 1.0 / r, seed, TENSOR_IDS["A_d"], dev, dt),
        "B_d": _normal((E, r, m), 0.01, seed, TENSOR_IDS["B_d"], dev, dt),
        "router_bias": None,
    }
    if cfg.zipf is not None:
        g = _generator(seed, TENSOR_IDS["rank"], "cpu")
        rank = torch.randperm(E, generator=g).to(torch.float64) + 1.0
        out["router_bias"] = (-cfg.zipf * torch.log(rank)).to(torch.float32).to(dev)
    want_dy = cfg.backward if with_grad_output is None else with_grad_output
    if want_dy:
        out["dY"] = _normal((s, m), 1.0, seed, TENSOR_IDS["dY"], dev, dt)
    return out
