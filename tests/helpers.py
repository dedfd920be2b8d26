"""Shared helpers for the parity tests: layer variants, tolerances, oracle runs on host copies."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from synth import config

# Tolerances on max|gpu - ref| / max|ref| per output tensor.
TOL = {"f32": 1e-5, "bf16": 2e-2}
LOGIT_TOL = 1e-5     # router logits, fp32 accumulation on both sides
WEIGHT_TOL = 1e-6    # routing weights from identical logits

# Reduced layers the oracle finishes in seconds; each spans several row and column tiles of the
# GPU kernels, has ragged last tiles, and keeps the structure of the full workload it is named for.
VARIANTS = {
    "tiny_fp32": config("tiny_fp32"),
    "tiny_fp32_bwd": config("tiny_fp32", backward=True),
    "qwen3_small": config("qwen3_30b_a3b", s=512, m=256, n=192, E=16, k=4),
    "qwen3_zipf_small": config("qwen3_30b_a3b_zipf", s=1024, m=256, n=128),
    "gpt_oss_small": config("gpt_oss_20b", s=384, m=320, n=320, E=8, k=4),
    "deepseek_small": config("deepseek_v3", s=512, m=448, n=128, E=32, k=8),
    # the largest supported rank: two-factor LoRA tails 2r = 128 reduction rows long
    "gpt_oss_r64": config("gpt_oss_20b", s=384, m=192, n=256, E=8, k=4, r=64, alpha=128.0),
    # an expert with more than one 256-row tile, and ragged last tiles
    "big_expert": config("qwen3_30b_a3b_zipf", s=1024, m=128, n=192, E=16, k=2, zipf=2.0),
    # an expert longer than several 1024-row chunks (chunked LoRA-gradient reductions)
    "chunked_expert": config("qwen3_30b_a3b_zipf", s=4096, m=128, n=64, E=8, k=2, zipf=2.0),
}


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = float(np.max(np.abs(ref))) if ref.size else 0.0
    if denom == 0.0:
        return float(np.max(np.abs(got))) if got.size else 0.0
    return float(np.max(np.abs(got - ref))) / denom


def host_weights(inp: dict) -> dict:
    return {k: np64(inp[k]) for k in ("W_gu", "W_d", "A_g", "B_g", "A_u", "B_u", "A_d", "B_d")}


def oracle_route_from(z: np.ndarray, cfg) -> dict:
    return oracle.route(z, cfg.k, cfg.E, cfg.score, cfg.renormalize)
