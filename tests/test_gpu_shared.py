"""GPU parity of the shared expert (moe_shared_forward / moe_shared_backward through the C ABI)
against the CPU oracle.

The shared expert adds into the caller's Y and dX, so each case starts them from a known tensor
(2^-6 times X and dY: exact scalings, of the same magnitude as the expert's own contribution, so
that both a missing addition and a missing contribution exceed the tolerance) and compares the
sums. The LoRA-factor gradients are compared directly.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from helpers import TOL, np64, rel_err
from synth import config, make_inputs

pytestmark = pytest.mark.gpu

FLAG_RSLORA, FLAG_OUT_IN, FLAG_RECOMPUTE, FLAG_FUSED_GU = 2, 4, 16, 32
WEIGHTS = ("W_gu", "W_d", "A_g", "B_g", "A_u", "B_u", "A_d", "B_d")

# shared-expert layers (E and k of the routed layer do not apply; expert 0's draws are used)
CASES = {
    # ragged last row tiles
    "bf16": config("qwen3_30b_a3b", s=600, m=256, n=192, E=8, k=1),
    # longer than two 1024-row chunks of the K-grouped gradient reductions
    "bf16_chunked": config("qwen3_30b_a3b", s=2500, m=128, n=64, E=8, k=1),
    # the largest rank
    "bf16_r64": config("gpt_oss_20b", s=384, m=192, n=256, E=8, k=1, r=64, alpha=128.0),
    "fp32": config("tiny_fp32", backward=True, k=1),
}
MODES = {"plain": 0, "rslora": FLAG_RSLORA, "out_in": FLAG_OUT_IN, "fused_gu": FLAG_FUSED_GU,
         "recompute": FLAG_RECOMPUTE, "reference": 1,
         "fused_out_in_recompute": FLAG_FUSED_GU | FLAG_OUT_IN | FLAG_RECOMPUTE}


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("name", list(CASES))
def test_shared_expert_parity(name, mode, cuda):
    from grouped_gemm_top_amd import layer
    cfg, flags = CASES[name], MODES[mode]
    _say(f"[shared] {name} {mode} s={cfg.s} m={cfg.m} n={cfg.n} r={cfg.r} {cfg.dtype}")
    inp = make_inputs(cfg, seed=0, device="cpu", with_grad_output=True)
    W1 = {k: inp[k][0].contiguous() for k in WEIGHTS}
    if flags & FLAG_FUSED_GU:  # one pair on gate_up_proj: A = A_g, B = [B_g | B_u]
        W1["B_g"] = torch.cat([W1["B_g"], W1["B_u"]], dim=1).contiguous()
        W1["A_u"] = W1["B_u"] = None
    d = {k: (v.to(cuda) if v is not None else None) for k, v in W1.items()}
    if flags & FLAG_OUT_IN:
        d["W_gu"] = d["W_gu"].t().contiguous()
        d["W_d"] = d["W_d"].t().contiguous()
    X, dY = inp["X"].to(cuda), inp["dY"].to(cuda)
    Y = (X * 2.0 ** -6).contiguous()
    dX = (dY * 2.0 ** -6).contiguous()
    Y0, dX0 = np64(Y), np64(dX)
    shape = layer.shape_of(cfg, flags=flags)
    keep = not (flags & FLAG_RECOMPUTE)
    saved = layer.shared_forward(shape, X, d, Y, training=keep)
    grads = layer.shared_backward(shape, dY, X, d, saved, dX)
    torch.cuda.synchronize()

    Wo = {k: np64(v) for k, v in W1.items() if v is not None}
    if flags & FLAG_FUSED_GU:
        Wo.update(oracle.fused_gate_up_pair(Wo["A_g"], Wo["B_g"]))
    rs = bool(flags & FLAG_RSLORA)
    Xh, dYh = np64(inp["X"]), np64(inp["dY"])
    f = oracle.shared_expert_forward(Xh, Wo, cfg.alpha, cfg.r, rslora=rs)
    g = oracle.shared_expert_backward(dYh, Xh, Wo, cfg.alpha, cfg.r, f, rslora=rs)
    errs = {"Y": rel_err(np64(Y), Y0 + f["o"]), "dX": rel_err(np64(dX), dX0 + g["dX"])}
    keys = ("dA_g", "dB_g", "dA_u", "dB_u", "dA_d", "dB_d")
    if flags & FLAG_FUSED_GU:
        g["dA_g"], g["dB_g"] = oracle.fused_gate_up_grads(g)
        keys = ("dA_g", "dB_g", "dA_d", "dB_d")
    for key in keys:
        errs[key] = rel_err(np64(grads[key]), g[key])
    _say("  rel errors: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    tol = TOL[cfg.dtype]
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"over tolerance {tol}: {bad}"
    # both the prior contents and the expert's contribution are needed to pass
    assert rel_err(np64(Y), f["o"]) > 10 * tol and rel_err(np64(Y), Y0) > 10 * tol


def test_shared_expert_no_tokens(cuda):
    """s == 0: the gradients are zeroed and nothing else is touched."""
    from grouped_gemm_top_amd import layer
    cfg = config("qwen3_30b_a3b", s=0, m=128, n=64, E=8, k=1)
    shape = layer.shape_of(cfg)
    m, n, r = cfg.m, cfg.n, cfg.r
    W1 = {"W_gu": torch.zeros(m, 2 * n), "W_d": torch.zeros(n, m), "A_g": torch.zeros(m, r),
          "B_g": torch.zeros(r, n), "A_u": torch.zeros(m, r), "B_u": torch.zeros(r, n),
          "A_d": torch.zeros(n, r), "B_d": torch.zeros(r, m)}
    d = {k: v.to(cuda, torch.bfloat16) for k, v in W1.items()}
    X = torch.zeros(0, m, dtype=torch.bfloat16, device=cuda)
    saved = layer.shared_forward(shape, X, d, X.clone())
    grads = {k: torch.full(v.shape, 7.0, device=cuda) for k, v in
             (("dA_g", d["A_g"]), ("dB_g", d["B_g"]), ("dA_u", d["A_u"]), ("dB_u", d["B_u"]),
              ("dA_d", d["A_d"]), ("dB_d", d["B_d"]))}
    layer.shared_backward(shape, X, X, d, saved, X.clone(), grads)
    torch.cuda.synchronize()
    for key, v in grads.items():
        assert torch.all(v == 0), key


@pytest.mark.timeout(600)
@pytest.mark.parametrize("flags", [0, FLAG_FUSED_GU], ids=["pairs", "fused_gu"])
def test_shared_expert_fullsize(flags, cuda):
    """The shared expert at the Qwen3-30B-A3B layer's size (4096 tokens, m 2048, n 768, r 16): every
    output row and every gradient against the fp64 oracle. Its gradient reductions split the one
    group into many chunks at this size."""
    from grouped_gemm_top_amd import layer
    cfg = config("qwen3_30b_a3b", E=8, k=1)
    _say(f"[shared fullsize] flags={flags} s={cfg.s} m={cfg.m} n={cfg.n} r={cfg.r}")
    inp = make_inputs(cfg, seed=0, device="cpu", with_grad_output=True)
    W1 = {k: inp[k][0].contiguous() for k in WEIGHTS}
    if flags & FLAG_FUSED_GU:
        W1["B_g"] = torch.cat([W1["B_g"], W1["B_u"]], dim=1).contiguous()
        W1["A_u"] = W1["B_u"] = None
    d = {k: (v.to(cuda) if v is not None else None) for k, v in W1.items()}
    X, dY = inp["X"].to(cuda), inp["dY"].to(cuda)
    Y = (X * 2.0 ** -6).contiguous()
    dX = (dY * 2.0 ** -6).contiguous()
    Y0, dX0 = np64(Y), np64(dX)
    shape = layer.shape_of(cfg, flags=flags)
    saved = layer.shared_forward(shape, X, d, Y)
    grads = layer.shared_backward(shape, dY, X, d, saved, dX)
    torch.cuda.synchronize()
    Wo = {k: np64(v) for k, v in W1.items() if v is not None}
    if flags & FLAG_FUSED_GU:
        Wo.update(oracle.fused_gate_up_pair(Wo["A_g"], Wo["B_g"]))
    Xh, dYh = np64(inp["X"]), np64(inp["dY"])
    f = oracle.shared_expert_forward(Xh, Wo, cfg.alpha, cfg.r)
    g = oracle.shared_expert_backward(dYh, Xh, Wo, cfg.alpha, cfg.r, f)
    errs = {"Y": rel_err(np64(Y), Y0 + f["o"]), "dX": rel_err(np64(dX), dX0 + g["dX"])}
    keys = ("dA_g", "dB_g", "dA_u", "dB_u", "dA_d", "dB_d")
    if flags & FLAG_FUSED_GU:
        g["dA_g"], g["dB_g"] = oracle.fused_gate_up_grads(g)
        keys = ("dA_g", "dB_g", "dA_d", "dB_d")
    for key in keys:
        errs[key] = rel_err(np64(grads[key]), g[key])
    _say("  rel errors: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL[cfg.dtype]}
    assert not bad, f"over tolerance: {bad}"
