"""GPU parity: libmoelora (through the C ABI) against the CPU oracle on reduced layers.

Routing protocol: GPU logits must match the oracle's to LOGIT_TOL; the oracle then selects,
weights and groups on the GPU's own logits, and ids / offsets / perm / inv must be bit-equal and
weights within WEIGHT_TOL. The layer outputs and gradients are compared per tensor with
max|gpu - ref| / max|ref| <= 1e-5 (fp32) or 2e-2 (bf16).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from helpers import (LOGIT_TOL, TOL, VARIANTS, WEIGHT_TOL, host_weights, np64, oracle_route_from,
                     rel_err)
from synth import config, make_inputs

pytestmark = pytest.mark.gpu

GRAD_KEYS = ("dA_g", "dB_g", "dA_u", "dB_u", "dA_d", "dB_d")


def _say(msg):
    print(msg, flush=True)


FLAG_RSLORA = 2
FLAG_WEIGHTS_OUT_IN = 4
FLAG_RECOMPUTE = 16
FLAG_FUSED_GU = 32


def fuse_gate_up(inp):
    """One LoRA pair on the fused gate/up projection from the generator's draws: A = A_g and
    B = [B_g | B_u] (E, r, 2n); the per-projection up factors are dropped."""
    return dict(inp, B_g=torch.cat([inp["B_g"], inp["B_u"]], dim=2).contiguous(), A_u=None, B_u=None)


def oracle_weights(inp, flags):
    if not flags & FLAG_FUSED_GU:
        return host_weights(inp)
    W = {k: np64(inp[k]) for k in ("W_gu", "W_d", "A_d", "B_d")}
    W.update(oracle.fused_gate_up_pair(np64(inp["A_g"]), np64(inp["B_g"])))
    return W


def run_gpu(cfg, device, flags=0, router_grad=True, mutate=None):
    """One route + forward (+ backward) of cfg's seeded layer through the C ABI. mutate(inp), when
    given, edits the host inputs first (tied logits, zero factors, non-numbers)."""
    from grouped_gemm_top_amd import layer
    inp = make_inputs(cfg, seed=0, device="cpu", with_grad_output=cfg.backward)
    if mutate is not None:
        mutate(inp)
    if flags & FLAG_FUSED_GU:
        inp = fuse_gate_up(inp)
    d = {k: (v.to(device) if v is not None else None) for k, v in inp.items()}
    if flags & FLAG_WEIGHTS_OUT_IN:  # the library gets W_gu [E, 2n, m] and W_d [E, m, n]
        d["W_gu"] = d["W_gu"].transpose(1, 2).contiguous()
        d["W_d"] = d["W_d"].transpose(1, 2).contiguous()
    shape = layer.shape_of(cfg, router_grad=router_grad, flags=flags)
    rt = layer.route(shape, d["X"], d["W_r"], d["router_bias"])
    # with FLAG_RECOMPUTE nothing is saved: the backward recomputes the forward's intermediates
    keep = cfg.backward and not (flags & FLAG_RECOMPUTE)
    Y, saved = layer.forward(shape, d["X"], rt, d, training=keep)
    out = {"rt": rt, "Y": Y}
    if cfg.backward:
        dX, grads = layer.backward(shape, d["dY"], d["X"], d["W_r"], rt, d, saved)
        out["dX"] = dX
        out.update(grads)
    torch.cuda.synchronize()
    return inp, out


def check_routing(cfg, inp, rt):
    X, Wr = np64(inp["X"]), np64(inp["W_r"])
    bias = np64(inp["router_bias"]) if inp["router_bias"] is not None else None
    z_ref = oracle.router_logits(X, Wr, bias)
    z_gpu = rt["logits"].cpu().numpy().astype(np.float64)
    # NaN logits (from a NaN input) must be NaN on both sides; the numbers are compared
    assert np.array_equal(np.isnan(z_gpu), np.isnan(z_ref))
    num = ~np.isnan(z_ref)
    assert rel_err(z_gpu[num], z_ref[num]) <= LOGIT_TOL
    ort = oracle_route_from(z_gpu, cfg)
    np.testing.assert_array_equal(rt["topk_idx"].cpu().numpy(), ort["idx"])
    np.testing.assert_array_equal(rt["expert_off"].cpu().numpy(), ort["off"])
    np.testing.assert_array_equal(rt["perm"].cpu().numpy(), ort["perm"])
    np.testing.assert_array_equal(rt["inv_perm"].cpu().numpy(), ort["inv"])
    assert rel_err(rt["topk_w"].cpu().numpy(), ort["w"]) <= WEIGHT_TOL
    # selections that would differ under the oracle's own logits (near ties); reported only
    diff = int(np.sum(np.any(np.sort(oracle.topk_experts(z_ref, cfg.k), 1) !=
                             np.sort(ort["idx"], 1), axis=1)))
    _say(f"  tokens whose top-k set differs under the oracle's own logits: {diff}")
    return ort


@pytest.mark.parametrize("flags", [0, 1], ids=["mfma", "reference"])
@pytest.mark.parametrize("name", list(VARIANTS))
def test_layer_parity(name, flags, cuda):
    _parity(VARIANTS[name], name, flags, cuda)


# rsLoRA scale; output-major base weights (forward GEMMs on the reduction-contiguous path,
# backward on the transposing one, LoRA factors transposed for the tails); both; and output-major
# weights on the reference kernels
FLAG_CASES = {"rslora": FLAG_RSLORA, "out_in": FLAG_WEIGHTS_OUT_IN,
              "out_in_rslora": FLAG_WEIGHTS_OUT_IN | FLAG_RSLORA, "out_in_reference": FLAG_WEIGHTS_OUT_IN | 1,
              "recompute": FLAG_RECOMPUTE, "recompute_out_in": FLAG_RECOMPUTE | FLAG_WEIGHTS_OUT_IN,
              # one LoRA pair on the fused gate/up projection, alone and with the other modes
              "fused_gu": FLAG_FUSED_GU, "fused_gu_out_in": FLAG_FUSED_GU | FLAG_WEIGHTS_OUT_IN,
              "fused_gu_recompute": FLAG_FUSED_GU | FLAG_RECOMPUTE, "fused_gu_reference": FLAG_FUSED_GU | 1}


@pytest.mark.parametrize("mode", list(FLAG_CASES))
@pytest.mark.parametrize("name", ["qwen3_small", "gpt_oss_r64", "tiny_fp32_bwd"])
def test_layer_parity_flags(name, mode, cuda):
    _parity(VARIANTS[name], name, FLAG_CASES[mode], cuda)


def _parity(cfg, name, flags, cuda, mutate=None):
    _say(f"[parity] {name} flags={flags} s={cfg.s} m={cfg.m} n={cfg.n} E={cfg.E} k={cfg.k} "
         f"r={cfg.r} {cfg.dtype} {cfg.score} backward={cfg.backward}")
    inp, out = run_gpu(cfg, cuda, flags=flags, mutate=mutate)
    ort = check_routing(cfg, inp, out["rt"])
    W = oracle_weights(inp, flags)
    X = np64(inp["X"])
    rs = bool(flags & FLAG_RSLORA)
    Y_ref, saved = oracle.forward(X, W, ort, cfg.alpha, cfg.r, rslora=rs)
    tol = TOL[cfg.dtype]
    errs = {"Y": rel_err(np64(out["Y"]), Y_ref)}
    if cfg.backward:
        g = oracle.backward(np64(inp["dY"]), X, np64(inp["W_r"]), W, ort, cfg.alpha, cfg.r,
                            cfg.score, cfg.renormalize, True, saved, rslora=rs)
        errs["dX"] = rel_err(np64(out["dX"]), g["dX"])
        keys = GRAD_KEYS
        if flags & FLAG_FUSED_GU:  # dA [E, m, r] in dA_g, dB [E, r, 2n] in dB_g
            g["dA_g"], g["dB_g"] = oracle.fused_gate_up_grads(g)
            keys = ("dA_g", "dB_g", "dA_d", "dB_d")
            assert out["dB_g"].shape == (cfg.E, cfg.r, 2 * cfg.n)
        for key in keys:
            errs[key] = rel_err(np64(out[key]), g[key])
    _say("  rel errors: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"over tolerance {tol}: {bad}"
    return inp, out


def test_router_grad_off(cuda):
    cfg = VARIANTS["qwen3_small"]
    _say("[parity] router_grad=0 qwen3_small")
    inp, out = run_gpu(cfg, cuda, router_grad=False)
    ort = check_routing(cfg, inp, out["rt"])
    W = host_weights(inp)
    X = np64(inp["X"])
    _, saved = oracle.forward(X, W, ort, cfg.alpha, cfg.r)
    g = oracle.backward(np64(inp["dY"]), X, np64(inp["W_r"]), W, ort, cfg.alpha, cfg.r,
                        cfg.score, cfg.renormalize, False, saved)
    assert rel_err(np64(out["dX"]), g["dX"]) <= TOL[cfg.dtype]


def test_zero_token_experts_get_zero_grads(cuda):
    cfg = VARIANTS["qwen3_zipf_small"]
    _say("[parity] zero-token experts")
    inp, out = run_gpu(cfg, cuda)
    off = out["rt"]["expert_off"].cpu().numpy()
    empty = np.where(off[1:] == off[:-1])[0]
    assert empty.size > 0, "the skewed layer should leave some experts without tokens"
    for key in GRAD_KEYS:
        assert torch.all(out[key][torch.as_tensor(empty, device=cuda)] == 0)


@pytest.mark.parametrize("name", ["qwen3_small", "chunked_expert", "big_expert"])
def test_determinism(name, cuda):
    """Two runs give bit-identical outputs and gradients: no float atomics anywhere, and the
    chunked LoRA-gradient reductions (experts longer than one 1024-row chunk) add their partials
    in chunk order."""
    cfg = VARIANTS[name]
    _say(f"[parity] determinism {name}")
    _, a = run_gpu(cfg, cuda)
    _, b = run_gpu(cfg, cuda)
    if name == "chunked_expert":
        cnt = np.diff(a["rt"]["expert_off"].cpu().numpy())
        assert cnt.max() > 1024, "the layer should have an expert longer than one gradient chunk"
    for key in ("Y", "dX") + GRAD_KEYS:
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("out_in", [False, True], ids=["x_w", "out_in"])
@pytest.mark.parametrize("name", ["qwen3_small", "tiny_fp32", "gpt_oss_r64"])
def test_merged_weights_forward(name, out_in, cuda):
    """The materialised PEFT form: moe_peft_merge against W + c A B on the host, and the forward on
    merged weights (no Split-LoRA work) against the oracle's Split-LoRA forward."""
    from grouped_gemm_top_amd import layer, moe_peft_merge
    cfg = VARIANTS[name]
    _say(f"[merged] {name} out_in={out_in}")
    flags = FLAG_WEIGHTS_OUT_IN if out_in else 0
    inp = make_inputs(cfg, seed=0, device="cpu", with_grad_output=False)
    d = {k: (v.to(cuda) if v is not None else None) for k, v in inp.items()}
    if out_in:
        d["W_gu"] = d["W_gu"].transpose(1, 2).contiguous()
        d["W_d"] = d["W_d"].transpose(1, 2).contiguous()
    shape = layer.shape_of(cfg, flags=flags)
    Wm_gu, Wm_d = torch.empty_like(d["W_gu"]), torch.empty_like(d["W_d"])
    moe_peft_merge(shape, d["W_gu"], d["W_d"], d["A_g"], d["B_g"], d["A_u"], d["B_u"], d["A_d"],
                   d["B_d"], Wm_gu, Wm_d)
    torch.cuda.synchronize()
    W = host_weights(inp)
    n = cfg.n
    ref = oracle.merged_weights(W, cfg.alpha, cfg.r)
    ref_gu, ref_d = ref["W_gu"], ref["W_d"]
    got_gu, got_d = np64(Wm_gu), np64(Wm_d)
    if out_in:
        got_gu, got_d = got_gu.transpose(0, 2, 1), got_d.transpose(0, 2, 1)
    tol = TOL[cfg.dtype]
    assert rel_err(got_gu, ref_gu) <= tol and rel_err(got_d, ref_d) <= tol
    assert ref_gu.shape[2] == 2 * n
    rt = layer.route(shape, d["X"], d["W_r"], d["router_bias"])
    dm = dict(d, W_gu=Wm_gu, W_d=Wm_d, A_g=None, B_g=None, A_u=None, B_u=None, A_d=None, B_d=None)
    Y, _ = layer.forward(layer.shape_of(cfg, flags=flags | 8), d["X"], rt, dm, training=False)
    torch.cuda.synchronize()
    ort = check_routing(cfg, inp, rt)
    Y_ref, _ = oracle.forward(np64(inp["X"]), W, ort, cfg.alpha, cfg.r, keep=False)
    err = rel_err(np64(Y), Y_ref)
    _say(f"  merge err gu {rel_err(got_gu, ref_gu):.2e} d {rel_err(got_d, ref_d):.2e}; Y {err:.2e}")
    assert err <= tol


@pytest.mark.parametrize("out_in", [False, True], ids=["x_w", "out_in"])
def test_merged_weights_fused_gate_up(out_in, cuda):
    """moe_peft_merge with one fused gate/up pair: W_gu + c A B over all 2n columns."""
    from grouped_gemm_top_amd import layer, moe_peft_merge
    cfg = VARIANTS["qwen3_small"]
    _say(f"[merged fused] qwen3_small out_in={out_in}")
    flags = FLAG_FUSED_GU | (FLAG_WEIGHTS_OUT_IN if out_in else 0)
    inp = fuse_gate_up(make_inputs(cfg, seed=0, device="cpu", with_grad_output=False))
    d = {k: (v.to(cuda) if v is not None else None) for k, v in inp.items()}
    if out_in:
        d["W_gu"] = d["W_gu"].transpose(1, 2).contiguous()
        d["W_d"] = d["W_d"].transpose(1, 2).contiguous()
    shape = layer.shape_of(cfg, flags=flags)
    Wm_gu, Wm_d = torch.empty_like(d["W_gu"]), torch.empty_like(d["W_d"])
    moe_peft_merge(shape, d["W_gu"], d["W_d"], d["A_g"], d["B_g"], None, None, d["A_d"], d["B_d"],
                   Wm_gu, Wm_d)
    torch.cuda.synchronize()
    W = oracle_weights(inp, flags)
    ref_gu = oracle.merged_weights({key: (np64(v) if v is not None else None) for key, v in inp.items()},
                                   cfg.alpha, cfg.r)["W_gu"]
    got_gu = np64(Wm_gu)
    if out_in:
        got_gu = got_gu.transpose(0, 2, 1)
    err = rel_err(got_gu, ref_gu)
    rt = layer.route(shape, d["X"], d["W_r"], d["router_bias"])
    dm = dict(d, W_gu=Wm_gu, W_d=Wm_d, A_g=None, B_g=None, A_u=None, B_u=None, A_d=None, B_d=None)
    Y, _ = layer.forward(layer.shape_of(cfg, flags=flags | 8), d["X"], rt, dm, training=False)
    torch.cuda.synchronize()
    ort = check_routing(cfg, inp, rt)
    Y_ref, _ = oracle.forward(np64(inp["X"]), W, ort, cfg.alpha, cfg.r, keep=False)
    yerr = rel_err(np64(Y), Y_ref)
    _say(f"  merge err gu {err:.2e}; Y {yerr:.2e}")
    assert err <= TOL[cfg.dtype] and yerr <= TOL[cfg.dtype]


# Degenerate and extreme shapes of the routing: every expert chosen by every token, one expert per
# token, a single token, the largest expert count (most experts empty), sigmoid scores without
# renormalisation (the router gradient then has no coupling between a token's slots), expert
# counts that are not a multiple of the wave width, and more slots per token than a wave has lanes.
EDGE = {
    "k_equals_E": config("qwen3_30b_a3b", s=64, m=128, n=64, E=8, k=8),
    "k_one": config("qwen3_30b_a3b", s=200, m=128, n=64, E=16, k=1),
    "one_token": config("qwen3_30b_a3b", s=1, m=128, n=64, E=8, k=2),
    "max_experts": config("qwen3_30b_a3b", s=300, m=128, n=64, E=1024, k=4),
    "sigmoid_no_renorm": config("deepseek_v3", s=256, m=128, n=64, E=16, k=4, renormalize=False),
    # expert counts that fill 4 and 8 slots per lane of the top-k wave, the last slot partly
    "experts_200_sigmoid_bias": config("deepseek_v3", s=160, m=128, n=64, E=200, k=8, zipf=0.8),
    "experts_320": config("qwen3_30b_a3b", s=160, m=128, n=64, E=320, k=6),
    # more than 64 slots per token: a token's slots span two waves' worth of lanes
    "k_over_64": config("qwen3_30b_a3b", s=40, m=128, n=64, E=96, k=72),
    # bf16 expert counts that are not a multiple of 8 (rows of W_r not 16-byte aligned): 60 experts
    # as in Qwen1.5-MoE, and 12
    "experts_60": config("qwen3_30b_a3b", s=300, m=192, n=128, E=60, k=4),
    "experts_12": config("qwen3_30b_a3b", s=200, m=128, n=64, E=12, k=2),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_shapes(name, cuda):
    _parity(EDGE[name], name, 0, cuda)


def test_empty_batch(cuda):
    """s == 0: every call succeeds, nothing is written but the gradients, which are zeroed."""
    from grouped_gemm_top_amd import layer
    cfg = config("qwen3_30b_a3b", s=0, m=128, n=64, E=8, k=2)
    _say("[edge] empty batch")
    inp = make_inputs(cfg, seed=0, device="cpu", with_grad_output=True)
    d = {k: (v.to(cuda) if v is not None else None) for k, v in inp.items()}
    shape = layer.shape_of(cfg)
    rt = layer.route(shape, d["X"], d["W_r"], d["router_bias"])
    Y, saved = layer.forward(shape, d["X"], rt, d)
    grads = {k: torch.full(v.shape, 7.0, device=cuda) for k, v in layer.alloc_grads(shape, cuda).items()}
    dX, grads = layer.backward(shape, d["dY"], d["X"], d["W_r"], rt, d, saved, grads=grads)
    torch.cuda.synchronize()
    assert Y.shape == (0, cfg.m) and dX.shape == (0, cfg.m)
    assert torch.all(rt["expert_off"] == 0)
    for key, v in grads.items():
        assert torch.all(v == 0), key


# ---------------------------------------------------------------- the method's own special cases

def _zero_rows(inp):
    """Every fifth token's x_t = 0 (no router bias): all E logits of those tokens are exactly 0."""
    inp["X"][::5] = 0


def _dup_router_columns(inp):
    """W_r[:, 2j+1] = W_r[:, 2j]: the two logits of each expert pair are equal for every token."""
    inp["W_r"][:, 1::2] = inp["W_r"][:, 0::2]


@pytest.mark.parametrize("name", ["qwen3_small", "deepseek_small"])
def test_exact_ties_go_to_the_lower_expert(name, cuda):
    """Exactly tied logits: all-zero logits select experts 0..k-1 with weights 1/k (softmax) or
    equal sigmoid weights, and tied expert pairs are taken lower id first. The ids are checked bit-exact
    against the oracle's selection on the GPU's logits, which holds the tie rule."""
    cfg = VARIANTS[name]
    _, out = _parity(cfg, f"{name}_zero_rows", 0, cuda, mutate=_zero_rows)
    idx = out["rt"]["topk_idx"].cpu().numpy()
    w = out["rt"]["topk_w"].cpu().numpy()
    z = out["rt"]["logits"].cpu().numpy()
    assert np.all(z[::5] == 0.0)
    assert np.all(idx[::5] == np.arange(cfg.k))
    np.testing.assert_allclose(w[::5], 1.0 / cfg.k, rtol=1e-6, atol=0)
    _, out = _parity(cfg, f"{name}_dup_columns", 0, cuda, mutate=_dup_router_columns)
    z = out["rt"]["logits"].cpu().numpy()
    assert np.array_equal(z[:, 0::2], z[:, 1::2]), "duplicated W_r columns should give equal logits"
    idx = out["rt"]["topk_idx"].cpu().numpy()
    pos = np.full((cfg.s, cfg.E), cfg.k)
    np.put_along_axis(pos, idx.astype(np.int64), np.arange(cfg.k)[None, :].repeat(cfg.s, 0), axis=1)
    even, odd = pos[:, 0::2], pos[:, 1::2]
    # of each tied pair, the lower id is selected whenever the higher one is, and before it
    assert np.all(even[odd < cfg.k] < odd[odd < cfg.k])


def test_alpha_zero_is_the_plain_moe_layer(cuda):
    """alpha = 0: Y is the MoE layer without adapters and every LoRA gradient is exactly zero."""
    cfg = config("qwen3_30b_a3b", s=512, m=256, n=192, E=16, k=4, alpha=0.0)
    _, out = _parity(cfg, "alpha_zero", 0, cuda)
    for key in GRAD_KEYS:
        assert torch.count_nonzero(out[key]).item() == 0, key


def _zero_B(inp):
    for key in ("B_g", "B_u", "B_d"):
        inp[key].zero_()


def test_zero_B_gives_zero_dA(cuda):
    """B = 0 (the usual LoRA initialisation): the adapters add nothing, dA is exactly zero and dB is
    not."""
    cfg = VARIANTS["qwen3_small"]
    _, out = _parity(cfg, "zero_B", 0, cuda, mutate=_zero_B)
    for key in ("dA_g", "dA_u", "dA_d"):
        assert torch.count_nonzero(out[key]).item() == 0, key
    for key in ("dB_g", "dB_u", "dB_d"):
        assert torch.count_nonzero(out[key]).item() > 0, key


def _nan_router_column(inp):
    inp["W_r"][:, 5] = float("nan")


def test_nan_router_column_is_never_selected(cuda):
    """A NaN column of W_r gives that expert NaN logits, which count as -inf: the expert is never
    selected, scores 0 in every softmax denominator, and the rest of the layer matches the oracle."""
    cfg = VARIANTS["qwen3_small"]
    _, out = _parity(cfg, "nan_router_column", 0, cuda, mutate=_nan_router_column)
    idx = out["rt"]["topk_idx"].cpu().numpy()
    assert not np.any(idx == 5)
    assert torch.isfinite(out["Y"]).all() and torch.isfinite(out["dX"]).all()


def test_nan_token_routes_to_valid_experts(cuda):
    """A token whose x_t is NaN has only NaN logits: it is routed to experts 0..k-1 (ties at -inf go
    to the lower id), every id stays in range, and every other token's output matches the oracle."""
    from grouped_gemm_top_amd import layer
    cfg = config("qwen3_30b_a3b", s=256, m=256, n=128, E=16, k=4, backward=False)
    _say("[edge] NaN token row")
    bad_t = 7
    inp = make_inputs(cfg, seed=0, device="cpu", with_grad_output=False)
    inp["X"][bad_t] = float("nan")
    d = {k: (v.to(cuda) if v is not None else None) for k, v in inp.items()}
    shape = layer.shape_of(cfg)
    rt = layer.route(shape, d["X"], d["W_r"], d["router_bias"])
    Y, _ = layer.forward(shape, d["X"], rt, d, training=False)
    torch.cuda.synchronize()
    idx = rt["topk_idx"].cpu().numpy()
    assert idx.min() >= 0 and idx.max() < cfg.E
    assert list(idx[bad_t]) == list(range(cfg.k))
    z_gpu = rt["logits"].cpu().numpy().astype(np.float64)
    assert np.all(np.isnan(z_gpu[bad_t]))
    ort = oracle_route_from(z_gpu, cfg)
    np.testing.assert_array_equal(idx, ort["idx"])
    np.testing.assert_array_equal(rt["perm"].cpu().numpy(), ort["perm"])
    good = np.arange(cfg.s) != bad_t
    Xh = np64(inp["X"])
    Xh[bad_t] = 0.0  # its rows' results are not compared
    Y_ref, _ = oracle.forward(Xh, host_weights(inp), ort, cfg.alpha, cfg.r, keep=False)
    assert rel_err(np64(Y)[good], Y_ref[good]) <= TOL[cfg.dtype]
