"""Full-size parity: every workload at its real shape, in the launch configuration the benchmark uses.

Routing is checked in full (ids, offsets, perm, inv bit-exact on the GPU's own logits; weights to
1e-6). The two Qwen3-30B-A3B layers compare every token of Y and dX and every expert's LoRA-factor
gradients with the oracle's whole layer in fp64. The larger layers are checked on sampled tokens
(y_t and dX_t depend only on x_t, dY_t and the token's k experts) and LoRA gradients on sampled
experts (an expert's gradients depend only on its own rows), computed by the oracle in fp64.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from helpers import LOGIT_TOL, TOL, WEIGHT_TOL, rel_err
from synth import config, make_inputs

pytestmark = pytest.mark.gpu

GRADS = ("dA_g", "dB_g", "dA_u", "dB_u", "dA_d", "dB_d")


def _say(msg):
    print(msg, flush=True)


class LazyExperts:
    """Expert slices of a device tensor, copied to host fp64 on first use and kept (only the
    experts of the sampled tokens and the sampled experts are ever touched)."""

    def __init__(self, t: torch.Tensor):
        self.t = t
        self.shape = tuple(t.shape)
        self.cache = {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            self.cache[e] = self.t[e].to(torch.float32).cpu().numpy().astype(np.float64)
        return self.cache[e]


class NoCache:
    """Expert slices of a device tensor, copied to host fp64 on every access (for layers whose
    experts do not all fit in host memory as fp64)."""

    def __init__(self, t: torch.Tensor):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, e):
        return self.t[int(e)].to(torch.float32).cpu().numpy().astype(np.float64)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


# (name, tokens, experts): "all" compares every token of Y and dX and every expert's gradients
# against the oracle's whole layer; a number samples that many tokens and experts, the experts
# chosen to include the busiest, an empty one and those whose last 128-row tile is the most
# ragged (1..a few rows past a tile boundary).
WORKLOADS = [
    ("qwen3_30b_a3b", "all", "all"),
    ("qwen3_30b_a3b_zipf", "all", "all"),
    ("gpt_oss_20b", 64, 16),
    ("deepseek_v3", 64, 16),
]


class Rows:
    """Row access X[t:t+1] / X[idx] on a device tensor, returned as host fp64."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, i):
        if isinstance(i, slice):
            return f64(self.t[i])
        return f64(self.t[torch.as_tensor(np.asarray(i), device=self.t.device)])


def _check_expert_grads(e, cnt, grads, ge, tol):
    errs = {key: rel_err(grads[key][e].cpu().numpy(), ge[key]) for key in GRADS}
    if cnt[e] == 0:
        assert all(torch.all(grads[key][e] == 0) for key in GRADS), e
    else:
        assert all(v <= tol for v in errs.values()), (e, errs)
    return errs


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,ntok,nexp", WORKLOADS, ids=[w[0] for w in WORKLOADS])
def test_fullsize_parity(name, ntok, nexp, cuda):
    from grouped_gemm_top_amd import layer
    cfg = config(name)
    _say(f"[fullsize] {name}: s={cfg.s} m={cfg.m} n={cfg.n} E={cfg.E} k={cfg.k} r={cfg.r} "
         f"{cfg.dtype} {cfg.score}")
    inp = make_inputs(cfg, seed=0, device=cuda, with_grad_output=True)
    shape = layer.shape_of(cfg)
    rt = layer.route(shape, inp["X"], inp["W_r"], inp["router_bias"])
    Y, saved = layer.forward(shape, inp["X"], rt, inp, training=True)
    dX, grads = layer.backward(shape, inp["dY"], inp["X"], inp["W_r"], rt, inp, saved)
    torch.cuda.synchronize()
    _say("  GPU pass done")
    tol = TOL[cfg.dtype]

    # ---- routing, in full
    z_gpu = rt["logits"].cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(7)
    Wr = f64(inp["W_r"])
    bias = f64(inp["router_bias"]) if inp["router_bias"] is not None else None
    if ntok == "all":
        tok = np.arange(cfg.s)
    else:
        tok = np.sort(rng.choice(cfg.s, size=ntok, replace=False))
    z_ref = oracle.router_logits(f64(inp["X"][torch.as_tensor(tok, device=cuda)]), Wr, bias)
    assert rel_err(z_gpu[tok], z_ref) <= LOGIT_TOL
    ort = oracle.route(z_gpu, cfg.k, cfg.E, cfg.score, cfg.renormalize)
    assert np.array_equal(rt["topk_idx"].cpu().numpy(), ort["idx"])
    assert np.array_equal(rt["expert_off"].cpu().numpy(), ort["off"])
    assert np.array_equal(rt["perm"].cpu().numpy(), ort["perm"])
    assert np.array_equal(rt["inv_perm"].cpu().numpy(), ort["inv"])
    assert rel_err(rt["topk_w"].cpu().numpy(), ort["w"]) <= WEIGHT_TOL
    cnt = ort["cnt"]
    _say(f"  routing bit-exact; expert load min/mean/max {cnt.min()}/{cnt.mean():.0f}/{cnt.max()}, "
         f"empty experts {(cnt == 0).sum()}")
    Xr, dYr = Rows(inp["X"]), Rows(inp["dY"])

    if ntok == "all":
        # ---- the whole layer: every token of Y and dX, every expert's LoRA gradients
        W = {key: LazyExperts(inp[key]) for key in ("W_gu", "W_d", "A_g", "B_g", "A_u", "B_u", "A_d", "B_d")}
        X64, dY64 = f64(inp["X"]), f64(inp["dY"])
        Y_ref, sv = oracle.forward(X64, W, ort, cfg.alpha, cfg.r)
        e_y = rel_err(f64(Y), Y_ref)
        del Y_ref
        g = oracle.backward(dY64, X64, Wr, W, ort, cfg.alpha, cfg.r, cfg.score, cfg.renormalize, True, sv)
        del sv
        e_dx = rel_err(f64(dX), g["dX"])
        _say(f"  all {cfg.s} tokens: Y {e_y:.2e}, dX {e_dx:.2e}")
        assert e_y <= tol and e_dx <= tol
        worst = {key: 0.0 for key in GRADS}
        for e in range(cfg.E):
            errs = _check_expert_grads(e, cnt, grads, {key: g[key][e] for key in GRADS}, tol)
            for key in GRADS:
                worst[key] = max(worst[key], errs[key])
        _say(f"  all {cfg.E} experts, worst: " + ", ".join(f"{k}={v:.1e}" for k, v in worst.items()))
        return

    # ---- sampled tokens: Y and dX, one expert's weights in host memory at a time
    W = {key: NoCache(inp[key]) for key in ("W_gu", "W_d", "A_g", "B_g", "A_u", "B_u", "A_d", "B_d")}
    y_ref, dx_ref = oracle.token_outputs(tok, Xr, W, ort, cfg.alpha, cfg.r, dYr, Wr, cfg.score,
                                         cfg.renormalize, True)
    tt = torch.as_tensor(tok, device=cuda)
    e_y = rel_err(f64(Y[tt]), y_ref)
    e_dx = rel_err(f64(dX[tt]), dx_ref)
    _say(f"  sampled tokens {len(tok)}: Y {e_y:.2e}, dX {e_dx:.2e}")
    assert e_y <= tol and e_dx <= tol

    # ---- sampled experts: LoRA-factor gradients
    used = np.where(cnt > 0)[0]
    # fewest rows in the last 128-row tile first (129 rows: 1, 128 rows: a full tile)
    ragged = used[np.argsort((cnt[used] - 1) % 128, kind="stable")]
    experts = [int(np.argmax(cnt))] + [int(e) for e in ragged[: nexp // 2]]
    experts += [int(e) for e in rng.choice(cfg.E, size=nexp, replace=False)]
    empty = np.where(cnt == 0)[0]
    if empty.size:
        experts.append(int(empty[0]))
    experts = list(dict.fromkeys(experts))
    assert len(experts) >= nexp
    for e in experts:
        ge = oracle.backward_expert(e, dYr, Xr, W, ort, cfg.alpha, cfg.r)
        errs = _check_expert_grads(e, cnt, grads, ge, tol)
        _say(f"  expert {e} ({cnt[e]} rows): " + ", ".join(f"{k}={v:.1e}" for k, v in errs.items()))


@pytest.mark.timeout(900)
def test_long_context_deepseek_layer(cuda):
    """The DeepSeek-V3 layer at 65 536 tokens (8x the benchmark's batch): 524 288 routed pairs, so the
    grouped activations o, dXp and gu hold up to 3.8e9 elements and their row offsets pass 2^31.
    Routing is checked in full; Y and dX on tokens whose pairs sit in the highest grouped rows (the
    last experts), and the gradients of the last expert and one more, against the oracle in fp64."""
    from grouped_gemm_top_amd import layer
    cfg = config("deepseek_v3", s=65536)
    _say(f"[long context] deepseek_v3 s={cfg.s}: P={cfg.s * cfg.k}")
    inp = make_inputs(cfg, seed=0, device=cuda, with_grad_output=True)
    shape = layer.shape_of(cfg)
    rt = layer.route(shape, inp["X"], inp["W_r"], inp["router_bias"])
    Y, saved = layer.forward(shape, inp["X"], rt, inp, training=True)
    dX, grads = layer.backward(shape, inp["dY"], inp["X"], inp["W_r"], rt, inp, saved)
    torch.cuda.synchronize()
    _say("  GPU pass done")
    del saved
    z_gpu = rt["logits"].cpu().numpy().astype(np.float64)
    ort = oracle.route(z_gpu, cfg.k, cfg.E, cfg.score, cfg.renormalize)
    assert np.array_equal(rt["topk_idx"].cpu().numpy(), ort["idx"])
    assert np.array_equal(rt["expert_off"].cpu().numpy(), ort["off"])
    assert np.array_equal(rt["perm"].cpu().numpy(), ort["perm"])
    assert np.array_equal(rt["inv_perm"].cpu().numpy(), ort["inv"])
    assert rel_err(rt["topk_w"].cpu().numpy(), ort["w"]) <= WEIGHT_TOL
    P = cfg.s * cfg.k
    assert (P - 1) * cfg.m >= 1 << 31
    # tokens holding the last grouped rows (each row's offset in o and dXp is row * m elements)
    top_rows = np.arange(P - 1, P - 6000, -1)
    tok = np.unique(ort["perm"][top_rows] // cfg.k)[-6:]
    tok = np.concatenate([tok, [cfg.s - 1, 0]])
    hi = max(int(ort["inv"][t * cfg.k + j]) for t in tok for j in range(cfg.k))
    _say(f"  tokens {tok.tolist()}, highest grouped row {hi} (offset {hi * cfg.m:.3e} elements)")
    assert hi * cfg.m >= 1 << 31
    W = {key: NoCache(inp[key]) for key in ("W_gu", "W_d", "A_g", "B_g", "A_u", "B_u", "A_d", "B_d")}
    Xr, dYr = Rows(inp["X"]), Rows(inp["dY"])
    Wr = f64(inp["W_r"])
    y_ref, dx_ref = oracle.token_outputs(tok, Xr, W, ort, cfg.alpha, cfg.r, dYr, Wr, cfg.score,
                                         cfg.renormalize, True)
    tt = torch.as_tensor(tok, device=cuda)
    e_y, e_dx = rel_err(f64(Y[tt]), y_ref), rel_err(f64(dX[tt]), dx_ref)
    _say(f"  tokens: Y {e_y:.2e}, dX {e_dx:.2e}")
    tol = TOL[cfg.dtype]
    assert e_y <= tol and e_dx <= tol
    cnt = ort["cnt"]
    for e in (cfg.E - 1, int(np.argmax(cnt))):
        ge = oracle.backward_expert(e, dYr, Xr, W, ort, cfg.alpha, cfg.r)
        errs = _check_expert_grads(e, cnt, grads, ge, tol)
        _say(f"  expert {e} ({cnt[e]} rows): " + ", ".join(f"{k}={v:.1e}" for k, v in errs.items()))
