"""Full-size parity: every workload at its real shape, in the launch configuration the benchmark uses.

Routing is checked in full (ids, offsets, perm, inv bit-exact on the GPU's own logits; weights to
1e-6). Layer outputs are checked on sampled tokens (y_t and dX_t depend only on x_t, dY_t and the
token's k experts) and LoRA gradients on sampled experts (an expert's gradients depend only on its
own rows), computed one by one by the oracle in fp64.
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


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


WORKLOADS = [
    ("qwen3_30b_a3b", 24, 6),
    ("qwen3_30b_a3b_zipf", 24, 6),
    ("gpt_oss_20b", 16, 4),
    ("deepseek_v3", 6, 3),
]


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

    # ---- routing, in full
    z_gpu = rt["logits"].cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(7)
    tok = np.sort(rng.choice(cfg.s, size=ntok, replace=False))
    Xs = f64(inp["X"][torch.as_tensor(tok, device=cuda)])
    Wr = f64(inp["W_r"])
    bias = f64(inp["router_bias"]) if inp["router_bias"] is not None else None
    z_ref = oracle.router_logits(Xs, Wr, bias)
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

    # ---- sampled tokens: Y and dX
    W = {key: LazyExperts(inp[key]) for key in ("W_gu", "W_d", "A_g", "B_g", "A_u", "B_u", "A_d", "B_d")}

    class Rows:  # row access X[t:t+1] / X[idx] on the device tensor, returned as host fp64
        def __init__(self, t):
            self.t = t
            self.shape = tuple(t.shape)

        def __getitem__(self, i):
            if isinstance(i, slice):
                return f64(self.t[i])
            return f64(self.t[torch.as_tensor(np.asarray(i), device=self.t.device)])

    Xr, dYr = Rows(inp["X"]), Rows(inp["dY"])
    y_ref = oracle.forward_tokens(tok, Xr, W, ort, cfg.alpha, cfg.r)
    tol = TOL[cfg.dtype]
    e_y = rel_err(f64(Y[torch.as_tensor(tok, device=cuda)]), y_ref)
    dx_ref = oracle.backward_tokens(tok, dYr, Xr, Wr, W, ort, cfg.alpha, cfg.r, cfg.score,
                                    cfg.renormalize, True)
    e_dx = rel_err(f64(dX[torch.as_tensor(tok, device=cuda)]), dx_ref)
    _say(f"  sampled tokens {len(tok)}: Y {e_y:.2e}, dX {e_dx:.2e}")
    assert e_y <= tol and e_dx <= tol

    # ---- sampled experts: LoRA-factor gradients (the busiest, random ones, and an empty one)
    experts = [int(np.argmax(cnt))] + [int(e) for e in rng.choice(cfg.E, size=nexp, replace=False)]
    empty = np.where(cnt == 0)[0]
    if empty.size:
        experts.append(int(empty[0]))
    for e in dict.fromkeys(experts):
        ge = oracle.backward_expert(e, dYr, Xr, W, ort, cfg.alpha, cfg.r)
        errs = {key: rel_err(grads[key][e].cpu().numpy(), ge[key]) for key in GRADS}
        _say(f"  expert {e} ({cnt[e]} rows): " + ", ".join(f"{k}={v:.1e}" for k, v in errs.items()))
        if cnt[e] == 0:
            assert all(torch.all(grads[key][e] == 0) for key in GRADS)
        else:
            assert all(v <= tol for v in errs.values()), errs
