"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test checks the oracle against something fixed by the pages or by mathematics: a brute-force
sort, the dense-merge form of LoRA the pages compare against, a per-token loop with no grouping,
fp64 central finite differences, closed forms and invariants, and the page's gate/up order.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng0 = np.random.default_rng(1234)


def _rand_layer(rng, s, m, n, E, k, r, scale_w=0.3):
    W = {
        "W_gu": rng.normal(0, scale_w, (E, m, 2 * n)),
        "W_d": rng.normal(0, scale_w, (E, n, m)),
        "A_g": rng.normal(0, 0.5, (E, m, r)), "B_g": rng.normal(0, 0.5, (E, r, n)),
        "A_u": rng.normal(0, 0.5, (E, m, r)), "B_u": rng.normal(0, 0.5, (E, r, n)),
        "A_d": rng.normal(0, 0.5, (E, n, r)), "B_d": rng.normal(0, 0.5, (E, r, m)),
    }
    X = rng.normal(0, 1, (s, m))
    W_r = rng.normal(0, 1, (m, E))
    dY = rng.normal(0, 1, (s, m))
    return X, W_r, W, dY


def _silu(v):
    return v / (1.0 + np.exp(-v))


def _merged(W, e, c):
    """Dense-merged expert weights W + c * A B (the materialised PEFT form)."""
    n = W["W_d"].shape[1]
    Wg = W["W_gu"][e][:, :n] + c * W["A_g"][e] @ W["B_g"][e]
    Wu = W["W_gu"][e][:, n:] + c * W["A_u"][e] @ W["B_u"][e]
    Wd = W["W_d"][e] + c * W["A_d"][e] @ W["B_d"][e]
    return Wg, Wu, Wd


def _min_gap(z, k):
    zs = -np.sort(-z, axis=1)
    return float(np.min(zs[:, k - 1] - zs[:, k])) if z.shape[1] > k else np.inf


# ------------------------------------------------------------------------------- routing

def test_topk_matches_bruteforce_sort():
    rng = np.random.default_rng(7)
    z = rng.integers(-2, 3, size=(300, 12)).astype(np.float64)  # many ties
    k = 5
    idx = oracle.topk_experts(z, k)
    for t in range(z.shape[0]):
        order = sorted(range(z.shape[1]), key=lambda e: (-z[t, e], e))
        assert list(idx[t]) == order[:k]


def test_topk_negative_zero_ties_with_zero():
    z = np.array([[0.0, -0.0, 1.0, -0.0]])
    assert list(oracle.topk_experts(z, 3)[0]) == [2, 0, 1]


def test_all_equal_logits_pick_first_experts_with_equal_weights():
    s, E, k = 5, 8, 4
    z = np.full((s, E), 0.37)
    rt = oracle.route(z, k, E, "softmax")
    assert np.all(rt["idx"] == np.arange(k))
    assert np.all(rt["w"] == 1.0 / k)
    rt = oracle.route(z, k, E, "sigmoid")
    assert np.all(rt["w"] == 1.0 / k)


def test_k_equals_E_renormalisation_is_identity_for_softmax():
    rng = np.random.default_rng(3)
    z = rng.normal(size=(40, 6))
    rt = oracle.route(z, 6, 6, "softmax")
    np.testing.assert_allclose(rt["w"], rt["p_sel"], rtol=1e-14, atol=0)
    # softmax restricted to the k selected logits equals the renormalised weights
    zs = np.take_along_axis(z, rt["idx"].astype(np.int64), 1)
    ref = np.exp(zs) / np.exp(zs).sum(1, keepdims=True)
    np.testing.assert_allclose(rt["w"], ref, rtol=1e-13)


def test_sigmoid_scores_closed_form():
    z = np.array([[0.0, math.log(3.0), -1.0, 2.0]])
    rt = oracle.route(z, 2, 4, "sigmoid", renormalize=False)
    assert list(rt["idx"][0]) == [3, 1]
    np.testing.assert_allclose(rt["w"][0], [1 / (1 + math.exp(-2.0)), 0.75], rtol=1e-15)


def test_grouping_invariants():
    rng = np.random.default_rng(11)
    s, E, k = 257, 13, 3
    z = rng.normal(size=(s, E))
    z[:, 4] -= 10.0  # expert 4 never selected
    rt = oracle.route(z, k, E)
    idx, cnt, off, perm, inv = rt["idx"], rt["cnt"], rt["off"], rt["perm"], rt["inv"]
    P = s * k
    assert cnt.sum() == P and off[0] == 0 and off[E] == P and cnt[4] == 0
    assert np.all(np.diff(off) == cnt)
    assert sorted(perm.tolist()) == list(range(P))
    for i in range(P):
        assert inv[perm[i]] == i
    for e in range(E):
        rows = perm[off[e]:off[e + 1]]
        assert all(idx.reshape(-1)[p] == e for p in rows)
        toks = [p // k for p in rows]
        assert all(a < b for a, b in zip(toks, toks[1:]))
    for t in range(s):
        assert len(set(idx[t].tolist())) == k
    assert np.max(np.abs(rt["w"].sum(1) - 1.0)) <= k * 2.0 ** -52


# ------------------------------------------------------------------------------- forward

# ------------------------------------------------------------------------ router bias
# The skewed-routing workload adds a fixed per-expert bias beta to the logits,
# beta_e = -zipf * ln(rank_e), so that the bias alone gives a Zipf law on the experts. These pins
# tie the oracle's logits to that law and to properties of softmax, so that a dropped or negated
# bias fails.

def test_router_bias_alone_gives_the_zipf_law():
    rng = np.random.default_rng(21)
    s, m, E, a = 7, 16, 12, 1.2
    rank = rng.permutation(E) + 1.0
    beta = -a * np.log(rank)
    X = rng.normal(size=(s, m))
    z = oracle.router_logits(X, np.zeros((m, E)), beta)
    rt = oracle.route(z, E, E, "softmax")           # k = E: every expert, weights = softmax
    zipf = rank ** -a / np.sum(rank ** -a)
    for t in range(s):
        assert list(rt["idx"][t]) == list(np.argsort(rank))  # rank 1 first
        np.testing.assert_allclose(rt["p_sel"][t], zipf[rt["idx"][t]], rtol=1e-13, atol=0)


def test_router_bias_shift_leaves_softmax_routing_unchanged():
    rng = np.random.default_rng(22)
    s, m, E, k = 40, 24, 10, 3
    X, W_r = rng.normal(size=(s, m)), rng.normal(size=(m, E))
    beta = rng.normal(size=E)
    a = oracle.route(oracle.router_logits(X, W_r, beta), k, E, "softmax")
    b = oracle.route(oracle.router_logits(X, W_r, beta + 3.25), k, E, "softmax")
    assert np.array_equal(a["idx"], b["idx"])
    np.testing.assert_allclose(a["w"], b["w"], rtol=1e-12, atol=0)
    # and the bias does act: the logits move by exactly beta against the unbiased ones
    z0 = oracle.router_logits(X, W_r)
    np.testing.assert_allclose(oracle.router_logits(X, W_r, beta) - z0, np.tile(beta, (s, 1)),
                               rtol=0, atol=1e-12)


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_large_positive_bias_puts_its_expert_first(score):
    rng = np.random.default_rng(23)
    s, m, E, k, j = 50, 16, 9, 3, 6
    X, W_r = rng.normal(size=(s, m)), rng.normal(size=(m, E))
    beta = np.zeros(E)
    beta[j] = 100.0
    rt = oracle.route(oracle.router_logits(X, W_r, beta), k, E, score)
    assert np.all(rt["idx"][:, 0] == j)
    assert np.all(rt["w"][:, 0] > 1.0 / k)


# ------------------------------------------------------------------------ non-numbers
# Reading: a NaN logit counts as -inf (never selected before a number, score 0).

def test_nan_logits_rank_below_numbers_and_ids_stay_valid():
    rng = np.random.default_rng(24)
    s, E, k = 30, 7, 3
    z = rng.normal(size=(s, E))
    z[:, 2] = np.nan                       # a NaN column: never selected while numbers remain
    z[5, :] = np.nan                       # a NaN row: all ties at -inf -> experts 0..k-1
    z[9, :5] = np.nan                      # fewer numbers than... still k of them
    rt = oracle.route(z, k, E, "softmax")
    idx = rt["idx"]
    assert idx.min() >= 0 and idx.max() < E
    assert all(len(set(r.tolist())) == k for r in idx)
    assert list(idx[5]) == [0, 1, 2]
    assert set(idx[9].tolist()) <= {5, 6, 0}  # the two numbers first, then the lowest NaN id
    assert list(idx[9][:2]) == list(np.argsort(-z[9, 5:])[:2] + 5)
    for t in range(s):
        if t not in (5, 9):
            assert 2 not in idx[t]
            # unaffected tokens: the same selection and weights as with the column removed
            keep = [e for e in range(E) if e != 2]
            sub = oracle.route(z[t:t + 1, keep], k, E - 1, "softmax")
            assert [keep[e] for e in sub["idx"][0]] == list(idx[t])
            np.testing.assert_allclose(sub["w"][0], rt["w"][t], rtol=1e-14, atol=0)


def test_gate_up_order_closed_form():
    fx = json.load(open(os.path.join(GOLDEN, "swiglu_gate_first.json")))
    m = n = 64
    r = 8
    W = {key: np.zeros(shape) for key, shape in
         (("W_gu", (1, m, 2 * n)), ("W_d", (1, n, m)), ("A_g", (1, m, r)), ("B_g", (1, r, n)),
          ("A_u", (1, m, r)), ("B_u", (1, r, n)), ("A_d", (1, n, r)), ("B_d", (1, r, m)))}
    W["W_gu"][0, 0, :n] = fx["gate"]
    W["W_gu"][0, 0, n:] = fx["up"]
    W["W_d"][0] = np.eye(n, m)
    X = np.zeros((1, m))
    X[0, 0] = 1.0
    rt = oracle.route(np.zeros((1, 1)), 1, 1)
    Y, saved = oracle.forward(X, W, rt, alpha=16.0, r=r)
    np.testing.assert_allclose(saved["h"][0], fx["expected_h"], rtol=1e-15)
    np.testing.assert_allclose(Y[0, :n], fx["expected_h"], rtol=1e-15)


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_split_lora_equals_dense_merge_and_per_token_loop(score):
    """Split LoRA (X W + c (X A) B) against the materialised form X (W + c A B), evaluated one
    token at a time over its k experts with no grouping (the per-expert loop semantics)."""
    rng = np.random.default_rng(5)
    s, m, n, E, k, r, alpha = 37, 16, 8, 5, 2, 3, 6.0
    X, W_r, W, _ = _rand_layer(rng, s, m, n, E, k, r)
    c = alpha / r
    rt = oracle.route(oracle.router_logits(X, W_r), k, E, score)
    Y, _ = oracle.forward(X, W, rt, alpha, r)
    ref = np.zeros((s, m))
    for t in range(s):
        for j in range(k):
            Wg, Wu, Wd = _merged(W, int(rt["idx"][t, j]), c)
            x = X[t]
            ref[t] += rt["w"][t, j] * ((_silu(x @ Wg) * (x @ Wu)) @ Wd)
    np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("rslora", [False, True], ids=["alpha_over_r", "rslora"])
def test_merged_weights_give_the_split_lora_forward(rslora):
    """merged_weights (the materialised W + c A B) against the Split-LoRA forward: the layer on the
    merged weights with zero low-rank factors equals the layer on the split weights (associativity of
    X W + c (X A) B), for the per-projection pairs and for one fused gate/up pair."""
    rng = np.random.default_rng(12)
    s, m, n, E, k, r, alpha = 31, 16, 8, 5, 2, 3, 6.0
    X, W_r, W, _ = _rand_layer(rng, s, m, n, E, k, r)
    rt = oracle.route(oracle.router_logits(X, W_r), k, E)
    for Wsplit in (W, dict(W, **oracle.fused_gate_up_pair(W["A_g"], np.concatenate([W["B_g"], W["B_u"]], axis=-1)))):
        Y, _ = oracle.forward(X, Wsplit, rt, alpha, r, keep=False, rslora=rslora)
        if Wsplit is W:
            Wm = oracle.merged_weights(W, alpha, r, rslora)
        else:  # the fused pair given as one [m, r] x [r, 2n] product
            Wm = oracle.merged_weights(dict(W, A_u=None, B_u=None,
                                            B_g=np.concatenate([W["B_g"], W["B_u"]], axis=-1)), alpha, r, rslora)
        zero = {key: np.zeros_like(W[key]) for key in ("A_g", "B_g", "A_u", "B_u", "A_d", "B_d")}
        Ym, _ = oracle.forward(X, dict(zero, W_gu=Wm["W_gu"], W_d=Wm["W_d"]), rt, alpha, r, keep=False,
                               rslora=rslora)
        np.testing.assert_allclose(Ym, Y, rtol=1e-12, atol=1e-12 * np.abs(Y).max())


def test_rslora_scale_is_alpha_over_sqrt_r():
    """Rank-stabilised LoRA (bluecore.net/archives/629, LoRA section, rsLoRA item) scales the
    low-rank update by alpha/sqrt(r): the forward equals the dense merge with that scale, and the
    backward equals the plain-scale one at the alpha that gives the same c."""
    rng = np.random.default_rng(6)
    s, m, n, E, k, r, alpha = 29, 16, 8, 4, 2, 4, 6.0
    X, W_r, W, dY = _rand_layer(rng, s, m, n, E, k, r)
    c = alpha / math.sqrt(r)
    rt = oracle.route(oracle.router_logits(X, W_r), k, E)
    Y, sv = oracle.forward(X, W, rt, alpha, r, rslora=True)
    ref = np.zeros((s, m))
    for t in range(s):
        for j in range(k):
            Wg, Wu, Wd = _merged(W, int(rt["idx"][t, j]), c)
            x = X[t]
            ref[t] += rt["w"][t, j] * ((_silu(x @ Wg) * (x @ Wu)) @ Wd)
    np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    assert oracle.lora_scale(alpha, r, True) == c and oracle.lora_scale(alpha, r) == alpha / r
    # backward: the same as the plain-scale oracle at alpha' = alpha sqrt(r) (same c)
    g = oracle.backward(dY, X, W_r, W, rt, alpha, r, saved=sv, rslora=True)
    g2 = oracle.backward(dY, X, W_r, W, rt, alpha * math.sqrt(r), r)
    for key in ("dX", "dA_g", "dB_g", "dA_u", "dB_u", "dA_d", "dB_d"):
        np.testing.assert_allclose(g[key], g2[key], rtol=1e-12, atol=1e-12 * np.abs(g2[key]).max())


def test_single_expert_is_a_dense_swiglu_mlp():
    rng = np.random.default_rng(9)
    s, m, n, r, alpha = 11, 12, 6, 2, 4.0
    X, W_r, W, _ = _rand_layer(rng, s, m, n, 1, 1, r)
    rt = oracle.route(oracle.router_logits(X, W_r), 1, 1)
    assert np.all(rt["w"] == 1.0)
    Y, _ = oracle.forward(X, W, rt, alpha, r)
    Wg, Wu, Wd = _merged(W, 0, alpha / r)
    np.testing.assert_allclose(Y, (_silu(X @ Wg) * (X @ Wu)) @ Wd, rtol=1e-12, atol=1e-13)


def test_alpha_zero_is_plain_moe_and_freezes_lora():
    rng = np.random.default_rng(10)
    s, m, n, E, k, r = 20, 8, 4, 4, 2, 2
    X, W_r, W, dY = _rand_layer(rng, s, m, n, E, k, r)
    rt = oracle.route(oracle.router_logits(X, W_r), k, E)
    Y0, sv = oracle.forward(X, W, rt, 0.0, r)
    Wz = dict(W)
    for key in ("B_g", "B_u", "B_d"):
        Wz[key] = np.zeros_like(W[key])
    Yb, _ = oracle.forward(X, Wz, rt, 5.0, r)
    np.testing.assert_allclose(Y0, Yb, rtol=1e-14, atol=0)
    g = oracle.backward(dY, X, W_r, W, rt, 0.0, r, saved=sv)
    for key in ("dA_g", "dB_g", "dA_u", "dB_u", "dA_d", "dB_d"):
        assert np.all(g[key] == 0.0)


def test_zero_B_gives_zero_dA_but_nonzero_dB():
    rng = np.random.default_rng(12)
    s, m, n, E, k, r = 20, 8, 4, 3, 2, 2
    X, W_r, W, dY = _rand_layer(rng, s, m, n, E, k, r)
    for key in ("B_g", "B_u", "B_d"):
        W[key] = np.zeros_like(W[key])
    rt = oracle.route(oracle.router_logits(X, W_r), k, E)
    g = oracle.backward(dY, X, W_r, W, rt, 4.0, r)
    for key in ("dA_g", "dA_u", "dA_d"):
        assert np.all(g[key] == 0.0)
    for key in ("dB_g", "dB_u", "dB_d"):
        assert np.abs(g[key]).max() > 1e-3


def test_zero_token_expert_has_exact_zero_gradients():
    rng = np.random.default_rng(13)
    s, m, n, E, k, r = 30, 8, 4, 5, 2, 2
    X, W_r, W, dY = _rand_layer(rng, s, m, n, E, k, r)
    z = oracle.router_logits(X, W_r)
    z[:, 2] = -1e3
    rt = oracle.route(z, k, E)
    assert rt["cnt"][2] == 0
    g = oracle.backward(dY, X, W_r, W, rt, 2.0, r)
    for key in ("dA_g", "dB_g", "dA_u", "dB_u", "dA_d", "dB_d"):
        assert np.all(g[key][2] == 0.0)


# ------------------------------------------------------------------------------- backward

def _loss(X, W_r, W, dY, k, E, alpha, r, score, renorm, frozen_rt=None):
    rt = frozen_rt if frozen_rt is not None else oracle.route(oracle.router_logits(X, W_r), k, E,
                                                               score, renorm)
    Y, _ = oracle.forward(X, W, rt, alpha, r, keep=False)
    return float(np.sum(dY * Y)), rt


@pytest.mark.parametrize("score,renorm", [("softmax", True), ("sigmoid", True), ("sigmoid", False)])
def test_gradients_match_central_finite_differences(score, renorm):
    rng = np.random.default_rng(21)
    s, m, n, E, k, r, alpha = 6, 8, 4, 4, 2, 2, 3.0
    for _ in range(50):
        X, W_r, W, dY = _rand_layer(rng, s, m, n, E, k, r)
        if _min_gap(oracle.router_logits(X, W_r), k) > 1e-2:
            break
    base_rt = oracle.route(oracle.router_logits(X, W_r), k, E, score, renorm)
    g = oracle.backward(dY, X, W_r, W, base_rt, alpha, r, score, renorm, router_grad=True)
    g0 = oracle.backward(dY, X, W_r, W, base_rt, alpha, r, score, renorm, router_grad=False)
    h = 1e-6

    def fd(arr, frozen):
        out = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            old = arr[i]
            arr[i] = old + h
            lp, rtp = _loss(X, W_r, W, dY, k, E, alpha, r, score, renorm, frozen)
            arr[i] = old - h
            lm, rtm = _loss(X, W_r, W, dY, k, E, alpha, r, score, renorm, frozen)
            arr[i] = old
            if frozen is None:
                assert np.array_equal(rtp["idx"], base_rt["idx"])
                assert np.array_equal(rtm["idx"], base_rt["idx"])
            out[i] = (lp - lm) / (2 * h)
        return out

    def close(a, b):
        return np.max(np.abs(a - b)) <= 1e-6 * max(np.max(np.abs(b)), 1e-3)

    assert close(g["dX"], fd(X, None)), "dX with the router path"
    assert close(g0["dX"], fd(X, base_rt)), "dX through the experts only"
    for key in ("A_g", "B_g", "A_u", "B_u", "A_d", "B_d"):
        assert close(g["d" + key], fd(W[key], base_rt)), key


def test_lora_grads_equal_projected_dense_weight_gradient():
    """With W' = W + c A B, dA = c (dL/dW') B^T and dB = c A^T (dL/dW'); dL/dW' = X_e^T dG_e."""
    rng = np.random.default_rng(31)
    s, m, n, E, k, r, alpha = 25, 8, 6, 3, 2, 2, 5.0
    c = alpha / r
    X, W_r, W, dY = _rand_layer(rng, s, m, n, E, k, r)
    rt = oracle.route(oracle.router_logits(X, W_r), k, E)
    g = oracle.backward(dY, X, W_r, W, rt, alpha, r)
    Xp = X[rt["perm"] // k]
    tok, slot = rt["perm"] // k, rt["perm"] % k
    dO = rt["w"][tok, slot][:, None] * dY[tok]
    for e in range(E):
        a, b = rt["off"][e], rt["off"][e + 1]
        ew = oracle._expert(W, e)
        f = oracle.expert_rows_forward(Xp[a:b], ew, c)
        res = oracle.expert_rows_backward(Xp[a:b], dO[a:b], ew, c, f)
        dWg = Xp[a:b].T @ res["dg"]
        dWd = f["h"].T @ dO[a:b]
        np.testing.assert_allclose(g["dA_g"][e], c * dWg @ W["B_g"][e].T, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(g["dB_g"][e], c * W["A_g"][e].T @ dWg, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(g["dA_d"][e], c * dWd @ W["B_d"][e].T, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(g["dB_d"][e], c * W["A_d"][e].T @ dWd, rtol=1e-12, atol=1e-14)


def test_softmax_router_gradient_sums_to_zero_per_token():
    rng = np.random.default_rng(41)
    s, m, n, E, k, r = 40, 8, 4, 6, 3, 2
    X, W_r, W, dY = _rand_layer(rng, s, m, n, E, k, r)
    rt = oracle.route(oracle.router_logits(X, W_r), k, E)
    g = oracle.backward(dY, X, W_r, W, rt, 2.0, r)
    assert np.max(np.abs(g["dz"].sum(1))) <= 1e-14 * np.abs(g["dz"]).max() * k


# ------------------------------------------------------------------------------- sampled outputs

def test_sampled_outputs_equal_full_layer():
    rng = np.random.default_rng(51)
    s, m, n, E, k, r, alpha = 30, 8, 4, 5, 2, 2, 4.0
    X, W_r, W, dY = _rand_layer(rng, s, m, n, E, k, r)
    for score in ("softmax", "sigmoid"):
        rt = oracle.route(oracle.router_logits(X, W_r), k, E, score)
        Y, sv = oracle.forward(X, W, rt, alpha, r)
        g = oracle.backward(dY, X, W_r, W, rt, alpha, r, score, True, True, sv)
        toks = [0, 7, 29]
        np.testing.assert_allclose(oracle.forward_tokens(toks, X, W, rt, alpha, r), Y[toks],
                                   rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(
            oracle.backward_tokens(toks, dY, X, W_r, W, rt, alpha, r, score), g["dX"][toks],
            rtol=1e-12, atol=1e-14)
        yt, dxt = oracle.token_outputs(toks, X, W, rt, alpha, r, dY, W_r, score)
        np.testing.assert_allclose(yt, Y[toks], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(dxt, g["dX"][toks], rtol=1e-12, atol=1e-14)
        for e in range(E):
            ge = oracle.backward_expert(e, dY, X, W, rt, alpha, r)
            for key, v in ge.items():
                np.testing.assert_allclose(v, g[key][e], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------ fused gate/up LoRA pair

def test_fused_gate_up_pair_equals_dense_merge():
    """One pair on gate_up_proj: y equals the per-token loop over W_gu + c A B (2n columns at once)."""
    rng = np.random.default_rng(41)
    s, m, n, E, k, r, alpha = 20, 8, 6, 3, 2, 2, 5.0
    c = alpha / r
    X, W_r, W, _ = _rand_layer(rng, s, m, n, E, k, r)
    A = rng.normal(0, 0.5, (E, m, r))
    B = rng.normal(0, 0.5, (E, r, 2 * n))
    W.update(oracle.fused_gate_up_pair(A, B))
    rt = oracle.route(oracle.router_logits(X, W_r), k, E)
    Y, _ = oracle.forward(X, W, rt, alpha, r, keep=False)
    ref = np.zeros((s, m))
    for t in range(s):
        for j in range(k):
            e = rt["idx"][t, j]
            gu = X[t] @ (W["W_gu"][e] + c * A[e] @ B[e])
            h = _silu(gu[:n]) * gu[n:]
            ref[t] += rt["w"][t, j] * (h @ (W["W_d"][e] + c * W["A_d"][e] @ W["B_d"][e]))
    np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-12)


def test_fused_gate_up_grads_match_central_finite_differences():
    """dA, dB of the fused pair (summed / concatenated from the per-projection gradients) equal fp64
    central differences of the loss taken with respect to the fused A and B themselves."""
    rng = np.random.default_rng(43)
    s, m, n, E, k, r, alpha = 6, 8, 4, 3, 2, 2, 3.0
    X, W_r, W, dY = _rand_layer(rng, s, m, n, E, k, r)
    A = rng.normal(0, 0.5, (E, m, r))
    B = rng.normal(0, 0.5, (E, r, 2 * n))
    rt = oracle.route(oracle.router_logits(X, W_r), k, E)

    def loss():
        Wf = dict(W, **oracle.fused_gate_up_pair(A, B))
        Y, _ = oracle.forward(X, Wf, rt, alpha, r, keep=False)
        return float(np.sum(dY * Y))

    g = oracle.backward(dY, X, W_r, dict(W, **oracle.fused_gate_up_pair(A, B)), rt, alpha, r)
    dA, dB = oracle.fused_gate_up_grads(g)
    h = 1e-6
    for arr, got in ((A, dA), (B, dB)):
        fd = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            old = arr[i]
            arr[i] = old + h
            lp = loss()
            arr[i] = old - h
            lm = loss()
            arr[i] = old
            fd[i] = (lp - lm) / (2 * h)
        assert got.shape == arr.shape
        assert np.max(np.abs(got - fd)) <= 1e-6 * max(np.max(np.abs(fd)), 1e-3)


# ------------------------------------------------------------------------------ shared expert

def test_shared_expert_is_the_routed_layer_with_one_expert_and_plain_mlp():
    """The shared expert equals the routed layer with E = k = 1 (weight 1 for every token), and the
    textbook SwiGLU MLP on merged weights; its gradients match fp64 central differences."""
    rng = np.random.default_rng(47)
    s, m, n, r, alpha = 7, 8, 4, 2, 3.0
    c = alpha / r
    X, W_r, W, dY = _rand_layer(rng, s, m, n, 1, 1, r)
    W1 = {k: v[0] for k, v in W.items()}
    f = oracle.shared_expert_forward(X, W1, alpha, r)
    rt = oracle.route(oracle.router_logits(X, W_r), 1, 1)
    Y, _ = oracle.forward(X, W, rt, alpha, r, keep=False)
    np.testing.assert_allclose(f["o"], Y, rtol=1e-13, atol=1e-13)
    Wg, Wu, Wd = _merged(W, 0, c)
    dense = (_silu(X @ Wg) * (X @ Wu)) @ Wd
    np.testing.assert_allclose(f["o"], dense, rtol=1e-12, atol=1e-12)
    g = oracle.shared_expert_backward(dY, X, W1, alpha, r)
    h = 1e-6

    def loss():
        return float(np.sum(dY * oracle.shared_expert_forward(X, W1, alpha, r)["o"]))

    for key, arr in (("dX", X), ("dA_g", W1["A_g"]), ("dB_u", W1["B_u"]), ("dA_d", W1["A_d"]),
                     ("dB_d", W1["B_d"])):
        fd = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            old = arr[i]
            arr[i] = old + h
            lp = loss()
            arr[i] = old - h
            lm = loss()
            arr[i] = old
            fd[i] = (lp - lm) / (2 * h)
        assert np.max(np.abs(g[key] - fd)) <= 1e-6 * max(np.max(np.abs(fd)), 1e-3), key
