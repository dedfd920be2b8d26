"""CPU oracle for the MoE-LoRA expert layer (test infrastructure, not part of the product).

A plain, slow, fp64 numpy restatement of what the layer computes, used only by the tests,
the smoke check and the benchmark's CPU-baseline leg. It shares no code with the HIP library
and imports nothing from it. Each function cites the passage it follows:

  [ALK] ailinkdeeptech.com cookbook page "Accelerating Mixture-of-Experts Fine-Tuning: Unsloth
        Faster MoE, Split LoRA, and Grouped GEMM".
  [UNS] unsloth.ai documentation page "Faster MoE" (Japanese edition, titled
        "UnslothでMoEモデルを12倍高速に微調整する"; German and French editions carry the same text).

Readings taken where the pages are silent (each is listed with its reason in the design notes):
  * Router: softmax over all E logits, keep the top k, renormalise the k kept weights; the
    sigmoid variant scores each logit with 1/(1+exp(-z)) and renormalises the same way.
  * Top-k selection compares logits, larger first; equal logits go to the lower expert id.
    The slot order j of a token is its selection order. A NaN logit counts as -inf.
  * LoRA update of an expert projection W (x.W orientation, W in R^{m x n}) is
    (alpha/r) * (x A) B with A in R^{m x r}, B in R^{r x n}.
  * Gate/up: gate_up = [gate | up] along the output axis, h = silu(gate) * up.
  * Backward: base weights and router are frozen; gradients are dX, dA_*, dB_*. dX includes the
    path through the routing weights (top-k set held fixed) unless router_grad is off.
  * Pairs are grouped by expert, token order ascending inside a group.

Parity pins (tests/test_oracle_pins.py): dense-merge equivalence, a per-token brute-force loop,
fp64 central finite differences for every gradient, brute-force sorting for top-k, textbook
special cases and invariants. The bf16 rounding of the GPU path has no pin beyond the stated
tolerance.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "router_logits", "nan_as_neg_inf", "topk_experts", "routing_weights", "group_by_expert", "route",
    "silu", "expert_rows_forward", "expert_rows_backward", "forward", "router_backward",
    "backward", "forward_tokens", "backward_tokens", "token_outputs", "backward_expert", "merged_weights",
    "fused_gate_up_pair",
    "fused_gate_up_grads", "shared_expert_forward", "shared_expert_backward",
]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------- routing

def router_logits(X, W_r, bias=None) -> np.ndarray:
    """Gating logits z = x_t W_r (+ a fixed per-expert bias), one row per token.

    [ALK] section "The Dynamic Dispatch Bottleneck in Mixture-of-Experts Architectures",
    routing equation (the router applies W_r to x_t).
    """
    z = _f64(X) @ _f64(W_r)
    if bias is not None:
        z = z + _f64(bias)[None, :]
    return z


def nan_as_neg_inf(z) -> np.ndarray:
    """Logits with every NaN replaced by -inf.

    The pages say nothing of non-numbers. Reading taken: a NaN logit (say from a NaN in x_t or
    in a column of W_r) counts as -inf, so it is never selected before a number and its score is
    0 under softmax and under sigmoid. Infinite logits keep their value.
    """
    z = np.array(z, dtype=np.float64, copy=True)
    z[np.isnan(z)] = -np.inf
    return z


def topk_experts(z, k: int) -> np.ndarray:
    """Indices of the k largest logits per token, in selection order.

    [ALK] routing equation, Top-k(.) over the router scores. Softmax and sigmoid are both
    increasing, so ranking the logits ranks the scores; ties go to the lower expert id
    (a stable sort keeps equal keys in index order). A NaN logit ranks as -inf (nan_as_neg_inf).
    """
    z = nan_as_neg_inf(z)
    s, E = z.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    order = np.argsort(-z, axis=1, kind="stable")  # descending logits, equal ones by id
    return order[:, :k].astype(np.int32)


def routing_weights(z, idx, score: str = "softmax", renormalize: bool = True):
    """Routing weights s_{t,j} of the selected experts, plus their raw scores p_sel.

    [ALK] routing equation: Softmax(x_t W_r) scores, weights s_{t,i} on the selected experts.
    softmax: p = exp(z - max z) / sum over all E; sigmoid: p = 1 / (1 + exp(-z)).
    With renormalize, s_{t,j} = p_j / sum_{j'} p_{j'} over the token's k selected experts.
    """
    z = nan_as_neg_inf(z)
    if score == "softmax":
        zmax = z.max(axis=1, keepdims=True)
        with np.errstate(invalid="ignore"):  # a token whose logits are all -inf: NaN weights
            ex = np.exp(z - zmax)
        p = ex / ex.sum(axis=1, keepdims=True)
        p_sel = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    elif score == "sigmoid":
        z_sel = np.take_along_axis(z, idx.astype(np.int64), axis=1)
        p_sel = 1.0 / (1.0 + np.exp(-z_sel))
    else:
        raise ValueError(score)
    w = p_sel / p_sel.sum(axis=1, keepdims=True) if renormalize else p_sel.copy()
    return w, p_sel


def group_by_expert(idx, E: int):
    """Contiguous per-expert groups of the token-expert pairs.

    Pair id p = t*k + j. Returns cnt [E], off [E+1] (exclusive prefix sum of cnt), perm [P]
    (group row -> pair id; expert ascending, token ascending inside an expert) and inv [P]
    (pair id -> group row). This is the grouping that grouped-GEMM execution over
    variable-sized expert groups relies on ([ALK] "Unsloth Faster MoE resolves these
    bottlenecks via ... grouped GEMM execution"; [UNS] section on torch._grouped_mm, which
    replaces the loop over experts).
    """
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    P = flat.size
    cnt = np.zeros(E, dtype=np.int64)
    for e in flat:
        cnt[e] += 1
    off = np.zeros(E + 1, dtype=np.int64)
    off[1:] = np.cumsum(cnt)
    # counting sort, visiting pairs in increasing pair id (= increasing token, since a token
    # holds at most one pair per expert)
    nxt = off[:-1].copy()
    perm = np.empty(P, dtype=np.int64)
    for p in range(P):
        e = flat[p]
        perm[nxt[e]] = p
        nxt[e] += 1
    inv = np.empty(P, dtype=np.int64)
    inv[perm] = np.arange(P)
    return cnt.astype(np.int32), off.astype(np.int32), perm.astype(np.int32), inv.astype(np.int32)


def route(z, k: int, E: int, score: str = "softmax", renormalize: bool = True) -> dict:
    """Selection, weights and grouping from given logits (steps of the routing equation)."""
    idx = topk_experts(z, k)
    w, p_sel = routing_weights(z, idx, score, renormalize)
    cnt, off, perm, inv = group_by_expert(idx, E)
    return dict(idx=idx, w=w, p_sel=p_sel, cnt=cnt, off=off, perm=perm, inv=inv, k=k, E=E)


# ----------------------------------------------------------------------------- expert MLP

def silu(v):
    return v / (1.0 + np.exp(-v))


def _expert(W, e):
    n = W["W_d"].shape[1]
    Wgu = _f64(W["W_gu"][e])
    return dict(W_g=Wgu[:, :n], W_u=Wgu[:, n:], W_d=_f64(W["W_d"][e]),
                A_g=_f64(W["A_g"][e]), B_g=_f64(W["B_g"][e]),
                A_u=_f64(W["A_u"][e]), B_u=_f64(W["B_u"][e]),
                A_d=_f64(W["A_d"][e]), B_d=_f64(W["B_d"][e]))


def expert_rows_forward(Xr, ew: dict, c: float) -> dict:
    """Expert MLP with Split LoRA on a block of rows routed to one expert.

    Split LoRA [ALK] section "2. Split LoRA Associative Transformation": Y = XW + (alpha/r)(XA)B,
    step 1 H_low = XA, step 2 H_low B, never forming the m x n product of the factors.
    Gate and up are the two halves of the fused gate_up projection, gate first ([UNS] section
    on torch._grouped_mm: linear with gate_up_proj, then chunk(2) into gate, up); the expert
    output is the down projection of silu(gate) * up, with its own Split-LoRA pair.
    """
    Xr = _f64(Xr)
    T_g = Xr @ ew["A_g"]
    T_u = Xr @ ew["A_u"]
    g = Xr @ ew["W_g"] + c * (T_g @ ew["B_g"])
    u = Xr @ ew["W_u"] + c * (T_u @ ew["B_u"])
    h = silu(g) * u
    T_d = h @ ew["A_d"]
    o = h @ ew["W_d"] + c * (T_d @ ew["B_d"])
    return dict(g=g, u=u, h=h, T_g=T_g, T_u=T_u, T_d=T_d, o=o)


def expert_rows_backward(Xr, dO, ew: dict, c: float, fwd: dict | None = None) -> dict:
    """Gradients of one expert's rows: dX rows and this expert's LoRA factor gradients.

    Only the LoRA factors train; the base expert weights are frozen ([UNS] section
    "Implementation details": LoRA tracks gradients for m*r + r*n parameters instead of m*n).
    Chain rule through o = h W_d + c (h A_d) B_d and [g|u] = x W_gu + c [(x A_g) B_g | (x A_u) B_u],
    h = silu(g) u, with silu'(g) = sigma(g) (1 + g (1 - sigma(g))).
    """
    Xr = _f64(Xr)
    dO = _f64(dO)
    f = fwd if fwd is not None else expert_rows_forward(Xr, ew, c)
    g, u, h = f["g"], f["u"], f["h"]
    # down projection
    dT_d = c * (dO @ ew["B_d"].T)
    dh = dO @ ew["W_d"].T + dT_d @ ew["A_d"].T
    dA_d = h.T @ dT_d
    dB_d = c * (f["T_d"].T @ dO)
    # SwiGLU
    sg = 1.0 / (1.0 + np.exp(-g))
    dg = dh * u * sg * (1.0 + g * (1.0 - sg))
    du = dh * g * sg
    # gate / up projections
    dT_g = c * (dg @ ew["B_g"].T)
    dT_u = c * (du @ ew["B_u"].T)
    dX = dg @ ew["W_g"].T + du @ ew["W_u"].T + dT_g @ ew["A_g"].T + dT_u @ ew["A_u"].T
    dA_g = Xr.T @ dT_g
    dB_g = c * (f["T_g"].T @ dg)
    dA_u = Xr.T @ dT_u
    dB_u = c * (f["T_u"].T @ du)
    return dict(dX=dX, dA_g=dA_g, dB_g=dB_g, dA_u=dA_u, dB_u=dB_u, dA_d=dA_d, dB_d=dB_d,
                dh=dh, dg=dg, du=du)


# ----------------------------------------------------------------------------- layer

def lora_scale(alpha: float, r: int, rslora: bool = False) -> float:
    """The LoRA scale c: alpha/r (Split LoRA [ALK] section "2. Split LoRA Associative
    Transformation"), or alpha/sqrt(r) for rank-stabilised LoRA (bluecore.net/archives/629,
    LoRA section, rsLoRA item)."""
    return alpha / np.sqrt(r) if rslora else alpha / r


def forward(X, W: dict, rt: dict, alpha: float, r: int, keep: bool = True, rslora: bool = False):
    """Layer output y_t = sum_j s_{t,j} Expert_{e_{t,j}}(x_t), evaluated over expert groups.

    [ALK] routing equation; experts run per contiguous group (perm), the combine sums the
    token's k rows in slot order. Returns (Y, saved) where saved holds the per-row
    intermediates (rows in group order) when keep is set.
    """
    X = _f64(X)
    c = lora_scale(alpha, r, rslora)
    k, E = rt["k"], rt["E"]
    s, m = X.shape
    P = s * k
    perm, inv, off, w = rt["perm"], rt["inv"], rt["off"], rt["w"]
    Xp = X[perm // k]
    o = np.zeros((P, m))
    saved = {}
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        f = expert_rows_forward(Xp[a:b], _expert(W, e), c)
        o[a:b] = f["o"]
        if keep:
            for key, v in f.items():
                if key not in saved:
                    saved[key] = np.zeros((P, v.shape[1]))
                saved[key][a:b] = v
    Y = np.zeros((s, m))
    tok = np.arange(s)
    for j in range(k):
        Y += w[:, j:j + 1] * o[inv[tok * k + j]]
    saved["o"] = o
    return Y, saved


def merged_weights(W: dict, alpha: float, r: int, rslora: bool = False) -> dict:
    """The materialised PEFT weights W + c A B of every expert: the dense form against which the pages
    set the Split-LoRA evaluation order ([ALK] section "2. Split LoRA Associative Transformation";
    the scale c is lora_scale's). Gate columns first, as in W_gu. With one fused gate/up pair
    (A_u and B_u absent) the update is c A_g B_g over all 2n columns ([UNS] section "Faster LoRA MoE
    training"). Returns fp64 {"W_gu": [E, m, 2n], "W_d": [E, n, m]}.
    """
    c = lora_scale(alpha, r, rslora)
    if W.get("A_u") is None:
        d_gu = _f64(W["A_g"]) @ _f64(W["B_g"])
    else:
        d_gu = np.concatenate([_f64(W["A_g"]) @ _f64(W["B_g"]), _f64(W["A_u"]) @ _f64(W["B_u"])], axis=-1)
    return {"W_gu": _f64(W["W_gu"]) + c * d_gu, "W_d": _f64(W["W_d"]) + c * (_f64(W["A_d"]) @ _f64(W["B_d"]))}


def fused_gate_up_pair(A, B) -> dict:
    """One LoRA pair on the fused gate/up projection written as the two per-projection pairs.

    [UNS] section "Faster LoRA MoE training": the adapter targets the single gate_up_proj tensor,
    so Delta W_gu = (alpha/r) A B with A in R^{m x r}, B in R^{r x 2n}. Its gate columns [0, n) are
    A B[:, :n] and its up columns A B[:, n:], which is the per-projection form with one shared A:
    A_g = A_u = A, B_g = B[:, :n], B_u = B[:, n:].
    """
    B = _f64(B)
    n = B.shape[-1] // 2
    A = _f64(A)
    return {"A_g": A, "A_u": A, "B_g": B[..., :n], "B_u": B[..., n:]}


def fused_gate_up_grads(g: dict):
    """Gradients (dA, dB) of the fused gate/up pair from those of its per-projection form.

    A enters both halves, so its gradient is the sum dA_g + dA_u (chain rule for a parameter used
    twice); B's gradient is the column concatenation [dB_g | dB_u].
    """
    return g["dA_g"] + g["dA_u"], np.concatenate([g["dB_g"], g["dB_u"]], axis=-1)


def _single_expert(W1: dict) -> dict:
    return _expert({k: _f64(v)[None] for k, v in W1.items()}, 0)


def shared_expert_forward(X, W1: dict, alpha: float, r: int, rslora: bool = False) -> dict:
    """A shared expert: one SwiGLU expert with Split LoRA that every token passes through, its
    output added to the routed experts' ([UNS] section "GLM 4.7 Benchmarks": GLM 4.7 Flash has 64
    routed experts and 1 shared expert, DeepSeek-MoE style). W1 holds one expert's weights
    (W_gu [m, 2n], W_d [n, m], A_*, B_*). Returns the intermediates; "o" is the contribution to Y.
    """
    return expert_rows_forward(X, _single_expert(W1), lora_scale(alpha, r, rslora))


def shared_expert_backward(dY, X, W1: dict, alpha: float, r: int, fwd: dict | None = None,
                           rslora: bool = False) -> dict:
    """Gradients of the shared expert: its output adds to Y with weight 1, so dO = dY for every
    token; "dX" is its contribution to the input gradient."""
    return expert_rows_backward(X, dY, _single_expert(W1), lora_scale(alpha, r, rslora), fwd)


def router_backward(ds, rt: dict, W_r, score: str = "softmax", renormalize: bool = True):
    """Gradient reaching X through the routing weights, top-k set held fixed.

    ds[t, j] = dY_t . o_{t,j} is the gradient of the loss with respect to s_{t,j}.
    softmax + renormalise: s_j = exp(z_j) / sum_sel exp(z), so dz_j = s_j (ds_j - sum_i s_i ds_i).
    sigmoid + renormalise: s_j = p_j / S, S = sum_sel p, dz_j = p_j (1 - p_j) / S (ds_j - sum_i s_i ds_i).
    sigmoid alone: dz_j = p_j (1 - p_j) ds_j. Logits of unselected experts get no gradient in
    these three cases. dX_r[t] = sum_j dz_{t,j} W_r[:, e_{t,j}].
    Returns (dX_r, dz).
    """
    ds = _f64(ds)
    w, p, idx = rt["w"], rt["p_sel"], rt["idx"]
    if score == "softmax" and renormalize:
        dz = w * (ds - (w * ds).sum(axis=1, keepdims=True))
    elif score == "sigmoid" and renormalize:
        S = p.sum(axis=1, keepdims=True)
        dz = p * (1.0 - p) / S * (ds - (w * ds).sum(axis=1, keepdims=True))
    elif score == "sigmoid":
        dz = p * (1.0 - p) * ds
    else:
        raise NotImplementedError("softmax without renormalisation: every logit gets a gradient")
    Wr = _f64(W_r)
    dX_r = np.zeros((ds.shape[0], Wr.shape[0]))
    for j in range(idx.shape[1]):
        dX_r += dz[:, j:j + 1] * Wr[:, idx[:, j]].T
    return dX_r, dz


def backward(dY, X, W_r, W: dict, rt: dict, alpha: float, r: int, score: str = "softmax",
             renormalize: bool = True, router_grad: bool = True, saved: dict | None = None,
             rslora: bool = False):
    """dX and the LoRA-factor gradients of the whole layer for upstream gradient dY.

    Returns dict with dX [s,m], dA_g/dA_u [E,m,r], dB_g/dB_u [E,r,n], dA_d [E,n,r],
    dB_d [E,r,m], plus ds [s,k] and dz [s,k].
    """
    dY = _f64(dY)
    X = _f64(X)
    c = lora_scale(alpha, r, rslora)
    k, E = rt["k"], rt["E"]
    s, m = X.shape
    P = s * k
    n = W["W_d"].shape[1]
    perm, inv, off, w = rt["perm"], rt["inv"], rt["off"], rt["w"]
    if saved is None:
        _, saved = forward(X, W, rt, alpha, r, keep=True, rslora=rslora)
    o = saved["o"]
    tok_of_row = perm // k
    slot_of_row = perm % k
    # combine backward: dO = s_{t,j} dY_t, ds_{t,j} = dY_t . o_{t,j}
    dO = w[tok_of_row, slot_of_row][:, None] * dY[tok_of_row]
    ds_rows = np.einsum("ij,ij->i", dY[tok_of_row], o)
    ds = np.zeros((s, k))
    ds[tok_of_row, slot_of_row] = ds_rows
    Xp = X[tok_of_row]
    dXp = np.zeros((P, m))
    grads = {"dA_g": np.zeros((E, m, r)), "dB_g": np.zeros((E, r, n)),
             "dA_u": np.zeros((E, m, r)), "dB_u": np.zeros((E, r, n)),
             "dA_d": np.zeros((E, n, r)), "dB_d": np.zeros((E, r, m))}
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        fwd = {key: saved[key][a:b] for key in ("g", "u", "h", "T_g", "T_u", "T_d")}
        res = expert_rows_backward(Xp[a:b], dO[a:b], _expert(W, e), c, fwd)
        dXp[a:b] = res["dX"]
        for key in grads:
            grads[key][e] = res[key]
    dX = np.zeros((s, m))
    tok = np.arange(s)
    for j in range(k):
        dX += dXp[inv[tok * k + j]]
    dz = np.zeros((s, k))
    if router_grad:
        dX_r, dz = router_backward(ds, rt, W_r, score, renormalize)
        dX += dX_r
    out = dict(dX=dX, ds=ds, dz=dz)
    out.update(grads)
    return out


# ----------------------------------------------------------------------------- sampled outputs
# Full-size layers are checked on sampled tokens and experts: y_t and dX_t depend only on x_t,
# dY_t and the k experts of token t; an expert's LoRA gradients only on that expert's rows.

def forward_tokens(tokens, X, W: dict, rt: dict, alpha: float, r: int) -> np.ndarray:
    """y_t for the listed tokens, one token at a time over its k experts (no grouping)."""
    c = alpha / r
    out = np.zeros((len(tokens), X.shape[1]))
    for q, t in enumerate(tokens):
        x = _f64(X[t:t + 1])
        for j in range(rt["k"]):
            e = int(rt["idx"][t, j])
            out[q] += rt["w"][t, j] * expert_rows_forward(x, _expert(W, e), c)["o"][0]
    return out


def backward_tokens(tokens, dY, X, W_r, W: dict, rt: dict, alpha: float, r: int,
                    score: str = "softmax", renormalize: bool = True, router_grad: bool = True):
    """dX_t for the listed tokens (expert paths plus, optionally, the router path)."""
    c = alpha / r
    k = rt["k"]
    Wr = _f64(W_r)
    out = np.zeros((len(tokens), X.shape[1]))
    for q, t in enumerate(tokens):
        x = _f64(X[t:t + 1])
        dy = _f64(dY[t:t + 1])
        ds = np.zeros(k)
        for j in range(k):
            e = int(rt["idx"][t, j])
            ew = _expert(W, e)
            f = expert_rows_forward(x, ew, c)
            ds[j] = float(dy[0] @ f["o"][0])
            res = expert_rows_backward(x, rt["w"][t, j] * dy, ew, c, f)
            out[q] += res["dX"][0]
        if router_grad:
            sub = dict(w=rt["w"][t:t + 1], p_sel=rt["p_sel"][t:t + 1], idx=rt["idx"][t:t + 1])
            dX_r, _ = router_backward(ds[None, :], sub, Wr, score, renormalize)
            out[q] += dX_r[0]
    return out


def token_outputs(tokens, X, W: dict, rt: dict, alpha: float, r: int, dY=None, W_r=None,
                  score: str = "softmax", renormalize: bool = True, router_grad: bool = True):
    """y_t (and, with dY, dX_t) for the listed tokens, visiting each expert the tokens use once.

    The same sums as forward_tokens / backward_tokens, ordered by expert instead of by token, so
    that a layer with large experts needs only one expert's weights in memory at a time. Returns
    (y [T, m], dX [T, m] or None).
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    c = alpha / r
    k = rt["k"]
    m = X.shape[1]
    T = len(tokens)
    y = np.zeros((T, m))
    dx = np.zeros((T, m)) if dY is not None else None
    ds = np.zeros((T, k))
    users = {}
    for q, t in enumerate(tokens):
        for j in range(k):
            users.setdefault(int(rt["idx"][t, j]), []).append((q, j))
    for e in sorted(users):
        q = np.array([u[0] for u in users[e]])
        j = np.array([u[1] for u in users[e]])
        ew = _expert(W, e)
        xr = _f64(X[tokens[q]])
        f = expert_rows_forward(xr, ew, c)
        w = rt["w"][tokens[q], j][:, None]
        y[q] += w * f["o"]              # a token uses an expert at most once: q has no repeats
        if dY is not None:
            dy = _f64(dY[tokens[q]])
            ds[q, j] = np.einsum("ij,ij->i", dy, f["o"])
            dx[q] += expert_rows_backward(xr, w * dy, ew, c, f)["dX"]
    if dY is not None and router_grad:
        sub = dict(w=rt["w"][tokens], p_sel=rt["p_sel"][tokens], idx=rt["idx"][tokens])
        dX_r, _ = router_backward(ds, sub, W_r, score, renormalize)
        dx += dX_r
    return y, dx


def backward_expert(e: int, dY, X, W: dict, rt: dict, alpha: float, r: int) -> dict:
    """LoRA-factor gradients of one expert, from that expert's group of rows only."""
    c = alpha / r
    k = rt["k"]
    a, b = int(rt["off"][e]), int(rt["off"][e + 1])
    n = W["W_d"].shape[1]
    m = X.shape[1]
    if a == b:
        return {"dA_g": np.zeros((m, r)), "dB_g": np.zeros((r, n)), "dA_u": np.zeros((m, r)),
                "dB_u": np.zeros((r, n)), "dA_d": np.zeros((n, r)), "dB_d": np.zeros((r, m))}
    pairs = rt["perm"][a:b]
    tok, slot = pairs // k, pairs % k
    Xr = _f64(X[tok])
    dO = rt["w"][tok, slot][:, None] * _f64(dY[tok])
    res = expert_rows_backward(Xr, dO, _expert(W, e), c)
    return {key: res[key] for key in ("dA_g", "dB_g", "dA_u", "dB_u", "dA_d", "dB_d")}
