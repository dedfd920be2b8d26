"""Buffer allocation around the C-ABI calls (torch provides device memory and the stream).

Nothing here computes any part of the layer: each helper allocates the output and scratch
tensors the C ABI expects and makes one call into libmoelora.
"""
from __future__ import annotations

import torch

from . import (make_shape, moe_bwd_ws_bytes, moe_fwd_saved_bytes, moe_fwd_ws_bytes,
               moe_lora_backward, moe_lora_forward, moe_route, moe_route_state_bytes,
               moe_shared_backward, moe_shared_bwd_ws_bytes, moe_shared_forward,
               moe_shared_fwd_ws_bytes, moe_shared_saved_bytes)

__all__ = ["shape_of", "alloc_route", "route", "forward", "backward", "alloc_grads", "shared_forward",
           "shared_grads", "shared_backward"]


def shape_of(cfg, router_grad=True, flags=0, s=None):
    """moe_shape for an object with s, m, n, E, k, r, alpha, dtype, score, renormalize fields."""
    return make_shape(cfg.s if s is None else s, cfg.m, cfg.n, cfg.E, cfg.k, cfg.r, cfg.alpha,
                      cfg.dtype, cfg.score, getattr(cfg, "renormalize", True), router_grad, flags)


def _bytes(n, device):
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)


def alloc_route(shape, device, with_logits=True) -> dict:
    s, E, k = shape.s, shape.E, shape.k
    return {
        "logits": torch.empty(s, E, dtype=torch.float32, device=device) if with_logits else None,
        "topk_idx": torch.empty(s, k, dtype=torch.int32, device=device),
        "topk_w": torch.empty(s, k, dtype=torch.float32, device=device),
        "expert_off": torch.empty(E + 1, dtype=torch.int32, device=device),
        "perm": torch.empty(s * k, dtype=torch.int32, device=device),
        "inv_perm": torch.empty(s * k, dtype=torch.int32, device=device),
        "route_state": _bytes(moe_route_state_bytes(shape), device),
    }


def route(shape, X, W_r, router_bias=None, bufs=None, stream=None) -> dict:
    rt = bufs if bufs is not None else alloc_route(shape, X.device)
    moe_route(shape, X, W_r, router_bias, rt["logits"], rt["topk_idx"], rt["topk_w"],
              rt["expert_off"], rt["perm"], rt["inv_perm"], rt["route_state"], stream)
    return rt


def forward(shape, X, rt, W, training=True, Y=None, saved=None, ws=None, stream=None):
    """Returns (Y, saved). W holds W_gu, W_d, A_g, B_g, A_u, B_u, A_d, B_d."""
    dev = X.device
    if Y is None:
        Y = torch.empty(shape.s, shape.m, dtype=X.dtype, device=dev)
    if training and saved is None:
        saved = _bytes(moe_fwd_saved_bytes(shape), dev)
    if ws is None:
        nws = moe_fwd_ws_bytes(shape, saved is not None)
        ws = _bytes(nws, dev) if nws else None
    moe_lora_forward(shape, X, rt["topk_idx"], rt["topk_w"], rt["expert_off"], rt["perm"],
                     rt["inv_perm"], rt["route_state"], W["W_gu"], W["W_d"], W["A_g"], W["B_g"],
                     W["A_u"], W["B_u"], W["A_d"], W["B_d"], Y, saved, ws, stream)
    return Y, saved


def alloc_grads(shape, device) -> dict:
    """Gradient buffers; with a fused gate/up LoRA pair dA_g is dA [E, m, r], dB_g is dB
    [E, r, 2n], and there are no dA_u, dB_u."""
    E, m, n, r = shape.E, shape.m, shape.n, shape.r
    f = dict(dtype=torch.float32, device=device)
    if shape.flags & 32:  # MOE_FLAG_FUSED_GU_LORA
        return {"dA_g": torch.empty(E, m, r, **f), "dB_g": torch.empty(E, r, 2 * n, **f),
                "dA_u": None, "dB_u": None,
                "dA_d": torch.empty(E, n, r, **f), "dB_d": torch.empty(E, r, m, **f)}
    return {"dA_g": torch.empty(E, m, r, **f), "dB_g": torch.empty(E, r, n, **f),
            "dA_u": torch.empty(E, m, r, **f), "dB_u": torch.empty(E, r, n, **f),
            "dA_d": torch.empty(E, n, r, **f), "dB_d": torch.empty(E, r, m, **f)}


def backward(shape, dY, X, W_r, rt, W, saved, dX=None, grads=None, ws=None, stream=None):
    """Returns (dX, grads dict)."""
    dev = X.device
    if dX is None:
        dX = torch.empty(shape.s, shape.m, dtype=X.dtype, device=dev)
    if grads is None:
        grads = alloc_grads(shape, dev)
    if ws is None:
        ws = _bytes(moe_bwd_ws_bytes(shape), dev)
    moe_lora_backward(shape, dY, X, W_r, rt["topk_idx"], rt["topk_w"], rt["expert_off"],
                      rt["perm"], rt["inv_perm"], rt["route_state"], W["W_gu"], W["W_d"],
                      W["A_g"], W["B_g"], W["A_u"], W["B_u"], W["A_d"], W["B_d"], saved, dX,
                      grads["dA_g"], grads["dB_g"], grads["dA_u"], grads["dB_u"], grads["dA_d"],
                      grads["dB_d"], ws, stream)
    return dX, grads


def shared_forward(shape, X, W, Y, training=True, saved=None, ws=None, stream=None):
    """Y += the shared expert's output (W: W_gu [m, 2n], W_d [n, m] and the LoRA factors of one
    expert). Returns the saved buffer (None when not training)."""
    dev = X.device
    if training and saved is None:
        saved = _bytes(moe_shared_saved_bytes(shape), dev)
    if ws is None:
        ws = _bytes(moe_shared_fwd_ws_bytes(shape, saved is not None), dev)
    moe_shared_forward(shape, X, W["W_gu"], W["W_d"], W["A_g"], W["B_g"], W.get("A_u"), W.get("B_u"),
                       W["A_d"], W["B_d"], Y, saved, ws, stream)
    return saved


def shared_grads(shape, device) -> dict:
    """Gradient buffers of the shared expert's LoRA factors (fp32)."""
    m, n, r = shape.m, shape.n, shape.r
    f = dict(dtype=torch.float32, device=device)
    if shape.flags & 32:  # MOE_FLAG_FUSED_GU_LORA
        return {"dA_g": torch.empty(m, r, **f), "dB_g": torch.empty(r, 2 * n, **f), "dA_u": None,
                "dB_u": None, "dA_d": torch.empty(n, r, **f), "dB_d": torch.empty(r, m, **f)}
    return {"dA_g": torch.empty(m, r, **f), "dB_g": torch.empty(r, n, **f),
            "dA_u": torch.empty(m, r, **f), "dB_u": torch.empty(r, n, **f),
            "dA_d": torch.empty(n, r, **f), "dB_d": torch.empty(r, m, **f)}


def shared_backward(shape, dY, X, W, saved, dX, grads=None, ws=None, stream=None):
    """dX += the shared expert's input gradient; returns the LoRA-factor gradients."""
    dev = X.device
    if grads is None:
        grads = shared_grads(shape, dev)
    if ws is None:
        ws = _bytes(moe_shared_bwd_ws_bytes(shape), dev)
    moe_shared_backward(shape, dY, X, W["W_gu"], W["W_d"], W["A_g"], W["B_g"], W.get("A_u"),
                        W.get("B_u"), W["A_d"], W["B_d"], saved, dX, grads["dA_g"], grads["dB_g"],
                        grads["dA_u"], grads["dB_u"], grads["dA_d"], grads["dB_d"], ws, stream)
    return grads
