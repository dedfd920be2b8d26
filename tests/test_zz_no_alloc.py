"""moe_lora_forward_noalloc (the inference forward whose scratch is the library's fixed device array)
against moe_lora_forward with a caller workspace, through the C ABI: two calls in a row, the second
on a smaller layer, must give the same Y (bit for bit: the same kernels on the same inputs), and a
layer too large for the fixed scratch is refused with nothing enqueued."""
from __future__ import annotations

import pytest
import torch

import grouped_gemm_top_amd as g
from grouped_gemm_top_amd import layer
from helpers import TOL, np64, rel_err
from synth import config, make_inputs

pytestmark = pytest.mark.gpu

WEIGHTS = ("W_gu", "W_d", "A_g", "B_g", "A_u", "B_u", "A_d", "B_d")


def _say(msg):
    print(msg, flush=True)


def _both(cfg, flags, cuda):
    inp = make_inputs(cfg, seed=3, device="cpu", with_grad_output=False)
    d = {k: (v.to(cuda) if v is not None else None) for k, v in inp.items()}
    if flags & g.MOE_FLAG_FUSED_GU_LORA:  # one pair: B [E, r, 2n] in B_g (B_g and B_u side by side)
        d["B_g"] = torch.cat([d["B_g"], d["B_u"]], dim=2).contiguous()
        d["A_u"] = d["B_u"] = None
    if flags & g.MOE_FLAG_WEIGHTS_OUT_IN:
        d["W_gu"] = d["W_gu"].transpose(1, 2).contiguous()
        d["W_d"] = d["W_d"].transpose(1, 2).contiguous()
    shape = layer.shape_of(cfg, flags=flags)
    assert g.moe_fwd_ws_bytes(shape, False) <= g.MOE_NOALLOC_SCRATCH_BYTES
    rt = layer.route(shape, d["X"], d["W_r"], d["router_bias"])
    Y_ref, _ = layer.forward(shape, d["X"], rt, d, training=False)
    Y = torch.full_like(Y_ref, float("nan"))
    g.moe_lora_forward_noalloc(shape, d["X"], rt["topk_idx"], rt["topk_w"], rt["expert_off"], rt["perm"],
                               rt["inv_perm"], rt["route_state"], *[d[k] for k in WEIGHTS], Y)
    torch.cuda.synchronize()
    return Y, Y_ref


@pytest.mark.parametrize("flags", [0, 4, 32], ids=["plain", "out_in", "fused_gu"])
def test_noalloc_forward_matches_workspace_forward(flags, cuda):
    big = config("qwen3_30b_a3b", s=1024, m=512, n=256, E=32, k=8)
    small = config("qwen3_30b_a3b", s=200, m=512, n=256, E=32, k=8)
    for cfg in (big, small):  # the second call reuses the array the first one filled
        _say(f"[noalloc] flags={flags} s={cfg.s} m={cfg.m} n={cfg.n} E={cfg.E} k={cfg.k}")
        Y, Y_ref = _both(cfg, flags, cuda)
        assert torch.equal(Y, Y_ref)
        assert rel_err(np64(Y), np64(Y_ref)) <= TOL[cfg.dtype]


def test_noalloc_forward_refuses_a_layer_beyond_its_scratch(cuda):
    cfg = config("qwen3_30b_a3b", s=4096)  # the full Qwen3-30B-A3B layer needs ~290 MB of scratch
    shape = layer.shape_of(cfg)
    assert g.moe_fwd_ws_bytes(shape, False) > g.MOE_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(16, device=cuda)
    Y = torch.full((cfg.s, cfg.m), 7.0, dtype=torch.bfloat16, device=cuda)
    with pytest.raises(g.MoeError) as err:
        g.moe_lora_forward_noalloc(shape, *([x] * 15), Y)
    assert err.value.status == g.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(Y == 7.0)
