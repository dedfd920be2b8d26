"""Python binding of libmoelora (MoE expert-MLP layer with Split LoRA, MI355X / gfx950).

Argument marshalling only: every function here converts torch tensors to device pointers and
calls the C ABI declared in include/moelora.h with the same name. All computation runs in the HIP
kernels of libmoelora.so; there is no other implementation to fall back on, and importing the
functions raises if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first so that libmoelora shares torch's HIP runtime

__all__ = [
    "MoeShape", "MoeError", "lib", "LIB_PATH", "make_shape", "moe_status_str", "moe_abi_version",
    "moe_check_shape", "moe_route_state_bytes", "moe_fwd_saved_bytes", "moe_fwd_ws_bytes",
    "moe_bwd_ws_bytes", "moe_route", "moe_lora_forward", "moe_lora_backward",
    "moe_lora_forward_noalloc", "MOE_NOALLOC_SCRATCH_BYTES",
    "MOE_OK", "MOE_ERR_INVALID_ARG", "MOE_ERR_UNSUPPORTED", "MOE_ERR_WORKSPACE", "MOE_ERR_HIP",
    "MOE_FLAG_REFERENCE_GEMM", "MOE_FLAG_RSLORA", "MOE_FLAG_WEIGHTS_OUT_IN", "MOE_FLAG_MERGED", "MOE_FLAG_RECOMPUTE",
    "MOE_FLAG_FUSED_GU_LORA",
    "moe_peft_merge", "moe_timing_enable", "moe_timing_read",
    "moe_shared_saved_bytes", "moe_shared_fwd_ws_bytes", "moe_shared_bwd_ws_bytes",
    "moe_shared_forward", "moe_shared_backward",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoelora.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, 1, 2, 3, 4
MOE_DTYPE = {"f32": 0, "bf16": 1}
MOE_SCORE = {"softmax": 0, "sigmoid": 1}
MOE_FLAG_REFERENCE_GEMM = 1
MOE_FLAG_RSLORA = 2
MOE_FLAG_WEIGHTS_OUT_IN = 4
MOE_FLAG_MERGED = 8
MOE_FLAG_RECOMPUTE = 16
MOE_FLAG_FUSED_GU_LORA = 32
MOE_NOALLOC_SCRATCH_BYTES = 128 << 20  # the fixed device scratch of moe_lora_forward_noalloc


class MoeShape(ctypes.Structure):
    _fields_ = [("s", ctypes.c_int32), ("m", ctypes.c_int32), ("n", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("r", ctypes.c_int32),
                ("alpha", ctypes.c_float), ("dtype", ctypes.c_int32), ("score", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("router_grad", ctypes.c_int32),
                ("flags", ctypes.c_int32)]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {moe_status_str(status)} ({status})")


_lib = None
_P = ctypes.c_void_p
_SZ = ctypes.c_size_t
_I32 = ctypes.c_int32
_SHAPE = ctypes.POINTER(MoeShape)

_SIGNATURES = {
    "moe_status_str": (ctypes.c_char_p, [_I32]),
    "moe_abi_version": (_I32, []),
    "moe_check_shape": (_I32, [_SHAPE]),
    "moe_route_state_bytes": (_SZ, [_SHAPE]),
    "moe_fwd_saved_bytes": (_SZ, [_SHAPE]),
    "moe_fwd_ws_bytes": (_SZ, [_SHAPE, _I32]),
    "moe_bwd_ws_bytes": (_SZ, [_SHAPE]),
    "moe_route": (_I32, [_SHAPE] + [_P] * 10 + [_SZ, _P]),
    "moe_lora_forward": (_I32, [_SHAPE] + [_P] * 17 + [_SZ, _P, _SZ, _P]),
    "moe_lora_forward_noalloc": (_I32, [_SHAPE] + [_P] * 17),
    "moe_lora_backward": (_I32, [_SHAPE] + [_P] * 18 + [_SZ] + [_P] * 8 + [_SZ, _P]),
    "moe_peft_merge": (_I32, [_SHAPE] + [_P] * 11),
    "moe_shared_saved_bytes": (_SZ, [_SHAPE]),
    "moe_shared_fwd_ws_bytes": (_SZ, [_SHAPE, _I32]),
    "moe_shared_bwd_ws_bytes": (_SZ, [_SHAPE]),
    "moe_shared_forward": (_I32, [_SHAPE] + [_P] * 11 + [_SZ, _P, _SZ, _P]),
    "moe_shared_backward": (_I32, [_SHAPE] + [_P] * 11 + [_SZ] + [_P] * 8 + [_SZ, _P]),
    "moe_timing_enable": (_I32, [_I32]),
    "moe_timing_stage_count": (_I32, []),
    "moe_timing_stage_name": (ctypes.c_char_p, [_I32]),
    "moe_timing_read": (_I32, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64), _I32]),
}


def lib():
    """The loaded libmoelora (ctypes.CDLL); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (__graft_entry__.build())")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def make_shape(s, m, n, E, k, r, alpha, dtype="bf16", score="softmax", renormalize=True,
               router_grad=True, flags=0) -> MoeShape:
    return MoeShape(int(s), int(m), int(n), int(E), int(k), int(r), float(alpha),
                    MOE_DTYPE[dtype] if isinstance(dtype, str) else int(dtype),
                    MOE_SCORE[score] if isinstance(score, str) else int(score),
                    int(bool(renormalize)), int(bool(router_grad)), int(flags))


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor or None")
    if t.device.type != "cuda":
        raise ValueError("tensors passed to libmoelora must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoelora must be contiguous")
    return t.data_ptr() or None


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _check(status, where):
    if status != MOE_OK:
        raise MoeError(status, where)


def moe_status_str(status: int) -> str:
    return lib().moe_status_str(int(status)).decode()


def moe_abi_version() -> int:
    return int(lib().moe_abi_version())


def moe_check_shape(shape: MoeShape) -> int:
    return int(lib().moe_check_shape(ctypes.byref(shape)))


def moe_route_state_bytes(shape: MoeShape) -> int:
    return int(lib().moe_route_state_bytes(ctypes.byref(shape)))


def moe_fwd_saved_bytes(shape: MoeShape) -> int:
    return int(lib().moe_fwd_saved_bytes(ctypes.byref(shape)))


def moe_fwd_ws_bytes(shape: MoeShape, with_saved: bool) -> int:
    return int(lib().moe_fwd_ws_bytes(ctypes.byref(shape), int(bool(with_saved))))


def moe_bwd_ws_bytes(shape: MoeShape) -> int:
    return int(lib().moe_bwd_ws_bytes(ctypes.byref(shape)))


def moe_route(shape, X, W_r, router_bias, logits, topk_idx, topk_w, expert_off, perm, inv_perm,
              route_state, stream=None):
    st = lib().moe_route(ctypes.byref(shape), _ptr(X), _ptr(W_r), _ptr(router_bias), _ptr(logits),
                         _ptr(topk_idx), _ptr(topk_w), _ptr(expert_off), _ptr(perm),
                         _ptr(inv_perm), _ptr(route_state), _nbytes(route_state), _stream(stream))
    _check(st, "moe_route")


def moe_lora_forward(shape, X, topk_idx, topk_w, expert_off, perm, inv_perm, route_state, W_gu,
                     W_d, A_g, B_g, A_u, B_u, A_d, B_d, Y, saved, ws, stream=None):
    st = lib().moe_lora_forward(
        ctypes.byref(shape), _ptr(X), _ptr(topk_idx), _ptr(topk_w), _ptr(expert_off), _ptr(perm),
        _ptr(inv_perm), _ptr(route_state), _ptr(W_gu), _ptr(W_d), _ptr(A_g), _ptr(B_g), _ptr(A_u),
        _ptr(B_u), _ptr(A_d), _ptr(B_d), _ptr(Y), _ptr(saved), _nbytes(saved), _ptr(ws),
        _nbytes(ws), _stream(stream))
    _check(st, "moe_lora_forward")


def moe_lora_forward_noalloc(shape, X, topk_idx, topk_w, expert_off, perm, inv_perm, route_state, W_gu,
                             W_d, A_g, B_g, A_u, B_u, A_d, B_d, Y, stream=None):
    st = lib().moe_lora_forward_noalloc(
        ctypes.byref(shape), _ptr(X), _ptr(topk_idx), _ptr(topk_w), _ptr(expert_off), _ptr(perm),
        _ptr(inv_perm), _ptr(route_state), _ptr(W_gu), _ptr(W_d), _ptr(A_g), _ptr(B_g), _ptr(A_u),
        _ptr(B_u), _ptr(A_d), _ptr(B_d), _ptr(Y), _stream(stream))
    _check(st, "moe_lora_forward_noalloc")


def moe_peft_merge(shape, W_gu, W_d, A_g, B_g, A_u, B_u, A_d, B_d, W_gu_merged, W_d_merged,
                   stream=None):
    st = lib().moe_peft_merge(
        ctypes.byref(shape), _ptr(W_gu), _ptr(W_d), _ptr(A_g), _ptr(B_g), _ptr(A_u), _ptr(B_u),
        _ptr(A_d), _ptr(B_d), _ptr(W_gu_merged), _ptr(W_d_merged), _stream(stream))
    _check(st, "moe_peft_merge")


def moe_lora_backward(shape, dY, X, W_r, topk_idx, topk_w, expert_off, perm, inv_perm, route_state,
                      W_gu, W_d, A_g, B_g, A_u, B_u, A_d, B_d, saved, dX, dA_g, dB_g, dA_u, dB_u,
                      dA_d, dB_d, ws, stream=None):
    st = lib().moe_lora_backward(
        ctypes.byref(shape), _ptr(dY), _ptr(X), _ptr(W_r), _ptr(topk_idx), _ptr(topk_w),
        _ptr(expert_off), _ptr(perm), _ptr(inv_perm), _ptr(route_state), _ptr(W_gu), _ptr(W_d),
        _ptr(A_g), _ptr(B_g), _ptr(A_u), _ptr(B_u), _ptr(A_d), _ptr(B_d), _ptr(saved),
        _nbytes(saved), _ptr(dX), _ptr(dA_g), _ptr(dB_g), _ptr(dA_u), _ptr(dB_u), _ptr(dA_d),
        _ptr(dB_d), _ptr(ws), _nbytes(ws), _stream(stream))
    _check(st, "moe_lora_backward")


def moe_shared_saved_bytes(shape: MoeShape) -> int:
    return int(lib().moe_shared_saved_bytes(ctypes.byref(shape)))


def moe_shared_fwd_ws_bytes(shape: MoeShape, with_saved: bool) -> int:
    return int(lib().moe_shared_fwd_ws_bytes(ctypes.byref(shape), int(bool(with_saved))))


def moe_shared_bwd_ws_bytes(shape: MoeShape) -> int:
    return int(lib().moe_shared_bwd_ws_bytes(ctypes.byref(shape)))


def moe_shared_forward(shape, X, W_gu, W_d, A_g, B_g, A_u, B_u, A_d, B_d, Y, saved, ws, stream=None):
    st = lib().moe_shared_forward(
        ctypes.byref(shape), _ptr(X), _ptr(W_gu), _ptr(W_d), _ptr(A_g), _ptr(B_g), _ptr(A_u),
        _ptr(B_u), _ptr(A_d), _ptr(B_d), _ptr(Y), _ptr(saved), _nbytes(saved), _ptr(ws),
        _nbytes(ws), _stream(stream))
    _check(st, "moe_shared_forward")


def moe_shared_backward(shape, dY, X, W_gu, W_d, A_g, B_g, A_u, B_u, A_d, B_d, saved, dX, dA_g, dB_g,
                        dA_u, dB_u, dA_d, dB_d, ws, stream=None):
    st = lib().moe_shared_backward(
        ctypes.byref(shape), _ptr(dY), _ptr(X), _ptr(W_gu), _ptr(W_d), _ptr(A_g), _ptr(B_g),
        _ptr(A_u), _ptr(B_u), _ptr(A_d), _ptr(B_d), _ptr(saved), _nbytes(saved), _ptr(dX),
        _ptr(dA_g), _ptr(dB_g), _ptr(dA_u), _ptr(dB_u), _ptr(dA_d), _ptr(dB_d), _ptr(ws),
        _nbytes(ws), _stream(stream))
    _check(st, "moe_shared_backward")


def moe_timing_enable(on: bool) -> None:
    _check(lib().moe_timing_enable(int(bool(on))), "moe_timing_enable")


def moe_timing_read() -> dict:
    """{stage name: (summed ms, count)} since the last read; waits for the recorded events."""
    n = int(lib().moe_timing_stage_count())
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(lib().moe_timing_read(ms, cnt, n), "moe_timing_read")
    return {lib().moe_timing_stage_name(i).decode(): (ms[i], int(cnt[i])) for i in range(n)}
