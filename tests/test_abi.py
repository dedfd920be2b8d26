"""C-ABI checks that need no GPU: exported symbols, size queries and argument validation.

Every call here fails validation on the host, so nothing is enqueued and no device is touched.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

import grouped_gemm_top_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moelora.h")

FAKE = 0x10000   # aligned non-null stand-in pointer (never dereferenced: validation fails first)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def exported_symbols():
    out = subprocess.run(["nm", "-D", "--defined-only", g.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    return {line.split()[-1] for line in out.splitlines() if line.strip()}


def test_library_exports_every_declared_function():
    decl = header_functions()
    assert {"moe_route", "moe_lora_forward", "moe_lora_backward"} <= set(decl)
    exported = exported_symbols()
    missing = [f for f in decl if f not in exported]
    assert not missing, missing
    lib = g.lib()
    for f in decl:
        assert getattr(lib, f) is not None


def test_status_strings_and_version():
    assert g.moe_status_str(g.MOE_OK) == "MOE_OK"
    assert g.moe_status_str(g.MOE_ERR_WORKSPACE) == "MOE_ERR_WORKSPACE"
    assert g.moe_status_str(99) == "MOE_ERR_UNKNOWN"
    assert g.moe_abi_version() == 1


def shape(**kw):
    base = dict(s=512, m=256, n=192, E=16, k=4, r=16, alpha=32.0, dtype="bf16")
    base.update(kw)
    return g.make_shape(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(k=17), g.MOE_ERR_INVALID_ARG),
    (dict(k=0), g.MOE_ERR_INVALID_ARG),
    (dict(s=-1), g.MOE_ERR_INVALID_ARG),
    (dict(r=0), g.MOE_ERR_INVALID_ARG),
    (dict(dtype=5), g.MOE_ERR_INVALID_ARG),
    (dict(score=3), g.MOE_ERR_INVALID_ARG),
    (dict(flags=64), g.MOE_ERR_INVALID_ARG),
    (dict(alpha=float("nan")), g.MOE_ERR_INVALID_ARG),
    (dict(m=200), g.MOE_ERR_UNSUPPORTED),
    (dict(n=100), g.MOE_ERR_UNSUPPORTED),
    (dict(E=2048, k=4), g.MOE_ERR_UNSUPPORTED),
    (dict(r=12), g.MOE_ERR_UNSUPPORTED),
    (dict(r=128), g.MOE_ERR_UNSUPPORTED),
    (dict(E=12), g.MOE_OK),    # bf16 W_r rows not 16-byte aligned: the router GEMM reads a padded copy
    (dict(E=60, k=4), g.MOE_OK),
    (dict(s=1 << 29, k=4), g.MOE_ERR_UNSUPPORTED),   # 2^31 pairs: pair ids are int32
    (dict(s=1 << 20, m=4096), g.MOE_OK),             # 2^32 activation elements: 64-bit offsets
    (dict(s=65536, m=7168, n=2048, E=256, k=8), g.MOE_OK),  # the DeepSeek-V3 layer at 64K tokens
    (dict(), g.MOE_OK),
    (dict(dtype="f32", r=4, E=12), g.MOE_OK),
    (dict(s=0), g.MOE_OK),
])
def test_check_shape(kw, status):
    sh = shape(**kw)
    assert g.moe_check_shape(sh) == status
    if status != g.MOE_OK:
        assert g.moe_route_state_bytes(sh) == 0
        assert g.moe_fwd_saved_bytes(sh) == 0
        assert g.moe_bwd_ws_bytes(sh) == 0


def test_null_shape():
    lib = g.lib()
    assert lib.moe_check_shape(None) == g.MOE_ERR_INVALID_ARG
    assert lib.moe_route_state_bytes(None) == 0


def test_sizes_grow_with_tokens_and_dtype():
    a, b = shape(s=512), shape(s=1024)
    for fn in (g.moe_route_state_bytes, g.moe_fwd_saved_bytes, g.moe_bwd_ws_bytes):
        assert 0 < fn(a) < fn(b)
    # the expert outputs o (P x m, only the forward's combine reads them) live in the workspace
    o_bytes = a.s * a.k * a.m * (2 if a.dtype == g.MOE_DTYPE["bf16"] else 4)
    assert g.moe_fwd_ws_bytes(a, True) == o_bytes
    assert g.moe_fwd_ws_bytes(a, False) == g.moe_fwd_saved_bytes(a) + o_bytes
    assert g.moe_fwd_saved_bytes(shape(dtype="f32")) > g.moe_fwd_saved_bytes(shape())


def _route(sh, X=FAKE, Wr=FAKE, state_bytes=None, state=FAKE):
    lib = g.lib()
    if state_bytes is None:
        state_bytes = g.moe_route_state_bytes(sh)
    return lib.moe_route(ctypes.byref(sh), X, Wr, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, state,
                         state_bytes, None)


def test_route_validation():
    sh = shape()
    assert _route(sh, X=None) == g.MOE_ERR_INVALID_ARG
    assert _route(sh, Wr=FAKE + 8) == g.MOE_ERR_INVALID_ARG
    assert _route(sh, state=None) == g.MOE_ERR_INVALID_ARG
    assert _route(sh, state_bytes=g.moe_route_state_bytes(sh) - 1) == g.MOE_ERR_WORKSPACE
    assert _route(shape(k=99)) == g.MOE_ERR_INVALID_ARG


def _forward(sh, saved=FAKE, saved_bytes=None, ws=None, ws_bytes=0, Y=FAKE):
    lib = g.lib()
    if saved_bytes is None:
        saved_bytes = g.moe_fwd_saved_bytes(sh)
    p = [FAKE] * 15
    return lib.moe_lora_forward(ctypes.byref(sh), *p, Y, saved, saved_bytes, ws, ws_bytes, None)


def test_forward_validation():
    sh = shape()
    assert _forward(sh, saved_bytes=g.moe_fwd_saved_bytes(sh) - 256) == g.MOE_ERR_WORKSPACE
    assert _forward(sh, saved=None, ws=FAKE, ws_bytes=10) == g.MOE_ERR_WORKSPACE
    assert _forward(sh, Y=None) == g.MOE_ERR_INVALID_ARG
    assert _forward(sh, saved=FAKE + 16) == g.MOE_ERR_INVALID_ARG


def test_noalloc_forward_refuses_layers_beyond_its_scratch():
    """The no-allocation forward checks the shape and its fixed scratch before touching a device."""
    lib = g.lib()
    big = shape(s=1 << 20)
    assert g.moe_fwd_ws_bytes(big, False) > g.MOE_NOALLOC_SCRATCH_BYTES
    assert lib.moe_lora_forward_noalloc(ctypes.byref(big), *([FAKE] * 16), None) == g.MOE_ERR_WORKSPACE
    bad = shape(m=100)
    assert lib.moe_lora_forward_noalloc(ctypes.byref(bad), *([FAKE] * 16), None) == g.MOE_ERR_UNSUPPORTED


def _backward(sh, ws_bytes=None, saved=FAKE, dX=FAKE):
    lib = g.lib()
    if ws_bytes is None:
        ws_bytes = g.moe_bwd_ws_bytes(sh)
    p = [FAKE] * 17
    grads = [FAKE] * 6
    return lib.moe_lora_backward(ctypes.byref(sh), *p, saved, g.moe_fwd_saved_bytes(sh), dX,
                                 *grads, FAKE, ws_bytes, None)


def test_backward_validation():
    sh = shape()
    assert _backward(sh, ws_bytes=g.moe_bwd_ws_bytes(sh) - 1) == g.MOE_ERR_WORKSPACE
    assert _backward(sh, saved=None) == g.MOE_ERR_INVALID_ARG
    assert _backward(sh, dX=None) == g.MOE_ERR_INVALID_ARG
    assert _backward(shape(renormalize=False)) == g.MOE_ERR_UNSUPPORTED
    assert _backward(shape(renormalize=False, router_grad=False), ws_bytes=0) == g.MOE_ERR_WORKSPACE


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(g, "_lib", None)
    monkeypatch.setattr(g, "LIB_PATH", "/nonexistent/libmoelora.so")
    with pytest.raises(RuntimeError, match="missing"):
        g.lib()


def test_product_code_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "grouped_gemm_top_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\boracle\b", text), f
