"""The library's host logic under AddressSanitizer and UBSan (no GPU needed).

A build of the library whose host code carries both sanitizers (grouped_gemm_top_amd/build.py,
build_host_sanitized) is loaded in a child process that preloads clang's ASan runtime and imports nothing
but ctypes. It drives every entry point
that answers without the GPU: the shape check and every size query over a few thousand valid and invalid
shapes, the status strings and timing-stage names, and every compute entry point with arguments that must
be rejected (null, misaligned or undersized buffers, a null shape). Any sanitizer report, or a rejection
with the wrong status, fails the test. The child rebuilds the binding's moe_shape layout and argument types
from what this process passes it, so the two cannot drift apart.
"""
import json
import os
import subprocess
import sys

import pytest

from grouped_gemm_top_amd import build as gbuild
import grouped_gemm_top_amd as g

CHILD = r'''
import ctypes, json, random, sys
spec = json.loads(sys.argv[2])
lib = ctypes.CDLL(sys.argv[1])
CT = {"i32": ctypes.c_int32, "f32": ctypes.c_float}
class Shape(ctypes.Structure):
    _fields_ = [(n, CT[t]) for n, t in spec["fields"]]
SP = ctypes.POINTER(Shape)
AT = {"shape": SP, "p": ctypes.c_void_p, "sz": ctypes.c_size_t, "i32": ctypes.c_int32, "cstr": ctypes.c_char_p,
      "pd": ctypes.POINTER(ctypes.c_double), "pi64": ctypes.POINTER(ctypes.c_int64)}
for name, (res, args) in spec["sigs"].items():
    fn = getattr(lib, name)
    fn.restype = AT[res]
    fn.argtypes = [AT[a] for a in args]
C = spec["const"]
OK, INVALID, UNSUP, WS = C["ok"], C["invalid"], C["unsupported"], C["workspace"]

assert lib.moe_abi_version() > 0
for st in range(-3, 12):
    assert lib.moe_status_str(st) is not None
nst = lib.moe_timing_stage_count()
assert nst > 0
for i in range(-2, nst + 2):
    name = lib.moe_timing_stage_name(i)
    assert (name is None) == (i < 0 or i >= nst), i
tot = (ctypes.c_double * nst)()
cnt = (ctypes.c_int64 * nst)()
assert lib.moe_timing_read(tot, cnt, nst) == OK

rng = random.Random(0)
flags_all = [0, 1, 2, 4, 8, 16, 32, 2 | 4, 16 | 32, 2 | 4 | 16 | 32, 64, -1]
n_ok = 0
for it in range(3000):
    if it % 3:  # mostly shapes the library accepts
        E = rng.choice([1, 2, 8, 12, 60, 128, 200, 256, 1024])
        s = Shape(rng.choice([0, 1, 7, 256, 4096, 65536]), 64 * rng.randint(1, 112), 64 * rng.randint(1, 45),
                  E, rng.randint(1, E), rng.choice([8, 16, 32, 64]), rng.choice([32.0, 0.0, 1.5]),
                  rng.choice([0, 1]), rng.choice([0, 1]), rng.choice([0, 1]), rng.choice([0, 1]),
                  rng.choice(flags_all[:10]))
    else:
        E = rng.choice([0, 1, 2, 8, 12, 60, 128, 200, 256, 1024, 1025, -4])
        s = Shape(rng.choice([0, 1, 7, 256, 4096, 65536, 300000, -1]),
                  rng.choice([64, 128, 2048, 2880, 7168, 100, 0, -64]),
                  rng.choice([64, 192, 768, 2048, 2880, 96, 0]),
                  E, rng.choice([1, 2, 4, 8, 72, max(E, 1), E + 1, 0, -1]),
                  rng.choice([4, 8, 12, 16, 32, 64, 65, 128, 0, -8]),
                  rng.choice([32.0, 0.0, 1.5, float("nan")]),
                  rng.choice([0, 1, 2, -1]), rng.choice([0, 1, 2]), rng.choice([0, 1]), rng.choice([0, 1]),
                  rng.choice(flags_all))
    st = lib.moe_check_shape(ctypes.byref(s))
    assert st in (OK, INVALID, UNSUP), st
    if st != OK:
        # a call with this shape must refuse it the same way, before looking at any buffer
        assert lib.moe_lora_forward(ctypes.byref(s), *([None] * 17), 0, None, 0, None) == st
        continue
    n_ok += 1
    sizes = [lib.moe_route_state_bytes(ctypes.byref(s)), lib.moe_fwd_saved_bytes(ctypes.byref(s)),
             lib.moe_fwd_ws_bytes(ctypes.byref(s), 0), lib.moe_fwd_ws_bytes(ctypes.byref(s), 1),
             lib.moe_bwd_ws_bytes(ctypes.byref(s)), lib.moe_shared_saved_bytes(ctypes.byref(s)),
             lib.moe_shared_fwd_ws_bytes(ctypes.byref(s), 0), lib.moe_shared_fwd_ws_bytes(ctypes.byref(s), 1),
             lib.moe_shared_bwd_ws_bytes(ctypes.byref(s))]
    assert all(v < (1 << 50) for v in sizes), sizes
    if s.s > 0:
        assert sizes[0] > 0 and sizes[2] > 0, sizes
    # every compute entry point refuses null buffers (or, for the routed forward, the missing route state)
    A = ctypes.c_void_p(4096)  # aligned, never dereferenced on the host
    assert lib.moe_route(ctypes.byref(s), *([None] * 10), 0, None) in (INVALID, WS) or s.s == 0
    assert lib.moe_lora_forward(ctypes.byref(s), *([None] * 17), 0, None, 0, None) in (INVALID, WS) or s.s == 0
    assert lib.moe_lora_forward_noalloc(ctypes.byref(s), *([None] * 17)) in (INVALID, WS, UNSUP) or s.s == 0
    # (the backward refuses merged weights, and softmax without renormalisation with router gradients)
    assert lib.moe_lora_backward(ctypes.byref(s), *([None] * 18), 0, *([None] * 8), 0, None) in (INVALID, WS, UNSUP) \
        or s.s == 0
    assert lib.moe_peft_merge(ctypes.byref(s), *([None] * 11)) in (INVALID, UNSUP, WS)
    # a route state one byte short of its size query
    if s.s > 0:
        need = sizes[0]
        st2 = lib.moe_route(ctypes.byref(s), *([A] * 9), None, need - 1 if need else 0, A)
        assert st2 in (INVALID, WS), st2
for fn, nargs in (("moe_check_shape", 0), ("moe_route_state_bytes", 0), ("moe_bwd_ws_bytes", 0)):
    r = getattr(lib, fn)(None)
    assert r in (INVALID, 0), (fn, r)
assert lib.moe_lora_forward(None, *([None] * 17), 0, None, 0, None) == INVALID
assert n_ok > 1000, n_ok
print("sanitized host checks:", n_ok, "valid shapes")
'''


def _spec():
    code = {ctypes_t: name for name, ctypes_t in (
        ("i32", g.ctypes.c_int32), ("f32", g.ctypes.c_float), ("p", g.ctypes.c_void_p), ("sz", g.ctypes.c_size_t),
        ("cstr", g.ctypes.c_char_p), ("pd", g.ctypes.POINTER(g.ctypes.c_double)),
        ("pi64", g.ctypes.POINTER(g.ctypes.c_int64)), ("shape", g.ctypes.POINTER(g.MoeShape)))}
    fields = [(n, code[t]) for n, t in g.MoeShape._fields_]
    sigs = {name: (code[res], [code[a] for a in args]) for name, (res, args) in g._SIGNATURES.items()}
    const = {"ok": g.MOE_OK, "invalid": g.MOE_ERR_INVALID_ARG, "unsupported": g.MOE_ERR_UNSUPPORTED,
             "workspace": g.MOE_ERR_WORKSPACE}
    return {"fields": fields, "sigs": sigs, "const": const}


def test_host_logic_under_asan_and_ubsan(tmp_path):
    try:
        gbuild.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    rt = gbuild.sanitizer_runtime()
    if rt is None:
        pytest.skip("clang's AddressSanitizer runtime not found")
    lib = gbuild.build_host_sanitized(str(tmp_path))
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    res = subprocess.run([sys.executable, "-c", CHILD, lib, json.dumps(_spec())], env=env,
                         stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=600)
    report = res.stdout[-3000:] + res.stderr[-6000:]
    assert res.returncode == 0, report
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, report
    assert "sanitized host checks:" in res.stdout, report
