"""Builds libmoelora.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libmoelora.so")
SOURCES = ("api.hip", "gemm.hip", "kernels.hip")
ARCH = "gfx950"

# Packed-fp32 instructions are disabled for all device code; hipcc's host pass warns that it does
# not know the feature, which is harmless.
FLAGS = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile every HIP source (in parallel) and link libmoelora.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [cc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if p.returncode != 0:
            failed.append((src, "\n".join(lines)))
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        msg = "\n".join(f"--- {s}\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout.decode(errors="replace"))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


# A build whose host code carries AddressSanitizer and UBSan (the device code is built as usual, without
# them), for checking the library's host logic (shape checks, workspace layouts, size queries, argument
# rejection) on a machine without a GPU.
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined"]


def sanitizer_runtime() -> str | None:
    """The clang AddressSanitizer runtime that a process must preload to load the sanitized library."""
    root = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "lib", "llvm", "lib", "clang")
    if not os.path.isdir(root):
        root = "/opt/rocm/lib/llvm/lib/clang"
    if not os.path.isdir(root):
        return None
    for ver in sorted(os.listdir(root), reverse=True):
        cand = os.path.join(root, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(cand):
            return cand
    return None


def build_host_sanitized(out_dir: str, verbose: bool = False) -> str:
    """Compile every source, the host code with ASan + UBSan, and link out_dir/libmoelora_san.so."""
    os.makedirs(out_dir, exist_ok=True)
    cc = hipcc()
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(out_dir, src.replace(".hip", ".san.o"))
        objs.append(obj)
        cmd = [cc, *SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = [(src, p.communicate()[0].decode(errors="replace")) for src, p in procs]
    failed = [(src, out) for (src, out), (_, p) in zip(failed, procs) if p.returncode != 0]
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(f"--- {s}\n{o}" for s, o in failed))
    out = os.path.join(out_dir, "libmoelora_san.so")
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", *objs, "-o", out]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout.decode(errors="replace"))
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
