"""Build libmoss.so in-tree with hipcc for gfx950.

``python -m diffusion_transformer_denoiser_amd.build`` compiles every HIP
source under ``csrc/`` (one object each, in parallel) and links the shared
library next to this file.  It always rebuilds.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoss.so")

SOURCES = ["elementwise.hip", "qk_norm_rope.hip", "gemm.hip", "attention.hip", "moss_api.hip"]

# Packed-fp32 VALU instructions are disabled for every kernel: hipcc otherwise
# forms them from ordinary float code.  (The host pass prints that it does not
# know the feature; that line is filtered below.)
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-I" + INCLUDE, "-I" + CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain (ROCm) is required to build libmoss.so")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the C ABI layer
# (argument validation, planning, launch sequencing); the device code is built
# as usual.  Each -fsanitize goes right after -Xarch_host.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer"]
ASAN_LIB = os.path.join(PKG, "_build_asan", "libmoss_asan.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every source and link libmoss.so (or, with sanitize, the host-sanitizer copy)."""
    hipcc = _hipcc()
    bdir = os.path.dirname(ASAN_LIB) if sanitize else BUILD
    out = ASAN_LIB if sanitize else LIB
    extra = HOST_SANITIZE if sanitize else []
    os.makedirs(bdir, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(min(len(cmds), 8)) as ex:
        outs = list(ex.map(_run, cmds))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = out + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *extra, "-o", tmp, *objs])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
