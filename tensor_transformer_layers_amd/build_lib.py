"""Build libtp.so (HIP for gfx950) in-tree with hipcc.

Usage: ``python -m tensor_transformer_layers_amd.build_lib`` or call ``build()``.
Every source is compiled on each call (hipcc cross-compiles without a GPU).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libtp.so")
BUILD = os.path.join(PKG, "_build")

SOURCES = ["gemm.hip", "mlp_fused.hip", "reduce.hip", "attention.hip", "norm.hip", "bwd.hip", "vocab.hip", "tp_api.cpp"]

ARCH = "gfx950"
# -packed-fp32-ops: keep the compiler from forming v_pk_*_f32 instructions.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libtp)")


def build(verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    t0 = time.time()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [cc, *FLAGS]
        if src.endswith(".cpp"):
            cmd += ["-x", "hip"]
        cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    errors = []
    for src, cmd, p in procs:
        out, _ = p.communicate()
        noise = "is not a recognized feature for this target"
        lines = [l for l in out.splitlines() if noise not in l]
        if p.returncode != 0:
            errors.append(f"== {src} (exit {p.returncode})\n" + "\n".join(lines))
        elif verbose and lines:
            print(f"== {src}\n" + "\n".join(lines))
    if errors:
        raise RuntimeError("libtp build failed:\n" + "\n".join(errors))
    tmp = OUT + ".tmp"
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("libtp link failed:\n" + r.stdout)
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT} in {time.time() - t0:.1f}s")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
