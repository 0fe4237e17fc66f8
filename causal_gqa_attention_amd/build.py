"""Build libxattn.so in-tree with hipcc for gfx950.

Usage: python -m causal_gqa_attention_amd.build   (or build() from Python).
Objects go to _build/ at the repository root; the shared library is written next to
this file, where the binding loads it (a copy of the tree carries it along).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libxattn.so")
SOURCES = ["attn.hip", "attn_bf16.hip", "prologue.hip", "decode.hip", "proj.hip", "gemm.hip",
           "xattn_api.cpp", "profile.cpp", "noalloc.hip"]
LINK_LIBS: list = []
# Per-source extra flags.  The attention and decode kernels: MFMA results go to VGPRs (the
# score tiles are consumed by VALU right away; AGPR results would need a copy per element).
SOURCE_FLAGS = {"attn_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
                "attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
                "decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libxattn)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source and link libxattn.so; always recompiles."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    flags = HIPCC_FLAGS + list(extra_flags or [])
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        extra = SOURCE_FLAGS.get(src, [])
        jobs.append((obj, [hipcc, *flags, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]))
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        outs = list(ex.map(lambda j: _run(j[1]), jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[j[0] for j in jobs],
          *LINK_LIBS])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
