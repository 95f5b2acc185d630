"""Compile the HIP library ``libkda.so`` (C ABI of include/kda.h) for gfx950.

Run ``python -m gated_delta_rule_88_amd.build``; the library lands in
``gated_delta_rule_88_amd/_build/`` next to the package so that it travels
with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(BUILD, "libkda.so")
SOURCES = ["kda_api.cpp", "kda_noalloc.hip", "kda_decode.hip", "kda_prefill.hip", "kda_prefill_bf16.hip", "kda_backward.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkda)")


def compile_flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # keep the compiler from forming packed-fp32 instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Wall", "-Wno-unused-function",
    ]


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libkda.so``; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [cc] + compile_flags() + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        noise = [ln for ln in (r.stderr or "").splitlines() if "packed-fp32-ops" not in ln]
        if r.returncode != 0:
            raise RuntimeError(f"compiling {src} failed:\n" + "\n".join(noise))
        if verbose and noise:
            print("\n".join(noise), flush=True)
        objs.append(obj)
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("linking libkda.so failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
