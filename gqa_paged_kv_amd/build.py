"""Compile the gpkv HIP library for gfx950 into gqa_paged_kv_amd/libgpkv.so.

Usage: python -m gqa_paged_kv_amd.build [--verbose]

hipcc cross-compiles for gfx950 on a machine without a GPU. Packed-FP32 VALU
instructions are disabled for all device code (-packed-fp32-ops); hipcc's host
pass ignores that feature with a warning.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgpkv.so")
SOURCES = ["status.cpp", "reshape_and_cache.hip", "paged_attention.hip", "varlen.hip", "quest.hip",
           "quest_decode.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def command(out: str = LIB) -> list[str]:
    return [
        HIPCC, "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-fhip-fp32-correctly-rounded-divide-sqrt",
        "-Wno-unused-command-line-argument",
        "-I", INCLUDE, "-I", CSRC,
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out,
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    if verbose and res.stderr.strip():
        lines = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
