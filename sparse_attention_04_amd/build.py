"""Build ``libdsa.so`` (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m sparse_attention_04_amd.build      # or build() from Python
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdsa.so")
SOURCES = ["dsa_capi.cpp", "indexer.hip", "topk.hip", "sparse_attn.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdsa.so)")


def command(out: str = LIB, extra=()) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 VALU forms are disabled on purpose: plain v_fma/v_mul only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
        "-I", os.path.join(os.path.dirname(HERE), "include"),
        *extra,
        "-o", out,
        "-x", "hip", *[os.path.join(CSRC, s) for s in SOURCES],
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; drop that noise
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
