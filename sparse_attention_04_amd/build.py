"""Build ``libdsa.so`` (the C-ABI library) for gfx950 with hipcc, in-tree.

    python sparse_attention_04_amd/build.py      # or build() from Python
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdsa.so")
OBJ_DIR = os.path.join(HERE, "_build")
ARCH = "gfx950"
# Per-source extra flags.  The indexer's MFMA results are consumed by vector
# fmas at once, so its MFMAs are built in the VGPR-destination form (an AGPR
# destination would need a copy-out instruction per element).  So are the
# 64/128-wide attention kernel's: its accumulators fit the VGPRs, and in AGPRs
# the compiler moved two O tiles out and back around every chunk's Q.K (4.5%
# of the kernel).  The 576/512 attention kernels keep their 256 accumulators
# in AGPRs.
SOURCES = [
    ("dsa_capi.cpp", []),
    ("indexer.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form"]),
    ("topk.hip", []),
    ("select.hip", []),
    ("sparse_attn.hip", []),
    ("attn_mla.hip", []),
    ("attn_mqa.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form"]),
    ("inputs.hip", []),
    ("kl.hip", []),
    ("attn_bwd.hip", []),
]
# The measurement-only MFMA / clock probe: a library of its own, which the
# benchmark loads; the forward path's library does not contain it.
PROBE_SRC = os.path.join(os.path.dirname(HERE), "measure", "mfma_probe.hip")
PROBE_LIB = os.path.join(os.path.dirname(HERE), "measure", "libdsa_probe.so")
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are disabled on purpose: plain v_fma/v_mul only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    "-I", os.path.join(os.path.dirname(HERE), "include"),
]
# hipcc's host pass does not know the packed-fp32 feature; that warning is noise
_NOISE = "'-packed-fp32-ops' is not a recognized feature"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdsa.so)")


def compile_command(src: str, obj: str, extra=()) -> list:
    flags = dict(SOURCES).get(src, [])
    path = src if os.path.isabs(src) else os.path.join(CSRC, src)
    return [hipcc(), *COMMON, *flags, *extra, "-c", "-x", "hip", path, "-o", obj]


def link_command(objs, out: str) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out, *objs]


def _run(cmds, verbose: bool):
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    errors = []
    for cmd, p in procs:
        out, err = p.communicate()
        err = "\n".join(l for l in err.splitlines() if _NOISE not in l)
        if p.returncode != 0:
            errors.append(f"{' '.join(cmd)}\n(exit {p.returncode}):\n{err}")
        elif verbose and err.strip():
            print(err, file=sys.stderr)
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n\n".join(errors))


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 (in parallel), link libdsa.so and the
    probe library."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = [os.path.join(OBJ_DIR, os.path.splitext(s)[0] + ".o") for s, _ in SOURCES]
    probe_obj = os.path.join(OBJ_DIR, "mfma_probe.o")
    _run([compile_command(s, o) for (s, _), o in zip(SOURCES, objs)] + [compile_command(PROBE_SRC, probe_obj)],
         verbose)
    for out, ins in ((LIB, objs), (PROBE_LIB, [probe_obj])):
        tmp = out + ".tmp"
        _run([link_command(ins, tmp)], verbose)
        os.replace(tmp, out)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
