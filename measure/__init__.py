"""Measurement-only helpers of the benchmark (not part of the forward path).

libdsa_probe.so (built from mfma_probe.hip by sparse_attention_04_amd/build.py)
issues back-to-back MFMAs with operands in registers at a chosen occupancy and
reads the shader clock against the constant 100 MHz counter, so that a
kernel's MFMA fraction can be set against what the matrix units sustain, and
at what clock, on the same box.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB = os.path.join(_HERE, "libdsa_probe.so")

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_LIB):
            raise ImportError(f"{PROBE_LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(PROBE_LIB)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.dsa_probe_mfma.argtypes = [i32, i32, i32, i32, vp, sz, vp, sz, ctypes.POINTER(ctypes.c_double), vp]
        L.dsa_probe_mfma.restype = i32
        L.dsa_probe_last_error.argtypes = []
        L.dsa_probe_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


class ProbeError(RuntimeError):
    pass


def probe_mfma(kind: int, waves_per_simd: int, iters: int, random_operands: bool = False, sink=None, clocks=None,
               stream=None) -> float:
    """Enqueue the probe (kind 0 = FP8 16x16x128, 1 = BF16 32x32x16) on
    `stream`; returns the launch's FLOPs.  sink: fp32 CUDA tensor, one value
    per wave; clocks: int64 CUDA tensor, two per workgroup (shader cycles,
    100 MHz ticks), or None."""
    import torch
    if sink is None:
        sink = torch.empty(256 * 8 * 4, dtype=torch.float32, device="cuda")
    if stream is None:
        stream = torch.cuda.current_stream()
    flop = ctypes.c_double(0.0)
    st = lib().dsa_probe_mfma(int(kind), int(waves_per_simd), int(iters), int(bool(random_operands)),
                              ctypes.c_void_p(sink.data_ptr()), sink.numel(),
                              None if clocks is None else ctypes.c_void_p(clocks.data_ptr()),
                              0 if clocks is None else clocks.numel(), ctypes.byref(flop),
                              ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise ProbeError(f"dsa_probe_mfma failed with status {st}: {lib().dsa_probe_last_error().decode()}")
    return flop.value


def clock_ghz(clocks) -> float:
    """Mean shader clock of a probe launch from its clocks tensor."""
    c = clocks.view(-1, 2).double().cpu()
    return float(c[:, 0].sum() / c[:, 1].sum() * 0.1)
