"""Seeded synthetic inputs shared by the GPU path's tests/bench and the CPU oracle.

Nothing here computes any part of the ternary matmul: the module draws ternary
codes, normals and signs (SplitMix64 in counter form, Box-Muller normals; see
synth.c) and rounds them to the storage dtypes with IEEE round-to-nearest-even.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile synth.c into libsynth.so next to it."""
    if force or not os.path.exists(_SO):
        cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", _SO + ".tmp",
               os.path.join(_HERE, "synth.c"), "-lm"]
        subprocess.check_call(cmd)
        os.replace(_SO + ".tmp", _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        lib = ctypes.CDLL(_SO)
        i64, u64, dbl, vp = ctypes.c_int64, ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p
        lib.synth_trits.argtypes = [u64, u64, i64, dbl, vp]
        lib.synth_normal.argtypes = [u64, u64, i64, vp]
        lib.synth_signs.argtypes = [u64, u64, i64, vp]
        lib.synth_u64.argtypes = [u64, u64, u64]
        lib.synth_u64.restype = u64
        for f in (lib.synth_trits, lib.synth_normal, lib.synth_signs):
            f.restype = None
        _lib = lib
    return _lib


def stream_id(*parts) -> int:
    """Stable 64-bit stream id (FNV-1a over the text of the parts)."""
    h = 0xCBF29CE484222325
    for byte in "/".join(str(p) for p in parts).encode():
        h ^= byte
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def trits(seed: int, stream: int, shape, p_zero: float) -> np.ndarray:
    """iid codes in {-1, 0, +1}: P(0) = p_zero, P(-1) = P(+1) = (1 - p_zero) / 2."""
    out = np.empty(shape, dtype=np.int8)
    _load().synth_trits(seed, stream, out.size, float(p_zero), out.ctypes.data)
    return out


def normal(seed: int, stream: int, shape) -> np.ndarray:
    out = np.empty(shape, dtype=np.float64)
    _load().synth_normal(seed, stream, out.size, out.ctypes.data)
    return out


def signs(seed: int, stream: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.int8)
    _load().synth_signs(seed, stream, count, out.ctypes.data)
    return out


def f16(values: np.ndarray) -> np.ndarray:
    """Round doubles to IEEE binary16 (round to nearest even); returns float16."""
    return np.asarray(values, dtype=np.float64).astype(np.float16)


def bf16_bits(values: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (via float32, each step round-to-nearest-even); returns uint16 bits."""
    f = np.asarray(values, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(f)
    rounded = np.where(nan, (u >> 16) | 0x40, rounded)
    return rounded.astype(np.uint16)


def scales_f16(seed: int, stream: int, shape, sigma: float = 0.02, offset: float = 1e-4) -> np.ndarray:
    """Group scales |N(0, sigma)| + offset rounded to fp16."""
    return f16(np.abs(normal(seed, stream, shape)) * sigma + offset)


def x_f16(seed: int, stream: int, shape) -> np.ndarray:
    """Activations N(0, 1) rounded to fp16."""
    return f16(normal(seed, stream, shape))


def x_bf16_bits(seed: int, stream: int, shape) -> np.ndarray:
    """Activations N(0, 1) rounded to bf16; returned as uint16 bit patterns."""
    return bf16_bits(normal(seed, stream, shape))
