"""CPU oracle for the ternary group-scaled matmul — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg
may import this package. It is a thin ctypes wrapper over ``oracle.c`` (plain C,
fp64, bit-by-bit packing loops, dense Hadamard rotation), which shares no code
with the GPU library. See ``oracle.c`` for what each function computes and which
page passage it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
# A test may point the wrapper at a deliberately broken copy of the oracle (see
# tests/test_oracle_mutants.py) to show that the pins catch planted mistakes.
_SO_OVERRIDE = os.environ.get("TGS_ORACLE_SO")
_lib = None

SLOT2 = 1
BASE3 = 2
BINARY = 3
X_F16 = 1
X_BF16 = 2

OK = 0
BAD_CODE = -1
BAD_SHAPE = -2
BAD_LAYOUT = -3


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    if force or not os.path.exists(_SO):
        cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", _SO + ".tmp",
               os.path.join(_HERE, "oracle.c"), "-lm"]
        subprocess.check_call(cmd)
        os.replace(_SO + ".tmp", _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if _SO_OVERRIDE:
            lib = ctypes.CDLL(_SO_OVERRIDE)
        else:
            if not os.path.exists(_SO):
                build(force=False)
            lib = ctypes.CDLL(_SO)
        i32, i64, vp, dbl, u16 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double, ctypes.c_uint16
        lib.orc_f16_to_f64.argtypes = [u16]
        lib.orc_f16_to_f64.restype = dbl
        lib.orc_bf16_to_f64.argtypes = [u16]
        lib.orc_bf16_to_f64.restype = dbl
        lib.orc_row_bytes.argtypes = [i32, i64]
        lib.orc_row_bytes.restype = i64
        for name in ("orc_pack_slot2", "orc_unpack_slot2", "orc_pack_base3", "orc_unpack_base3", "orc_pack_binary",
                     "orc_unpack_binary"):
            f = getattr(lib, name)
            f.argtypes = [vp, i64, i64, vp]
            f.restype = ctypes.c_int
        lib.orc_hadamard.argtypes = [i32, vp]
        lib.orc_hadamard.restype = None
        lib.orc_rotate_f64.argtypes = [vp, vp, i64, i64, i64, vp]
        lib.orc_rotate_f64.restype = None
        lib.orc_matmul_f64.argtypes = [i32, vp, i64, vp, i64, i64, vp, i32, i64, vp, i64, vp, i64, vp, vp]
        lib.orc_matmul_f64.restype = ctypes.c_int
        lib.orc_matmul_norm_f64.argtypes = [i32, vp, i64, vp, i64, i64, vp, i32, i64, vp, dbl, vp, i64, vp, i64, vp,
                                            vp]
        lib.orc_matmul_norm_f64.restype = ctypes.c_int
        lib.orc_rmsnorm_f64.argtypes = [vp, vp, dbl, i64, i64, vp]
        lib.orc_rmsnorm_f64.restype = ctypes.c_int
        lib.orc_rmsnorm_rotate_f64.argtypes = [vp, i32, vp, dbl, vp, i64, i64, i64, vp]
        lib.orc_rmsnorm_rotate_f64.restype = ctypes.c_int
        lib.orc_code_flips.argtypes = [i32, vp, i64, vp, i64, i64, i64, vp]
        lib.orc_code_flips.restype = i64
        _lib = lib
    return _lib


def _check(rc: int, what: str):
    if rc != OK:
        raise OracleError(f"{what}: oracle status {rc}")


def f16_to_f64(bits: int) -> float:
    return _load().orc_f16_to_f64(int(bits))


def bf16_to_f64(bits: int) -> float:
    return _load().orc_bf16_to_f64(int(bits))


def row_bytes(layout: int, k: int) -> int:
    return int(_load().orc_row_bytes(layout, k))


def pack(layout: int, trits: np.ndarray) -> np.ndarray:
    """trits int8 [n][k] -> codes uint8 [n][row_bytes] (binary: values must be -1 or +1)."""
    t = np.ascontiguousarray(trits, dtype=np.int8)
    n, k = t.shape
    rb = row_bytes(layout, k)
    if rb == 0:
        raise OracleError("bad layout or k")
    out = np.zeros((n, rb), dtype=np.uint8)
    fn = {SLOT2: _load().orc_pack_slot2, BASE3: _load().orc_pack_base3, BINARY: _load().orc_pack_binary}[layout]
    _check(fn(t.ctypes.data, n, k, out.ctypes.data), "pack")
    return out


def unpack(layout: int, codes: np.ndarray, k: int) -> np.ndarray:
    """codes uint8 [n][row_bytes] -> trits int8 [n][k]."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    n = c.shape[0]
    if c.shape[1] != row_bytes(layout, k):
        raise OracleError("codes row length does not match k")
    out = np.zeros((n, k), dtype=np.int8)
    fn = {SLOT2: _load().orc_unpack_slot2, BASE3: _load().orc_unpack_base3, BINARY: _load().orc_unpack_binary}[layout]
    _check(fn(c.ctypes.data, n, k, out.ctypes.data), "unpack")
    return out


def hadamard(n: int = 128) -> np.ndarray:
    h = np.zeros((n, n), dtype=np.int8)
    _load().orc_hadamard(n, h.ctypes.data)
    return h


def rotate(x: np.ndarray, signs: np.ndarray, block: int = 128) -> np.ndarray:
    """x float64 [m][k] (or [k]) -> R x per block of `block` (128 or 1024) elements, float64."""
    xd = np.ascontiguousarray(x, dtype=np.float64)
    shape = xd.shape
    xd = xd.reshape(-1, shape[-1])
    m, k = xd.shape
    s = np.ascontiguousarray(signs, dtype=np.int8)
    assert s.shape == (k,) and block in (128, 1024) and k % block == 0
    out = np.zeros_like(xd)
    _load().orc_rotate_f64(xd.ctypes.data, s.ctypes.data, m, k, block, out.ctypes.data)
    return out.reshape(shape)


def rmsnorm(x: np.ndarray, gamma_bits: np.ndarray, eps: float) -> np.ndarray:
    """x float64 [m][k] -> gamma * x / sqrt(mean(x^2) + eps) per row; gamma as bf16 bits [k]."""
    xd = np.ascontiguousarray(x, dtype=np.float64)
    shape = xd.shape
    xd = xd.reshape(-1, shape[-1])
    g = np.ascontiguousarray(gamma_bits).view(np.uint16)
    assert g.shape == (xd.shape[1],)
    out = np.zeros_like(xd)
    _check(_load().orc_rmsnorm_f64(xd.ctypes.data, g.ctypes.data, float(eps), xd.shape[0], xd.shape[1],
                                   out.ctypes.data), "rmsnorm")
    return out.reshape(shape)


def rmsnorm_rotate(x_bits: np.ndarray, x_dtype: int, gamma_bits: np.ndarray, eps: float,
                   signs: np.ndarray | None, block: int = 128) -> np.ndarray:
    """The fused operation R (RMSNorm x) (or RMSNorm x when signs is None), float64 [m][k]."""
    xb = np.ascontiguousarray(x_bits).view(np.uint16)
    xb = xb.reshape(-1, xb.shape[-1])
    m, k = xb.shape
    g = np.ascontiguousarray(gamma_bits).view(np.uint16)
    sg = None if signs is None else np.ascontiguousarray(signs, dtype=np.int8)
    out = np.zeros((m, k), dtype=np.float64)
    _check(_load().orc_rmsnorm_rotate_f64(xb.ctypes.data, x_dtype, g.ctypes.data, float(eps),
                                          sg.ctypes.data if sg is not None else None, m, k, block,
                                          out.ctypes.data), "rmsnorm_rotate")
    return out


def matmul(layout: int, codes: np.ndarray, scales: np.ndarray, k: int, x_bits: np.ndarray,
           x_dtype: int, signs: np.ndarray | None = None, rows: np.ndarray | None = None, block: int = 128,
           gamma: np.ndarray | None = None, eps: float = 0.0):
    """Reference product. Returns (y, bound), both float64 [m][n_sel].

    codes uint8 [n][stride]; scales fp16 (float16 or uint16 bits) [n][k/128];
    x_bits uint16 bit patterns [m][k] (fp16 or bf16 per x_dtype); signs int8 [k] or None;
    rows: int64 row indices to evaluate, or None for all rows; block: rotation block (128 or
    1024) when signs are given; gamma: bf16 bits [k] to RMS-normalise x first (with eps > 0).
    """
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    n, stride = c.shape
    s = np.ascontiguousarray(scales).view(np.uint16)
    assert s.shape == (n, k // 128)
    xb = np.ascontiguousarray(x_bits).view(np.uint16)
    xb = xb.reshape(-1, k)
    m = xb.shape[0]
    if rows is None:
        r_ptr, n_sel = None, n
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        r_ptr, n_sel = rows.ctypes.data, rows.size
    sg = None
    if signs is not None:
        sg = np.ascontiguousarray(signs, dtype=np.int8)
        assert sg.shape == (k,)
    g = None
    if gamma is not None:
        g = np.ascontiguousarray(gamma).view(np.uint16)
        assert g.shape == (k,)
    y = np.zeros((m, n_sel), dtype=np.float64)
    bound = np.zeros((m, n_sel), dtype=np.float64)
    rc = _load().orc_matmul_norm_f64(layout, c.ctypes.data, stride, s.ctypes.data, n, k, xb.ctypes.data,
                                     x_dtype, m, g.ctypes.data if g is not None else None, float(eps),
                                     sg.ctypes.data if sg is not None else None, block, r_ptr, n_sel,
                                     y.ctypes.data, bound.ctypes.data)
    _check(rc, "matmul")
    return y, bound


def code_flips(layout: int, codes_a: np.ndarray, codes_b: np.ndarray, k: int):
    """Code flips between two packed matrices: (total, per-row counts int64 [n]).

    codes_a, codes_b: uint8 [n][stride_a], [n][stride_b] of the same layout and k.
    """
    a = np.ascontiguousarray(codes_a, dtype=np.uint8)
    b = np.ascontiguousarray(codes_b, dtype=np.uint8)
    n = a.shape[0]
    assert b.shape[0] == n
    counts = np.zeros(n, dtype=np.int64)
    total = _load().orc_code_flips(layout, a.ctypes.data, a.shape[1], b.ctypes.data, b.shape[1], n, k,
                                   counts.ctypes.data)
    if total < 0:
        raise OracleError(f"code_flips: oracle status {total}")
    return int(total), counts
