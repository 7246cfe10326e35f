"""Python binding of libtgs.so, the ternary group-scaled matmul library for MI355X (gfx950).

The binding only marshals arguments into the C ABI declared in include/tgs.h; every step of
the computation runs in the library's HIP kernels (device calls) or its host packer. PyTorch
provides device memory and streams. If the built library is missing, importing this package
raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtgs.so")

SLOT2 = 1
BASE3 = 2
BINARY = 3
F16 = 1
BF16 = 2
F32 = 3
MAGIC = 0x31534754
VERSION = 1
MAX_M_GEMV = 8
MAX_BATCH = 32

STATUS = {0: "TGS_OK", 1: "TGS_E_NULL", 2: "TGS_E_SHAPE", 3: "TGS_E_ALIGN", 4: "TGS_E_CODE", 5: "TGS_E_LAYOUT",
          6: "TGS_E_BASIS", 7: "TGS_E_SIZE", 8: "TGS_E_DTYPE", 9: "TGS_E_DEVICE"}


class TgsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class Matrix(ctypes.Structure):
    """ctypes mirror of tgs_matrix."""
    _fields_ = [("magic", ctypes.c_uint32), ("version", ctypes.c_uint32), ("layout", ctypes.c_int32),
                ("rotated", ctypes.c_int32), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("code_row_stride", ctypes.c_int64), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python ternary_group_scaled_amd/build.py` "
                      "(or __graft_entry__.build()) first")
_lib = ctypes.CDLL(LIB_PATH)

_i32, _i64, _vp, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
_lib.tgs_code_row_bytes.argtypes = [_i32, _i64]
_lib.tgs_code_row_bytes.restype = _sz
_lib.tgs_matrix_init.argtypes = [ctypes.POINTER(Matrix), _i32, _i32, _i64, _i64, _vp, _vp]
_lib.pack_ternary.argtypes = [_i32, _vp, _vp, _i64, _i64, _vp, _sz, _vp]
_lib.unpack_ternary.argtypes = [ctypes.POINTER(Matrix), _vp, _vp]
_lib.ternary_gemv.argtypes = [ctypes.POINTER(Matrix), _vp, _i32, _i64, _vp, _vp, _vp]
_lib.ternary_gemv_batched.argtypes = [ctypes.POINTER(Matrix), _i32, ctypes.POINTER(_vp), _i32, _i64,
                                      ctypes.POINTER(_vp), ctypes.POINTER(_vp), _vp]
_lib.ternary_gemm.argtypes = [ctypes.POINTER(Matrix), _vp, _i32, _i64, _vp, _vp, _vp]
_lib.hadamard_rotate_g128.argtypes = [_vp, _i32, _i64, _i64, _vp, _vp, _i32, _vp]
_lib.hadamard_rotate.argtypes = [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _i32, _vp]
_lib.ternary_gemv_rmsnorm.argtypes = [ctypes.POINTER(Matrix), _vp, _i32, _i64, _vp, ctypes.c_float, _vp, _vp, _vp]
_lib.ternary_gemv_rmsnorm_batched.argtypes = [ctypes.POINTER(Matrix), _i32, ctypes.POINTER(_vp), _i32, _i64,
                                              ctypes.POINTER(_vp), ctypes.c_float, ctypes.POINTER(_vp),
                                              ctypes.POINTER(_vp), _vp]
_lib.rmsnorm_hadamard_rotate.argtypes = [_vp, _i32, _i64, _i64, _i64, _vp, ctypes.c_float, _vp, _vp, _i32, _vp]
_lib.ternary_code_flips.argtypes = [ctypes.POINTER(Matrix), ctypes.POINTER(Matrix), _vp, _vp, _vp]
_lib.ternary_code_flips_batched.argtypes = [ctypes.POINTER(Matrix), ctypes.POINTER(Matrix), _i32,
                                            ctypes.POINTER(_vp), ctypes.POINTER(_vp), _vp]
for _name in ("tgs_matrix_init", "pack_ternary", "unpack_ternary", "ternary_gemv", "ternary_gemv_batched",
              "ternary_gemm", "hadamard_rotate_g128", "hadamard_rotate", "ternary_code_flips",
              "ternary_code_flips_batched", "ternary_gemv_rmsnorm", "ternary_gemv_rmsnorm_batched",
              "rmsnorm_hadamard_rotate"):
    getattr(_lib, _name).restype = ctypes.c_int
_lib.tgs_status_string.argtypes = [ctypes.c_int]
_lib.tgs_status_string.restype = ctypes.c_char_p
_lib.tgs_last_error.argtypes = []
_lib.tgs_last_error.restype = ctypes.c_char_p

EXPORTS = ("tgs_code_row_bytes", "tgs_matrix_init", "pack_ternary", "unpack_ternary", "ternary_gemv",
           "ternary_gemv_batched", "ternary_gemm", "hadamard_rotate_g128", "hadamard_rotate", "ternary_code_flips",
           "ternary_code_flips_batched", "ternary_gemv_rmsnorm", "ternary_gemv_rmsnorm_batched",
           "rmsnorm_hadamard_rotate", "tgs_status_string", "tgs_last_error")


def _check(status: int):
    if status != 0:
        raise TgsError(status, _lib.tgs_last_error().decode())


def lib() -> ctypes.CDLL:
    return _lib


def status_string(status: int) -> str:
    return _lib.tgs_status_string(status).decode()


def code_row_bytes(layout: int, k: int) -> int:
    return int(_lib.tgs_code_row_bytes(layout, k))


# ------------------------------------------------------------------------------ host packing

def pack_ternary(layout: int, trits: np.ndarray, scales: np.ndarray | None = None):
    """Pack int8 trits [n][k] on the host. Returns (codes uint8 [n][row_bytes], scales fp16 or None)."""
    t = np.ascontiguousarray(trits, dtype=np.int8)
    n, k = t.shape
    rb = code_row_bytes(layout, k)  # 0 for an invalid layout or k: the library reports which
    codes = np.empty((n, rb), dtype=np.uint8)
    s_in = s_out = None
    if scales is not None:
        s_in = np.ascontiguousarray(scales).view(np.uint16)
        s_out = np.empty_like(s_in)
    _check(_lib.pack_ternary(layout, t.ctypes.data, s_in.ctypes.data if s_in is not None else None, n, k,
                             codes.ctypes.data, codes.nbytes, s_out.ctypes.data if s_out is not None else None))
    return codes, (s_out.view(np.float16) if s_out is not None else None)


def host_matrix(layout: int, codes: np.ndarray, scales: np.ndarray, k: int, rotated: bool = False) -> Matrix:
    """Descriptor for host-resident packed data (for unpack_ternary)."""
    m = Matrix()
    _check(_lib.tgs_matrix_init(ctypes.byref(m), layout, int(rotated), codes.shape[0], k, codes.ctypes.data,
                                scales.ctypes.data))
    m.code_row_stride = codes.shape[1]
    return m


def unpack_ternary(layout: int, codes: np.ndarray, scales: np.ndarray, k: int):
    """Unpack host codes [n][stride] back to int8 trits [n][k] (+ a copy of the scales)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(scales).view(np.uint16)
    desc = host_matrix(layout, c, s, k)
    trits = np.empty((c.shape[0], k), dtype=np.int8)
    s_out = np.empty_like(s)
    _check(_lib.unpack_ternary(ctypes.byref(desc), trits.ctypes.data, s_out.ctypes.data))
    return trits, s_out.view(np.float16)


# ------------------------------------------------------------------------------ device calls

def _torch():
    import torch  # imported lazily: host packing works without it
    return torch


def _stream_handle(stream) -> int | None:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class PackedMatrix:
    """Packed ternary weights resident on the GPU: codes [n][stride] uint8, scales [n][k/128] fp16."""

    def __init__(self, layout: int, codes, scales, k: int, rotated=False):
        """rotated: False/0 (plain basis), True/1/128 (128-element rotation blocks) or 1024."""
        self.layout = layout
        self.codes = codes
        self.scales = scales
        self.n = int(codes.shape[0])
        self.k = int(k)
        self.rotated = bool(rotated)
        self.desc = Matrix()
        _check(_lib.tgs_matrix_init(ctypes.byref(self.desc), layout, int(rotated), self.n, self.k,
                                    codes.data_ptr(), scales.data_ptr()))
        self.block = 1024 if self.desc.rotated == 1024 else (128 if self.rotated else 0)
        self.desc.code_row_stride = int(codes.stride(0))

    @classmethod
    def from_trits(cls, layout: int, trits: np.ndarray, scales_f16: np.ndarray, device="cuda", rotated=False):
        torch = _torch()
        codes, scales = pack_ternary(layout, trits, scales_f16)
        return cls(layout, torch.from_numpy(codes).to(device), torch.from_numpy(scales.view(np.int16)).to(device),
                   trits.shape[1], rotated)

    @property
    def nbytes(self) -> int:
        return int(self.codes.numel() + 2 * self.scales.numel())


def ternary_gemv(w: PackedMatrix, x, signs=None, y=None, stream=None):
    """y[m][n] (fp32) = W (R) x for fp16 x [m][k], m <= 8. Returns y."""
    torch = _torch()
    x2 = x.reshape(-1, w.k)
    m = x2.shape[0]
    if y is None:
        y = torch.empty((m, w.n), dtype=torch.float32, device=x.device)
    _check(_lib.ternary_gemv(ctypes.byref(w.desc), x2.data_ptr(), F16, m,
                             signs.data_ptr() if signs is not None else None, y.data_ptr(), _stream_handle(stream)))
    return y


def ternary_gemv_batched(ws, xs, ys, signs=None, stream=None):
    """Independent GEMVs sharing m (fp16 inputs, fp32 outputs), issued as few launches as possible."""
    count = len(ws)
    descs = (Matrix * count)(*[w.desc for w in ws])
    m = xs[0].reshape(-1, ws[0].k).shape[0]
    xp = (_vp * count)(*[x.data_ptr() for x in xs])
    yp = (_vp * count)(*[y.data_ptr() for y in ys])
    sp = None
    if signs is not None:
        sp = (_vp * count)(*[s.data_ptr() if s is not None else None for s in signs])
    _check(_lib.ternary_gemv_batched(descs, count, xp, F16, m, sp, yp, _stream_handle(stream)))
    return ys


def ternary_gemv_rmsnorm(w: PackedMatrix, x, gamma, eps, signs=None, y=None, stream=None):
    """y[m][n] (fp32) = W (R) RMSNorm(x) for fp16 x [m][k], m <= 8; gamma: bf16 [k]. Returns y."""
    torch = _torch()
    x2 = x.reshape(-1, w.k)
    m = x2.shape[0]
    if y is None:
        y = torch.empty((m, w.n), dtype=torch.float32, device=x.device)
    _check(_lib.ternary_gemv_rmsnorm(ctypes.byref(w.desc), x2.data_ptr(), F16, m, gamma.data_ptr(), float(eps),
                                     signs.data_ptr() if signs is not None else None, y.data_ptr(),
                                     _stream_handle(stream)))
    return y


def ternary_gemv_rmsnorm_batched(ws, xs, gammas, eps, ys, signs=None, stream=None):
    """ternary_gemv_batched with the RMSNorm prologue (one bf16 gamma [k] per matrix)."""
    count = len(ws)
    descs = (Matrix * count)(*[w.desc for w in ws])
    m = xs[0].reshape(-1, ws[0].k).shape[0]
    xp = (_vp * count)(*[x.data_ptr() for x in xs])
    gp = (_vp * count)(*[g.data_ptr() for g in gammas])
    yp = (_vp * count)(*[y.data_ptr() for y in ys])
    sp = None
    if signs is not None:
        sp = (_vp * count)(*[s.data_ptr() if s is not None else None for s in signs])
    _check(_lib.ternary_gemv_rmsnorm_batched(descs, count, xp, F16, m, gp, float(eps), sp, yp, _stream_handle(stream)))
    return ys


def rmsnorm_hadamard_rotate(x, gamma, eps, signs, block=128, y=None, out_dtype=None, stream=None):
    """R RMSNorm(x) per row of x [m][k] (fp16/bf16/fp32), gamma bf16 [k]; fp16/bf16/fp32 output."""
    torch = _torch()
    dt = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}
    k = x.shape[-1]
    x2 = x.reshape(-1, k)
    if y is None:
        y = torch.empty(x2.shape, dtype=out_dtype or torch.float32, device=x.device)
    _check(_lib.rmsnorm_hadamard_rotate(x2.data_ptr(), dt[x2.dtype], x2.shape[0], k, block, gamma.data_ptr(),
                                        float(eps), signs.data_ptr(), y.data_ptr(), dt[y.dtype],
                                        _stream_handle(stream)))
    return y


def ternary_gemm(w: PackedMatrix, x, y=None, stream=None):
    """y[m][n] (fp32) = W x for bf16 x [m][k]. Returns y."""
    torch = _torch()
    x2 = x.reshape(-1, w.k)
    m = x2.shape[0]
    if y is None:
        y = torch.empty((m, w.n), dtype=torch.float32, device=x.device)
    _check(_lib.ternary_gemm(ctypes.byref(w.desc), x2.data_ptr(), BF16, m, None, y.data_ptr(), _stream_handle(stream)))
    return y


def hadamard_rotate(x, signs, block=128, y=None, out_dtype=None, stream=None):
    """Block-wise signed Walsh-Hadamard rotation (128 or 1024 per block) of x [m][k]; fp16/bf16/fp32
    output."""
    torch = _torch()
    dt = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}
    k = x.shape[-1]
    x2 = x.reshape(-1, k)
    if y is None:
        y = torch.empty(x2.shape, dtype=out_dtype or torch.float32, device=x.device)
    _check(_lib.hadamard_rotate(x2.data_ptr(), dt[x2.dtype], x2.shape[0], k, block, signs.data_ptr(), y.data_ptr(),
                                dt[y.dtype], _stream_handle(stream)))
    return y


def hadamard_rotate_g128(x, signs, y=None, out_dtype=None, stream=None):
    """Block-wise signed Walsh-Hadamard rotation (128 per block) of x [m][k]; fp16/bf16/fp32 output."""
    torch = _torch()
    dt = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}
    k = x.shape[-1]
    x2 = x.reshape(-1, k)
    if y is None:
        y = torch.empty(x2.shape, dtype=out_dtype or torch.float32, device=x.device)
    _check(_lib.hadamard_rotate_g128(x2.data_ptr(), dt[x2.dtype], x2.shape[0], k, signs.data_ptr(), y.data_ptr(),
                                     dt[y.dtype], _stream_handle(stream)))
    return y


def ternary_code_flips(a: PackedMatrix, b: PackedMatrix, rows=True, total=True, stream=None):
    """Code flips between two packed matrices on the GPU: (total uint64 [1] or None,
    per-row counts int32 [n] holding uint32 values, or None)."""
    torch = _torch()
    dev = a.codes.device
    r = torch.empty(a.n, dtype=torch.int32, device=dev) if rows else None
    t = torch.empty(1, dtype=torch.int64, device=dev) if total else None
    _check(_lib.ternary_code_flips(ctypes.byref(a.desc), ctypes.byref(b.desc), r.data_ptr() if r is not None else None,
                                   t.data_ptr() if t is not None else None, _stream_handle(stream)))
    return t, r


def ternary_code_flips_batched(pairs, totals, rows=None, stream=None):
    """Code flips of several pairs (a, b) of one layout in one launch. totals: int64 [1] tensors
    (or None entries); rows: int32 [n] tensors (or None entries), or None."""
    count = len(pairs)
    da = (Matrix * count)(*[a.desc for a, _ in pairs])
    db = (Matrix * count)(*[b.desc for _, b in pairs])
    tp = (_vp * count)(*[t.data_ptr() if t is not None else None for t in totals])
    rp = None
    if rows is not None:
        rp = (_vp * count)(*[r.data_ptr() if r is not None else None for r in rows])
    _check(_lib.ternary_code_flips_batched(da, db, count, rp, tp, _stream_handle(stream)))
    return totals, rows
