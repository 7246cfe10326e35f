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


CHAIN_MAX_STEPS = 16
CHAIN_MAX_MATRICES = 3


class ChainStep(ctypes.Structure):
    """ctypes mirror of tgs_chain_step."""
    _fields_ = [("count", ctypes.c_int32), ("x_dtype", ctypes.c_int32), ("norm", ctypes.c_int32),
                ("eps", ctypes.c_float), ("x", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("w", Matrix * CHAIN_MAX_MATRICES), ("y", ctypes.c_void_p * CHAIN_MAX_MATRICES)]


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
_lib.ternary_gemm_ws.argtypes = [ctypes.POINTER(Matrix), _vp, _i32, _i64, _vp, _vp, _vp, _sz, _vp]
_lib.ternary_gemm_workspace_size.argtypes = [ctypes.POINTER(Matrix), _i64]
_lib.ternary_gemm_workspace_size.restype = _sz
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
              "ternary_gemm", "ternary_gemm_ws", "hadamard_rotate_g128", "hadamard_rotate", "ternary_code_flips",
              "ternary_code_flips_batched", "ternary_gemv_rmsnorm", "ternary_gemv_rmsnorm_batched",
              "rmsnorm_hadamard_rotate"):
    getattr(_lib, _name).restype = ctypes.c_int
_lib.tgs_chain_workspace_bytes.argtypes = []
_lib.tgs_chain_workspace_bytes.restype = _sz
_lib.ternary_gemv_chain.argtypes = [ctypes.POINTER(ChainStep), _i32, _vp, _sz, _vp]
_lib.ternary_gemv_chain.restype = ctypes.c_int
_lib.ternary_gemv_chain_static.argtypes = [ctypes.POINTER(ChainStep), _i32, _vp, _vp]
_lib.ternary_gemv_chain_static.restype = ctypes.c_int
_lib.tgs_stream_read_sink_words.argtypes = []
_lib.tgs_stream_read_sink_words.restype = _sz
_lib.tgs_stream_read.argtypes = [_vp, _sz, _vp, _vp]
_lib.tgs_stream_read.restype = ctypes.c_int
_lib.tgs_status_string.argtypes = [ctypes.c_int]
_lib.tgs_status_string.restype = ctypes.c_char_p
_lib.tgs_last_error.argtypes = []
_lib.tgs_last_error.restype = ctypes.c_char_p

EXPORTS = ("tgs_code_row_bytes", "tgs_matrix_init", "pack_ternary", "unpack_ternary", "ternary_gemv",
           "ternary_gemv_batched", "ternary_gemm", "ternary_gemm_ws", "ternary_gemm_workspace_size",
           "hadamard_rotate_g128", "hadamard_rotate", "ternary_code_flips",
           "ternary_code_flips_batched", "ternary_gemv_rmsnorm", "ternary_gemv_rmsnorm_batched",
           "rmsnorm_hadamard_rotate", "tgs_chain_workspace_bytes", "ternary_gemv_chain", "ternary_gemv_chain_static",
           "tgs_stream_read_sink_words", "tgs_stream_read", "tgs_status_string", "tgs_last_error")


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
#
# The C ABI sees raw pointers only, so it cannot know a buffer's size, type or device: the wrappers
# below check every tensor before the call (dtype, element count, contiguity, then device), and
# raise TgsError with the status the library uses for that kind of error. A rejected call queues
# nothing.

_CODE = {name: code for code, name in STATUS.items()}


def _torch():
    import torch  # imported lazily: host packing works without it
    return torch


def _stream_handle(stream) -> int | None:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _raise(name: str, message: str):
    raise TgsError(_CODE[name], message)


def _need(t, what: str, dtypes, numel: int | None = None, min_numel: int | None = None):
    """Check one tensor argument of a device call: dtype, element count, contiguity."""
    if t is None:
        _raise("TGS_E_NULL", f"{what} is None")
    if t.dtype not in dtypes:
        _raise("TGS_E_DTYPE", f"{what} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        _raise("TGS_E_SHAPE", f"{what} holds {t.numel()} elements, expected {numel}")
    if min_numel is not None and t.numel() < min_numel:
        _raise("TGS_E_SIZE", f"{what} holds {t.numel()} elements, needs at least {min_numel}")
    if not t.is_contiguous():
        _raise("TGS_E_SHAPE", f"{what} must be contiguous")


def _on_device(device, **tensors):
    """Every tensor argument must be device memory of the call's device (checked last, so that a
    call with host tensors still reports its other argument errors first)."""
    for what, t in tensors.items():
        if t is not None and (not t.is_cuda or t.device != device):
            _raise("TGS_E_DEVICE", f"{what} is on {t.device}; the call runs on {device} (device memory only)")


def _signs_ok(signs, k: int):
    if signs is not None:
        _need(signs, "signs", (_torch().int8,), numel=k)


def _gamma_ok(gamma, k: int):
    torch = _torch()
    _need(gamma, "gamma", (torch.bfloat16, torch.int16), numel=k)


class PackedMatrix:
    """Packed ternary weights resident on the GPU: codes [n][stride] uint8, scales [n][k/128] fp16."""

    def __init__(self, layout: int, codes, scales, k: int, rotated=False):
        """rotated: False/0 (plain basis), True/1/128 (128-element rotation blocks) or 1024."""
        torch = _torch()
        if codes.dtype != torch.uint8 or codes.dim() != 2 or codes.stride(1) != 1:
            _raise("TGS_E_SHAPE", "codes must be a uint8 [n][stride] tensor with contiguous rows")
        if scales.dtype not in (torch.float16, torch.int16) or not scales.is_contiguous():
            _raise("TGS_E_DTYPE", "scales must be a contiguous fp16 (or int16 bit-pattern) tensor")
        if scales.numel() != codes.shape[0] * (int(k) // 128) or scales.device != codes.device:
            _raise("TGS_E_SHAPE", "scales must hold n * k / 128 values on the codes' device")
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
    def device(self):
        return self.codes.device

    @property
    def nbytes(self) -> int:
        return int(self.codes.numel() + 2 * self.scales.numel())


def _rows_of(x, k: int, what: str = "x") -> int:
    if x is None:
        _raise("TGS_E_NULL", f"{what} is None")
    if k <= 0 or x.numel() % k != 0 or x.numel() == 0:
        _raise("TGS_E_SHAPE", f"{what} holds {x.numel()} elements, not a positive multiple of k = {k}")
    return x.numel() // k


def _out(y, m: int, n: int, device):
    """The fp32 output [m][n]: allocated on the call's device when y is None, else checked."""
    torch = _torch()
    if y is None:
        return torch.empty((m, n), dtype=torch.float32, device=device)
    _need(y, "y", (torch.float32,), min_numel=m * n)
    return y


def ternary_gemv(w: PackedMatrix, x, signs=None, y=None, stream=None):
    """y[m][n] (fp32) = W (R) x for fp16 x [m][k], m <= 8. Returns y."""
    torch = _torch()
    m = _rows_of(x, w.k)
    _need(x, "x", (torch.float16,))
    _signs_ok(signs, w.k)
    y = _out(y, m, w.n, w.device)
    _on_device(w.device, codes=w.codes, scales=w.scales, x=x, signs=signs, y=y)
    _check(_lib.ternary_gemv(ctypes.byref(w.desc), x.data_ptr(), F16, m,
                             signs.data_ptr() if signs is not None else None, y.data_ptr(), _stream_handle(stream)))
    return y


def _batched_ptrs(ws, xs, ys, signs, gammas=None):
    """Checks and pointer arrays of a batched call: m is taken from xs[0], and every x must then
    hold m * k_i fp16 values, every y at least m * n_i fp32 values."""
    torch = _torch()
    count = len(ws)
    if count == 0 or len(xs) != count or len(ys) != count:
        _raise("TGS_E_SHAPE", "ws, xs and ys must be non-empty lists of one length")
    if signs is not None and len(signs) != count:
        _raise("TGS_E_SHAPE", "signs must have one entry per matrix")
    m = _rows_of(xs[0], ws[0].k, "xs[0]")
    for i, (w, x, y) in enumerate(zip(ws, xs, ys)):
        _need(x, f"xs[{i}]", (torch.float16,), numel=m * w.k)
        _need(y, f"ys[{i}]", (torch.float32,), min_numel=m * w.n)
        if signs is not None:
            _signs_ok(signs[i], w.k)
        if gammas is not None:
            _gamma_ok(gammas[i], w.k)
    for i, (w, x, y) in enumerate(zip(ws, xs, ys)):
        _on_device(ws[0].device, codes=w.codes, scales=w.scales, x=x, y=y,
                   signs=signs[i] if signs is not None else None, gamma=gammas[i] if gammas is not None else None)
    descs = (Matrix * count)(*[w.desc for w in ws])
    xp = (_vp * count)(*[x.data_ptr() for x in xs])
    yp = (_vp * count)(*[y.data_ptr() for y in ys])
    sp = None
    if signs is not None:
        sp = (_vp * count)(*[s.data_ptr() if s is not None else None for s in signs])
    gp = None
    if gammas is not None:
        gp = (_vp * count)(*[g.data_ptr() for g in gammas])
    return count, m, descs, xp, yp, sp, gp


def ternary_gemv_batched(ws, xs, ys, signs=None, stream=None):
    """Independent GEMVs sharing m (fp16 inputs, fp32 outputs), issued as few launches as possible."""
    count, m, descs, xp, yp, sp, _ = _batched_ptrs(ws, xs, ys, signs)
    _check(_lib.ternary_gemv_batched(descs, count, xp, F16, m, sp, yp, _stream_handle(stream)))
    return ys


def ternary_gemv_rmsnorm(w: PackedMatrix, x, gamma, eps, signs=None, y=None, stream=None):
    """y[m][n] (fp32) = W (R) RMSNorm(x) for fp16 x [m][k], m <= 8; gamma: bf16 [k]. Returns y."""
    torch = _torch()
    m = _rows_of(x, w.k)
    _need(x, "x", (torch.float16,))
    _gamma_ok(gamma, w.k)
    _signs_ok(signs, w.k)
    y = _out(y, m, w.n, w.device)
    _on_device(w.device, codes=w.codes, scales=w.scales, x=x, gamma=gamma, signs=signs, y=y)
    _check(_lib.ternary_gemv_rmsnorm(ctypes.byref(w.desc), x.data_ptr(), F16, m, gamma.data_ptr(), float(eps),
                                     signs.data_ptr() if signs is not None else None, y.data_ptr(),
                                     _stream_handle(stream)))
    return y


def ternary_gemv_rmsnorm_batched(ws, xs, gammas, eps, ys, signs=None, stream=None):
    """ternary_gemv_batched with the RMSNorm prologue (one bf16 gamma [k] per matrix)."""
    if gammas is None or len(gammas) != len(ws):
        _raise("TGS_E_NULL", "one gamma per matrix is required")
    count, m, descs, xp, yp, sp, gp = _batched_ptrs(ws, xs, ys, signs, gammas)
    _check(_lib.ternary_gemv_rmsnorm_batched(descs, count, xp, F16, m, gp, float(eps), sp, yp, _stream_handle(stream)))
    return ys


def _float_dtypes():
    torch = _torch()
    return {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}


def _rotation_args(x, signs, y, out_dtype, gamma=None):
    dt = _float_dtypes()
    if x is None:
        _raise("TGS_E_NULL", "x is None")
    if x.dim() < 1:
        _raise("TGS_E_SHAPE", "x must have a last dimension k")
    k = x.shape[-1]
    m = _rows_of(x, k)
    _need(x, "x", tuple(dt))
    if signs is None:
        _raise("TGS_E_NULL", "signs are required")
    _signs_ok(signs, k)
    if gamma is not None:
        _gamma_ok(gamma, k)
    if y is None:
        y = _torch().empty((m, k), dtype=out_dtype or _torch().float32, device=x.device)
    else:
        _need(y, "y", tuple(dt), min_numel=m * k)
    _on_device(x.device, x=x, signs=signs, gamma=gamma, y=y)
    return dt, k, m, y


def rmsnorm_hadamard_rotate(x, gamma, eps, signs, block=128, y=None, out_dtype=None, stream=None):
    """R RMSNorm(x) per row of x [m][k] (fp16/bf16/fp32), gamma bf16 [k]; fp16/bf16/fp32 output."""
    if gamma is None:
        _raise("TGS_E_NULL", "gamma is None")
    dt, k, m, y = _rotation_args(x, signs, y, out_dtype, gamma)
    _check(_lib.rmsnorm_hadamard_rotate(x.data_ptr(), dt[x.dtype], m, k, block, gamma.data_ptr(), float(eps),
                                        signs.data_ptr(), y.data_ptr(), dt[y.dtype], _stream_handle(stream)))
    return y


def gemm_workspace_bytes(w: PackedMatrix, m: int) -> int:
    """Bytes of workspace the split product (ternary_gemm_ws) uses for W and m rows; 0: not split."""
    return int(_lib.ternary_gemm_workspace_size(ctypes.byref(w.desc), int(m)))


def ternary_gemm(w: PackedMatrix, x, y=None, stream=None, workspace=None, split=True):
    """y[m][n] (fp32) = W x for bf16 x [m][k]. Returns y.

    split: a product that would leave compute units idle splits K across workgroups, with the
    parts' sums in a workspace: `workspace` (a device tensor of at least gemm_workspace_bytes(w, m)
    bytes, used by no other call at the same time) or, when None, a temporary from torch's
    allocator on the call's stream. split=False: the single-launch product (ternary_gemm).
    """
    torch = _torch()
    m = _rows_of(x, w.k)
    _need(x, "x", (torch.bfloat16,))
    y = _out(y, m, w.n, w.device)
    _on_device(w.device, codes=w.codes, scales=w.scales, x=x, y=y)
    handle = _stream_handle(stream)
    need = gemm_workspace_bytes(w, m) if split else 0
    if need == 0:
        _check(_lib.ternary_gemm(ctypes.byref(w.desc), x.data_ptr(), BF16, m, None, y.data_ptr(), handle))
        return y
    if workspace is None:
        on = stream if isinstance(stream, torch.cuda.Stream) else (
            torch.cuda.current_stream(w.device) if stream is None else torch.cuda.ExternalStream(handle, device=w.device))
        with torch.cuda.stream(on):
            workspace = torch.empty((need + 3) // 4, dtype=torch.float32, device=w.device)
    elif workspace.numel() * workspace.element_size() < need or not workspace.is_contiguous():
        _raise("TGS_E_SIZE", f"workspace must be a contiguous tensor of at least {need} bytes")
    _on_device(w.device, workspace=workspace)
    _check(_lib.ternary_gemm_ws(ctypes.byref(w.desc), x.data_ptr(), BF16, m, None, y.data_ptr(), workspace.data_ptr(),
                                workspace.numel() * workspace.element_size(), handle))
    return y


def hadamard_rotate(x, signs, block=128, y=None, out_dtype=None, stream=None):
    """Block-wise signed Walsh-Hadamard rotation (128 or 1024 per block) of x [m][k]; fp16/bf16/fp32
    output."""
    dt, k, m, y = _rotation_args(x, signs, y, out_dtype)
    _check(_lib.hadamard_rotate(x.data_ptr(), dt[x.dtype], m, k, block, signs.data_ptr(), y.data_ptr(),
                                dt[y.dtype], _stream_handle(stream)))
    return y


def hadamard_rotate_g128(x, signs, y=None, out_dtype=None, stream=None):
    """Block-wise signed Walsh-Hadamard rotation (128 per block) of x [m][k]; fp16/bf16/fp32 output."""
    dt, k, m, y = _rotation_args(x, signs, y, out_dtype)
    _check(_lib.hadamard_rotate_g128(x.data_ptr(), dt[x.dtype], m, k, signs.data_ptr(), y.data_ptr(),
                                     dt[y.dtype], _stream_handle(stream)))
    return y


def ternary_code_flips(a: PackedMatrix, b: PackedMatrix, rows=True, total=True, stream=None):
    """Code flips between two packed matrices on the GPU: (total uint64 [1] or None,
    per-row counts int32 [n] holding uint32 values, or None)."""
    torch = _torch()
    dev = a.device
    _on_device(dev, a_codes=a.codes, b_codes=b.codes)
    r = torch.empty(a.n, dtype=torch.int32, device=dev) if rows else None
    t = torch.empty(1, dtype=torch.int64, device=dev) if total else None
    _check(_lib.ternary_code_flips(ctypes.byref(a.desc), ctypes.byref(b.desc), r.data_ptr() if r is not None else None,
                                   t.data_ptr() if t is not None else None, _stream_handle(stream)))
    return t, r


def ternary_code_flips_batched(pairs, totals, rows=None, stream=None):
    """Code flips of several pairs (a, b) of one layout in one launch. totals: int64 [1] tensors
    (or None entries); rows: int32 [n] tensors (or None entries), or None."""
    torch = _torch()
    count = len(pairs)
    if count == 0 or len(totals) != count or (rows is not None and len(rows) != count):
        _raise("TGS_E_SHAPE", "pairs, totals (and rows) must be non-empty lists of one length")
    for i, (a, b) in enumerate(pairs):
        if totals[i] is not None:
            _need(totals[i], f"totals[{i}]", (torch.int64,), min_numel=1)
        if rows is not None and rows[i] is not None:
            _need(rows[i], f"rows[{i}]", (torch.int32,), min_numel=a.n)
    for i, (a, b) in enumerate(pairs):
        _on_device(pairs[0][0].device, a_codes=a.codes, b_codes=b.codes, total=totals[i],
                   rows=rows[i] if rows is not None else None)
    da = (Matrix * count)(*[a.desc for a, _ in pairs])
    db = (Matrix * count)(*[b.desc for _, b in pairs])
    tp = (_vp * count)(*[t.data_ptr() if t is not None else None for t in totals])
    rp = None
    if rows is not None:
        rp = (_vp * count)(*[r.data_ptr() if r is not None else None for r in rows])
    _check(_lib.ternary_code_flips_batched(da, db, count, rp, tp, _stream_handle(stream)))
    return totals, rows


def stream_read(buf, sink=None, stream=None):
    """Read the whole device tensor `buf` once (the streaming-read probe); returns the sink tensor."""
    torch = _torch()
    if buf is None or not buf.is_contiguous() or buf.numel() * buf.element_size() % 16 != 0:
        _raise("TGS_E_SHAPE", "buf must be a contiguous tensor of a multiple of 16 bytes")
    words = int(_lib.tgs_stream_read_sink_words())
    if sink is None:
        sink = torch.empty(words, dtype=torch.int32, device=buf.device)
    _need(sink, "sink", (torch.int32,), min_numel=words)
    _on_device(buf.device, buf=buf, sink=sink)
    _check(_lib.tgs_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                                _stream_handle(stream)))
    return sink


def chain_workspace(device="cuda"):
    """A zero-filled chain workspace for the current device (int32 words; see ternary_gemv_chain)."""
    torch = _torch()
    nbytes = int(_lib.tgs_chain_workspace_bytes())
    if nbytes == 0:
        _raise("TGS_E_DEVICE", "no usable device for the chain workspace")
    return torch.zeros(nbytes // 4, dtype=torch.int32, device=device)


def _chain_steps(steps):
    """The ctypes step array of a chain, its length and the device its tensors are on."""
    torch = _torch()
    count = len(steps)
    if not 1 <= count <= CHAIN_MAX_STEPS:
        _raise("TGS_E_SHAPE", f"1..{CHAIN_MAX_STEPS} steps per chain, got {count}")
    arr = (ChainStep * count)()
    dev = None
    for i, st in enumerate(steps):
        ws, x, ys, gamma = st["ws"], st["x"], st["ys"], st.get("gamma")
        if not 1 <= len(ws) <= CHAIN_MAX_MATRICES or len(ys) != len(ws):
            _raise("TGS_E_SHAPE", f"step {i}: 1..{CHAIN_MAX_MATRICES} matrices and one y each")
        k = ws[0].k
        dev = dev or ws[0].device
        _need(x, f"steps[{i}].x", (torch.float16, torch.float32), numel=k)
        for j, (w, y) in enumerate(zip(ws, ys)):
            _need(y, f"steps[{i}].ys[{j}]", (torch.float32,), min_numel=w.n)
        if gamma is not None:
            _gamma_ok(gamma, k)
        _on_device(dev, x=x, gamma=gamma, **{f"codes{j}": w.codes for j, w in enumerate(ws)},
                   **{f"y{j}": y for j, y in enumerate(ys)})
        a = arr[i]
        a.count = len(ws)
        a.x_dtype = F32 if x.dtype == torch.float32 else F16
        a.norm = 1 if gamma is not None else 0
        a.eps = float(st.get("eps", 0.0))
        a.x = x.data_ptr()
        a.gamma = gamma.data_ptr() if gamma is not None else None
        for j, (w, y) in enumerate(zip(ws, ys)):
            a.w[j] = w.desc
            a.y[j] = y.data_ptr()
    return arr, count, dev


def ternary_gemv_chain(steps, workspace, stream=None):
    """Run up to CHAIN_MAX_STEPS single-token GEMV steps in order in one launch.

    steps: a list of dicts with keys "ws" (1..3 slot-2 PackedMatrix of one k), "x" (fp16 or fp32
    tensor of k elements: the step's input, which may be an earlier step's output), "ys" (fp32
    tensors of n_i elements) and optionally "gamma" (bf16 [k], as bfloat16 or int16 bits) with
    "eps" for the RMSNorm. workspace: from chain_workspace(), shared by consecutive chains.
    """
    torch = _torch()
    arr, count, dev = _chain_steps(steps)
    _need(workspace, "workspace", (torch.int32,), min_numel=int(_lib.tgs_chain_workspace_bytes()) // 4)
    _on_device(dev, workspace=workspace)
    _check(_lib.ternary_gemv_chain(arr, count, workspace.data_ptr(), workspace.numel() * 4, _stream_handle(stream)))


def ternary_gemv_chain_static(steps, error=None, stream=None):
    """ternary_gemv_chain on the library's own per-device workspace: allocates nothing.

    error: None, or an int32 device tensor of at least one element that receives the chain's
    error word (0 when every wait between steps completed). Calls that overlap on one device race.
    """
    torch = _torch()
    arr, count, dev = _chain_steps(steps)
    if error is not None:
        _need(error, "error", (torch.int32,), min_numel=1)
        _on_device(dev, error=error)
    _check(_lib.ternary_gemv_chain_static(arr, count, None if error is None else error.data_ptr(),
                                          _stream_handle(stream)))
