"""The Python binding checks every tensor argument before calling the C ABI (which sees raw pointers
only and cannot know a buffer's size, type or device).

These run on the CPU: every tensor is host memory, so each call must raise before the library is
called at all (a host pointer handed to a device call would be a bad address). The argument errors
are reported first, and the device check last, so each error can be provoked on its own.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
import ternary_group_scaled_amd as tgs  # noqa: E402


def _w(layout=tgs.SLOT2, n=8, k=256, rotated=0):
    t = np.zeros((n, k), dtype=np.int8)
    s = np.ones((n, k // 128), dtype=np.float16)
    codes, sc = tgs.pack_ternary(layout, t, s)
    return tgs.PackedMatrix(layout, torch.from_numpy(codes), torch.from_numpy(sc.view(np.int16)), k, rotated=rotated)


def _expect(name, fn, *args, **kw):
    with pytest.raises(tgs.TgsError) as info:
        fn(*args, **kw)
    assert info.value.name == name, str(info.value)


def _h(n, dtype=torch.float16):
    return torch.zeros(n, dtype=dtype)


def test_gemv_checks():
    w = _w()
    _expect("TGS_E_DTYPE", tgs.ternary_gemv, w, _h(256, torch.bfloat16))      # bf16 read as fp16 otherwise
    _expect("TGS_E_DTYPE", tgs.ternary_gemv, w, _h(256, torch.float32))
    _expect("TGS_E_SHAPE", tgs.ternary_gemv, w, _h(200))                       # not a multiple of k
    _expect("TGS_E_SHAPE", tgs.ternary_gemv, w, torch.zeros((2, 512), dtype=torch.float16)[:, ::2])
    _expect("TGS_E_DTYPE", tgs.ternary_gemv, w, _h(256), y=_h(8, torch.float64))
    _expect("TGS_E_SIZE", tgs.ternary_gemv, w, _h(512), y=_h(8, torch.float32))  # m = 2 needs 16
    _expect("TGS_E_SHAPE", tgs.ternary_gemv, w, _h(256), y=torch.zeros((8, 2))[:, 0])
    wr = _w(rotated=1)
    _expect("TGS_E_DTYPE", tgs.ternary_gemv, wr, _h(256), signs=_h(256, torch.int16))
    _expect("TGS_E_SHAPE", tgs.ternary_gemv, wr, _h(256), signs=_h(128, torch.int8))
    _expect("TGS_E_DEVICE", tgs.ternary_gemv, w, _h(256))                       # host memory: never called
    _expect("TGS_E_DEVICE", tgs.ternary_gemv, w, _h(256), y=_h(8, torch.float32))


def test_batched_checks():
    ws = [_w(n=8, k=256), _w(n=4, k=512)]
    x0, x1 = _h(256), _h(512)
    y0, y1 = _h(8, torch.float32), _h(4, torch.float32)
    _expect("TGS_E_SHAPE", tgs.ternary_gemv_batched, ws, [x0, _h(256)], [y0, y1])   # m * k_1 = 512 expected
    _expect("TGS_E_DTYPE", tgs.ternary_gemv_batched, ws, [x0, _h(512, torch.bfloat16)], [y0, y1])
    _expect("TGS_E_SIZE", tgs.ternary_gemv_batched, ws, [x0, x1], [y0, _h(3, torch.float32)])
    _expect("TGS_E_DTYPE", tgs.ternary_gemv_batched, ws, [x0, x1], [y0, _h(4, torch.float16)])
    _expect("TGS_E_SHAPE", tgs.ternary_gemv_batched, ws, [x0], [y0, y1])
    _expect("TGS_E_SHAPE", tgs.ternary_gemv_batched, ws, [x0, x1], [y0, y1], signs=[None])
    _expect("TGS_E_DEVICE", tgs.ternary_gemv_batched, ws, [x0, x1], [y0, y1])
    g = [_h(256, torch.int16), _h(256, torch.int16)]
    _expect("TGS_E_SHAPE", tgs.ternary_gemv_rmsnorm_batched, ws, [x0, x1], g, 1e-6, [y0, y1])  # gamma 1 is [512]
    _expect("TGS_E_NULL", tgs.ternary_gemv_rmsnorm_batched, ws, [x0, x1], None, 1e-6, [y0, y1])


def test_rmsnorm_gemv_checks():
    w = _w()
    _expect("TGS_E_DTYPE", tgs.ternary_gemv_rmsnorm, w, _h(256), _h(256, torch.float32), 1e-6)
    _expect("TGS_E_SHAPE", tgs.ternary_gemv_rmsnorm, w, _h(256), _h(255, torch.bfloat16), 1e-6)
    _expect("TGS_E_DEVICE", tgs.ternary_gemv_rmsnorm, w, _h(256), _h(256, torch.bfloat16), 1e-6)


def test_gemm_checks():
    w = _w()
    _expect("TGS_E_DTYPE", tgs.ternary_gemm, w, _h(16 * 256))                      # fp16 read as bf16 otherwise
    _expect("TGS_E_SHAPE", tgs.ternary_gemm, w, _h(300, torch.bfloat16))
    _expect("TGS_E_SIZE", tgs.ternary_gemm, w, _h(16 * 256, torch.bfloat16), y=_h(16 * 8 - 1, torch.float32))
    _expect("TGS_E_DEVICE", tgs.ternary_gemm, w, _h(16 * 256, torch.bfloat16))


def test_rotation_checks():
    x = torch.zeros((2, 256), dtype=torch.float16)
    sg = torch.ones(256, dtype=torch.int8)
    _expect("TGS_E_DTYPE", tgs.hadamard_rotate, x.to(torch.int16), sg)
    _expect("TGS_E_SHAPE", tgs.hadamard_rotate, x, torch.ones(128, dtype=torch.int8))
    _expect("TGS_E_NULL", tgs.hadamard_rotate, x, None)
    _expect("TGS_E_SIZE", tgs.hadamard_rotate, x, sg, y=torch.zeros(300))
    _expect("TGS_E_DTYPE", tgs.hadamard_rotate_g128, x, sg, y=torch.zeros(512, dtype=torch.float64))
    _expect("TGS_E_SHAPE", tgs.rmsnorm_hadamard_rotate, x, _h(128, torch.bfloat16), 1e-6, sg)
    _expect("TGS_E_NULL", tgs.rmsnorm_hadamard_rotate, x, None, 1e-6, sg)
    _expect("TGS_E_DEVICE", tgs.hadamard_rotate, x, sg)
    _expect("TGS_E_DEVICE", tgs.hadamard_rotate_g128, x, sg)
    _expect("TGS_E_DEVICE", tgs.rmsnorm_hadamard_rotate, x, _h(256, torch.bfloat16), 1e-6, sg)


def test_code_flip_checks():
    a, b = _w(), _w()
    _expect("TGS_E_DTYPE", tgs.ternary_code_flips_batched, [(a, b)], [_h(1, torch.int32)])
    _expect("TGS_E_SIZE", tgs.ternary_code_flips_batched, [(a, b)], [None], [_h(7, torch.int32)])
    _expect("TGS_E_SHAPE", tgs.ternary_code_flips_batched, [(a, b)], [])
    _expect("TGS_E_DEVICE", tgs.ternary_code_flips_batched, [(a, b)], [_h(1, torch.int64)])
    _expect("TGS_E_DEVICE", tgs.ternary_code_flips, a, b)


def test_packed_matrix_checks():
    codes = torch.zeros((8, 64), dtype=torch.uint8)
    _expect("TGS_E_SHAPE", tgs.PackedMatrix, tgs.SLOT2, codes.to(torch.int8), torch.zeros(16, dtype=torch.int16), 256)
    _expect("TGS_E_SHAPE", tgs.PackedMatrix, tgs.SLOT2, torch.zeros((8, 128), dtype=torch.uint8)[:, ::2],
            torch.zeros(16, dtype=torch.int16), 256)
    _expect("TGS_E_DTYPE", tgs.PackedMatrix, tgs.SLOT2, codes, torch.zeros(16, dtype=torch.float32), 256)
    _expect("TGS_E_SHAPE", tgs.PackedMatrix, tgs.SLOT2, codes, torch.zeros(15, dtype=torch.int16), 256)
