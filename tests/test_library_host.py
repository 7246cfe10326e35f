"""Host-side tests of the C-ABI library: load, exports, packing and argument checks.

No device work is queued here: every call either runs on the host (pack/unpack) or is
rejected by the host-side checks before any HIP call, so these run without a GPU.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth
import ternary_group_scaled_amd as tgs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CONFIG_K = (128, 1024, 4096, 5120, 12288, 17408)


def test_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "tgs.h")).read()
    declared = set(re.findall(r"^\s*(?:tgs_status|size_t|const char\*)\s+(\w+)\s*\(", header, re.M))
    assert {"pack_ternary", "unpack_ternary", "ternary_gemv", "ternary_gemm", "hadamard_rotate_g128"} <= declared
    lib = ctypes.CDLL(tgs.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == set(tgs.EXPORTS)


def test_status_strings():
    for code in range(10):
        assert tgs.status_string(code)
    assert tgs.status_string(0) == "ok"


@pytest.mark.parametrize("k", CONFIG_K)
def test_row_bytes_match_oracle(k):
    for layout in (tgs.SLOT2, tgs.BASE3, tgs.BINARY):
        assert tgs.code_row_bytes(layout, k) == oracle.row_bytes(layout, k)
    assert tgs.code_row_bytes(tgs.SLOT2, 100) == 0
    assert tgs.code_row_bytes(7, 128) == 0


@pytest.mark.parametrize("layout", [tgs.SLOT2, tgs.BASE3])
@pytest.mark.parametrize("k", CONFIG_K)
def test_pack_bit_exact_vs_oracle(layout, k):
    n = 37
    t = synth.trits(1, k * 10 + layout, (n, k), 0.4 if layout == tgs.SLOT2 else 0.5)
    s = synth.scales_f16(1, k, (n, k // 128))
    codes, s_out = tgs.pack_ternary(layout, t, s)
    assert (codes == oracle.pack(layout, t)).all()
    assert (s_out.view(np.uint16) == s.view(np.uint16)).all()
    back, s_back = tgs.unpack_ternary(layout, codes, s, k)
    assert (back == t).all()
    assert (s_back.view(np.uint16) == s.view(np.uint16)).all()


@pytest.mark.parametrize("k", CONFIG_K)
def test_binary_pack_bit_exact_vs_oracle(k):
    n = 37
    t = synth.trits(1, k * 10 + 3, (n, k), 0.0)  # {-1, +1}
    s = synth.scales_f16(1, k, (n, k // 128))
    codes, _ = tgs.pack_ternary(tgs.BINARY, t, s)
    assert codes.shape == (n, k // 8)
    assert (codes == oracle.pack(tgs.BINARY, t)).all()
    back, _ = tgs.unpack_ternary(tgs.BINARY, codes, s, k)
    assert (back == t).all()
    # every byte value decodes (the binary layout has no invalid codes)
    every = np.arange(n * k // 8, dtype=np.uint64).astype(np.uint8).reshape(n, k // 8)
    back, _ = tgs.unpack_ternary(tgs.BINARY, every, s, k)
    assert (back == oracle.unpack(tgs.BINARY, every, k)).all()


def test_pack_large_parallel_path_is_exact():
    # big enough for the multi-threaded packer
    t = synth.trits(2, 3, (300, 12288), 0.4)
    for layout in (tgs.SLOT2, tgs.BASE3):
        codes, _ = tgs.pack_ternary(layout, t)
        assert (codes == oracle.pack(layout, t)).all()
    t = synth.trits(2, 4, (300, 12288), 0.0)
    codes, _ = tgs.pack_ternary(tgs.BINARY, t)
    assert (codes == oracle.pack(tgs.BINARY, t)).all()


def test_unpack_reads_the_oracle_bytes():
    t = synth.trits(3, 3, (5, 1024), 0.4)
    for layout in (tgs.SLOT2, tgs.BASE3):
        s = np.ones((5, 8), dtype=np.float16)
        back, _ = tgs.unpack_ternary(layout, oracle.pack(layout, t), s, 1024)
        assert (back == t).all()


def _expect(status_name, fn, *args):
    with pytest.raises(tgs.TgsError) as info:
        fn(*args)
    assert info.value.name == status_name, str(info.value)


def test_pack_errors():
    t = np.zeros((2, 128), dtype=np.int8)
    t[1, 77] = 2
    _expect("TGS_E_CODE", tgs.pack_ternary, tgs.SLOT2, t)
    _expect("TGS_E_CODE", tgs.pack_ternary, tgs.BASE3, t)
    _expect("TGS_E_SHAPE", tgs.pack_ternary, tgs.SLOT2, np.zeros((2, 100), dtype=np.int8))
    _expect("TGS_E_LAYOUT", tgs.pack_ternary, 4, np.zeros((2, 128), dtype=np.int8))
    _expect("TGS_E_CODE", tgs.pack_ternary, tgs.BINARY, np.ones((2, 128), dtype=np.int8) - (t == 2))  # a zero
    _expect("TGS_E_CODE", tgs.pack_ternary, tgs.BINARY, np.zeros((2, 128), dtype=np.int8))
    lib = tgs.lib()
    out = np.zeros(10, dtype=np.uint8)
    good = np.zeros((2, 128), dtype=np.int8)
    assert lib.pack_ternary(tgs.SLOT2, good.ctypes.data, None, 2, 128, out.ctypes.data, out.nbytes, None) == 7
    assert lib.pack_ternary(tgs.SLOT2, None, None, 2, 128, out.ctypes.data, out.nbytes, None) == 1


def test_unpack_errors():
    s = np.ones((1, 1), dtype=np.float16)
    slot = np.full((1, 32), 0x55, dtype=np.uint8)
    slot[0, 9] = 0x7F  # slot value 3
    _expect("TGS_E_CODE", tgs.unpack_ternary, tgs.SLOT2, slot, s, 128)
    b3 = np.full((1, 32), 121, dtype=np.uint8)
    b3[0, 3] = 243
    _expect("TGS_E_CODE", tgs.unpack_ternary, tgs.BASE3, b3, s, 128)
    b3 = np.full((1, 32), 121, dtype=np.uint8)
    b3[0, 30] = 0  # pad byte must be 121
    _expect("TGS_E_CODE", tgs.unpack_ternary, tgs.BASE3, b3, s, 128)
    b3 = np.full((1, 32), 121, dtype=np.uint8)
    b3[0, 25] = 121 + 2 * 27  # trit 128 (past K) set to +1
    _expect("TGS_E_CODE", tgs.unpack_ternary, tgs.BASE3, b3, s, 128)


def _fake_matrix(layout=tgs.SLOT2, rotated=0, n=4, k=256, codes=0x100000, scales=0x200000):
    m = tgs.Matrix()
    assert tgs.lib().tgs_matrix_init(ctypes.byref(m), layout, rotated, n, k, codes, scales) == 0
    return m


def _gemv(m, x=0x300000, x_dtype=tgs.F16, rows=1, signs=None, y=0x400000):
    return tgs.lib().ternary_gemv(ctypes.byref(m), x, x_dtype, rows, signs, y, None)


def test_device_call_argument_checks_happen_before_any_device_work():
    lib = tgs.lib()
    assert _gemv(_fake_matrix(rotated=1)) == 6            # rotated weights need signs
    assert _gemv(_fake_matrix(rotated=0), signs=0x500000) == 6  # plain weights refuse signs
    assert _gemv(_fake_matrix(), x_dtype=tgs.BF16) == 8
    assert _gemv(_fake_matrix(), rows=0) == 2
    assert _gemv(_fake_matrix(), rows=9) == 2
    assert _gemv(_fake_matrix(), x=0x300004) == 3          # x must be 16-byte aligned
    assert _gemv(_fake_matrix(), y=0x400002) == 3
    assert _gemv(_fake_matrix(codes=0x100008)) == 3        # codes 16-byte aligned
    assert _gemv(_fake_matrix(), x=None) == 1
    bad = _fake_matrix()
    bad.magic = 0
    assert _gemv(bad) == 5
    bad = _fake_matrix()
    bad.layout = 9
    assert _gemv(bad) == 5
    bad = _fake_matrix()
    bad.k = 200
    assert _gemv(bad) == 2
    bad = _fake_matrix()
    bad.code_row_stride = 48  # < 64 bytes per row at k = 256
    assert _gemv(bad) == 2
    assert "rotated" in lib.tgs_last_error().decode() or lib.tgs_last_error()
    # ternary_gemm
    m = _fake_matrix()
    assert lib.ternary_gemm(ctypes.byref(m), 0x300000, tgs.F16, 4, None, 0x400000, None) == 8
    assert lib.ternary_gemm(ctypes.byref(_fake_matrix(rotated=1)), 0x300000, tgs.BF16, 4, 0x500000, 0x400000,
                            None) == 6
    assert lib.ternary_gemm(ctypes.byref(m), 0x300000, tgs.BF16, 0, None, 0x400000, None) == 2
    big = _fake_matrix(k=1 << 23)
    assert lib.ternary_gemm(ctypes.byref(big), 0x300000, tgs.BF16, 4, None, 0x400000, None) == 2  # k <= 2^23 - 4096
    # hadamard_rotate_g128
    assert lib.hadamard_rotate_g128(0x300000, tgs.F16, 2, 200, 0x500000, 0x400000, tgs.F32, None) == 2
    assert lib.hadamard_rotate_g128(0x300000, tgs.F16, 2, 256, 0x500000, 0x400000, 99, None) == 8  # no such dtype
    assert lib.hadamard_rotate_g128(0x300000, tgs.F16, 2, 256, None, 0x400000, tgs.F32, None) == 1
    assert lib.hadamard_rotate_g128(0x300000, tgs.F16, 2, 256, 0x500000, 0x300100, tgs.F32, None) == 2  # overlap
    # hadamard_rotate: the block is 128 or 1024 and divides k
    rot = lambda k, block, signs=0x500000: lib.hadamard_rotate(0x300000, tgs.F16, 2, k, block, signs, 0x400000,
                                                                 tgs.F32, None)
    assert rot(2048, 512) == 2
    assert rot(1536, 1024) == 2
    assert rot(512, 1024) == 2
    assert rot(2048, 1024, signs=None) == 1
    assert rot(2048, 1024, signs=0x500008) == 3                   # signs 16-byte aligned
    assert rot(2048, 128, signs=0x500001) == 3
    # rotated GEMV: signs 16-byte aligned; 1024-element blocks need k % 1024 == 0
    assert _gemv(_fake_matrix(rotated=1), signs=0x500004) == 3
    assert _gemv(_fake_matrix(rotated=1024, k=2048), signs=0x500008) == 3
    bad = _fake_matrix(rotated=1024, k=2048)
    bad.k = 1536
    bad.code_row_stride = 384
    assert _gemv(bad, signs=0x500000) == 2
    # RMSNorm prologue: gamma required and 16-byte aligned, eps positive and finite
    norm = lambda m, gamma=0x600000, eps=1e-6, signs=None: lib.ternary_gemv_rmsnorm(
        ctypes.byref(m), 0x300000, tgs.F16, 1, gamma, eps, signs, 0x400000, None)
    assert norm(_fake_matrix(), gamma=None) == 1
    assert norm(_fake_matrix(), gamma=0x600008) == 3
    assert norm(_fake_matrix(), eps=0.0) == 2
    assert norm(_fake_matrix(), eps=-1e-6) == 2
    assert norm(_fake_matrix(), eps=float("inf")) == 2
    assert norm(_fake_matrix(), eps=float("nan")) == 2
    assert norm(_fake_matrix(rotated=1)) == 6                    # rotated weights still need signs
    assert norm(_fake_matrix(rotated=0), signs=0x500000) == 6
    gp = (ctypes.c_void_p * 1)(None)
    assert lib.ternary_gemv_rmsnorm_batched((tgs.Matrix * 1)(_fake_matrix()), 1, (ctypes.c_void_p * 1)(0x300000),
                                            tgs.F16, 1, gp, 1e-6, None, (ctypes.c_void_p * 1)(0x400000), None) == 1
    assert lib.ternary_gemv_rmsnorm_batched((tgs.Matrix * 1)(_fake_matrix()), 1, (ctypes.c_void_p * 1)(0x300000),
                                            tgs.F16, 1, None, 1e-6, None, (ctypes.c_void_p * 1)(0x400000), None) == 1
    # the fused standalone norm + rotation
    nrot = lambda k=2048, block=1024, gamma=0x600000, eps=1e-6, y=0x400000, signs=0x500000: \
        lib.rmsnorm_hadamard_rotate(0x300000, tgs.F16, 2, k, block, gamma, eps, signs, y, tgs.F32, None)
    assert nrot(gamma=0x600002) == 3                              # gamma 16-byte aligned
    assert nrot(signs=0x500004) == 3                              # signs 16-byte aligned
    assert nrot(block=512) == 2
    assert nrot(k=1536) == 2
    assert nrot(gamma=None) == 1
    assert nrot(eps=0.0) == 2
    assert nrot(y=0x300100) == 2                                  # overlaps x
    assert nrot(k=1 << 24, block=128) == 2                        # k below 2^24
    # batched
    ms = (tgs.Matrix * 2)(_fake_matrix(), _fake_matrix(rotated=1))
    xp = (ctypes.c_void_p * 2)(0x300000, 0x300000)
    yp = (ctypes.c_void_p * 2)(0x400000, 0x410000)
    assert lib.ternary_gemv_batched(ms, 2, xp, tgs.F16, 1, None, yp, None) == 6
    assert lib.ternary_gemv_batched(ms, 0, xp, tgs.F16, 1, None, yp, None) == 2
    assert lib.ternary_gemv_batched(ms, 33, xp, tgs.F16, 1, None, yp, None) == 2


def test_code_flip_argument_checks_happen_before_any_device_work():
    lib = tgs.lib()
    a, b = _fake_matrix(), _fake_matrix()
    flips = lambda x, y, rows=0x600000, total=0x700000: lib.ternary_code_flips(ctypes.byref(x), ctypes.byref(y),
                                                                                rows, total, None)
    assert flips(a, b, rows=None, total=None) == 1         # nothing requested
    assert flips(a, b, rows=0x600002) == 3                 # row counts 4-byte aligned
    assert flips(a, b, total=0x700004) == 3                # total 8-byte aligned
    other = _fake_matrix()
    other.k = 384
    other.code_row_stride = 96
    assert flips(a, other) == 2                            # shapes differ
    other = _fake_matrix()
    other.layout = tgs.BASE3
    other.code_row_stride = 64
    assert flips(a, other) == 2                            # layouts differ
    assert flips(a, _fake_matrix(rotated=1)) == 6          # bases differ
    bad = _fake_matrix()
    bad.magic = 0
    assert flips(bad, b) == 5
    ms = (tgs.Matrix * 2)(_fake_matrix(), _fake_matrix())
    tp = (ctypes.c_void_p * 2)(0x700000, 0x700008)
    assert lib.ternary_code_flips_batched(ms, ms, 0, None, tp, None) == 2
    assert lib.ternary_code_flips_batched(ms, ms, 33, None, tp, None) == 2
    assert lib.ternary_code_flips_batched(ms, ms, 2, None, None, None) == 1
    tp_gap = (ctypes.c_void_p * 2)(0x700000, None)
    assert lib.ternary_code_flips_batched(ms, ms, 2, None, tp_gap, None) == 1  # pair 1 requests nothing


def test_matrix_init_rejects_bad_shapes():
    m = tgs.Matrix()
    assert tgs.lib().tgs_matrix_init(ctypes.byref(m), tgs.SLOT2, 0, 0, 128, 1, 1) == 2
    assert tgs.lib().tgs_matrix_init(ctypes.byref(m), tgs.SLOT2, 0, 4, 129, 1, 1) == 2
    assert tgs.lib().tgs_matrix_init(ctypes.byref(m), 5, 0, 4, 128, 1, 1) == 5
    assert m.magic == 0
    assert tgs.lib().tgs_matrix_init(ctypes.byref(m), tgs.SLOT2, 1024, 4, 1536, 1, 1) == 2  # k % 1024 != 0
    assert tgs.lib().tgs_matrix_init(ctypes.byref(m), tgs.SLOT2, 512, 4, 2048, 1, 1) == 5   # no 512-blocks
    assert m.magic == 0


def test_bad_rotation_block_has_one_status_everywhere():
    """An invalid `rotated` field is an invalid descriptor: TGS_E_LAYOUT from tgs_matrix_init and from
    every call that checks a descriptor (the header documents the same status)."""
    m = tgs.Matrix()
    for rotated in (2, 512, -1, 2048):
        assert tgs.lib().tgs_matrix_init(ctypes.byref(m), tgs.SLOT2, rotated, 4, 2048, 1, 1) == 5
    bad = _fake_matrix(rotated=1, k=2048)
    bad.rotated = 512
    assert _gemv(bad, signs=0x500000) == 5
    assert tgs.lib().ternary_gemm(ctypes.byref(bad), 0x300000, tgs.BF16, 4, None, 0x400000, None) == 5
    codes = np.zeros((4, 512), dtype=np.uint8)
    assert tgs.lib().unpack_ternary(ctypes.byref(bad), codes.ctypes.data, None) == 5


@pytest.mark.parametrize("rotated,stored", [(0, 0), (1, 1), (128, 1), (1024, 1024)])
def test_matrix_init_records_the_rotation_block(rotated, stored):
    m = _fake_matrix(rotated=rotated, k=2048)
    assert m.rotated == stored


# Workspace bytes of ternary_gemm_ws for the 27B prefill shapes, as the launch plan splits K on a
# device of 256 compute units (MI355X; also the count the host assumes when no device is visible):
# - 17408 x 5120 (40 groups): too few groups to split up to 32 rows (one block of 16 rows, or two
#   above 16, per workgroup); 64 x 64 tiles at 128 rows (544 tiles: 512 whole, the 32 left over
#   in four parts); 128 x 128 tiles at 2048 rows (2176 tiles: 128 left over, four parts);
# - 5120 x 17408 (136 groups): FB = 5 and four K parts up to 32 rows, (4 - 1) m n fp32 values;
#   every 64 x 64 tile in four parts at 33 and 128 rows (80 and 160 tiles); 128 left-over
#   128 x 128 tiles in four parts at 2048 rows.
GEMM_WORKSPACE_27B = [
    (17408, 5120, 1, 0), (17408, 5120, 16, 0), (17408, 5120, 17, 0), (17408, 5120, 32, 0), (17408, 5120, 33, 0),
    (17408, 5120, 128, 3 * 32 * 64 * 64 * 4), (17408, 5120, 2048, 3 * 128 * 128 * 128 * 4),
    (5120, 17408, 1, 3 * 1 * 5120 * 4), (5120, 17408, 16, 3 * 16 * 5120 * 4), (5120, 17408, 17, 3 * 17 * 5120 * 4),
    (5120, 17408, 32, 3 * 32 * 5120 * 4), (5120, 17408, 33, 3 * 80 * 64 * 64 * 4),
    (5120, 17408, 128, 3 * 160 * 64 * 64 * 4), (5120, 17408, 2048, 3 * 128 * 128 * 128 * 4),
]


@pytest.mark.parametrize("n,k,m,expected", GEMM_WORKSPACE_27B)
def test_gemm_workspace_follows_the_launch_plan(n, k, m, expected):
    """The size query runs the same plan as the launch, so it pins how K is split (skinny kernel
    up to 32 rows, tiled kernel above) without a device."""
    w = _fake_matrix(n=n, k=k)
    assert tgs.lib().ternary_gemm_workspace_size(ctypes.byref(w), m) == expected
    assert tgs.lib().ternary_gemm_workspace_size(ctypes.byref(w), 0) == 0
