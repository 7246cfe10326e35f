"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Tolerance per element: |y - y_ref| <= 1e-3 * sum_k |s t xr| + 1e-6 (the oracle's `bound`), with xr the
rotated activation for rotated weights. Packing must be bit-exact. Exact equalities hold where every
partial sum is exactly representable in fp32 (integer activations, power-of-two scales).
"""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from gpu_util import (assert_within_bound, make_signs, make_weights, make_x_bf16_bits, make_x_f16,
                      oracle_product)

torch = pytest.importorskip("torch")
import ternary_group_scaled_amd as tgs  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"
LAYOUTS = [tgs.SLOT2, tgs.BASE3]
LNAME = {tgs.SLOT2: "slot2", tgs.BASE3: "base3"}


def _packed(layout, t, s, rotated=False):
    return tgs.PackedMatrix.from_trits(layout, t, s, device=DEV, rotated=rotated)


def _x_dev(x16):
    return torch.from_numpy(x16.view(np.int16).copy()).to(DEV).view(torch.float16)


def _gemv(layout, t, s, x16, signs=None, block=128):
    w = _packed(layout, t, s, rotated=block if signs is not None else 0)
    sg = torch.from_numpy(signs).to(DEV) if signs is not None else None
    y = tgs.ternary_gemv(w, _x_dev(x16), signs=sg)
    torch.cuda.synchronize()
    return y.cpu().numpy()


# ------------------------------------------------------------------------------ small configuration

def test_single_gemv_256x1024_slot2():
    """256 x 1024 GEMV, codes P(0)=0.4, scales |N(0,0.02)|+1e-4, x fp16 N(0,1), seed 0."""
    t, s = make_weights(0, "gemv256x1024", 256, 1024, 0.4)
    x16 = make_x_f16(0, "gemv256x1024", 1, 1024)
    codes, _ = tgs.pack_ternary(tgs.SLOT2, t, s)
    assert (codes == oracle.pack(tgs.SLOT2, t)).all()
    back, _ = tgs.unpack_ternary(tgs.SLOT2, codes, s, 1024)
    assert (back == t).all()
    y = _gemv(tgs.SLOT2, t, s, x16)
    y_ref, bound = oracle_product(tgs.SLOT2, t, s, x16.view(np.uint16), oracle.X_F16)
    assert_within_bound(y, y_ref, bound, "256x1024 GEMV")
    y2 = _gemv(tgs.SLOT2, t, s, x16)
    assert (y2.view(np.uint32) == y.view(np.uint32)).all()  # run-to-run bitwise determinism


SHAPES = [(1, 128), (17, 256), (300, 1024), (129, 4096), (64, 5120), (33, 12288), (40, 17408), (70, 640),
          (9, 30720), (130, 2048), (257, 2560), (1000, 3968)]


@pytest.mark.parametrize("layout", LAYOUTS, ids=LNAME.get)
@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("m", [1, 2, 3, 8])
def test_gemv_matches_oracle(layout, n, k, m):
    t, s = make_weights(n + k, f"gemv{layout}", n, k, 0.4 if layout == tgs.SLOT2 else 0.5)
    x16 = make_x_f16(m, f"gemv{n}x{k}", m, k)
    y = _gemv(layout, t, s, x16)
    y_ref, bound = oracle_product(layout, t, s, x16.view(np.uint16), oracle.X_F16)
    assert_within_bound(y, y_ref, bound, f"{LNAME[layout]} {n}x{k} m={m}")


@pytest.mark.parametrize("layout", LAYOUTS, ids=LNAME.get)
@pytest.mark.parametrize("n,k", [(1, 128), (33, 640), (100, 5120), (20, 17408), (65, 4096)])
@pytest.mark.parametrize("m", [1, 3, 5, 8])
def test_rotated_gemv_matches_oracle(layout, n, k, m):
    t, s = make_weights(n * 3 + k, f"rot{layout}", n, k, 0.5)
    x16 = make_x_f16(m + 7, f"rot{n}x{k}", m, k)
    sg = make_signs(k, "rot", k)
    y = _gemv(layout, t, s, x16, signs=sg)
    y_ref, bound = oracle_product(layout, t, s, x16.view(np.uint16), oracle.X_F16, signs=sg)
    assert_within_bound(y, y_ref, bound, f"rotated {LNAME[layout]} {n}x{k} m={m}")


@pytest.mark.parametrize("layout", LAYOUTS, ids=LNAME.get)
@pytest.mark.parametrize("n,k", [(1, 1024), (33, 2048), (100, 5120), (20, 17408), (65, 4096), (300, 3072)])
@pytest.mark.parametrize("m", [1, 2, 3, 8])
def test_rotated_1024_gemv_matches_oracle(layout, n, k, m):
    """1024-element rotation blocks (eight scale groups per block)."""
    t, s = make_weights(n * 5 + k, f"rot1024{layout}", n, k, 0.5)
    x16 = make_x_f16(m + 11, f"rot1024{n}x{k}", m, k)
    sg = make_signs(k, "rot1024", k)
    y = _gemv(layout, t, s, x16, signs=sg, block=1024)
    y_ref, bound = oracle_product(layout, t, s, x16.view(np.uint16), oracle.X_F16, signs=sg, block=1024)
    assert_within_bound(y, y_ref, bound, f"rotated-1024 {LNAME[layout]} {n}x{k} m={m}")


@pytest.mark.parametrize("layout", LAYOUTS, ids=LNAME.get)
def test_rotation_block_changes_the_product(layout):
    """The same weights and signs under 128- and 1024-element blocks give different products, each
    matching its own oracle (a kernel that ignored the block size would fail one of the two)."""
    n, k, m = 40, 2048, 2
    t, s = make_weights(3, f"rotblk{layout}", n, k, 0.5)
    x16 = make_x_f16(3, "rotblk", m, k)
    sg = make_signs(3, "rotblk", k)
    for block in (128, 1024):
        y = _gemv(layout, t, s, x16, signs=sg, block=block)
        y_ref, bound = oracle_product(layout, t, s, x16.view(np.uint16), oracle.X_F16, signs=sg, block=block)
        assert_within_bound(y, y_ref, bound, f"block {block}")
        other, _ = oracle_product(layout, t, s, x16.view(np.uint16), oracle.X_F16, signs=sg,
                                  block=1152 - block)
        assert (np.abs(y - other) > bound).any()


@pytest.mark.parametrize("layout", LAYOUTS, ids=LNAME.get)
def test_integer_inputs_are_exact(layout):
    # integer x in [-4, 4] and power-of-two scales: every partial sum is an fp32-exact integer
    # multiple of a power of two, so any summation order gives the oracle's value bit for bit
    n, k, m = 200, 12288, 2
    t, _ = make_weights(5, "exact", n, k, 0.4)
    expo = synth.trits(5, 77, (n, k // 128), 0.0).astype(np.int64) - 3
    s = np.ldexp(1.0, expo).astype(np.float16)
    xi = synth.trits(6, 1, (m, k), 0.2).astype(np.int64) * 4 + synth.trits(6, 2, (m, k), 0.3)
    x16 = xi.astype(np.float16)
    y = _gemv(layout, t, s, x16)
    y_ref, _ = oracle_product(layout, t, s, x16.view(np.uint16), oracle.X_F16)
    assert (y.astype(np.float64) == y_ref).all()


@pytest.mark.parametrize("layout", LAYOUTS, ids=LNAME.get)
def test_special_rows(layout):
    # all +1 rows give s * sum x, all -1 rows -s * sum x, all-zero rows 0, and one-hot rows s * t * x_j,
    # each within the tolerance bound (the oracle's values are exact; see test_oracle_pins)
    k = 1024
    t = np.zeros((5, k), dtype=np.int8)
    t[0] = 1
    t[1] = -1
    t[3, 517] = 1
    t[4, 1023] = -1
    s = synth.scales_f16(1, 2, (5, k // 128))
    x16 = make_x_f16(3, "special", 1, k)
    y = _gemv(layout, t, s, x16)
    y_ref, bound = oracle_product(layout, t, s, x16.view(np.uint16), oracle.X_F16)
    assert_within_bound(y, y_ref, bound, "special rows")


@pytest.mark.parametrize("layout", LAYOUTS, ids=LNAME.get)
def test_batched_equals_single_calls(layout):
    shapes = [(300, 4096), (64, 4096), (96, 12288), (5, 1024)]
    ws, xs, ys, singles = [], [], [], []
    for i, (n, k) in enumerate(shapes):
        t, s = make_weights(i, f"batch{layout}", n, k, 0.4)
        x16 = make_x_f16(i, "batch", 1, k)
        ws.append(_packed(layout, t, s))
        xs.append(_x_dev(x16))
        ys.append(torch.empty((1, n), dtype=torch.float32, device=DEV))
        singles.append(_gemv(layout, t, s, x16))
    tgs.ternary_gemv_batched(ws, xs, ys)
    torch.cuda.synchronize()
    for y, ref in zip(ys, singles):
        assert (y.cpu().numpy().view(np.uint32) == ref.view(np.uint32)).all()


def test_batched_mixed_layouts_and_bases():
    k = 2048
    sg = make_signs(1, "mixed", k)
    cases = [(tgs.SLOT2, 0), (tgs.BASE3, 128), (tgs.SLOT2, 1024), (tgs.SLOT2, 128), (tgs.BASE3, 1024),
             (tgs.BASE3, 0)]
    ws, xs, ys, signs, refs = [], [], [], [], []
    for i, (layout, rot) in enumerate(cases):
        t, s = make_weights(i, "mixed", 50 + i, k, 0.5)
        x16 = make_x_f16(i, "mixed", 2, k)
        ws.append(_packed(layout, t, s, rotated=rot))
        xs.append(_x_dev(x16))
        ys.append(torch.empty((2, 50 + i), dtype=torch.float32, device=DEV))
        signs.append(torch.from_numpy(sg).to(DEV) if rot else None)
        refs.append(oracle_product(layout, t, s, x16.view(np.uint16), oracle.X_F16, signs=sg if rot else None,
                                   block=rot or 128))
    tgs.ternary_gemv_batched(ws, xs, ys, signs=signs)
    torch.cuda.synchronize()
    for y, (y_ref, bound) in zip(ys, refs):
        assert_within_bound(y.cpu().numpy(), y_ref, bound, "mixed batch")


def test_wrong_basis_is_refused_on_the_device_path():
    t, s = make_weights(1, "basis", 8, 256, 0.4)
    w = _packed(tgs.SLOT2, t, s, rotated=True)
    with pytest.raises(tgs.TgsError) as info:
        tgs.ternary_gemv(w, _x_dev(make_x_f16(1, "basis", 1, 256)))
    assert info.value.name == "TGS_E_BASIS"


# ------------------------------------------------------------------------------ Hadamard

@pytest.mark.parametrize("in_dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("out_dtype", ["f32", "f16"])
def test_hadamard_rotate_matches_oracle(in_dtype, out_dtype):
    m, k = 3, 1280
    sg = make_signs(2, "had", k)
    xd = synth.normal(2, 9, (m, k))
    if in_dtype == "f16":
        host = xd.astype(np.float16)
        xt = torch.from_numpy(host.copy()).to(DEV)
        xref = host.astype(np.float64)
    elif in_dtype == "bf16":
        bits = synth.bf16_bits(xd)
        xt = torch.from_numpy(bits.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
        xref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        host = xd.astype(np.float32)
        xt = torch.from_numpy(host.copy()).to(DEV)
        xref = host.astype(np.float64)
    od = torch.float32 if out_dtype == "f32" else torch.float16
    y = tgs.hadamard_rotate_g128(xt, torch.from_numpy(sg).to(DEV), out_dtype=od)
    torch.cuda.synchronize()
    ref = oracle.rotate(xref, sg)
    got = y.float().cpu().numpy().astype(np.float64)
    blk_l1 = np.repeat(np.abs(xref).reshape(m, -1, 128).sum(axis=2), 128, axis=1) / np.sqrt(128)
    if out_dtype == "f32":
        assert (np.abs(got - ref) <= 1e-6 * blk_l1 + 1e-30).all()
    else:
        assert (np.abs(got - ref) <= 2.0 ** -11 * np.abs(ref) + 1e-6 * blk_l1 + 2.0 ** -25).all()


@pytest.mark.parametrize("in_dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("out_dtype", ["f32", "f16"])
def test_hadamard_rotate_1024_matches_oracle(in_dtype, out_dtype):
    m, k = 3, 3072
    sg = make_signs(4, "had1024", k)
    xd = synth.normal(4, 10, (m, k))
    if in_dtype == "f16":
        host = xd.astype(np.float16)
        xt = torch.from_numpy(host.copy()).to(DEV)
        xref = host.astype(np.float64)
    elif in_dtype == "bf16":
        bits = synth.bf16_bits(xd)
        xt = torch.from_numpy(bits.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
        xref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        host = xd.astype(np.float32)
        xt = torch.from_numpy(host.copy()).to(DEV)
        xref = host.astype(np.float64)
    od = torch.float32 if out_dtype == "f32" else torch.float16
    y = tgs.hadamard_rotate(xt, torch.from_numpy(sg).to(DEV), block=1024, out_dtype=od)
    torch.cuda.synchronize()
    ref = oracle.rotate(xref, sg, block=1024)
    got = y.float().cpu().numpy().astype(np.float64)
    blk_l1 = np.repeat(np.abs(xref).reshape(m, -1, 1024).sum(axis=2), 1024, axis=1) / np.sqrt(1024)
    if out_dtype == "f32":
        assert (np.abs(got - ref) <= 1e-6 * blk_l1 + 1e-30).all()
    else:
        assert (np.abs(got - ref) <= 2.0 ** -11 * np.abs(ref) + 1e-6 * blk_l1 + 2.0 ** -25).all()
    # the 128-block entry point is the general one at block 128
    y128 = tgs.hadamard_rotate(xt, torch.from_numpy(sg).to(DEV), block=128, out_dtype=od)
    y128b = tgs.hadamard_rotate_g128(xt, torch.from_numpy(sg).to(DEV), out_dtype=od)
    torch.cuda.synchronize()
    assert torch.equal(y128.view(torch.int16 if out_dtype == "f16" else torch.int32),
                       y128b.view(torch.int16 if out_dtype == "f16" else torch.int32))


@pytest.mark.parametrize("block,k", [(128, 128), (128, 384), (128, 640), (1024, 1024), (1024, 5120)])
@pytest.mark.parametrize("m", [1, 5, 13])
def test_hadamard_rotate_ragged_tiles(block, k, m):
    """A wave rotates 512 consecutive elements (four 128-blocks) or one 1024-block of the
    flattened rows: tiles that span rows, and a last tile with only some 128-blocks in it."""
    sg = make_signs(m + k, "hadrag", k)
    x16 = make_x_f16(m + k, f"hadrag{block}", m, k)
    y = tgs.hadamard_rotate(_x_dev(x16), torch.from_numpy(sg).to(DEV), block=block)
    gamma = synth.bf16_bits(1.0 + 0.3 * synth.normal(m + k, 13, (k,)))
    yn = tgs.rmsnorm_hadamard_rotate(_x_dev(x16), _gamma_dev(gamma), 1e-6, torch.from_numpy(sg).to(DEV),
                                     block=block)
    torch.cuda.synchronize()
    xref = x16.astype(np.float64)
    ref = oracle.rotate(xref, sg, block)
    blk_l1 = np.repeat(np.abs(xref).reshape(m, -1, block).sum(axis=2), block, axis=1) / np.sqrt(block)
    assert (np.abs(y.cpu().numpy() - ref) <= 1e-6 * blk_l1 + 1e-30).all()
    xhat = oracle.rmsnorm(xref, gamma, float(np.float32(1e-6)))
    refn = oracle.rmsnorm_rotate(x16.view(np.uint16), oracle.X_F16, gamma, float(np.float32(1e-6)), sg, block)
    blk_n = np.repeat(np.abs(xhat).reshape(m, -1, block).sum(axis=2), block, axis=1) / np.sqrt(block)
    assert (np.abs(yn.cpu().numpy() - refn) <= 2e-6 * blk_n + 1e-30).all()


def _bf16_rne(f32):
    """fp32 values -> bf16 bits, round to nearest with ties to even (finite inputs)."""
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("block", [128, 1024])
@pytest.mark.parametrize("norm", [False, True])
def test_rotation_bf16_output_is_the_rounded_fp32_output(block, norm):
    """bf16 output is the fp32 output rounded once to nearest-even, and within bf16's unit
    roundoff (2^-8) of the oracle's rotation."""
    m, k = 5, 3072
    sg = torch.from_numpy(make_signs(8, "rotbf16", k)).to(DEV)
    xd = synth.normal(8, 11, (m, k)) * np.array([[1e-3], [0.5], [3.0], [40.0], [900.0]])
    host = xd.astype(np.float16)
    xt = torch.from_numpy(host.copy()).to(DEV)
    xref = host.astype(np.float64)
    if norm:
        gamma = synth.bf16_bits(1.0 + 0.3 * synth.normal(8, 12, (k,)))
        rot = lambda od: tgs.rmsnorm_hadamard_rotate(xt, _gamma_dev(gamma), 1e-6, sg, block=block, out_dtype=od)
        ref = oracle.rmsnorm_rotate(host.view(np.uint16), oracle.X_F16, gamma, float(np.float32(1e-6)),
                                    make_signs(8, "rotbf16", k), block)
        src = oracle.rmsnorm(xref, gamma, float(np.float32(1e-6)))
    else:
        rot = lambda od: tgs.hadamard_rotate(xt, sg, block=block, out_dtype=od)
        ref = oracle.rotate(xref, make_signs(8, "rotbf16", k), block)
        src = xref
    y32, y16 = rot(torch.float32), rot(torch.bfloat16)
    torch.cuda.synchronize()
    got32 = y32.cpu().numpy()
    got16 = y16.view(torch.int16).cpu().numpy().view(np.uint16)
    assert (got16 == _bf16_rne(got32)).all()
    got = (got16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    blk_l1 = np.repeat(np.abs(src).reshape(m, -1, block).sum(axis=2), block, axis=1) / np.sqrt(block)
    assert (np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 2e-6 * blk_l1 + 1e-38).all()


ROT_LAYOUTS = [tgs.SLOT2, tgs.BASE3, tgs.BINARY]


@pytest.mark.parametrize("layout", ROT_LAYOUTS, ids=["slot2", "base3", "binary"])
@pytest.mark.parametrize("block", [128, 1024])
@pytest.mark.parametrize("m", [1, 24, 130])
def test_rotated_prefill_two_pass_matches_oracle(layout, block, m):
    """Prefill with rotated weights: rotate the activations once into bf16, then ternary_gemm
    with a plain-basis descriptor of the same codes. Two references:
    - the oracle's rotation rounded to bf16 (via fp32, as the kernel rounds), multiplied by the
      oracle: within the usual bound;
    - the oracle's rotated product itself (no rounding of R x): within the bound derived for one
      bf16 rounding of every rotated activation. With B = sum |s t (R x)| and bf16's unit roundoff
      2^-8, |y - y_exact| <= 2^-8 B + 1e-3 (1 + 2^-8) B + 1e-6; the plain bound alone
      (1e-3 B + 1e-6) does not hold on this route, and the header says so."""
    n, k = 200, 3072
    if layout == tgs.BINARY:
        t, s = _binary_weights(m, f"rotpre{block}", n, k)
    else:
        t, s = make_weights(m, f"rotpre{layout}{block}", n, k, 0.4)
    sg = make_signs(m, f"rotpre{block}", k)
    x16 = make_x_f16(m, f"rotpre{block}", m, k)
    xr = tgs.hadamard_rotate(_x_dev(x16), torch.from_numpy(sg).to(DEV), block=block, out_dtype=torch.bfloat16)
    y = tgs.ternary_gemm(_packed(layout, t, s), xr)
    torch.cuda.synchronize()
    xr_bits = synth.bf16_bits(oracle.rotate(x16.astype(np.float64), sg, block))
    y_ref, bound = oracle_product(layout, t, s, xr_bits, oracle.X_BF16)
    assert_within_bound(y.cpu().numpy(), y_ref, bound, f"rotated prefill {layout} block {block} m={m}")
    y_exact, bound_exact = oracle_product(layout, t, s, x16.view(np.uint16), oracle.X_F16, signs=sg, block=block)
    b = (bound_exact - 1e-6) / 1e-3  # sum |s t (R x)| per output
    derived = (2.0 ** -8 + 1e-3 * (1 + 2.0 ** -8)) * b + 1e-6
    assert_within_bound(y.cpu().numpy(), y_exact, derived, f"rotated prefill vs unrounded rotation {layout} {block} m={m}")


def test_misaligned_signs_are_refused():
    k = 2048
    t, s = make_weights(1, "sgal", 8, k, 0.4)
    w = _packed(tgs.BASE3, t, s, rotated=1024)
    sg = torch.from_numpy(np.ones(k + 16, dtype=np.int8)).to(DEV)
    with pytest.raises(tgs.TgsError) as info:
        tgs.ternary_gemv(w, _x_dev(make_x_f16(1, "sgal", 1, k)), signs=sg[4:4 + k])
    assert info.value.name == "TGS_E_ALIGN"


# ------------------------------------------------------------------------------ GEMM

def _gemm(layout, t, s, xbits, split=True):
    w = _packed(layout, t, s)
    xt = torch.from_numpy(xbits.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    y = tgs.ternary_gemm(w, xt, split=split)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("layout", LAYOUTS, ids=LNAME.get)
@pytest.mark.parametrize("n,k", [(128, 128), (300, 1024), (129, 2048), (64, 640), (70, 4352), (90, 2176)])
@pytest.mark.parametrize("m", [1, 8, 16, 24, 32, 50, 128, 200])
def test_gemm_matches_oracle(layout, n, k, m):
    t, s = make_weights(n + k + m, f"gemm{layout}", n, k, 0.4)
    xb = make_x_bf16_bits(m, f"gemm{n}", m, k)
    y = _gemm(layout, t, s, xb)
    y_ref, bound = oracle_product(layout, t, s, xb, oracle.X_BF16)
    assert_within_bound(y, y_ref, bound, f"gemm {LNAME[layout]} {n}x{k} m={m}")


@pytest.mark.parametrize("n", [4100, 9000, 13000, 17000, 33000])
@pytest.mark.parametrize("m", [5, 16, 20])
def test_gemm_wide_matrices(n, m):
    """Wide matrices take the few-row product: up to 16 rows with 2..6 output blocks per
    workgroup (n / 4096 rounded up), 17..32 rows with 1, 2 or 4."""
    k = 384
    t, s = make_weights(n + m, "gemmwide", n, k, 0.4)
    xb = make_x_bf16_bits(m, f"gemmwide{n}", m, k)
    y = _gemm(tgs.SLOT2, t, s, xb)
    y_ref, bound = oracle_product(tgs.SLOT2, t, s, xb, oracle.X_BF16)
    assert_within_bound(y, y_ref, bound, f"gemm wide {n}x{k} m={m}")


@pytest.mark.parametrize("n,k,m", [(16400, 1024, 16), (8200, 3072, 7), (1000, 2560, 16), (333, 512, 3),
                                   (4096, 9216, 16), (17, 4608, 12), (8192, 512, 1), (300, 8192, 16),
                                   (24000, 1024, 9)])
def test_gemm_few_rows_shapes(n, k, m):
    """Up to 16 activation rows over partial 16-output blocks, 1 to 16 rows, K from one to 18
    windows of 512 and n from 17 to 24000 (2 to 6 output blocks per workgroup)."""
    t, s = make_weights(n + k + 3 * m, "gemmfew", n, k, 0.4)
    xb = make_x_bf16_bits(n + m, "gemmfewx", m, k)
    y = _gemm(tgs.SLOT2, t, s, xb)
    rows = None if n <= 4096 else np.unique(np.r_[0, n - 1, np.linspace(0, n - 1, 300).astype(np.int64)])
    y_ref, bound = oracle_product(tgs.SLOT2, t, s, xb, oracle.X_BF16, rows=rows)
    got = y if rows is None else y[:, rows]
    assert_within_bound(got, y_ref, bound, f"gemm few rows {n}x{k} m={m}")


def test_gemm_sixteen_rows_integer_inputs_are_exact():
    """Integer activations and power-of-two scales with 16 rows and K = 4096: every partial is
    exact in fp32, so the result equals the oracle bit for bit."""
    n, k, m = 1040, 4096, 16
    t, _ = make_weights(13, "gemmexact16", n, k, 0.4)
    s = np.ldexp(1.0, synth.trits(13, 7, (n, k // 128), 0.0).astype(np.int64)).astype(np.float16)
    xi = (synth.trits(13, 8, (m, k), 0.2).astype(np.int64) * 3).astype(np.float32)
    y_gemm = _gemm(tgs.SLOT2, t, s, synth.bf16_bits(xi))
    y_ref, _ = oracle_product(tgs.SLOT2, t, s, synth.bf16_bits(xi), oracle.X_BF16)
    assert (y_gemm.astype(np.float64) == y_ref).all()


@pytest.mark.parametrize("split", [False, True], ids=["in_workgroup", "across_workgroups"])
@pytest.mark.parametrize("layout", ROT_LAYOUTS, ids=["slot2", "base3", "binary"])
@pytest.mark.parametrize("n,k,m", [(300, 8192, 100), (200, 8448, 40), (1000, 16384, 128)])
def test_gemm_four_k_parts(layout, n, k, m, split):
    """Few 64 x 64 tiles over a long K (at least 64 groups) split K in four parts: inside the
    workgroup without a workspace (8448 = 66 groups leaves the last parts' final group past the
    end: loaded, not multiplied), or across workgroups with one. Either way the parts' sums are
    added in part order."""
    t, s = make_weights(n + k + m, f"gemm4k{layout}", n, k, 0.0 if layout == tgs.BINARY else 0.4)
    xb = make_x_bf16_bits(n + m, "gemm4kx", m, k)
    y = _gemm(layout, t, s, xb, split=split)
    y_ref, bound = oracle_product(layout, t, s, xb, oracle.X_BF16)
    assert_within_bound(y, y_ref, bound, f"gemm four K parts layout {layout} {n}x{k} m={m}")


# (n, k, m, parts): K split across workgroups. Skinny kernel (m <= 32; one block of 16 rows, or
# two above 16): FB in 2..6 (2..5 for two blocks) and parts in 1..min(4, groups / 32), the most
# workgroups ceil(n / 16 FB) * parts that fit one per CU (256), ties to the larger FB
# (4100 x 8192: FB = 3 in two parts). Tiled kernel (64 x 64 tiles, 33 <= m <= 128):
# parts = min(ceil(640 / tiles), 4, groups / 32). Ragged n, parts that do not divide the groups
# (130 / 4, 65 / 2, 66 / 2), one row, 17 to 32 rows, parts of exactly 32 groups, and a product
# with too few groups to split.
SPLIT_CASES = [(512, 16384, 1, 4), (1000, 16640, 16, 4), (70, 8320, 5, 2), (4100, 8192, 16, 2), (600, 16384, 100, 4),
               (130, 8448, 64, 2), (64, 4096, 33, 1), (1000, 16640, 24, 4), (70, 8320, 32, 2), (4100, 8192, 17, 2)]


def _split_bytes(n, m, parts, skinny):
    """Workspace of a split product: an [m][n] fp32 slice per extra part (skinny kernel), or one
    [64][64] slice per tile and extra part (tiled kernel, every 64 x 64 tile split)."""
    per = m * n if skinny else -(-n // 64) * -(-m // 64) * 64 * 64
    return (parts - 1) * per * 4


def _tile_parts(n, k, m):
    """Parts of the tiled kernel's split for 64 x 64 tiles: min(ceil(640 / tiles), 4, groups / 32)."""
    tiles = -(-n // 64) * -(-m // 64)
    return max(1, min(-(-640 // tiles), 4, (k // 128) // 32))


@pytest.mark.parametrize("layout", ROT_LAYOUTS, ids=["slot2", "base3", "binary"])
@pytest.mark.parametrize("n,k,m,parts", SPLIT_CASES)
def test_gemm_split_across_workgroups(layout, n, k, m, parts):
    """The K split across workgroups (ternary_gemm_ws): within the bound of the oracle, the
    workspace size is (parts - 1) * m * n fp32, and repeated calls are bit-identical (the parts
    are added in part order, no atomics). The single-launch product is within the bound too."""
    skinny = m <= 32 and layout != tgs.BASE3  # base-3 always takes the tiled kernel
    if layout == tgs.BASE3 and m <= 32:
        parts = _tile_parts(n, k, m)
    t, s = make_weights(n + k + m, f"gemmsplit{layout}", n, k, 0.0 if layout == tgs.BINARY else 0.4)
    xb = make_x_bf16_bits(n + m, "gemmsplitx", m, k)
    w = _packed(layout, t, s)
    assert tgs.gemm_workspace_bytes(w, m) == _split_bytes(n, m, parts, skinny)
    xt = torch.from_numpy(xb.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    y1 = tgs.ternary_gemm(w, xt).cpu().numpy()
    ws = torch.full((max(1, _split_bytes(n, m, parts, skinny) // 4),), float("nan"), device=DEV)  # no state kept
    y2 = tgs.ternary_gemm(w, xt, workspace=ws).cpu().numpy()
    y0 = tgs.ternary_gemm(w, xt, split=False).cpu().numpy()
    y_ref, bound = oracle_product(layout, t, s, xb, oracle.X_BF16)
    assert_within_bound(y1, y_ref, bound, f"gemm split layout {layout} {n}x{k} m={m} parts={parts}")
    assert_within_bound(y0, y_ref, bound, f"gemm unsplit layout {layout} {n}x{k} m={m}")
    assert (y1.view(np.uint32) == y2.view(np.uint32)).all()


def test_gemm_split_workspace_checks():
    """A workspace below the needed size is refused (binding and C entry point) before any launch;
    a NULL workspace is the single-launch product; a product that is not split needs none."""
    n, k, m = 512, 16384, 16
    t, s = make_weights(5, "gemmsplitws", n, k, 0.4)
    w = _packed(tgs.SLOT2, t, s)
    need = tgs.gemm_workspace_bytes(w, m)
    assert need == 3 * m * n * 4
    xt = torch.from_numpy(make_x_bf16_bits(5, "gemmsplitwsx", m, k).view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    y = torch.zeros(m, n, device=DEV)
    with pytest.raises(tgs.TgsError) as e:
        tgs.ternary_gemm(w, xt, y, workspace=torch.empty(need // 4 - 1, device=DEV))
    assert e.value.status == 7
    small = torch.empty(need // 4 - 1, device=DEV)
    st = tgs.lib().ternary_gemm_ws(ctypes.byref(w.desc), xt.data_ptr(), tgs.BF16, m, None, y.data_ptr(),
                                   small.data_ptr(), need - 4, None)
    assert st == 7 and not y.any()
    st = tgs.lib().ternary_gemm_ws(ctypes.byref(w.desc), xt.data_ptr(), tgs.BF16, m, None, y.data_ptr(), None, 0,
                                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    y0 = tgs.ternary_gemm(w, xt, split=False)
    assert torch.equal(y, y0)
    w_short = _packed(tgs.SLOT2, *make_weights(6, "gemmsplitws2", 512, 5120, 0.4))
    assert tgs.gemm_workspace_bytes(w_short, m) == 0  # 40 groups: too few to split


def test_gemm_split_large_tiles_sampled():
    """540 tiles of 128 x 128 (9 x 60) over 64 groups: 512 tiles (one full round of two
    workgroups per CU) taken whole, the last 28 in four parts across workgroups; checked on
    sampled output columns, with the workspace size (3 extra parts x 28 tiles x 128 x 128)."""
    n, k, m = 7680, 8192, 1040
    t, s = make_weights(37, "gemmsplitbig", n, k, 0.4)
    xb = make_x_bf16_bits(37, "gemmsplitbigx", m, k)
    w = _packed(tgs.SLOT2, t, s)
    assert tgs.gemm_workspace_bytes(w, m) == 3 * 28 * 128 * 128 * 4
    xt = torch.from_numpy(xb.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    y = tgs.ternary_gemm(w, xt).cpu().numpy()
    cols = np.sort(np.random.default_rng(5).choice(n, size=64, replace=False))
    cols[0], cols[-1] = 0, n - 1
    y_ref, bound = oracle_product(tgs.SLOT2, t, s, xb, oracle.X_BF16, rows=cols)
    assert_within_bound(y[:, cols], y_ref, bound, f"gemm split {n}x{k} m={m} sampled")


def test_gemm_split_on_a_side_stream():
    """A split product on a stream of its own (its temporary workspace allocated on that stream),
    twice in a row with the stream's own work between: bit-identical to the product on the
    current stream."""
    n, k, m = 512, 16384, 16
    t, s = make_weights(43, "gemmsplitstream", n, k, 0.4)
    w = _packed(tgs.SLOT2, t, s)
    assert tgs.gemm_workspace_bytes(w, m) > 0
    xt = torch.from_numpy(make_x_bf16_bits(43, "gemmsplitstreamx", m, k).view(np.int16).copy()).to(DEV)
    xt = xt.view(torch.bfloat16)
    ref = tgs.ternary_gemm(w, xt)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    with torch.cuda.stream(side):
        for _ in range(2):
            y = tgs.ternary_gemm(w, xt, stream=side)
            outs.append(y.clone())
            y.zero_()
    torch.cuda.synchronize()
    for y in outs:
        assert torch.equal(y, ref)


def test_gemm_split_balance_sampled():
    """532 tiles of 64 x 64 (2 x 266) over 16 groups: 512 taken whole (two per CU) and the last 20
    (row tile 1, columns 15744..16999) in two K parts; checked on sampled columns that include
    all of the split tiles' last 64 and some of the rest."""
    n, k, m = 17000, 2048, 100
    t, s = make_weights(41, "gemmbal", n, k, 0.4)
    xb = make_x_bf16_bits(41, "gemmbalx", m, k)
    w = _packed(tgs.SLOT2, t, s)
    assert tgs.gemm_workspace_bytes(w, m) == 20 * 64 * 64 * 4
    xt = torch.from_numpy(xb.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    y = tgs.ternary_gemm(w, xt).cpu().numpy()
    rng = np.random.default_rng(7)
    cols = np.unique(np.r_[np.arange(n - 64, n), rng.choice(15744, 48, replace=False),
                           15744 + rng.choice(n - 64 - 15744, 48, replace=False), 0])
    y_ref, bound = oracle_product(tgs.SLOT2, t, s, xb, oracle.X_BF16, rows=cols)
    assert_within_bound(y[:, cols], y_ref, bound, f"gemm balanced split {n}x{k} m={m} sampled")


@pytest.mark.parametrize("layout", [tgs.SLOT2, tgs.BINARY], ids=["slot2", "binary"])
@pytest.mark.parametrize("n,k,m", [(8192, 256, 1040), (8190, 384, 1100), (4200, 128, 2100)])
def test_gemm_large_tiles_sampled(layout, n, k, m):
    """Many rows and columns take 128 x 128 tiles: slot-2 and binary codes, ragged m and n, one to
    three groups; checked on sampled output columns."""
    t, s = make_weights(31, "gemmbig", n, k, 0.0 if layout == tgs.BINARY else 0.4)
    xb = make_x_bf16_bits(31, "gemmbigx", m, k)
    y = _gemm(layout, t, s, xb)
    cols = np.sort(np.random.default_rng(3).choice(n, size=96, replace=False))
    cols[0], cols[-1] = 0, n - 1
    y_ref, bound = oracle_product(layout, t, s, xb, oracle.X_BF16, rows=cols)
    assert_within_bound(y[:, cols], y_ref, bound, f"gemm layout {layout} {n}x{k} m={m} sampled")


@pytest.mark.parametrize("m", [1, 20, 40])
def test_gemm_integer_inputs_are_exact(m):
    """Integer activations and power-of-two scales: every partial sum is exact in fp32, so each
    GEMM path (skinny and tiled) must equal the oracle bit for bit."""
    n, k = 200, 2304
    t, _ = make_weights(11 + m, "gemmexactm", n, k, 0.4)
    s = np.ldexp(1.0, synth.trits(11, 7, (n, k // 128), 0.0).astype(np.int64)).astype(np.float16)
    xi = (synth.trits(11 + m, 8, (m, k), 0.2).astype(np.int64) * 3).astype(np.float32)
    y_gemm = _gemm(tgs.SLOT2, t, s, synth.bf16_bits(xi))
    y_ref, _ = oracle_product(tgs.SLOT2, t, s, synth.bf16_bits(xi), oracle.X_BF16)
    assert (y_gemm.astype(np.float64) == y_ref).all()


def test_gemm_integer_inputs_are_exact_and_match_gemv():
    n, k, m = 160, 2048, 1
    t, _ = make_weights(9, "gemmexact", n, k, 0.4)
    s = np.ldexp(1.0, synth.trits(9, 5, (n, k // 128), 0.0).astype(np.int64)).astype(np.float16)
    xi = (synth.trits(9, 6, (m, k), 0.2).astype(np.int64) * 3).astype(np.float32)
    y_gemm = _gemm(tgs.SLOT2, t, s, synth.bf16_bits(xi))
    y_gemv = _gemv(tgs.SLOT2, t, s, xi.astype(np.float16))
    y_ref, _ = oracle_product(tgs.SLOT2, t, s, xi.astype(np.float16).view(np.uint16), oracle.X_F16)
    assert (y_gemm.astype(np.float64) == y_ref).all()
    assert (y_gemm.view(np.uint32) == y_gemv.view(np.uint32)).all()


# ------------------------------------------------------------------------------ code flips

def _flip_pair(layout, n, k, frac, seed, pad=0):
    """Two packed checkpoints: t and t with a seeded fraction of trits changed. Returns
    (PackedMatrix a, PackedMatrix b, codes_a, codes_b) where codes_a and codes_b are the oracle's
    own packing (the library's bytes must equal them; the padded stride copies the oracle's)."""
    t = synth.trits(seed, n * 7 + k, (n, k), 0.4)
    rng = np.random.default_rng(seed)
    mask = rng.random((n, k)) < frac
    step = rng.integers(1, 3, size=(n, k))
    u = t.copy()
    u[mask] = ((t[mask].astype(np.int64) + 1 + step[mask]) % 3 - 1).astype(np.int8)
    s = synth.scales_f16(seed, 5, (n, k // 128))
    ca, _ = tgs.pack_ternary(layout, t, s)
    cb, _ = tgs.pack_ternary(layout, u, s)
    assert np.array_equal(ca, oracle.pack(layout, t)) and np.array_equal(cb, oracle.pack(layout, u))
    ca, cb = oracle.pack(layout, t), oracle.pack(layout, u)
    if pad:  # a wider row stride for the first matrix, with garbage past its codes
        wide = np.full((n, ca.shape[1] + pad), 0xEE, dtype=np.uint8)
        wide[:, :ca.shape[1]] = ca
        ca = wide
    sd = torch.from_numpy(s.view(np.int16)).to(DEV)
    a = tgs.PackedMatrix(layout, torch.from_numpy(ca).to(DEV), sd, k)
    b = tgs.PackedMatrix(layout, torch.from_numpy(cb).to(DEV), sd, k)
    return a, b, ca, cb


@pytest.mark.parametrize("layout", LAYOUTS, ids=LNAME.get)
@pytest.mark.parametrize("n,k,frac", [(1, 128, 0.5), (17, 384, 0.05), (300, 1280, 0.007), (33, 4096, 0.1),
                                      (129, 12288, 0.003), (5, 17408, 0.02)])
def test_code_flips_match_oracle(layout, n, k, frac):
    a, b, ca, cb = _flip_pair(layout, n, k, frac, seed=n + k)
    total, rows = tgs.ternary_code_flips(a, b)
    torch.cuda.synchronize()
    ref_total, ref_rows = oracle.code_flips(layout, ca, cb, k)
    assert int(total.item()) == ref_total
    assert (rows.cpu().numpy().astype(np.int64) == ref_rows).all()
    total2, rows2 = tgs.ternary_code_flips(a, b)
    assert int(total2.item()) == ref_total and torch.equal(rows, rows2)  # identical run to run


@pytest.mark.parametrize("layout", LAYOUTS, ids=LNAME.get)
def test_code_flips_extremes_strides_and_outputs(layout):
    n, k = 70, 640
    a, _, ca, _ = _flip_pair(layout, n, k, 0.0, seed=3, pad=48)
    t = tgs.unpack_ternary(layout, ca[:, :tgs.code_row_bytes(layout, k)], np.zeros((n, k // 128), np.float16), k)[0]
    every = ((t.astype(np.int64) + 2) % 3 - 1).astype(np.int8)
    cb = tgs.pack_ternary(layout, every, None)[0]
    b = tgs.PackedMatrix(layout, torch.from_numpy(cb).to(DEV), a.scales, k)
    assert int(tgs.ternary_code_flips(a, a)[0].item()) == 0
    total, rows = tgs.ternary_code_flips(a, b)
    assert int(total.item()) == n * k and (rows.cpu().numpy() == k).all()
    # only a total, only rows
    t_only, none_rows = tgs.ternary_code_flips(a, b, rows=False)
    none_total, r_only = tgs.ternary_code_flips(a, b, total=False)
    assert none_rows is None and none_total is None
    assert int(t_only.item()) == n * k and (r_only.cpu().numpy() == k).all()


def test_code_flips_batched_equals_single_calls():
    pairs, refs = [], []
    for i, (n, k) in enumerate([(40, 1024), (300, 4096), (7, 12288)]):
        a, b, ca, cb = _flip_pair(tgs.SLOT2, n, k, 0.01 * (i + 1), seed=20 + i)
        pairs.append((a, b))
        refs.append(oracle.code_flips(tgs.SLOT2, ca, cb, k))
    totals = [torch.empty(1, dtype=torch.int64, device=DEV) for _ in pairs]
    rows = [torch.empty(a.n, dtype=torch.int32, device=DEV) for a, _ in pairs]
    tgs.ternary_code_flips_batched(pairs, totals, rows)
    torch.cuda.synchronize()
    for t, r, (ref_t, ref_r) in zip(totals, rows, refs):
        assert int(t.item()) == ref_t
        assert (r.cpu().numpy().astype(np.int64) == ref_r).all()


def test_code_flips_full_size_matrix():
    """A 12288 x 4096 gate/up-sized matrix at the 0.7% flip rate the fine-tuning page reports."""
    a, b, ca, cb = _flip_pair(tgs.SLOT2, 12288, 4096, 0.007, seed=77)
    total, rows = tgs.ternary_code_flips(a, b)
    ref_total, ref_rows = oracle.code_flips(tgs.SLOT2, ca, cb, 4096)
    assert int(total.item()) == ref_total
    assert (rows.cpu().numpy().astype(np.int64) == ref_rows).all()


# ------------------------------------------------------------------------------ binary codes
# The two-level sibling format: t in {-1, +1}, one bit per weight, the same fp16 group scales.


def _binary_weights(seed, stream, n, k):
    t = synth.trits(seed, synth.stream_id(stream, "codes"), (n, k), 0.0)  # {-1, +1}
    s = synth.scales_f16(seed, synth.stream_id(stream, "scales"), (n, k // 128))
    return t, s


def test_binary_packing_on_the_device_path_round_trips():
    t, s = _binary_weights(0, "binpack", 64, 1024)
    codes, _ = tgs.pack_ternary(tgs.BINARY, t, s)
    assert (codes == oracle.pack(tgs.BINARY, t)).all()
    assert (tgs.unpack_ternary(tgs.BINARY, codes, s, 1024)[0] == t).all()


@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("m", [1, 2, 3, 8])
def test_binary_gemv_matches_oracle(n, k, m):
    t, s = _binary_weights(n + k, "bingemv", n, k)
    x16 = make_x_f16(m, f"bingemv{n}x{k}", m, k)
    y = _gemv(tgs.BINARY, t, s, x16)
    y_ref, bound = oracle_product(tgs.BINARY, t, s, x16.view(np.uint16), oracle.X_F16)
    assert_within_bound(y, y_ref, bound, f"binary {n}x{k} m={m}")


@pytest.mark.parametrize("block", [128, 1024])
@pytest.mark.parametrize("n,k", [(33, 1024), (100, 5120), (20, 17408)])
@pytest.mark.parametrize("m", [1, 3, 8])
def test_binary_rotated_gemv_matches_oracle(block, n, k, m):
    t, s = _binary_weights(n + k + block, "binrot", n, k)
    x16 = make_x_f16(m + 5, f"binrot{n}x{k}", m, k)
    sg = make_signs(k, "binrot", k)
    y = _gemv(tgs.BINARY, t, s, x16, signs=sg, block=block)
    y_ref, bound = oracle_product(tgs.BINARY, t, s, x16.view(np.uint16), oracle.X_F16, signs=sg, block=block)
    assert_within_bound(y, y_ref, bound, f"binary rotated-{block} {n}x{k} m={m}")


@pytest.mark.parametrize("m", [1, 3])
def test_binary_special_rows_and_integer_exactness(m):
    # all +1 rows give s * sum x, all -1 rows -s * sum x; alternating signs and a single -1 among
    # +1s too. Integer x in [-4, 4] with power-of-two scales: every partial sum is exact in fp32,
    # so the GPU must equal the oracle bit for bit.
    k = 4096
    t = np.ones((6, k), dtype=np.int8)
    t[1] = -1
    t[2, 1::2] = -1
    t[3, 2049] = -1
    t[4, :] = synth.trits(7, 1, (k,), 0.0)
    t[5, 64:] = -1
    s = np.ldexp(1.0, synth.trits(7, 2, (6, k // 128), 0.0).astype(np.int64)).astype(np.float16)
    xi = synth.trits(7, 3, (m, k), 0.2).astype(np.int64) * 4 + synth.trits(7, 4, (m, k), 0.3)
    x16 = xi.astype(np.float16)
    y = _gemv(tgs.BINARY, t, s, x16)
    y_ref, _ = oracle_product(tgs.BINARY, t, s, x16.view(np.uint16), oracle.X_F16)
    assert (y.astype(np.float64) == y_ref).all()


def test_binary_batched_with_other_layouts():
    k = 2048
    sg = make_signs(2, "binmix", k)
    cases = [(tgs.BINARY, 0), (tgs.SLOT2, 0), (tgs.BINARY, 128), (tgs.BASE3, 0), (tgs.BINARY, 1024)]
    ws, xs, ys, signs, refs = [], [], [], [], []
    for i, (layout, rot) in enumerate(cases):
        if layout == tgs.BINARY:
            t, s = _binary_weights(i, "binmix", 40 + i, k)
        else:
            t, s = make_weights(i, "binmix", 40 + i, k, 0.4)
        x16 = make_x_f16(i, "binmix", 2, k)
        ws.append(_packed(layout, t, s, rotated=rot))
        xs.append(_x_dev(x16))
        ys.append(torch.empty((2, 40 + i), dtype=torch.float32, device=DEV))
        signs.append(torch.from_numpy(sg).to(DEV) if rot else None)
        refs.append(oracle_product(layout, t, s, x16.view(np.uint16), oracle.X_F16, signs=sg if rot else None,
                                   block=rot or 128))
    tgs.ternary_gemv_batched(ws, xs, ys, signs=signs)
    torch.cuda.synchronize()
    for y, (y_ref, bound) in zip(ys, refs):
        assert_within_bound(y.cpu().numpy(), y_ref, bound, "binary mixed batch")


@pytest.mark.parametrize("n,k", [(64, 256), (200, 2048), (130, 1280), (257, 640)])
@pytest.mark.parametrize("m", [1, 16, 40, 128, 200])
def test_binary_gemm_matches_oracle(n, k, m):
    t, s = _binary_weights(n + m, "bingemm", n, k)
    xb = make_x_bf16_bits(m, f"bingemm{n}", m, k)
    y = _gemm(tgs.BINARY, t, s, xb)
    y_ref, bound = oracle_product(tgs.BINARY, t, s, xb, oracle.X_BF16)
    assert_within_bound(y, y_ref, bound, f"binary gemm {n}x{k} m={m}")


def test_binary_gemm_integer_inputs_are_exact_and_match_gemv():
    n, k, m = 160, 2048, 1
    t, _ = _binary_weights(9, "bingemmexact", n, k)
    s = np.ldexp(1.0, synth.trits(9, 5, (n, k // 128), 0.0).astype(np.int64)).astype(np.float16)
    xi = (synth.trits(9, 6, (m, k), 0.2).astype(np.int64) * 3).astype(np.float32)
    y_gemm = _gemm(tgs.BINARY, t, s, synth.bf16_bits(xi))
    y_gemv = _gemv(tgs.BINARY, t, s, xi.astype(np.float16))
    y_ref, _ = oracle_product(tgs.BINARY, t, s, xi.astype(np.float16).view(np.uint16), oracle.X_F16)
    assert (y_gemm.astype(np.float64) == y_ref).all()
    assert (y_gemm.view(np.uint32) == y_gemv.view(np.uint32)).all()


@pytest.mark.parametrize("n,k,frac", [(1, 128, 0.5), (17, 384, 0.05), (300, 1280, 0.007), (129, 12288, 0.003)])
def test_binary_code_flips_match_oracle(n, k, frac):
    t, s = _binary_weights(n + k, "binflip", n, k)
    mask = np.random.default_rng(n + k).random((n, k)) < frac
    u = np.where(mask, -t, t).astype(np.int8)
    ca, _ = tgs.pack_ternary(tgs.BINARY, t, s)
    cb, _ = tgs.pack_ternary(tgs.BINARY, u, s)
    assert np.array_equal(ca, oracle.pack(tgs.BINARY, t)) and np.array_equal(cb, oracle.pack(tgs.BINARY, u))
    ca, cb = oracle.pack(tgs.BINARY, t), oracle.pack(tgs.BINARY, u)
    sd = torch.from_numpy(s.view(np.int16)).to(DEV)
    a = tgs.PackedMatrix(tgs.BINARY, torch.from_numpy(ca).to(DEV), sd, k)
    b = tgs.PackedMatrix(tgs.BINARY, torch.from_numpy(cb).to(DEV), sd, k)
    total, rows = tgs.ternary_code_flips(a, b)
    torch.cuda.synchronize()
    ref_total, ref_rows = oracle.code_flips(tgs.BINARY, ca, cb, k)
    assert ref_total == int(mask.sum())
    assert int(total.item()) == ref_total
    assert (rows.cpu().numpy().astype(np.int64) == ref_rows).all()


# ------------------------------------------------------------------------------ RMSNorm prologue
# xhat = gamma * x / sqrt(mean(x^2) + eps), gamma in bf16, then the rotation (if any) and the product.


def _norm_inputs(seed, m, k):
    """Activations with a different scale per row (hidden states, not unit normals) and bf16 gamma."""
    scale = np.array([0.05, 3.0, 40.0, 0.7, 11.0, 0.2, 6.0, 1.5])[:m, None]
    x16 = (synth.normal(seed, 1, (m, k)) * scale).astype(np.float16)
    gamma = synth.bf16_bits(1.0 + 0.25 * synth.normal(seed, 2, (k,)))
    return x16, gamma


def _gamma_dev(gamma):
    return torch.from_numpy(gamma.view(np.int16).copy()).to(DEV)


NORM_LAYOUT_BLOCKS = [(tgs.SLOT2, 0), (tgs.SLOT2, 128), (tgs.SLOT2, 1024), (tgs.BASE3, 0), (tgs.BASE3, 128),
                      (tgs.BASE3, 1024), (tgs.BINARY, 0), (tgs.BINARY, 1024)]


@pytest.mark.parametrize("layout,block", NORM_LAYOUT_BLOCKS, ids=lambda v: str(v))
@pytest.mark.parametrize("n,k", [(33, 1024), (100, 5120), (70, 2048), (20, 40960)])
@pytest.mark.parametrize("m", [1, 3, 8])
def test_rmsnorm_gemv_matches_oracle(layout, block, n, k, m):
    """Every kernel path takes the prologue: the single-token kernel (plain slot-2/binary, m = 1,
    K <= 32768), the general slot-2/binary kernel (the rest: K = 40960 for m = 1) and the base-3
    matrix-core kernel, each plain and with both rotation blocks."""
    if block == 1024 and k % 1024:
        pytest.skip("k is not a multiple of the rotation block")
    if layout == tgs.BINARY:
        t, s = _binary_weights(n + k, "norm", n, k)
    else:
        t, s = make_weights(n + k, f"norm{layout}", n, k, 0.4)
    x16, gamma = _norm_inputs(m + k, m, k)
    sg = make_signs(k, "norm", k) if block else None
    w = _packed(layout, t, s, rotated=block)
    eps = 1e-6
    y = tgs.ternary_gemv_rmsnorm(w, _x_dev(x16), _gamma_dev(gamma), eps,
                                 signs=torch.from_numpy(sg).to(DEV) if block else None)
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul(layout, oracle.pack(layout, t), s, k, x16.view(np.uint16), oracle.X_F16, signs=sg,
                                 block=block or 128, gamma=gamma, eps=float(np.float32(eps)))
    assert_within_bound(y.cpu().numpy(), y_ref, bound, f"rmsnorm {LNAME.get(layout, 'binary')} b{block} {n}x{k} m={m}")


def test_rmsnorm_gemv_zero_rows_and_batched():
    # an all-zero activation row normalises to zero (eps keeps the factor finite): y is exactly 0;
    # the batched call equals single calls bit for bit, gammas may differ per matrix
    k, m = 2048, 3
    sg = make_signs(5, "normb", k)
    x16, gamma = _norm_inputs(5, m, k)
    x16[1] = 0
    cases = [(tgs.SLOT2, 0), (tgs.BASE3, 128), (tgs.SLOT2, 1024), (tgs.BINARY, 128)]
    ws, gs, ys, signs, singles = [], [], [], [], []
    for i, (layout, rot) in enumerate(cases):
        if layout == tgs.BINARY:
            t, s = _binary_weights(i, "normb", 40 + i, k)
        else:
            t, s = make_weights(i, "normb", 40 + i, k, 0.4)
        w = _packed(layout, t, s, rotated=rot)
        g = _gamma_dev(synth.bf16_bits(1.0 + 0.1 * i + 0.2 * synth.normal(i, 7, (k,))))
        sgd = torch.from_numpy(sg).to(DEV) if rot else None
        ws.append(w)
        gs.append(g)
        signs.append(sgd)
        ys.append(torch.empty((m, 40 + i), dtype=torch.float32, device=DEV))
        singles.append(tgs.ternary_gemv_rmsnorm(w, _x_dev(x16), g, 1e-5, signs=sgd))
    tgs.ternary_gemv_rmsnorm_batched(ws, [_x_dev(x16)] * len(ws), gs, 1e-5, ys, signs=signs)
    torch.cuda.synchronize()
    for y, single in zip(ys, singles):
        assert torch.equal(y.view(torch.int32), single.view(torch.int32))
        assert (y[1] == 0).all()


@pytest.mark.parametrize("in_dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("block", [128, 1024])
def test_rmsnorm_hadamard_rotate_matches_oracle(in_dtype, block):
    m, k = 3, 3072
    sg = make_signs(6, "nrot", k)
    xd = synth.normal(6, 9, (m, k)) * np.array([[0.1], [5.0], [60.0]])
    gamma = synth.bf16_bits(1.0 + 0.3 * synth.normal(6, 10, (k,)))
    if in_dtype == "f16":
        host = xd.astype(np.float16)
        xt = torch.from_numpy(host.copy()).to(DEV)
        bits, xdt = host.view(np.uint16), oracle.X_F16
        xref = host.astype(np.float64)
    elif in_dtype == "bf16":
        bits = synth.bf16_bits(xd)
        xt = torch.from_numpy(bits.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
        xdt = oracle.X_BF16
        xref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        host = xd.astype(np.float32)
        xt = torch.from_numpy(host.copy()).to(DEV)
        bits, xdt = None, None
        xref = host.astype(np.float64)
    eps = 1e-6
    xhat = oracle.rmsnorm(xref, gamma, float(np.float32(eps)))
    blk_l1 = np.repeat(np.abs(xhat).reshape(m, -1, block).sum(axis=2), block, axis=1) / np.sqrt(block)
    for od in (torch.float32, torch.float16):
        y = tgs.rmsnorm_hadamard_rotate(xt, _gamma_dev(gamma), eps, torch.from_numpy(sg).to(DEV), block=block,
                                        out_dtype=od)
        torch.cuda.synchronize()
        got = y.float().cpu().numpy().astype(np.float64)
        if bits is not None:
            ref = oracle.rmsnorm_rotate(bits, xdt, gamma, float(np.float32(eps)), sg, block)
        else:  # fp32 input: the oracle's rotation of its own RMSNorm of the fp32 values
            ref = oracle.rotate(xhat, sg, block)
        tol = 2e-6 * blk_l1 + 1e-30 if od == torch.float32 else 2.0 ** -11 * np.abs(ref) + 2e-6 * blk_l1 + 2.0 ** -25
        assert (np.abs(got - ref) <= tol).all(), f"{in_dtype} block {block} {od}"
