"""Pins for the CPU oracle, independent of the oracle's own code.

Each check ties the oracle to something it does not compute itself: hand-worked bytes
(tests/golden), numpy/scipy library routines (IEEE decoding, Sylvester Hadamard, dense
matmul), closed forms of the group-scaled product, exhaustive enumeration and brute force
on tiny shapes. Citations name the page and section whose definition each check follows:
  P3 = "Ternary Bonsai 2 27B, 5.93GB ... (feat. PrismML)" (discuss.pytorch.kr)
  P2 = "Bonsai 27B and how 1-bit survives" (velog.io)
  P1 = "Fine-tuning the ternary Bonsai-8B on Metal" (molayo1419.me)
"""
import math
import os

import numpy as np
import pytest
import scipy.linalg

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_fixture(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split(";")
            rows.append(([int(v) for v in lhs.split()], rhs.strip()))
    return rows


# ---------------------------------------------------------------- storage dtypes

def test_f16_decode_matches_numpy_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_bf16_decode_matches_float32_top_half_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        ref = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    got = np.array([oracle.bf16_to_f64(int(b)) for b in bits])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


# ---------------------------------------------------------------- slot-2 bytes (P3, "Two packings")

def _row_with_prefix(prefix, k=128):
    t = np.zeros((1, k), dtype=np.int8)
    t[0, :len(prefix)] = prefix
    return t


@pytest.mark.parametrize("trits,hexbyte", _read_fixture("slot2_bytes.txt"))
def test_slot2_hand_bytes(trits, hexbyte):
    codes = oracle.pack(oracle.SLOT2, _row_with_prefix(trits))
    assert codes[0, 0] == int(hexbyte, 16)
    assert (codes[0, 1:] == 0x55).all()  # zero trits elsewhere: q = 1 in every slot


def test_slot2_all_zero_dword():
    codes = oracle.pack(oracle.SLOT2, np.zeros((1, 128), dtype=np.int8))
    assert codes[0, :4].view(np.uint32)[0] == 0x55555555


def test_slot2_every_byte_round_trips_or_is_rejected():
    valid = 0
    for b in range(256):
        slots = [(b >> (2 * i)) & 3 for i in range(4)]
        codes = np.full((1, 32), 0x55, dtype=np.uint8)
        codes[0, 0] = b
        if 3 in slots:
            with pytest.raises(oracle.OracleError):
                oracle.unpack(oracle.SLOT2, codes, 128)
            continue
        valid += 1
        t = oracle.unpack(oracle.SLOT2, codes, 128)
        assert list(t[0, :4]) == [s - 1 for s in slots]
        assert (oracle.pack(oracle.SLOT2, t) == codes).all()
    assert valid == 81


def test_slot2_random_round_trip_and_position():
    t = synth.trits(0, 11, (5, 384), 0.4)
    codes = oracle.pack(oracle.SLOT2, t)
    assert codes.shape == (5, 96)
    assert (oracle.unpack(oracle.SLOT2, codes, 384) == t).all()
    # element k lives in byte k//4 at bit 2*(k%4): check directly with numpy bit arithmetic
    for k in (0, 1, 2, 3, 4, 127, 128, 383):
        q = (codes[:, k // 4] >> (2 * (k % 4))) & 3
        assert (q.astype(np.int16) - 1 == t[:, k]).all()


def test_pack_rejects_bad_trits():
    t = np.zeros((1, 128), dtype=np.int8)
    t[0, 5] = 2
    for layout in (oracle.SLOT2, oracle.BASE3, oracle.BINARY):
        with pytest.raises(oracle.OracleError):
            oracle.pack(layout, t)


# ---------------------------------------------------------------- base-3 bytes

@pytest.mark.parametrize("trits,value", _read_fixture("base3_bytes.txt"))
def test_base3_hand_bytes(trits, value):
    codes = oracle.pack(oracle.BASE3, _row_with_prefix(trits))
    assert codes[0, 0] == int(value)
    assert codes.shape == (1, 32)  # ceil(128/5) = 26 bytes, padded to 32
    assert (codes[0, 1:26] == 121).all()
    assert (codes[0, 26:] == 121).all()


def test_base3_every_byte_round_trips_or_is_rejected():
    for b in range(256):
        codes = np.full((1, 32), 121, dtype=np.uint8)
        codes[0, 0] = b
        if b > 242:
            with pytest.raises(oracle.OracleError):
                oracle.unpack(oracle.BASE3, codes, 128)
            continue
        t = oracle.unpack(oracle.BASE3, codes, 128)
        digits = [(b // 3 ** j) % 3 for j in range(5)]
        assert list(t[0, :5]) == [d - 1 for d in digits]
        assert (oracle.pack(oracle.BASE3, t) == codes).all()


def test_base3_last_byte_of_k4096():
    # K = 4096: byte 819 holds trit 4095 and four positions past K (trit 0, digit 1 each):
    # value = (t_4095 + 1) + 3 + 9 + 27 + 81 = (t_4095 + 1) + 120
    for last in (-1, 0, 1):
        t = np.zeros((1, 4096), dtype=np.int8)
        t[0, -1] = last
        codes = oracle.pack(oracle.BASE3, t)
        assert codes.shape == (1, 832)
        assert codes[0, 819] == (last + 1) + 120
        assert (codes[0, 820:] == 121).all()


def test_base3_rejects_noncanonical_padding():
    t = synth.trits(0, 12, (1, 4096), 0.5)
    codes = oracle.pack(oracle.BASE3, t)
    bad = codes.copy()
    bad[0, 825] = 120  # pad byte must be 121
    with pytest.raises(oracle.OracleError):
        oracle.unpack(oracle.BASE3, bad, 4096)
    bad = codes.copy()
    bad[0, 819] = (t[0, -1] + 1) + 3 * 2  # a position past K carrying a nonzero trit
    with pytest.raises(oracle.OracleError):
        oracle.unpack(oracle.BASE3, bad, 4096)


def test_base3_random_round_trip():
    for k in (128, 1024, 4096, 5120, 12288):
        t = synth.trits(3, k, (3, k), 0.5)
        codes = oracle.pack(oracle.BASE3, t)
        assert (oracle.unpack(oracle.BASE3, codes, k) == t).all()
        # the digit rule written with numpy over the whole row
        used = (k + 4) // 5
        digits = np.ones((3, used * 5), dtype=np.int64)
        digits[:, :k] = t.astype(np.int64) + 1
        expect = (digits.reshape(3, used, 5) * (3 ** np.arange(5))).sum(axis=2)
        assert (codes[:, :used] == expect).all()


# ---------------------------------------------------------------- byte counts (P3 "Group-scaled ternary format",
#                                                                   "Two packings")

def _bits_per_weight(layout, n, k):
    return (n * oracle.row_bytes(layout, k) + n * (k // 128) * 2) * 8 / (n * k)


def test_slot2_costs_34_bytes_per_128_weights():
    for k in (128, 1024, 4096, 5120, 12288, 17408):
        assert oracle.row_bytes(oracle.SLOT2, k) / (k / 128) + 2 == 34
        assert _bits_per_weight(oracle.SLOT2, 7, k) == 2.125


def test_base3_density():
    b_eff = math.log2(3) + 16 / 128  # the information bound plus the fp16 scale (P3, b_eff equation)
    for k in (128, 1024, 4096, 5120, 12288, 17408):
        for layout in (oracle.SLOT2, oracle.BASE3):
            assert _bits_per_weight(layout, 3, k) >= b_eff
    # exactly 8/5 + 16/128 = 1.725 where ceil(K/5) is already a multiple of 16
    assert _bits_per_weight(oracle.BASE3, 1, 5120) == pytest.approx(1.725, abs=1e-15)
    assert oracle.row_bytes(oracle.BASE3, 4096) == 832
    assert oracle.row_bytes(oracle.BASE3, 12288) == 2464
    assert oracle.row_bytes(oracle.BASE3, 17408) == 3488


def test_single_gemv_256x1024_bytes():
    assert 256 * oracle.row_bytes(oracle.SLOT2, 1024) + 256 * 8 * 2 == 69632


def test_published_file_sizes_fit_34_bytes_per_group():
    # P3 "Points to note when reading": the two released files are 7,206,168,928 B (2-bit slots)
    # and 5,946,648,928 B (dense). With 34 B per 128-group for the slot layout and 28 B for a
    # dense layout of ceil(128/5) = 26 code bytes + 2 scale bytes, the difference must be a whole
    # number of groups times 6 B, and the implied weight count plus the 26,238,464 parameters kept
    # in high precision (P3 table in "The 0.0976% left in high precision") must match the 53.80 GB
    # FP16 size (P3 introduction) to within the rounding of that figure.
    diff = 7_206_168_928 - 5_946_648_928
    slot_bytes_per_group = oracle.row_bytes(oracle.SLOT2, 128) + 2
    assert slot_bytes_per_group == 34
    dense_bytes_per_group = math.ceil(128 / 5) + 2
    groups, rem = divmod(diff, slot_bytes_per_group - dense_bytes_per_group)
    assert rem == 0
    assert abs((groups * 128 + 26_238_464) * 2 / 53.80e9 - 1) < 1e-3


# ---------------------------------------------------------------- Hadamard and rotation (P3 "Block-wise Hadamard rotation")

def test_hadamard_is_sylvester():
    for n in (1, 2, 4, 8, 16, 32, 64, 128, 1024):
        h = oracle.hadamard(n).astype(np.int64)
        assert (h == scipy.linalg.hadamard(n)).all()
        assert (h @ h.T == n * np.eye(n, dtype=np.int64)).all()
        assert (h == h.T).all()
        if n >= 2:
            half = oracle.hadamard(n // 2).astype(np.int64)
            assert (h == np.block([[half, half], [half, -half]])).all()


def _dense_rotation(signs, block=128):
    k = signs.size
    h = scipy.linalg.hadamard(block).astype(np.float64) / math.sqrt(block)
    r = np.zeros((k, k))
    for b in range(k // block):
        sl = slice(b * block, (b + 1) * block)
        r[sl, sl] = h * signs[sl].astype(np.float64)[None, :]  # H S: sign on the input side
    return r


@pytest.mark.parametrize("block,k", [(128, 512), (1024, 2048)])
def test_rotation_matches_dense_block_matrix(block, k):
    sg = synth.signs(0, 1, k)
    x = synth.normal(0, 2, (3, k))
    got = oracle.rotate(x, sg, block)
    ref = x @ _dense_rotation(sg, block).T
    assert np.abs(got - ref).max() < 1e-12


@pytest.mark.parametrize("block,k", [(128, 256), (1024, 1024)])
def test_rotation_is_orthogonal(block, k):
    sg = synth.signs(5, 1, k)
    rcols = oracle.rotate(np.eye(k), sg, block)  # row i = R e_i = column i of R
    r = rcols.T
    assert np.abs(r.T @ r - np.eye(k)).max() < 1e-13
    x = synth.normal(1, 3, (4, k))
    assert np.allclose(np.linalg.norm(oracle.rotate(x, sg, block), axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


@pytest.mark.parametrize("block", [128, 1024])
def test_rotation_of_one_hot(block):
    k = block
    sg = synth.signs(7, 1, k)
    h = scipy.linalg.hadamard(block)
    for j in (0, 1, 77, block - 1):
        e = np.zeros(k)
        e[j] = 1.0
        assert np.allclose(oracle.rotate(e, sg, block), sg[j] * h[:, j] / math.sqrt(block), atol=1e-15)


def test_1024_block_is_the_kronecker_product_of_8_and_128():
    # natural-order Sylvester: H_1024 = H_8 (x) H_128, so one 1024-block rotation equals the
    # 128-block rotations of its 8 groups followed by an 8-point transform across the groups
    k = 2048
    sg = synth.signs(9, 2, k)
    x = synth.normal(9, 3, (2, k))
    small = oracle.rotate(x, sg, 128).reshape(2, k // 1024, 8, 128) * math.sqrt(128)
    h8 = scipy.linalg.hadamard(8).astype(np.float64)
    mixed = np.einsum("ij,rbjc->rbic", h8, small).reshape(2, k) / math.sqrt(1024)
    assert np.abs(mixed - oracle.rotate(x, sg, 1024)).max() < 1e-12
    assert np.abs(mixed - oracle.rotate(x, sg, 128)).max() > 1e-3  # and the two block sizes differ


def test_rotation_identities():
    # (W H)(H^T x) / 128 = W x  and  (W R^T)(R x) = W x, on dense fp64 W
    k = 256
    w = synth.normal(2, 1, (5, k))
    x = synth.normal(2, 2, (k,))
    h = np.kron(np.eye(k // 128), scipy.linalg.hadamard(128).astype(np.float64))
    assert np.allclose((w @ h) @ (h.T @ x) / 128, w @ x, atol=1e-12)
    sg = synth.signs(2, 3, k)
    rt = _dense_rotation(sg).T
    assert np.allclose((w @ rt) @ oracle.rotate(x, sg), w @ x, atol=1e-12)


# ---------------------------------------------------------------- binary bits (P2, "What ternary and binary are")

def _binary_row_with_prefix(prefix, k=128):
    t = -np.ones((1, k), dtype=np.int8)
    t[0, :len(prefix)] = prefix
    return t


def _signs(seed, stream, shape):
    """Seeded weights in {-1, +1} (the binary format has no zero)."""
    return synth.trits(seed, stream, shape, 0.0)


@pytest.mark.parametrize("bits,hexbyte", _read_fixture("binary_bytes.txt"))
def test_binary_hand_bytes(bits, hexbyte):
    codes = oracle.pack(oracle.BINARY, _binary_row_with_prefix(bits))
    assert codes.shape == (1, 16)
    assert codes[0, 0] == int(hexbyte, 16)
    assert (codes[0, 1:] == 0).all()  # -1 elsewhere: every bit clear


def test_binary_every_byte_round_trips():
    for b in range(256):
        codes = np.zeros((1, 16), dtype=np.uint8)
        codes[0, 0] = b
        t = oracle.unpack(oracle.BINARY, codes, 128)
        assert list(t[0, :8]) == [1 if (b >> i) & 1 else -1 for i in range(8)]
        assert (t[0, 8:] == -1).all()
        assert (oracle.pack(oracle.BINARY, t) == codes).all()


def test_binary_random_round_trip_and_position():
    t = _signs(0, 12, (5, 384))
    codes = oracle.pack(oracle.BINARY, t)
    assert codes.shape == (5, 48)
    assert (oracle.unpack(oracle.BINARY, codes, 384) == t).all()
    # element k lives in bit k%8 of byte k//8: numpy's little-endian bit unpacking
    bits = np.unpackbits(codes, axis=1, bitorder="little")
    assert (np.where(bits == 1, 1, -1) == t).all()


def test_binary_rejects_zero_and_out_of_range():
    for bad in (0, 2, -2):
        t = np.ones((1, 128), dtype=np.int8)
        t[0, 77] = bad
        with pytest.raises(oracle.OracleError):
            oracle.pack(oracle.BINARY, t)


def test_binary_costs_one_and_an_eighth_bits_per_weight():
    # P2 "What ternary and binary are": 1.125 bits per weight with the group scales
    for k in (128, 1024, 4096, 5120, 12288, 17408):
        total_bits = 8 * (oracle.row_bytes(oracle.BINARY, k) + 2 * (k // 128))
        assert total_bits / k == 1.125


@pytest.mark.parametrize("block", [None, 128, 1024])
def test_binary_product_equals_the_slot2_product_of_the_same_signs(block):
    # the same {-1, +1} weights stored in either layout define the same product, bit for bit
    k = 1024
    t = _signs(3, 4, (6, k))
    s = synth.scales_f16(3, 5, (6, k // 128))
    x16 = synth.x_f16(3, 6, (2, k))
    sg = synth.signs(3, 7, k) if block else None
    yb, bb = oracle.matmul(oracle.BINARY, oracle.pack(oracle.BINARY, t), s, k, x16.view(np.uint16), oracle.X_F16,
                           signs=sg, block=block or 128)
    ys, bs = oracle.matmul(oracle.SLOT2, oracle.pack(oracle.SLOT2, t), s, k, x16.view(np.uint16), oracle.X_F16,
                           signs=sg, block=block or 128)
    assert (yb == ys).all() and (bb == bs).all()


def test_binary_closed_forms():
    # all +1 gives s * sum x per group, all -1 gives -s * sum x; +1 on even positions and -1 on
    # odd ones gives s * (sum of even - sum of odd)
    k = 256
    x16 = synth.x_f16(0, 2, (k,))
    xs = x16.astype(np.float64)
    t = np.ones((3, k), dtype=np.int8)
    t[1] = -1
    t[2, 1::2] = -1
    s = np.array([[0.5, 3.0], [0.25, 2.0], [1.0, 4.0]], dtype=np.float16)
    y, _ = oracle.matmul(oracle.BINARY, oracle.pack(oracle.BINARY, t), s, k, x16.view(np.uint16), oracle.X_F16)
    assert y[0, 0] == pytest.approx(0.5 * xs[:128].sum() + 3.0 * xs[128:].sum(), rel=1e-15, abs=1e-15)
    assert y[0, 1] == pytest.approx(-0.25 * xs[:128].sum() - 2.0 * xs[128:].sum(), rel=1e-15, abs=1e-15)
    alt = xs[0::2] - xs[1::2]
    assert y[0, 2] == pytest.approx(alt[:64].sum() + 4.0 * alt[64:].sum(), rel=1e-14, abs=1e-14)


@pytest.mark.parametrize("k", [128, 384])
@pytest.mark.parametrize("m", [1, 3])
def test_binary_brute_force_tiny(k, m):
    n = 5
    t = _signs(k + m, 21, (n, k))
    s = synth.scales_f16(k + m, 22, (n, k // 128))
    x16 = synth.x_f16(k + m, 23, (m, k))
    y, bound = oracle.matmul(oracle.BINARY, oracle.pack(oracle.BINARY, t), s, k, x16.view(np.uint16), oracle.X_F16)
    terms = x16.astype(np.float64)[:, None, :] * _dense_weights(t, s)[None, :, :]
    assert np.allclose(y, terms.sum(axis=2), rtol=1e-13, atol=1e-16)
    assert np.allclose(bound, 1e-3 * np.abs(terms).sum(axis=2) + 1e-6, rtol=1e-13)


# ---------------------------------------------------------------- the product (P3 "Group-scaled ternary format")

def _dense_weights(trits, scales_f16):
    s = np.asarray(scales_f16, dtype=np.float16).astype(np.float64)
    return trits.astype(np.float64) * np.repeat(s, 128, axis=1)


@pytest.mark.parametrize("layout", [oracle.SLOT2, oracle.BASE3])
def test_closed_forms(layout):
    k = 256
    x16 = synth.x_f16(0, 1, (k,))
    xs = x16.astype(np.float64)
    t = np.zeros((4, k), dtype=np.int8)
    t[0, :128] = 1          # all +1 in group 0, zero in group 1
    t[1, 128:] = -1         # all -1 in group 1
    t[3, 200] = -1          # one-hot
    s = np.array([[0.5, 3.0], [0.25, 2.0], [1.0, 1.0], [7.0, 0.125]], dtype=np.float16)
    codes = oracle.pack(layout, t)
    y, bound = oracle.matmul(layout, codes, s, k, x16.view(np.uint16), oracle.X_F16)
    assert y[0, 0] == pytest.approx(0.5 * xs[:128].sum(), rel=1e-15, abs=1e-15)
    assert y[0, 1] == pytest.approx(-2.0 * xs[128:].sum(), rel=1e-15, abs=1e-15)
    assert y[0, 2] == 0.0
    assert y[0, 3] == -0.125 * xs[200]
    assert bound[0, 2] == 1e-6


@pytest.mark.parametrize("layout", [oracle.SLOT2, oracle.BASE3])
def test_integer_inputs_give_exact_integers(layout):
    k = 512
    t = synth.trits(4, 1, (6, k), 0.4)
    x = (synth.trits(4, 2, (2, k), 0.0).astype(np.int64) * 3 + synth.trits(4, 3, (2, k), 0.2)).astype(np.int64)
    expo = synth.trits(4, 4, (6, k // 128), 0.0).astype(np.int64)  # scales 2^-1 or 2^+1
    s = np.ldexp(1.0, expo).astype(np.float16)
    codes = oracle.pack(layout, t)
    y, _ = oracle.matmul(layout, codes, s, k, x.astype(np.float16).view(np.uint16), oracle.X_F16)
    ref = x.astype(np.float64) @ _dense_weights(t, s).T
    assert (y == ref).all()


@pytest.mark.parametrize("layout", [oracle.SLOT2, oracle.BASE3])
@pytest.mark.parametrize("k", [128, 256])
@pytest.mark.parametrize("m", [1, 3])
def test_brute_force_tiny(layout, k, m):
    n = 4
    t = synth.trits(k + m, layout, (n, k), 0.4)
    s = synth.scales_f16(k + m, 9, (n, k // 128))
    x16 = synth.x_f16(k + m, 10, (m, k))
    codes = oracle.pack(layout, t)
    y, bound = oracle.matmul(layout, codes, s, k, x16.view(np.uint16), oracle.X_F16)
    terms = x16.astype(np.float64)[:, None, :] * _dense_weights(t, s)[None, :, :]
    assert np.allclose(y, terms.sum(axis=2), rtol=1e-13, atol=1e-16)
    assert np.allclose(bound, 1e-3 * np.abs(terms).sum(axis=2) + 1e-6, rtol=1e-13)


def test_bf16_activations():
    k = 256
    t = synth.trits(1, 1, (3, k), 0.4)
    s = synth.scales_f16(1, 2, (3, 2))
    xb = synth.x_bf16_bits(1, 3, (2, k))
    xf = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    y, _ = oracle.matmul(oracle.SLOT2, oracle.pack(oracle.SLOT2, t), s, k, xb, oracle.X_BF16)
    assert np.allclose(y, xf @ _dense_weights(t, s).T, rtol=1e-13, atol=1e-16)


@pytest.mark.parametrize("layout", [oracle.SLOT2, oracle.BASE3])
@pytest.mark.parametrize("block,k", [(128, 256), (1024, 1024)])
def test_rotated_product_brute_force(layout, block, k):
    m = 2
    t = synth.trits(8, 1, (3, k), 0.5)
    s = synth.scales_f16(8, 2, (3, k // 128))
    x16 = synth.x_f16(8, 3, (m, k))
    sg = synth.signs(8, 4, k)
    y, bound = oracle.matmul(layout, oracle.pack(layout, t), s, k, x16.view(np.uint16), oracle.X_F16, signs=sg,
                             block=block)
    xr = x16.astype(np.float64) @ _dense_rotation(sg, block).T
    terms = xr[:, None, :] * _dense_weights(t, s)[None, :, :]
    assert np.allclose(y, terms.sum(axis=2), rtol=1e-12, atol=1e-15)
    assert np.allclose(bound, 1e-3 * np.abs(terms).sum(axis=2) + 1e-6, rtol=1e-12)


def test_rotated_hand_example():
    # sigma = +1 everywhere, x = e_0: R x = H[:, 0] / sqrt(128) = (1, ..., 1) / sqrt(128).
    # Row of all +1 codes at scale 1 gives 128 / sqrt(128) = sqrt(128); a row equal to any other
    # Hadamard row gives 0 (rows of H are orthogonal to the all-ones row 0).
    # sigma_3 = -1, x = e_3: R x = -H[:, 3] / sqrt(128); the row t = H[3] then gives -sqrt(128).
    k = 128
    h = scipy.linalg.hadamard(128).astype(np.int8)
    t = np.stack([np.ones(k, dtype=np.int8), h[5], h[3]])
    s = np.ones((3, 1), dtype=np.float16)
    sg = np.ones(k, dtype=np.int8)
    x = np.zeros((2, k), dtype=np.float16)
    x[0, 0] = 1
    x[1, 3] = 1
    sg[3] = -1
    y, _ = oracle.matmul(oracle.SLOT2, oracle.pack(oracle.SLOT2, t), s, k, x.view(np.uint16), oracle.X_F16, signs=sg)
    assert y[0, 0] == pytest.approx(math.sqrt(128), rel=1e-15)
    assert y[0, 1] == pytest.approx(0.0, abs=1e-15)
    assert y[1, 2] == pytest.approx(-math.sqrt(128), rel=1e-15)


def test_row_sampling_matches_full():
    k = 384
    t = synth.trits(2, 5, (50, k), 0.4)
    s = synth.scales_f16(2, 6, (50, 3))
    x16 = synth.x_f16(2, 7, (2, k))
    codes = oracle.pack(oracle.BASE3, t)
    full, _ = oracle.matmul(oracle.BASE3, codes, s, k, x16.view(np.uint16), oracle.X_F16)
    rows = np.array([49, 0, 17, 17, 3])
    part, _ = oracle.matmul(oracle.BASE3, codes, s, k, x16.view(np.uint16), oracle.X_F16, rows=rows)
    assert (part == full[:, rows]).all()


def test_golden_small_product():
    # tests/golden/small_product.txt: a K = 128 example worked by hand.
    path = os.path.join(GOLDEN, "small_product.txt")
    spec = {}
    with open(path) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if line:
                key, val = line.split("=")
                spec[key.strip()] = val.strip()
    k = 128
    x = np.array([int(v) for v in spec["x"].split()], dtype=np.float16)
    assert x.size == k
    rows = [r for r in spec if r.startswith("row")]
    t = np.zeros((len(rows), k), dtype=np.int8)
    s = np.zeros((len(rows), 1), dtype=np.float16)
    expect = np.zeros(len(rows))
    for i, name in enumerate(sorted(rows)):
        kind, scale, want = spec[name].split()
        if kind == "plus":
            t[i] = 1
        elif kind == "minus":
            t[i] = -1
        elif kind == "alternate":
            t[i, 0::2] = 1
            t[i, 1::2] = -1
        elif kind.startswith("onehot"):
            t[i, int(kind[len("onehot"):])] = -1
        s[i, 0] = float(scale)
        expect[i] = float(want)
    for layout in (oracle.SLOT2, oracle.BASE3):
        y, _ = oracle.matmul(layout, oracle.pack(layout, t), s, k, x.view(np.uint16), oracle.X_F16)
        assert (y[0] == expect).all()


# ---------------------------------------------------------------- RMSNorm (P3, "Running in the browser with WebGPU")
# The fused BlockHadamard + RMSNorm variant; norm weights gamma in bf16 (P3, "The 0.0976% kept at
# high precision"). Reading: xhat = gamma * x / sqrt(mean(x^2) + eps) per row.

def _bf16(values):
    return synth.bf16_bits(np.asarray(values, dtype=np.float64))


def _rmsnorm_cases():
    cases = []
    with open(os.path.join(GOLDEN, "rmsnorm_example.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, xs, eps, gs, outs = [part.strip() for part in line.split(";")]
            cases.append((name, [float(v) for v in xs.split()], float(eps), [float(v) for v in gs.split()],
                          [float(v) for v in outs.split()]))
    return cases


@pytest.mark.parametrize("name,x_prefix,eps,g_prefix,expect", _rmsnorm_cases())
def test_rmsnorm_hand_examples(name, x_prefix, eps, g_prefix, expect):
    k = 128
    if name == "A":
        x = np.zeros(k)
        gamma = np.ones(k)
    else:
        x = np.ones(k)
        gamma = np.where(np.arange(k) % 2 == 0, 1.0, -1.0)
    x[:len(x_prefix)] = x_prefix
    gamma[:len(g_prefix)] = g_prefix
    out = oracle.rmsnorm(x[None, :], _bf16(gamma), eps)[0]
    assert list(out[:len(expect)]) == expect
    if name == "A":
        assert (out[len(expect):] == 0).all()
    else:
        assert (np.abs(out) == 0.5).all()


def test_rmsnorm_gives_unit_root_mean_square():
    x = synth.normal(5, 1, (3, 1024)) * np.array([[0.01], [1.0], [300.0]])
    out = oracle.rmsnorm(x, _bf16(np.ones(1024)), 1e-300)
    assert np.allclose(np.sqrt((out ** 2).mean(axis=1)), 1.0, rtol=1e-14)


def test_rmsnorm_is_invariant_to_power_of_two_scaling():
    # gamma * (a x) / sqrt(mean((a x)^2) + a^2 eps) = gamma * x / sqrt(mean(x^2) + eps) exactly for a = 2^j
    x = synth.normal(5, 2, (2, 640))
    g = _bf16(synth.normal(5, 3, (640,)))
    base = oracle.rmsnorm(x, g, 1e-3)
    for j in (-3, 4):
        a = 2.0 ** j
        assert (oracle.rmsnorm(a * x, g, 1e-3 * a * a) == base).all()


def test_rmsnorm_applies_gamma_per_element_and_rows_independently():
    x = synth.normal(6, 1, (3, 384))
    gvals = synth.normal(6, 2, (384,))
    g = _bf16(gvals)
    g_exact = (g.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    out = oracle.rmsnorm(x, g, 1e-5)
    ones = oracle.rmsnorm(x, _bf16(np.ones(384)), 1e-5)
    assert np.allclose(out, ones * g_exact[None, :], rtol=1e-15, atol=0)
    for r in range(3):  # each row is normalised by its own root mean square
        assert (oracle.rmsnorm(x[r:r + 1], g, 1e-5)[0] == out[r]).all()


def test_rmsnorm_refuses_nonpositive_eps():
    with pytest.raises(oracle.OracleError):
        oracle.rmsnorm(np.ones((1, 128)), _bf16(np.ones(128)), 0.0)


@pytest.mark.parametrize("layout", [oracle.SLOT2, oracle.BASE3, oracle.BINARY])
@pytest.mark.parametrize("block", [None, 128, 1024])
def test_rmsnorm_product_brute_force(layout, block):
    k, n, m = 1024, 4, 2
    t = synth.trits(9, layout, (n, k), 0.0 if layout == oracle.BINARY else 0.4)
    s = synth.scales_f16(9, 2, (n, k // 128))
    x16 = (synth.x_f16(9, 3, (m, k)).astype(np.float32) * 20).astype(np.float16)
    gvals = synth.normal(9, 4, (k,))
    g = _bf16(gvals)
    sg = synth.signs(9, 5, k) if block else None
    eps = 1e-6
    y, bound = oracle.matmul(layout, oracle.pack(layout, t), s, k, x16.view(np.uint16), oracle.X_F16, signs=sg,
                             block=block or 128, gamma=g, eps=eps)
    xd = x16.astype(np.float64)
    g_exact = (g.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    xn = g_exact * xd / np.sqrt((xd ** 2).mean(axis=1, keepdims=True) + np.float64(np.float32(eps)))
    if block:
        xn = xn @ _dense_rotation(sg, block).T
    terms = xn[:, None, :] * _dense_weights(t, s)[None, :, :]
    assert np.allclose(y, terms.sum(axis=2), rtol=1e-12, atol=1e-13)
    assert np.allclose(bound, 1e-3 * np.abs(terms).sum(axis=2) + 1e-6, rtol=1e-12)
    # the standalone fused operation gives the same activation
    if block:
        fused = oracle.rmsnorm_rotate(x16.view(np.uint16), oracle.X_F16, g, eps, sg, block)
        assert np.allclose(fused, xn, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- code flips (P1, opening section)
# A code flip is a weight whose code changed between two checkpoints. The pins plant flips at
# positions the test chooses and compare with that known count, so a count of changed bytes or
# of changed words instead of changed trits, or a dropped position, fails.


def _flipped(t, rng, frac):
    """t with a random set of positions changed to another trit; returns (u, planted mask)."""
    mask = rng.random(t.shape) < frac
    step = rng.integers(1, 3, size=t.shape)  # +1 or +2 modulo 3: always a different trit
    u = t.copy()
    u[mask] = ((t[mask].astype(np.int64) + 1 + step[mask]) % 3 - 1).astype(np.int8)
    return u, mask


@pytest.mark.parametrize("layout", [oracle.SLOT2, oracle.BASE3])
@pytest.mark.parametrize("k", [128, 640, 4096])
def test_code_flips_count_the_planted_positions(layout, k):
    rng = np.random.default_rng(k + layout)
    n = 37
    t = synth.trits(11, k, (n, k), 0.4)
    u, mask = _flipped(t, rng, 0.03)
    a, b = oracle.pack(layout, t), oracle.pack(layout, u)
    total, rows = oracle.code_flips(layout, a, b, k)
    assert total == int(mask.sum())
    assert (rows == mask.sum(axis=1)).all()


@pytest.mark.parametrize("layout", [oracle.SLOT2, oracle.BASE3])
def test_code_flips_extremes_and_symmetry(layout):
    k, n = 384, 9
    t = synth.trits(12, 3, (n, k), 0.4)
    a = oracle.pack(layout, t)
    assert oracle.code_flips(layout, a, a, k)[0] == 0
    every = ((t.astype(np.int64) + 2) % 3 - 1).astype(np.int8)  # each trit moved to another value
    assert oracle.code_flips(layout, a, oracle.pack(layout, every), k)[0] == n * k
    rng = np.random.default_rng(5)
    u, _ = _flipped(t, rng, 0.1)
    v, _ = _flipped(u, rng, 0.1)
    b, c = oracle.pack(layout, u), oracle.pack(layout, v)
    ab, ba = oracle.code_flips(layout, a, b, k)[0], oracle.code_flips(layout, b, a, k)[0]
    assert ab == ba
    assert oracle.code_flips(layout, a, c, k)[0] <= ab + oracle.code_flips(layout, b, c, k)[0]


@pytest.mark.parametrize("k", [128, 1280])
def test_binary_code_flips_count_the_planted_sign_changes(k):
    n = 23
    t = _signs(14, k, (n, k))
    mask = np.random.default_rng(k).random((n, k)) < 0.05
    u = np.where(mask, -t, t).astype(np.int8)
    a, b = oracle.pack(oracle.BINARY, t), oracle.pack(oracle.BINARY, u)
    total, rows = oracle.code_flips(oracle.BINARY, a, b, k)
    assert total == int(mask.sum())
    assert (rows == mask.sum(axis=1)).all()
    assert oracle.code_flips(oracle.BINARY, a, a, k)[0] == 0
    assert oracle.code_flips(oracle.BINARY, a, oracle.pack(oracle.BINARY, -t), k)[0] == n * k
    # the same sign changes counted in the slot-2 layout give the same numbers
    s_total, s_rows = oracle.code_flips(oracle.SLOT2, oracle.pack(oracle.SLOT2, t), oracle.pack(oracle.SLOT2, u), k)
    assert s_total == total and (s_rows == rows).all()


def test_code_flips_do_not_depend_on_the_layout_or_the_row_padding():
    k, n = 1280, 21
    t = synth.trits(13, 4, (n, k), 0.5)
    u, mask = _flipped(t, np.random.default_rng(9), 0.02)
    counts = []
    for layout in (oracle.SLOT2, oracle.BASE3):
        a, b = oracle.pack(layout, t), oracle.pack(layout, u)
        # wider rows on one side, with bytes past the codes that differ from the other side
        wide = np.full((n, a.shape[1] + 48), 0xFF, dtype=np.uint8)
        wide[:, :a.shape[1]] = a
        counts.append(oracle.code_flips(layout, wide, b, k))
    assert counts[0][0] == counts[1][0] == int(mask.sum())
    assert (counts[0][1] == counts[1][1]).all()
