"""The rotation kernels' lane choreography, simulated on the CPU and checked against the oracle.

The GPU kernels split each Walsh-Hadamard block ("Ternary Bonsai 2 27B, 5.93GB ... (feat.
PrismML)", subsection "Block-wise Hadamard rotation") over the 64 lanes of a wave: butterfly
stages inside a lane, lane exchanges for the others, and for the stages across lanes 16 and 32
apart a lane-half swap that pairs two of a lane's own registers, which moves elements to new
(lane, register) places. These tests replay that data movement with numpy on integer inputs and
compare the result, put back in element order by the same index maps the kernels use, with the
oracle's dense rotation. They exercise the layout arithmetic, not the GPU code.
"""
import numpy as np

import oracle

LANES = np.arange(64)


def _swap_rows16(a, b):
    """a's odd 16-lane rows <-> b's even rows (v_permlane16_swap)."""
    odd = (LANES & 16) != 0
    na, nb = a.copy(), b.copy()
    na[odd] = b[LANES[odd] - 16]
    nb[~odd] = a[LANES[~odd] + 16]
    return na, nb


def _swap_halves32(a, b):
    """a's lanes 32..63 <-> b's lanes 0..31 (v_permlane32_swap)."""
    up = LANES >= 32
    na, nb = a.copy(), b.copy()
    na[up] = b[LANES[up] - 32]
    nb[~up] = a[LANES[~up] + 32]
    return na, nb


def _cross(v, stride):
    """Butterfly across lanes `stride` apart: the lower lane keeps own + partner, the upper
    partner - own."""
    sgn = np.where(LANES & stride, -1.0, 1.0)
    return [r * sgn + r[LANES ^ stride] for r in v]


def _inputs(seed, n):
    rng = np.random.default_rng(seed)
    x = rng.integers(-9, 10, n).astype(np.float64)
    signs = np.where(rng.random(n) < 0.5, -1, 1).astype(np.int8)
    return x, signs


def test_one_token_group_rotation_with_paired_lane_half_stages():
    """128-element group, one token: lane p holds elements 2p and 2p + 1; the stages across lanes
    16 and 32 apart pair the lane's two registers. Element of (lane p, register r) afterwards:
    bit 0 = lane bit 4, bits 1..4 = lane bits 0..3, bit 5 = lane bit 5, bit 6 = r."""
    x, signs = _inputs(1, 128)
    xs = x * signs
    v = [xs[0::2].copy(), xs[1::2].copy()]
    v = [v[0] + v[1], v[0] - v[1]]  # in-lane stage
    for s in (1, 2, 4, 8):
        v = _cross(v, s)
    a, b = _swap_rows16(v[0], v[1])
    v = [a + b, a - b]
    a, b = _swap_halves32(v[0], v[1])
    v = [a + b, a - b]

    def element(p, r):
        return ((p >> 4) & 1) | ((p & 15) << 1) | (((p >> 5) & 1) << 5) | (r << 6)

    places = {element(p, r) for p in range(64) for r in range(2)}
    assert places == set(range(128))
    out = np.empty(128)
    for p in range(64):
        for r in range(2):
            out[element(p, r)] = v[r][p]
    ref = oracle.rotate(x[None, :], signs, 128)[0] * np.sqrt(128)
    assert np.abs(out - ref).max() < 1e-9


def test_block_rotation_1024_with_paired_lane_half_stages():
    """1024-element block: lane l holds elements 16 l .. 16 l + 15; registers i, i + 8 pair across
    lanes 16 apart, then i, i + 4 across lanes 32 apart. Element of (lane l, register i)
    afterwards: bits 0, 1 = i bits 0, 1; bit 2 = lane bit 5; bit 3 = lane bit 4; bits 4..7 = lane
    bits 0..3; bit 8 = i bit 3; bit 9 = i bit 2."""
    x, signs = _inputs(3, 1024)
    xs = x * signs
    v = [xs[16 * LANES + i].copy() for i in range(16)]
    for h in (1, 2, 4, 8):
        for i in range(16):
            if i & h == 0:
                a, b = v[i].copy(), v[i + h].copy()
                v[i], v[i + h] = a + b, a - b
    for s in (1, 2, 4, 8):
        v = _cross(v, s)
    for i in range(8):
        a, b = _swap_rows16(v[i], v[i + 8])
        v[i], v[i + 8] = a + b, a - b
    for i in (0, 1, 2, 3, 8, 9, 10, 11):
        a, b = _swap_halves32(v[i], v[i + 4])
        v[i], v[i + 4] = a + b, a - b
    out = np.empty(1024)
    seen = set()
    for lane in range(64):
        e0 = (((lane >> 5) & 1) << 2) | (((lane >> 4) & 1) << 3) | ((lane & 15) << 4)
        for q in range(4):  # the four 4-element runs a lane stores
            base = e0 + 512 * (q & 1) + 256 * (q >> 1)
            for j in range(4):
                out[base + j] = v[4 * q + j][lane]
                seen.add(base + j)
    assert seen == set(range(1024))
    ref = oracle.rotate(x[None, :], signs, 1024)[0] * 32
    assert np.abs(out - ref).max() < 1e-9


def test_standalone_rotation_tiles():
    """Standalone rotation: a wave takes 512 consecutive elements of the flattened rows (four
    128-blocks, or half of a 1024-block), lane l holding elements 8 l .. 8 l + 7 of each half;
    strides 1, 2, 4 run in the lane, 8 .. 256 across lanes, 512 between a lane's two halves.
    Tiles may span rows."""
    for block, m, k in ((128, 3, 384), (128, 5, 128), (1024, 2, 2048)):
        x, _ = _inputs(block + k, m * k)
        _, signs = _inputs(block + k + 1, k)
        x = x.reshape(m, k)
        flat = (x * signs[None, :]).ravel()
        halves = 2 if block == 1024 else 1
        out = np.empty_like(flat)
        for t0 in range(0, flat.size, 512 * halves):
            v = np.zeros((64, 8 * halves))
            for lane in range(64):
                for h in range(halves):
                    e = t0 + 512 * h + 8 * lane
                    if e < flat.size:
                        v[lane, 8 * h:8 * h + 8] = flat[e:e + 8]
            for hh in (1, 2, 4):
                for i in range(8 * halves):
                    if i & hh == 0:
                        a, b = v[:, i].copy(), v[:, i + hh].copy()
                        v[:, i], v[:, i + hh] = a + b, a - b
            strides = (1, 2, 4, 8, 16, 32) if block == 1024 else (1, 2, 4, 8)
            for s in strides:
                sgn = np.where(LANES & s, -1.0, 1.0)[:, None]
                v = v * sgn + v[LANES ^ s]
            if block == 1024:
                a, b = v[:, :8].copy(), v[:, 8:].copy()
                v[:, :8], v[:, 8:] = a + b, a - b
            for lane in range(64):
                for h in range(halves):
                    e = t0 + 512 * h + 8 * lane
                    if e < flat.size:
                        out[e:e + 8] = v[lane, 8 * h:8 * h + 8]
        ref = oracle.rotate(x, signs, block) * np.sqrt(block)
        assert np.abs(out.reshape(m, k) - ref).max() < 1e-9, (block, m, k)
