"""GPU parity at the edges of the number format, every kernel path against the fp64 oracle.

The format is w = s_g * t with one fp16 scale per 128 weights ("Ternary Bonsai 2 27B, 5.93GB ...
(feat. PrismML)", section "Group-scaled ternary format"); the pages put no limit on the scale's
value, so any fp16 scale is accepted, subnormals are not flushed and NaN / Inf propagate.

- One-hot rows: a row with a single nonzero code gives s * t * x_k exactly (an fp16 x fp16 product
  needs 22 significant bits, an fp16 x bf16 product 19, so the fp32 result is exact), whatever the
  row's other activations hold. The activation at the hot position is small (1e-3 or 1e-4) among
  N(0, 9) neighbours, and the scale is 1 or the largest fp16 value 65504: a kernel that formed
  sum t x as a difference of two rounded sums over all weights would miss by about ulp(sum |x|).
- Two-hot rows (two nonzero codes, in the same or different groups): within the bound, which for
  such rows is about 1e-3 of |s x| at the two positions.
- Subnormal fp16 scales with activations near 1e3, and subnormal fp16 activations with scales
  near 1e3: the products are far above the bound's 1e-6 floor, so a flush to zero fails.
- Infinite and NaN scales: an output is non-finite exactly where the oracle's is. (The oracle
  forms each weight s * t before summing, so a zero code under an infinite scale gives NaN there;
  the kernels scale each group's partial sum, which gives +-Inf or NaN. Which non-finite value
  results is not compared.) Outputs of rows with finite scales stay within the bound.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import oracle_product

torch = pytest.importorskip("torch")
import ternary_group_scaled_amd as tgs  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"

# GEMV kernel paths: (layout, m, rotation block). slot-2 m = 1 plain is the single-token kernel;
# m = 2 and 8 (and rotated) the general slot-2/binary kernel; every base-3 case the matrix-core kernel.
GEMV_PATHS = [(tgs.SLOT2, 1, 0), (tgs.SLOT2, 2, 0), (tgs.SLOT2, 8, 0), (tgs.BASE3, 1, 0), (tgs.BASE3, 8, 0)]
GEMV_PATHS_ALL = GEMV_PATHS + [(tgs.SLOT2, 1, 128), (tgs.BASE3, 1, 128), (tgs.BASE3, 8, 128),
                               (tgs.BASE3, 8, 1024), (tgs.BINARY, 1, 0), (tgs.BINARY, 8, 0)]
LNAME = {tgs.SLOT2: "slot2", tgs.BASE3: "base3", tgs.BINARY: "binary"}


def _pid(p):
    return f"{LNAME[p[0]]}-m{p[1]}-rot{p[2]}"


def _x_dev(bits, dtype):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).to(DEV).view(dtype)


def _run_gemv(layout, t, s, x16, block=0, signs=None):
    w = tgs.PackedMatrix.from_trits(layout, t, s, device=DEV, rotated=block)
    sg = torch.from_numpy(signs).to(DEV) if block else None
    y = tgs.ternary_gemv(w, _x_dev(x16, torch.float16), signs=sg)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _run_gemm(layout, t, s, xb_bits):
    w = tgs.PackedMatrix.from_trits(layout, t, s, device=DEV)
    y = tgs.ternary_gemm(w, _x_dev(xb_bits, torch.bfloat16))
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _check_bound(y, y_ref, bound, what):
    err = np.abs(y.astype(np.float64) - y_ref)
    bad = ~(err <= bound)
    assert not bad.any(), (f"{what}: {int(bad.sum())} outside the bound; worst err/bound "
                           f"{float(np.nanmax(err / bound)):.3g}")


# ------------------------------------------------------------------------------ one-hot / two-hot rows

def _hot_case(seed, n, k, m):
    """Codes, scales and activations (doubles, before rounding) with one-hot rows (0 .. n/4), two-hot
    rows (n/4 .. n/2) and dense rows (the rest). Returns (t, s16, x, hot) with hot[r] = (position,
    code) of the one-hot rows."""
    rs = np.random.default_rng(seed)
    t = synth.trits(seed, synth.stream_id("hot", n, k, "codes"), (n, k), 0.4)
    s16 = synth.scales_f16(seed, synth.stream_id("hot", n, k, "scales"), (n, k // 128))
    x = 3.0 * synth.normal(seed, synth.stream_id("hot", n, k, m, "x"), (m, k))
    hot = {}
    n1, n2 = n // 4, n // 2
    # positions: first / last of a group, the last of the row, and random ones
    fixed = [0, 127, 128, 255, k - 1, k - 128, 64, 63]
    for r in range(n2):
        p = fixed[r % len(fixed)] if r < len(fixed) else int(rs.integers(0, k))
        code = 1 if r % 2 == 0 else -1
        t[r] = 0
        t[r, p] = code
        big = (r // 2) % 2 == 1
        s16[r, p // 128] = np.float16(65504.0 if big else 1.0)
        small = 1e-3 if r % 3 else 1e-4
        x[:, p] = small * np.where(np.arange(m) % 2 == 0, 1.0, -1.0)
        if r < n1:
            hot[r] = (p, code)
        else:
            q = int(rs.integers(0, k))
            t[r, q] = -code
            s16[r, q // 128] = np.float16(65504.0 if big else 1.0)
            x[:, q] = 2e-4
    return t, s16, x, hot


def _assert_one_hot_exact(y, s16, xv, hot, what):
    for r, (p, code) in hot.items():
        want = (np.float64(s16[r, p // 128]) * code * xv[:, p].astype(np.float64)).astype(np.float32)
        got = y[:, r].astype(np.float32)
        assert (got.view(np.uint32) == want.view(np.uint32)).all(), \
            f"{what}: one-hot row {r} (position {p}): got {got[:2]}, want s*t*x = {want[:2]}"


@pytest.mark.parametrize("path", GEMV_PATHS, ids=_pid)
@pytest.mark.parametrize("k", [1024, 4096, 12288])
def test_one_hot_rows_exact_gemv(path, k):
    layout, m, _ = path
    n = 96
    t, s16, x, hot = _hot_case(7, n, k, m)
    x16 = x.astype(np.float16)
    y = _run_gemv(layout, t, s16, x16)
    y_ref, bound = oracle_product(layout, t, s16, x16.view(np.uint16), oracle.X_F16)
    _check_bound(y, y_ref, bound, f"{_pid(path)} k={k}")
    _assert_one_hot_exact(y, s16, x16, hot, f"{_pid(path)} k={k}")


@pytest.mark.parametrize("m", [16, 128])
@pytest.mark.parametrize("k", [1024, 5120])
def test_one_hot_rows_exact_gemm(m, k):
    n = 96
    t, s16, x, hot = _hot_case(11, n, k, m)
    xb = synth.bf16_bits(x)
    y = _run_gemm(tgs.SLOT2, t, s16, xb)
    y_ref, bound = oracle_product(tgs.SLOT2, t, s16, xb, oracle.X_BF16)
    _check_bound(y, y_ref, bound, f"gemm m={m} k={k}")
    xv = (xb.astype(np.uint32) << 16).view(np.float32)
    _assert_one_hot_exact(y, s16, xv, hot, f"gemm m={m} k={k}")


# ------------------------------------------------------------------------------ subnormals

def _subnormal_f16(seed, stream, shape, negative=True):
    """fp16 subnormals: random nonzero mantissas with a zero exponent field (and random signs)."""
    u = synth.normal(seed, stream, shape)
    mant = (np.floor(np.abs(u) * 300.0).astype(np.int64) % 1023 + 1).astype(np.uint16)
    sign = (u < 0).astype(np.uint16) << 15 if negative else np.zeros(shape, np.uint16)
    return (mant | sign).view(np.float16)


def _near(seed, stream, shape, value):
    return (value * (1.0 + 0.25 * synth.normal(seed, stream, shape))).astype(np.float16)


@pytest.mark.parametrize("path", GEMV_PATHS_ALL, ids=_pid)
def test_subnormal_scales_gemv(path):
    layout, m, block = path
    n, k = 80, 4096
    p0 = 0.0 if layout == tgs.BINARY else 0.4
    t = synth.trits(1, synth.stream_id("subs", layout, "codes"), (n, k), p0)
    s16 = _subnormal_f16(1, synth.stream_id("subs", "s"), (n, k // 128), negative=False)
    x16 = _near(1, synth.stream_id("subs", m, "x"), (m, k), 1000.0) * np.where(
        synth.normal(1, 5, (m, k)) < 0, -1, 1).astype(np.float16)
    sg = synth.signs(1, 9, k) if block else None
    y = _run_gemv(layout, t, s16, x16, block, sg)
    y_ref, bound = oracle_product(layout, t, s16, x16.view(np.uint16), oracle.X_F16, signs=sg, block=block or 128)
    assert (bound > 1e-5).all()  # the relative part dominates: a flushed scale would fail
    _check_bound(y, y_ref, bound, f"subnormal scales {_pid(path)}")


@pytest.mark.parametrize("path", GEMV_PATHS_ALL, ids=_pid)
def test_subnormal_activations_gemv(path):
    layout, m, block = path
    n, k = 80, 4096
    p0 = 0.0 if layout == tgs.BINARY else 0.4
    t = synth.trits(2, synth.stream_id("subx", layout, "codes"), (n, k), p0)
    s16 = _near(2, synth.stream_id("subx", "s"), (n, k // 128), 1000.0)
    x16 = _subnormal_f16(2, synth.stream_id("subx", m, "x"), (m, k))
    sg = synth.signs(2, 9, k) if block else None
    y = _run_gemv(layout, t, s16, x16, block, sg)
    y_ref, bound = oracle_product(layout, t, s16, x16.view(np.uint16), oracle.X_F16, signs=sg, block=block or 128)
    assert (bound > 1e-5).all()
    _check_bound(y, y_ref, bound, f"subnormal activations {_pid(path)}")


@pytest.mark.parametrize("layout", [tgs.SLOT2, tgs.BINARY], ids=LNAME.get)
@pytest.mark.parametrize("m", [16, 128])
def test_subnormal_scales_gemm(layout, m):
    """(bf16 subnormal activations lie below 1.2e-38, so their products with any fp16 scale sit far
    under the bound's 1e-6 floor and would test nothing; the scales are the subnormal operand here.)"""
    n, k = 80, 5120
    p0 = 0.0 if layout == tgs.BINARY else 0.4
    t = synth.trits(3, synth.stream_id("subg", layout, "codes"), (n, k), p0)
    s16 = _subnormal_f16(3, synth.stream_id("subg", "s"), (n, k // 128), negative=False)
    xb = synth.bf16_bits(1000.0 * synth.normal(3, synth.stream_id("subg", m, "x"), (m, k)))
    y = _run_gemm(layout, t, s16, xb)
    y_ref, bound = oracle_product(layout, t, s16, xb, oracle.X_BF16)
    assert (bound > 1e-5).all()
    _check_bound(y, y_ref, bound, f"gemm subnormal scales {LNAME[layout]} m={m}")


# ------------------------------------------------------------------------------ Inf / NaN scales

def _special_scales(seed, n, k):
    s16 = synth.scales_f16(seed, synth.stream_id("inf", n, k), (n, k // 128))
    special = np.zeros(n, dtype=bool)
    for r, v in ((3, np.inf), (10, -np.inf), (17, np.nan), (30, np.inf), (45, np.nan)):
        if r < n:
            s16[r, (r * 7) % (k // 128)] = np.float16(v)
            special[r] = True
    return s16, special


def _check_nonfinite(y, y_ref, bound, special, what):
    fin_ref = np.isfinite(y_ref)
    assert (np.isfinite(y) == fin_ref).all(), f"{what}: finiteness differs from the oracle's"
    assert not fin_ref[:, special].any(), f"{what}: the oracle left a row with a non-finite scale finite"
    ok = fin_ref
    err = np.abs(y.astype(np.float64) - y_ref)
    assert (err[ok] <= bound[ok]).all(), f"{what}: finite outputs outside the bound"


@pytest.mark.parametrize("path", GEMV_PATHS_ALL, ids=_pid)
def test_inf_nan_scales_gemv(path):
    layout, m, block = path
    n, k = 64, 2048
    p0 = 0.0 if layout == tgs.BINARY else 0.4
    t = synth.trits(4, synth.stream_id("inf", layout, "codes"), (n, k), p0)
    s16, special = _special_scales(4, n, k)
    x16 = synth.x_f16(4, synth.stream_id("inf", m, "x"), (m, k))
    sg = synth.signs(4, 9, k) if block else None
    y = _run_gemv(layout, t, s16, x16, block, sg)
    with np.errstate(invalid="ignore"):
        y_ref, bound = oracle_product(layout, t, s16, x16.view(np.uint16), oracle.X_F16, signs=sg,
                                      block=block or 128)
        _check_nonfinite(y, y_ref, bound, special, f"inf/nan scales {_pid(path)}")


@pytest.mark.parametrize("layout", [tgs.SLOT2, tgs.BINARY], ids=LNAME.get)
@pytest.mark.parametrize("m", [16, 128])
def test_inf_nan_scales_gemm(layout, m):
    n, k = 64, 2048
    p0 = 0.0 if layout == tgs.BINARY else 0.4
    t = synth.trits(5, synth.stream_id("infg", layout, "codes"), (n, k), p0)
    s16, special = _special_scales(5, n, k)
    xb = synth.x_bf16_bits(5, synth.stream_id("infg", m, "x"), (m, k))
    y = _run_gemm(layout, t, s16, xb)
    with np.errstate(invalid="ignore"):
        y_ref, bound = oracle_product(layout, t, s16, xb, oracle.X_BF16)
        _check_nonfinite(y, y_ref, bound, special, f"gemm inf/nan scales {LNAME[layout]} m={m}")
