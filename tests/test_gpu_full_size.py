"""GPU parity at the benchmark workloads' full sizes, in the launches the benchmark times.

The oracle evaluates every output row, except for the prefill GEMM at 2048 activation rows, where
it takes 512 of them (first, last and a seeded sample in between); the tolerance is the oracle's
per-element bound, |y - y_ref| <= 1e-3 * sum_k |s t xr| + 1e-6.
Workloads (synthetic, seeded, the benchmark's shapes and value distributions):
  - 8B-class decode layer: q, k, v, o 4096 x 4096 / 1024 x 4096, gate and up 12288 x 4096, down
    4096 x 12288, M = 1, fp16 N(0, 1) activations, launched one layer at a time as q/k/v, o,
    gate/up, down; all three layouts (slot-2 with P(0) = 0.4, base-3 with P(0) = 0.5, binary
    with +1 and -1 equally likely).
  - 27B-class rotated-basis GEMV: base-3 gate 17408 x 5120 and down 5120 x 17408, M = 1 and 8,
    128- and 1024-element rotation blocks.
  - 27B-class prefill GEMM: slot-2 17408 x 5120 and 5120 x 17408, bf16 activations, M = 16, 128, 2048.
  - The RMSNorm prologue: q/k/v of the 8B layer in one batched call, and the 27B gate projection with
    1024-element rotation blocks at M = 8.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
import ternary_group_scaled_amd as tgs  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"
LNAME = {tgs.SLOT2: "slot2", tgs.BASE3: "base3", tgs.BINARY: "binary"}

LAYER_8B = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
            ("gate", 12288, 4096), ("up", 12288, 4096), ("down", 4096, 12288)]
GROUPS_8B = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]


def _sample_rows(n, count, seed):
    rows = np.sort(np.random.default_rng(seed).choice(n, size=min(count, n), replace=False))
    rows[0], rows[-1] = 0, n - 1
    return np.unique(rows)


def _matrix(layout, tag, n, k, p_zero, rotated=0):
    """The device matrix (packed by the library) and the oracle's own packing of the same trits,
    which must be identical; the oracle is only ever given its own bytes."""
    t = synth.trits(0, synth.stream_id(tag, "codes"), (n, k), p_zero)
    s = synth.scales_f16(0, synth.stream_id(tag, "scales"), (n, k // 128))
    codes, scales = tgs.pack_ternary(layout, t, s)
    ref_codes = oracle.pack(layout, t)
    assert np.array_equal(codes, ref_codes)
    w = tgs.PackedMatrix(layout, torch.from_numpy(codes).to(DEV), torch.from_numpy(scales.view(np.int16)).to(DEV),
                         k, rotated=rotated)
    return w, ref_codes, s


def _x_f16(tag, m, k):
    x = synth.x_f16(0, synth.stream_id(tag, "x"), (m, k))
    return torch.from_numpy(x.view(np.int16).copy()).to(DEV).view(torch.float16), x


def _check_rows(layout, codes, scales, k, x_bits, x_dtype, y, rows, what, signs=None, block=128):
    y_ref, bound = oracle.matmul(layout, codes, scales, k, x_bits, x_dtype, signs=signs, rows=rows, block=block)
    got = y[:, rows].astype(np.float64)
    err = np.abs(got - y_ref)
    bad = ~(err <= bound)
    assert not bad.any(), f"{what}: {bad.sum()} sampled outputs outside tolerance, max err/bound " \
                          f"{float(np.nanmax(err / bound)):.3g}"


@pytest.mark.parametrize("layout", [tgs.SLOT2, tgs.BASE3, tgs.BINARY], ids=LNAME.get)
def test_8b_layer_as_launched_by_the_benchmark(layout):
    p_zero = {tgs.SLOT2: 0.4, tgs.BASE3: 0.5, tgs.BINARY: 0.0}[layout]
    mats, host = {}, {}
    for name, n, k in LAYER_8B:
        w, codes, scales = _matrix(layout, f"full8b/{layout}/{name}", n, k, p_zero)
        mats[name] = w
        host[name] = (codes, scales, n, k)
    xs = {grp: _x_f16(f"full8b/{grp[0]}", 1, mats[grp[0]].k) for grp in GROUPS_8B}
    ys = {name: torch.empty((1, n), dtype=torch.float32, device=DEV) for name, n, _ in LAYER_8B}
    for grp in GROUPS_8B:  # one launch per group, as the benchmark's layer mode does
        tgs.ternary_gemv_batched([mats[nm] for nm in grp], [xs[grp][0]] * len(grp), [ys[nm] for nm in grp])
    torch.cuda.synchronize()
    got = {name: ys[name].cpu().numpy() for name in ys}
    for i, (name, n, k) in enumerate(LAYER_8B):
        codes, scales, _, _ = host[name]
        x_host = xs[[g for g in GROUPS_8B if name in g][0]][1]
        _check_rows(layout, codes, scales, k, x_host.view(np.uint16), oracle.X_F16, got[name],
                    np.arange(n), f"8B {LNAME[layout]} {name} {n}x{k}")
    # the whole layer in one batched call (the set mode's grouping) gives the same bits
    order = [nm for g in GROUPS_8B for nm in g]
    ys2 = {name: torch.empty_like(ys[name]) for name in ys}
    tgs.ternary_gemv_batched([mats[nm] for nm in order],
                             [xs[[g for g in GROUPS_8B if nm in g][0]][0] for nm in order], [ys2[nm] for nm in order])
    torch.cuda.synchronize()
    for name in ys:
        assert torch.equal(ys[name].view(torch.int32), ys2[name].view(torch.int32)), name


@pytest.mark.parametrize("block", [128, 1024])
@pytest.mark.parametrize("m", [1, 8])
def test_27b_rotated_gemv(block, m):
    shapes = [("gate", 17408, 5120), ("down", 5120, 17408)]
    for i, (name, n, k) in enumerate(shapes):
        w, codes, scales = _matrix(tgs.BASE3, f"full27r/{name}", n, k, 0.5, rotated=block)
        sg = synth.signs(0, synth.stream_id("full27r/signs", k), k)
        xd, xh = _x_f16(f"full27r/{name}/{m}", m, k)
        y = torch.empty((m, n), dtype=torch.float32, device=DEV)
        tgs.ternary_gemv_batched([w], [xd], [y], signs=[torch.from_numpy(sg).to(DEV)])
        torch.cuda.synchronize()
        _check_rows(tgs.BASE3, codes, scales, k, xh.view(np.uint16), oracle.X_F16, y.cpu().numpy(),
                    np.arange(n), f"27B rotated {name} m={m} block={block}", signs=sg, block=block)


def test_8b_attention_inputs_with_the_rmsnorm_prologue():
    """q, k, v of the 8B-class layer in one batched call with the RMSNorm prologue (slot-2, M = 1),
    and the 27B gate projection, base-3 with 1024-element rotation blocks, M = 8."""
    x, xh = _x_f16("full8bn/x", 1, 4096)
    x = (x.float() * 7.0).half()
    xh = (xh.astype(np.float32) * 7.0).astype(np.float16)
    gamma = synth.bf16_bits(1.0 + 0.25 * synth.normal(0, 77, (4096,)))
    gd = torch.from_numpy(gamma.view(np.int16).copy()).to(DEV)
    mats, ys = [], []
    for name, n, k in LAYER_8B[:3]:
        w, codes, scales = _matrix(tgs.SLOT2, f"full8bn/{name}", n, k, 0.4)
        mats.append((w, codes, scales, n))
        ys.append(torch.empty((1, n), dtype=torch.float32, device=DEV))
    tgs.ternary_gemv_rmsnorm_batched([w for w, _, _, _ in mats], [x] * 3, [gd] * 3, 1e-6, ys)
    torch.cuda.synchronize()
    for i, ((w, codes, scales, n), y) in enumerate(zip(mats, ys)):
        rows = np.arange(n)
        y_ref, bound = oracle.matmul(tgs.SLOT2, codes, scales, 4096, xh.view(np.uint16), oracle.X_F16, rows=rows,
                                     gamma=gamma, eps=float(np.float32(1e-6)))
        assert (np.abs(y.cpu().numpy()[:, rows] - y_ref) <= bound).all(), LAYER_8B[i][0]
    n, k, m = 17408, 5120, 8
    w, codes, scales = _matrix(tgs.BASE3, "full27n/gate", n, k, 0.5, rotated=1024)
    sg = synth.signs(0, synth.stream_id("full27n/signs", k), k)
    xd, xh = _x_f16("full27n/x", m, k)
    gamma = synth.bf16_bits(1.0 + 0.25 * synth.normal(0, 78, (k,)))
    y = tgs.ternary_gemv_rmsnorm(w, xd, torch.from_numpy(gamma.view(np.int16).copy()).to(DEV), 1e-6,
                                 signs=torch.from_numpy(sg).to(DEV))
    torch.cuda.synchronize()
    rows = np.arange(n)
    y_ref, bound = oracle.matmul(tgs.BASE3, codes, scales, k, xh.view(np.uint16), oracle.X_F16, signs=sg, block=1024,
                                 rows=rows, gamma=gamma, eps=float(np.float32(1e-6)))
    assert (np.abs(y.cpu().numpy()[:, rows] - y_ref) <= bound).all()


@pytest.mark.parametrize("m", [16, 32, 128, 2048])
def test_27b_prefill_gemm(m):
    shapes = [("gate", 17408, 5120), ("down", 5120, 17408)]
    for i, (name, n, k) in enumerate(shapes):
        w, codes, scales = _matrix(tgs.SLOT2, f"full27g/{name}", n, k, 0.4)
        xb = synth.x_bf16_bits(0, synth.stream_id(f"full27g/{name}/{m}", "x"), (m, k))
        xt = torch.from_numpy(xb.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
        y = tgs.ternary_gemm(w, xt)
        torch.cuda.synchronize()
        # every output column up to 128 rows (the oracle takes about 1.5 s per matrix there),
        # 512 sampled columns at 2048 rows
        rows = np.arange(n) if m <= 128 else _sample_rows(n, 512, 20 + i)
        _check_rows(tgs.SLOT2, codes, scales, k, xb, oracle.X_BF16, y.cpu().numpy(), rows, f"27B GEMM {name} m={m}")


@pytest.mark.parametrize("layout", [tgs.SLOT2, tgs.BINARY, tgs.BASE3], ids=LNAME.get)
@pytest.mark.parametrize("k", [65536, 65536 + 128, 32768, 32768 + 1024])
def test_gemv_at_the_single_token_kernel_limits(layout, k):
    """K at and just past the largest K of the single-token kernel (65536 plain, 32768 with the
    RMSNorm prologue): either kernel must give the oracle's rows, with and without the norm."""
    n = 96
    p_zero = {tgs.SLOT2: 0.4, tgs.BASE3: 0.5, tgs.BINARY: 0.0}[layout]
    w, codes, scales = _matrix(layout, f"limk/{layout}/{k}", n, k, p_zero)
    xd, xh = _x_f16(f"limk/{k}", 1, k)
    y = torch.empty((1, n), dtype=torch.float32, device=DEV)
    tgs.ternary_gemv_batched([w], [xd], [y])
    gamma = synth.bf16_bits(1.0 + 0.25 * synth.normal(1, k, (k,)))
    yn = tgs.ternary_gemv_rmsnorm(w, xd, torch.from_numpy(gamma.view(np.int16).copy()).to(DEV), 1e-6)
    torch.cuda.synchronize()
    rows = np.arange(n)
    _check_rows(layout, codes, scales, k, xh.view(np.uint16), oracle.X_F16, y.cpu().numpy(), rows, f"k={k}")
    y_ref, bound = oracle.matmul(layout, codes, scales, k, xh.view(np.uint16), oracle.X_F16, rows=rows,
                                 gamma=gamma, eps=float(np.float32(1e-6)))
    assert (np.abs(yn.cpu().numpy()[:, rows] - y_ref) <= bound).all(), f"rmsnorm k={k}"


@pytest.mark.parametrize("layout", [tgs.SLOT2, tgs.BINARY, tgs.BASE3], ids=LNAME.get)
def test_gemv_with_a_million_rows(layout):
    """n = 2^20 rows of K = 256: tens of thousands of workgroups, first and last rows included."""
    n, k = 1 << 20, 256
    p_zero = {tgs.SLOT2: 0.4, tgs.BASE3: 0.5, tgs.BINARY: 0.0}[layout]
    w, codes, scales = _matrix(layout, f"mrows/{layout}", n, k, p_zero)
    for m in (1, 8):
        xd, xh = _x_f16(f"mrows/{m}", m, k)
        y = torch.empty((m, n), dtype=torch.float32, device=DEV)
        tgs.ternary_gemv_batched([w], [xd], [y])
        torch.cuda.synchronize()
        _check_rows(layout, codes, scales, k, xh.view(np.uint16), oracle.X_F16, y.cpu().numpy(),
                    np.arange(n), f"{n}x{k} m={m}")
