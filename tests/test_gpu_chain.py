"""GPU parity of ternary_gemv_chain: single-token GEMV steps run in order by one launch.

Each step is checked on its own against the fp64 oracle: its input is rounded to fp16 on the host
exactly as the kernel rounds it (an fp32 input is the GPU's own output of an earlier step, read
back after the chain; nearest-even rounding on both sides), RMS-normalised by the oracle when the
step asks for it, and multiplied; every output must lie within the oracle's per-element bound
|y - y_ref| <= 1e-3 * sum_k |s t xh| + 1e-6. The chain must also be identical run to run, leave
the workspace's error word at zero, and count its steps in every workgroup's word.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
import ternary_group_scaled_amd as tgs  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _matrix(tag, n, k, p_zero=0.4):
    t = synth.trits(0, synth.stream_id("chain", tag, "codes"), (n, k), p_zero)
    s = synth.scales_f16(0, synth.stream_id("chain", tag, "scales"), (n, k // 128))
    w = tgs.PackedMatrix.from_trits(tgs.SLOT2, t, s, device=DEV)
    return w, oracle.pack(tgs.SLOT2, t), s


def _gamma(tag, k):
    g = synth.bf16_bits(1.0 + 0.25 * synth.normal(0, synth.stream_id("chain", tag, "gamma"), (k,)))
    return torch.from_numpy(g.view(np.int16).copy()).to(DEV), g


def _x16(tag, k):
    x = synth.x_f16(0, synth.stream_id("chain", tag, "x"), (1, k))
    return torch.from_numpy(x.view(np.int16).copy()).to(DEV).view(torch.float16)


def _check_step(i, step, host, sample=None):
    """The oracle's product of step i's fp16-rounded input; host[i] = [(codes, scales, gamma bits)]
    per matrix. sample: check this many evenly spaced rows of each matrix (and its first and last)
    instead of all of them."""
    x = step["x"].detach().float().cpu().numpy().reshape(1, -1).astype(np.float16)
    for j, (w, y) in enumerate(zip(step["ws"], step["ys"])):
        codes, s, gbits = host[i][j]
        rows = None
        if sample:
            rows = np.unique(np.r_[0, w.n - 1, np.linspace(0, w.n - 1, sample).astype(np.int64)])
        y_ref, bound = oracle.matmul(tgs.SLOT2, codes, s, w.k, x.view(np.uint16), oracle.X_F16, rows=rows,
                                     gamma=gbits, eps=step.get("eps", 0.0))
        got = y.cpu().numpy().astype(np.float64).reshape(1, -1)[:, :w.n]
        if rows is not None:
            got = got[:, rows]
        err = np.abs(got - y_ref)
        bad = ~(err <= bound)
        assert not bad.any(), (f"step {i} matrix {j} (n={w.n}, k={w.k}): {int(bad.sum())} outputs outside the "
                               f"bound, worst err/bound {float(np.nanmax(err / bound)):.3g}")


def _odd_chain():
    """Six steps over K = 512 .. 16384, one to three matrices per step, partial 16-row blocks,
    external fp16 inputs and fp32 outputs of earlier steps (whole buffers and slices), with and
    without the norm."""
    mats = {}
    for tag, n, k in (("A", 1536, 1024), ("B", 37, 1024), ("C", 64, 1024), ("D", 600, 1536), ("E", 2048, 512),
                      ("F", 333, 2048), ("G", 16, 2048), ("H", 16384, 512), ("I", 40, 16384)):
        mats[tag] = _matrix(tag, n, k)
    ys = {tag: torch.full((m[0].n,), float("nan"), dtype=torch.float32, device=DEV) for tag, m in mats.items()}
    g0, g0b = _gamma("g0", 1024)
    g2, g2b = _gamma("g2", 512)
    g5, g5b = _gamma("g5", 16384)
    plan = [(["A", "B", "C"], _x16("x0", 1024), (g0, g0b)),
            (["D"], ys["A"], None),
            (["E"], ys["D"][:512], (g2, g2b)),
            (["F", "G"], ys["E"], None),
            (["H"], _x16("x4", 512), None),
            (["I"], ys["H"], (g5, g5b))]
    steps, host = [], []
    for names, x, g in plan:
        st = {"ws": [mats[nm][0] for nm in names], "x": x, "ys": [ys[nm] for nm in names]}
        if g is not None:
            st["gamma"], st["eps"] = g[0], 1e-5
        steps.append(st)
        host.append([(mats[nm][1], mats[nm][2], g[1] if g is not None else None) for nm in names])
    return steps, host, ys


def test_chain_matches_oracle_step_by_step():
    steps, host, ys = _odd_chain()
    wsp = tgs.chain_workspace()
    tgs.ternary_gemv_chain(steps, wsp)
    torch.cuda.synchronize()
    words = wsp.cpu().numpy().view(np.uint32)
    assert words[-1] == 0, "a wait between steps gave up"
    assert (words[:-1] == len(steps)).all(), "every workgroup counts every step"
    for i, st in enumerate(steps):
        _check_step(i, st, host)
    first = {tag: y.cpu().numpy().copy() for tag, y in ys.items()}
    # again, on the same workspace: identical results, counts carried on
    tgs.ternary_gemv_chain(steps, wsp)
    torch.cuda.synchronize()
    words = wsp.cpu().numpy().view(np.uint32)
    assert words[-1] == 0 and (words[:-1] == 2 * len(steps)).all()
    for tag, y in ys.items():
        assert (y.cpu().numpy().view(np.uint32) == first[tag].view(np.uint32)).all(), f"{tag}: not deterministic"


def test_chain_of_one_step_and_of_sixteen():
    w, codes, s = _matrix("one", 300, 4096)
    y = torch.empty(300, dtype=torch.float32, device=DEV)
    x = _x16("one", 4096)
    wsp = tgs.chain_workspace()
    tgs.ternary_gemv_chain([{"ws": [w], "x": x, "ys": [y]}], wsp)
    torch.cuda.synchronize()
    _check_step(0, {"ws": [w], "x": x, "ys": [y]}, [[(codes, s, None)]])
    # sixteen steps, each reading the previous one's output (k = n = 1024)
    mats = [_matrix(f"s{i}", 1024, 1024) for i in range(16)]
    ys = [torch.empty(1024, dtype=torch.float32, device=DEV) for _ in range(16)]
    g, gb = _gamma("s", 1024)
    steps = [{"ws": [mats[i][0]], "x": _x16("s", 1024) if i == 0 else ys[i - 1], "ys": [ys[i]], "gamma": g,
              "eps": 1e-6} for i in range(16)]
    tgs.ternary_gemv_chain(steps, wsp)
    torch.cuda.synchronize()
    assert wsp.cpu().numpy().view(np.uint32)[-1] == 0
    for i, st in enumerate(steps):
        _check_step(i, st, [[(mats[j][1], mats[j][2], gb)] for j in range(16)])


LAYER_8B = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
            ("gate", 12288, 4096), ("up", 12288, 4096), ("down", 4096, 12288)]


def test_chain_8b_layers():
    """Two 8B-class layers in layer order, wired as the benchmark wires them: q/k/v read the
    normalised layer input, o reads q's output, gate/up the normalised output of o, down gate's
    output, and the next layer's q/k/v the normalised output of down. Outputs are checked on
    sampled rows of every matrix."""
    layers = 2
    mats, ys, host_m = {}, {}, {}
    for L in range(layers):
        for nm, n, k in LAYER_8B:
            w, c, s = _matrix(f"8b{L}{nm}", n, k)
            mats[L, nm], host_m[L, nm] = w, (c, s)
            ys[L, nm] = torch.empty(n, dtype=torch.float32, device=DEV)
    g_in, g_in_b = _gamma("gin", 4096)
    g_post, g_post_b = _gamma("gpost", 4096)
    steps, host = [], []
    for L in range(layers):
        x_in = _x16("8bx", 4096) if L == 0 else ys[L - 1, "down"]
        plan = [(("q", "k", "v"), x_in, (g_in, g_in_b)), (("o",), ys[L, "q"], None),
                (("gate", "up"), ys[L, "o"], (g_post, g_post_b)), (("down",), ys[L, "gate"], None)]
        for names, x, g in plan:
            st = {"ws": [mats[L, nm] for nm in names], "x": x, "ys": [ys[L, nm] for nm in names]}
            if g is not None:
                st["gamma"], st["eps"] = g[0], 1e-6
            steps.append(st)
            host.append([(host_m[L, nm][0], host_m[L, nm][1], g[1] if g is not None else None) for nm in names])
    wsp = tgs.chain_workspace()
    tgs.ternary_gemv_chain(steps, wsp)
    torch.cuda.synchronize()
    assert wsp.cpu().numpy().view(np.uint32)[-1] == 0
    for i, st in enumerate(steps):
        _check_step(i, st, host, sample=257)


def test_chain_refuses_bad_steps():
    w, _, _ = _matrix("bad", 64, 1024)
    y = torch.empty(64, dtype=torch.float32, device=DEV)
    wsp = tgs.chain_workspace()
    x = _x16("bad", 1024)
    for bad_w, code in ((_matrix("bad3", 64, 640)[0], "TGS_E_SHAPE"),):
        with pytest.raises(tgs.TgsError) as info:
            tgs.ternary_gemv_chain([{"ws": [bad_w], "x": _x16("b", 640), "ys": [y]}], wsp)
        assert info.value.name == code
    w3 = tgs.PackedMatrix.from_trits(tgs.BASE3, np.zeros((64, 1024), np.int8), np.ones((64, 8), np.float16),
                                     device=DEV)
    with pytest.raises(tgs.TgsError) as info:
        tgs.ternary_gemv_chain([{"ws": [w3], "x": x, "ys": [y]}], wsp)
    assert info.value.name == "TGS_E_LAYOUT"
    with pytest.raises(tgs.TgsError) as info:
        tgs.ternary_gemv_chain([{"ws": [w], "x": x, "ys": [y]}], wsp[:3])
    assert info.value.name == "TGS_E_SIZE"
    with pytest.raises(tgs.TgsError) as info:
        tgs.ternary_gemv_chain([{"ws": [w], "x": x, "ys": [y]}] * 17, wsp)
    assert info.value.name == "TGS_E_SHAPE"
