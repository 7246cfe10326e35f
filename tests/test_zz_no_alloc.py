"""ternary_gemv_chain_static (the chain on the library's own workspace, allocating nothing) against
ternary_gemv_chain on a caller's workspace: two calls in a row, the second smaller, each identical
bit for bit to the workspace entry point on the same steps, with the error word at zero, and each
step's outputs within the oracle's bound |y - y_ref| <= 1e-3 * sum_k |s t xh| + 1e-6.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
import ternary_group_scaled_amd as tgs  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _matrix(tag, n, k):
    t = synth.trits(0, synth.stream_id("noalloc", tag, "codes"), (n, k), 0.4)
    s = synth.scales_f16(0, synth.stream_id("noalloc", tag, "scales"), (n, k // 128))
    return tgs.PackedMatrix.from_trits(tgs.SLOT2, t, s, device=DEV), oracle.pack(tgs.SLOT2, t), s


def _x16(tag, k):
    x = synth.x_f16(0, synth.stream_id("noalloc", tag, "x"), (1, k))
    return torch.from_numpy(x.view(np.int16).copy()).to(DEV).view(torch.float16)


def _chain(tag, shapes, norm_steps):
    """Steps over shapes [(n, k) per matrix of a step]; step s > 0 reads step s - 1's first output
    when its k matches, else an external input. Returns (steps for the workspace call, steps for
    the static call with their own outputs, host copies per step)."""
    g_bits = synth.bf16_bits(1.0 + 0.25 * synth.normal(0, synth.stream_id("noalloc", tag, "gamma"), (16384,)))
    steps_a, steps_b, host = [], [], []
    prev = None
    for s, mats in enumerate(shapes):
        k = mats[0][1]
        built = [_matrix(f"{tag}{s}{j}", n, k) for j, (n, _) in enumerate(mats)]
        ya = [torch.full((n,), float("nan"), dtype=torch.float32, device=DEV) for n, _ in mats]
        yb = [torch.full((n,), float("nan"), dtype=torch.float32, device=DEV) for n, _ in mats]
        xa = xb = _x16(f"{tag}{s}", k)
        if prev is not None and prev[0][0].numel() >= k:
            xa, xb = prev[0][0][:k], prev[1][0][:k]
        sa = {"ws": [b[0] for b in built], "x": xa, "ys": ya}
        sb = {"ws": [b[0] for b in built], "x": xb, "ys": yb}
        gb = None
        if s in norm_steps:
            gb = g_bits[:k].copy()
            gt = torch.from_numpy(gb.view(np.int16).copy()).to(DEV)
            for st in (sa, sb):
                st["gamma"], st["eps"] = gt, 1e-5
        steps_a.append(sa)
        steps_b.append(sb)
        host.append([(b[1], b[2], gb) for b in built])
        prev = (ya, yb)
    return steps_a, steps_b, host


def _check_oracle(i, step, host):
    x = step["x"].detach().float().cpu().numpy().reshape(1, -1).astype(np.float16)
    for j, (w, y) in enumerate(zip(step["ws"], step["ys"])):
        codes, s, gbits = host[i][j]
        rows = np.unique(np.r_[0, w.n - 1, np.linspace(0, w.n - 1, 97).astype(np.int64)])
        y_ref, bound = oracle.matmul(tgs.SLOT2, codes, s, w.k, x.view(np.uint16), oracle.X_F16, rows=rows,
                                     gamma=gbits, eps=step.get("eps", 0.0))
        got = y.cpu().numpy().astype(np.float64).reshape(1, -1)[:, rows]
        assert (np.abs(got - y_ref) <= bound).all(), f"step {i} matrix {j}: outside the oracle's bound"


def _run_and_compare(tag, shapes, norm_steps, wsp, err):
    steps_a, steps_b, host = _chain(tag, shapes, norm_steps)
    print(f"[no-alloc] {tag}: {len(shapes)} steps", flush=True)
    tgs.ternary_gemv_chain(steps_a, wsp)
    err.fill_(-1)
    tgs.ternary_gemv_chain_static(steps_b, error=err)
    torch.cuda.synchronize()
    assert wsp.cpu().numpy().view(np.uint32)[-1] == 0
    assert int(err.cpu()[0]) == 0, "a wait between steps gave up"
    for i, (sa, sb) in enumerate(zip(steps_a, steps_b)):
        for j, (ya, yb) in enumerate(zip(sa["ys"], sb["ys"])):
            a = ya.cpu().numpy().view(np.uint32)
            b = yb.cpu().numpy().view(np.uint32)
            assert (a == b).all(), f"{tag} step {i} matrix {j}: {int((a != b).sum())} outputs differ"
        _check_oracle(i, sb, host)


def test_static_chain_matches_workspace_chain_twice():
    wsp = tgs.chain_workspace()
    err = torch.empty(1, dtype=torch.int32, device=DEV)
    big = [[(4096, 4096), (1024, 4096), (1024, 4096)], [(4096, 4096)], [(12288, 4096), (333, 4096)],
           [(4096, 12288)], [(2048, 4096)], [(600, 1536)]]
    _run_and_compare("big", big, {0, 2}, wsp, err)
    small = [[(256, 1024)], [(40, 1024), (17, 1024)]]
    _run_and_compare("small", small, {1}, wsp, err)


def test_static_chain_refuses_what_the_workspace_chain_refuses():
    w, _, _ = _matrix("bad", 64, 640)
    y = torch.empty(64, dtype=torch.float32, device=DEV)
    with pytest.raises(tgs.TgsError) as info:
        tgs.ternary_gemv_chain_static([{"ws": [w], "x": _x16("bad", 640), "ys": [y]}])
    assert info.value.name == "TGS_E_SHAPE"
    w2, _, _ = _matrix("ok", 64, 1024)
    with pytest.raises(tgs.TgsError) as info:
        tgs.ternary_gemv_chain_static([{"ws": [w2], "x": _x16("ok", 1024), "ys": [y]}] * 17)
    assert info.value.name == "TGS_E_SHAPE"
