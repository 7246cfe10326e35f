"""Helpers for GPU parity tests: seeded inputs -> library on the GPU and oracle on the CPU."""
from __future__ import annotations

import numpy as np

import oracle
import synth


def make_weights(seed, stream, n, k, p_zero):
    t = synth.trits(seed, synth.stream_id(stream, "codes"), (n, k), p_zero)
    s = synth.scales_f16(seed, synth.stream_id(stream, "scales"), (n, k // 128))
    return t, s


def make_x_f16(seed, stream, m, k):
    return synth.x_f16(seed, synth.stream_id(stream, "x"), (m, k))


def make_x_bf16_bits(seed, stream, m, k):
    return synth.x_bf16_bits(seed, synth.stream_id(stream, "x"), (m, k))


def make_signs(seed, stream, k):
    return synth.signs(seed, synth.stream_id(stream, "signs"), k)


def oracle_product(layout, trits, scales, x_bits, x_dtype, signs=None, rows=None, block=128):
    codes = oracle.pack(layout, trits)
    return oracle.matmul(layout, codes, scales, trits.shape[1], x_bits, x_dtype, signs=signs, rows=rows,
                         block=block)


def assert_within_bound(y_gpu, y_ref, bound, what=""):
    y = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y - y_ref)
    bad = ~(err <= bound)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first at {tuple(i)}: "
                             f"gpu={y[tuple(i)]!r} ref={y_ref[tuple(i)]!r} bound={bound[tuple(i)]!r}")
    return float((err / bound).max())
