"""Planted mistakes in the oracle must be caught by its pins.

Each case copies oracle/oracle.c, changes one line the way a plausible slip would
(a wrong sign, index, order, normalisation or a dropped term), builds it on the CPU,
and runs tests/test_oracle_pins.py against the broken copy. The pin suite must fail.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "slot2_code_sign": ("int q = v + 1;", "int q = 1 - v;"),
    "slot2_bit_order": ("int bit = 2 * (int)(c % 4);", "int bit = 2 * (int)(3 - c % 4);"),
    "slot2_unpack_offset": ("t[r * k + c] = (int8_t)(q - 1);", "t[r * k + c] = (int8_t)(1 - q);"),
    "base3_digit_order": [("int value = 0, power = 1;", "int value = 0, power = 81;"), ("power *= 3;", "power /= 3;")],
    "base3_pad_value": ("int digit = 1; /* trit 0", "int digit = 0; /* trit 0"),
    "scale_group_index": ("scales[r * (k / 128) + c / 128]", "scales[r * (k / 128) + (c / 128 + 1) % (k / 128)]"),
    "rotation_sign_side": ("((double)sb[j] * xb[j])", "((double)sb[i] * xb[j])"),
    "rotation_norm": ("xr[r * k + b * n + i] = acc / norm;", "xr[r * k + b * n + i] = acc / (double)n;"),
    "rotation_hadamard_index": ("(double)h[i * n + j]", "(double)h[i * n + ((j + 1) & (n - 1))]"),
    "dropped_last_term": ("for (int64_t c = 0; c < k; ++c) {\n          double p", "for (int64_t c = 0; c + 1 < k; ++c) {\n          double p"),
    "bound_without_abs": ("mag += fabs(p);", "mag += p;"),
    "f16_exponent_bias": ("v = ldexp((double)(1024 + m), e - 25);", "v = ldexp((double)(1024 + m), e - 24);"),
    "f16_subnormal_scale": ("v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    "bf16_mantissa_width": ("v = ldexp((double)(128 + m), e - 134);", "v = ldexp((double)(256 + m), e - 135);"),
    "rotation_block_ignored": ("orc_rotate_f64(xd, sign, m, k, block, out);", "orc_rotate_f64(xd, sign, m, k, 128, out);"),
    "rmsnorm_mean_denominator": ("sqrt(sq / (double)k + eps)", "sqrt(sq / (double)(k - 1) + eps)"),
    "rmsnorm_eps_outside_sqrt": ("sqrt(sq / (double)k + eps)", "(sqrt(sq / (double)k) + eps)"),
    "rmsnorm_gamma_index": ("orc_bf16_to_f64(gamma[c]) * xr[c]", "orc_bf16_to_f64(gamma[k - 1 - c]) * xr[c]"),
    "rmsnorm_skipped_in_product": ("if (rc == ORC_OK && gamma) {", "if (rc == ORC_OK && gamma && 0) {"),
    "flips_dropped_last_trit": ("for (int64_t i = 0; i < k; ++i) c += ta[i] != tb[i];",
                                "for (int64_t i = 0; i + 1 < k; ++i) c += ta[i] != tb[i];"),
    "binary_bit_order": ("codes[r * rb + c / 8] |= (uint8_t)(1u << (c % 8));",
                         "codes[r * rb + c / 8] |= (uint8_t)(1u << (7 - c % 8));"),
    "binary_sign": ("t[r * k + c] = ((codes[r * rb + c / 8] >> (c % 8)) & 1) ? 1 : -1;",
                    "t[r * k + c] = ((codes[r * rb + c / 8] >> (c % 8)) & 1) ? -1 : 1;"),
    "binary_row_bytes": ("if (layout == ORC_BINARY) return k / 8;", "if (layout == ORC_BINARY) return k / 4;"),
    "flips_row_stride": ("unpack_row(layout, b + r * row_stride_b, k, tb)", "unpack_row(layout, b + r * row_stride_a, k, tb)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    edits = MUTANTS[name]
    if isinstance(edits, tuple):
        edits = [edits]
    src = open(SRC).read()
    for before, after in edits:
        assert src.count(before) == 1, f"mutation anchor for {name} not found exactly once"
        src = src.replace(before, after)
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(src)
    so = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-o", str(so), str(mutated), "-lm"])
    env = dict(os.environ, TGS_ORACLE_SO=str(so), OMP_NUM_THREADS="2")
    proc = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert proc.returncode != 0, f"pins did not catch mutant {name}:\n{proc.stdout[-2000:]}"
    assert "failed" in proc.stdout or "Error" in proc.stdout
