"""Planted mistakes: each mutant is a copy of the oracle source with one plausible
error (a dropped term, a wrong index or sign, another rounding mode), compiled on
the CPU into a temporary library.  Every mutant must make at least one pin fail;
the unmodified oracle passes them all (test_oracle_pins.py).
"""
from __future__ import annotations

import os
import subprocess
import tempfile

import pytest

import oracle
import test_oracle_pins as pins
import test_oracle_pins_next as pn

MUTANTS = {
    "half-away rounding of activations": (
        "float r = rintf(t);", "float r = roundf(t);",
        [pins.test_act_quant_tie_fixture]),
    "reciprocal multiply instead of division": (
        "float t = bf16_to_float(row[k]) / s;", "float t = bf16_to_float(row[k]) * (1.0f / s);",
        [pins.test_act_quant_exact_rational]),
    "scale over 128 instead of 127": (
        "float s = amax / 127.0f;", "float s = amax / 128.0f;",
        [pins.test_act_quant_integer_row_is_identity]),
    "big-endian code order in a word": (
        "int code = (int)((word >> (bits * (int)(k % per))) & mask);",
        "int code = (int)((word >> (bits * (per - 1 - (int)(k % per)))) & mask);",
        [lambda m: pins.test_unpack_against_byte_view(m, 8)]),
    "two's-complement codes instead of offset binary": (
        "q_out[k * N + n] = (int8_t)(code - offset);", "q_out[k * N + n] = (int8_t)code;",
        [lambda m: pins.test_unpack_against_byte_view(m, 8)]),
    "dropped first element of each group": (
        "for (int64_t k = g * GROUP; k < (g + 1) * GROUP; ++k) {\n                int64_t a = qa[m * K + k];\n                const int8_t *wrow = q + k * N;\n                for (int64_t n = 0; n < N; ++n) acc[n] += a * (int64_t)wrow[n];\n            }\n            for (int64_t n = 0; n < N; ++n) {\n                if",
        "for (int64_t k = g * GROUP + 1; k < (g + 1) * GROUP; ++k) {\n                int64_t a = qa[m * K + k];\n                const int8_t *wrow = q + k * N;\n                for (int64_t n = 0; n < N; ++n) acc[n] += a * (int64_t)wrow[n];\n            }\n            for (int64_t n = 0; n < N; ++n) {\n                if",
        [pins.test_partials_brute_force_tiny]),
    "group scale of the wrong group": (
        "const float *srow = w_scale + g * N;\n            for (int64_t n = 0; n < N; ++n) {\n                double s = (double)srow[n];\n                ys[n] += s * (double)acc[n];",
        "const float *srow = w_scale + (G - 1 - g) * N;\n            for (int64_t n = 0; n < N; ++n) {\n                double s = (double)srow[n];\n                ys[n] += s * (double)acc[n];",
        [pins.test_w8a8_exact_rational_tiny]),
    "activation scale not applied": (
        "for (int64_t n = 0; n < N; ++n) { ys[n] *= as; ts[n] *= fabs(as); }",
        "for (int64_t n = 0; n < N; ++n) { ts[n] *= fabs(as); }",
        [pins.test_w8a8_constant_scale_reduces_to_per_channel]),
    "w4a16 sign of products lost": (
        "acc[n] += p;", "acc[n] += fabs(p);",
        [pins.test_w4a16_unit_scale_is_plain_gemm]),
    "bf16 output ties away from zero": (
        "double r = nearbyint(ldexp(a, -qexp));", "double r = round(ldexp(a, -qexp));",
        [pins.test_bf16_from_double_exact]),
    "rtn grid over qmax + 1": (
        "float s = amax / qmax;", "float s = amax / (qmax + 1.0f);",
        [lambda m: pins.test_rtn_exact_rational(m, 8)]),
    "dequant scale from the wrong group": (
        "float s = w_scale[(k / GROUP) * N + n];", "float s = w_scale[(k % 2) * N + n];",
        [lambda m: pins.test_dequant_is_rounded_product(m, 8)]),
    "weight-only groups counted as 128 wide": (
        "if (group <= 0 || K % group != 0 || ldx < K) return 1;\n    const int64_t G = K / group;",
        "if (group <= 0 || K % group != 0 || ldx < K) return 1;\n    const int64_t G = K / 128;",
        [pn.test_weight_only_group32_exact_rational]),
    "weight-only last element of each group dropped": (
        "for (int64_t k = g * group; k < (g + 1) * group; ++k) {\n                double a",
        "for (int64_t k = g * group; k < (g + 1) * group - 1; ++k) {\n                double a",
        [lambda m: pn.test_weight_only_unit_scale_is_plain_gemm(m, 32)]),
    "rtn with groups over qmax + 1": (
        "if (group <= 0 || K % group != 0 || group % per != 0) return 1;\n    const float qmax = bits == 8 ? 127.0f : 7.0f;",
        "if (group <= 0 || K % group != 0 || group % per != 0) return 1;\n    const float qmax = bits == 8 ? 128.0f : 8.0f;",
        [lambda m: pn.test_rtn_group_exact_rational(m, 8, 32)]),
    "rmsnorm without eps": (
        "double r = 1.0 / sqrt(mean + eps);", "double r = 1.0 / sqrt(mean);",
        [pn.test_rmsnorm_eps_and_mean]),
    "rmsnorm over the sum instead of the mean": (
        "double mean = ss / (double)K;", "double mean = ss;",
        [pn.test_rmsnorm_constant_row, pn.test_rmsnorm_eps_and_mean]),
    "rmsnorm with one rounding instead of the bf16 cast before gamma": (
        "uint16_t t = oracle_bf16_from_double(v * r);\n            double prod = (double)bf16_to_float(gamma[k]) * (double)bf16_to_float(t);",
        "uint16_t t = oracle_bf16_from_double(v * r);\n            (void)t;\n            double prod = (double)bf16_to_float(gamma[k]) * (v * r);",
        [pn.test_rmsnorm_against_decimal_square_root]),
    "rmsnorm without gamma": (
        "double prod = (double)bf16_to_float(gamma[k]) * (double)bf16_to_float(t);",
        "double prod = (double)bf16_to_float(t);",
        [pn.test_rmsnorm_constant_row]),
    "qk grouped-query heads mapped round robin": (
        "const int64_t hk = h / rep;", "const int64_t hk = h % Hkv;",
        [pn.test_attn_qk_int8_brute_force]),
    "qk dot over 127 of the 128 dimensions": (
        "for (int d = 0; d < 128; ++d) dot += (int64_t)qrow[d] * (int64_t)krow[d];",
        "for (int d = 0; d < 127; ++d) dot += (int64_t)qrow[d] * (int64_t)krow[d];",
        [pn.test_attn_qk_int8_brute_force]),
    "pv block scale taken before the V scale moves onto p": (
        "float v = fabsf(prow[t] * vs[t * Hkv + hk]);", "float v = fabsf(prow[t]);",
        [pn.test_attn_pv_int8_exact]),
    "pv block scale not applied": (
        "o[d] += (double)ps * (double)acc[d];", "o[d] += (double)acc[d];",
        [pn.test_attn_pv_int8_exact, pn.test_attn_pv_uniform_probabilities_average_v]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, oracle_mod, tmp_path):
    old, new, checks = MUTANTS[name]
    src = oracle_mod.source_text()
    assert src.count(old) >= 1, f"mutation site for {name!r} not found"
    mutated = src.replace(old, new, 1)
    c = tmp_path / "mutant.c"
    c.write_text(mutated)
    so = tmp_path / f"mutant_{abs(hash(name))}.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
                    "-o", str(so), str(c), "-lm"], check=True)
    prev = oracle_mod.use_library(str(so))
    try:
        caught = False
        for check in checks:
            try:
                check(oracle_mod)
            except (AssertionError, ValueError):
                caught = True
        assert caught, f"no pin caught the planted mistake: {name}"
    finally:
        oracle_mod.use_library(None)
        oracle_mod._lib = prev
