"""Pins for the CPU oracle: each oracle function is checked against something other
than itself -- hand-derived fixtures, exact rational arithmetic, closed forms,
brute force on tiny inputs, float64 BLAS on integer-valued matrices, and special
cases that reduce to a plain library GEMM.  All run on the CPU.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest

import synth
from exact import fl32, fl_bf16, frac, rne_int, bf16_bits, ulp_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_row(values):
    return synth.bf16_bits_from_f32(np.asarray(values, dtype=np.float32))


# ---------------------------------------------------------------- activation quant

def test_act_quant_tie_fixture(oracle_mod):
    """Hand-derived RNE codes on exact .5 ties (absmax 127 => scale exactly 1)."""
    rows = []
    for line in open(os.path.join(GOLDEN, "act_quant_ties.txt")):
        line = line.split("#")[0].strip()
        if line:
            x, even, away = line.split()
            rows.append((float(x), int(even), int(away)))
    x = _bf16_row([r[0] for r in rows])[None, :]
    assert np.array_equal(synth.f32_from_bf16_bits(x)[0], np.float32([r[0] for r in rows]))
    qa, s = oracle_mod.quant_act_per_token(x)
    assert s[0] == np.float32(1.0)
    assert qa[0].tolist() == [r[1] for r in rows]
    assert qa[0].tolist() != [r[2] for r in rows]


def test_act_quant_integer_row_is_identity(oracle_mod):
    """A bf16 row of integers in [-127, 127] containing 127 gives scale 1 and codes = x."""
    g = np.random.default_rng(1)
    v = g.integers(-127, 128, size=(3, 1000)).astype(np.float32)
    v[0, 17] = 127.0
    v[1, 5] = -127.0
    v[2, 999] = 127.0
    qa, s = oracle_mod.quant_act_per_token(_bf16_row(v))
    assert np.all(s == np.float32(1.0))
    assert np.array_equal(qa.astype(np.float32), v)


def test_act_quant_power_of_two_scaling(oracle_mod):
    """Scaling a row by 2^e leaves the codes unchanged and scales a_s by exactly 2^e."""
    x = synth.activations_bf16(3, "pow2", 6, 768, outliers=True)
    qa0, s0 = oracle_mod.quant_act_per_token(x)
    xf = synth.f32_from_bf16_bits(x)
    for e in (-7, -1, 1, 5):
        xs = synth.bf16_bits_from_f32(xf * np.float32(2.0 ** e))
        qa1, s1 = oracle_mod.quant_act_per_token(xs)
        assert np.array_equal(qa0, qa1)
        assert np.array_equal(s1, s0 * np.float32(2.0 ** e))


def test_act_quant_zero_row(oracle_mod):
    x = np.zeros((2, 256), dtype=np.uint16)
    x[1, 3] = 0x8000  # -0.0
    qa, s = oracle_mod.quant_act_per_token(x)
    assert np.all(s == 0) and np.all(qa == 0)


def test_act_quant_absmax_maps_to_127(oracle_mod):
    x = synth.activations_bf16(0, "amax", 64, 5120, outliers=True)
    qa, s = oracle_mod.quant_act_per_token(x)
    xf = synth.f32_from_bf16_bits(x)
    idx = np.argmax(np.abs(xf), axis=1)
    assert np.array_equal(np.abs(qa[np.arange(64), idx]), np.full(64, 127, np.int8))
    assert np.all(np.abs(qa.astype(np.int32)) <= 127)


def test_act_quant_exact_rational(oracle_mod):
    """Every code equals round_half_even(fl32(x / fl32(absmax / 127))) computed with exact rationals.

    The rows checked include elements where multiplying by a rounded reciprocal
    (1/s or 127/absmax), or rounding half away from zero, gives a different code,
    so the check separates those readings from true division with ties to even.
    """
    M, K = 512, 5120
    x = synth.activations_bf16(0, "exact-act", M, K, outliers=True)
    qa, s = oracle_mod.quant_act_per_token(x)
    xf = synth.f32_from_bf16_bits(x)
    rows = [0, 1, 30, 67, 201, 253]
    recip_differs = recip2_differs = away_differs = 0
    for m in rows:
        amax = max(abs(frac(v)) for v in xf[m])
        sm = fl32(amax / 127)
        assert frac(s[m]) == sm
        recip = fl32(1 / sm)
        recip2 = fl32(127 / amax)
        for k in range(K):
            xv = frac(xf[m, k])
            t = fl32(xv / sm)
            q = max(-127, min(127, rne_int(t)))
            assert int(qa[m, k]) == q, (m, k)
            if max(-127, min(127, rne_int(fl32(xv * recip)))) != q:
                recip_differs += 1
            if max(-127, min(127, rne_int(fl32(xv * recip2)))) != q:
                recip2_differs += 1
            away = int(abs(t) + Fraction(1, 2)) * (1 if t >= 0 else -1)
            if max(-127, min(127, away)) != q:
                away_differs += 1
    assert recip_differs > 0 and recip2_differs > 0 and away_differs > 0


# ---------------------------------------------------------------- unpack / dequant

@pytest.mark.parametrize("bits", [8, 4])
def test_unpack_against_byte_view(oracle_mod, bits):
    """Codes from the oracle equal those read from the words' little-endian memory bytes."""
    per = 32 // bits
    K, N = 512, 96
    words = synth.uniform_words(0, f"unpack{bits}", (K // per) * N).reshape(K // per, N)
    q = oracle_mod.gptq_unpack(words, bits, K)
    b = words.view(np.uint8).reshape(K // per, N, 4)  # byte j of word [r, n]
    if bits == 8:
        codes = np.transpose(b, (0, 2, 1)).reshape(K, N).astype(np.int32)  # k = 4r + j
        ref = codes - 128
    else:
        lo = (b & 0xF).astype(np.int32)
        hi = (b >> 4).astype(np.int32)
        nib = np.stack([lo, hi], axis=3).reshape(K // per, N, 8)  # nibble 2j, 2j+1
        ref = np.transpose(nib, (0, 2, 1)).reshape(K, N) - 8
    assert np.array_equal(q.astype(np.int32), ref)
    # the extremes of the code range occur and survive
    assert q.min() == -(1 << (bits - 1)) and q.max() == (1 << (bits - 1)) - 1


@pytest.mark.parametrize("bits", [8, 4])
def test_dequant_is_rounded_product(oracle_mod, bits):
    per = 32 // bits
    K, N = 256, 40
    words = synth.uniform_words(1, f"deq{bits}", (K // per) * N).reshape(K // per, N)
    ws = np.abs(synth.normal_f32(1, f"deqs{bits}", (K // 128) * N, 0.001)).reshape(K // 128, N)
    w = oracle_mod.gptq_dequant(words, ws, bits, K)
    q = oracle_mod.gptq_unpack(words, bits, K)
    for k in range(0, K, 7):
        for n in range(N):
            assert frac(w[k, n]) == fl32(frac(ws[k // 128, n]) * int(q[k, n]))


def test_dequant_requant_round_trip(oracle_mod):
    """rint(fl32(s*q) / s) == q for |q| <= 127: the grid survives a dequant / requant cycle."""
    K, N = 1024, 64
    w = synth.weights_f32(2, "rt", K, N)
    qw, ws = oracle_mod.gptq_quantize_rtn(w, 8)
    q = oracle_mod.gptq_unpack(qw, 8, K)
    wd = oracle_mod.gptq_dequant(qw, ws, 8, K)
    s_full = np.repeat(ws, 128, axis=0)
    back = np.rint(wd / s_full)
    assert np.array_equal(back.astype(np.int32), q.astype(np.int32))


# ---------------------------------------------------------------- RTN weight quantiser

@pytest.mark.parametrize("bits", [8, 4])
def test_rtn_exact_rational(oracle_mod, bits):
    K, N = 256, 24
    qmax = 127 if bits == 8 else 7
    qmin = -127 if bits == 8 else -8
    w = synth.weights_f32(4, f"rtn{bits}", K, N)
    w[0:128, 3] = 0.0  # an all-zero group
    qw, ws = oracle_mod.gptq_quantize_rtn(w, bits)
    q = oracle_mod.gptq_unpack(qw, bits, K)
    for g in range(K // 128):
        for n in range(N):
            col = [frac(v) for v in w[g * 128:(g + 1) * 128, n]]
            amax = max(abs(c) for c in col)
            s = fl32(amax / qmax)
            assert frac(ws[g, n]) == s
            for i, c in enumerate(col):
                want = 0 if s == 0 else max(qmin, min(qmax, rne_int(fl32(c / s))))
                assert int(q[g * 128 + i, n]) == want
    assert ws[0, 3] == 0 and np.all(q[0:128, 3] == 0)


def test_rtn_error_class(oracle_mod):
    """Round-to-nearest G128 INT8 on N(0, 0.02) weights: every element within half a step,
    relative Frobenius error in the 0.6-0.7% class the Flint model card audits."""
    K, N = 5120, 256
    w = synth.weights_f32(0, "rtn-class", K, N)
    qw, ws = oracle_mod.gptq_quantize_rtn(w, 8)
    wd = oracle_mod.gptq_dequant(qw, ws, 8, K)
    s_full = np.repeat(ws, 128, axis=0).astype(np.float64)
    err = np.abs(wd.astype(np.float64) - w.astype(np.float64))
    # half a step, plus the fp32 rounding of s*q (|q| <= 127, so at most 2^-17 s)
    assert np.all(err <= s_full * (0.5 + 2.0 ** -16))
    rel = np.linalg.norm(wd - w) / np.linalg.norm(w)
    assert 0.006 < rel < 0.007


# ---------------------------------------------------------------- group partials

def test_partials_brute_force_tiny(oracle_mod):
    """Pure-Python integer triple loop on the single-linear shape (8 x 512 x 256)."""
    M, K, N = 8, 512, 256
    x = synth.activations_bf16(0, "bf-x", M, K, outliers=False)
    qa, _ = oracle_mod.quant_act_per_token(x)
    words = synth.uniform_words(0, "bf-w", (K // 4) * N).reshape(K // 4, N)
    q = oracle_mod.gptq_unpack(words, 8, K)
    P = oracle_mod.group_partials(qa, q)
    qa_l = qa.astype(int).tolist()
    q_l = q.astype(int).tolist()
    for m in range(M):
        for g in range(K // 128):
            for n in range(N):
                acc = 0
                for k in range(g * 128, (g + 1) * 128):
                    acc += qa_l[m][k] * q_l[k][n]
                assert P[m, g, n] == acc


def test_partials_match_float64_blas(oracle_mod):
    """Integer-valued float64 GEMM per group is exact (|P| < 2^53)."""
    M, K, N = 64, 5120, 192
    x = synth.activations_bf16(0, "blas-x", M, K, outliers=True)
    qa, _ = oracle_mod.quant_act_per_token(x)
    words = synth.uniform_words(0, "blas-w", (K // 4) * N).reshape(K // 4, N)
    q = oracle_mod.gptq_unpack(words, 8, K)
    P = oracle_mod.group_partials(qa, q)
    A = qa.astype(np.float64)
    B = q.astype(np.float64)
    for g in range(K // 128):
        ref = A[:, g * 128:(g + 1) * 128] @ B[g * 128:(g + 1) * 128, :]
        assert np.array_equal(P[:, g, :].astype(np.float64), ref)
    # extremes: |P| stays far inside int32
    assert np.abs(P).max() <= 127 * 128 * 128


# ---------------------------------------------------------------- W8A8 output

def test_w8a8_exact_rational_tiny(oracle_mod):
    M, K, N = 3, 384, 16
    x = synth.activations_bf16(5, "er-x", M, K, outliers=True)
    qa, s = oracle_mod.quant_act_per_token(x)
    w = synth.weights_f32(5, "er-w", K, N)
    qw, ws = oracle_mod.gptq_quantize_rtn(w, 8)
    q = oracle_mod.gptq_unpack(qw, 8, K)
    y, T = oracle_mod.gemm_w8a8_g128(qa, s, q, ws)
    yb = oracle_mod.bf16_from_double(y)
    qa_l = qa.astype(int).tolist()
    q_l = q.astype(int).tolist()
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            mag = Fraction(0)
            for g in range(K // 128):
                p = sum(qa_l[m][k] * q_l[k][n] for k in range(g * 128, (g + 1) * 128))
                tot += frac(ws[g, n]) * p
                mag += abs(frac(ws[g, n])) * abs(p)
            exact = frac(s[m]) * tot
            assert abs(frac(y[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 50)
            assert abs(frac(T[m, n]) - abs(frac(s[m])) * mag) <= abs(frac(s[m])) * mag * Fraction(1, 2 ** 50)
            assert int(yb[m, n]) == bf16_bits(fl_bf16(exact))


def test_w8a8_constant_scale_reduces_to_per_channel(oracle_mod):
    """With one scale per column for all groups, y = a_s * s_n * (qa @ q) (a plain float64 GEMM)."""
    M, K, N = 16, 2048, 64
    x = synth.activations_bf16(6, "pc-x", M, K, outliers=True)
    qa, s = oracle_mod.quant_act_per_token(x)
    words = synth.uniform_words(6, "pc-w", (K // 4) * N).reshape(K // 4, N)
    q = oracle_mod.gptq_unpack(words, 8, K)
    col = np.abs(synth.normal_f32(6, "pc-s", N, 0.001)) + np.float32(1e-4)
    ws = np.tile(col[None, :], (K // 128, 1))
    y, T = oracle_mod.gemm_w8a8_g128(qa, s, q, ws)
    ref = (qa.astype(np.float64) @ q.astype(np.float64)) * col.astype(np.float64)[None, :]
    ref *= s.astype(np.float64)[:, None]
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13 * np.abs(T).max())


def test_w8a8_row_subset_matches_full(oracle_mod):
    M, K, N = 20, 256, 48
    x = synth.activations_bf16(7, "rs-x", M, K, outliers=False)
    qa, s = oracle_mod.quant_act_per_token(x)
    words = synth.uniform_words(7, "rs-w", (K // 4) * N).reshape(K // 4, N)
    q = oracle_mod.gptq_unpack(words, 8, K)
    ws = np.abs(synth.normal_f32(7, "rs-s", (K // 128) * N, 0.001)).reshape(K // 128, N)
    y, T = oracle_mod.gemm_w8a8_g128(qa, s, q, ws)
    rows = np.array([19, 0, 7])
    y2, T2 = oracle_mod.gemm_w8a8_g128(qa, s, q, ws, rows=rows)
    assert np.array_equal(y2, y[rows]) and np.array_equal(T2, T[rows])


# ---------------------------------------------------------------- W4A16 output

def test_w4a16_unit_scale_is_plain_gemm(oracle_mod):
    """All scales 1: y = x @ q (bf16 activations times small integers, float64 BLAS)."""
    M, K, N = 8, 1024, 80
    x = synth.activations_bf16(8, "w4u-x", M, K, outliers=True)
    words = synth.uniform_words(8, "w4u-w", (K // 8) * N).reshape(K // 8, N)
    q = oracle_mod.gptq_unpack(words, 4, K)
    ws = np.ones((K // 128, N), dtype=np.float32)
    y, T = oracle_mod.gemm_w4a16_g128(x, q, ws)
    ref = synth.f32_from_bf16_bits(x).astype(np.float64) @ q.astype(np.float64)
    assert np.allclose(y, ref, rtol=0, atol=1e-12 * T.max())


def test_w4a16_exact_rational_tiny(oracle_mod):
    M, K, N = 2, 256, 8
    x = synth.activations_bf16(9, "w4e-x", M, K, outliers=True)
    w = synth.weights_f32(9, "w4e-w", K, N)
    qw, ws = oracle_mod.gptq_quantize_rtn(w, 4)
    q = oracle_mod.gptq_unpack(qw, 4, K)
    y, T = oracle_mod.gemm_w4a16_g128(x, q, ws)
    xf = synth.f32_from_bf16_bits(x)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for g in range(K // 128):
                part = sum(frac(xf[m, k]) * int(q[k, n]) for k in range(g * 128, (g + 1) * 128))
                tot += frac(ws[g, n]) * part
            assert abs(frac(y[m, n]) - tot) <= frac(T[m, n]) * Fraction(1, 2 ** 48)


# ---------------------------------------------------------------- bf16 output rounding

def test_bf16_from_double_exact(oracle_mod):
    g = np.random.default_rng(11)
    vals = list(g.standard_normal(2000) * 10.0 ** g.integers(-30, 30, 2000))
    one = 1.0
    vals += [one + 2 ** -8, one + 3 * 2 ** -8, -(one + 2 ** -8), 2.0 ** -130, 3 * 2.0 ** -134,
             255.5 * 2 ** -7 * 2 ** 10, 0.0, -0.0]
    got = oracle_mod.bf16_from_double(np.array(vals))
    for v, b in zip(vals, got):
        want = bf16_bits(fl_bf16(Fraction(v)))
        if v == 0 and np.signbit(v):
            want = 0x8000
        assert int(b) == want, v
    assert int(got[len(vals) - 8]) == 0x3F80  # 1 + 2^-8 is a tie -> even (1.0)
    assert int(got[len(vals) - 7]) == 0x3F82  # 1 + 3*2^-8 -> 1 + 2^-6


def test_ulp_helper():
    assert ulp_bf16(Fraction(1)) == Fraction(1, 128)
    assert ulp_bf16(Fraction(3, 2)) == Fraction(1, 128)
    assert ulp_bf16(Fraction(-2)) == Fraction(1, 64)


# ---------------------------------------------------------------- shapes

def test_drafter_shapes_fixture():
    kv = {}
    for line in open(os.path.join(GOLDEN, "drafter_shapes.txt")):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split()
            kv[k] = float(v)
    L = synth.LAYERS
    assert L["qkv"].N == (kv["q_heads"] + 2 * kv["kv_heads"]) * kv["head_dim"] == 6144
    assert L["qkv"].K == L["gate_up"].K == L["lm_head"].K == kv["hidden_size"]
    assert L["o_proj"].K == kv["q_heads"] * kv["head_dim"]
    assert L["gate_up"].N == 2 * kv["intermediate_size"]
    assert L["down"].K == kv["intermediate_size"] and L["down"].N == kv["hidden_size"]
    assert L["fc"].K == kv["fc_in"] and L["fc"].N == kv["fc_out"]
    assert L["lm_head"].N == kv["vocab_size"]
    for l in synth.PREFILL_LAYERS + (L["lm_head"], L["single"]):
        assert l.K % int(kv["group_size"]) == 0 and l.N % 8 == 0
    per_layer = sum(l.K * l.N for l in synth.DECODE_LAYERS)
    quantised = int(kv["draft_layers"]) * per_layer + L["fc"].K * L["fc"].N
    assert quantised == 1_730_150_400
    # "I32 1.7B, 90%" of "1.9B"
    assert round(quantised / 1e9, 1) == kv["params_i32_billion"]
    assert abs(quantised / (kv["params_total_billion"] * 1e9) * 100 - kv["params_i32_percent"]) < 2
    # bf16 size ~ 2 bytes per parameter; INT4 g128 checkpoint ~ 3.2x smaller
    assert abs(kv["params_total_billion"] * 2 - kv["bf16_gb"]) / kv["bf16_gb"] < 0.02
    other = kv["params_total_billion"] * 1e9 - quantised
    int4_bytes = quantised / 2 + quantised / 128 * 2 + other * 2
    assert abs(int4_bytes / 1e9 - kv["quantized_gb"]) / kv["quantized_gb"] < 0.05


def test_tp4_shard_shapes():
    """One GPU's share at tensor-parallel size 4: four column shards (qkv, gate/up, vocabulary
    head) or four row shards (o_proj, down) rebuild the full layer, and every shard keeps
    whole 128-wide groups and a column count the kernels accept."""
    L = synth.LAYERS
    for full, shard, axis in (("qkv", "qkv_tp4", "N"), ("gate_up", "gate_up_tp4", "N"), ("lm_head", "lm_head_tp4", "N"),
                              ("o_proj", "o_proj_tp4", "K"), ("down", "down_tp4", "K")):
        f, s = L[full], L[shard]
        other = "K" if axis == "N" else "N"
        assert getattr(s, axis) * 4 == getattr(f, axis) and getattr(s, other) == getattr(f, other)
        assert s.K % 128 == 0 and s.N % 8 == 0
    # the row shards cut K on group boundaries: 8 and 34 groups per GPU
    assert L["o_proj_tp4"].K // 128 == 8 and L["down_tp4"].K // 128 == 34
    assert synth.SHARD_LAYERS == tuple(L[n] for n in ("qkv_tp4", "o_proj_tp4", "gate_up_tp4", "down_tp4"))
