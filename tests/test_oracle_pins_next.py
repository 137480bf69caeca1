"""Pins for the oracle functions of the weight-only INT8 GEMM (any group size), the RMS
normalisation that feeds the activation quantiser, and the INT8 attention products on the
block-g128 INT8 KV cache.  As in test_oracle_pins.py, each is checked against something
other than itself: exact rational arithmetic, high-precision decimal square roots,
closed forms, brute-force integer loops and float64 BLAS on exactly representable data.
"""
from __future__ import annotations

import decimal
from fractions import Fraction

import numpy as np
import pytest

import synth
from exact import bf16_bits, bf16_value, fl32, fl_bf16, frac, rne_int


def _bf16(values):
    return synth.bf16_bits_from_f32(np.asarray(values, dtype=np.float32))


# ---------------------------------------------------------------- weight-only GEMM, any group size

@pytest.mark.parametrize("group", [32, 128])
def test_weight_only_unit_scale_is_plain_gemm(oracle_mod, group):
    """All scales 1: y = x @ q for 8-bit codes (bf16 times integers, float64 BLAS)."""
    M, K, N = 8, 1024, 72
    x = synth.activations_bf16(20, "wo-u-x", M, K, outliers=True)
    words = synth.uniform_words(20, "wo-u-w", (K // 4) * N).reshape(K // 4, N)
    q = oracle_mod.gptq_unpack(words, 8, K)
    ws = np.ones((K // group, N), dtype=np.float32)
    y, T = oracle_mod.gemm_weight_only(x, q, ws, group)
    ref = synth.f32_from_bf16_bits(x).astype(np.float64) @ q.astype(np.float64)
    assert np.allclose(y, ref, rtol=0, atol=1e-12 * T.max())


def test_weight_only_group32_exact_rational(oracle_mod):
    """Group 32: every output equals the exact rational sum_g s[g] * sum_{k in g} x*q, with the
    scale of group k // 32 (a group-128 reading gives other values on this data)."""
    M, K, N = 2, 256, 6
    x = synth.activations_bf16(21, "wo-e-x", M, K, outliers=True)
    w = synth.weights_f32(21, "wo-e-w", K, N)
    qw, ws = oracle_mod.gptq_quantize_rtn_group(w, 8, 32)
    assert ws.shape == (K // 32, N)
    q = oracle_mod.gptq_unpack(qw, 8, K)
    y, T = oracle_mod.gemm_weight_only(x, q, ws, 32)
    xf = synth.f32_from_bf16_bits(x)
    differs = 0
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            wrong = Fraction(0)
            for g in range(K // 32):
                part = sum(frac(xf[m, k]) * int(q[k, n]) for k in range(g * 32, (g + 1) * 32))
                tot += frac(ws[g, n]) * part
                wrong += frac(ws[(g // 4) * 4, n]) * part
            assert abs(frac(y[m, n]) - tot) <= frac(T[m, n]) * Fraction(1, 2 ** 48)
            differs += wrong != tot
    assert differs > 0


def test_weight_only_4bit_group128_matches_w4a16(oracle_mod):
    """At 4 bits and group 128 the weight-only output is the W4A16 g128 output."""
    M, K, N = 4, 512, 40
    x = synth.activations_bf16(22, "wo-4-x", M, K, outliers=True)
    words = synth.uniform_words(22, "wo-4-w", (K // 8) * N).reshape(K // 8, N)
    q = oracle_mod.gptq_unpack(words, 4, K)
    ws = np.abs(synth.normal_f32(22, "wo-4-s", (K // 128) * N, 0.01)).reshape(K // 128, N)
    y1, T1 = oracle_mod.gemm_weight_only(x, q, ws, 128)
    y2, T2 = oracle_mod.gemm_w4a16_g128(x, q, ws)
    assert np.array_equal(y1, y2) and np.array_equal(T1, T2)


@pytest.mark.parametrize("bits,group", [(8, 32), (8, 128), (4, 32)])
def test_rtn_group_exact_rational(oracle_mod, bits, group):
    K, N = 256, 12
    qmax = 127 if bits == 8 else 7
    qmin = -127 if bits == 8 else -8
    w = synth.weights_f32(23, f"rtng{bits}-{group}", K, N)
    w[0:group, 2] = 0.0  # an all-zero group
    qw, ws = oracle_mod.gptq_quantize_rtn_group(w, bits, group)
    q = oracle_mod.gptq_unpack(qw, bits, K)
    for g in range(K // group):
        for n in range(N):
            col = [frac(v) for v in w[g * group:(g + 1) * group, n]]
            s = fl32(max(abs(c) for c in col) / qmax)
            assert frac(ws[g, n]) == s
            for i, c in enumerate(col):
                want = 0 if s == 0 else max(qmin, min(qmax, rne_int(fl32(c / s))))
                assert int(q[g * group + i, n]) == want
    assert ws[0, 2] == 0 and np.all(q[0:group, 2] == 0)


# ---------------------------------------------------------------- RMS normalisation

def _rms_reference(xrow, grow, eps):
    """h = bf16(gamma * bf16(x / sqrt(mean(x^2) + eps))) from the exact sum of squares and a
    60-digit decimal square root; also returns, per element, how close x*r lies to a bf16
    rounding midpoint (relative), and whether a single rounding would give another h."""
    ctx = decimal.Context(prec=60)
    xs = [frac(v) for v in xrow]
    ss = sum(v * v for v in xs)
    v = ss / len(xs) + Fraction(eps)
    dv = ctx.divide(decimal.Decimal(v.numerator), decimal.Decimal(v.denominator))
    r = Fraction(ctx.divide(decimal.Decimal(1), ctx.sqrt(dv)))
    out, margin, single_differs = [], [], 0
    for xv, gv in zip(xs, grow):
        xr = xv * r
        t = fl_bf16(xr)
        # distance of x*r from the nearest bf16 midpoint, relative
        if xr != 0:
            lo = fl_bf16(xr)
            other = fl_bf16(xr + (xr - lo)) if xr != lo else lo
            mid = (lo + other) / 2 if other != lo else None
            margin.append(abs(xr - mid) / abs(xr) if mid is not None else Fraction(1))
        else:
            margin.append(Fraction(1))
        g = bf16_value(gv)
        h = fl_bf16(g * t)
        single_differs += fl_bf16(g * xr) != h
        out.append(bf16_bits(h) if h != 0 else (0x8000 if (g * t) < 0 or (h == 0 and g * xr < 0) else 0))
    return out, margin, single_differs


def test_rmsnorm_against_decimal_square_root(oracle_mod):
    """Each output equals bf16(gamma * bf16(x / sqrt(mean(x^2) + eps))) evaluated from the exact
    sum of squares with a 60-digit square root, wherever x*r is not within 2^-45 of a bf16
    rounding midpoint; the rows include elements where rounding once (bf16(gamma*x*r)) differs."""
    M, K, eps = 4, 512, 1e-6
    x = synth.activations_bf16(24, "rms-x", M, K, outliers=True)
    gamma = _bf16(1.0 + 0.3 * synth.normal_f32(24, "rms-g", K))
    h = oracle_mod.rmsnorm_bf16(x, gamma, eps)
    xf = synth.f32_from_bf16_bits(x)
    close = single = 0
    for m in range(M):
        want, margin, sd = _rms_reference(xf[m], gamma, eps)
        single += sd
        for k in range(K):
            if margin[k] < Fraction(1, 2 ** 45):
                close += 1
                continue
            got = int(h[m, k])
            if want[k] in (0, 0x8000):
                assert got in (0, 0x8000)
            else:
                assert got == want[k], (m, k)
    assert close <= 2 and single > 0


def test_rmsnorm_constant_row(oracle_mod):
    """A row of 2.0 with eps = 2^-30: x / sqrt(4 + 2^-30) = 1 - 2^-33 rounds to 1.0, so h = gamma."""
    K = 256
    x = np.full((1, K), _bf16([2.0])[0], dtype=np.uint16)
    gamma = _bf16(synth.normal_f32(25, "rms-c", K))
    h = oracle_mod.rmsnorm_bf16(x, gamma, 2.0 ** -30)
    assert np.array_equal(h[0], gamma)
    # and -2.0 gives -gamma
    h2 = oracle_mod.rmsnorm_bf16(np.full((1, K), _bf16([-2.0])[0], dtype=np.uint16), gamma, 2.0 ** -30)
    assert np.array_equal(synth.f32_from_bf16_bits(h2[0]), -synth.f32_from_bf16_bits(gamma))


def test_rmsnorm_power_of_four_scaling(oracle_mod):
    """Scaling x by 4 and eps by 16 scales sum / K + eps by exactly 16 and r by exactly 1/4:
    the output is unchanged."""
    M, K = 6, 640
    x = synth.activations_bf16(26, "rms-s", M, K, outliers=True)
    gamma = _bf16(1.0 + 0.2 * synth.normal_f32(26, "rms-sg", K))
    h1 = oracle_mod.rmsnorm_bf16(x, gamma, 1e-6)
    x4 = synth.bf16_bits_from_f32(synth.f32_from_bf16_bits(x) * np.float32(4.0))
    h4 = oracle_mod.rmsnorm_bf16(x4, gamma, 16.0 * 1e-6)
    assert np.array_equal(h1, h4)


def test_rmsnorm_zero_row_quantises_to_zero(oracle_mod):
    x = np.zeros((2, 128), dtype=np.uint16)
    gamma = _bf16(np.ones(128))
    h = oracle_mod.rmsnorm_bf16(x, gamma, 1e-6)
    assert np.all(synth.f32_from_bf16_bits(h) == 0)
    qa, s = oracle_mod.quant_act_per_token(h)
    assert np.all(qa == 0) and np.all(s == 0)


def test_rmsnorm_eps_and_mean(oracle_mod):
    """eps enters as mean + eps (not sum + eps): a row of 1/8 with eps = 3/64 has mean 1/64,
    r = 1/sqrt(1/16) = 4, x*r = 1/2 exactly."""
    K = 128
    x = np.full((1, K), _bf16([0.125])[0], dtype=np.uint16)
    gamma = _bf16(np.full(K, 3.0))
    h = oracle_mod.rmsnorm_bf16(x, gamma, 3.0 / 64.0)
    assert np.all(synth.f32_from_bf16_bits(h) == 1.5)


# ---------------------------------------------------------------- INT8 attention on the block-g128 KV cache

def test_kv_codec_round_trip_and_scale(oracle_mod):
    """The block-g128 codec: one scale per 128-wide row, its absmax element at +-127, and the
    dequantised values within half a step of the inputs."""
    T, H = 37, 3
    kv = synth.activations_bf16(27, "kv", T * H, 128, outliers=True).reshape(T, H, 128)
    codes, scales = oracle_mod.kv_quant_block128(kv)
    assert codes.shape == (T, H, 128) and scales.shape == (T, H)
    xf = synth.f32_from_bf16_bits(kv).astype(np.float64)
    amax = np.abs(xf).max(axis=2)
    assert np.array_equal(scales, (amax / 127.0).astype(np.float32)) or np.allclose(scales, amax / 127, rtol=2e-7)
    assert np.all(np.abs(codes).max(axis=2) == 127)
    deq = codes.astype(np.float64) * scales[..., None].astype(np.float64)
    # half a step, plus the rounding of the fp32 scale and quotient (at most 127 * 2^-23 steps)
    assert np.all(np.abs(deq - xf) <= scales[..., None] * (0.5 + 2.0 ** -16))


def test_attn_qk_int8_brute_force(oracle_mod):
    """Integer dots by a Python loop and scores as exact rationals, with grouped-query heads
    (4 query heads on 2 KV heads: head h reads KV head h // 2)."""
    Mq, T, Hq, Hkv = 3, 5, 4, 2
    qb = synth.activations_bf16(28, "qk-q", Mq * Hq, 128, outliers=False).reshape(Mq, Hq, 128)
    kb = synth.activations_bf16(28, "qk-k", T * Hkv, 128, outliers=False).reshape(T, Hkv, 128)
    qq, qs = oracle_mod.kv_quant_block128(qb)
    kq, ks = oracle_mod.kv_quant_block128(kb)
    scale = 1.0 / np.sqrt(128.0)
    s, dots = oracle_mod.attn_qk_int8(qq, qs, kq, ks, scale)
    for h in range(Hq):
        for i in range(Mq):
            for t in range(T):
                d = sum(int(a) * int(b) for a, b in zip(qq[i, h], kq[t, h // 2]))
                assert dots[h, i, t] == d
                exact = frac(scale) * frac(qs[i, h]) * frac(ks[t, h // 2]) * d
                assert abs(frac(s[h, i, t]) - exact) <= abs(exact) * Fraction(1, 2 ** 50)


def test_attn_pv_int8_exact(oracle_mod):
    """INT8 PV over two 128-token blocks (the second partial): the V scale moves onto the
    probabilities, each block of them is quantised with its own scale (bit-exact codes and
    scales against exact rationals), and the output is the exact group-scaled sum."""
    Mq, T, Hq, Hkv = 2, 200, 2, 1
    logits = synth.normal_f32(29, "pv-l", Hq * Mq * T).reshape(Hq, Mq, T).astype(np.float64)
    p = np.exp(logits - logits.max(axis=2, keepdims=True))
    p = (p / p.sum(axis=2, keepdims=True)).astype(np.float32)
    vb = synth.activations_bf16(29, "pv-v", T * Hkv, 128, outliers=True).reshape(T, Hkv, 128)
    vq, vs = oracle_mod.kv_quant_block128(vb)
    out, mag, pq, ps = oracle_mod.attn_pv_int8(p, vq, vs)
    assert ps.shape == (Hq, Mq, 2)
    for h in range(Hq):
        for i in range(Mq):
            pp = [fl32(frac(p[h, i, t]) * frac(vs[t, 0])) for t in range(T)]
            for b in range(2):
                t0, t1 = b * 128, min(T, b * 128 + 128)
                s = fl32(max(abs(v) for v in pp[t0:t1]) / 127)
                assert frac(ps[h, i, b]) == s
                for t in range(t0, t1):
                    assert int(pq[h, i, t]) == max(-127, min(127, rne_int(fl32(pp[t] / s))))
            for d in (0, 1, 64, 127):
                exact = sum(frac(ps[h, i, t // 128]) * int(pq[h, i, t]) * int(vq[t, 0, d]) for t in range(T))
                assert abs(frac(out[h, i, d]) - exact) <= frac(mag[h, i, d]) * Fraction(1, 2 ** 50)


def test_attn_pv_uniform_probabilities_average_v(oracle_mod):
    """Uniform probabilities 1/T on unit V scales quantise to 127 everywhere, so the output is
    127 * fl32(fl32(1/T) / 127) times the column sums of the codes: the average of V."""
    Mq, T, Hq, Hkv = 1, 256, 1, 1
    p = np.full((Hq, Mq, T), np.float32(1.0 / T))
    words = synth.uniform_words(30, "pv-u", T * 128 // 4).view(np.int8).reshape(T, 1, 128)
    vq = np.clip(words, -127, 127).astype(np.int8)
    vs = np.ones((T, 1), dtype=np.float32)
    out, _, pq, ps = oracle_mod.attn_pv_int8(p, vq, vs)
    assert np.all(pq == 127)
    s = float(np.float32(np.float32(1.0 / T) / np.float32(127.0)))
    want = 127 * s * vq[:, 0, :].astype(np.float64).sum(axis=0)
    assert np.allclose(out[0, 0], want, rtol=1e-15, atol=0)
    assert np.allclose(out[0, 0], vq[:, 0, :].mean(axis=0), rtol=1e-6)
