"""GPU parity: the INT8 block-g128 KV codec and the INT8 QK / PV attention products
(kv_quant_int8_block128, attn_qk_int8, attn_pv_int8) against the oracle.

Bars: codes, scales, QK int32 dots, and PV probability codes and block scales
bit-exact; QK scores within 3 * 2^-24 relative (three fp32 products of exact
factors); PV outputs within (B + 2) * 2^-24 times the a-priori magnitude of the fp32
fold over B = ceil(T/128) token blocks.  Shapes: the drafter's attention (32 query
heads over 8 KV heads, head dimension 128), one block of 8 queries against a
2048-token window and a 16384-token context, plus ragged sizes that leave partial
tiles and partial token blocks, and the empty cases.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import int8_group_scaled_amd as i8
import oracle
import synth
from parity import dev, dev_bf16

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _kv(seed, tag, T, H, outliers=True):
    return synth.activations_bf16(seed, tag, T * H, 128, outliers).reshape(T, H, 128)


def _probs(seed, tag, Hq, Mq, T, temp=2.0):
    """Softmax rows over T tokens of seeded N(0, temp^2) logits (test-side input recipe)."""
    logits = synth.normal_f32(seed, tag, Hq * Mq * T, temp).reshape(Hq, Mq, T).astype(np.float64)
    if T == 0:
        return np.zeros((Hq, Mq, 0), dtype=np.float32)
    p = np.exp(logits - logits.max(axis=2, keepdims=True))
    return (p / p.sum(axis=2, keepdims=True)).astype(np.float32)


def _codec(kvb, heads=None):
    codes, scales = i8.kv_quant_int8_block128(dev_bf16(kvb) if heads is None else kvb, heads)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


@pytest.mark.parametrize("T,H", [(2048, 8), (1, 1), (17, 3), (2049, 8), (16, 32)])
def test_kv_codec_bit_exact(T, H):
    kvb = _kv(1, f"kv{T}x{H}", T, H)
    kvb[0, 0] = 0                                   # an all-zero head vector: scale 0, codes 0
    codes, scales = _codec(kvb)
    c_o, s_o = oracle.kv_quant_block128(kvb)
    assert np.array_equal(scales.view(np.uint32), s_o.view(np.uint32))
    assert np.array_equal(codes, c_o)
    assert scales[0, 0] == 0 and not codes[0, 0].any()


def test_kv_codec_reads_a_slice_of_the_fused_qkv_output():
    """K and V are column slices of the fused qkv projection output [T, (32 + 2*8) * 128]."""
    T, Hq, Hkv = 257, 32, 8
    qkv = synth.activations_bf16(2, "qkv-out", T, (Hq + 2 * Hkv) * 128, True)
    y = dev_bf16(qkv)
    for off, H in ((0, Hq), (Hq * 128, Hkv), ((Hq + Hkv) * 128, Hkv)):
        codes, scales = i8.kv_quant_int8_block128(y[:, off:off + H * 128], H)
        torch.cuda.synchronize()
        c_o, s_o = oracle.kv_quant_block128(qkv[:, off:off + H * 128].reshape(T, H, 128))
        assert np.array_equal(scales.cpu().numpy().view(np.uint32), s_o.view(np.uint32)), off
        assert np.array_equal(codes.cpu().numpy(), c_o), off


def _qk_case(Mq, T, Hq, Hkv, seed, scale=128 ** -0.5):
    qb = _kv(seed, f"q{Mq}", Mq, Hq)
    kb = _kv(seed, f"k{T}", T, Hkv)
    qq, qs = oracle.kv_quant_block128(qb)
    kq, ks = oracle.kv_quant_block128(kb)
    s, dots = i8.attn_qk_int8(dev(qq), dev(qs), dev(kq), dev(ks), scale, want_dots=True)
    torch.cuda.synchronize()
    s_o, d_o = oracle.attn_qk_int8(qq, qs, kq, ks, float(np.float32(scale)))
    return s.cpu().numpy(), dots.cpu().numpy(), s_o, d_o


@pytest.mark.parametrize("Mq,T,Hq,Hkv", [(8, 2048, 32, 8), (3, 77, 4, 1), (17, 129, 2, 2), (1, 1, 1, 1),
                                         (64, 300, 8, 8), (8, 16384, 32, 8),
                                         (8, 4100, 32, 8),     # two waves per workgroup, ragged last block
                                         (8, 32768, 32, 8),    # the benchmark's long context
                                         (40, 161, 8, 2),      # 160 rows per KV head: three row blocks
                                         (3, 200, 32, 1),      # one KV head shared by 32 query heads
                                         (2, 130, 64, 64)])    # one query head per KV head
def test_attn_qk_int8(Mq, T, Hq, Hkv):
    s, dots, s_o, d_o = _qk_case(Mq, T, Hq, Hkv, 3)
    assert np.array_equal(dots, d_o), "int32 dots"
    err = np.abs(s.astype(np.float64) - s_o)
    bound = 3.01 * U * np.abs(s_o)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, f"scores beyond 3 ulp at {bad[:5].tolist()}"


def test_attn_qk_without_dots_matches():
    Mq, T, Hq, Hkv = 5, 200, 4, 2
    qq, qs = oracle.kv_quant_block128(_kv(4, "q", Mq, Hq))
    kq, ks = oracle.kv_quant_block128(_kv(4, "k", T, Hkv))
    a, _ = i8.attn_qk_int8(dev(qq), dev(qs), dev(kq), dev(ks), 0.5, want_dots=False)
    b, _ = i8.attn_qk_int8(dev(qq), dev(qs), dev(kq), dev(ks), 0.5, want_dots=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def _pv_check(p, vq, vs, what):
    out, pq, ps = i8.attn_pv_int8(dev(p), dev(vq), dev(vs), want_codes=True)
    torch.cuda.synchronize()
    o_o, mag, pq_o, ps_o = oracle.attn_pv_int8(p, vq, vs)
    assert np.array_equal(ps.cpu().numpy().view(np.uint32), ps_o.view(np.uint32)), f"{what}: ps"
    assert np.array_equal(pq.cpu().numpy(), pq_o), f"{what}: pq"
    B = ps_o.shape[2]
    err = np.abs(out.cpu().numpy().astype(np.float64) - o_o)
    bad = np.argwhere(err > (B + 2) * U * mag)
    assert bad.size == 0, f"{what}: out beyond tolerance at {bad[:5].tolist()}"
    return out


@pytest.mark.parametrize("Mq,T,Hq,Hkv", [(8, 2048, 32, 8), (3, 77, 4, 1), (17, 129, 2, 2), (1, 1, 1, 1),
                                         (20, 300, 8, 4), (8, 16384, 32, 8), (8, 5000, 32, 8), (2, 1000, 4, 4),
                                         (512, 700, 32, 8),
                                         (8, 32768, 32, 8),    # the benchmark's long context
                                         (3, 200, 32, 1),      # 96 rows on one KV head: three row tiles
                                         (2, 130, 64, 64)])    # one query head per KV head
def test_attn_pv_int8(Mq, T, Hq, Hkv):
    p = _probs(5, f"p{Mq}x{T}", Hq, Mq, T)
    vq, vs = oracle.kv_quant_block128(_kv(5, f"v{T}", T, Hkv))
    _pv_check(p, vq, vs, f"{Mq}x{T}x{Hq}/{Hkv}")


def test_attn_pv_split_is_deterministic():
    """With the token blocks split over workgroups (few rows, long context) the split sums
    are added in a fixed order: repeated calls give the same bits, also with a call of
    another shape on the same workspace in between."""
    Mq, T, Hq, Hkv = 8, 9000, 32, 8
    assert i8.load_library().attn_pv_int8_workspace_bytes(Mq, T, Hq, Hkv) > 0
    p = dev(_probs(8, "pdet", Hq, Mq, T))
    vq, vs = oracle.kv_quant_block128(_kv(8, "vdet", T, Hkv))
    vq, vs = dev(vq), dev(vs)
    a, _, _ = i8.attn_pv_int8(p, vq, vs)
    small = dev(_probs(8, "pdet2", 4, 3, 300))
    vq2, vs2 = oracle.kv_quant_block128(_kv(8, "vdet2", 300, 1))
    i8.attn_pv_int8(small, dev(vq2), dev(vs2))
    b, _, _ = i8.attn_pv_int8(p, vq, vs)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_attn_pv_leaves_the_gemm_counters_alone():
    """PV and the split-K GEMMs share the binding's workspace: the GEMM's arrival counters
    at its start stay zero across a split PV call, so a split-K GEMM after it is unchanged."""
    from parity import rtn_weights
    K, N, M = 5120, 6144, 8
    xb = synth.activations_bf16(9, "pv-ws-x", M, K, True)
    qw, ws = rtn_weights(9, "pv-ws", K, N, 4)
    x, qw, ws = dev_bf16(xb), dev(qw), dev(ws)
    y1 = i8.gemm_w4a16_g128(x, qw, ws)
    Mq, T, Hq, Hkv = 8, 9000, 32, 8
    p = dev(_probs(9, "pv-ws-p", Hq, Mq, T))
    vq, vs = oracle.kv_quant_block128(_kv(9, "pv-ws-v", T, Hkv))
    i8.attn_pv_int8(p, dev(vq), dev(vs))
    y2 = i8.gemm_w4a16_g128(x, qw, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_attn_pv_degenerate_rows():
    """A query row of zero probabilities (every block scale 0, output 0), a one-hot row
    (the output is that token's V row times its scale, up to the codec), and a row whose
    mass sits in the last partial block."""
    Mq, T, Hq, Hkv = 3, 260, 2, 1
    p = _probs(6, "pdeg", Hq, Mq, T)
    p[:, 0] = 0.0
    p[:, 1] = 0.0
    p[:, 1, 131] = 1.0
    p[:, 2, :256] = 0.0
    vq, vs = oracle.kv_quant_block128(_kv(6, "vdeg", T, Hkv))
    out = _pv_check(p, vq, vs, "degenerate").cpu().numpy()
    assert not out[:, 0].any()
    one_hot = 127 * np.float32(np.float32(vs[131, 0]) / np.float32(127)) * vq[131, 0].astype(np.float64)
    assert np.allclose(out[:, 1], one_hot[None, :], rtol=4 * U, atol=0)


def test_attn_pv_empty_context_writes_zeros():
    out = torch.full((2, 3, 128), 7.0, device="cuda:0")
    p = torch.empty((2, 3, 0), dtype=torch.float32, device="cuda:0")
    vq = torch.empty((0, 1, 128), dtype=torch.int8, device="cuda:0")
    vs = torch.empty((0, 1), dtype=torch.float32, device="cuda:0")
    i8.attn_pv_int8(p, vq, vs, out=out)
    torch.cuda.synchronize()
    assert not out.any()


def test_int8_attention_end_to_end_matches_oracle_chain():
    """Codec -> QK -> softmax (test side, fp64 from the same scores) -> PV, each device
    stage fed the previous device stage's output, against the oracle chain on the same
    inputs; the scores agree to 3 ulp, so the probabilities are recomputed from the
    oracle's scores for both sides and the PV codes stay bit-exact."""
    Mq, T, Hq, Hkv = 8, 1000, 8, 2
    qb, kb, vb = _kv(7, "e2e-q", Mq, Hq), _kv(7, "e2e-k", T, Hkv), _kv(7, "e2e-v", T, Hkv)
    qq, qs = i8.kv_quant_int8_block128(dev_bf16(qb))
    kq, ks = i8.kv_quant_int8_block128(dev_bf16(kb))
    vq, vs = i8.kv_quant_int8_block128(dev_bf16(vb))
    s, _ = i8.attn_qk_int8(qq, qs, kq, ks, 128 ** -0.5)
    torch.cuda.synchronize()
    qq_o, qs_o = oracle.kv_quant_block128(qb)
    kq_o, ks_o = oracle.kv_quant_block128(kb)
    vq_o, vs_o = oracle.kv_quant_block128(vb)
    s_o, _ = oracle.attn_qk_int8(qq_o, qs_o, kq_o, ks_o, float(np.float32(128 ** -0.5)))
    assert np.all(np.abs(s.cpu().numpy() - s_o) <= 3.01 * U * np.abs(s_o))
    p = np.exp(s_o - s_o.max(axis=2, keepdims=True))
    p = (p / p.sum(axis=2, keepdims=True)).astype(np.float32)
    assert np.array_equal(vq.cpu().numpy(), vq_o)
    _pv_check(p, vq.cpu().numpy(), vs.cpu().numpy(), "e2e")
