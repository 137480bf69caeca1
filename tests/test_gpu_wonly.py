"""GPU parity of the weight-only GEMM (gemm_weight_only: 4-bit group 128, 8-bit group 128
and group 32) against the fp64 oracle, within the weight-only tolerance of parity.py: the
decode layer shapes at 8 and 64 tokens, the 248320-column INT4 and INT8 vocabulary heads
(sampled rows), and ragged, strided and full-code-range edge cases; plus the group-size
RTN packer, bit-exact."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import int8_group_scaled_amd as i8
import oracle
import synth
from parity import assert_within_tolerance, dev, dev_bf16, host_bf16_bits, rtn_weights_group

pytestmark = pytest.mark.gpu

SCHEMES = [(4, 128), (8, 128), (8, 32)]


def _check(xb, words, ws, bits, group, K, what, rows=None, y=None):
    yd = i8.gemm_weight_only(dev_bf16(xb), dev(words), dev(ws), bits, group, y=y)
    torch.cuda.synchronize()
    q = oracle.gptq_unpack(words, bits, K)
    y_exact, T = oracle.gemm_weight_only(xb, q, ws, group, rows=rows)
    yb = host_bf16_bits(yd)
    if rows is not None:
        yb = yb[rows]
    beyond, maxulp = assert_within_tolerance(yb, y_exact, T, K, what=what, group=group)
    print(f"{what}: {beyond} of {y_exact.size} beyond a bare ulp, max {maxulp:.3f} ulp")
    assert beyond <= max(1, y_exact.size // 10_000), (beyond, maxulp)
    return yd


@pytest.mark.parametrize("bits,group", SCHEMES)
@pytest.mark.parametrize("M", [8, 64])
@pytest.mark.parametrize("layer", ["qkv", "o_proj", "gate_up", "down"])
def test_decode_layer(layer, M, bits, group):
    L = synth.LAYERS[layer]
    xb = synth.activations_bf16(0, f"wo-{layer}-{M}", M, L.K, outliers=True)
    qw, ws = rtn_weights_group(0, f"wo-{layer}-{bits}", L.K, L.N, bits, group)
    _check(xb, qw, ws, bits, group, L.K, f"w{bits} g{group} {layer} M={M}")


@pytest.mark.parametrize("bits,group", SCHEMES)
@pytest.mark.parametrize("M,K,N", [(1, 128, 8), (13, 384, 40), (16, 640, 264), (16, 1024, 264), (17, 256, 520),
                                   (33, 1152, 136), (64, 384, 1032), (65, 640, 264), (130, 1024, 72)])
def test_ragged(M, K, N, bits, group):
    """Uniformly random codes (every code value) and positive scales; K with a half last
    chunk (384, 640, 1152), N not a multiple of the 256-column tile, M across the 16-row tiles
    and past 64 (several row chunks)."""
    per = 32 // bits
    xb = synth.activations_bf16(2, f"wor{M}-{K}-{N}", M, K, outliers=True)
    words = synth.uniform_words(2, f"worw{bits}-{M}-{K}-{N}", (K // per) * N).reshape(K // per, N)
    ws = np.abs(synth.normal_f32(2, f"wors{group}-{M}-{K}-{N}", (K // group) * N, 0.003)).reshape(K // group, N)
    _check(xb, words, ws, bits, group, K, f"ragged w{bits} g{group} {M}x{K}x{N}")


@pytest.mark.parametrize("bits,group", SCHEMES)
@pytest.mark.parametrize("M,K,N", [(8, 640, 264), (64, 1280, 392), (70, 384, 136)])
def test_strided_rows(M, K, N, bits, group):
    """x and y with row strides larger than K and N: the padding columns of y stay untouched."""
    xb = synth.activations_bf16(3, f"wos{M}-{K}-{N}", M, K, outliers=True)
    qw, ws = rtn_weights_group(3, f"wos{M}-{K}-{N}-{bits}", K, N, bits, group)
    xfull = torch.zeros((M, K + 64), dtype=torch.bfloat16, device="cuda")
    xfull[:, :K] = dev_bf16(xb)
    yfull = torch.full((M, N + 24), 7.0, dtype=torch.bfloat16, device="cuda")
    i8.gemm_weight_only(xfull[:, :K], dev(qw), dev(ws), bits, group, y=yfull[:, :N])
    torch.cuda.synchronize()
    q = oracle.gptq_unpack(qw, bits, K)
    y_exact, T = oracle.gemm_weight_only(xb, q, ws, group)
    assert_within_tolerance(host_bf16_bits(yfull[:, :N].contiguous()), y_exact, T, K, group=group,
                            what=f"strided w{bits} g{group} {M}x{K}x{N}")
    assert bool((yfull[:, N:] == 7.0).all())


@pytest.mark.parametrize("bits,group", SCHEMES)
def test_repeatable(bits, group):
    M, K, N = 64, 5120, 512
    xb = synth.activations_bf16(4, "worep", M, K, outliers=True)
    qw, ws = rtn_weights_group(4, f"worep{bits}", K, N, bits, group)
    a = i8.gemm_weight_only(dev_bf16(xb), dev(qw), dev(ws), bits, group)
    b = i8.gemm_weight_only(dev_bf16(xb), dev(qw), dev(ws), bits, group)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(a), host_bf16_bits(b))


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M", [1, 8, 64])
def test_vocabulary_head(M, bits):
    """INT4 / INT8 group-128 vocabulary head: M tokens x 248320 columns; 4 sampled rows
    (every column) against the oracle."""
    L = synth.LAYERS["lm_head"]
    xb = synth.activations_bf16(0, f"wo-lm-{M}", M, L.K, outliers=False)
    qw, ws = rtn_weights_group(0, f"wo-lm-{bits}", L.K, L.N, bits, 128)
    rows = synth.sample_rows(0, f"wo-lm-{M}", M, 4)
    _check(xb, qw, ws, bits, 128, L.K, f"vocab w{bits} M={M}", rows=rows)


@pytest.mark.parametrize("bits,group", SCHEMES)
@pytest.mark.parametrize("K,N", [(512, 256), (5120, 6144), (384, 24)])
def test_rtn_group_bit_exact(bits, group, K, N):
    w = synth.weights_f32(5, f"rtng{K}x{N}", K, N)
    w[:group, 5] = 0.0  # an all-zero group
    qw, ws = i8.gptq_quantize_rtn_group(dev(w), bits, group)
    torch.cuda.synchronize()
    qw_o, ws_o = oracle.gptq_quantize_rtn_group(w, bits, group)
    assert np.array_equal(ws.cpu().numpy().view(np.uint32), ws_o.view(np.uint32))
    assert np.array_equal(qw.cpu().numpy(), qw_o)
