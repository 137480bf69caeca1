"""GPU parity of the W4A16 g128 GEMM against the fp64 oracle (tolerance in parity.py),
on the decode layer shapes at 8 and 64 tokens and on ragged edge cases."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import int8_group_scaled_amd as i8
import oracle
import synth
from parity import assert_within_tolerance, dev, dev_bf16, host_bf16_bits, rtn_weights, unpacked

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M", [8, 64])
@pytest.mark.parametrize("layer", ["qkv", "o_proj", "gate_up", "down"])
def test_w4a16_decode_layer(layer, M):
    L = synth.LAYERS[layer]
    xb = synth.activations_bf16(0, f"w4-{layer}-{M}", M, L.K, outliers=True)
    qw, ws = rtn_weights(0, f"w4-{layer}", L.K, L.N, 4)
    y = i8.gemm_w4a16_g128(dev_bf16(xb), dev(qw), dev(ws))
    torch.cuda.synchronize()
    y_exact, T = oracle.gemm_w4a16_g128(xb, unpacked(0, f"w4-{layer}", L.K, L.N, 4), ws)
    beyond, maxulp = assert_within_tolerance(host_bf16_bits(y), y_exact, T, L.K, w4=True, what=f"w4 {layer} M={M}")
    print(f"w4a16 {layer} M={M}: {beyond} beyond a bare ulp, max {maxulp:.3f} ulp")
    # Scaling each group's exact-product sum (not the weights) leaves only fp32 rounding of
    # group sums and of the fold: outputs more than one bf16 unit from the exact value can
    # only come from cancellation, at most 1 in 10^4 elements.
    assert beyond <= max(1, y_exact.size // 10_000), (beyond, maxulp)


@pytest.mark.parametrize("M,K,N", [(1, 128, 8), (8, 512, 256), (13, 384, 40), (13, 768, 40), (16, 2816, 264),
                                   (65, 256, 136), (130, 640, 264)])
def test_w4a16_ragged(M, K, N):
    xb = synth.activations_bf16(1, f"w4r{M}-{K}-{N}", M, K, outliers=True)
    words = synth.uniform_words(1, f"w4rw{M}-{K}-{N}", (K // 8) * N).reshape(K // 8, N)  # all 16 nibble values
    ws = np.abs(synth.normal_f32(1, f"w4rs{M}-{K}-{N}", (K // 128) * N, 0.003)).reshape(K // 128, N)
    y = i8.gemm_w4a16_g128(dev_bf16(xb), dev(words), dev(ws))
    torch.cuda.synchronize()
    y_exact, T = oracle.gemm_w4a16_g128(xb, oracle.gptq_unpack(words, 4, K), ws)
    assert_within_tolerance(host_bf16_bits(y), y_exact, T, K, w4=True, what=f"w4 ragged {M}x{K}x{N}")


def test_w4a16_repeatable():
    M, K, N = 64, 5120, 512
    xb = synth.activations_bf16(2, "w4rep", M, K, outliers=True)
    qw, ws = rtn_weights(2, "w4rep", K, N, 4)
    a = i8.gemm_w4a16_g128(dev_bf16(xb), dev(qw), dev(ws))
    b = i8.gemm_w4a16_g128(dev_bf16(xb), dev(qw), dev(ws))
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(a), host_bf16_bits(b))


@pytest.mark.parametrize("M,K,N", [(8, 640, 264), (8, 1280, 264), (64, 1280, 392), (70, 384, 136)])
def test_w4a16_strided_rows(M, K, N):
    """x and y addressed with row strides larger than K and N (ldx = K + 64, ldy = N + 24):
    the padding columns of y stay untouched."""
    xb = synth.activations_bf16(3, f"w4s{M}-{K}-{N}", M, K, outliers=True)
    qw, ws = rtn_weights(3, f"w4s{M}-{K}-{N}", K, N, 4)
    xfull = torch.zeros((M, K + 64), dtype=torch.bfloat16, device="cuda")
    xfull[:, :K] = dev_bf16(xb)
    yfull = torch.full((M, N + 24), 7.0, dtype=torch.bfloat16, device="cuda")
    i8.gemm_w4a16_g128(xfull[:, :K], dev(qw), dev(ws), y=yfull[:, :N])
    torch.cuda.synchronize()
    y_exact, T = oracle.gemm_w4a16_g128(xb, unpacked(3, f"w4s{M}-{K}-{N}", K, N, 4), ws)
    assert_within_tolerance(host_bf16_bits(yfull[:, :N].contiguous()), y_exact, T, K, w4=True,
                            what=f"w4 strided {M}x{K}x{N}")
    assert bool((yfull[:, N:] == 7.0).all())
