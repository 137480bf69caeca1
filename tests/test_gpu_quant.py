"""GPU parity, bit-exact: per-token activation quantisation, GPTQ unpack /
dequant, and RTN G128 packing, against the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import int8_group_scaled_amd as i8
import oracle
import synth
from parity import dev, dev_bf16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,outliers", [
    (8, 512, False),      # single linear
    (64, 5120, True),     # decode activations into qkv / gate_up
    (64, 4096, True),     # into o_proj
    (64, 17408, True),    # into down
    (4096, 5120, True),   # prefill
    (4096, 25600, True),  # prefill context projection (two-pass path)
    (1, 8, False),        # smallest row
    (3, 2056, True),      # ragged: not a multiple of the 2048-element thread stride
    (130, 33000, True),   # above the in-register limit
])
def test_quant_act_bit_exact(M, K, outliers):
    xb = synth.activations_bf16(0, f"q{M}x{K}", M, K, outliers)
    qa, s = i8.quant_act_per_token(dev_bf16(xb))
    torch.cuda.synchronize()
    qa_o, s_o = oracle.quant_act_per_token(xb)
    assert np.array_equal(s.cpu().numpy(), s_o)
    assert np.array_equal(qa.cpu().numpy(), qa_o)


def test_quant_act_special_rows_and_stride():
    K = 1024
    xb = synth.activations_bf16(1, "special", 6, K, outliers=True)
    xf = synth.f32_from_bf16_bits(xb)
    xf[0] = 0.0                                      # all-zero row
    xf[1, :] = np.resize(np.float32([0.5, -0.5, 1.5, -2.5, 126.5, 127.0]), K)  # ties
    xf[2] = xf[3] * np.float32(2.0 ** -20)           # tiny values
    xf[4] = xf[5] * np.float32(2.0 ** -130)          # subnormal a_scale: 1/a_scale overflows
    xb = synth.bf16_bits_from_f32(xf)
    big = np.zeros((6, K + 64), dtype=np.uint16)     # ldx > K
    big[:, :K] = xb
    xt = dev_bf16(big)[:, :K]
    qa, s = i8.quant_act_per_token(xt)
    torch.cuda.synchronize()
    qa_o, s_o = oracle.quant_act_per_token(xb)
    assert np.array_equal(s.cpu().numpy(), s_o)
    assert np.array_equal(qa.cpu().numpy(), qa_o)
    assert np.all(qa.cpu().numpy()[0] == 0) and s_o[0] == 0


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("K,N", [(512, 256), (5120, 6144), (384, 40)])
def test_gptq_unpack_bit_exact(bits, K, N):
    per = 32 // bits
    words = synth.uniform_words(2, f"u{bits}-{K}-{N}", (K // per) * N).reshape(K // per, N)
    ws = np.abs(synth.normal_f32(2, f"us{bits}-{K}-{N}", (K // 128) * N, 0.001)).reshape(K // 128, N)
    q, w = i8.gptq_unpack(dev(words), bits, dev(ws), want_codes=True, want_dequant=True)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), oracle.gptq_unpack(words, bits, K))
    assert np.array_equal(w.cpu().numpy().view(np.uint32), oracle.gptq_dequant(words, ws, bits, K).view(np.uint32))


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("K,N", [(512, 256), (17408, 5120), (256, 24)])
def test_gptq_rtn_bit_exact(bits, K, N):
    w = synth.weights_f32(3, f"rtn{K}x{N}", K, N)
    w[128:256, 5] = 0.0  # an all-zero group
    qw, ws = i8.gptq_quantize_rtn(dev(w), bits)
    torch.cuda.synchronize()
    qw_o, ws_o = oracle.gptq_quantize_rtn(w, bits)
    assert np.array_equal(ws.cpu().numpy().view(np.uint32), ws_o.view(np.uint32))
    assert np.array_equal(qw.cpu().numpy(), qw_o)
