"""GPU parity, bit-exact: RMS normalisation fused with the per-token INT8 quantisation
(rmsnorm_quant_per_token) against the oracle's RMS normalisation followed by its
per-token quantiser, on the decode and prefill activation shapes and edge rows."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import int8_group_scaled_amd as i8
import oracle
import synth
from parity import dev, dev_bf16, host_bf16_bits

pytestmark = pytest.mark.gpu


def _gamma(seed, K):
    return synth.bf16_bits_from_f32(1.0 + 0.25 * synth.normal_f32(seed, f"gamma{K}", K))


def _check(xb, gb, eps, what):
    qa, s, h = i8.rmsnorm_quant_per_token(dev_bf16(xb), dev_bf16(gb), eps, want_h=True)
    torch.cuda.synchronize()
    h_o = oracle.rmsnorm_bf16(xb, gb, float(np.float32(eps)))
    qa_o, s_o = oracle.quant_act_per_token(h_o)
    hb = host_bf16_bits(h)
    bad = np.argwhere(hb != h_o)
    assert bad.size == 0, f"{what}: h differs at {bad[:5].tolist()}"
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_o.view(np.uint32)), what
    assert np.array_equal(qa.cpu().numpy(), qa_o), what
    return qa, s, h


@pytest.mark.parametrize("M,K,outliers", [
    (64, 5120, True),     # decode: the inputs of qkv and gate/up
    (8, 5120, True),      # one draft block
    (4096, 5120, True),   # prefill
    (1, 8, False), (3, 2056, True), (130, 8192, True), (17, 32768, True), (600, 26624, True),
])
def test_rmsnorm_quant_bit_exact(M, K, outliers):
    xb = synth.activations_bf16(0, f"rms{M}x{K}", M, K, outliers)
    _check(xb, _gamma(0, K), 1e-6, f"{M}x{K}")


def test_fused_equals_separate_quantisation():
    """The fused codes equal the standalone quantisation kernel applied to the fused h."""
    M, K = 64, 5120
    xb = synth.activations_bf16(1, "rms-sep", M, K, True)
    qa, s, h = _check(xb, _gamma(1, K), 1e-6, "sep")
    qa2, s2 = i8.quant_act_per_token(h)
    torch.cuda.synchronize()
    assert torch.equal(qa, qa2) and torch.equal(s, s2)


def test_edge_rows_and_stride():
    K = 1024
    xb = synth.activations_bf16(2, "rms-edge", 6, K, True)
    xf = synth.f32_from_bf16_bits(xb)
    xf[0] = 0.0                                  # zero row: h = 0, codes 0, scale 0
    xf[1] = 2.0                                  # constant row
    xf[2] = xf[3] * np.float32(2.0 ** -60)       # tiny values
    xf[4] = xf[5] * np.float32(2.0 ** 60)        # huge values
    xb = synth.bf16_bits_from_f32(xf)
    big = np.zeros((6, K + 64), dtype=np.uint16)
    big[:, :K] = xb
    gb = _gamma(2, K)
    qa, s, h = i8.rmsnorm_quant_per_token(dev_bf16(big)[:, :K], dev_bf16(gb), 1e-6, want_h=True)
    torch.cuda.synchronize()
    h_o = oracle.rmsnorm_bf16(xb, gb, float(np.float32(1e-6)))
    qa_o, s_o = oracle.quant_act_per_token(h_o)
    assert np.array_equal(host_bf16_bits(h), h_o)
    assert np.array_equal(qa.cpu().numpy(), qa_o) and np.array_equal(s.cpu().numpy(), s_o)
    assert s_o[0] == 0 and np.all(qa_o[0] == 0)


@pytest.mark.parametrize("eps", [1e-6, 1e-5, 0.5])
def test_eps_values(eps):
    M, K = 16, 4096
    xb = synth.activations_bf16(3, f"rms-eps{eps}", M, K, True)
    _check(xb, _gamma(3, K), eps, f"eps={eps}")
