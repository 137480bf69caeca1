"""The W8A8 entry point that allocates nothing (gemm_w8a8_g128_noalloc): its output is
bit-identical to gemm_w8a8_g128's on the same inputs (same kernels and plan, scratch in
the library's static device array), on consecutive calls whose second input is
smaller, and within the output tolerance of the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import int8_group_scaled_amd as i8
import oracle
import synth
from parity import assert_within_tolerance, dev, dev_bf16, host_bf16_bits, rtn_weights

pytestmark = pytest.mark.gpu


def _check(M, K, N, tag, quantised=False):
    xb = synth.activations_bf16(11, tag, M, K, outliers=True)
    qw, ws = rtn_weights(11, tag, K, N, 8)
    qwd, wsd = dev(qw), dev(ws)
    if quantised:
        qa, s = oracle.quant_act_per_token(xb)
        args = dict(qa=dev(qa), a_scale=dev(s))
    else:
        args = dict(x=dev_bf16(xb))
    y_ref = i8.gemm_w8a8_g128(qwd, wsd, **args)
    y = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    i8.gemm_w8a8_g128_noalloc(qwd, wsd, y, **args)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(y), host_bf16_bits(y_ref)), tag
    qa_o, s_o = oracle.quant_act_per_token(xb)
    y_exact, T = oracle.gemm_w8a8_g128(qa_o, s_o, oracle.gptq_unpack(qw, 8, K), ws)
    assert_within_tolerance(host_bf16_bits(y), y_exact, T, K, what=tag)


def test_noalloc_two_calls_second_smaller():
    """A K-split decode layer (qkv: 48 tiles x 4 splits, fp32 pieces in the scratch array),
    then a smaller single linear: the second call reuses the array the first one left."""
    assert i8.noalloc_scratch_bytes() == 16 << 20
    _check(64, 5120, 6144, "na-qkv")
    _check(8, 512, 256, "na-single")


def test_noalloc_down_and_prequantised():
    _check(64, 17408, 5120, "na-down")          # 6 K splits: the largest decode scratch (8.6 MiB)
    _check(40, 1024, 520, "na-q", quantised=True)
    _check(300, 4096, 520, "na-prefill", quantised=True)  # prefill kernel: 6 tiles, K split 2 ways


def test_noalloc_rejects_oversized_scratch():
    M, K, N = 4096, 5120, 256
    xb = synth.activations_bf16(11, "na-big", M, K, outliers=False)
    qw, ws = rtn_weights(11, "na-big", K, N, 8)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="scratch"):
        i8.gemm_w8a8_g128_noalloc(dev(qw), dev(ws), y, x=dev_bf16(xb))
