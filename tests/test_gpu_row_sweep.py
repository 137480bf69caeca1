"""GPU parity at every row count: the row count picks the W8A8 kernel (decode up to 64
rows, with one or two 32-row m tiles; the 256 x 256 prefill kernel above), the m tiles
and row chunks of the LDS-staged weight-only kernel, and the m tiles of the register-
streaming weight-only kernel (up to 16 rows on a vocabulary-wide N), and every kernel
masks the rows past M of its last tile.  Each case compares the whole output with the
oracle (W8A8: the per-group int32 partials bit-exact as well) on a small shape whose
columns end in a partial tile."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import int8_group_scaled_amd as i8
import oracle
import synth
from parity import assert_within_tolerance, dev, dev_bf16, host_bf16_bits, rtn_weights, rtn_weights_group

pytestmark = pytest.mark.gpu

SCHEMES = [(4, 128), (8, 128), (8, 32)]


@pytest.mark.parametrize("M", range(1, 73))
def test_w8a8_every_row_count(M):
    """K = 384 (three groups), N = 264 (a last 8-column fragment): y within tolerance and
    the partials from the kernel that serves the call bit-exact."""
    K, N = 384, 264
    qw, ws = rtn_weights(7, "row-sweep", K, N, 8)
    xb = synth.activations_bf16(7, f"row-sweep-{M}", M, K, outliers=True)
    qa, s = oracle.quant_act_per_token(xb)
    q = oracle.gptq_unpack(qw, 8, K)
    y = i8.gemm_w8a8_g128(dev(qw), dev(ws), x=dev_bf16(xb))
    P = i8.gemm_w8a8_g128_group_partials(dev(qa), dev(qw))
    torch.cuda.synchronize()
    assert np.array_equal(P.cpu().numpy(), oracle.group_partials(qa, q)), f"partials, M={M}"
    y_exact, T = oracle.gemm_w8a8_g128(qa, s, q, ws)
    assert_within_tolerance(host_bf16_bits(y), y_exact, T, K, what=f"w8a8 M={M}")


def _weight_only(M, K, N, bits, group, tag):
    qw, ws = rtn_weights_group(7, tag, K, N, bits, group)
    xb = synth.activations_bf16(7, f"{tag}-{M}", M, K, outliers=True)
    y = i8.gemm_weight_only(dev_bf16(xb), dev(qw), dev(ws), bits, group)
    torch.cuda.synchronize()
    y_exact, T = oracle.gemm_weight_only(xb, oracle.gptq_unpack(qw, bits, K), ws, group)
    beyond, maxulp = assert_within_tolerance(host_bf16_bits(y), y_exact, T, K, what=f"w{bits} g{group} M={M}",
                                             group=group)
    assert beyond <= max(1, y_exact.size // 10_000), (beyond, maxulp)


@pytest.mark.parametrize("bits,group", SCHEMES)
@pytest.mark.parametrize("M", range(1, 73))
def test_weight_only_lds_kernel_every_row_count(M, bits, group):
    """The LDS-staged kernel: K = 640 (at 4 bits with one m tile, two-group stages and a
    last one-group stage), N = 136 (one full 128-column tile and 8 columns)."""
    _weight_only(M, 640, 136, bits, group, "row-sweep-lds")


@pytest.mark.parametrize("bits,group", SCHEMES)
@pytest.mark.parametrize("M", range(1, 17))
def test_weight_only_register_kernel_every_row_count(M, bits, group):
    """The register-streaming kernel (vocabulary-wide N, up to 16 rows): N = 65544, 256
    full 256-column tiles and a last one of 8 columns; K = 1024, four 256-wide chunks
    split two ways, so the last split to arrive sums the pieces of the partial tile too."""
    _weight_only(M, 1024, 65544, bits, group, "row-sweep-reg")
