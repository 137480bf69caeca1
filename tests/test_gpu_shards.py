"""GPU parity of the W8A8 G128 GEMM on one GPU's share at tensor-parallel size 4 (the
size both serving recipes fix: Flint card, serving recipe; target model card, serving
section).

Column shards (qkv, gate/up, vocabulary head) are plain layers with N/4 columns.  Row
shards (o_proj, down) take K/4 on group boundaries; their activations are quantised over
the full K (the per-token maximum all-reduced first, so a shard's codes and scale equal
those of one GPU) and the shard's slice of the codes goes in with the full-K scale.  The
kernels see only the shard's shape: these are the launch plans a TP4 deployment would
run, with few column tiles (qkv: 1536 columns) or few groups (o_proj: 8)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import int8_group_scaled_amd as i8
import oracle
import synth
from parity import assert_within_tolerance, dev, dev_bf16, host_bf16_bits, rtn_weights, unpacked

pytestmark = pytest.mark.gpu

ROW_SHARDS = {"o_proj_tp4": "o_proj", "down_tp4": "down"}
SHARD = 1  # which of the four row shards (K slice) is checked


def _shard_inputs(name, M, seed=0):
    """(qa, a_scale, q, w_scale, qweight, x-or-None) for one GPU's share; x is given for the
    column shards (the library quantises), None for the row shards (pre-quantised codes)."""
    L = synth.LAYERS[name]
    tag = f"tp4-{name}-{M}"
    qw, ws = rtn_weights(seed, tag, L.K, L.N, 8)
    q = unpacked(seed, tag, L.K, L.N, 8)
    if name in ROW_SHARDS:
        Kfull = synth.LAYERS[ROW_SHARDS[name]].K
        xb = synth.activations_bf16(seed, tag, M, Kfull, True)
        qa_full, s = oracle.quant_act_per_token(xb)
        qa = np.ascontiguousarray(qa_full[:, SHARD * L.K:(SHARD + 1) * L.K])
        return qa, s, q, ws, qw, None
    xb = synth.activations_bf16(seed, tag, M, L.K, True)
    qa, s = oracle.quant_act_per_token(xb)
    return qa, s, q, ws, qw, xb


@pytest.mark.parametrize("name", [L.name for L in synth.SHARD_LAYERS])
def test_tp4_shard_decode(name):
    """64 tokens through one GPU's share of each drafter linear: full output within the
    tolerance, and the exact group sums of the same kernel bit-exact."""
    L = synth.LAYERS[name]
    M = 64
    qa, s, q, ws, qw, xb = _shard_inputs(name, M)
    if xb is None:
        y = i8.gemm_w8a8_g128(dev(qw), dev(ws), qa=dev(qa), a_scale=dev(s))
    else:
        y = i8.gemm_w8a8_g128(dev(qw), dev(ws), x=dev_bf16(xb))
    torch.cuda.synchronize()
    y_exact, T = oracle.gemm_w8a8_g128(qa, s, q, ws)
    beyond, maxulp = assert_within_tolerance(host_bf16_bits(y), y_exact, T, L.K, what=f"decode {name}")
    print(f"decode {name}: {beyond} of {y_exact.size} beyond a bare ulp, max {maxulp:.3f} ulp")
    P = i8.gemm_w8a8_g128_group_partials(dev(qa), dev(qw))
    torch.cuda.synchronize()
    assert np.array_equal(P.cpu().numpy(), oracle.group_partials(qa, q))


def test_tp4_lm_head_shard_sampled_rows():
    """A quarter of the vocabulary head (62080 columns) at 64 tokens; 6 sampled rows."""
    L = synth.LAYERS["lm_head_tp4"]
    M = 64
    qa, s, q, ws, qw, xb = _shard_inputs("lm_head_tp4", M)
    y = i8.gemm_w8a8_g128(dev(qw), dev(ws), x=dev_bf16(xb))
    torch.cuda.synchronize()
    rows = synth.sample_rows(0, "lm_head_tp4", M, 6)
    y_exact, T = oracle.gemm_w8a8_g128(qa, s, q, ws, rows=rows)
    assert_within_tolerance(host_bf16_bits(y)[rows], y_exact, T, L.K, what="lm_head_tp4")


@pytest.mark.parametrize("name", [L.name for L in synth.SHARD_LAYERS])
def test_tp4_shard_prefill_sampled_rows(name):
    """4096 tokens through one GPU's share: the prefill kernel on 16 row tiles by 6 to 34
    column tiles (fewer than one round of workgroups for qkv, so every tile is split along
    K); 16 sampled rows of y and of the exact group sums."""
    L = synth.LAYERS[name]
    M = 4096
    qa, s, q, ws, qw, xb = _shard_inputs(name, M)
    if xb is None:
        y = i8.gemm_w8a8_g128(dev(qw), dev(ws), qa=dev(qa), a_scale=dev(s))
    else:
        y = i8.gemm_w8a8_g128(dev(qw), dev(ws), x=dev_bf16(xb))
    torch.cuda.synchronize()
    rows = synth.sample_rows(0, f"tp4-prefill-{name}", M, 16)
    y_exact, T = oracle.gemm_w8a8_g128(qa, s, q, ws, rows=rows)
    yb = host_bf16_bits(y)[rows]
    del y
    assert_within_tolerance(yb, y_exact, T, L.K, what=f"prefill {name}")
    P = i8.gemm_w8a8_g128_group_partials(dev(qa), dev(qw))
    Prows = P[torch.from_numpy(rows).to(P.device)].cpu().numpy()
    del P
    torch.cuda.empty_cache()
    assert np.array_equal(Prows, oracle.group_partials(qa[rows], q))
