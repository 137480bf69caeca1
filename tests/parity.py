"""Helpers shared by the GPU parity tests: seeded inputs, device transfer, and the
output tolerance.

Tolerance for bf16 outputs (one reading of "within one bf16 unit", made exact):
an element passes iff
    |y_gpu - y_exact| <= ulp_bf16(y_exact) + c * 2^-24 * T
where y_exact and T come from the fp64 oracle, T is the a-priori magnitude of the
fp32 evaluation (a_scale * sum_g |w_scale * P| for W8A8; sum_g |w_scale| *
sum_k |x*q| for W4A16) and c counts the fp32 roundings any summation order can
add: K/128 + 2 for W8A8 (the fold over groups, the scale products, the row
scale), K/128 + 130 for W4A16 (plus the 128-term fp32 sum inside each group), and
K/group + group + 2 for a weight-only GEMM with another group size.
Where |y| is comparable to T this is one bf16 unit; only elements whose terms
cancel get the (tiny) extra allowance, which no fp32 implementation can avoid.
"""
from __future__ import annotations

import functools

import numpy as np
import torch

import oracle
import synth

DEV = "cuda:0"


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def ulp_bf16(y: np.ndarray) -> np.ndarray:
    a = np.abs(y)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(np.maximum(e - 7, -133)), 2.0 ** -133)


def tolerance_report(y_bits: np.ndarray, y_exact: np.ndarray, T: np.ndarray, K: int, w4: bool = False,
                     group: int | None = None):
    """(pass mask, number beyond a bare 1 ulp, max error in ulps).  group: weight-only GEMM
    with that group size (c = K/group + group + 2: the fold, the in-group fp32 sum, the
    scale products)."""
    yg = synth.f32_from_bf16_bits(y_bits).astype(np.float64)
    if group is not None:
        c = K // group + group + 2
    else:
        c = K // 128 + (130 if w4 else 2)
    ulp = ulp_bf16(y_exact)
    err = np.abs(yg - y_exact)
    ok = err <= ulp + c * 2.0 ** -24 * T
    return ok, int((err > ulp).sum()), float((err / ulp).max()) if err.size else 0.0


def assert_within_tolerance(y_bits, y_exact, T, K, w4=False, what="", group=None):
    ok, beyond, maxulp = tolerance_report(y_bits, y_exact, T, K, w4, group)
    bad = np.argwhere(~ok)
    assert ok.all(), (f"{what}: {len(bad)} elements outside tolerance, first {bad[:5].tolist()}, "
                      f"max {maxulp:.2f} ulp")
    return beyond, maxulp


@functools.lru_cache(maxsize=16)
def rtn_weights(seed: int, tag: str, K: int, N: int, bits: int):
    """Seeded N(0, 0.02) weights packed by the oracle's RTN G128 quantiser."""
    w = synth.weights_f32(seed, tag, K, N)
    qw, ws = oracle.gptq_quantize_rtn(w, bits)
    return qw, ws


@functools.lru_cache(maxsize=16)
def unpacked(seed: int, tag: str, K: int, N: int, bits: int):
    qw, _ = rtn_weights(seed, tag, K, N, bits)
    return oracle.gptq_unpack(qw, bits, K)


@functools.lru_cache(maxsize=8)
def rtn_weights_group(seed: int, tag: str, K: int, N: int, bits: int, group: int):
    """Seeded N(0, 0.02) weights packed by the oracle's RTN quantiser with `group` K values per scale."""
    w = synth.weights_f32(seed, tag, K, N)
    return oracle.gptq_quantize_rtn_group(w, bits, group)
