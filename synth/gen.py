"""Counter-based, slice-reproducible random inputs.

Every tensor is a pure function of (seed, tag, shape). Values come from
numpy's Philox-4x32-10 bit generator (Salmon et al., "Parallel random numbers:
as easy as 1, 2, 3", SC'11): the 128-bit key is (seed, crc64-like hash of the
tag) and each chunk of ``CHUNK`` elements starts at its own counter, so chunks
are generated independently (in threads) and any chunk can be regenerated
alone.  Normal variates use numpy's ziggurat sampler on that stream.

Workload recipe (the drafter layers of the Qwen3.8-27B DFlash2 model card):
activations are N(0, 1) fp32 rounded to bf16 (round-to-nearest-even), with
round(0.01*K) input channels -- chosen by a seeded permutation, the same for
every row -- multiplied by 20 before the rounding when outliers are asked for;
weights are N(0, 0.02) fp32 laid out [K, N] (input dimension first).
"""
from __future__ import annotations

import hashlib
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22


def _tag_key(seed: int, tag: str) -> np.ndarray:
    h = hashlib.blake2b(tag.encode(), digest_size=8).digest()
    return np.array([int(seed) & ((1 << 64) - 1), int.from_bytes(h, "little")], dtype=np.uint64)


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _chunked(seed: int, tag: str, n: int, fill) -> np.ndarray:
    """Run ``fill(generator, out_slice)`` over independent Philox chunks."""
    key = _tag_key(seed, tag)
    nchunks = (n + CHUNK - 1) // CHUNK

    def work(c: int, out: np.ndarray) -> None:
        bg = np.random.Philox(key=key, counter=np.array([0, 0, c, 0], dtype=np.uint64))
        fill(np.random.Generator(bg), out)

    return key, nchunks, work


def normal_f32(seed: int, tag: str, n: int, std: float = 1.0) -> np.ndarray:
    """``n`` float32 samples of N(0, std^2); chunk c depends only on (seed, tag, c)."""
    out = np.empty(n, dtype=np.float32)
    _, nchunks, work = _chunked(seed, tag, n, lambda g, o: g.standard_normal(out=o, dtype=np.float32))
    slices = [out[c * CHUNK:(c + 1) * CHUNK] for c in range(nchunks)]
    if nchunks == 1:
        work(0, slices[0])
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks), slices))
    if std != 1.0:
        out *= np.float32(std)
    return out


def uniform_words(seed: int, tag: str, n: int) -> np.ndarray:
    """``n`` uniformly random 32-bit words (returned as int32)."""
    out = np.empty(n, dtype=np.uint32)

    def fill(g, o):
        o[:] = g.integers(0, 1 << 32, size=o.shape[0], dtype=np.uint32)

    _, nchunks, work = _chunked(seed, tag, n, fill)
    slices = [out[c * CHUNK:(c + 1) * CHUNK] for c in range(nchunks)]
    if nchunks == 1:
        work(0, slices[0])
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks), slices))
    return out.view(np.int32)


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns the uint16 bit patterns.

    Inputs here are finite; NaN handling is not needed for generated data.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def outlier_channels(seed: int, tag: str, K: int) -> np.ndarray:
    """The round(0.01*K) input channels that carry x20 outliers (sorted)."""
    count = int(round(0.01 * K))
    g = np.random.Generator(np.random.Philox(key=_tag_key(seed, tag + "/outlier-channels")))
    return np.sort(g.permutation(K)[:count])


def activations_bf16(seed: int, tag: str, M: int, K: int, outliers: bool) -> np.ndarray:
    """bf16 bit patterns [M, K] of N(0,1) activations, optionally with x20 outlier channels."""
    x = normal_f32(seed, tag + "/x", M * K).reshape(M, K)
    if outliers:
        ch = outlier_channels(seed, tag, K)
        x[:, ch] *= np.float32(20.0)
    return bf16_bits_from_f32(x)


def weights_f32(seed: int, tag: str, K: int, N: int, std: float = 0.02) -> np.ndarray:
    """fp32 weights [K, N] drawn from N(0, std^2)."""
    return normal_f32(seed, tag + "/w", K * N, std).reshape(K, N)


def sample_rows(seed: int, tag: str, M: int, count: int) -> np.ndarray:
    """A sorted seeded sample of ``count`` distinct row indices in [0, M); always includes 0 and M-1."""
    if count >= M:
        return np.arange(M, dtype=np.int64)
    g = np.random.Generator(np.random.Philox(key=_tag_key(seed, tag + "/rows")))
    rows = set(int(r) for r in g.choice(M, size=count - 2, replace=False))
    rows.update((0, M - 1))
    return np.array(sorted(rows), dtype=np.int64)
