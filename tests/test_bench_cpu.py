"""Host-side checks of bench.py (no GPU): the algorithmic byte counts it divides by, the
stored traffic figures' source key, and the single-GPU contract."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    sys.path.insert(0, ROOT)
    import bench as b
    return b


def test_byte_counts_by_hand(bench):
    # qkv at M = 64: codes K*N, fp32 scales per 128-group, int8 qa + fp32 row scales in, bf16 y out
    M, K, N = 64, 5120, 6144
    assert bench.gemm_bytes(M, K, N) == 5120 * 6144 + 4 * 6144 * 40 + 64 * 5120 + 4 * 64 + 2 * 64 * 6144
    # the full linear reads bf16 x instead of qa
    assert bench.linear_bytes(M, K, N) == 5120 * 6144 + 4 * 6144 * 40 + 2 * 64 * 5120 + 2 * 64 * 6144
    # 4-bit codes: half a byte each
    assert bench.w4_bytes(8, K, N) == 5120 * 6144 // 2 + 4 * 6144 * 40 + 2 * 8 * 5120 + 2 * 8 * 6144
    # weight-only at group 32: four times the scales of group 128
    assert bench.wo_bytes(8, K, N, 8, 32) - bench.wo_bytes(8, K, N, 8, 128) == 4 * N * (K // 32 - K // 128)
    assert bench.wo_bytes(8, K, N, 4, 128) == bench.w4_bytes(8, K, N)


def test_traffic_key_ignores_comments_and_whitespace(bench, tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int a = 1; // one\n/* block\ncomment */ int b = 2;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "DECODE_SOURCES", ("k.hip",))
    h1 = bench.decode_sources_sha256()
    src.write_text("int a = 1;   // another comment\n\n   int b = 2;  /* x */\n")
    assert bench.decode_sources_sha256() == h1
    src.write_text("int a = 1; int b = 3;\n")
    assert bench.decode_sources_sha256() != h1


def test_stored_traffic_covers_the_four_layers(bench):
    names = {"qkv", "o_proj", "gate_up", "down"}
    assert set(bench.DECODE_TRAFFIC["fetch"]) == names and set(bench.DECODE_TRAFFIC["write"]) == names
    assert len(bench.DECODE_TRAFFIC["sources_sha256"]) == 64
    # measured traffic is at least the algorithmic bytes of each layer
    import synth
    for L in synth.DECODE_LAYERS:
        t = bench.DECODE_TRAFFIC["fetch"][L.name] + bench.DECODE_TRAFFIC["write"][L.name]
        assert t >= bench.gemm_bytes(64, L.K, L.N)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
