"""Benchmark of the W8A8 G128 linear on one MI355X.

One step = the decode workload: 64 tokens (8 sequences x a draft block of 8)
through the four drafter linears (fused qkv 5120->6144, o_proj 4096->5120, fused
gate/up 5120->34816, down 17408->5120), each as the full W8A8 G128 linear from
bf16 activations: per-token quantisation kernel, then the GEMM kernel.  Weights
are N(0, 0.02) fp32 packed on the GPU by the library's RTN G128 kernel; the
activations are N(0, 1) bf16 with 1% of channels scaled x20.  Weight copies are
rotated so that more than 1 GB of distinct weights is streamed between reuses
(more than the 256 MB last-level cache), i.e. every step reads its weights from
HBM.

Timing: W untimed steps, then exactly K steps between two synchronisations.
Before the K steps a short spin kernel is queued so the host can enqueue all of
them ahead of the GPU; the step time is then the GPU time between HIP events
recorded on the launch stream before the first and after the last step, and the
per-kernel durations come from events around every launch of every 8th timed
step on that stream (an event between two kernels adds a gap of its own).

value = algorithmic bytes of the step / step time, with per-layer bytes
K*N (codes) + 4*N*K/128 (fp32 scales) + 2*M*K (bf16 x) + 2*M*N (bf16 y).
The roofline entry is for the GEMM kernel: bytes per launch K*N + 4*N*K/128 +
M*K + 4*M (qa, a_scale) + 2*M*N, over its average duration, against 8 TB/s;
`traffic` is the HBM bytes per launch measured with rocprofv3 counters (see
DECODE_TRAFFIC), null when the kernel sources have changed since.
Secondary figures, each against its roofline: prefill (4096 tokens, five layers,
GEMM kernel on pre-quantised activations) in TOP/s against the 5.0 POP/s dense INT8
peak; the INT8 vocabulary head (64 tokens x 248320 columns); the weight-only GEMMs
(W4A16 g128 and W8A16 g128 / g32 on the decode shapes at 8 and 64 tokens, and the
INT4 / INT8 weight-only vocabulary heads at 1, 8 and 64 tokens); the RMS
normalisation fused with the quantisation; one GPU's share at tensor-parallel size 4
(qkv and gate/up by columns, o_proj and down by K, a quarter of the vocabulary head;
decode and prefill GEMM); the achievable peaks measured in the same
run (a streaming-read kernel and an INT8 MFMA loop, libi8gs_peaks.so); clocks and
software versions; and the CPU oracle on the host cores (the decode step, per layer,
and single-threaded on the single linear and qkv).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W8A8-G128 GEMM: GB/s at decode M=64 + INT8 TOPS at prefill M=4096, % peak"
HBM_PEAK_GBS = 8000.0

# HBM bytes per launch of the decode GEMM kernel on the four layers, from two
# rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE) over `bench.py --traffic-probe`,
# each counter scaled by its own reading for the probe's 256 MiB device copy
# (FETCH_SIZE counts half the bytes read: x2.0; WRITE_SIZE: x1.0).  The figures hold
# for the kernel sources they were taken with, identified by the SHA-256 of the code in
# DECODE_SOURCES (comments and whitespace aside); after any change to that code `traffic`
# is reported as null.
DECODE_SOURCES = ("int8_group_scaled_amd/csrc/w8a8.hip", "int8_group_scaled_amd/csrc/internal.h")
DECODE_TRAFFIC = {
    "sources_sha256": "ac7e56bb4167989302daf04c9747fddf5fb48bb8008b8d7b4e504ace78d4b09d",
    "fetch": {"qkv": 39961920, "o_proj": 26539296, "gate_up": 190730048, "down": 107590336},
    "write": {"qkv": 7085568, "o_proj": 4597760, "gate_up": 4456448, "down": 8528640},
}
EVENT_EVERY = 8  # per-kernel HIP events on every 8th timed step (each event adds a gap)
INT8_PEAK_TOPS = 5000.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prefill-reps", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extras", action="store_true", help="skip prefill and W4A16 figures")
    ap.add_argument("--no-lm-head", action="store_true", help="skip the 248320-column vocabulary heads")
    ap.add_argument("--min-cold-bytes", type=float, default=1.0e9)
    ap.add_argument("--traffic-probe", action="store_true",
                    help="no timing: 4 decode steps plus a 256 MiB device copy (the calibration kernel), for "
                         "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs")
    ap.add_argument("--counter-probe", choices=("prefill", "w4a16"),
                    help="no timing: two launches of each prefill GEMM (M=4096, five layers) or of each W4A16 "
                         "GEMM (M=8 and 64, four decode layers), for rocprofv3 --pmc runs")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def decode_sources_sha256():
    """SHA-256 of the code in DECODE_SOURCES: comments removed and whitespace collapsed,
    so that only a change to the code itself invalidates the stored counters."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def gemm_bytes(M, K, N):
    return K * N + 4 * N * K // 128 + M * K + 4 * M + 2 * M * N


def linear_bytes(M, K, N):
    return K * N + 4 * N * K // 128 + 2 * M * K + 2 * M * N


def w4_bytes(M, K, N):
    return K * N // 2 + 4 * N * K // 128 + 2 * M * K + 2 * M * N


def wo_bytes(M, K, N, bits, group):
    """Weight-only GEMM: codes, fp32 scales, bf16 x in, bf16 y out."""
    return K * N * bits // 8 + 4 * N * K // group + 2 * M * K + 2 * M * N


def environment():
    """Software versions and the GPU clocks (rocm-smi) at the time of the call."""
    import subprocess

    import torch
    env = {"torch": torch.__version__, "hip": torch.version.hip, "device": torch.cuda.get_device_name(0)}
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip()
    except OSError:
        env["rocm"] = None
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        card = next(iter(json.loads(r.stdout).values()))
        env["clocks"] = {k: v for k, v in card.items() if "clock" in k.lower() or k.lower().startswith(("sclk", "mclk", "fclk"))}
    except Exception as e:  # rocm-smi absent or not parseable: report why
        env["clocks"] = f"unavailable ({type(e).__name__})"
    return env


def measured_peaks(torch, dev):
    """Achievable HBM read bandwidth and dense INT8 MFMA rate on this GPU, from the
    in-repo microbenchmarks (libi8gs_peaks.so), timed with HIP events on the current stream."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "int8_group_scaled_amd", "libi8gs_peaks.so"))
    P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.i8gs_peak_stream_read.argtypes = [P, S, P, I, P]
    lib.i8gs_peak_mfma_i8.argtypes = [I, P, I, P]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = cus * 8
    sink = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    nbytes = 4 << 30  # 4 GiB: far beyond the 256 MB last-level cache
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def run(f, reps):
        f()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    t = run(lambda: lib.i8gs_peak_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                              ctypes.c_void_p(sink.data_ptr()), blocks, stream), 5)
    hbm = nbytes / t / 1e9
    del buf
    torch.cuda.empty_cache()
    iters = 4096
    t = run(lambda: lib.i8gs_peak_mfma_i8(iters, ctypes.c_void_p(sink.data_ptr()), blocks, stream), 3)
    tops = blocks * 4 * iters * 4 * 65536 / t / 1e12
    return {"hbm_read_GBps": round(hbm, 1), "int8_mfma_TOPS": round(tops, 1),
            "kernels": "i8gs_peak_stream_read (4 GiB, 16-byte non-temporal loads), "
                       "i8gs_peak_mfma_i8 (4 independent v_mfma_i32_32x32x32_i8 chains per wave)"}


class Timer:
    """HIP events around launches on the current stream, kept until the end of the run."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def mark(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def add(self, key, a, b):
        self.pairs.setdefault(key, []).append((a, b))

    def mean_us(self, key):
        v = [a.elapsed_time(b) * 1e3 for a, b in self.pairs[key]]
        return float(np.mean(v)), float(np.median(v)), len(v)


def spin(torch, ms):
    """Queue roughly `ms` of GPU busy time so the host can run ahead of the device."""
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(int(ms * 1e-3 * 2.4e9))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (sharding is a "
              "design note only); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import int8_group_scaled_amd as i8
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    i8.load_library()
    M = 64
    layers = list(synth.DECODE_LAYERS)

    # ---------------- inputs
    t0 = time.time()
    xs, ys, wsets = [], [], []
    base = []
    for L in layers:
        xb = synth.activations_bf16(0, f"bench-decode-{L.name}", M, L.K, outliers=True)
        xs.append(torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev))
        ys.append(torch.empty((M, L.N), dtype=torch.bfloat16, device=dev))
        w = torch.from_numpy(synth.weights_f32(0, f"bench-decode-{L.name}", L.K, L.N)).to(dev)
        base.append(i8.gptq_quantize_rtn(w, 8))
        del w
    set_bytes = sum(qw.numel() * 4 + ws.numel() * 4 for qw, ws in base)
    nsets = max(2, math.ceil(args.min_cold_bytes / set_bytes))
    wsets.append(base)
    for _ in range(nsets - 1):
        wsets.append([(qw.clone(), ws.clone()) for qw, ws in base])
    qas = [torch.empty((M, L.K), dtype=torch.int8, device=dev) for L in layers]
    scs = [torch.empty((M,), dtype=torch.float32, device=dev) for L in layers]
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s: {nsets} weight sets of {set_bytes / 1e6:.1f} MB")

    timer = Timer(torch)

    if args.counter_probe:
        # Counter runs on the secondary kernels: two launches per layer and size, in order.
        del wsets
        torch.cuda.empty_cache()
        if args.counter_probe == "prefill":
            for L in synth.PREFILL_LAYERS:
                xb = synth.activations_bf16(0, f"bench-prefill-{L.name}", 4096, L.K, outliers=True)
                x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
                w = torch.from_numpy(synth.weights_f32(0, f"bench-prefill-{L.name}", L.K, L.N)).to(dev)
                qw, sc = i8.gptq_quantize_rtn(w, 8)
                qa, s = i8.quant_act_per_token(x)
                y = torch.empty((4096, L.N), dtype=torch.bfloat16, device=dev)
                for _ in range(2):
                    i8.gemm_w8a8_g128(qw, sc, qa=qa, a_scale=s, y=y)
                torch.cuda.synchronize()
                del x, w, qw, sc, qa, s, y
        else:
            for L in layers:
                w = torch.from_numpy(synth.weights_f32(0, f"bench-w4-{L.name}", L.K, L.N)).to(dev)
                qw, sc = i8.gptq_quantize_rtn(w, 4)
                for Mw in (8, 64):
                    xb = synth.activations_bf16(0, f"bench-w4-{L.name}-{Mw}", Mw, L.K, outliers=True)
                    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
                    y = torch.empty((Mw, L.N), dtype=torch.bfloat16, device=dev)
                    for _ in range(2):
                        i8.gemm_w4a16_g128(x, qw, sc, y)
                torch.cuda.synchronize()
                del w, qw, sc
        print(json.dumps({"counter_probe": args.counter_probe}), flush=True)
        return

    if args.traffic_probe:
        # Counter runs: a plain copy of known size first (its FETCH_SIZE / WRITE_SIZE give
        # the counters' scale), then 4 decode steps in layer order qkv, o_proj, gate_up, down.
        copy_bytes = 256 << 20
        src = torch.empty(copy_bytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        for i in range(4):
            ws = wsets[i % nsets]
            for li, L in enumerate(layers):
                qw, sc = ws[li]
                i8.gemm_w8a8_g128(qw, sc, qa=qas[li], a_scale=scs[li], y=ys[li])
        torch.cuda.synchronize()
        print(json.dumps({"traffic_probe": True, "copy_bytes": copy_bytes,
                          "gemm_bytes": {L.name: gemm_bytes(M, L.K, L.N) for L in layers}}), flush=True)
        return

    def step(i, timed):
        ws = wsets[i % nsets]
        for li, L in enumerate(layers):
            qw, sc = ws[li]
            if timed:
                e0 = timer.mark()
            i8.quant_act_per_token(xs[li], qas[li], scs[li])
            if timed:
                e1 = timer.mark()
            i8.gemm_w8a8_g128(qw, sc, qa=qas[li], a_scale=scs[li], y=ys[li])
            if timed:
                e2 = timer.mark()
                timer.add(("quant", L.name), e0, e1)
                timer.add(("gemm", L.name), e1, e2)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    spin(torch, 20 + 0.15 * args.steps)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        step(args.warmup + i, i % EVENT_EVERY == 0)
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps

    step_bytes = sum(linear_bytes(M, L.K, L.N) for L in layers)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    per_layer = {}
    g_bytes = g_us = 0.0
    for L in layers:
        gm, gmed, n = timer.mean_us(("gemm", L.name))
        qm, _, _ = timer.mean_us(("quant", L.name))
        b = gemm_bytes(M, L.K, L.N)
        g_bytes += b
        g_us += gm
        per_layer[L.name] = {"K": L.K, "N": L.N, "gemm_us": round(gm, 3), "gemm_us_median": round(gmed, 3),
                             "quant_us": round(qm, 3), "gemm_GBps": round(b / (gm * 1e-6) / 1e9, 1),
                             "gemm_frac_hbm": round(b / (gm * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    achieved = g_bytes / (g_us * 1e-6) / 1e9
    # Cross-check without an event around every launch: per layer, 32 back-to-back GEMM
    # launches (weight sets rotated, so still read from HBM) between two events.  The
    # difference to gemm_us is the dispatch time an event pair brackets.
    for li, L in enumerate(layers):
        torch.cuda.synchronize()
        spin(torch, 2)
        e0 = timer.mark()
        for r in range(32):
            qw, sc = wsets[r % nsets][li]
            i8.gemm_w8a8_g128(qw, sc, qa=qas[li], a_scale=scs[li], y=ys[li])
        e1 = timer.mark()
        timer.add(("b2b", L.name), e0, e1)
        torch.cuda.synchronize()
        per_layer[L.name]["gemm_us_back_to_back"] = round(timer.mean_us(("b2b", L.name))[0] / 32, 3)
    b2b_us = sum(per_layer[L.name]["gemm_us_back_to_back"] for L in layers)
    log(f"decode step {ms_per_step * 1e3:.1f} us, {value:.0f} GB/s; GEMM kernels {achieved:.0f} GB/s "
        f"(back to back: " + ", ".join(f"{L.name} {per_layer[L.name]['gemm_us_back_to_back']:.1f}" for L in layers)
        + " us)")
    traffic = None
    if decode_sources_sha256() == DECODE_TRAFFIC["sources_sha256"]:
        traffic = round(sum(DECODE_TRAFFIC["fetch"][L.name] + DECODE_TRAFFIC["write"][L.name] for L in layers)
                        / len(layers))
    else:
        log("decode kernel sources differ from those the traffic counters were taken with: traffic = null")

    # Context for the roofline: what a plain device-to-device copy reaches on this GPU
    # (read + write bytes over time, 1 GiB each way), outside the timed region.
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * 5 * src.numel() / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": "decode M=64 (8 seqs x block 8), W8A8 G128 linear from bf16 x: "
                               "qkv 5120->6144, o_proj 4096->5120, gate_up 5120->34816, down 17408->5120",
                   "M": M, "layers": [[L.name, L.K, L.N] for L in layers], "weights": "N(0,0.02) RTN G128 sym",
                   "activations": "bf16 N(0,1), 1% channels x20", "cold_weight_sets": nsets,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "w8a8_decode_kernel", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "traffic_unit": "bytes per launch (mean of the 4 layers; FETCH_SIZE x2.0 + WRITE_SIZE x1.0)",
                     "bytes_per_launch": "K*N + 4*N*K/128 + M*K + 4*M + 2*M*N (mean of the 4 layers: %d)"
                                         % int(g_bytes / len(layers)),
                     "avg_launch_us": round(g_us / len(layers), 3),
                     "measured_copy_GBps": round(copy_gbs, 1),
                     "frac_of_measured_copy": round(achieved / copy_gbs, 4),
                     # the same bytes over the back-to-back launch times (no event between two
                     # kernels: close to the kernel trace's durations)
                     "achieved_back_to_back": round(g_bytes / (b2b_us * 1e-6) / 1e9, 1),
                     "frac_back_to_back": round(g_bytes / (b2b_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "per_layer": per_layer,
    }

    # ---------------- prefill (secondary)
    if not args.no_extras:
        del wsets
        torch.cuda.empty_cache()
        pre = {}
        tot_ops = tot_us = 0.0
        Mp = 4096
        for L in synth.PREFILL_LAYERS:
            xb = synth.activations_bf16(0, f"bench-prefill-{L.name}", Mp, L.K, outliers=True)
            x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
            w = torch.from_numpy(synth.weights_f32(0, f"bench-prefill-{L.name}", L.K, L.N)).to(dev)
            qw, sc = i8.gptq_quantize_rtn(w, 8)
            del w
            qa, s = i8.quant_act_per_token(x)
            y = torch.empty((Mp, L.N), dtype=torch.bfloat16, device=dev)
            for _ in range(3):
                i8.gemm_w8a8_g128(qw, sc, qa=qa, a_scale=s, y=y)
            torch.cuda.synchronize()
            spin(torch, 5)
            for _ in range(args.prefill_reps):
                e0 = timer.mark()
                i8.quant_act_per_token(x, qa, s)
                e1 = timer.mark()
                i8.gemm_w8a8_g128(qw, sc, qa=qa, a_scale=s, y=y)
                e2 = timer.mark()
                timer.add(("pquant", L.name), e0, e1)
                timer.add(("pgemm", L.name), e1, e2)
            torch.cuda.synchronize()
            gm, gmed, _ = timer.mean_us(("pgemm", L.name))
            qm, _, _ = timer.mean_us(("pquant", L.name))
            ops = 2.0 * Mp * L.N * L.K
            tot_ops += ops
            tot_us += gm
            pre[L.name] = {"K": L.K, "N": L.N, "gemm_us": round(gm, 2), "TOPS": round(ops / (gm * 1e-6) / 1e12, 1),
                           "frac_int8_peak": round(ops / (gm * 1e-6) / 1e12 / INT8_PEAK_TOPS, 4),
                           "quant_us": round(qm, 2)}
            del x, qw, sc, qa, s, y
            torch.cuda.empty_cache()
        tops = tot_ops / (tot_us * 1e-6) / 1e12
        out["prefill"] = {"M": Mp, "TOPS": round(tops, 1), "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4),
                          "kernel": "w8a8_prefill_kernel", "per_layer": pre}
        log(f"prefill GEMMs {tops:.0f} TOP/s ({tops / INT8_PEAK_TOPS:.1%} of dense INT8 peak)")

        # ---------------- W4A16 g128 on the decode shapes (secondary)
        w4 = {}
        for L in layers:
            w = torch.from_numpy(synth.weights_f32(0, f"bench-w4-{L.name}", L.K, L.N)).to(dev)
            qw, sc = i8.gptq_quantize_rtn(w, 4)
            del w
            reps = max(2, math.ceil(args.min_cold_bytes / (qw.numel() * 4)))
            copies = [(qw, sc)] + [(qw.clone(), sc.clone()) for _ in range(reps - 1)]
            for Mw in (8, 64):
                xb = synth.activations_bf16(0, f"bench-w4-{L.name}-{Mw}", Mw, L.K, outliers=True)
                x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
                y = torch.empty((Mw, L.N), dtype=torch.bfloat16, device=dev)
                for c in copies[:2]:
                    i8.gemm_w4a16_g128(x, c[0], c[1], y)
                torch.cuda.synchronize()
                spin(torch, 5)
                for r in range(50):
                    c = copies[r % len(copies)]
                    e0 = timer.mark()
                    i8.gemm_w4a16_g128(x, c[0], c[1], y)
                    e1 = timer.mark()
                    timer.add(("w4", L.name, Mw), e0, e1)
                torch.cuda.synchronize()
                gm, _, _ = timer.mean_us(("w4", L.name, Mw))
                b = w4_bytes(Mw, L.K, L.N)
                # bf16 MFMA work: 2*M*N*K useful flops (the 16-row tiles pad M = 8 to 16)
                tfl = 2.0 * Mw * L.N * L.K / (gm * 1e-6) / 1e12
                w4[f"{L.name}_M{Mw}"] = {"us": round(gm, 3), "GBps": round(b / (gm * 1e-6) / 1e9, 1),
                                         "frac_hbm": round(b / (gm * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                         "bf16_TFLOPS": round(tfl, 1),
                                         "frac_bf16_peak": round(tfl / BF16_PEAK_TFLOPS, 4)}
            del copies, qw, sc
            torch.cuda.empty_cache()
        out["w4a16"] = w4

    def timed(key, calls, reps):
        """Average event-timed duration (us) of reps launches, cycling through calls."""
        for c in calls[:2]:
            c()
        torch.cuda.synchronize()
        spin(torch, 5)
        for r in range(reps):
            e0 = timer.mark()
            calls[r % len(calls)]()
            e1 = timer.mark()
            timer.add(key, e0, e1)
        torch.cuda.synchronize()
        return timer.mean_us(key)[0]

    def cold_copies(t_pair, nbytes):
        reps = max(2, math.ceil(args.min_cold_bytes / nbytes))
        return [t_pair] + [tuple(t.clone() for t in t_pair) for _ in range(reps - 1)]

    if not args.no_extras:
        # ---------------- W8A16 (weight-only INT8) at group 128 and 32 on the decode shapes
        w8 = {}
        for L in layers:
            w = torch.from_numpy(synth.weights_f32(0, f"bench-w8-{L.name}", L.K, L.N)).to(dev)
            for group in (128, 32):
                qw, sc = i8.gptq_quantize_rtn_group(w, 8, group)
                copies = cold_copies((qw, sc), qw.numel() * 4)
                for Mw in (8, 64):
                    xb = synth.activations_bf16(0, f"bench-w8-{L.name}-{Mw}", Mw, L.K, outliers=True)
                    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
                    y = torch.empty((Mw, L.N), dtype=torch.bfloat16, device=dev)
                    calls = [lambda c=c: i8.gemm_weight_only(x, c[0], c[1], 8, group, y) for c in copies]
                    gm = timed(("w8", L.name, group, Mw), calls, 50)
                    b = wo_bytes(Mw, L.K, L.N, 8, group)
                    w8[f"{L.name}_g{group}_M{Mw}"] = {"us": round(gm, 3), "GBps": round(b / (gm * 1e-6) / 1e9, 1),
                                                      "frac_hbm": round(b / (gm * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
                del copies, qw, sc
            del w
            torch.cuda.empty_cache()
        out["w8a16"] = w8

        # ---------------- RMS normalisation fused with the quantisation (decode: 64 x 5120)
        xb = synth.activations_bf16(0, "bench-rms", M, 5120, outliers=True)
        x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
        gamma = torch.ones(5120, dtype=torch.bfloat16, device=dev)
        qa_b = torch.empty((M, 5120), dtype=torch.int8, device=dev)
        s_b = torch.empty((M,), dtype=torch.float32, device=dev)
        us_f = timed(("rmsq",), [lambda: i8.rmsnorm_quant_per_token(x, gamma, 1e-6, qa=qa_b, a_scale=s_b)], 50)
        us_q = timed(("q5120",), [lambda: i8.quant_act_per_token(x, qa_b, s_b)], 50)
        out["rmsnorm_quant"] = {"M": M, "K": 5120, "fused_us": round(us_f, 3), "quant_only_us": round(us_q, 3),
                                "bytes": 2 * M * 5120 + 2 * 5120 + M * 5120 + 4 * M,
                                "note": "one launch per layer input in place of a normalisation kernel "
                                        "followed by the quantisation kernel"}

    if not args.no_extras:
        # ---------------- INT8 block-g128 KV cache: codec, QK and PV for one block of 8 draft
        # queries (32 query heads over 8 KV heads) against a 2048-token window and a 32768-token
        # context; inputs cycle through cold copies
        kv = {}
        Hq, Hkv, Mq = 32, 8, 8
        for T in (2048, 32768):
            kb = torch.from_numpy(synth.activations_bf16(0, f"bench-k{T}", T * Hkv, 128, True).view(np.int16)) \
                .view(torch.bfloat16).reshape(T, Hkv, 128).to(dev)
            qb = torch.from_numpy(synth.activations_bf16(0, f"bench-q{T}", Mq * Hq, 128, True).view(np.int16)) \
                .view(torch.bfloat16).reshape(Mq, Hq, 128).to(dev)
            kq, ks = i8.kv_quant_int8_block128(kb)
            qq, qs = i8.kv_quant_int8_block128(qb)
            codes_b = T * Hkv * (256 + 128 + 4)
            us_c = timed(("kvq", T), [lambda c=c: i8.kv_quant_int8_block128(c[0], codes=kq, scales=ks)
                                      for c in cold_copies((kb,), codes_b)], 50)
            sc = torch.empty((Hq, Mq, T), dtype=torch.float32, device=dev)
            qk_b = Mq * Hq * 132 + T * Hkv * 132 + Hq * Mq * T * 4
            us_qk = timed(("qk", T), [lambda c=c: i8.attn_qk_int8(qq, qs, c[0], c[1], 128 ** -0.5, s=sc)
                                      for c in cold_copies((kq, ks), qk_b)], 50)
            p = torch.softmax(sc, dim=2)
            o = torch.empty((Hq, Mq, 128), dtype=torch.float32, device=dev)
            pv_b = Hq * Mq * T * 4 + T * Hkv * 132 + Hq * Mq * 128 * 4
            us_pv = timed(("pv", T), [lambda c=c: i8.attn_pv_int8(c[0], c[1], c[2], out=o)
                                      for c in cold_copies((p, kq, ks), pv_b)], 50)
            for name, us, b in (("codec", us_c, codes_b), ("qk", us_qk, qk_b), ("pv", us_pv, pv_b)):
                kv[f"{name}_T{T}"] = {"us": round(us, 3), "bytes": b, "GBps": round(b / (us * 1e-6) / 1e9, 1),
                                      "frac_hbm": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            del kb, qb, kq, ks, qq, qs, sc, p, o
            torch.cuda.empty_cache()
        kv["shape"] = {"Mq": Mq, "Hq": Hq, "Hkv": Hkv, "head_dim": 128}
        out["kv_int8"] = kv
        log("kv int8: " + ", ".join(f"{k} {v['us']:.1f} us" for k, v in kv.items() if "us" in v))

    if not args.no_lm_head:
        # ---------------- vocabulary heads: 248320 columns (naturally cold: 0.64-1.27 GB of codes)
        L = synth.LAYERS["lm_head"]
        heads = {}
        w = torch.from_numpy(synth.weights_f32(0, "bench-lm", L.K, L.N)).to(dev)
        qw, sc = i8.gptq_quantize_rtn(w, 8)
        xb = synth.activations_bf16(0, "bench-lm", M, L.K, outliers=False)
        x64 = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
        qa, s = i8.quant_act_per_token(x64)
        y = torch.empty((M, L.N), dtype=torch.bfloat16, device=dev)
        gm = timed(("lm",), [lambda: i8.gemm_w8a8_g128(qw, sc, qa=qa, a_scale=s, y=y)], 20)
        b = gemm_bytes(M, L.K, L.N)
        heads["w8a8_M64"] = {"us": round(gm, 2), "GBps": round(b / (gm * 1e-6) / 1e9, 1),
                             "frac_hbm": round(b / (gm * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                             "kernel": "w8a8_decode_kernel"}
        out["lm_head"] = heads["w8a8_M64"]
        for bits in (4, 8):
            qw2, sc2 = (i8.gptq_quantize_rtn(w, 4) if bits == 4 else (qw, sc))
            for Mw in (1, 8, 64):
                xw = x64[:Mw].contiguous()
                yw = torch.empty((Mw, L.N), dtype=torch.bfloat16, device=dev)
                gm = timed(("lmw", bits, Mw), [lambda: i8.gemm_weight_only(xw, qw2, sc2, bits, 128, yw)], 20)
                b = wo_bytes(Mw, L.K, L.N, bits, 128)
                heads[f"w{bits}a16_M{Mw}"] = {"us": round(gm, 2), "GBps": round(b / (gm * 1e-6) / 1e9, 1),
                                              "frac_hbm": round(b / (gm * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            del qw2, sc2
        out["vocab_heads"] = heads
        del w, qw, sc, x64, qa, s, y
        torch.cuda.empty_cache()
        log(f"vocabulary heads: " + ", ".join(f"{k} {v['GBps']:.0f} GB/s" for k, v in heads.items()))

    if not args.no_extras:
        # ---------------- one GPU's share at tensor-parallel size 4: the decode (64 tokens) and
        # prefill (4096 tokens) GEMM on the shard shapes, pre-quantised activations, cold weights
        shards = {}
        for L in synth.SHARD_LAYERS + (synth.LAYERS["lm_head_tp4"],):
            w = torch.from_numpy(synth.weights_f32(0, f"bench-tp4-{L.name}", L.K, L.N)).to(dev)
            qw, sc = i8.gptq_quantize_rtn(w, 8)
            del w
            copies = cold_copies((qw, sc), qw.numel() * 4)
            e = {"K": L.K, "N": L.N}
            for Ms in ((64,) if L.name == "lm_head_tp4" else (64, 4096)):
                xb = synth.activations_bf16(0, f"bench-tp4-{L.name}-{Ms}", Ms, L.K, outliers=True)
                x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
                qa, s = i8.quant_act_per_token(x)
                y = torch.empty((Ms, L.N), dtype=torch.bfloat16, device=dev)
                calls = [lambda c=c: i8.gemm_w8a8_g128(c[0], c[1], qa=qa, a_scale=s, y=y) for c in copies]
                gm = timed(("tp4", L.name, Ms), calls, 50 if Ms == 64 else 10)
                if Ms == 64:
                    b = gemm_bytes(Ms, L.K, L.N)
                    e.update(decode_us=round(gm, 3), decode_GBps=round(b / (gm * 1e-6) / 1e9, 1),
                             decode_frac_hbm=round(b / (gm * 1e-6) / 1e9 / HBM_PEAK_GBS, 4))
                else:
                    tops = 2.0 * Ms * L.N * L.K / (gm * 1e-6) / 1e12
                    e.update(prefill_us=round(gm, 2), prefill_TOPS=round(tops, 1),
                             prefill_frac_int8_peak=round(tops / INT8_PEAK_TOPS, 4))
                del x, qa, s, y, calls
            shards[L.name] = e
            del copies, qw, sc
            torch.cuda.empty_cache()
        out["tp4_shard"] = shards
        log("tensor-parallel-4 shards: " + ", ".join(
            f"{k} {v['decode_GBps']:.0f} GB/s" + (f" / {v['prefill_TOPS']:.0f} TOP/s" if "prefill_TOPS" in v else "")
            for k, v in shards.items()))

    # ---------------- measured ceilings and environment
    peaks = measured_peaks(torch, dev)
    out["measured_peaks"] = peaks
    out["roofline"]["measured_peak"] = peaks["hbm_read_GBps"]
    out["roofline"]["frac_of_measured_peak"] = round(achieved / peaks["hbm_read_GBps"], 4)
    if "prefill" in out:
        out["prefill"]["measured_peak_TOPS"] = peaks["int8_mfma_TOPS"]
        out["prefill"]["frac_of_measured_peak"] = round(out["prefill"]["TOPS"] / peaks["int8_mfma_TOPS"], 4)
    out["environment"] = environment()
    log(f"measured peaks: {peaks['hbm_read_GBps']:.0f} GB/s HBM read, {peaks['int8_mfma_TOPS']:.0f} TOP/s INT8 MFMA")

    # ---------------- CPU oracle baseline (rank 0, N=1 only)
    if not args.no_cpu:
        import oracle

        oracle.build(force=False)
        host = []
        for L in layers:
            xb = synth.activations_bf16(0, f"bench-decode-{L.name}", M, L.K, outliers=True)
            w = synth.weights_f32(0, f"bench-decode-{L.name}", L.K, L.N)
            qw, sc = oracle.gptq_quantize_rtn(w, 8)
            host.append((xb, qw, sc, L))

        def oracle_linear(xb, qw, sc, L):
            qa, s = oracle.quant_act_per_token(xb)
            q = oracle.gptq_unpack(qw, 8, L.K)
            yex, _ = oracle.gemm_w8a8_g128(qa, s, q, sc)
            oracle.bf16_from_double(yex)

        per = {L.name: 0.0 for L in layers}
        reps = 0
        t0 = time.perf_counter()
        while True:
            for xb, qw, sc, L in host:
                ta = time.perf_counter()
                oracle_linear(xb, qw, sc, L)
                per[L.name] += time.perf_counter() - ta
            reps += 1
            el = time.perf_counter() - t0
            if el >= 10.0 or reps >= 50:
                break
        cpu_gbs = step_bytes * reps / el / 1e9
        threads = oracle.num_threads()
        per_layer_cpu = {L.name: round(linear_bytes(M, L.K, L.N) * reps / per[L.name] / 1e9, 3) for L in layers}
        # single-threaded: the single linear (8 x 512 x 256) and the decode qkv layer
        oracle.set_num_threads(1)
        xs = synth.activations_bf16(0, "bench-single", 8, 512, outliers=False)
        qws, scs = oracle.gptq_quantize_rtn(synth.weights_f32(0, "bench-single", 512, 256), 8)
        single = synth.LAYERS["single"]
        ta = time.perf_counter()
        n_single = 0
        while time.perf_counter() - ta < 1.0:
            oracle_linear(xs, qws, scs, single)
            n_single += 1
        t_single = (time.perf_counter() - ta) / n_single
        xb, qw, sc, L = host[0]
        ta = time.perf_counter()
        oracle_linear(xb, qw, sc, L)
        t_qkv = time.perf_counter() - ta
        oracle.set_num_threads(threads)
        # prefill: the qkv layer at M = 4096, exact group sums and fold for 64 sampled rows
        PL = synth.LAYERS["qkv"]
        qa_p = np.maximum(synth.uniform_words(0, "bench-prefill-cpu", 4096 * PL.K // 4).view(np.int8), -127)
        qa_p = qa_p.reshape(4096, PL.K)
        s_p = np.abs(synth.normal_f32(0, "bench-prefill-cpu-s", 4096)) + 1e-3
        q_p = oracle.gptq_unpack(host[0][1], 8, PL.K)
        rows_p = synth.sample_rows(0, "bench-prefill-cpu", 4096, 64)
        ta = time.perf_counter()
        oracle.gemm_w8a8_g128(qa_p, s_p, q_p, host[0][2], rows=rows_p)
        t_pf = time.perf_counter() - ta
        pf_tops = 2.0 * len(rows_p) * PL.N * PL.K / t_pf / 1e12
        out["cpu_baseline"] = {"value": round(cpu_gbs, 3), "unit": "GB/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"the full decode step (64 tokens x 4 layers: quantise, unpack, exact "
                                         f"group sums, fold, bf16) repeated {reps}x in {el:.1f}s",
                               "per_layer_GBps": per_layer_cpu,
                               "single_thread": {"single_linear_8x512x256_ms": round(t_single * 1e3, 3),
                                                 "qkv_64x5120x6144_s": round(t_qkv, 3)},
                               "prefill_TOPS": round(pf_tops, 4),
                               "prefill_sample": f"qkv 5120->6144 at M=4096, 64 sampled rows (exact group sums "
                                                 f"and fold, {threads} threads) in {t_pf:.2f}s"}
        log(f"cpu oracle: {cpu_gbs:.2f} GB/s on {threads} threads; single thread: single linear "
            f"{t_single * 1e3:.2f} ms, qkv {t_qkv:.2f} s; prefill sample {pf_tops:.3f} TOP/s")

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
