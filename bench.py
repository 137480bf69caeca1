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
Secondary figures: prefill (4096 tokens, five layers, GEMM kernel on
pre-quantised activations) in TOP/s against the 5.0 POP/s dense INT8 peak, the
W4A16 g128 sibling on the decode shapes, and the CPU oracle on the host cores.
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
DECODE_SOURCES = ("int8_group_scaled_amd/csrc/w8a8.hip", "int8_group_scaled_amd/csrc/internal.h", "include/i8gs.h")
DECODE_TRAFFIC = {
    "sources_sha256": "84a9eb0eea502d269f5604bcde36860788df78a2f63b532cdf897a2b3465c55b",
    "fetch": {"qkv": 36814661, "o_proj": 26535249, "gate_up": 192737799, "down": 107581243},
    "write": {"qkv": 3941376, "o_proj": 4597760, "gate_up": 4456544, "down": 8528640},
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
    ap.add_argument("--lm-head", action="store_true", help="also time the 248320-column INT8 vocabulary head")
    ap.add_argument("--min-cold-bytes", type=float, default=1.0e9)
    ap.add_argument("--traffic-probe", action="store_true",
                    help="no timing: 4 decode steps plus a 256 MiB device copy (the calibration kernel), for "
                         "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs")
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
    log(f"decode step {ms_per_step * 1e3:.1f} us, {value:.0f} GB/s; GEMM kernels {achieved:.0f} GB/s")
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
                     "frac_of_measured_copy": round(achieved / copy_gbs, 4)},
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
                w4[f"{L.name}_M{Mw}"] = {"us": round(gm, 3), "GBps": round(b / (gm * 1e-6) / 1e9, 1),
                                         "frac_hbm": round(b / (gm * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            del copies, qw, sc
            torch.cuda.empty_cache()
        out["w4a16"] = w4

    if args.lm_head:
        L = synth.LAYERS["lm_head"]
        xb = synth.activations_bf16(0, "bench-lm", M, L.K, outliers=False)
        x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
        w = torch.from_numpy(synth.weights_f32(0, "bench-lm", L.K, L.N)).to(dev)
        qw, sc = i8.gptq_quantize_rtn(w, 8)
        del w
        qa, s = i8.quant_act_per_token(x)
        y = torch.empty((M, L.N), dtype=torch.bfloat16, device=dev)
        i8.gemm_w8a8_g128(qw, sc, qa=qa, a_scale=s, y=y)
        torch.cuda.synchronize()
        for _ in range(20):
            e0 = timer.mark()
            i8.gemm_w8a8_g128(qw, sc, qa=qa, a_scale=s, y=y)
            e1 = timer.mark()
            timer.add(("lm",), e0, e1)
        torch.cuda.synchronize()
        gm, _, _ = timer.mean_us(("lm",))
        b = gemm_bytes(M, L.K, L.N)
        out["lm_head"] = {"us": round(gm, 2), "GBps": round(b / (gm * 1e-6) / 1e9, 1),
                          "frac_hbm": round(b / (gm * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}

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
        reps = 0
        t0 = time.perf_counter()
        while True:
            for xb, qw, sc, L in host:
                qa, s = oracle.quant_act_per_token(xb)
                q = oracle.gptq_unpack(qw, 8, L.K)
                yex, _ = oracle.gemm_w8a8_g128(qa, s, q, sc)
                oracle.bf16_from_double(yex)
            reps += 1
            el = time.perf_counter() - t0
            if el >= 10.0 or reps >= 50:
                break
        cpu_gbs = step_bytes * reps / el / 1e9
        out["cpu_baseline"] = {"value": round(cpu_gbs, 3), "unit": "GB/s", "cores": oracle.num_threads(),
                               "kind": "oracle",
                               "sample": f"the full decode step (64 tokens x 4 layers: quantise, unpack, exact "
                                         f"group sums, fold, bf16) repeated {reps}x in {el:.1f}s"}
        log(f"cpu oracle: {cpu_gbs:.2f} GB/s on {oracle.num_threads()} threads")

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
