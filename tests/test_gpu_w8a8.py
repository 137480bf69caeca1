"""GPU parity of the W8A8 G128 GEMM: per-group int32 partials bit-exact, bf16
outputs within the tolerance in parity.py, on the workloads' layer shapes (in
the launch configuration the benchmark times) and on ragged edge cases."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import int8_group_scaled_amd as i8
import oracle
import synth
from parity import assert_within_tolerance, dev, dev_bf16, host_bf16_bits, rtn_weights, unpacked

pytestmark = pytest.mark.gpu


def _case(seed, tag, M, K, N, outliers):
    xb = synth.activations_bf16(seed, tag, M, K, outliers)
    qw, ws = rtn_weights(seed, tag, K, N, 8)
    return xb, qw, ws


# Partials come from the kernel that serves the same call: the decode kernel for M <= 64,
# the 256 x 256 prefill kernel above (AUTO), or the 128 x 128 tiled kernel when asked for.
KERNELS = {"auto": i8.KERNEL_AUTO, "decode": i8.KERNEL_DECODE, "tiled": i8.KERNEL_TILED}


@pytest.mark.parametrize("M,K,N,kern", [
    (8, 512, 256, "auto"), (8, 512, 256, "tiled"),          # the single linear
    (1, 128, 8, "auto"), (33, 384, 72, "auto"), (64, 1024, 520, "auto"),
    (100, 384, 72, "auto"), (100, 384, 72, "tiled"),        # prefill kernel, ragged tile
    (300, 4096, 520, "auto"),                               # 6 tiles, K split 2 ways in the last round
    (600, 2048, 264, "auto"),                               # 6 tiles, split 2 ways
])
def test_group_partials_bit_exact(M, K, N, kern):
    xb, qw, _ = _case(0, f"p{M}-{K}-{N}", M, K, N, True)
    qa, _ = oracle.quant_act_per_token(xb)
    P = i8.gemm_w8a8_g128_group_partials(dev(qa), dev(qw), kernel=KERNELS[kern])
    torch.cuda.synchronize()
    assert np.array_equal(P.cpu().numpy(), oracle.group_partials(qa, oracle.gptq_unpack(qw, 8, K)))


@pytest.mark.parametrize("wgs", [1, 3, 7, 97, 256, 10000])
def test_group_partials_decode_splits(wgs):
    """The decode kernel's tiles and K splits for every grid size write the same exact sums."""
    M, K, N = 64, 5120, 512
    xb, qw, _ = _case(2, "splits", M, K, N, True)
    qa, _ = oracle.quant_act_per_token(xb)
    P = i8.gemm_w8a8_g128_group_partials(dev(qa), dev(qw), kernel=i8.KERNEL_DECODE, decode_workgroups=wgs)
    torch.cuda.synchronize()
    assert np.array_equal(P.cpu().numpy(), oracle.group_partials(qa, oracle.gptq_unpack(qw, 8, K)))


@pytest.mark.parametrize("M,K,N,kern", [(48, 1024, 96, "auto"), (48, 1024, 96, "tiled"), (5, 256, 40, "auto"),
                                        (300, 4096, 520, "auto"), (257, 640, 264, "auto")])
def test_group_partials_full_code_range(M, K, N, kern):
    """Uniformly random codes (all 256, including q = -128) and random activation codes in
    [-127, 127], through the decode kernel (M <= 64), the prefill kernel with split tiles
    (M > 64) and the tiled kernel."""
    words = synth.uniform_words(5, f"pcodes{M}-{K}-{N}", (K // 4) * N).reshape(K // 4, N)
    qa = (synth.uniform_words(5, f"pqa{M}-{K}-{N}", M * K // 4).view(np.uint8).reshape(M, K).astype(np.int16) - 128)
    qa = np.clip(qa, -127, 127).astype(np.int8)
    q = oracle.gptq_unpack(words, 8, K)
    assert (q == -128).any() and (q == 127).any()
    P = i8.gemm_w8a8_g128_group_partials(dev(qa), dev(words), kernel=KERNELS[kern])
    torch.cuda.synchronize()
    assert np.array_equal(P.cpu().numpy(), oracle.group_partials(qa, q))


def test_group_partials_extreme_sums():
    """Rows of +-127 against columns of codes 0 and 255 (q = -128 and 127): group sums at the
    ends of their range, +-127*128*128 = +-2080768, through the decode kernel's seeded
    accumulator and the prefill kernel."""
    K, N = 512, 64
    q = np.full((K, N), 127, np.int16)
    q[:, ::2] = -128
    codes = (q + 128).astype(np.uint32).reshape(K // 4, 4, N)
    words = (codes[:, 0] | (codes[:, 1] << 8) | (codes[:, 2] << 16) | (codes[:, 3] << 24)).view(np.int32)
    for M in (64, 300):
        qa = np.full((M, K), 127, np.int8)
        qa[1::2] = -127
        P = i8.gemm_w8a8_g128_group_partials(dev(qa), dev(words))
        torch.cuda.synchronize()
        ref = oracle.group_partials(qa, oracle.gptq_unpack(words, 8, K))
        assert ref.max() == 127 * 128 * 128 and ref.min() == -127 * 128 * 128
        assert np.array_equal(P.cpu().numpy(), ref)


@pytest.mark.parametrize("layer", ["qkv", "o_proj", "gate_up", "down"])
def test_group_partials_decode_layer(layer):
    """Decode workload: the exact group sums of all 64 tokens x every column, from the decode
    kernel in the launch plan the benchmark times."""
    L = synth.LAYERS[layer]
    M = 64
    xb, qw, _ = _case(0, f"decode-{layer}", M, L.K, L.N, True)
    qa, _ = oracle.quant_act_per_token(xb)
    P = i8.gemm_w8a8_g128_group_partials(dev(qa), dev(qw))
    torch.cuda.synchronize()
    assert np.array_equal(P.cpu().numpy(), oracle.group_partials(qa, unpacked(0, f"decode-{layer}", L.K, L.N, 8)))


@pytest.mark.parametrize("layer", ["qkv", "o_proj", "gate_up", "down"])
def test_decode_layer(layer):
    """Decode workload: 64 tokens through each drafter linear, full output, from bf16 x."""
    L = synth.LAYERS[layer]
    M = 64
    xb, qw, ws = _case(0, f"decode-{layer}", M, L.K, L.N, True)
    y = i8.gemm_w8a8_g128(dev(qw), dev(ws), x=dev_bf16(xb))
    torch.cuda.synchronize()
    qa, s = oracle.quant_act_per_token(xb)
    y_exact, T = oracle.gemm_w8a8_g128(qa, s, unpacked(0, f"decode-{layer}", L.K, L.N, 8), ws)
    beyond, maxulp = assert_within_tolerance(host_bf16_bits(y), y_exact, T, L.K, what=f"decode {layer}")
    print(f"decode {layer}: {beyond} of {y_exact.size} beyond a bare ulp, max {maxulp:.3f} ulp")


def test_single_linear_both_modes():
    M, K, N = 8, 512, 256
    xb, qw, ws = _case(0, "single", M, K, N, False)
    qa, s = oracle.quant_act_per_token(xb)
    y_exact, T = oracle.gemm_w8a8_g128(qa, s, oracle.gptq_unpack(qw, 8, K), ws)
    y1 = i8.gemm_w8a8_g128(dev(qw), dev(ws), x=dev_bf16(xb))
    y2 = i8.gemm_w8a8_g128(dev(qw), dev(ws), qa=dev(qa), a_scale=dev(s))
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(y1), host_bf16_bits(y2))
    assert_within_tolerance(host_bf16_bits(y1), y_exact, T, K, what="single")


@pytest.mark.parametrize("M,K,N", [
    (1, 128, 8), (17, 384, 40), (63, 1024, 264), (64, 256, 520), (65, 640, 136), (100, 1152, 200), (3, 17408, 64),
    (65, 4096, 8), (100, 8192, 200),
])
def test_ragged_shapes(M, K, N):
    xb, qw, ws = _case(1, f"rag{M}-{K}-{N}", M, K, N, True)
    qa, s = oracle.quant_act_per_token(xb)
    y_exact, T = oracle.gemm_w8a8_g128(qa, s, oracle.gptq_unpack(qw, 8, K), ws)
    y = i8.gemm_w8a8_g128(dev(qw), dev(ws), x=dev_bf16(xb))
    torch.cuda.synchronize()
    assert_within_tolerance(host_bf16_bits(y), y_exact, T, K, what=f"ragged {M}x{K}x{N}")


@pytest.mark.parametrize("wgs", [1, 2, 3, 7, 40, 97, 256, 10000])
def test_decode_workgroup_counts(wgs):
    """Every stream-K grid size gives an in-tolerance result, and repeating a call is bitwise identical."""
    M, K, N = 64, 5120, 512
    xb, qw, ws = _case(2, "splits", M, K, N, True)
    qa, s = oracle.quant_act_per_token(xb)
    y_exact, T = oracle.gemm_w8a8_g128(qa, s, oracle.gptq_unpack(qw, 8, K), ws)
    args = (dev(qw), dev(ws))
    ya = i8.gemm_w8a8_g128_ex(*args, x=dev_bf16(xb), kernel=i8.KERNEL_DECODE, decode_workgroups=wgs)
    yb = i8.gemm_w8a8_g128_ex(*args, x=dev_bf16(xb), kernel=i8.KERNEL_DECODE, decode_workgroups=wgs)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(ya), host_bf16_bits(yb))
    assert_within_tolerance(host_bf16_bits(ya), y_exact, T, K, what=f"{wgs} workgroups")


@pytest.mark.parametrize("N,wgs", [(4096, 2), (2048, 1), (1000, 1)])
def test_decode_short_chunks(N, wgs):
    """One group per chunk (K = 128) and tiles of several chunks: the first chunk ends right after
    the first stage, so the row scales must already be in LDS then."""
    M, K = 64, 128
    xb, qw, ws = _case(7, f"chunks{N}", M, K, N, True)
    qa, s = oracle.quant_act_per_token(xb)
    y_exact, T = oracle.gemm_w8a8_g128(qa, s, oracle.gptq_unpack(qw, 8, K), ws)
    y = i8.gemm_w8a8_g128_ex(dev(qw), dev(ws), x=dev_bf16(xb), kernel=i8.KERNEL_DECODE, decode_workgroups=wgs)
    torch.cuda.synchronize()
    assert_within_tolerance(host_bf16_bits(y), y_exact, T, K, what=f"N={N} with {wgs} workgroups")


@pytest.mark.parametrize("M,K,N,wgs", [
    (64, 128, 48, 1), (64, 1024, 40, 1), (64, 1024, 72, 1), (64, 1024, 72, 2), (64, 1024, 136, 1),
    (64, 1024, 136, 3), (64, 1024, 280, 1), (64, 2048, 264, 1), (20, 1024, 136, 1), (20, 1024, 136, 3),
    (33, 1024, 72, 2),
])
def test_decode_partial_last_fragment(M, K, N, wgs):
    """Chunks 48, 80 and 144 columns wide, whose last 32-column fragment reaches past the chunk:
    whole and K-split tiles, one or two m tiles, chunks of 40, 72, 136 and 144 columns."""
    xb, qw, ws = _case(8, f"half{M}-{K}-{N}", M, K, N, True)
    qa, s = oracle.quant_act_per_token(xb)
    y_exact, T = oracle.gemm_w8a8_g128(qa, s, oracle.gptq_unpack(qw, 8, K), ws)
    y = i8.gemm_w8a8_g128_ex(dev(qw), dev(ws), x=dev_bf16(xb), kernel=i8.KERNEL_DECODE, decode_workgroups=wgs)
    torch.cuda.synchronize()
    assert_within_tolerance(host_bf16_bits(y), y_exact, T, K, what=f"{M}x{K}x{N} with {wgs} workgroups")


def test_decode_and_tiled_kernels_agree_with_oracle():
    M, K, N = 64, 2048, 384
    xb, qw, ws = _case(3, "kernels", M, K, N, True)
    qa, s = oracle.quant_act_per_token(xb)
    y_exact, T = oracle.gemm_w8a8_g128(qa, s, oracle.gptq_unpack(qw, 8, K), ws)
    for kern in (i8.KERNEL_DECODE, i8.KERNEL_TILED):
        y = i8.gemm_w8a8_g128_ex(dev(qw), dev(ws), qa=dev(qa), a_scale=dev(s), kernel=kern)
        torch.cuda.synchronize()
        assert_within_tolerance(host_bf16_bits(y), y_exact, T, K, what=f"kernel {kern}")


@pytest.mark.parametrize("M,K,N", [(600, 640, 520), (257, 256, 264), (512, 1280, 768), (300, 128, 264),
                                   (300, 4096, 520), (130, 8192, 264)])
def test_prefill_and_tiled_kernels_multi_tile(M, K, N):
    """M > 64: the 256x256 prefill kernel (auto) and the 128x128 tiled kernel, over
    several tiles with ragged last rows and columns, against the oracle."""
    xb, qw, ws = _case(4, f"pf{M}-{K}-{N}", M, K, N, True)
    qa, s = oracle.quant_act_per_token(xb)
    y_exact, T = oracle.gemm_w8a8_g128(qa, s, oracle.gptq_unpack(qw, 8, K), ws)
    for kern in (i8.KERNEL_AUTO, i8.KERNEL_TILED):
        y = i8.gemm_w8a8_g128_ex(dev(qw), dev(ws), qa=dev(qa), a_scale=dev(s), kernel=kern)
        torch.cuda.synchronize()
        assert_within_tolerance(host_bf16_bits(y), y_exact, T, K, what=f"kernel {kern} {M}x{K}x{N}")


def test_identity_probe_recovers_dequantised_rows():
    """Running an identity matrix through the layer returns the dense dequantised
    weight rows (the W8A8-W8A16 drafter card's identity probe): row m is e_m, so
    a_scale = fl(1/127), qa = 127 e_m, and y[m, :] = bf16(fl(1/127) * 127 * w_scale * q)."""
    K, N = 512, 256
    _, qw, ws = _case(4, "probe", 8, K, N, False)
    eye = synth.bf16_bits_from_f32(np.eye(K, dtype=np.float32))
    y = i8.gemm_w8a8_g128(dev(qw), dev(ws), x=dev_bf16(eye))
    _, w = i8.gptq_unpack(dev(qw), 8, dev(ws), want_codes=False, want_dequant=True)
    torch.cuda.synchronize()
    qa, s = oracle.quant_act_per_token(eye)
    y_exact, T = oracle.gemm_w8a8_g128(qa, s, oracle.gptq_unpack(qw, 8, K), ws)
    yb = host_bf16_bits(y)
    assert_within_tolerance(yb, y_exact, T, K, what="identity probe")
    dense = synth.bf16_bits_from_f32(w.cpu().numpy())
    # the probe and the unpacked rows agree to within one bf16 unit
    diff = np.abs(synth.f32_from_bf16_bits(yb).astype(np.float64) - synth.f32_from_bf16_bits(dense))
    from parity import ulp_bf16
    assert np.all(diff <= ulp_bf16(w.cpu().numpy().astype(np.float64)))


@pytest.mark.parametrize("layer", ["qkv", "o_proj", "gate_up", "down", "fc"])
def test_prefill_layer_sampled_rows(layer):
    """Prefill workload (4096 tokens): full GPU output, 24 sampled rows checked (incl. first and
    last); the exact group sums of those rows from the prefill kernel run on all 4096 rows in
    the benchmark's launch plan (o_proj, down and fc split their last round's tiles along K:
    columns 4096 and up; qkv: columns 4096 and up of row tiles 8-15)."""
    L = synth.LAYERS[layer]
    M = 4096
    xb, qw, ws = _case(0, f"prefill-{layer}", M, L.K, L.N, True)
    y = i8.gemm_w8a8_g128(dev(qw), dev(ws), x=dev_bf16(xb))
    torch.cuda.synchronize()
    rows = synth.sample_rows(0, f"prefill-{layer}", M, 24)
    qa, s = oracle.quant_act_per_token(xb)
    q = unpacked(0, f"prefill-{layer}", L.K, L.N, 8)
    y_exact, T = oracle.gemm_w8a8_g128(qa, s, q, ws, rows=rows)
    yb = host_bf16_bits(y)[rows]
    del y
    assert_within_tolerance(yb, y_exact, T, L.K, what=f"prefill {layer}")
    P = i8.gemm_w8a8_g128_group_partials(dev(qa), dev(qw))
    Prows = P[torch.from_numpy(rows).to(P.device)].cpu().numpy()
    del P
    torch.cuda.empty_cache()
    assert np.array_equal(Prows, oracle.group_partials(qa[rows], q))


def test_lm_head_sampled_rows():
    """INT8 vocabulary head: 64 tokens x 248320 columns; 6 sampled rows checked against the oracle."""
    L = synth.LAYERS["lm_head"]
    M = 64
    xb, qw, ws = _case(0, "lm_head", M, L.K, L.N, False)
    y = i8.gemm_w8a8_g128(dev(qw), dev(ws), x=dev_bf16(xb))
    torch.cuda.synchronize()
    rows = synth.sample_rows(0, "lm_head", M, 6)
    qa, s = oracle.quant_act_per_token(xb)
    y_exact, T = oracle.gemm_w8a8_g128(qa, s, unpacked(0, "lm_head", L.K, L.N, 8), ws, rows=rows)
    assert_within_tolerance(host_bf16_bits(y)[rows], y_exact, T, L.K, what="lm_head")


@pytest.mark.parametrize("M,K,N,kern", [(64, 1280, 392, 0), (300, 640, 520, 0), (300, 640, 520, 2), (17, 384, 40, 1)])
def test_strided_rows(M, K, N, kern):
    """x and y with row strides larger than K and N (ldx = K + 64, ldy = N + 24), through
    the decode (M <= 64), prefill and 128x128 tiled kernels: the padding columns of y
    stay untouched."""
    xb, qw, ws = _case(5, f"st{M}-{K}-{N}", M, K, N, True)
    qa, s = oracle.quant_act_per_token(xb)
    y_exact, T = oracle.gemm_w8a8_g128(qa, s, oracle.gptq_unpack(qw, 8, K), ws)
    xfull = torch.zeros((M, K + 64), dtype=torch.bfloat16, device="cuda")
    xfull[:, :K] = dev_bf16(xb)
    yfull = torch.full((M, N + 24), 7.0, dtype=torch.bfloat16, device="cuda")
    i8.gemm_w8a8_g128_ex(dev(qw), dev(ws), x=xfull[:, :K], y=yfull[:, :N], kernel=kern)
    torch.cuda.synchronize()
    assert_within_tolerance(host_bf16_bits(yfull[:, :N].contiguous()), y_exact, T, K,
                            what=f"strided {M}x{K}x{N} kernel {kern}")
    assert bool((yfull[:, N:] == 7.0).all())


@pytest.mark.parametrize("M,K,N", [(64, 1024, 264), (7, 512, 256), (300, 640, 520)])
def test_zero_activation_rows_give_zero(M, K, N):
    """An all-zero token row has a_scale 0 and codes 0, so its output row is exactly zero
    (decode kernel for M <= 64, prefill kernel above), the other rows as usual."""
    xb, qw, ws = _case(6, f"zero{M}-{K}-{N}", M, K, N, True)
    xb = xb.copy()
    zero = [0, M // 2, M - 1]
    xb[zero] = 0
    y = i8.gemm_w8a8_g128(dev(qw), dev(ws), x=dev_bf16(xb))
    torch.cuda.synchronize()
    yf = y.float().cpu().numpy()
    assert np.all(yf[zero] == 0.0)
    qa, s = oracle.quant_act_per_token(xb)
    y_exact, T = oracle.gemm_w8a8_g128(qa, s, oracle.gptq_unpack(qw, 8, K), ws)
    assert_within_tolerance(host_bf16_bits(y), y_exact, T, K, what=f"zero rows {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N,ldy", [(7, 512, 256, 1 << 27), (40, 512, 264, (1 << 24) + 8),
                                       (40, 512, 264, 1 << 23), (100, 384, 264, 10_000_000),
                                       (300, 384, 264, (1 << 21) - 8)])
def test_large_row_stride_y(M, K, N, ldy):
    """Row strides of y near the 32-bit offset limit.  Where the rows a launch pads up to (32 or
    64 for the decode kernel, 256 for the prefill kernel) would pass 2^31 bytes, the call takes
    the 128 x 128 tiled kernel (64-bit addressing); below it (40 rows at 2^23, 300 rows at
    2^21 - 8) the decode and prefill kernels drop the padded rows by their range check.  Every
    real row holds its own result."""
    xb, qw, ws = _case(9, f"ldy{M}-{K}-{N}", M, K, N, True)
    qa, s = oracle.quant_act_per_token(xb)
    y_exact, T = oracle.gemm_w8a8_g128(qa, s, oracle.gptq_unpack(qw, 8, K), ws)
    ybuf = torch.empty(((M - 1) * ldy + N,), dtype=torch.bfloat16, device="cuda")
    y = ybuf.as_strided((M, N), (ldy, 1))
    i8.gemm_w8a8_g128(dev(qw), dev(ws), x=dev_bf16(xb), y=y)
    torch.cuda.synchronize()
    assert_within_tolerance(host_bf16_bits(y.contiguous()), y_exact, T, K, what=f"ldy={ldy} {M}x{K}x{N}")
    del ybuf
    torch.cuda.empty_cache()


@pytest.mark.parametrize("layer", ["qkv", "down"])
def test_graph_replays_match_eager(layer):
    """The decode linear from bf16 x (quantisation into the workspace, then the K-split
    GEMM whose arrival counters must return to zero) captured as a HIP graph: three
    replays, with eager calls of another shape and host synchronisations between them,
    each give the eager result bit for bit."""
    L = synth.LAYERS[layer]
    M = 64
    xb = synth.activations_bf16(3, f"graph-{layer}", M, L.K, True)
    qw, ws = rtn_weights(3, f"graph-{layer}", L.K, L.N, 8)
    x, qw, ws = dev_bf16(xb), dev(qw), dev(ws)
    y_eager = i8.gemm_w8a8_g128(qw, ws, x=x)
    other = synth.LAYERS["o_proj"]
    xo = dev_bf16(synth.activations_bf16(3, "graph-other", 8, other.K, True))
    qwo, wso = (dev(a) for a in rtn_weights(3, "graph-other", other.K, other.N, 8))
    cap = torch.cuda.Stream()
    y = torch.empty_like(y_eager)
    with torch.cuda.stream(cap):
        i8.gemm_w8a8_g128(qw, ws, x=x, y=y)  # the binding's workspace for this stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        i8.gemm_w8a8_g128(qw, ws, x=x, y=y)
    for r in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {r}"
        i8.gemm_w8a8_g128(qwo, wso, x=xo)
        torch.cuda.synchronize()


@pytest.mark.parametrize("M,K,N,kern", [(64, 1024, 264, "auto"), (300, 2048, 264, "auto"), (100, 512, 136, "tiled")])
def test_extreme_weight_scales(M, K, N, kern):
    """Weight scales across the whole range the contract admits, from fp32 subnormals to
    2^99, mixed per group and column: the decode kernel folds with w_scale * 2^26 (exact for
    |w_scale| < 2^100), the prefill and tiled kernels with w_scale itself."""
    xb = synth.activations_bf16(7, f"xs{M}", M, K, True)
    qw, _ = rtn_weights(7, f"xs{K}x{N}", K, N, 8)
    G = K // 128
    g = np.random.Generator(np.random.Philox(key=7))
    e = g.integers(-149, 99, size=(G, N))                       # subnormal to 2^99
    ws = (np.ldexp(1.0, e) * g.uniform(1.0, 2.0, size=(G, N))).astype(np.float32)
    ws[0, :8] = np.float32(2.0 ** -149)                            # the smallest subnormal
    ws[-1, -8:] = np.float32(np.nextafter(np.float32(2.0 ** 100), np.float32(0)))
    ws = np.where(np.isfinite(ws), ws, np.float32(1.0)).astype(np.float32)
    y = i8.gemm_w8a8_g128_ex(dev(qw), dev(ws), x=dev_bf16(xb), kernel=KERNELS[kern])
    torch.cuda.synchronize()
    qa, s = oracle.quant_act_per_token(xb)
    y_exact, T = oracle.gemm_w8a8_g128(qa, s, oracle.gptq_unpack(qw, 8, K), ws)
    assert_within_tolerance(host_bf16_bits(y), y_exact, T, K, what=f"extreme scales {M}x{K}x{N} {kern}")
