// W4A16 g128 weight-only GEMM on gfx950 bf16 MFMA.
//
// Qwen3.8-27B-DFlash2-W4A16-g128-sym-GPTQ model card, property table (W4A16,
// group_size 128, symmetric) and quantised-layer table (all attention / MLP
// linears and fc in INT4 g128 sym).  y[m,n] = bf16(sum_g w_scale[g,n] *
// sum_{k in g} x[m,k] * q[k,n]) with q = nibble - 8.
//
// Each nibble is turned into the exact bf16 value of 16*q (q an integer in [-8, 7]):
// masking a word's high nibbles in place, or its low nibbles shifted up by 4, and
// flipping bit 7 of every byte leaves 16*q as a signed byte; a sign-extending byte
// convert (SDWA) gives the fp32 value, whose top half is its bf16 pattern.  One
// 128-wide group is summed by four v_mfma_f32_16x16x32_bf16 into a fresh fp32
// accumulator (the products are exact in fp32), then scaled by that group's
// per-column scale / 16 (exact) and added to the running fp32 sum.  Scaling after
// the group keeps the error relative to sum |x*q| rather than to the cancelling
// scaled terms.
//
// MFMA layout (16x16x32 bf16): lane l holds row (l % 16) of A and column (l % 16)
// of B, 8 consecutive K values starting at 8 * (l / 16) within the 32-wide K step;
// with GPTQ's packing those 8 values of one column are exactly one int32 word.
//
// Data flow (as in the W8A8 decode kernel): a workgroup of 8 waves owns a tile of
// 128 columns (16 per wave) and up to 64 rows, and walks its K groups through a
// D-stage LDS ring filled by buffer_load ... lds copies -- a stage holds the group's
// 16 packed weight rows of the tile, its activation rows (bf16, 256 bytes each) and
// the tile's scales -- with the wait for a stage issued D - 2 stages behind the
// copies, so D - 1 groups are in flight.  K is split across S workgroups when the
// column tiles alone cannot fill the GPU; the splits publish fp32 partials with
// device-coherent stores and the last to arrive sums them in split order.  Rows
// are processed in chunks of 64 (gridDim.y).
#include "internal.h"

namespace i8gs {
namespace {

constexpr int kTN = 128;  // columns per tile (16 per wave)

// The 8 codes of one word as bf16 of 16*q, in K order.  Byte i of the word holds
// codes 2i (low nibble) and 2i+1 (high nibble); (code ^ 8) is q as a 4-bit two's-
// complement field, so a byte holding it in its high nibble reads as 16*q.
__device__ __forceinline__ v8bf dequant8x16(uint32_t w) {
    const uint32_t odd = (w & 0xF0F0F0F0u) ^ 0x80808080u;
    const uint32_t even = ((w << 4) & 0xF0F0F0F0u) ^ 0x80808080u;
    v4i out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t fe = __float_as_uint((float)(signed char)(even >> (8 * i)));
        const uint32_t fo = __float_as_uint((float)(signed char)(odd >> (8 * i)));
        out[i] = (int)__builtin_amdgcn_perm(fo, fe, 0x07060302u);  // top halves: (fe >> 16) | (fo & 0xFFFF0000)
    }
    return __builtin_bit_cast(v8bf, out);
}

__device__ __forceinline__ v4f mfma_bf16(v4i a, v8bf b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), b, c, 0, 0, 0);
}

// Stage layout (bytes): the 16 x 128 weight words, row-major, with the 16-byte pieces
// of packed row r permuted by XOR with 4 * (r % 4) (a B read's four lane groups read
// rows 4 apart: they land in different banks); then the activation rows, 256 bytes
// each, pieces permuted by XOR with row % 16; then the 128 scales.
template <int MT>
struct W4Stage {
    static constexpr int ROWS = 16 * MT;
    static constexpr int WB = 16 * kTN * 4;
    static constexpr int AB = ROWS * 256;
    static constexpr int SB = kTN * 4;
    static constexpr int BYTES = WB + AB + SB;
    static constexpr int ACOPIES = AB / 1024;              // 1 KiB activation copies per stage
    static constexpr int AI = (ACOPIES + 7) / 8;           // per wave (extra ones repeat the last)
};

// The copies of one stage (group g) by this wave.
template <int MT>
__device__ __forceinline__ void w4_issue(char *st, int g, int wave, int N, __amdgpu_buffer_rsrc_t wr,
                                         __amdgpu_buffer_rsrc_t xr, __amdgpu_buffer_rsrc_t sr, int w_voff,
                                         const int (&a_voff)[W4Stage<MT>::AI], const int (&a_ins)[W4Stage<MT>::AI],
                                         int s_half, int s_voff) {
    using SG = W4Stage<MT>;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, I8GS_LDS(st + wave * 1024), 16, w_voff,
                                             (int)((uint32_t)g * 16u * (uint32_t)N * 4u), 0, kCpolNT);
#pragma unroll
    for (int j = 0; j < SG::AI; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, I8GS_LDS(st + SG::WB + a_ins[j] * 1024), 16, a_voff[j], g * 256,
                                                 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, I8GS_LDS(st + SG::WB + SG::AB + s_half * 256), 4, s_voff,
                                             (int)((uint32_t)g * (uint32_t)N * 4u), 0, 0);
}

// The copies of wave + 4's share, issued by wave (0-3) too: its weight rows lie 8
// further down, its activation copies are given by a_voff / a_ins (its scales repeat
// those of this wave and are not copied again).
template <int MT>
__device__ __forceinline__ void w4_issue_partner(char *st, int g, int wave, int N, __amdgpu_buffer_rsrc_t wr,
                                                 __amdgpu_buffer_rsrc_t xr, int w_voff,
                                                 const int (&a_voff)[W4Stage<MT>::AI],
                                                 const int (&a_ins)[W4Stage<MT>::AI]) {
    using SG = W4Stage<MT>;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, I8GS_LDS(st + (wave + 4) * 1024), 16, w_voff,
                                             (int)(((uint32_t)g * 16u + 8u) * (uint32_t)N * 4u), 0, kCpolNT);
#pragma unroll
    for (int j = 0; j < SG::AI; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, I8GS_LDS(st + SG::WB + a_ins[j] * 1024), 16, a_voff[j], g * 256,
                                                 0, 0);
}

template <int MT, int D>
__global__ __launch_bounds__(512) void w4a16_stream_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, const int32_t *__restrict__ qweight,
    const float *__restrict__ w_scale, uint16_t *__restrict__ y, int64_t ldy, int M, int N, int K, int S,
    int tiles, float *__restrict__ part, size_t part_bytes, int *__restrict__ cnt) {
    using SG = W4Stage<MT>;
    constexpr int RING = D * SG::BYTES;
    // One LDS object only (see the W8A8 decode kernel); the split flag sits after the ring.
    __shared__ __attribute__((aligned(1024))) char lds[RING + 16];

    // XCD-aware placement: logical workgroup L (tile-major) at launch index (L % Q) * 8 + L / Q.
    const int P = tiles * S, Q = (P + 7) >> 3;
    const int L = (blockIdx.x & 7) * Q + (blockIdx.x >> 3);
    if (L >= P) return;
    const int t = L / S, s = L - (L / S) * S;
    const int m0 = blockIdx.y * SG::ROWS;
    const int mrows = min(M - m0, SG::ROWS);
    const int n0 = t * kTN;
    const int G = K >> 7;
    const int g0 = (int)((int64_t)s * G / S), g1 = (int)((int64_t)(s + 1) * G / S);
    const int ng = g1 - g0;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 15, lb = lane >> 4;

    // byte offsets fit 32 bits: K*N < 2^32 is checked before launch, and x is
    // addressed from this chunk's first row
    const uint16_t *xc = x + (int64_t)m0 * ldx;
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc((void *)qweight, 0, (int)((uint32_t)K / 8u * (uint32_t)N * 4u), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)xc, 0, (int)(((uint32_t)(mrows - 1) * (uint32_t)ldx + (uint32_t)K) * 2u), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t sr =
        __builtin_amdgcn_make_buffer_rsrc((void *)w_scale, 0, (int)((uint32_t)G * (uint32_t)N * 4u), kRsrcWord3);

    // Copy roles.  The shares are per wave w: weights: packed rows 2w, 2w+1 (32 pieces of
    // 4 columns each); activations: copies a_ins; scales: half w % 2.  Waves 0-3 issue
    // their own share and that of wave + 4: the SIMD's issue arbitration favours the
    // older of its two waves, and the copies' issue stalls then fall on the favoured one
    // (1-4% faster on six of the eight decode cases, the other two unchanged).  Every
    // copying wave issues LPSW copies per stage, so one wait count serves all.
    int w_voff;
    {
        const int r = 2 * wave + (lane >> 5), sl = lane & 31;
        const int piece = sl ^ ((r & 3) << 2);
        w_voff = (int)(((uint32_t)r * (uint32_t)N + (uint32_t)min(n0 + 4 * piece, N - 4)) * 4u);
    }
    // Activations: copy c fills rows 4c .. 4c+3 (16 pieces each); rows past the chunk
    // repeat its last row (never stored).
    int a_voff[SG::AI], a_ins[SG::AI];
#pragma unroll
    for (int j = 0; j < SG::AI; ++j) {
        a_ins[j] = min(wave * SG::AI + j, SG::ACOPIES - 1);
        const int row = 4 * a_ins[j] + (lane >> 4), sl = lane & 15;
        const int piece = sl ^ (row & 15);
        a_voff[j] = (int)(((uint32_t)min(row, mrows - 1) * (uint32_t)ldx + (uint32_t)piece * 8u) * 2u);
    }
    int a_voffp[SG::AI], a_insp[SG::AI];  // the activation copies of wave + 4
#pragma unroll
    for (int j = 0; j < SG::AI; ++j) {
        a_insp[j] = min((wave + 4) * SG::AI + j, SG::ACOPIES - 1);
        const int row = 4 * a_insp[j] + (lane >> 4), sl = lane & 15;
        const int piece = sl ^ (row & 15);
        a_voffp[j] = (int)(((uint32_t)min(row, mrows - 1) * (uint32_t)ldx + (uint32_t)piece * 8u) * 2u);
    }
    constexpr int LPSW = 2 * (1 + SG::AI) + 1;
    // Scales: half k = wave % 2 of the tile's 128 (waves 2..7 repeat them).
    const int s_half = wave & 1;
    const int s_voff = min(n0 + 64 * s_half + lane, N - 1) * 4;

    float acc[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mt][r] = 0.0f;

#pragma unroll
    for (int k = 0; k < D - 1; ++k)
        if (k < ng && wave < 4) {
            w4_issue<MT>(lds + k * SG::BYTES, g0 + k, wave, N, wr, xr, sr, w_voff, a_voff, a_ins, s_half, s_voff);
            w4_issue_partner<MT>(lds + k * SG::BYTES, g0 + k, wave, N, wr, xr, w_voff, a_voffp, a_insp);
        }

    // This lane's B words: column 16*wave + li of packed rows 4*ks + lb.
    const int cl = 16 * wave + li;
    int b_off[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int r = 4 * ks + lb;
        b_off[ks] = (r * kTN + (((cl >> 2) ^ ((r & 3) << 2)) << 2) + (cl & 3)) * 4;
    }
    int slot = 0;
    for (int u = 0; u < ng; ++u) {
        // Copies complete in issue order and the next D-2 stages are the youngest ones.
        if (u + D - 2 < ng) wait_vmcnt<(D - 2) * LPSW>();
        else wait_vmcnt<0>();
        barrier_only();  // this stage is in; every wave is done with the previous slot
        __builtin_amdgcn_sched_barrier(0);
        if (u + D - 1 < ng && wave < 4) {
            char *const nst = lds + (slot == 0 ? D - 1 : slot - 1) * SG::BYTES;
            w4_issue<MT>(nst, g0 + u + D - 1, wave, N, wr, xr, sr, w_voff, a_voff, a_ins, s_half, s_voff);
            w4_issue_partner<MT>(nst, g0 + u + D - 1, wave, N, wr, xr, w_voff, a_voffp, a_insp);
        }
        __builtin_amdgcn_sched_barrier(0);
        const char *st = lds + slot * SG::BYTES;
        // The group's four words are dequantised first, at raised wave priority: with
        // the two waves of a SIMD both holding VALU work, the dequantisation goes first
        // and the MFMAs that need it start sooner (measured 2-6% faster on the decode
        // layers at M = 8 and 64, except qkv at M = 8, 2% slower).
        v8bf bw[4];
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) bw[ks] = dequant8x16((uint32_t)*reinterpret_cast<const int *>(st + b_off[ks]));
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        v4f p[MT];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const v8bf b = bw[ks];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int row = mt * 16 + li;
                const v4i a = *reinterpret_cast<const v4i *>(st + SG::WB + row * 256 + (((4 * ks + lb) ^ li) << 4));
                p[mt] = mfma_bf16(a, b, ks == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : p[mt]);
            }
        }
        const float sc = reinterpret_cast<const float *>(st + SG::WB + SG::AB)[cl] * 0.0625f;  // sums are 16x
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[mt][r] += sc * p[mt][r];
        slot = slot == D - 1 ? 0 : slot + 1;
    }

    if (S > 1) {
        // Partial of split q, wave w: MT*4 fp32 cells of 64 lanes at
        // ((tile * S + q) * 8 + w) * MT*4 * 64 (device-coherent stores and loads: the
        // splits may run on different XCDs).
        constexpr int NACC = MT * 4;
        const int tile_id = blockIdx.y * tiles + t;
        const __amdgpu_buffer_rsrc_t pr =
            __builtin_amdgcn_make_buffer_rsrc((void *)part, 0, (int)part_bytes, kRsrcWord3);
        const uint32_t qstride = 8u * NACC * 64 * 4;
        const uint32_t cell0 = (uint32_t)tile_id * (uint32_t)S * qstride + ((uint32_t)wave * NACC * 64 + lane) * 4u;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(acc[mt][r]), pr,
                                                      (int)(cell0 + (uint32_t)(mt * 4 + r) * 256u),
                                                      (int)((uint32_t)s * qstride), kCpolSC1);
        wait_vmcnt<0>();
        __syncthreads();
        int *const s_last = reinterpret_cast<int *>(lds + RING);
        if (threadIdx.x == 0) {
            const int last =
                __hip_atomic_fetch_add(cnt + tile_id, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
            if (last) __hip_atomic_store(cnt + tile_id, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *s_last = last;
        }
        __syncthreads();
        if (!*s_last) return;
        // Sum in split order; the other splits' cells are loaded QB splits at a time, all
        // in flight together (this split's own come from registers: the values it stored).
        constexpr int QB = MT > 2 ? 2 : 4;
        float sum[NACC];
        for (int q0 = 0; q0 < S; q0 += QB) {
            float v[QB][NACC];
#pragma unroll
            for (int k = 0; k < QB; ++k) {
                const int q = min(q0 + k, S - 1);
#pragma unroll
                for (int i = 0; i < NACC; ++i)
                    v[k][i] = q == s ? acc[i / 4][i % 4]
                                     : __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                           pr, (int)(cell0 + (uint32_t)i * 256u), (int)((uint32_t)q * qstride),
                                           kCpolSC1));
            }
#pragma unroll
            for (int k = 0; k < QB; ++k) {
                if (q0 + k >= S) break;
#pragma unroll
                for (int i = 0; i < NACC; ++i) sum[i] = q0 + k == 0 ? v[k][i] : sum[i] + v[k][i];
            }
        }
#pragma unroll
        for (int i = 0; i < NACC; ++i) acc[i / 4][i % 4] = sum[i];
    }

    const int col = n0 + cl;
    if (col < N) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = mt * 16 + lb * 4 + r;
                if (row < mrows) y[(int64_t)(m0 + row) * ldy + col] = f32_to_bf16_bits(acc[mt][r]);
            }
    }
}

struct W4Plan {
    int MT, S, tiles, blocks, chunks;
};

W4Plan w4_plan(int M, int N, int K) {
    W4Plan p;
    p.tiles = (N + kTN - 1) / kTN;
    const int G = K / kGroup;
    // Target 1.5 workgroups per CU: two fit on a CU (LDS), and the second one's waves
    // hide the first one's dequantisation and barrier latencies (measured best of 1, 1.5, 2).
    // Layers with more tiles than CUs take 3 per CU (gate_up: 34.5 -> 31.8 us at M = 8).
    const int cus = device_cu_count();
    const int P = p.tiles > cus ? 3 * cus : 3 * cus / 2;
    auto plan = [&](int mt) {
        p.MT = mt;
        p.chunks = (M + 16 * mt - 1) / (16 * mt);
        int S = (P + p.tiles * p.chunks - 1) / (p.tiles * p.chunks);
        if (S > G) S = G;
        if (S < 1) S = 1;
        if (p.tiles * p.chunks > kMaxCounters) S = 1;
        p.S = S;
    };
    plan(M >= 64 ? 4 : (M + 15) / 16);
    // Narrow layers at M > 32: when the splits would leave a workgroup fewer than 8 groups,
    // chunks of 32 rows (twice the workgroups per tile, half the splits) are faster
    // (measured at M = 64: qkv 20.2 -> 18.1 us, o_proj 20.3 -> 15.9 us; wide layers lose).
    if (p.MT > 2 && G < 8 * p.S) plan(2);
    p.blocks = ((p.tiles * p.S + 7) / 8) * 8;
    return p;
}

// As many stages as fit in 80 KiB (two workgroups per CU), at most 6.
template <int MT, int D>
hipError_t launch_w4_mt(const W4A16Args &a, const W4Plan &p, hipStream_t st) {
    static_assert(D * W4Stage<MT>::BYTES + 16 <= 80 * 1024 && (D == 6 || (D + 1) * W4Stage<MT>::BYTES + 16 > 80 * 1024),
                  "stage count must be the largest that fits 80 KiB");
    int *cnt = p.S > 1 ? a.counters : nullptr;
    float *part = p.S > 1 ? (float *)a.ws : nullptr;
    dim3 grid(p.blocks, p.chunks);
    w4a16_stream_kernel<MT, D><<<grid, 512, 0, st>>>(a.x, a.ldx, a.qweight, a.w_scale, a.y, a.ldy, a.M, a.N, a.K,
                                                    p.S, p.tiles, part, p.S > 1 ? a.ws_bytes : 0, cnt);
    return hipGetLastError();
}

}  // namespace

// Partial-sum bytes after the counter region (0 when K is not split).
size_t w4a16_gemm_workspace(int M, int N, int K) {
    const W4Plan p = w4_plan(M, N, K);
    if (p.S <= 1) return 0;
    return align256(size_t(p.tiles) * p.chunks * p.S * 8 * p.MT * 4 * 64 * sizeof(float));
}

hipError_t launch_w4a16_gemm(const W4A16Args &a, hipStream_t s) {
    const W4Plan p = w4_plan(a.M, a.N, a.K);
    switch (p.MT) {
        case 1: return launch_w4_mt<1, 6>(a, p, s);
        case 2: return launch_w4_mt<2, 4>(a, p, s);
        case 3: return launch_w4_mt<3, 3>(a, p, s);
        default: return launch_w4_mt<4, 3>(a, p, s);
    }
}

}  // namespace i8gs
