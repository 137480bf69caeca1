// LDS-staged weight-only GEMM on gfx950 bf16 MFMA: W4A16 g128 and W8A16 g128 / g32 on the
// decode and prefill layer shapes (the vocabulary heads at few tokens take the
// register-streaming kernel of wonly.hip).
//
// Qwen3.8-27B-DFlash2-W4A16-g128-sym-GPTQ model card, property table (W4A16,
// group_size 128, symmetric) and quantised-layer table (all attention / MLP
// linears and fc in INT4 g128 sym); Qwen3.5-4B-DFlash-W8A16 model card (int8 weights,
// bf16 activations); qwen38/dflash2 recipe, quantisation settings (int8 projections at
// group 32).  y[m,n] = bf16(sum_g w_scale[g,n] * sum_{k in g} x[m,k] * q[k,n]) with
// q = code - 2^(bits-1).
//
// 4 bits: each nibble is turned into the exact bf16 value of 16*q (q an integer in
// [-8, 7]): masking a word's high nibbles in place, or its low nibbles shifted up by 4,
// and flipping bit 7 of every byte leaves 16*q as a signed byte; a sign-extending byte
// convert (SDWA) gives the fp32 value, whose top half is its bf16 pattern.  8 bits: XOR
// 0x80 per byte leaves q itself as a signed byte, converted the same way.  One 128-wide
// group (or, at group 32, each 32-wide K step) is summed by v_mfma_f32_16x16x32_bf16 into
// a fresh fp32 accumulator (the products are exact in fp32), then scaled by that group's
// per-column scale (/ 16 at 4 bits, exact) and added to the running fp32 sum.  Scaling
// after the group keeps the error relative to sum |x*q| rather than to the cancelling
// scaled terms.
//
// MFMA layout (16x16x32 bf16): lane l holds row (l % 16) of A and column (l % 16)
// of B, 8 consecutive K values starting at 8 * (l / 16) within the 32-wide K step;
// with GPTQ's packing those 8 values of one column are exactly one int32 word at 4 bits
// and two consecutive words at 8 bits.
//
// Data flow (as in the W8A8 decode kernel): a workgroup of 8 waves owns a tile of
// 128 columns (16 per wave) and up to 64 rows, and walks its K range through a
// D-stage LDS ring filled by buffer_load ... lds copies -- a stage holds one group's
// 16 (4 bits) or 32 (8 bits) packed weight rows of the tile (two groups, 32 rows, at
// 4 bits with one 16-row m tile), its activation rows (bf16) and the tile's scales --
// with the wait for a stage issued D - 2 stages behind the copies, so D - 1 stages are
// in flight.  K is split across S workgroups when the column tiles alone cannot fill
// the GPU; the splits publish fp32 partials with device-coherent stores and the last
// to arrive sums them in split order.  Rows are processed in chunks of up to 64
// (gridDim.y).
#include <algorithm>

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

// Stage layout (bytes): the PR x 128 weight words of KS 32-wide K steps (one 128-wide
// group: PR = 16 packed rows at 4 bits, 32 at 8 bits; two groups at 4 bits with KS = 8),
// row-major, with the 16-byte pieces of packed row r permuted by XOR with swz(r) (a B
// read's four lane groups read rows that land in different banks); then the activation
// rows, 2 * 32 * KS bytes each, pieces permuted by XOR with row % 16; then the 128 scales
// of each of the stage's scale rows.
//
// TAG (the kernel's ring depth) only gives each kernel instantiation shape types of its
// own: a device function template taking buffer resources, used with one shape from two
// kernel instantiations, fails overload resolution in hipcc's host pass.
template <int BITS, int GS, int MT, int KS = 4, int TAG = 0>
struct W4Stage {
    static_assert((BITS == 4 && GS == 128 && (KS == 4 || KS == 8)) ||
                      (BITS == 8 && (GS == 128 || GS == 32) && KS == 4),
                  "weight-only LDS shape");
    static constexpr int KPS = 32 * KS;                      // K values per stage (KS MFMA K steps)
    static constexpr int PR = KPS * BITS / 32;               // packed rows per stage
    static constexpr int ROWS = 16 * MT;
    static constexpr int ROWB = KPS * 2;                     // bytes of one activation row
    static constexpr int WB = PR * kTN * 4;
    static constexpr int AB = ROWS * ROWB;
    static constexpr int NSG = KPS / GS;                     // scale rows per stage
    static constexpr int SB = NSG * kTN * 4;
    static constexpr int BYTES = WB + AB + SB;
    static constexpr int WPW = PR / 16;                      // 1 KiB weight copies per wave (8 waves)
    static constexpr int ACOPIES = AB / 1024;              // 1 KiB activation copies per stage
    static constexpr int AI = (ACOPIES + 7) / 8;           // per wave (extra ones repeat the last)
    static constexpr int RPC = 1024 / ROWB;                  // activation rows per copy
    static constexpr int SPW = NSG == 1 ? 1 : 2;             // 256-byte scale copies per copying wave
};

// Piece permutation of packed row r: rows 4 apart (4 bits: a lane group's row 4*ks +
// lb) or 2 apart (8 bits: rows 8*ks + 2*lb and the next) are spread over the banks.
template <int BITS>
__device__ __forceinline__ int w4_swz(int r) {
    return BITS == 4 ? ((r & 3) << 2) : (((r >> 1) & 3) << 2);
}

// The copies of one stage (stage g) by this wave: its WPW weight copies (packed rows
// 2*(WPW*wave + j) and the next), its activation copies and its scale copies (one scale
// row: half wave % 2 of the tile's 128 scales; several: both halves of scale row
// wave % NSG).
template <int BITS, int GS, int MT, int KS, int TAG>
__device__ __forceinline__ void w4_issue(char *st, int g, int wave, int N, __amdgpu_buffer_rsrc_t wr,
                                         __amdgpu_buffer_rsrc_t xr, __amdgpu_buffer_rsrc_t sr,
                                         const int (&w_voff)[W4Stage<BITS, GS, MT, KS, TAG>::WPW],
                                         const int (&a_voff)[W4Stage<BITS, GS, MT, KS, TAG>::AI],
                                         const int (&a_ins)[W4Stage<BITS, GS, MT, KS, TAG>::AI], int s_half, int s_voff) {
    using SG = W4Stage<BITS, GS, MT, KS, TAG>;
#pragma unroll
    for (int j = 0; j < SG::WPW; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, I8GS_LDS(st + (wave * SG::WPW + j) * 1024), 16, w_voff[j],
                                                 (int)((uint32_t)g * (uint32_t)SG::PR * (uint32_t)N * 4u), 0, kCpolNT);
#pragma unroll
    for (int j = 0; j < SG::AI; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, I8GS_LDS(st + SG::WB + a_ins[j] * 1024), 16, a_voff[j],
                                                 g * SG::ROWB, 0, 0);
    if constexpr (SG::NSG == 1) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, I8GS_LDS(st + SG::WB + SG::AB + s_half * 256), 4, s_voff,
                                                 (int)((uint32_t)g * (uint32_t)N * 4u), 0, 0);
    } else {
        // scale row wave % NSG, both halves: s_voff addresses the first half (with two
        // scale rows, waves 2 and 3 copy the same bytes as waves 0 and 1)
        const int sri = wave % SG::NSG;
#pragma unroll
        for (int h = 0; h < 2; ++h)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                sr, I8GS_LDS(st + SG::WB + SG::AB + sri * 512 + h * 256), 4, s_voff + h * 256,
                (int)(((uint32_t)g * (uint32_t)SG::NSG + (uint32_t)sri) * (uint32_t)N * 4u), 0, 0);
    }
}

// The copies of wave + 4's share, issued by wave (0-3) too: its weight rows lie 8*WPW
// further down, its activation copies are given by a_voff / a_ins (its scales repeat
// those of this wave, or are copied by waves 0-3 themselves, and are not copied again).
template <int BITS, int GS, int MT, int KS, int TAG>
__device__ __forceinline__ void w4_issue_partner(char *st, int g, int wave, int N, __amdgpu_buffer_rsrc_t wr,
                                                 __amdgpu_buffer_rsrc_t xr,
                                                 const int (&w_voff)[W4Stage<BITS, GS, MT, KS, TAG>::WPW],
                                                 const int (&a_voff)[W4Stage<BITS, GS, MT, KS, TAG>::AI],
                                                 const int (&a_ins)[W4Stage<BITS, GS, MT, KS, TAG>::AI]) {
    using SG = W4Stage<BITS, GS, MT, KS, TAG>;
#pragma unroll
    for (int j = 0; j < SG::WPW; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wr, I8GS_LDS(st + ((wave + 4) * SG::WPW + j) * 1024), 16, w_voff[j],
            (int)(((uint32_t)g * (uint32_t)SG::PR + 8u * (uint32_t)SG::WPW) * (uint32_t)N * 4u), 0, kCpolNT);
#pragma unroll
    for (int j = 0; j < SG::AI; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, I8GS_LDS(st + SG::WB + a_ins[j] * 1024), 16, a_voff[j],
                                                 g * SG::ROWB, 0, 0);
}

// The 8 codes of two 8-bit words (K order: word 0 bytes 0..3, word 1 bytes 0..3) as
// bf16 of q = code - 128: XOR 0x80 per byte makes q a signed byte, a sign-extending
// byte convert gives the exact fp32 value, whose top half is its bf16 pattern.
__device__ __forceinline__ v8bf dequant8x8(uint32_t w0, uint32_t w1) {
    v4i out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w = (i < 2 ? w0 : w1) ^ 0x80808080u;
        const int sh = 16 * (i & 1);
        const uint32_t fe = __float_as_uint((float)(signed char)(w >> sh));
        const uint32_t fo = __float_as_uint((float)(signed char)(w >> (sh + 8)));
        out[i] = (int)__builtin_amdgcn_perm(fo, fe, 0x07060302u);  // top halves: (fe >> 16) | (fo & 0xFFFF0000)
    }
    return __builtin_bit_cast(v8bf, out);
}

template <int BITS, int GS, int MT, int KS, int D>
__global__ __launch_bounds__(512) void w4a16_stream_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, const int32_t *__restrict__ qweight,
    const float *__restrict__ w_scale, uint16_t *__restrict__ y, int64_t ldy, int M, int N, int K, int S,
    int tiles, float *__restrict__ part, size_t part_bytes, int *__restrict__ cnt) {
    using SG = W4Stage<BITS, GS, MT, KS, D>;
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
    const int G = K / SG::KPS;  // stages
    const int g0 = (int)((int64_t)s * G / S), g1 = (int)((int64_t)(s + 1) * G / S);
    const int ng = g1 - g0;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 15, lb = lane >> 4;

    // byte offsets fit 32 bits: K*N < 2^32 is checked before launch, and x is
    // addressed from this chunk's first row
    const uint16_t *xc = x + (int64_t)m0 * ldx;
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)qweight, 0, (int)((uint32_t)K / (32u / BITS) * (uint32_t)N * 4u), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)xc, 0, (int)(((uint32_t)(mrows - 1) * (uint32_t)ldx + (uint32_t)K) * 2u), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)w_scale, 0, (int)((uint32_t)K / (uint32_t)GS * (uint32_t)N * 4u), kRsrcWord3);

    // Copy roles.  The shares are per wave w: weights: packed rows 2w, 2w+1 (32 pieces of
    // 4 columns each); activations: copies a_ins; scales: half w % 2.  Waves 0-3 issue
    // their own share and that of wave + 4: the SIMD's issue arbitration favours the
    // older of its two waves, and the copies' issue stalls then fall on the favoured one
    // (1-4% faster on six of the eight decode cases, the other two unchanged).  Every
    // copying wave issues LPSW copies per stage, so one wait count serves all.
    int w_voff[SG::WPW];
#pragma unroll
    for (int j = 0; j < SG::WPW; ++j) {
        const int r = 2 * (SG::WPW * wave + j) + (lane >> 5), sl = lane & 31;
        const int piece = sl ^ w4_swz<BITS>(r);
        w_voff[j] = (int)(((uint32_t)r * (uint32_t)N + (uint32_t)min(n0 + 4 * piece, N - 4)) * 4u);
    }
    // Activations: copy c fills rows RPC*c .. RPC*c + RPC-1 (64/RPC pieces each); rows
    // past the chunk repeat its last row (never stored).
    constexpr int LPR = 64 / SG::RPC;  // lanes (16-byte pieces) per activation row
    int a_voff[SG::AI], a_ins[SG::AI];
#pragma unroll
    for (int j = 0; j < SG::AI; ++j) {
        a_ins[j] = min(wave * SG::AI + j, SG::ACOPIES - 1);
        const int row = SG::RPC * a_ins[j] + lane / LPR, sl = lane % LPR;
        const int piece = sl ^ (row & 15);
        a_voff[j] = (int)(((uint32_t)min(row, mrows - 1) * (uint32_t)ldx + (uint32_t)piece * 8u) * 2u);
    }
    int a_voffp[SG::AI], a_insp[SG::AI];  // the activation copies of wave + 4
#pragma unroll
    for (int j = 0; j < SG::AI; ++j) {
        a_insp[j] = min((wave + 4) * SG::AI + j, SG::ACOPIES - 1);
        const int row = SG::RPC * a_insp[j] + lane / LPR, sl = lane % LPR;
        const int piece = sl ^ (row & 15);
        a_voffp[j] = (int)(((uint32_t)min(row, mrows - 1) * (uint32_t)ldx + (uint32_t)piece * 8u) * 2u);
    }
    constexpr int LPSW = 2 * (SG::WPW + SG::AI) + SG::SPW;
    // Scales (one row per group): half k = wave % 2 of the tile's 128 (waves 2..7 repeat
    // them).  Group 32: scale row wave of the stage's four, both halves from s_voff.
    const int s_half = SG::NSG == 1 ? wave & 1 : 0;
    const int s_voff = min(n0 + 64 * s_half + lane, N - 1) * 4;

    float acc[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mt][r] = 0.0f;

#pragma unroll
    for (int k = 0; k < D - 1; ++k)
        if (k < ng && wave < 4) {
            w4_issue<BITS, GS, MT, KS, D>(lds + k * SG::BYTES, g0 + k, wave, N, wr, xr, sr, w_voff, a_voff, a_ins,
                                       s_half, s_voff);
            w4_issue_partner<BITS, GS, MT, KS, D>(lds + k * SG::BYTES, g0 + k, wave, N, wr, xr, w_voff, a_voffp,
                                               a_insp);
        }

    // This lane's B words: column 16*wave + li of packed row 4*ks + lb (4 bits) or of
    // packed rows 8*ks + 2*lb and the next (8 bits): the K values 32*ks + 8*lb .. +7.
    const int cl = 16 * wave + li;
    constexpr int BW = BITS == 4 ? 1 : 2;
    int b_off[KS][BW];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < BW; ++e) {
            const int r = BITS == 4 ? 4 * ks + lb : 8 * ks + 2 * lb + e;
            b_off[ks][e] = (r * kTN + (((cl >> 2) ^ w4_swz<BITS>(r)) << 2) + (cl & 3)) * 4;
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
            w4_issue<BITS, GS, MT, KS, D>(nst, g0 + u + D - 1, wave, N, wr, xr, sr, w_voff, a_voff, a_ins, s_half,
                                       s_voff);
            w4_issue_partner<BITS, GS, MT, KS, D>(nst, g0 + u + D - 1, wave, N, wr, xr, w_voff, a_voffp, a_insp);
        }
        __builtin_amdgcn_sched_barrier(0);
        const char *st = lds + slot * SG::BYTES;
        // The stage's KS words are dequantised first, at raised wave priority: with
        // the two waves of a SIMD both holding VALU work, the dequantisation goes first
        // and the MFMAs that need it start sooner (measured 2-6% faster on the decode
        // layers at M = 8 and 64, except qkv at M = 8, 2% slower).
        v8bf bw[KS];
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if constexpr (BITS == 4)
                bw[ks] = dequant8x16((uint32_t)*reinterpret_cast<const int *>(st + b_off[ks][0]));
            else
                bw[ks] = dequant8x8((uint32_t)*reinterpret_cast<const int *>(st + b_off[ks][0]),
                                    (uint32_t)*reinterpret_cast<const int *>(st + b_off[ks][1]));
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        v4f p[MT];
        const float *const srow = reinterpret_cast<const float *>(st + SG::WB + SG::AB);
        constexpr int KSG = GS / 32;  // K steps per group
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const v8bf b = bw[ks];
            // a group's first K step starts a fresh sum
            const bool fresh = ks % KSG == 0;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int row = mt * 16 + li;
                const v4i a =
                    *reinterpret_cast<const v4i *>(st + SG::WB + row * SG::ROWB + (((4 * ks + lb) ^ li) << 4));
                p[mt] = mfma_bf16(a, b, fresh ? v4f{0.f, 0.f, 0.f, 0.f} : p[mt]);
            }
            if (ks % KSG == KSG - 1) {
                // the group's sum, scaled (4 bits: the sums are of 16*q, the scale takes the
                // 1/16, exact)
                const float sc = srow[(ks / KSG) * kTN + cl] * (BITS == 4 ? 0.0625f : 1.0f);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[mt][r] += sc * p[mt][r];
            }
        }
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
    int MT, KS, S, tiles, blocks, chunks;
    bool one_per_cu;  // the CU's whole LDS is this workgroup's
};

W4Plan w4_plan(int M, int N, int K, int bits) {
    W4Plan p;
    p.tiles = (N + kTN - 1) / kTN;
    // Layers whose tiles and row chunks fill at most half the CUs (the narrow decode layers)
    // take one workgroup per CU: as many K splits as fit, rounded down.  Measured against
    // the 1.5 per CU they took before (whose rounding up left some CUs with two workgroups):
    // qkv 2-9%, o_proj 10-16% and down up to 14% faster at 1 to 64 rows.  Wider layers
    // target 1.5 workgroups per CU (two fit on a CU, and the second one's waves hide the
    // first one's dequantisation and barrier latencies), or 3 per CU with more tiles than
    // CUs (gate_up: 34.5 -> 31.8 us at M = 8).
    const int cus = device_cu_count();
    const int P = p.tiles > cus ? 3 * cus : 3 * cus / 2;
    auto plan = [&](int mt) {
        p.MT = mt;
        // 4 bits with one 16-row m tile: two groups per stage (the stage then carries as
        // many weight bytes as an 8-bit one, and the per-stage hand-off is paid half as often)
        p.KS = bits == 4 && mt == 1 && K % 256 == 0 ? 8 : 4;
        const int G = K / (32 * p.KS);  // stages
        p.chunks = (M + 16 * mt - 1) / (16 * mt);
        const int units = p.tiles * p.chunks;
        p.one_per_cu = 2 * units <= cus;
        int S = p.one_per_cu ? cus / units : (P + units - 1) / units;
        if (S > G) S = G;
        if (S < 1) S = 1;
        if (units > kMaxCounters) S = 1;
        p.S = S;
    };
    plan(M >= 64 ? 4 : (M + 15) / 16);
    // Narrow layers at M > 32: when the splits would leave a workgroup fewer than 8 groups,
    // chunks of 32 rows (twice the workgroups per tile, half the splits) are faster
    // (measured at M = 64: qkv 20.2 -> 18.1 us, o_proj 20.3 -> 15.9 us; wide layers lose).
    if (p.MT > 2 && K / kGroup < 8 * p.S) plan(2);
    p.blocks = ((p.tiles * p.S + 7) / 8) * 8;
    return p;
}

// As many stages as fit in BUDGET KiB, at most 6.
template <int BITS, int GS, int MT, int KS, int BUDGET>
hipError_t launch_w4_ring(const W4A16Args &a, const W4Plan &p, hipStream_t st) {
    constexpr int FIT = (BUDGET * 1024 - 16) / W4Stage<BITS, GS, MT, KS>::BYTES;
    constexpr int D = FIT < 6 ? FIT : 6;
    static_assert(D >= 2, "at least two stages");
    int *cnt = p.S > 1 ? a.counters : nullptr;
    float *part = p.S > 1 ? (float *)a.ws : nullptr;
    dim3 grid(p.blocks, p.chunks);
    w4a16_stream_kernel<BITS, GS, MT, KS, D><<<grid, 512, 0, st>>>(a.x, a.ldx, a.qweight, a.w_scale, a.y, a.ldy,
                                                                  a.M, a.N, a.K, p.S, p.tiles, part,
                                                                  p.S > 1 ? a.ws_bytes : 0, cnt);
    return hipGetLastError();
}

// The ring takes 80 KiB, so that two workgroups share a CU, except where 80 KiB holds
// only two stages (8-bit codes at 48 or 64 rows) and the workgroup has the CU to itself:
// then the whole LDS (four stages at 64 rows: down at M = 64 38.2 -> 33.3 us, qkv
// 19.9 -> 18.8 us; deeper rings where 80 KiB already holds three stages measured 5-12%
// slower).
template <int BITS, int GS, int MT, int KS>
hipError_t launch_w4_mt(const W4A16Args &a, const W4Plan &p, hipStream_t st) {
    if constexpr ((80 * 1024 - 16) / W4Stage<BITS, GS, MT, KS>::BYTES < 3)
        if (p.one_per_cu) return launch_w4_ring<BITS, GS, MT, KS, 160>(a, p, st);
    return launch_w4_ring<BITS, GS, MT, KS, 80>(a, p, st);
}

template <int BITS, int GS>
hipError_t launch_w4_bits(const W4A16Args &a, const W4Plan &p, hipStream_t s) {
    switch (p.MT) {
        case 1:
            if constexpr (BITS == 4)
                if (p.KS == 8) return launch_w4_mt<BITS, GS, 1, 8>(a, p, s);
            return launch_w4_mt<BITS, GS, 1, 4>(a, p, s);
        case 2: return launch_w4_mt<BITS, GS, 2, 4>(a, p, s);
        case 3: return launch_w4_mt<BITS, GS, 3, 4>(a, p, s);
        default: return launch_w4_mt<BITS, GS, 4, 4>(a, p, s);
    }
}

}  // namespace

// Partial-sum bytes after the counter region (0 when K is not split).
// Enough for either code width (the 4-bit plan splits K at most as often as the 8-bit one).
size_t w4a16_gemm_workspace(int M, int N, int K) {
    size_t bytes = 0;
    for (const int bits : {4, 8}) {
        const W4Plan p = w4_plan(M, N, K, bits);
        if (p.S > 1)
            bytes = std::max(bytes, align256(size_t(p.tiles) * p.chunks * p.S * 8 * p.MT * 4 * 64 * sizeof(float)));
    }
    return bytes;
}

hipError_t launch_w4a16_gemm(const W4A16Args &a, hipStream_t s) {
    const W4Plan p = w4_plan(a.M, a.N, a.K, a.bits);
    if (a.bits == 8) return a.group == 32 ? launch_w4_bits<8, 32>(a, p, s) : launch_w4_bits<8, 128>(a, p, s);
    return launch_w4_bits<4, 128>(a, p, s);
}

}  // namespace i8gs
