// W8A8 G128 GEMM for prefill shapes (M > 64): 256 x 256 output tiles on 32x32x32 int8
// MFMA (the operation and its citations are in w8a8.hip and include/i8gs.h).
#include <algorithm>
#include <type_traits>

#include "internal.h"

namespace i8gs {
namespace {

typedef int v16i __attribute__((ext_vector_type(16)));

// v_mfma_i32_32x32x32_i8: lane l holds row l % 32 of A and column l % 32 of B, 16
// consecutive K bytes at 16*(l / 32) of the 32-wide K step; register i of the result
// holds column l % 32, row 8*(i / 4) + 4*(l / 32) + i % 4.
__device__ __forceinline__ v16i mfma32_i8(v4i a, v4i b, v16i c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// // Bound by the MFMA units and, as much, by the VALU: folding a 32x32 int32 group sum
// into fp32 takes a convert and an FMA per value, 32 wave-wide VALU ops per lane that
// cost as many cycles as the tile's four MFMAs.  A workgroup (8 waves, one per CU: its
// LDS takes 130 KiB) owns a 256 x 256 output tile and walks the K groups with a
// 2-stage LDS ring filled by buffer_load ... lds: a stage holds the group's 256
// activation rows (128 bytes, pieces XOR-swizzled by row % 8), the 32 packed weight
// rows of the tile's 256 columns (rows 4..7 of every 8 shifted by 8 pieces, so the two
// lane halves of a B read hit different banks) and their scales.  The next stage's
// copies go into the slot that the barrier at the top of the group has freed, issued
// in pairs (one activation and one weight copy each) behind the MFMAs of the group's
// first four chains: issued all at once right after the barrier, they stalled every
// wave for about a fifth of the group while the vector memory path took them in.
// Waves 0-3 issue all of them, their own share and that of wave + 4 on the same SIMD:
// the SIMD's issue arbitration favours the older wave, so waves 0-3 finished each
// group's compute about a third sooner than waves 4-7 and then idled at the barrier;
// taking the copies' issue stalls on themselves, they now finish closer together.
//
// Wave w owns rows 128*(w / 4) .. +127 and columns 64*(w % 4) .. +63 of the tile:
// 4 m tiles x 2 column fragments of 32x32.  Per group it reads its B fragments (the
// words of packed rows 8*ks + 4*h + i of its column, as in the decode kernel) and, one
// m tile ahead, its A fragments.  Two waves per SIMD let one wave's folds run under
// the other's MFMAs.

constexpr int kPB = 256;                      // prefill tile rows and columns
constexpr int kPrefillMaxSplits = 4;          // K splits of a tile in the last round
constexpr int kPrefillMinGroups = 16;         // K groups per split, at least (the pieces'
                                              // traffic outweighs shorter ones: o_proj)
constexpr int kPStageA = kPB * 128;           // activation bytes of a stage
constexpr int kPStageB = 32 * kPB * 4;        // weight bytes of a stage
constexpr int kPStage = kPStageA + kPStageB + kPB * 4;

// The kernel body, built twice: folding into y (PARTIALS false) and writing the exact
// group sums to Pout (PARTIALS true), each called by a plain kernel: lambdas that call
// AMDGPU builtins inside a kernel template lose the host-side launch stub.
template <bool PARTIALS>
__device__ __forceinline__ void prefill_body(const int8_t *__restrict__ qa, const float *__restrict__ a_scale,
                                             const int32_t *__restrict__ qweight, const float *__restrict__ w_scale,
                                             uint16_t *__restrict__ y, int64_t ldy, int M, int N, int K, int full,
                                             int S, float *__restrict__ part, int *__restrict__ cnt,
                                             int32_t *__restrict__ Pout) {
    __shared__ __attribute__((aligned(1024))) char lds[2 * kPStage];
    const int mtiles = (M + kPB - 1) / kPB, ntiles = (N + kPB - 1) / kPB;
    const int P = mtiles * ntiles;
    // Work items, in launch order: the first `full` tiles whole, then each of the last
    // P - full tiles as S K-splits (they fill the last round of workgroups; a split
    // tile's pieces are summed as in the decode kernel).  Logical tile L = nt * mtiles +
    // mt; the whole tiles are placed XCD-aware (see the decode kernel), so the m tiles of
    // one column tile -- which read the same weights -- share an XCD.
    const int F8 = (full + 7) & ~7;
    int L, s = 0;
    if ((int)blockIdx.x < F8) {
        L = (blockIdx.x & 7) * (F8 >> 3) + (blockIdx.x >> 3);
        if (L >= full) return;
    } else {
        const int q = blockIdx.x - F8;
        L = full + q / S;
        s = q - (q / S) * S;
        if (L >= P) return;
    }
    const bool split = L >= full;
    const int mt = L % mtiles, nt = L / mtiles;
    const int m0 = mt * kPB, n0 = nt * kPB;
    const int G = K >> 7;
    const int g0 = split ? s * G / S : 0, g1 = split ? (s + 1) * G / S : G;  // this item's groups

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 31, h = lane >> 5;
    const int wm = wave >> 2, wn = wave & 3;

    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc((void *)qweight, 0, (int)((uint32_t)K * (uint32_t)N), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t ar =
        __builtin_amdgcn_make_buffer_rsrc((void *)qa, 0, (int)((uint32_t)M * (uint32_t)K), kRsrcWord3);
    // (partials mode: no scales are read; an empty range turns those copies into zeros)
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)w_scale, 0, PARTIALS ? 0 : (int)((uint32_t)G * (uint32_t)N * 4u), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)y, 0, (int)(((uint32_t)(M - 1) * (uint32_t)ldy + (uint32_t)N) * 2u), kRsrcWord3);

    // Copy roles: 32 activation copies (8 rows each) and 32 weight copies (half a
    // packed row each) per stage, 4 + 4 per wave, plus the 256 scales (waves 0..3).
    // LDS slot p of the 32 x 256 weight block holds row p / 64, piece (p % 64) ^ swz(row):
    // rows 4..7 of every 8 are shifted by 8 pieces (32 words), so the two halves of a
    // wave, which read rows 4 apart, use different banks.  A wave's four weight rows
    // 4*wave .. +3 share the swizzle, so one lane offset serves them all.
    int a_voff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = (wave * 4 + j) * 8 + (lane >> 3);
        const int piece = (lane & 7) ^ (row & 7);
        a_voff[j] = (int)((uint32_t)min(m0 + row, M - 1) * (uint32_t)K + (uint32_t)piece * 16u);
    }
    const int cp = min(n0 + (lane ^ (wave & 1 ? 8 : 0)) * 4, N - 4);
    const int w_voff = (int)(((uint32_t)(wave * 4) * (uint32_t)N + (uint32_t)cp) * 4u);
    const int s_voff = min(n0 + (wave & 3) * 64 + lane, N - 1) * 4;

    auto issue = [&](char *st, int g) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, I8GS_LDS(st + (wave * 4 + j) * 1024), 16, a_voff[j], g * 128,
                                                     0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, I8GS_LDS(st + kPStageA + (wave * 4 + j) * 1024), 16, w_voff,
                                                     (int)(((uint32_t)g * 32u + (uint32_t)j) * (uint32_t)N * 4u), 0, 0);
        if (wave < 4)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, I8GS_LDS(st + kPStageA + kPStageB + wave * 256), 4, s_voff,
                                                     (int)((uint32_t)g * (uint32_t)N * 4u), 0, 0);
    };
    // Copy pair j of group g into stage st: activation copy j, weight copy j, and the
    // scales with j = 0.
    auto issue_pair = [&](char *st, int g, int j) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, I8GS_LDS(st + (wave * 4 + j) * 1024), 16, a_voff[j], g * 128, 0,
                                                 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, I8GS_LDS(st + kPStageA + (wave * 4 + j) * 1024), 16, w_voff,
                                                 (int)(((uint32_t)g * 32u + (uint32_t)j) * (uint32_t)N * 4u), 0, 0);
        if (j == 0 && wave < 4)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, I8GS_LDS(st + kPStageA + kPStageB + wave * 256), 4, s_voff,
                                                     (int)((uint32_t)g * (uint32_t)N * 4u), 0, 0);
    };

    // Copy pair j of the share of wave + 4: its activation rows lie 128 further down, its
    // weight rows 16 further down.  Rows past M read zeros (past the end of qa) or, where
    // the 32-bit offset wraps, other bytes of qa; their results are never stored.
    auto issue_partner = [&](char *st, int g, int j) {
        uint32_t down = 128u * (uint32_t)K;
        __asm__ volatile("" : "+s"(down));  // added here, not kept in registers across the loop
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, I8GS_LDS(st + ((wave + 4) * 4 + j) * 1024), 16,
                                                 (int)((uint32_t)a_voff[j] + down), g * 128, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, I8GS_LDS(st + kPStageA + ((wave + 4) * 4 + j) * 1024), 16, w_voff,
                                                 (int)(((uint32_t)g * 32u + (uint32_t)j + 16u) * (uint32_t)N * 4u), 0, 0);
    };
    float acc[4][2][16];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][f][i] = 0.0f;

    // The fold here converts the plain int32 sums (v_cvt_f32_i32).  The seeded form the
    // decode kernel uses times the same but here holds its seed in 16 registers, which
    // the A prefetch needs.
    v16i pp = {};     // the chain folded under the next one and its scale (zero: adds an exact 0)
    float scp = 0.0f;
    issue(lds, g0);
    // The group loop, built twice: for the copying waves 0-3 (COPIER) and for waves 4-7.
    auto run = [&](auto copier_tag) {
    constexpr bool COPIER = decltype(copier_tag)::value;
    for (int g = g0; g < g1; ++g) {
        char *st = lds + ((g - g0) & 1) * kPStage;
        wait_vmcnt<0>();
        barrier_only();  // this stage is in; every wave is done with the other slot
        __builtin_amdgcn_sched_barrier(0);
        // The next group's copies, into the slot this barrier freed.  The last group copies
        // itself again into the idle slot instead of skipping them: a branch around the
        // copies splits the compiler's schedule and spills registers.
        char *const nst = lds + ((g + 1 - g0) & 1) * kPStage;
        const int gn = min(g + 1, g1 - 1);

        // B fragments of this wave's two 32-column fragments, offset binary -> int8.  Lane
        // half h reads rows 8*ks + 4*h + i, whose pieces are swizzled by 8*h.
        v4i b[2][4];
        float sc[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const int c = wn * 64 + f * 32 + col;
            const int cs = c ^ (h ? 32 : 0);
            const int *wcol = reinterpret_cast<const int *>(st + kPStageA) + cs;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int i = 0; i < 4; ++i) b[f][ks][i] = wcol[(8 * ks + 4 * h + i) * kPB];
            sc[f] = reinterpret_cast<const float *>(st + kPStageA + kPStageB)[c];
        }
        // Eight chains per group, chain c = (m tile c / 2, fragment c % 2): four dependent
        // MFMAs (the exact int32 group sum of one 32x32 tile), then the fold of chain
        // c - 1 into its fp32 accumulator (the last chain of a group is folded after the
        // first chain of the next), so the fold's VALU work has no MFMA result to wait
        // for and runs beside the MFMAs of this wave and of the other wave on the SIMD.
        // A fragments are read one m tile ahead.
        v4i a[4], an[4];
        {
            const int arow = wm * 128 + col;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                a[ks] = *reinterpret_cast<const v4i *>(st + arow * 128 + (((ks * 2 + h) ^ (arow & 7)) * 16));
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int mi = c >> 1, f = c & 1;
            if (f == 0 && mi < 3) {
                const int arow = wm * 128 + (mi + 1) * 32 + col;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    an[ks] = *reinterpret_cast<const v4i *>(st + arow * 128 + (((ks * 2 + h) ^ (arow & 7)) * 16));
            }
            v16i p;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) p = mfma32_i8(a[ks], b[f][ks] ^ (int)0x80808080, ks == 0 ? v16i{} : p);
            // The fold runs at raised wave priority, so that on a SIMD whose two waves both
            // have VALU work the fold goes first and the next MFMA chain is reached sooner
            // (measured 2-3% faster than without).
            const int pm = c == 0 ? 3 : (c - 1) >> 1, pf = c == 0 ? 1 : (c - 1) & 1;
            // copy pairs c of the next group, issued while this chain's MFMAs run
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (COPIER) {
                if (c < 4) {
                    issue_pair(nst, gn, c);
                    issue_partner(nst, gn, c);
                }
            }
            if constexpr (PARTIALS) {
                // this chain's exact group sums: rows m0 + 128*wm + 32*mi + 8*(i/4) + 4*h + i%4,
                // column n0 + 64*wn + 32*f + col
                const int rbase = m0 + wm * 128 + mi * 32 + 4 * h;
                const int cn = n0 + wn * 64 + f * 32 + col;
                if (cn < N) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int row = rbase + 8 * (i / 4) + i % 4;
                        if (row < M) Pout[((int64_t)row * G + g) * N + cn] = p[i];
                    }
                }
            } else {
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_setprio(1);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[pm][pf][i] += scp * (float)pp[i];
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_setprio(0);
                __builtin_amdgcn_sched_barrier(0);
                pp = p;
                scp = sc[f];
            }
            if (f == 1) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) a[ks] = an[ks];
            }
        }
    }
    };
    if (wave < 4)
        run(std::true_type{});
    else
        run(std::false_type{});
    wait_vmcnt<0>();  // the last group's extra copies: none may still be writing LDS when the waves end
    if constexpr (PARTIALS) return;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[3][1][i] += scp * (float)pp[i];

    if (split) {
        // Publish this split's piece (fp32, lane-interleaved: value i of lane l of wave w
        // at ((w * 128 + i) * 64 + l) floats; device-coherent), count arrivals, and let the
        // last split to arrive sum the S pieces in split order, so the result does not
        // depend on timing.
        const int tt = L - full;
        constexpr uint32_t kPiece = 8u * 128u * 64u * 4u;
        const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)part, 0, (int)((uint32_t)(P - full) * (uint32_t)S * kPiece), kRsrcWord3);
        const uint32_t cell0 = (uint32_t)tt * (uint32_t)S * kPiece + ((uint32_t)wave * 128u * 64u + lane) * 4u;
#pragma unroll
        for (int i = 0; i < 128; ++i)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, acc[i >> 5][(i >> 4) & 1][i & 15]), pr,
                                                  (int)cell0, (int)((uint32_t)s * kPiece + (uint32_t)i * 256u),
                                                  kCpolSC1);
        wait_vmcnt<0>();
        __syncthreads();
        int *const s_last = reinterpret_cast<int *>(lds);
        if (threadIdx.x == 0) {
            const int last = __hip_atomic_fetch_add(cnt + tt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
            if (last) __hip_atomic_store(cnt + tt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *s_last = last;
        }
        __syncthreads();
        if (!*s_last) return;
        // 16 values at a time: the S pieces' cells (this split's own too, already stored)
        // all in flight, then summed in split order
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float v[kPrefillMaxSplits][16];
#pragma unroll
            for (int q = 0; q < kPrefillMaxSplits; ++q)
                if (q < S) {
#pragma unroll
                    for (int k = 0; k < 16; ++k)
                        v[q][k] = __builtin_bit_cast(
                            float, __builtin_amdgcn_raw_buffer_load_b32(
                                       pr, (int)cell0, (int)((uint32_t)q * kPiece + (uint32_t)(c * 16 + k) * 256u),
                                       kCpolSC1));
                }
            // y = bf16(a_scale[row] * sum) for this chunk (m tile c / 2, fragment c % 2; the
            // layout of the whole-tile store below)
            const int rbase = m0 + wm * 128 + (c >> 1) * 32 + 4 * h;
            const int cn = n0 + wn * 64 + (c & 1) * 32 + col;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                float sum = v[0][k];
#pragma unroll
                for (int q = 1; q < kPrefillMaxSplits; ++q)
                    if (q < S) sum += v[q][k];
                const int row = rbase + 8 * (k / 4) + k % 4;
                const uint32_t off = ((uint32_t)row * (uint32_t)ldy + (uint32_t)cn) * 2u;
                __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(a_scale[min(row, M - 1)] * sum), yr,
                                                      (int)(cn < N ? off : 0x80000000u), 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);  // one chunk's loads in flight at a time
        }
        return;
    }

    // y = bf16(a_scale[row] * acc): lane (col, h) holds column n0 + 64*wn + 32*f + col,
    // rows m0 + 128*wm + 32*mi + 8*(i/4) + 4*h + i%4.
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int rbase = m0 + wm * 128 + mi * 32 + 4 * h;
        float as[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) as[i] = a_scale[min(rbase + 8 * (i / 4) + i % 4, M - 1)];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const int cn = n0 + wn * 64 + f * 32 + col;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = rbase + 8 * (i / 4) + i % 4;
                const uint32_t off = ((uint32_t)row * (uint32_t)ldy + (uint32_t)cn) * 2u;
                __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(as[i] * acc[mi][f][i]), yr,
                                                      (int)(cn < N ? off : 0x80000000u), 0, 0);
            }
        }
    }
}

__global__ __launch_bounds__(512) void w8a8_prefill_kernel(const int8_t *__restrict__ qa,
                                                           const float *__restrict__ a_scale,
                                                           const int32_t *__restrict__ qweight,
                                                           const float *__restrict__ w_scale,
                                                           uint16_t *__restrict__ y, int64_t ldy, int M, int N,
                                                           int K, int full, int S, float *__restrict__ part,
                                                           int *__restrict__ cnt) {
    prefill_body<false>(qa, a_scale, qweight, w_scale, y, ldy, M, N, K, full, S, part, cnt, nullptr);
}

__global__ __launch_bounds__(512) void w8a8_prefill_partials_kernel(const int8_t *__restrict__ qa,
                                                                    const int32_t *__restrict__ qweight, int M,
                                                                    int N, int K, int full, int S,
                                                                    int32_t *__restrict__ P) {
    // the scale pointers are not read (empty copy range); they point at valid memory
    prefill_body<true>(qa, (const float *)qa, qweight, (const float *)qweight, nullptr, 0, M, N, K, full, S, nullptr,
                       nullptr, P);
}

// ------------------------------------------------------------------ tiled kernel (group partials; M > 64 fallback)


// Prefill launch plan: whole tiles fill whole rounds of workgroups (one per CU); the
// tiles of a last, partial round are split along K, up to kPrefillMaxSplits ways and
// into at least kPrefillMinGroups groups each, so that round is about full too.
struct PrefillPlan {
    int tiles, full, S;
};

PrefillPlan prefill_plan(int M, int N, int K) {
    const int tiles = ((M + kPB - 1) / kPB) * ((N + kPB - 1) / kPB);
    const int cus = device_cu_count(), G = K / kGroup;
    const int tail = tiles % cus;
    const int S = tail ? std::min(std::min(kPrefillMaxSplits, G / kPrefillMinGroups), cus / tail) : 1;
    if (S < 2) return {tiles, tiles, 1};
    return {tiles, tiles - tail, S};
}

// The split tiles' fp32 pieces: 256 x 256 values per split.
size_t prefill_workspace(const PrefillPlan &p) {
    return p.S > 1 ? align256(size_t(p.tiles - p.full) * p.S * kPB * kPB * sizeof(float)) : 0;
}

}  // namespace

// The prefill kernel addresses y with 32-bit offsets and drops the rows past M by the y
// descriptor's range check, so the offsets of all the rows a launch covers -- M rounded
// up to the 256-row tiles -- must stay below 2^31 (no wrap back into range).
bool prefill_y_fits(int64_t M, int64_t ldy) { return (M + kPB - 1) / kPB * kPB * ldy * 2 < (int64_t(1) << 31); }

size_t prefill_gemm_workspace(int M, int N, int K) { return prefill_workspace(prefill_plan(M, N, K)); }

hipError_t launch_prefill(const W8A8Args &a, hipStream_t s) {
    PrefillPlan p = prefill_plan(a.M, a.N, a.K);
    if (a.P != nullptr) {
        // partials: each K split writes its own groups (no reduction)
        const int grid = ((p.full + 7) & ~7) + (p.tiles - p.full) * p.S;
        w8a8_prefill_partials_kernel<<<grid, 512, 0, s>>>(a.qa, a.qweight, a.M, a.N, a.K, p.full, p.S, a.P);
        return hipGetLastError();
    }
    if (p.S > 1 && (a.ws == nullptr || a.ws_bytes < prefill_workspace(p) || a.counters == nullptr))
        p = {p.tiles, p.tiles, 1};  // no room for the split pieces: whole tiles only
    const int grid = ((p.full + 7) & ~7) + (p.tiles - p.full) * p.S;
    w8a8_prefill_kernel<<<grid, 512, 0, s>>>(a.qa, a.a_scale, a.qweight, a.w_scale, a.y, a.ldy, a.M, a.N, a.K,
                                              p.full, p.S, (float *)a.ws, a.counters);
    return hipGetLastError();
}

}  // namespace i8gs
