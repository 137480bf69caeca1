// W8A8 G128 GEMM on gfx950 MFMA.
//
// Qwen3.8-27B GPTQ INT8 W8A8 GS128 PTQR model card, "Quantization details": true
// int8 x int8 compute at every decode and prefill shape with one weight scale per
// 128-wide K block.  Flint INT8 card, format table: GPTQ qweight/scales, symmetric,
// group 128, no g_idx.  For each 128-wide group the int8 products are summed exactly
// in an int32 MFMA accumulator, converted to fp32 and folded with that group's
// per-column scale; the row scale and the bf16 rounding are applied once at the end.
//
// GPTQ codes are offset binary (q + 128); XOR 0x80 per byte turns a code into the
// two's-complement int8 value of q.
//
// Three kernels:
//  * decode (M <= 64, w8a8_decode_kernel): bound by streaming the weights from HBM.
//    About one workgroup per CU streams its columns (and, for narrow layers, a part
//    of K) through an LDS ring filled by direct buffer-to-LDS copies;
//    v_mfma_i32_32x32x32_i8, four per 32x32 block and group.
//  * prefill (M > 64, w8a8_prefill_kernel, in w8a8_prefill.hip): 256 x 256 output
//    tiles, eight waves of 128 x 64; v_mfma_i32_32x32x32_i8 as in the decode kernel.
//  * tiled (w8a8_tiled_kernel): 128 x 128 tiles, four waves of 64 x 64,
//    v_mfma_i32_16x16x64_i8; the fallback when y is too large for 32-bit offsets
//    (or when asked for by I8GS_KERNEL_TILED).
// Each kernel also has a partials mode that writes the exact int32 group sums
// P[m, g, n] instead of folding them: the same loads, LDS layout and MFMA chains,
// with the fold and the output stage replaced by a store of each chain's result.
#include <algorithm>
#include <type_traits>

#include "internal.h"

namespace i8gs {
namespace {

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4i flip(v4i v) {
    return v ^ (int)0x80808080;
}

// ------------------------------------------------------------------ decode kernel
//
// Work split.  The launch is a grid of T column tiles x S K-splits, about one
// workgroup per CU.  Tile t covers columns [8*floor(t*N/8/T), 8*floor((t+1)*N/8/T));
// split s covers groups [floor(s*G/S), floor((s+1)*G/S)) of the G = K/128 groups.
// Wide layers take S = 1: every workgroup owns whole columns, streams all of K for
// them and writes y itself; its columns are walked in chunks of at most TN.  Narrow
// layers take S > 1 so that a tile stays about 64 columns wide or more (each streamed
// weight byte then costs at most one activation byte); the S workgroups of a tile
// each write an fp32 piece and the last of them to finish sums the pieces in split
// order, so the result does not depend on timing.
//
// Streaming.  Each workgroup (8 waves, two per SIMD; one workgroup per CU, the LDS
// ring takes most of the CU's 160 KiB) pulls its units -- (chunk, group) pairs, chunk-major -- through a
// D-stage ring in LDS filled by buffer_load ... lds: a stage holds the chunk's 32
// packed weight rows of the group (row-major, TN*4 bytes per row), the group's
// 32*M2 activation rows (128 bytes each) and the chunk's column scales.  The copies
// go straight from memory to LDS, so D-1 stages stay in flight without holding
// registers; four waves issue the copies, each waits for its own copies of the
// current stage (vmcnt), a barrier makes all of them visible, and the slot is
// refilled only after every wave is done with it.  Copies beyond the chunk's columns repeat its last piece (a cache
// hit), so every wave issues the same number of copies per stage.
//
// MFMA.  v_mfma_i32_32x32x32_i8: lane l holds row (l % 32) of A and column (l % 32)
// of B, 16 consecutive K bytes at 16*(l / 32) of a 32-wide K step (A and B use the
// same placement, so the product is the plain dot product); the 32x32 int32 result
// puts column l % 32, rows 8*(i / 4) + 4*(l / 32) + i % 4 in register i of lane l.
// On gfx950 this shape runs at about 2.6x the rate of the 16x16x64 one (measured).
// A is the activation rows (m tile of 32 tokens); B is a 32-column fragment of the
// chunk: lane (col, h) = (l % 32, l / 32) reads, for K step ks, the words of packed
// rows 8*ks + 4*h + i (i = 0..3) of its column -- 16 consecutive K bytes.  Wave w
// takes m tile w % M2 and fragments w / M2 + j * (8 / M2).
// Activations are stored with the 16-byte pieces of row r permuted by XOR with r % 8,
// so the rows read together fall in different bank groups.


constexpr int kMaxSplits = 8;

typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v16i mfma32_i8(v4i a, v4i b, v16i c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// Group sums leave the MFMA already shaped for a cheap fold.  A group's MFMA chain starts
// from the accumulator value kSumSeed (the fp32 bit pattern of 1/(2*pi), an inline
// constant of the MFMA's C operand) instead of 0.  Read as an fp32 number, the int32
// result kSumSeed + S equals f_seed + S * 2^-26 exactly while it stays in the seed's
// binade [1/8, 1/4) (bit patterns 0x3E000000 .. 0x3E7FFFFF), i.e. for
// -2292099 <= S <= 6096508, and a sum of 128 products of two int8 values lies within
// +-2097152.  f_seed minus that number is then exact
// (Sterbenz): -S * 2^-26 for one full-rate VALU op with an inline constant, where an
// int-to-float convert costs a half-rate one, and multiplying it by -scale * 2^26
// gives exactly the product scale * S that the fold adds.  (Scales must keep
// scale * 2^26 finite: |scale| < 2^100.)
constexpr int kSumSeed = 0x3E22F983;
constexpr float kSumScale = -67108864.0f;  // -2^26

__device__ __forceinline__ v16i sum_seed() {
    v16i c;
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = kSumSeed;
    return c;
}

// -S * 2^-26 from a seeded group sum (exact).
__device__ __forceinline__ float seeded_sum(int r) {
    return __builtin_bit_cast(float, kSumSeed) - __builtin_bit_cast(float, r);
}

// PARTIALS is part of the shape so that each kernel instantiation has shape types of
// its own: a device function template taking buffer resources, used with the same
// shape from two kernel instantiations, fails overload resolution in hipcc's host pass.
template <int M2, int TN, int W, bool PARTIALS>
struct DecodeShape {
    static_assert((M2 == 1 || M2 == 2) && W == 8 && TN % 8 == 0 && TN >= 8 && TN <= 256,
                  "unsupported decode shape");
    static constexpr int NF = (TN + 31) / 32;          // 32-column fragments of a chunk
    static constexpr int WPM = W / M2;                 // waves per m tile
    static constexpr int NFW = (NF + WPM - 1) / WPM;   // fragments per wave
    static constexpr int PPR = TN / 4;                 // 16-byte pieces per weight row
    // Copies are issued by four of the waves (the others only compute).
    static constexpr int WI = (TN + 31) / 32;          // 1 KiB weight copies per copying wave per stage
    static constexpr int WB = WI * 4096;               // weight bytes of a stage (TN*128 used)
    static constexpr int AI = M2;                      // 1 KiB activation copies per copying wave
    static constexpr int AB = M2 * 32 * 128;           // activation bytes of a stage
    static constexpr int SB = 1024;                    // scales (TN floats; copies past TN unused)
    static constexpr int STAGE = WB + AB + SB;
    static constexpr int LPS = WI + AI + 1;            // memory instructions per copying wave per stage
    static constexpr int TNV = TN;
    __device__ static int frag(int w, int j) { return w / M2 + j * WPM; }
    __device__ static int mtile(int w) { return w % M2; }
};


// Copies of one stage by this wave.  cb/cw: first column and width of the chunk.
template <class S>
__device__ __forceinline__ void decode_issue(char *st, __amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t ar,
                                             __amdgpu_buffer_rsrc_t sr, int wave, int lane, const int (&a_voff)[S::AI],
                                             int cb, int cw, int g, int N) {
    const int last_piece = (cw >> 2) - 1;
#pragma unroll
    for (int j = 0; j < S::WI; ++j) {
        const int ins = wave * S::WI + j;
        const int p = ins * 64 + lane;
        const int row = min(p / S::PPR, 31), cp = min(p % S::PPR, last_piece);
        const int voff = (int)(((uint32_t)row * (uint32_t)N + (uint32_t)(cb + 4 * cp)) * 4u);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, I8GS_LDS(st + ins * 1024), 16, voff,
                                                 (int)((uint32_t)g * 32u * (uint32_t)N * 4u), 0, kCpolNT);
    }
#pragma unroll
    for (int j = 0; j < S::AI; ++j) {
        const int ins = wave * S::AI + j;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, I8GS_LDS(st + S::WB + ins * 1024), 16, a_voff[j], g * 128, 0, 0);
    }
    const int sc = cb + min(wave * 64 + lane, cw - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, I8GS_LDS(st + S::WB + S::AB + wave * 256), 4, sc * 4,
                                             (int)((uint32_t)g * (uint32_t)N * 4u), 0, 0);
}

// One stage on the MFMA units: all of this wave's LDS reads for the stage, then the
// MFMAs of every fragment -- four K steps giving the exact int32 group sums p, seeded
// (see sum_seed) -- and the fragments' column scales sc, times -2^26.  last_live is false when the wave's last fragment
// lies past the chunk (then it is skipped).
template <class S>
__device__ __forceinline__ void decode_mfma(const char *st, int wave, int lane, bool last_live, v16i (&p)[S::NFW],
                                            float (&sc)[S::NFW]) {
    const int col = lane & 31, h = lane >> 5;
    const int arow = S::mtile(wave) * 32 + col;
    v4i a[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        a[ks] = *reinterpret_cast<const v4i *>(st + S::WB + arow * 128 + (((ks * 2 + h) ^ (arow & 7)) * 16));
    v4i b[S::NFW][4];
#pragma unroll
    for (int j = 0; j < S::NFW; ++j) {
        if (j == S::NFW - 1 && !last_live) break;
        // columns past the chunk read a valid word; their results are never stored
        const int c = min(S::frag(wave, j) * 32 + col, S::TNV - 1);
        const int *wcol = reinterpret_cast<const int *>(st) + c;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int i = 0; i < 4; ++i) b[j][ks][i] = wcol[(8 * ks + 4 * h + i) * (S::PPR * 4)];
        sc[j] = reinterpret_cast<const float *>(st + S::WB + S::AB)[c] * kSumScale;
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int j = 0; j < S::NFW; ++j) {
            if (j == S::NFW - 1 && !last_live) break;
            p[j] = mfma32_i8(a[ks], b[j][ks] ^ (int)0x80808080, ks == 0 ? sum_seed() : p[j]);
        }
}

// The fold of one stage: acc += scale * group sum (sc holds scale * -2^26, p the seeded
// sums; a zero p with a zero sc adds an exact 0).
template <class S>
__device__ __forceinline__ void decode_fold(float (&acc)[S::NFW][16], const v16i (&p)[S::NFW],
                                            const float (&sc)[S::NFW], bool last_live) {
#pragma unroll
    for (int j = 0; j < S::NFW; ++j) {
        if (j == S::NFW - 1 && !last_live) break;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][i] += sc[j] * seeded_sum(p[j][i]);
    }
}

// Partials mode: the exact int32 group sums of one stage, decoded from the seeded
// MFMA results exactly as the fold decodes them (seeded_sum times -2^26 is the sum
// itself), written to P[row, g, column] for the rows below M and the chunk's columns.
template <class S>
__device__ __forceinline__ void decode_store_partials(int32_t *__restrict__ P, const v16i (&p)[S::NFW], int wave,
                                                      int lane, bool last_live, int row0, int kb, int kw, int g,
                                                      int M, int N, int G) {
    const int col = lane & 31;
#pragma unroll
    for (int j = 0; j < S::NFW; ++j) {
        if (j == S::NFW - 1 && !last_live) break;
        const int cl = S::frag(wave, j) * 32 + col;
        if (cl >= kw) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = row0 + 8 * (i / 4) + i % 4;
            if (row < M) P[((int64_t)row * G + g) * N + kb + cl] = (int)(seeded_sum(p[j][i]) * kSumScale);
        }
    }
}

template <int M2, int TN, int W, int D, bool PARTIALS>
__global__ __launch_bounds__(W * 64) void w8a8_decode_kernel(const int8_t *__restrict__ qa,
                                                          const float *__restrict__ a_scale,
                                                          const int32_t *__restrict__ qweight,
                                                          const float *__restrict__ w_scale,
                                                          uint16_t *__restrict__ y, int64_t ldy, int M, int N, int K,
                                                          int T, int S, float *__restrict__ part,
                                                          int *__restrict__ cnt) {
    using SH = DecodeShape<M2, TN, W, PARTIALS>;
    // partials mode: `part` is the int32 output P [M, K/128, N] (there is no split reduction)
    int32_t *const Pout = reinterpret_cast<int32_t *>(part);
    constexpr int NFW = SH::NFW;
    // At least 82 KiB, so that no CU takes two of these workgroups while another has
    // none (the grid is about one workgroup per CU).
    // After the ring: the split-arrival flag (16 bytes) and the 64 row scales (256 bytes).
    constexpr int RING = D * SH::STAGE;
    constexpr int LDS_BYTES = RING + 512 > 82 * 1024 ? RING + 512 : 82 * 1024;
    static_assert(D >= 2 && LDS_BYTES <= 160 * 1024, "LDS ring too large");
    // One LDS object only: with a second one the compiler can no longer tell the
    // ring's reads from the copies in flight and waits for all of them.
    __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];

    // XCD-aware placement: workgroups are dealt to the 8 XCDs round-robin by launch
    // index, so logical workgroup L (tile-major: L = t*S + s) is launched at index
    // (L % Q) * 8 + L / Q with Q = ceil(P/8).  Each XCD then holds a contiguous run
    // of tiles: neighbouring tiles share the cache lines at their borders in one L2,
    // and the S splits of a tile meet in one L2 too.  (Only speed depends on this.)
    const int P = T * S, Q = (P + 7) >> 3;
    const int L = (blockIdx.x & 7) * Q + (blockIdx.x >> 3);
    if (L >= P) return;
    const int t = L / S, s = L - (L / S) * S;
    const int G = K >> 7, NG = N >> 3;
    const int c0 = 8 * (int)((int64_t)t * NG / T), c1 = 8 * (int)((int64_t)(t + 1) * NG / T);
    const int g0 = s * G / S, g1 = (s + 1) * G / S;
    if (c0 >= c1 || g0 >= g1) return;
    const int wg8 = (c1 - c0) >> 3;           // 8-column granules of the tile
    const int nch = (c1 - c0 + TN - 1) / TN;  // chunks of at most TN columns
    const int ng = g1 - g0;
    const int units = nch * ng;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 31, h = lane >> 5;
    const int row0 = SH::mtile(wave) * 32 + 4 * h;  // this lane's output rows: row0 + 8*(i/4) + i%4

    // byte offsets fit 32 bits: K*N < 2^32, M*K < 2^32 and 32*M2*ldy*2 < 2^31 are checked
    // before launch
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc((void *)qweight, 0, (int)((uint32_t)K * (uint32_t)N), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t ar =
        __builtin_amdgcn_make_buffer_rsrc((void *)qa, 0, (int)((uint32_t)M * (uint32_t)K), kRsrcWord3);
    // (partials mode: no scales are read; an empty range turns those copies into zeros)
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)w_scale, 0, PARTIALS ? 0 : (int)((uint32_t)G * (uint32_t)N * 4u), kRsrcWord3);
    // y stores go through a descriptor whose range check drops rows >= M: their offsets
    // are at least M*ldy*2 and below 2^31 (the padded rows, 32*M2 of them, are checked
    // before launch); columns past the chunk are sent past the end explicitly.
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)y, 0, (int)(((uint32_t)(M - 1) * (uint32_t)ldy + (uint32_t)N) * 2u), kRsrcWord3);

    // Activation copies: LDS slot lane % 8 of row 8*copy + lane / 8 holds piece
    // slot ^ (row % 8) of that row (rows past M repeat row M - 1; their results are
    // never stored).
    // With 8 waves, four of them issue the copies.  Where every wave computes exactly one
    // fragment those are waves 0-3: the SIMD's issue arbitration favours the older of its
    // two waves, and the copies' issue stalls then fall on the favoured one (3% faster
    // on the 128-column down tiles).  Otherwise waves 4-7: the first waves carry the
    // extra fragments (frag(w, j) = w / M2 + j * 8 / M2), or, with 64-column chunks,
    // waves 4-7 have no fragment at all.
    const int cwave = wave & 3;
    const bool copier = SH::NF == SH::WPM ? wave < 4 : wave >= 4;
    int a_voff[SH::AI];
#pragma unroll
    for (int j = 0; j < SH::AI; ++j) {
        const int row = (cwave * SH::AI + j) * 8 + (lane >> 3);
        const int piece = (lane & 7) ^ (row & 7);
        a_voff[j] = (int)((uint32_t)min(row, M - 1) * (uint32_t)K + (uint32_t)piece * 16u);
    }

    // The 64 row scales are copied into LDS by the first copying wave ahead of its first
    // stage (rows past M read as 0): that wave's wait for the first stage covers this older
    // copy too (copies complete in order), so the scales are in LDS, behind the first
    // barrier, before any chunk can end.
    float *const lds_as = reinterpret_cast<float *>(lds + RING + 256);
    if (copier && cwave == 0) {
        const __amdgpu_buffer_rsrc_t asr =
            __builtin_amdgcn_make_buffer_rsrc((void *)a_scale, 0, PARTIALS ? 0 : (int)((uint32_t)M * 4u), kRsrcWord3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(asr, I8GS_LDS(lds_as), 4, lane * 4, 0, 0, 0);
    }

    // All tiles walk their groups in the same order, so neighbouring tiles read the
    // cache lines they share at about the same time.
    const int gstart = g0;
    // copy cursor: chunk ci (columns [cb, cb + cw)), group gi, step ki within the chunk
    int ci = 0, gi = gstart, ki = 0;
    int cb = c0, cw = 8 * (wg8 / nch);
#pragma unroll
    for (int k = 0; k < D - 1; ++k) {
        if (k < units) {
            if (copier) decode_issue<SH>(lds + k * SH::STAGE, wr, ar, sr, cwave, lane, a_voff, cb, cw, gi, N);
            if (++gi == g1) gi = g0;
            if (++ki == ng) {
                ki = 0;
                ++ci;
                cb = c0 + 8 * (ci * wg8 / nch);
                cw = c0 + 8 * ((ci + 1) * wg8 / nch) - cb;
            }
        }
    }

    // Only a wave's last fragment can lie past the chunk's last fragment.
    const bool last_live = SH::frag(wave, NFW - 1) < SH::NF;
    float acc[NFW][16];
    v16i p_prev[NFW];  // group sums of the previous stage, not yet folded
    float sc_prev[NFW];
#pragma unroll
    for (int j = 0; j < NFW; ++j) {
        sc_prev[j] = 0.0f;
        p_prev[j] = v16i{};
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][i] = 0.0f;
    }

    int kc = 0, kk = 0;  // chunk and step being computed
    int slot = 0;
    for (int u = 0; u < units; ++u) {
        // Memory operations complete in order and the next D-2 stages are the youngest
        // copies, so this count waits for this stage.  A store issued at the end of a
        // chunk is younger still and makes the wait longer, not shorter.
        if (u + D - 2 < units) wait_vmcnt<(D - 2) * SH::LPS>();
        else wait_vmcnt<0>();
        barrier_only();
        __builtin_amdgcn_sched_barrier(0);
        if (u + D - 1 < units) {
            const int ns = slot == 0 ? D - 1 : slot - 1;  // slot of the previous stage, now free
            if (copier) decode_issue<SH>(lds + ns * SH::STAGE, wr, ar, sr, cwave, lane, a_voff, cb, cw, gi, N);
            if (++gi == g1) gi = g0;
            if (++ki == ng) {
                ki = 0;
                ++ci;
                cb = c0 + 8 * (ci * wg8 / nch);
                cw = c0 + 8 * ((ci + 1) * wg8 / nch) - cb;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // Software pipeline: this stage's MFMAs run while the previous stage is folded
        // (zeros at a chunk's first stage: that fold adds exact +0).
        v16i p_cur[NFW];
        float sc_cur[NFW];
        decode_mfma<SH>(lds + slot * SH::STAGE, wave, lane, last_live, p_cur, sc_cur);
        if constexpr (PARTIALS) {
            const int pb = c0 + 8 * (kc * wg8 / nch), pw = c0 + 8 * ((kc + 1) * wg8 / nch) - pb;
            decode_store_partials<SH>(Pout, p_cur, wave, lane, last_live, row0, pb, pw, g0 + kk, M, N, G);
            slot = slot == D - 1 ? 0 : slot + 1;
            if (++kk == ng) {
                kk = 0;
                ++kc;
            }
            continue;
        } else {
            decode_fold<SH>(acc, p_prev, sc_prev, last_live);
        }
#pragma unroll
        for (int j = 0; j < NFW; ++j) {
            p_prev[j] = p_cur[j];
            sc_prev[j] = sc_cur[j];
        }
        slot = slot == D - 1 ? 0 : slot + 1;

        if (++kk < ng) continue;
        // ---- end of chunk kc
        decode_fold<SH>(acc, p_prev, sc_prev, last_live);
#pragma unroll
        for (int j = 0; j < NFW; ++j) {
            p_prev[j] = v16i{};
            sc_prev[j] = 0.0f;
        }
        kk = 0;
        const int kb = c0 + 8 * (kc * wg8 / nch), kw = c0 + 8 * ((kc + 1) * wg8 / nch) - kb;
        ++kc;
        if (S == 1) {
            // y = bf16(a_scale[row] * sum): this lane's column, 16 rows
            v4f as[4];  // as[i / 4][i % 4]: row row0 + 8*(i/4) + i%4
#pragma unroll
            for (int q = 0; q < 4; ++q) as[q] = *reinterpret_cast<const v4f *>(lds_as + row0 + 8 * q);
#pragma unroll
            for (int j = 0; j < NFW; ++j) {
                const int cl = SH::frag(wave, j) * 32 + col;  // column within the chunk
                const uint32_t cbyte = cl < kw ? (uint32_t)(kb + cl) * 2u : 0x80000000u;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = row0 + 8 * (i / 4) + i % 4;
                    const uint32_t off = cbyte + (uint32_t)row * (uint32_t)ldy * 2u;
                    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(as[i / 4][i % 4] * acc[j][i]), yr,
                                                          (int)(cl < kw ? off : 0x80000000u), 0, 0);
                    acc[j][i] = 0.0f;
                }
            }
        }
    }
    if (S == 1 || PARTIALS) return;

    // ---- split tile (one chunk): publish this split's piece (fp32 [row][32*NF]; every
    // fragment lane, also those past the chunk, has its own place; device-coherent),
    // count arrivals, and let the last split to arrive sum all pieces in split order
    // (its own from registers: the same values it stored).
    constexpr int PW = 32 * SH::NF;  // piece row pitch in floats
    const int piece_bytes = 64 * PW * 4;
    const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)part, 0, (int)((uint32_t)T * (uint32_t)S * (uint32_t)piece_bytes), kRsrcWord3);
#pragma unroll
    for (int j = 0; j < NFW; ++j) {
        if (SH::frag(wave, j) >= SH::NF) break;
        const int cell0 = (row0 * PW + SH::frag(wave, j) * 32 + col) * 4;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, acc[j][i]), pr,
                                                  cell0 + ((8 * (i / 4) + i % 4) * PW) * 4, (s * T + t) * piece_bytes,
                                                  kCpolSC1);
    }
    wait_vmcnt<0>();
    __syncthreads();
    int *const s_last = reinterpret_cast<int *>(lds + RING);
    if (threadIdx.x == 0) {
        const int last = __hip_atomic_fetch_add(cnt + t, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
        if (last) __hip_atomic_store(cnt + t, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_last = last;
    }
    __syncthreads();
    if (!*s_last) return;

    // The last split sums the pieces in split order: the other splits' cells are
    // loaded QB pieces at a time, all in flight together, and its own come from
    // registers (the same values it stored).
    constexpr int QB = NFW > 1 ? 2 : 4;
    v4f as[4];  // as[i / 4][i % 4]: row row0 + 8*(i/4) + i%4
#pragma unroll
    for (int q = 0; q < 4; ++q) as[q] = *reinterpret_cast<const v4f *>(lds_as + row0 + 8 * q);
    float sum[NFW][16];
    for (int q0 = 0; q0 < S; q0 += QB) {
        float v[QB][NFW][16];
#pragma unroll
        for (int k = 0; k < QB; ++k) {
            const int q = q0 + k;
            if (q >= S) break;
#pragma unroll
            for (int j = 0; j < NFW; ++j) {
                if (SH::frag(wave, j) >= SH::NF) break;
                const int cell0 = (row0 * PW + SH::frag(wave, j) * 32 + col) * 4;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    v[k][j][i] = q == s ? acc[j][i]
                                        : __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                                        pr, cell0 + ((8 * (i / 4) + i % 4) * PW) * 4,
                                                                        (q * T + t) * piece_bytes, kCpolSC1));
            }
        }
#pragma unroll
        for (int k = 0; k < QB; ++k) {
            const int q = q0 + k;
            if (q >= S) break;
#pragma unroll
            for (int j = 0; j < NFW; ++j) {
                if (SH::frag(wave, j) >= SH::NF) break;
#pragma unroll
                for (int i = 0; i < 16; ++i) sum[j][i] = q == 0 ? v[k][j][i] : sum[j][i] + v[k][j][i];
            }
        }
    }
#pragma unroll
    for (int j = 0; j < NFW; ++j) {
        if (SH::frag(wave, j) >= SH::NF) break;
        const int cl = SH::frag(wave, j) * 32 + col;
        const uint32_t cbyte = (uint32_t)(c0 + cl) * 2u;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = row0 + 8 * (i / 4) + i % 4;
            const uint32_t off = cbyte + (uint32_t)row * (uint32_t)ldy * 2u;
            __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(as[i / 4][i % 4] * sum[j][i]), yr,
                                                  (int)(cl < c1 - c0 ? off : 0x80000000u), 0, 0);
        }
    }
}


#ifndef I8GS_DECODE_STAGES
#define I8GS_DECODE_STAGES 3  // upper bound on the LDS ring's stages
#endif

// Chunk widths the decode kernel is built for (multiples of 8 columns).
constexpr int kDecodeTN[] = {32, 48, 64, 80, 96, 128, 144, 192, 256};

struct DecodePlan {
    int T, S;  // column tiles x K splits (the grid)
    int tn;    // chunk width the kernel is built for
    int m2;    // 32-row m tiles (1 or 2)
};

DecodePlan decode_plan(int M, int N, int K, int workgroups) {
    DecodePlan p;
    const int G = K / kGroup, NG = N / 8;
    const int64_t P = workgroups > 0 ? workgroups : (int64_t)device_cu_count();
    // K splits so that a tile keeps about 64 columns: S = ceil(64 P / N)
    int64_t S = (64 * P + N - 1) / N;
    S = std::max<int64_t>(1, std::min<int64_t>(S, std::min(kMaxSplits, G)));
    int64_t T = std::max<int64_t>(1, std::min<int64_t>(P / S, NG));
    if (S > 1 && T > kMaxCounters) T = kMaxCounters;
    int maxw = 8 * (int)((NG + T - 1) / T);  // widest tile
    if (S > 1 && maxw > 256) {  // a split tile is one chunk
        S = 1;
        T = std::max<int64_t>(1, std::min<int64_t>(P, NG));
        maxw = 8 * (int)((NG + T - 1) / T);
    }
    // Narrow layers: tiles of whole 32-column fragments work best (measured on the drafter
    // layers).  128-column tiles give every wave exactly one fragment x m tile per group,
    // so they win when each split still has at least 16 groups to stream; otherwise
    // 64-column tiles with at least 8 groups per split, else the split above.
    bool whole_fragments = false;
    if (S > 1) {
        for (const int w : {128, 64}) {
            const int64_t Tw = (N + w - 1) / w;
            const int64_t Sw = std::min<int64_t>(std::min<int64_t>(kMaxSplits, G), P / Tw);
            if (Sw >= 2 && Tw <= kMaxCounters && G >= (w == 128 ? 16 : 8) * Sw) {
                T = Tw;
                S = Sw;
                maxw = 8 * (int)((NG + T - 1) / T);
                whole_fragments = true;
                break;
            }
            // 128-column tiles with about 10 groups per split, when that still makes at least
            // 4 splits and fills three quarters of the grid: fewer tiles re-read the
            // activations (qkv: 48 x 4 measured 7% faster than 96 x 2 of 64 columns; o_proj
            // and down keep their plans, which measured faster than any other)
            const int64_t S10 = std::min<int64_t>(std::min<int64_t>(kMaxSplits, G / 10), P / Tw);
            if (w == 128 && S10 >= 4 && Tw <= kMaxCounters && 4 * Tw * S10 >= 3 * P) {
                T = Tw;
                S = S10;
                maxw = 8 * (int)((NG + T - 1) / T);
                whole_fragments = true;
                break;
            }
        }
    }
    // Few columns and few groups at once (one GPU's share of a tensor-parallel layer:
    // 1536 or 8704 columns, or 8 groups): neither width above keeps its groups per split
    // at the full grid.  Rather than many splits of 2-5 groups, whose pieces then cost
    // more to sum than they save, cap the splits: 64-column tiles with at least 8 groups
    // per split (G/2 when K is that short), else 128-column tiles with at least 16, as
    // long as a quarter of the target grid stays busy (qkv, o_proj and gate/up shares
    // measured 10%, 12% and 7% faster than with the split above).
    if (S > 1 && !whole_fragments) {
        for (const int w : {64, 128}) {
            const int64_t Tw = (N + w - 1) / w;
            const int minG = std::min(w == 128 ? 16 : 8, G / 2);
            if (minG < 1) continue;
            const int64_t Sw = std::min<int64_t>(std::min<int64_t>(kMaxSplits, P / Tw), G / minG);
            if (Sw >= 2 && Tw <= kMaxCounters && Tw * Sw * 4 >= P) {
                T = Tw;
                S = Sw;
                maxw = 8 * (int)((NG + T - 1) / T);
                break;
            }
        }
    }
    const int nch = (maxw + 255) / 256;
    const int chunk = 8 * ((maxw / 8 + nch - 1) / nch);
    p.tn = 256;
    for (int tn : kDecodeTN)
        if (tn >= chunk) { p.tn = tn; break; }
    p.T = (int)T;
    p.S = (int)S;
    p.m2 = M <= 32 ? 1 : 2;
    return p;
}

// One fp32 piece (64 rows x the chunk width rounded up to 32) per workgroup when K
// is split.
size_t decode_workspace(const DecodePlan &p) {
    return p.S > 1 ? align256(size_t(p.T) * p.S * 64 * ((p.tn + 31) / 32 * 32) * sizeof(float)) : 0;
}

template <int M2, int TN, bool PARTIALS>
hipError_t launch_decode_tn(const W8A8Args &a, const DecodePlan &p, hipStream_t st) {
    constexpr int W = 8;  // two per SIMD, so one wave's latencies hide behind the other's work
    // as many stages as fit in LDS, up to I8GS_DECODE_STAGES
    constexpr int FIT = (160 * 1024 - 16) / DecodeShape<M2, TN, W, PARTIALS>::STAGE;
    constexpr int D = FIT < I8GS_DECODE_STAGES ? FIT : I8GS_DECODE_STAGES;
    w8a8_decode_kernel<M2, TN, W, D, PARTIALS><<<(p.T * p.S + 7) / 8 * 8, W * 64, 0, st>>>(
        a.qa, a.a_scale, a.qweight, a.w_scale, a.y, a.ldy, a.M, a.N, a.K, p.T, p.S,
        PARTIALS ? reinterpret_cast<float *>(a.P) : (float *)a.ws, a.counters);
    return hipGetLastError();
}

template <int M2, bool PARTIALS>
hipError_t launch_decode(const W8A8Args &a, const DecodePlan &p, hipStream_t st) {
    switch (p.tn) {
        case 32: return launch_decode_tn<M2, 32, PARTIALS>(a, p, st);
        case 48: return launch_decode_tn<M2, 48, PARTIALS>(a, p, st);
        case 64: return launch_decode_tn<M2, 64, PARTIALS>(a, p, st);
        case 80: return launch_decode_tn<M2, 80, PARTIALS>(a, p, st);
        case 96: return launch_decode_tn<M2, 96, PARTIALS>(a, p, st);
        case 128: return launch_decode_tn<M2, 128, PARTIALS>(a, p, st);
        case 144: return launch_decode_tn<M2, 144, PARTIALS>(a, p, st);
        case 192: return launch_decode_tn<M2, 192, PARTIALS>(a, p, st);
        default: return launch_decode_tn<M2, 256, PARTIALS>(a, p, st);
    }
}

constexpr int kTB = 128;       // tile rows and columns
constexpr int kPitch = 144;    // LDS row pitch in bytes (128 + 16)

template <bool PARTIALS>
__global__ __launch_bounds__(256) void w8a8_tiled_kernel(const int8_t *__restrict__ qa,
                                                         const float *__restrict__ a_scale,
                                                         const int32_t *__restrict__ qweight,
                                                         const float *__restrict__ w_scale,
                                                         uint16_t *__restrict__ y, int64_t ldy,
                                                         int32_t *__restrict__ P, int M, int N, int K) {
    constexpr int MT = 4, NT = 4;  // each wave: 64 x 64
    __shared__ __attribute__((aligned(16))) int8_t As[kTB * kPitch];
    __shared__ __attribute__((aligned(16))) int8_t Bs[kTB * kPitch];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lb = lane >> 4;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    const int m0 = blockIdx.y * kTB, n0 = blockIdx.x * kTB;
    const int G = K >> 7;

    float acc[MT][NT][4];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;

    for (int g = 0; g < G; ++g) {
        __syncthreads();
        // A tile: 128 rows x 128 bytes, 16 bytes per thread per step.
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int c = tid + it * 256;
            const int row = c >> 3, c16 = c & 7;
            const int gm = m0 + row;
            v4i v = v4i{0, 0, 0, 0};
            if (gm < M) v = *reinterpret_cast<const v4i *>(qa + (int64_t)gm * K + g * 128 + c16 * 16);
            *reinterpret_cast<v4i *>(As + row * kPitch + c16 * 16) = v;
        }
        // B tile: 32 word rows x 128 columns, transposed into [column][k] bytes.
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int c = tid + it * 256;
            const int rl = c >> 5, cq = c & 31;
            const int gn = n0 + cq * 4;
            v4i v = v4i{0, 0, 0, 0};
            if (gn < N) v = flip(*reinterpret_cast<const v4i *>(qweight + (int64_t)(g * 32 + rl) * N + gn));
#pragma unroll
            for (int i = 0; i < 4; ++i) *reinterpret_cast<int *>(Bs + (cq * 4 + i) * kPitch + rl * 4) = v[i];
        }
        __syncthreads();
        v4i pi[MT][NT];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            v4i af[MT], bf[NT];
#pragma unroll
            for (int i = 0; i < MT; ++i)
                af[i] = *reinterpret_cast<const v4i *>(As + (wm + i * 16 + li) * kPitch + ks * 64 + lb * 16);
#pragma unroll
            for (int j = 0; j < NT; ++j)
                bf[j] = *reinterpret_cast<const v4i *>(Bs + (wn + j * 16 + li) * kPitch + ks * 64 + lb * 16);
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j) pi[i][j] = mfma_i8(af[i], bf[j], ks == 0 ? v4i{0, 0, 0, 0} : pi[i][j]);
        }
        if constexpr (PARTIALS) {
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const int col = n0 + wn + j * 16 + li;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = m0 + wm + i * 16 + lb * 4 + r;
                        if (row < M && col < N) P[((int64_t)row * G + g) * N + col] = pi[i][j][r];
                    }
                }
        } else {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int col = min(n0 + wn + j * 16 + li, N - 1);
                const float sc = w_scale[(int64_t)g * N + col];
#pragma unroll
                for (int i = 0; i < MT; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[i][j][r] += sc * (float)pi[i][j][r];
            }
        }
    }
    if constexpr (!PARTIALS) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm + i * 16 + lb * 4 + r;
                if (row >= M) continue;
                const float as = a_scale[row];
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const int col = n0 + wn + j * 16 + li;
                    if (col < N) y[(int64_t)row * ldy + col] = f32_to_bf16_bits(as * acc[i][j][r]);
                }
            }
    }
}

}  // namespace

// Compute units of the current device (cached per device; 256 if unknown).
int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

static bool use_decode(int M, int kernel) {
    if (kernel == I8GS_KERNEL_DECODE) return true;
    if (kernel == I8GS_KERNEL_TILED) return false;
    return M <= 64;
}

// The decode kernel addresses y with 32-bit offsets and drops the rows past M by the y
// descriptor's range check, so the offsets of all the rows a launch covers -- M rounded
// up to the 32-row m tiles -- must stay below 2^31 (no wrap back into range).
bool decode_y_fits(int64_t M, int64_t ldy) { return (M <= 32 ? 32 : 64) * ldy * 2 < (int64_t(1) << 31); }

size_t w8a8_gemm_workspace(int M, int N, int K, int kernel, int workgroups) {
    if (use_decode(M, kernel)) return decode_workspace(decode_plan(M, N, K, workgroups));
    if (kernel != I8GS_KERNEL_TILED) return prefill_gemm_workspace(M, N, K);
    return 0;
}

hipError_t launch_w8a8_gemm(const W8A8Args &a, hipStream_t s) {
    if (a.P != nullptr) {
        // Partials: the kernel and plan the same call would use for y (no y, so no
        // output-size limit, and no split reduction: each K split writes its own groups).
        if (use_decode(a.M, a.kernel)) {
            const DecodePlan p = decode_plan(a.M, a.N, a.K, a.workgroups);
            if (p.m2 == 1) return launch_decode<1, true>(a, p, s);
            return launch_decode<2, true>(a, p, s);
        }
        if (a.kernel != I8GS_KERNEL_TILED) return launch_prefill(a, s);
    } else if (use_decode(a.M, a.kernel) && decode_y_fits(a.M, a.ldy)) {
        const DecodePlan p = decode_plan(a.M, a.N, a.K, a.workgroups);
        if (p.m2 == 1) return launch_decode<1, false>(a, p, s);
        return launch_decode<2, false>(a, p, s);
    }
    if (a.P == nullptr && a.kernel != I8GS_KERNEL_TILED && prefill_y_fits(a.M, a.ldy)) return launch_prefill(a, s);
    dim3 grid((a.N + kTB - 1) / kTB, (a.M + kTB - 1) / kTB);
    if (a.P)
        w8a8_tiled_kernel<true><<<grid, 256, 0, s>>>(a.qa, nullptr, a.qweight, nullptr, nullptr, 0, a.P, a.M, a.N,
                                                    a.K);
    else
        w8a8_tiled_kernel<false><<<grid, 256, 0, s>>>(a.qa, a.a_scale, a.qweight, a.w_scale, a.y, a.ldy, nullptr,
                                                     a.M, a.N, a.K);
    return hipGetLastError();
}

}  // namespace i8gs
