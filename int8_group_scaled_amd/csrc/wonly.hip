// Weight-only group-scaled GEMM on gfx950 bf16 MFMA: W4A16 g128 and W8A16 g128 / g32,
// register-streamed.  Calls of up to 16 rows on layers of at least 65536 columns (the
// vocabulary heads) take this kernel; the others take the LDS-staged kernel in
// w4a16.hip, faster on the decode layer shapes.
//
// Qwen3.8-27B-DFlash2-W4A16-g128-sym-GPTQ model card, property and quantised-layer
// tables (4-bit weights, bf16 activations, group 128, symmetric); Qwen3.5-4B-DFlash-
// W8A16 model card (int8 weights, bf16 activations, RTN); qwen38/dflash2 recipe,
// quantisation settings (int8 drafter projections at group 32; int4 vocabulary head at
// group 128).  y[m,n] = bf16(sum_g w_scale[g,n] * sum_{k in g} x[m,k] * q[k,n]) with
// q = code - 2^(bits-1).
//
// The weights are exact integers in bf16 (4-bit: 16*q, rescaled by 1/16 in the fold;
// 8-bit: q itself), so each MFMA product x*q is exact in fp32; one group is summed by
// v_mfma_f32_16x16x32_bf16 into a fresh fp32 accumulator and then scaled by that
// group's per-column scale and added to the running fp32 sum (scaling after the group
// keeps the error relative to sum |x*q|).
//
// Data flow.  The weights go straight from memory into the registers of the wave that
// uses them (no LDS round trip): a lane loads 16 bytes -- four adjacent columns of one
// packed row -- with buffer_load_dwordx4, and each of the four words feeds a different
// MFMA: the wave computes four 16-column sets at once, column set t holding columns
// 4*j + t (j = lane % 16) of its 64-column strip.  One load instruction then reads
// whole 256-byte pieces of four (4-bit) or of two consecutive (8-bit, two loads) packed
// rows.  A wave keeps one chunk of 256 K values of its weights in flight (8 MFMA
// K-steps), loading step j of the next chunk as soon as step j of this one is
// dequantised.  The activations of a chunk (bf16, shared by all waves of the
// workgroup) and the chunk's scales go through a two-slot LDS ring filled by
// buffer_load ... lds copies, with one barrier per chunk.
//
// MFMA layout (16x16x32 bf16): lane l holds row l % 16 of A and column l % 16 of B,
// 8 consecutive K values starting at 8 * (l / 16) of the 32-wide K step; the 16x16 fp32
// result puts column l % 16, rows 4 * (l / 16) + i in register i.  With GPTQ packing,
// the 8 K values of one column are one 4-bit word (packed row 4*s + l/16 of step s) or
// two 8-bit words (packed rows 8*s + 2*(l/16) and the next).
#include "internal.h"

namespace i8gs {
namespace {

constexpr int kWoChunk = 256;             // K values per activation chunk (one barrier each)
constexpr int kWoSteps = kWoChunk / 32;   // MFMA K-steps per chunk
constexpr int kWoWaves = 4;               // waves per workgroup (one per SIMD)

template <int BITS, int MT, int GS>
struct WoShape {
    static_assert((BITS == 4 || BITS == 8) && MT >= 1 && MT <= 4 && (GS == 32 || GS == 128), "weight-only shape");
    static constexpr int ROWS = 16 * MT;                  // rows of a workgroup's m chunk
    static constexpr int COLS = 64 * kWoWaves;            // columns of a workgroup's tile
    static constexpr int AB = ROWS * kWoChunk * 2;        // activation bytes of a slot
    static constexpr int NG = kWoChunk / GS;              // groups per chunk
    static constexpr int SB = NG * COLS * 4;              // scale bytes of a slot
    static constexpr int SLOT = AB + SB;
    static constexpr int L = BITS == 4 ? 1 : 2;           // weight loads per lane per step
    static constexpr int SPG = GS / 32;                   // steps per group
    static constexpr int ACOPY = AB / 1024;               // 1 KiB activation copies per chunk
    static constexpr int SCOPY = NG * COLS / 256;         // scale copies per chunk (256 columns each)
    static constexpr int APW = (ACOPY + kWoWaves - 1) / kWoWaves;  // activation copies per wave
    static constexpr int SPW = (SCOPY + kWoWaves - 1) / kWoWaves;  // scale copies per wave
    static constexpr int CPW = APW + SPW;                          // memory operations per wave
    static constexpr int NACC = 4 * MT * 4;               // fp32 values per lane (4 column sets)
};

// The 8 codes of one 4-bit word as bf16 of 16*q, in K order.  Byte i of the word holds
// codes 2i (low nibble) and 2i+1 (high nibble); (code ^ 8) is q as a 4-bit two's-
// complement field, so a byte holding it in its high nibble reads as 16*q.
__device__ __forceinline__ v4i wo_dequant4(uint32_t w) {
    const uint32_t odd = (w & 0xF0F0F0F0u) ^ 0x80808080u;
    const uint32_t even = ((w << 4) & 0xF0F0F0F0u) ^ 0x80808080u;
    v4i out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t fe = __float_as_uint((float)(signed char)(even >> (8 * i)));
        const uint32_t fo = __float_as_uint((float)(signed char)(odd >> (8 * i)));
        out[i] = (int)__builtin_amdgcn_perm(fo, fe, 0x07060302u);  // (fe >> 16) | (fo & 0xFFFF0000)
    }
    return out;
}

// The 4 codes of one 8-bit word as bf16 of q (exact: |q| <= 128), two per dword.
__device__ __forceinline__ v2i wo_dequant8(uint32_t w) {
    const uint32_t s = w ^ 0x80808080u;  // offset binary -> two's complement bytes
    v2i out;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t f0 = __float_as_uint((float)(signed char)(s >> (16 * i)));
        const uint32_t f1 = __float_as_uint((float)(signed char)(s >> (16 * i + 8)));
        out[i] = (int)__builtin_amdgcn_perm(f1, f0, 0x07060302u);
    }
    return out;
}

__device__ __forceinline__ v4f wo_mfma(v4i a, v4i b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0,
                                                   0, 0);
}

// The LDS copies of chunk `ch` (absolute chunk index) by this wave: APW activation
// copies (pieces of row r swizzled by XOR with r % 16) then SPW scale copies; every wave
// issues the same sequence, and copies past the chunk's count repeat the last one (the
// same bytes to the same place).
template <class SH>
__device__ __forceinline__ void wo_issue(char *slot, int ch, int wave, __amdgpu_buffer_rsrc_t xr,
                                         __amdgpu_buffer_rsrc_t sr, const int (&a_voff)[SH::APW],
                                         const int (&a_lim)[SH::APW], int s_voff, int N) {
#pragma unroll
    for (int j = 0; j < SH::APW; ++j) {
        // lane -> row 2c + lane/32, physical piece lane % 32; the voffset holds the row and
        // piece for chunk 0 and each chunk moves it by 512 bytes; from chunk a_lim on the
        // lane's K values lie past K and read zeros (offset out of range)
        const int c = min(wave * SH::APW + j, SH::ACOPY - 1);
        const int voff = ch < a_lim[j] ? a_voff[j] + ch * (kWoChunk * 2) : (int)0x80000000u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, I8GS_LDS(slot + c * 1024), 16, voff, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < SH::SPW; ++j) {
        // scale copy sc: group sc / (COLS/256) of the chunk, 256 columns; groups past the
        // end read zeros (past the descriptor's range)
        const int sc = min(wave * SH::SPW + j, SH::SCOPY - 1);
        const uint32_t g = (uint32_t)(ch * SH::NG + sc / (SH::COLS / 256));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            sr, I8GS_LDS(slot + SH::AB + sc * 1024), 16,
            (int)((uint32_t)s_voff + (uint32_t)(sc % (SH::COLS / 256)) * 1024u + g * (uint32_t)N * 4u), 0, 0, 0);
    }
}

// One K-step of this lane's weights: 16 bytes of packed row r (4-bit) or of rows r and
// r + 1 (8-bit), streamed (non-temporal).
template <class SH>
__device__ __forceinline__ void wo_load_w(v4i (&dst)[SH::L], __amdgpu_buffer_rsrc_t wr, uint32_t voff, uint32_t row,
                                          uint32_t soff) {
    dst[0] = __builtin_amdgcn_raw_buffer_load_b128(wr, (int)voff, (int)soff, kCpolNT);
    if constexpr (SH::L == 2) dst[1] = __builtin_amdgcn_raw_buffer_load_b128(wr, (int)(voff + row), (int)soff, kCpolNT);
}

template <int BITS, int MT, int GS>
__global__ __launch_bounds__(kWoWaves * 64) void wo_stream_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, const int32_t *__restrict__ qweight,
    const float *__restrict__ w_scale, uint16_t *__restrict__ y, int64_t ldy, int M, int N, int K, int S, int tiles,
    float *__restrict__ part, size_t part_bytes, int *__restrict__ cnt) {
    using SH = WoShape<BITS, MT, GS>;
    __shared__ __attribute__((aligned(1024))) char lds[2 * SH::SLOT + 16];

    // XCD-aware placement: logical workgroup L (tile-major: L = t*S + s) at launch index
    // (L % Q) * 8 + L / Q, so that the K splits of a tile and neighbouring tiles share an
    // XCD's L2 (only speed depends on this).
    const int P = tiles * S, Q = (P + 7) >> 3;
    const int L = (blockIdx.x & 7) * Q + (blockIdx.x >> 3);
    if (L >= P) return;
    const int t = L / S, s = L - (L / S) * S;
    const int m0 = blockIdx.y * SH::ROWS;
    const int mrows = min(M - m0, SH::ROWS);
    const int n0 = t * SH::COLS;
    const int NCH = (K + kWoChunk - 1) / kWoChunk;
    const int ch0 = (int)((int64_t)s * NCH / S), ch1 = (int)((int64_t)(s + 1) * NCH / S);
    const int nch = ch1 - ch0;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 15, lb = lane >> 4;

    // 32-bit byte offsets: K*N < 2^32 (checked before launch); x is addressed from this
    // chunk's first row, and (rows - 1) * ldx + K stays below 2^30 elements (checked)
    const uint16_t *xc = x + (int64_t)m0 * ldx;
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)qweight, 0, (int)((uint32_t)K * (uint32_t)N / (8u / BITS)), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)xc, 0, (int)(((uint32_t)(mrows - 1) * (uint32_t)ldx + (uint32_t)K) * 2u), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)w_scale, 0, (int)((uint32_t)(K / GS) * (uint32_t)N * 4u), kRsrcWord3);

    // Copy roles (offsets for chunk 0; see wo_issue)
    int a_voff[SH::APW], a_lim[SH::APW];
#pragma unroll
    for (int j = 0; j < SH::APW; ++j) {
        const int c = min(wave * SH::APW + j, SH::ACOPY - 1);
        const int row = 2 * c + (lane >> 5);
        const int piece = (lane & 31) ^ (row & 15);
        a_voff[j] = (int)(((uint32_t)min(row, mrows - 1) * (uint32_t)ldx + (uint32_t)piece * 8u) * 2u);
        a_lim[j] = (K - 8 * piece + kWoChunk - 1) / kWoChunk;  // first chunk whose piece lies past K
    }
    // scales: lane -> columns n0 + 4*lane .. +3 of a 256-column block (the last four when
    // past N: never used)
    const int s_voff = min(n0 + 4 * lane, N - 4) * 4;

    // This lane's weights: 4 adjacent columns cb .. cb+3 (one per column set) of the
    // packed rows of K-block lb; columns past N repeat the last four (never stored).
    const int cb = n0 + 64 * wave + 4 * li;
    const int cbc = min(cb, N - 4);
    const uint32_t w_voff = ((uint32_t)(BITS == 4 ? lb : 2 * lb) * (uint32_t)N + (uint32_t)cbc) * 4u;
    const uint32_t w_step = (uint32_t)(BITS == 4 ? 4 : 8) * (uint32_t)N * 4u;  // bytes per K-step
    const uint32_t w_row = (uint32_t)N * 4u;


    float acc[4][MT][4];
    v4f p[4][MT];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            p[c][mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[c][mt][i] = 0.0f;
        }

    // Prologue: chunk 0's copies, then its weights.
    v4i wbuf[kWoSteps][SH::L];
    wo_issue<SH>(lds, ch0, wave, xr, sr, a_voff, a_lim, s_voff, N);
#pragma unroll
    for (int j = 0; j < kWoSteps; ++j) wo_load_w<SH>(wbuf[j], wr, w_voff, w_row, (uint32_t)(ch0 * kWoSteps + j) * w_step);

    const int a_row0 = li;  // A rows 16*mt + li
    for (int c = 0; c < nch; ++c) {
        // This chunk's copies were issued before its 8 steps of weights, the youngest
        // memory operations of this wave (in-order completion).
        wait_vmcnt<kWoSteps * SH::L>();
        barrier_only();  // every wave's copies are in; every wave is done with the other slot
        __builtin_amdgcn_sched_barrier(0);
        char *const st = lds + (c & 1) * SH::SLOT;
        // The next chunk's copies and weights, issued unconditionally (no branch in the
        // loop, so the compiler's waits stay exact): the last chunk loads itself again,
        // from L2, into the slot and registers nothing reads any more.
        const int cn = ch0 + min(c + 1, nch - 1);
        wo_issue<SH>(lds + ((c + 1) & 1) * SH::SLOT, cn, wave, xr, sr, a_voff, a_lim, s_voff, N);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < kWoSteps; ++j) {
            // B operands of the four column sets
            v4i b[4];
            if constexpr (BITS == 4) {
#pragma unroll
                for (int cs = 0; cs < 4; ++cs) b[cs] = wo_dequant4((uint32_t)wbuf[j][0][cs]);
            } else {
#pragma unroll
                for (int cs = 0; cs < 4; ++cs) {
                    const v2i lo = wo_dequant8((uint32_t)wbuf[j][0][cs]);
                    const v2i hi = wo_dequant8((uint32_t)wbuf[j][1][cs]);
                    b[cs] = v4i{lo[0], lo[1], hi[0], hi[1]};
                }
            }
            wo_load_w<SH>(wbuf[j], wr, w_voff, w_row, (uint32_t)(cn * kWoSteps + j) * w_step);
            const bool first = j % SH::SPG == 0;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int row = 16 * mt + a_row0;
                const int piece = (4 * j + lb) ^ (row & 15);
                const v4i a = *reinterpret_cast<const v4i *>(st + row * (kWoChunk * 2) + piece * 16);
#pragma unroll
                for (int cs = 0; cs < 4; ++cs)
                    p[cs][mt] = wo_mfma(a, b[cs], first ? v4f{0.f, 0.f, 0.f, 0.f} : p[cs][mt]);
            }
            if (j % SH::SPG == SH::SPG - 1) {
                // fold this group: its scales for the lane's four columns (4-bit sums are 16x)
                const int gi = j / SH::SPG;
                v4f sc = *reinterpret_cast<const v4f *>(st + SH::AB + (gi * SH::COLS + 64 * wave + 4 * li) * 4);
                if constexpr (BITS == 4) sc *= 0.0625f;
#pragma unroll
                for (int cs = 0; cs < 4; ++cs)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[cs][mt][i] += sc[cs] * p[cs][mt][i];
            }
            // one step at a time: interleaving the unrolled steps would keep several
            // steps' operands and group sums live at once
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    if (S > 1) {
        // Partial of split q, wave w: NACC fp32 cells of 64 lanes at
        // ((tile_id * S + q) * 4 + w) * NACC * 64 (device-coherent stores and loads: the
        // splits may run on different XCDs); the last split to arrive sums them in split order.
        const int tile_id = blockIdx.y * tiles + t;
        const __amdgpu_buffer_rsrc_t pr =
            __builtin_amdgcn_make_buffer_rsrc((void *)part, 0, (int)part_bytes, kRsrcWord3);
        const uint32_t qstride = (uint32_t)kWoWaves * SH::NACC * 64 * 4;
        const uint32_t cell0 =
            (uint32_t)tile_id * (uint32_t)S * qstride + ((uint32_t)wave * SH::NACC * 64 + lane) * 4u;
        // (only the rows below M: the others are never stored)
#pragma unroll
        for (int cs = 0; cs < 4; ++cs)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * mt + 4 * lb + i < mrows)
                        __builtin_amdgcn_raw_buffer_store_b32(
                            __float_as_int(acc[cs][mt][i]), pr,
                            (int)(cell0 + (uint32_t)((cs * MT + mt) * 4 + i) * 256u), (int)((uint32_t)s * qstride),
                            kCpolSC1);
        wait_vmcnt<0>();
        __syncthreads();
        int *const s_last = reinterpret_cast<int *>(lds + 2 * SH::SLOT);
        if (threadIdx.x == 0) {
            const int last =
                __hip_atomic_fetch_add(cnt + tile_id, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
            if (last) __hip_atomic_store(cnt + tile_id, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *s_last = last;
        }
        __syncthreads();
        if (!*s_last) return;
        // QB pieces in flight at a time; cells of rows past M are not loaded (never stored)
        constexpr int QB = MT > 2 ? 2 : (MT == 2 ? 4 : 8);
        float sum[SH::NACC];
        for (int q0 = 0; q0 < S; q0 += QB) {
            float v[QB][SH::NACC];
#pragma unroll
            for (int k = 0; k < QB; ++k) {
                const int q = min(q0 + k, S - 1);
#pragma unroll
                for (int i = 0; i < SH::NACC; ++i) {
                    const bool live = 16 * ((i / 4) % MT) + 4 * lb + i % 4 < mrows;
                    v[k][i] = q == s || !live ? acc[i / (4 * MT)][(i / 4) % MT][i % 4]
                                              : __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                                    pr, (int)(cell0 + (uint32_t)i * 256u),
                                                    (int)((uint32_t)q * qstride), kCpolSC1));
                }
            }
#pragma unroll
            for (int k = 0; k < QB; ++k) {
                if (q0 + k >= S) break;
#pragma unroll
                for (int i = 0; i < SH::NACC; ++i) sum[i] = q0 + k == 0 ? v[k][i] : sum[i] + v[k][i];
            }
        }
#pragma unroll
        for (int i = 0; i < SH::NACC; ++i) acc[i / (4 * MT)][(i / 4) % MT][i % 4] = sum[i];
    }

    // y: for each of the lane's rows 16*mt + 4*lb + i, its four columns cb .. cb+3 as one
    // 8-byte store.
    if (cb < N) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * mt + 4 * lb + i;
                if (row < mrows) {
                    const uint32_t lo = (uint32_t)f32_to_bf16_bits(acc[0][mt][i]) |
                                        ((uint32_t)f32_to_bf16_bits(acc[1][mt][i]) << 16);
                    const uint32_t hi = (uint32_t)f32_to_bf16_bits(acc[2][mt][i]) |
                                        ((uint32_t)f32_to_bf16_bits(acc[3][mt][i]) << 16);
                    *reinterpret_cast<v2i *>(y + (int64_t)(m0 + row) * ldy + cb) = v2i{(int)lo, (int)hi};
                }
            }
    }
}

struct WoPlan {
    int MT, S, tiles, blocks, chunks;
};

WoPlan wo_plan(int M, int N, int K) {
    WoPlan p;
    p.MT = M >= 64 ? 4 : (M + 15) / 16;
    p.chunks = (M + 16 * p.MT - 1) / (16 * p.MT);
    p.tiles = (N + 64 * kWoWaves - 1) / (64 * kWoWaves);
    const int NCH = (K + kWoChunk - 1) / kWoChunk;
    // Target two workgroups per CU (their LDS rings fit); four for small m chunks was
    // slower (longer weight streams per workgroup win: gate_up at M = 8 55.9 -> 48.6 us,
    // the 8-bit vocabulary head at M = 1 228.7 -> 201.6 us).  K splits of at least two
    // chunks each and at most 16 (the last split to arrive sums all the pieces).
    const int cus = device_cu_count();
    const int target = 2 * cus;
    int S = (target + p.tiles * p.chunks - 1) / (p.tiles * p.chunks);
    S = std::max(1, std::min(S, std::min(16, NCH / 2)));
    if (p.tiles * p.chunks > kMaxCounters) S = 1;
    p.S = S;
    p.blocks = ((p.tiles * p.S + 7) / 8) * 8;
    return p;
}

template <int BITS, int MT, int GS>
hipError_t launch_wo_mt(const WoArgs &a, const WoPlan &p, hipStream_t st) {
    int *cnt = p.S > 1 ? a.counters : nullptr;
    float *part = p.S > 1 ? (float *)a.ws : nullptr;
    dim3 grid(p.blocks, p.chunks);
    wo_stream_kernel<BITS, MT, GS><<<grid, kWoWaves * 64, 0, st>>>(a.x, a.ldx, a.qweight, a.w_scale, a.y, a.ldy, a.M,
                                                                   a.N, a.K, p.S, p.tiles, part,
                                                                   p.S > 1 ? a.ws_bytes : 0, cnt);
    return hipGetLastError();
}

template <int BITS, int GS>
hipError_t launch_wo_bits(const WoArgs &a, const WoPlan &p, hipStream_t st) {
    switch (p.MT) {
        case 1: return launch_wo_mt<BITS, 1, GS>(a, p, st);
        case 2: return launch_wo_mt<BITS, 2, GS>(a, p, st);
        case 3: return launch_wo_mt<BITS, 3, GS>(a, p, st);
        default: return launch_wo_mt<BITS, 4, GS>(a, p, st);
    }
}

}  // namespace

// Partial-sum bytes after the counter region (0 when K is not split).
size_t wo_gemm_workspace(int M, int N, int K) {
    const WoPlan p = wo_plan(M, N, K);
    if (p.S <= 1) return 0;
    return align256(size_t(p.tiles) * p.chunks * p.S * kWoWaves * (16 * p.MT) * 64 * sizeof(float));
}

hipError_t launch_wo_gemm(const WoArgs &a, hipStream_t s) {
    const WoPlan p = wo_plan(a.M, a.N, a.K);
    if (a.bits == 4) return launch_wo_bits<4, 128>(a, p, s);
    if (a.group == 32) return launch_wo_bits<8, 32>(a, p, s);
    return launch_wo_bits<8, 128>(a, p, s);
}

}  // namespace i8gs
