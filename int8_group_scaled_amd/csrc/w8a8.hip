// W8A8 G128 GEMM on gfx950 MFMA.
//
// Qwen3.8-27B GPTQ INT8 W8A8 GS128 PTQR model card, "Quantization details": true
// int8 x int8 compute at every decode and prefill shape with one weight scale per
// 128-wide K block.  Flint INT8 card, format table: GPTQ qweight/scales, symmetric,
// group 128, no g_idx.  For each 128-wide group the int8 products are summed exactly
// in an int32 MFMA accumulator (v_mfma_i32_16x16x64_i8, two per group), converted to
// fp32 and folded with that group's per-column scale; the row scale and the bf16
// rounding are applied once at the end.
//
// MFMA operand layout used here (16x16x64 i8): lane l holds row (l % 16) of A and
// column (l % 16) of B, 16 consecutive K bytes starting at 16 * (l / 16) within a
// 64-wide K step.  A and B use the same K placement, so the product is the plain
// dot product whatever order the hardware walks K in.  The 16x16 int32 result puts
// column (l % 16), rows 4 * (l / 16) + r (r = 0..3) in lane l.
//
// GPTQ codes are offset binary (q + 128); XOR 0x80 per byte turns a code into the
// two's-complement int8 value of q.
//
// Two kernels:
//  * decode (M <= 64): bound by streaming the weights from HBM.  A workgroup owns a
//    tile of 64 columns and a range of K groups; its W waves split that range, and
//    every wave loads its weights straight from HBM into registers as 16-byte row
//    pieces (one wave instruction = 256 contiguous bytes of 4 rows) and its
//    activation fragments from L2, with the next group's loads in flight while the
//    current group runs on the MFMA units.  Waves reduce through LDS in a fixed
//    order.  When the tiles alone cannot fill the GPU, K is also split across S
//    workgroups: each writes an fp32 partial tile to the workspace, and the last of
//    the S to arrive (a per-tile atomic counter) sums the partials in split order
//    and writes y, so results do not depend on timing.
//  * tiled (M > 64): LDS-staged 128x128 tiles, four waves of 64x64.
#include "internal.h"

namespace i8gs {
namespace {

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Workgroup barrier that orders only LDS: waits for this wave's LDS accesses, not for
// its global loads (the fence of __syncthreads would drain the prefetches too).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ v4i flip(v4i v) {
    return v ^ (int)0x80808080;
}

// ------------------------------------------------------------------ decode kernel
//
// Weight operand.  A 64-column slab is read as 16-byte row pieces: lane (li, lb) =
// (lane % 16, lane / 16) owns the four adjacent columns c = n0 + 4*li .. +3 and, for
// the 64-wide K step s of group g, loads rows 32g + 16s + 4*lb + i (i = 0..3) of
// those columns; one wave instruction reads 256 contiguous bytes of 4 rows.  For
// column c + cc the four words are 16 consecutive K bytes (k = 128g + 64s + 16*lb ..
// +15): exactly the B operand of lane (li, lb) of an MFMA whose 16 columns are
// n0 + 4*j + cc.  So a slab is 4 MFMA fragments with column stride 4 and no data
// moves between lanes; fragment cc's result in lane (li, lb) is column
// n0 + 4*li + cc, rows 4*lb + r.
//
// Activation operand.  The 64 x 128-byte group of quantised activations is the same
// for every column, so each workgroup covers CQ slabs (a 64*CQ-column tile) and
// stages the group once in LDS with whole-row reads; every wave then reads its A
// fragments (row l % 16, bytes 16*(l / 16) .. of the K step) from LDS.  Reading it
// straight from L2 for every 64 columns doubled the L1 traffic and halved the rate.
//
// Work split (stream-K).  Work units are (tile, group) pairs in tile-major order and
// the P workgroups take equal contiguous ranges, so every CU streams the same number
// of weight bytes whatever the layer shape.  Inside a workgroup the W = CQ*KS waves
// are CQ column slabs x KS K-parts: the KS parts of a tile segment run side by side
// (all waves take the same number of steps; a part that is one group shorter takes
// a step with zero scales), then reduce through LDS in K order.  A tile that lies in
// one workgroup's range is written directly; a tile split over several workgroups is
// summed by the last of them to arrive (a per-tile counter), in workgroup order, so
// the result does not depend on timing.

constexpr int kAPitch = 144;           // LDS row pitch of a staged activation group (128 + 16)
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, gfx9-family format word
constexpr int kCpolNT = 2;             // non-temporal: streamed weights are not reused

struct DecodePlan {
    int cq;      // 64-column slabs per tile
    int tiles;   // column tiles
    int blocks;  // workgroups sharing the (tile, group) work items
};

struct DecodeRegs {
    v4i b[2][4];  // [k step][row i]: 4 columns each (offset-binary codes)
    v4f sc;       // scales of the 4 columns
    bool live;    // false on a padding step: its scales are taken as zero when used
};

// Loads of one step: the activation pieces this thread stages, then the weight rows
// and scales of this wave's slab (activations first, so the wait before staging them
// leaves the weight loads in flight).
template <int APT>
__device__ __forceinline__ void decode_load(DecodeRegs &d, v4i (&areg)[APT], __amdgpu_buffer_rsrc_t wr,
                                            __amdgpu_buffer_rsrc_t ar, __amdgpu_buffer_rsrc_t sr,
                                            const int (&a_src)[APT], int g, bool pad, uint32_t row_bytes, int w_lane,
                                            int s_lane) {
#pragma unroll
    for (int j = 0; j < APT; ++j) areg[j] = __builtin_amdgcn_raw_buffer_load_b128(ar, a_src[j], g * 128, 0);
    // Same issue order everywhere (also in the prologue), so the compiler's wait
    // counts at the loop head stay exact.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            d.b[s][i] = __builtin_amdgcn_raw_buffer_load_b128(wr, w_lane, (int)((uint32_t)(g * 32 + s * 16 + i) * row_bytes),
                                                              kCpolNT);
    __builtin_amdgcn_sched_barrier(0);
    d.sc = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(sr, s_lane, (int)((uint32_t)g * row_bytes), 0));
    // Not applied to the loaded scales here: a select on them right after the load
    // would make the compiler wait for every load in flight.
    d.live = !pad;
}

template <int APT, int STRIDE>
__device__ __forceinline__ void decode_stage(char *lds_buf, const v4i (&areg)[APT], const int (&a_dst)[APT], int tks,
                                             int pieces) {
#pragma unroll
    for (int j = 0; j < APT; ++j)
        if (tks + j * STRIDE < pieces) *reinterpret_cast<v4i *>(lds_buf + a_dst[j]) = areg[j];
}

// One step on the MFMA units: the activation fragments of both K steps are read
// from LDS once, then per column quad cc both K steps for every m tile (int32,
// exact), then the fold acc += scale * float(group sum).
template <int MT>
__device__ __forceinline__ void decode_compute(const DecodeRegs &d, const char *abase, float (&acc)[4][MT][4]) {
    v4i af[2][MT];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) af[s][mt] = *reinterpret_cast<const v4i *>(abase + mt * 16 * kAPitch + s * 64);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
        v4i p[MT];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const v4i bf = v4i{d.b[s][0][cc], d.b[s][1][cc], d.b[s][2][cc], d.b[s][3][cc]} ^ (int)0x80808080;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) p[mt] = mfma_i8(af[s][mt], bf, s == 0 ? v4i{0, 0, 0, 0} : p[mt]);
        }
        const float sc = d.live ? d.sc[cc] : 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[cc][mt][r] += sc * (float)p[mt][r];
    }
}

// Device-coherent stores and loads (scope "agent": the sc1 cache-policy bit) for the
// partial tiles exchanged between workgroups.  They are coherent across the XCDs'
// separate L2 caches, so no cache-wide writeback or invalidate is needed; the writer
// waits for its stores to complete before it bumps the tile's counter.
__device__ __forceinline__ void store_coherent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup that owns unit u when U units are split evenly over P workgroups
// (workgroup b owns [floor(b*U/P), floor((b+1)*U/P))).
__device__ __forceinline__ int owner_of(int64_t u, int64_t U, int P) { return (int)(((u + 1) * P - 1) / U); }

template <int MT, int CQ, int KS>
__global__ __launch_bounds__(CQ * KS * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void w8a8_decode_kernel(
    const int8_t *__restrict__ qa, const float *__restrict__ a_scale, const int32_t *__restrict__ qweight,
    const float *__restrict__ w_scale, uint16_t *__restrict__ y, int64_t ldy, int M, int N, int K, int tiles,
    int P, float *__restrict__ part, int *__restrict__ cnt) {
    constexpr int TN = 64 * CQ;
    constexpr int NACC = 16 * MT;                                 // fp32 accumulators per lane
    constexpr int ROWS = 16 * MT;
    constexpr int APIECES = ROWS * 8;                             // 16-byte pieces of one staged group
    constexpr int APT = (APIECES + CQ * 64 - 1) / (CQ * 64);      // pieces per thread of a K part
    constexpr int ABUF = ROWS * kAPitch;                          // bytes of one staged group
    constexpr int A_LDS = 2 * KS * ABUF;
    constexpr int R_LDS = (KS - 1) * CQ * NACC * 64 * 4;
    constexpr int LDS_BYTES = A_LDS > R_LDS ? A_LDS : R_LDS;
    static_assert((16 * MT / KS) % 4 == 0, "each wave must finish whole (row, 4-column) pieces");
    __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
    __shared__ int s_flag;

    const int b = blockIdx.x;
    const int G = K >> 7;
    const int64_t U = (int64_t)tiles * G;
    const int64_t u0 = (int64_t)b * U / P, u1 = (int64_t)(b + 1) * U / P;
    if (u0 >= u1) return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keeps group offsets in SGPRs
    const int cq = wave % CQ, ks = wave / CQ;
    const int li = lane & 15, lb = lane >> 4;
    const int tks = cq * 64 + lane;  // thread index among the CQ waves of this K part
    const int t_first = (int)(u0 / G), t_last = (int)((u1 - 1) / G);

    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc((void *)qweight, 0, (int)((uint32_t)K * (uint32_t)N), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t ar =
        __builtin_amdgcn_make_buffer_rsrc((void *)qa, 0, (int)((uint32_t)M * (uint32_t)K), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t sr =
        __builtin_amdgcn_make_buffer_rsrc((void *)w_scale, 0, (int)((uint32_t)(K >> 7) * (uint32_t)N * 4u), kRsrcWord3);

    // Activation staging: piece pc = tks + j*CQ*64 is row pc / 8, bytes (pc % 8) * 16.
    int a_src[APT], a_dst[APT];
#pragma unroll
    for (int j = 0; j < APT; ++j) {
        const int pc = min(tks + j * CQ * 64, APIECES - 1);
        a_src[j] = (int)((uint32_t)min(pc >> 3, M - 1) * (uint32_t)K + (uint32_t)(pc & 7) * 16u);
        a_dst[j] = ks * ABUF + (pc >> 3) * kAPitch + (pc & 7) * 16;
    }
    const int a_frag = li * kAPitch + lb * 16;  // + ks*ABUF + mt*16*kAPitch + s*64

    for (int t = t_first; t <= t_last; ++t) {
        const int64_t tb = (int64_t)t * G;
        const int ga = (int)(max(u0, tb) - tb), gb = (int)(min(u1, tb + G) - tb);
        const int ng = gb - ga;
        const int ka = ga + (ks * ng) / KS, nk = ga + ((ks + 1) * ng) / KS - ka;
        const int steps = (ng + KS - 1) / KS;  // same for every wave
        const int n0 = t * TN + cq * 64;
        const int col0 = min(n0 + 4 * li, N - 4);  // N % 8 == 0, so a clamped quad stays inside the row
        // byte offsets fit 32 bits: K*N < 2^32 is checked before launch
        const int w_lane = (int)(((uint32_t)(4 * lb) * (uint32_t)N + (uint32_t)col0) * 4u), s_lane = col0 * 4;

        float acc[4][MT][4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[cc][mt][r] = 0.0f;

        // Ping-pong over steps: while step i computes, the loads of step i+1 are in
        // flight.  The body is straight-line -- a step past this part's end re-reads a
        // valid group and has zero scales, also for the second half of the last pair
        // -- so the compiler's wait counts stay exact; sched_barrier keeps each
        // prefetch from sinking below the current step's waits.
        {
            const uint32_t row_bytes = (uint32_t)N * 4u;
            char *abuf0 = lds + ks * ABUF;
            char *abuf1 = lds + KS * ABUF + ks * ABUF;
            DecodeRegs r0, r1;
            v4i areg[APT];
            decode_load<APT>(r0, areg, wr, ar, sr, a_src, nk > 0 ? ka : ga, nk <= 0, row_bytes, w_lane, s_lane);
            for (int i = 0; i < steps; i += 2) {
                decode_stage<APT, CQ * 64>(lds, areg, a_dst, tks, APIECES);
                decode_load<APT>(r1, areg, wr, ar, sr, a_src, nk > 0 ? ka + min(i + 1, nk - 1) : ga, i + 1 >= nk,
                                 row_bytes, w_lane, s_lane);
                __builtin_amdgcn_sched_barrier(0);
                lds_barrier();
                decode_compute<MT>(r0, abuf0 + a_frag, acc);
                __builtin_amdgcn_sched_barrier(0);
                decode_stage<APT, CQ * 64>(lds + KS * ABUF, areg, a_dst, tks, APIECES);
                decode_load<APT>(r0, areg, wr, ar, sr, a_src, nk > 0 ? ka + min(i + 2, nk - 1) : ga, i + 2 >= nk,
                                 row_bytes, w_lane, s_lane);
                __builtin_amdgcn_sched_barrier(0);
                lds_barrier();
                decode_compute<MT>(r1, abuf1 + a_frag, acc);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // Reduce the K parts into the ks == 0 waves, in K order.
        if constexpr (KS > 1) {
            __syncthreads();  // the LDS staging area is reused below
            float *red = reinterpret_cast<float *>(lds);
            if (ks > 0) {
                float *dst = red + ((ks - 1) * CQ + cq) * NACC * 64;
                int i = 0;
#pragma unroll
                for (int cc = 0; cc < 4; ++cc)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int r = 0; r < 4; ++r, ++i) dst[i * 64 + lane] = acc[cc][mt][r];
            }
            __syncthreads();
            if (ks == 0) {
#pragma unroll
                for (int k2 = 1; k2 < KS; ++k2) {
                    const float *src = red + ((k2 - 1) * CQ + cq) * NACC * 64;
                    int i = 0;
#pragma unroll
                    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                            for (int r = 0; r < 4; ++r, ++i) acc[cc][mt][r] += src[i * 64 + lane];
                }
            }
            __syncthreads();  // before the next segment stages activations again
        }

        if (ng < G) {
            // Split tile: publish this workgroup's partial (layout [cq][m tile][row][quad]),
            // count arrivals, and let the last arrival sum the partials in workgroup order.
            // The sum is spread over all W waves, each re-reading its share of every
            // partial (its own included) with the loads of up to four workgroups in flight.
            const int slot = (t == t_first) ? 0 : 1;
            if (ks == 0) {
                float *mine = part + (((int64_t)b * 2 + slot) * CQ + cq) * NACC * 64;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int cc = 0; cc < 4; ++cc)
                            store_coherent(mine + ((mt * 4 + r) * 4 + cc) * 64 + lane, acc[cc][mt][r]);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            __syncthreads();
            const int bf = owner_of(tb, U, P), bl = owner_of(tb + G - 1, U, P);
            if (threadIdx.x == 0) s_flag = atomicAdd(cnt + t, 1);
            __syncthreads();
            if (s_flag != bl - bf) continue;
            asm volatile("" ::: "memory");
            constexpr int VPW = CQ * NACC / (CQ * KS);  // values per lane per wave (a multiple of 4)
            constexpr int QB = VPW >= 64 ? 1 : (VPW >= 32 ? 2 : 4);  // partials loaded at once (register budget)
            const int v0 = wave * VPW;                  // first value of this wave in [cq][m tile][row][quad] order
            float sum[VPW];
            for (int q0 = bf; q0 <= bl; q0 += QB) {
                float v[QB][VPW];
#pragma unroll
                for (int j = 0; j < QB; ++j) {
                    const int q = min(q0 + j, bl);
                    const int64_t qb = (int64_t)q * U / P;
                    const int qslot = (t == (int)(qb / G)) ? 0 : 1;
                    const float *src = part + ((int64_t)q * 2 + qslot) * CQ * NACC * 64 + (int64_t)v0 * 64;
#pragma unroll
                    for (int k = 0; k < VPW; ++k) v[j][k] = load_coherent(src + k * 64 + lane);
                }
#pragma unroll
                for (int j = 0; j < QB; ++j)
                    if (q0 + j <= bl) {
#pragma unroll
                        for (int k = 0; k < VPW; ++k) sum[k] = (q0 + j == bf) ? v[j][k] : sum[k] + v[j][k];
                    }
            }
            // Write this wave's share: VPW/4 (m tile, row) pairs x 4 adjacent columns.
            const int wcq = v0 / NACC;
            const int colw = t * TN + wcq * 64 + 4 * li;
            if (colw < N) {
#pragma unroll
                for (int k = 0; k < VPW; k += 4) {
                    const int pr = ((v0 % NACC) + k) >> 2;  // m tile * 4 + row index r
                    const int row = (pr >> 2) * 16 + lb * 4 + (pr & 3);
                    if (row < M) {
                        const float as = a_scale[row];
                        const uint32_t lo = f32_to_bf16_bits(as * sum[k]) | ((uint32_t)f32_to_bf16_bits(as * sum[k + 1]) << 16);
                        const uint32_t hi =
                            f32_to_bf16_bits(as * sum[k + 2]) | ((uint32_t)f32_to_bf16_bits(as * sum[k + 3]) << 16);
                        *reinterpret_cast<v2i *>(y + (int64_t)row * ldy + colw) = v2i{(int)lo, (int)hi};
                    }
                }
            }
            if (threadIdx.x == 0) cnt[t] = 0;  // leave the counter at zero for the next call
            continue;
        }

        // Epilogue (ks == 0 waves): y = bf16(a_scale[row] * sum), 4 adjacent columns per 8-byte store.
        const int col = n0 + 4 * li;
        if (ks == 0 && col < N) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = mt * 16 + lb * 4 + r;
                    if (row < M) {
                        const float as = a_scale[row];
                        const uint32_t lo = f32_to_bf16_bits(as * acc[0][mt][r]) |
                                            ((uint32_t)f32_to_bf16_bits(as * acc[1][mt][r]) << 16);
                        const uint32_t hi = f32_to_bf16_bits(as * acc[2][mt][r]) |
                                            ((uint32_t)f32_to_bf16_bits(as * acc[3][mt][r]) << 16);
                        *reinterpret_cast<v2i *>(y + (int64_t)row * ldy + col) = v2i{(int)lo, (int)hi};
                    }
                }
        }
    }
}

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

#ifndef I8GS_DECODE_CQ
#define I8GS_DECODE_CQ 0  // 0 = choose per shape
#endif
#ifndef I8GS_DECODE_KS
#define I8GS_DECODE_KS 1
#endif
#ifndef I8GS_DECODE_WG_PER_CU
#define I8GS_DECODE_WG_PER_CU 2
#endif

DecodePlan decode_plan(int M, int N, int K, int workgroups) {
    (void)M;
    DecodePlan p;
    // Wider tiles share each staged activation group across more columns (less L2
    // traffic); narrower tiles make smaller partial tiles where tiles are split.
    int cq = I8GS_DECODE_CQ;
    if (cq == 0) cq = 4;
    if (cq != 2) cq = 4;
    p.cq = cq;
    p.tiles = (N + 64 * cq - 1) / (64 * cq);
    const int64_t U = (int64_t)p.tiles * (K / kGroup);
    int64_t P = workgroups > 0 ? workgroups : (int64_t)device_cu_count() * I8GS_DECODE_WG_PER_CU;
    if (P > U) P = U;
    if (P < 1) P = 1;
    // Split tiles need a counter each; with one workgroup per tile no tile is split.
    if (p.tiles > kMaxCounters) P = p.tiles;
    p.blocks = (int)P;
    return p;
}

// Partial-sum bytes after the counter region: two partial tiles per workgroup.
size_t decode_workspace(const DecodePlan &p, int M) {
    const int MT = (M + 15) / 16;
    return align256(size_t(p.blocks) * 2 * p.cq * 16 * MT * 64 * sizeof(float));
}

template <int MT, int CQ>
hipError_t launch_decode_cq(const W8A8Args &a, const DecodePlan &p, hipStream_t st) {
    constexpr int KS = I8GS_DECODE_KS;
    w8a8_decode_kernel<MT, CQ, KS><<<p.blocks, CQ * KS * 64, 0, st>>>(a.qa, a.a_scale, a.qweight, a.w_scale, a.y, a.ldy, a.M,
                                                            a.N, a.K, p.tiles, p.blocks, (float *)a.ws, a.counters);
    return hipGetLastError();
}

template <int MT>
hipError_t launch_decode_mt(const W8A8Args &a, const DecodePlan &p, hipStream_t st) {
    switch (p.cq) {
        case 2: return launch_decode_cq<MT, 2>(a, p, st);
        default: return launch_decode_cq<MT, 4>(a, p, st);
    }
}

// ------------------------------------------------------------------ tiled kernel (M > 64)

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

static bool use_decode(int M, int kernel) {
    if (kernel == I8GS_KERNEL_DECODE) return true;
    if (kernel == I8GS_KERNEL_TILED) return false;
    return M <= 64;
}

size_t w8a8_gemm_workspace(int M, int N, int K, int kernel, int workgroups) {
    if (use_decode(M, kernel)) return decode_workspace(decode_plan(M, N, K, workgroups), M);
    return 0;
}

hipError_t launch_w8a8_gemm(const W8A8Args &a, hipStream_t s) {
    if (a.P == nullptr && use_decode(a.M, a.kernel)) {
        const DecodePlan p = decode_plan(a.M, a.N, a.K, a.workgroups);
        switch ((a.M + 15) / 16) {
            case 1: return launch_decode_mt<1>(a, p, s);
            case 2: return launch_decode_mt<2>(a, p, s);
            case 3: return launch_decode_mt<3>(a, p, s);
            default: return launch_decode_mt<4>(a, p, s);
        }
    }
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
