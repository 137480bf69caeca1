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
//  * decode (M <= 64): bound by streaming the weights from HBM.  One workgroup per
//    CU streams an equal share of (tile, group) units through an LDS ring filled by
//    direct buffer-to-LDS copies; tiles split between workgroups are summed in a
//    fixed order by a small reduction kernel.
//  * tiled (M > 64): LDS-staged 128x128 tiles, four waves of 64x64.
#include "internal.h"

namespace i8gs {
namespace {

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Workgroup barrier without the fence of __syncthreads (which would also wait for
// every copy in flight); the compiler keeps memory accesses on their side of it.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ v4i flip(v4i v) {
    return v ^ (int)0x80808080;
}

// ------------------------------------------------------------------ decode kernel
//
// Streaming.  Every workgroup (4 waves, one per CU: the LDS ring below takes most of
// the CU's 160 KiB) pulls its share of the weights through a D-stage ring in LDS with
// buffer_load ... lds: a stage is one 128-wide K group of a TN-column tile -- its
// 32 packed weight rows (TN*128 bytes), the group's 16*MT activation rows (128 bytes
// each) and its TN column scales.  The copies go straight from memory into LDS, so
// D-1 stages stay in flight without holding registers; each wave waits for its own
// copies of the current stage (vmcnt), a barrier makes all of them visible, and the
// stage's slot is refilled only after every wave is done with it.
//
// Work split (stream-K).  Work units are (tile, group) pairs in tile-major order and
// the P workgroups take equal contiguous ranges, so every CU streams the same number
// of weight bytes whatever the layer shape.  A tile that lies inside one workgroup's
// range is finished there; the pieces of a tile split between workgroups are written
// as fp32 partial tiles and summed in workgroup order by a small reduction kernel
// launched right after, so the result does not depend on timing.  Summing them in
// the same kernel (the last workgroup of a tile to finish reads the others' pieces)
// measured slower: all of that work falls on a few workgroups at the very end.
//
// Operand reads from LDS.  Wave w covers the 64-column slab w % CQ of the tile and the
// m tiles of part w / CQ of the rows.  Weights: lane (li, lb) = (lane % 16, lane / 16)
// reads the 16-byte row pieces of rows 16s + 4*lb + i (i = 0..3), columns
// slab*64 + 4*li .. +3; for column c + cc the four words are 16 consecutive K bytes,
// i.e. the B operand of an MFMA whose 16 columns are slab*64 + 4*j + cc.  Activations
// are stored with the 16-byte pieces of row r permuted by XOR with (r / 2) % 8, so the
// 16 rows of an A fragment fall in 16 different bank groups.

#define I8GS_LDS(p) ((__attribute__((address_space(3))) void *)(p))

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, gfx9-family format word
constexpr int kCpolNT = 2;             // non-temporal: streamed weights are not reused

template <int MT, int TN>
struct DecodeShape {
    static constexpr int CQ = TN / 64;              // 64-column slabs per tile
    static constexpr int MS = 4 / CQ;               // row parts (4 waves = CQ x MS)
    static constexpr int MTW = MT / MS;             // 16-row m tiles per wave
    static constexpr int WB = TN * 128;             // weight bytes of a stage
    static constexpr int AB = MT * 16 * 128;        // activation bytes of a stage
    static constexpr int SB = 1024;                 // scale slot (TN floats + copies)
    static constexpr int STAGE = WB + AB + SB;
    static constexpr int WI = WB / 4096;            // 1 KiB copies per wave: weights
    static constexpr int AI = AB / 4096;            //   activations
    static constexpr int LPS = WI + AI + 1;         // memory instructions per wave per stage
    static constexpr int LPR = TN / 4;              // lanes per packed weight row
    static constexpr int RPI = 256 / TN;            // packed rows per 1 KiB copy
    static_assert(CQ * MS == 4 && MT % MS == 0 && AB % 4096 == 0, "unsupported decode shape");
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Copies of one stage by this wave: its WI pieces of the weight rows, AI pieces of the
// activation rows and one dword per lane of the scales.
template <int MT, int TN>
__device__ __forceinline__ void decode_issue(char *st, __amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t ar,
                                             __amdgpu_buffer_rsrc_t sr, int wave, int w_voff,
                                             const int (&a_voff)[DecodeShape<MT, TN>::AI], int s_voff, int t, int g,
                                             int N) {
    using S = DecodeShape<MT, TN>;
#pragma unroll
    for (int j = 0; j < S::WI; ++j) {
        const int ins = wave * S::WI + j;
        const uint32_t so = ((uint32_t)(g * 32 + ins * S::RPI) * (uint32_t)N + (uint32_t)(t * TN)) * 4u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, I8GS_LDS(st + ins * 1024), 16, w_voff, (int)so, 0, kCpolNT);
    }
#pragma unroll
    for (int j = 0; j < S::AI; ++j) {
        const int ins = wave * S::AI + j;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, I8GS_LDS(st + S::WB + ins * 1024), 16, a_voff[j], g * 128, 0, 0);
    }
    const uint32_t so = ((uint32_t)g * (uint32_t)N + (uint32_t)(t * TN)) * 4u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, I8GS_LDS(st + S::WB + S::AB + wave * 256), 4, s_voff, (int)so, 0, 0);
}

// One stage on the MFMA units: per column quad cc both K steps for every m tile of
// this wave (int32, exact), then the fold acc += scale * float(group sum).
template <int MT, int TN>
__device__ __forceinline__ void decode_compute(const char *st, int slab, int mpart, int li, int lb,
                                               float (&acc)[4][DecodeShape<MT, TN>::MTW][4]) {
    using S = DecodeShape<MT, TN>;
    v4i b[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            b[s][i] = *reinterpret_cast<const v4i *>(st + (16 * s + 4 * lb + i) * (TN * 4) + (slab * 64 + 4 * li) * 4);
    v4i af[2][S::MTW];
    const int swz = (li >> 1) & 7;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int m = 0; m < S::MTW; ++m) {
            const int row = (mpart * S::MTW + m) * 16 + li;
            af[s][m] = *reinterpret_cast<const v4i *>(st + S::WB + row * 128 + (((s * 4 + lb) ^ swz) * 16));
        }
    const v4f sc = *reinterpret_cast<const v4f *>(st + S::WB + S::AB + (slab * 64 + 4 * li) * 4);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
        v4i p[S::MTW];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const v4i bf = v4i{b[s][0][cc], b[s][1][cc], b[s][2][cc], b[s][3][cc]} ^ (int)0x80808080;
#pragma unroll
            for (int m = 0; m < S::MTW; ++m) p[m] = mfma_i8(af[s][m], bf, s == 0 ? v4i{0, 0, 0, 0} : p[m]);
        }
#pragma unroll
        for (int m = 0; m < S::MTW; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[cc][m][r] += sc[cc] * (float)p[m][r];
    }
}

// Units of workgroup b when U units are split evenly over P workgroups:
// [floor(b*U/P), floor((b+1)*U/P)).  The launch keeps P*U below 2^32.
__device__ __forceinline__ int range_begin(int b, int U, int P) { return (int)((uint32_t)b * (uint32_t)U / (uint32_t)P); }
__device__ __forceinline__ int owner_of(int u, int U, int P) {
    return (int)((((uint32_t)u + 1u) * (uint32_t)P - 1u) / (uint32_t)U);
}

// bf16(a_scale[row] * acc) of this lane's 4 adjacent columns, packed for one 8-byte store.
__device__ __forceinline__ v2i pack_y(float a, float c0, float c1, float c2, float c3) {
    return v2i{(int)(f32_to_bf16_bits(a * c0) | ((uint32_t)f32_to_bf16_bits(a * c1) << 16)),
               (int)(f32_to_bf16_bits(a * c2) | ((uint32_t)f32_to_bf16_bits(a * c3) << 16))};
}

template <int MT, int TN, int D>
__global__ __launch_bounds__(256) void w8a8_decode_kernel(const int8_t *__restrict__ qa,
                                                          const float *__restrict__ a_scale,
                                                          const int32_t *__restrict__ qweight,
                                                          const float *__restrict__ w_scale,
                                                          uint16_t *__restrict__ y, int64_t ldy, int M, int N, int K,
                                                          int tiles, int P, float *__restrict__ part) {
    using S = DecodeShape<MT, TN>;
    constexpr int MTW = S::MTW;
    static_assert(D >= 2 && D <= 8 && D * S::STAGE <= 160 * 1024, "LDS ring too large");
    // One LDS object only: with a second one the compiler can no longer tell the
    // ring's reads from the copies in flight and waits for all of them.
    __shared__ __attribute__((aligned(1024))) char lds[D * S::STAGE];

    const int b = blockIdx.x;
    const int G = K >> 7;
    const int U = tiles * G;
    const int u0 = range_begin(b, U, P), u1 = range_begin(b + 1, U, P);
    if (u0 >= u1) return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slab = wave % S::CQ, mpart = wave / S::CQ;
    const int li = lane & 15, lb = lane >> 4;
    const int row0 = mpart * MTW * 16 + 4 * lb;  // this lane's rows: row0 + 16*m + r
    const int lcol = slab * 64 + 4 * li;         // this lane's 4 columns within a tile

    // byte offsets fit 32 bits: K*N < 2^32, M*K < 2^32 and M*ldy*2 < 2^31 are checked
    // before launch
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc((void *)qweight, 0, (int)((uint32_t)K * (uint32_t)N), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t ar =
        __builtin_amdgcn_make_buffer_rsrc((void *)qa, 0, (int)((uint32_t)M * (uint32_t)K), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t sr =
        __builtin_amdgcn_make_buffer_rsrc((void *)w_scale, 0, (int)((uint32_t)G * (uint32_t)N * 4u), kRsrcWord3);
    // Output stores go through a buffer descriptor whose range check drops those
    // outside y (rows >= M; columns >= N are sent past the end explicitly).
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)y, 0, (int)(((uint32_t)(M - 1) * (uint32_t)ldy + (uint32_t)N) * 2u), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)part, 0, (int)((uint32_t)P * 2u * (uint32_t)(64 * TN * 4)), kRsrcWord3);

    // Per-lane parts of the copy addresses.  Weights: packed row lane / LPR of the
    // copy, columns 4*(lane % LPR) .. +3.  Activations: LDS slot lane % 8 of row
    // 8*copy + lane / 8 holds piece slot ^ ((row / 2) % 8) of that row (rows past M
    // repeat row M - 1; their results are never stored).  Scales: column
    // (64*wave + lane) % TN.
    const int w_voff = (lane / S::LPR) * N * 4 + (lane % S::LPR) * 16;
    int a_voff[S::AI];
#pragma unroll
    for (int j = 0; j < S::AI; ++j) {
        const int row = (wave * S::AI + j) * 8 + (lane >> 3);
        const int piece = (lane & 7) ^ ((row >> 1) & 7);
        a_voff[j] = (int)((uint32_t)min(row, M - 1) * (uint32_t)K + (uint32_t)piece * 16u);
    }
    const int s_voff = ((wave * 64 + lane) % TN) * 4;

    // Row scales of this lane's output rows (4 consecutive rows per m tile; rows past
    // M read as 0), loaded and waited for before the ring starts: memory operations
    // complete in order, so a wait for a load issued later would drain the ring.
    const __amdgpu_buffer_rsrc_t asr =
        __builtin_amdgcn_make_buffer_rsrc((void *)a_scale, 0, (int)((uint32_t)M * 4u), kRsrcWord3);
    v4f as[MTW];
#pragma unroll
    for (int m = 0; m < MTW; ++m)
        as[m] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(asr, (row0 + 16 * m) * 4, 0, 0));
#pragma unroll
    for (int m = 0; m < MTW; ++m) asm volatile("" ::"v"(as[m]));

    int ti = u0 / G, gi = u0 - (u0 / G) * G;  // next unit to copy
#pragma unroll
    for (int s = 0; s < D - 1; ++s) {
        if (u0 + s < u1) {
            decode_issue<MT, TN>(lds + s * S::STAGE, wr, ar, sr, wave, w_voff, a_voff, s_voff, ti, gi, N);
            if (++gi == G) { gi = 0; ++ti; }
        }
    }

    const int t_first = u0 / G;
    int tc = t_first, gc = u0 - t_first * G;  // unit being computed
    int seg_g0 = gc;                          // first group of the current tile segment
    float acc[4][MTW][4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
        for (int m = 0; m < MTW; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[cc][m][r] = 0.0f;

    int slot = 0;
    for (int u = u0; u < u1; ++u) {
        // Memory operations complete in order; the D-2 stages after this one are the
        // youngest copies, so this count waits for this stage.  Stores issued at the
        // end of a tile segment are younger still and make this wait longer, not
        // shorter (counting them exactly, so they stay in flight, measured slower).
        if (u + D - 2 < u1) wait_vmcnt<(D - 2) * S::LPS>();
        else wait_vmcnt<0>();
        barrier_only();
        __builtin_amdgcn_sched_barrier(0);
        if (u + D - 1 < u1) {
            const int ns = slot == 0 ? D - 1 : slot - 1;  // slot of the previous stage, now free
            decode_issue<MT, TN>(lds + ns * S::STAGE, wr, ar, sr, wave, w_voff, a_voff, s_voff, ti, gi, N);
            if (++gi == G) { gi = 0; ++ti; }
        }
        __builtin_amdgcn_sched_barrier(0);
        decode_compute<MT, TN>(lds + slot * S::STAGE, slab, mpart, li, lb, acc);
        slot = slot == D - 1 ? 0 : slot + 1;

        if (gc == G - 1 || u == u1 - 1) {
            const int col = tc * TN + lcol;
            if (seg_g0 == 0 && gc == G - 1) {
                // whole tile: y = bf16(a_scale[row] * sum), 4 columns per store
                const uint32_t cbase = col < N ? (uint32_t)col * 2u : 0x80000000u;
#pragma unroll
                for (int m = 0; m < MTW; ++m)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const uint32_t off = cbase + (uint32_t)(row0 + 16 * m + r) * (uint32_t)ldy * 2u;
                        __builtin_amdgcn_raw_buffer_store_b64(
                            pack_y(as[m][r], acc[0][m][r], acc[1][m][r], acc[2][m][r], acc[3][m][r]), yr,
                            (int)(col < N ? off : 0x80000000u), 0, 0);
                    }
            } else {
                // piece of a split tile: fp32 [row][TN] in slot 0 (first tile of this
                // range) or 1 (last tile)
                const int soff = (b * 2 + (tc == t_first ? 0 : 1)) * (64 * TN * 4);
#pragma unroll
                for (int m = 0; m < MTW; ++m)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        __builtin_amdgcn_raw_buffer_store_b128(
                            __builtin_bit_cast(v4i, v4f{acc[0][m][r], acc[1][m][r], acc[2][m][r], acc[3][m][r]}),
                            pr, ((row0 + 16 * m + r) * TN + lcol) * 4, soff, 0);
            }
#pragma unroll
            for (int cc = 0; cc < 4; ++cc)
#pragma unroll
                for (int m = 0; m < MTW; ++m)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[cc][m][r] = 0.0f;
            seg_g0 = 0;
        }
        if (++gc == G) { gc = 0; ++tc; }
    }
}

// Sums the pieces of every split tile in workgroup order and writes y.  Block x takes
// the tile holding the boundary between workgroups x and x + 1 when that boundary lies
// strictly inside a tile and is the first such boundary of the tile; block y covers
// 256 (row, 4-column) pieces of it.
template <int TN>
__global__ __launch_bounds__(256) void w8a8_splitk_reduce(const float *__restrict__ part,
                                                          const float *__restrict__ a_scale,
                                                          uint16_t *__restrict__ y, int64_t ldy, int M, int N,
                                                          int tiles, int G, int P) {
    const int U = tiles * G;
    const int bi = blockIdx.x + 1;
    const int ub = range_begin(bi, U, P);
    const int t = ub / G;
    if (ub == t * G) return;
    if (bi > 1 && range_begin(bi - 1, U, P) > t * G) return;
    constexpr int QPR = TN / 4;
    const int idx = blockIdx.y * 256 + threadIdx.x;
    const int row = idx / QPR, q = idx % QPR;
    const int col = t * TN + 4 * q;
    if (row >= M || col >= N) return;
    const int bf = owner_of(t * G, U, P), bl = owner_of(t * G + G - 1, U, P);
    const float *src = part + row * TN + 4 * q;
    v4f sum;
    for (int w0 = bf; w0 <= bl; w0 += 8) {
        // up to 8 pieces in flight at once, summed in workgroup order
        v4f v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int w = w0 + j;
            if (w > bl) break;
            const int sl = range_begin(w, U, P) / G == t ? 0 : 1;
            v[j] = *reinterpret_cast<const v4f *>(src + (int64_t)(w * 2 + sl) * (64 * TN));
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (w0 + j <= bl) sum = (w0 + j == bf) ? v[j] : sum + v[j];
    }
    *reinterpret_cast<v2i *>(y + (int64_t)row * ldy + col) = pack_y(a_scale[row], sum[0], sum[1], sum[2], sum[3]);
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

#ifndef I8GS_DECODE_TN
#define I8GS_DECODE_TN 128
#endif
#ifndef I8GS_DECODE_STAGES
#define I8GS_DECODE_STAGES 3
#endif

struct DecodePlan {
    int tn;      // tile columns
    int tiles;   // column tiles
    int blocks;  // workgroups sharing the (tile, group) units
};

DecodePlan decode_plan(int M, int N, int K, int workgroups) {
    (void)M;
    DecodePlan p;
    p.tn = I8GS_DECODE_TN;
    p.tiles = (N + p.tn - 1) / p.tn;
    const int64_t U = (int64_t)p.tiles * (K / kGroup);
    int64_t P = workgroups > 0 ? workgroups : (int64_t)device_cu_count();
    if (P > U) P = U;
    if (P * U >= (int64_t(1) << 32)) P = ((int64_t(1) << 32) - 1) / U;  // 32-bit range arithmetic
    if (P < 1) P = 1;
    p.blocks = (int)P;
    return p;
}

// Two fp32 partial tiles (64 rows) per workgroup.
size_t decode_workspace(const DecodePlan &p) { return align256(size_t(p.blocks) * 2 * 64 * p.tn * sizeof(float)); }

template <int MT, int TN>
hipError_t launch_decode(const W8A8Args &a, const DecodePlan &p, hipStream_t st) {
    constexpr int D = I8GS_DECODE_STAGES;
    float *part = (float *)a.ws;
    w8a8_decode_kernel<MT, TN, D><<<p.blocks, 256, 0, st>>>(a.qa, a.a_scale, a.qweight, a.w_scale, a.y, a.ldy, a.M,
                                                             a.N, a.K, p.tiles, p.blocks, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.blocks < 2) return e;
    const dim3 grid(p.blocks - 1, (a.M * (TN / 4) + 255) / 256);
    w8a8_splitk_reduce<TN><<<grid, 256, 0, st>>>(part, a.a_scale, a.y, a.ldy, a.M, a.N, p.tiles, a.K / kGroup,
                                                 p.blocks);
    return hipGetLastError();
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

// The decode kernel addresses y with 32-bit offsets.
bool decode_y_fits(int64_t M, int64_t ldy) { return M * ldy * 2 < (int64_t(1) << 31); }

size_t w8a8_gemm_workspace(int M, int N, int K, int kernel, int workgroups) {
    if (use_decode(M, kernel)) return decode_workspace(decode_plan(M, N, K, workgroups));
    return 0;
}

hipError_t launch_w8a8_gemm(const W8A8Args &a, hipStream_t s) {
    if (a.P == nullptr && use_decode(a.M, a.kernel) && decode_y_fits(a.M, a.ldy)) {
        const DecodePlan p = decode_plan(a.M, a.N, a.K, a.workgroups);
        if (a.M <= 32) return launch_decode<2, I8GS_DECODE_TN>(a, p, s);
        return launch_decode<4, I8GS_DECODE_TN>(a, p, s);
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
