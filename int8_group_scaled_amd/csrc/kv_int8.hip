// INT8 block-g128 KV cache: the codec and the INT8 attention products (QK and PV).
//
// Flint-DFlash2-GPTQ-INT8-PTQR model card, serving recipe and notes: the target and the
// draft keep their KV cache as "int8_block_g128" -- INT8 codes with one scale per
// 128-wide group, i.e. per head vector of 128 -- and take INT8 dot products for QK and
// for PV (the recipe's INT8 DOT / PV flags).  The codec is the per-token quantiser of
// the linear layer applied to each 128-wide row: scale = absmax / 127 (fp32),
// codes = clamp(rint(x / scale), -127, 127).
//
// QK: s[h, i, t] = scale * qs[i, h] * ks[t, hk] * sum_d qq[i, h, d] * kq[t, hk, d], with
// hk = h / (Hq / Hkv); the dot is exact in int32 (v_mfma_i32_32x32x32_i8, four per 32x32
// tile of queries x tokens), the three scale products are fp32.
//
// PV (INT8 PV): for probabilities p [Hq, Mq, T] and the INT8 V cache, the V scale of
// each token moves onto its probability, p' = fl32(p * vs), and p' is quantised per
// block of 128 tokens with the same codec (ps = max |p'| / 127, pq = clamp(rint(p' / ps)));
// out[h, i, d] = sum_b ps[h, i, b] * sum_{t in b} pq[h, i, t] * vq[t, hk, d], the int32
// block sums exact (MFMA) and folded in fp32 -- the group-scaled INT8 product of the
// linear layer with K = tokens.
#include <algorithm>

#include "act_quant.h"

namespace i8gs {
namespace {

// Maximum over each row of 16 lanes (non-negative floats compared as bit patterns):
// the two quad permutations and the half-row and row mirrors.
__device__ __forceinline__ float row16_max(float m) {
    int v = __builtin_bit_cast(int, m);
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false));  // row_half_mirror
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false));  // row_mirror
    return __builtin_bit_cast(float, v);
}

// Codec: 16 lanes per 128-wide row, 8 values each; 16 rows per workgroup of 256.
// Row r = t * H + hh is the head vector hh of token t, read at kv + t * ld + 128 * hh.
__global__ __launch_bounds__(256) void kv_quant_kernel(const uint16_t *__restrict__ kv, int64_t T, int H, int64_t ld,
                                                       int8_t *__restrict__ codes, float *__restrict__ scales) {
    const int64_t r = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int j = threadIdx.x & 15;
    const bool live = r < T * H;
    const int64_t t = live ? r / H : 0, hh = live ? r - t * H : 0;
    const v4i v = live ? *reinterpret_cast<const v4i *>(kv + t * ld + 128 * hh + 8 * j) : v4i{0, 0, 0, 0};
    const float amax = row16_max(absmax8(v, 0.0f));
    const float s = amax / 127.0f;
    const v2i q = quant8(v, s, row_inverse(s));
    if (live) {
        *reinterpret_cast<v2i *>(codes + r * 128 + 8 * j) = q;
        if (j == 0) scales[r] = s;
    }
}

// Rows of one KV head group.  The Hq/Hkv query heads of KV head hk and the Mq queries
// form R = (Hq/Hkv) * Mq rows r = (h - hk*Hq/Hkv) * Mq + i; row r is row hk*R + r of
// the [Hq*Mq, ...] score, probability and output matrices.

// QK: a workgroup covers 32 tokens per wave (four waves, fewer for short contexts) and
// up to 64 rows of one group (two 32-row tiles).  A wave loads its tokens' K vectors once as the B operand of
// v_mfma_i32_32x32x32_i8 (lane l: token l % 32, 16 bytes of the head dimension at
// 16*(l/32) + 32*step, four steps) and multiplies them with each row tile's query
// vectors (the A operand, the same byte placement).  Register i of the result holds
// token l % 32 of row 8*(i/4) + 4*(l/32) + i%4, so each store instruction writes two
// rows of 32 consecutive scores (128 bytes each).
typedef int v16i_kv __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void attn_qk_kernel(const int8_t *__restrict__ qq, const float *__restrict__ qs,
                                                      const int8_t *__restrict__ kq, const float *__restrict__ ks,
                                                      float scale, int Mq, int T, int Hq, int Hkv,
                                                      float *__restrict__ s_out, int32_t *__restrict__ dots) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hk = blockIdx.y, rep = Hq / Hkv, R = rep * Mq;
    const int t0 = (blockIdx.x * (blockDim.x >> 6) + wave) * 32;
    if (t0 >= T) return;
    const int li = lane & 31, h = lane >> 5;
    const int kt = min(t0 + li, T - 1);  // tokens past the end: never stored
    const int8_t *krow = kq + ((int64_t)kt * Hkv + hk) * 128 + 16 * h;
    v4i b[4];
#pragma unroll
    for (int ks2 = 0; ks2 < 4; ++ks2) b[ks2] = *reinterpret_cast<const v4i *>(krow + 32 * ks2);
    const int t = t0 + li;
    const float kscale = ks[(int64_t)kt * Hkv + hk];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int r0 = blockIdx.z * 64 + rt * 32;
        if (r0 >= R) break;
        // lane li's row of the tile: its query vector (A operand) and scale * qs (shared by
        // shuffles with the lanes that store that row)
        const int ra = min(r0 + li, R - 1);
        const int qi = ra % Mq, qh = hk * rep + ra / Mq;
        const int8_t *qrow = qq + ((int64_t)qi * Hq + qh) * 128 + 16 * h;
        const float sq = scale * qs[(int64_t)qi * Hq + qh];
        v16i_kv acc;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = 0;
#pragma unroll
        for (int ks2 = 0; ks2 < 4; ++ks2)
            acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(*reinterpret_cast<const v4i *>(qrow + 32 * ks2), b[ks2], acc,
                                                        0, 0, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int rr = 8 * (i >> 2) + 4 * h + (i & 3);  // row within the tile
            const float sqr = __shfl(sq, rr, 64);
            const int r = r0 + rr;
            if (t < T && r < R) {
                const int64_t o = ((int64_t)hk * R + r) * T + t;
                s_out[o] = sqr * kscale * (float)acc[i];
                if (dots) dots[o] = acc[i];
            }
        }
    }
}

// PV: a workgroup computes 32 rows x 128 output columns of one group over a range of
// token blocks.  Per block of 128 tokens:
//  1. quantise p' = p * vs for its 32 rows: thread (row tid/8, q = tid%8) takes tokens
//     q + 8j (j = 0..15), so each load instruction reads 8 consecutive floats of a row;
//     the block maximum is taken over the 8 lanes of the row;
//  2. copy V transposed into LDS, column-major by token;
//  3. four 32x32x32 int8 MFMA per wave (wave w: columns 32w .. 32w+31), then the fold
//     acc += ps[row] * block sum.
// In LDS the tokens of a block sit in the order u = 16q + j <-> token q + 8j, for the
// probability codes and the V columns alike, so a lane's 16 codes are one 16-byte row
// piece and the MFMA operands (16 consecutive positions) pair the same tokens.
// The next block's probabilities, V scales and V pieces are loaded into registers while
// the current block's products run.
constexpr int kPvLd = 144;  // LDS row pitch in bytes (128 + 16: spreads rows over the banks)

struct PvStage {
    float p[16], vs[16];
    v4i v[4];
};

__device__ __forceinline__ void pv_load(PvStage &st, const float *__restrict__ prow, bool row_live,
                                        const int8_t *__restrict__ vq, const float *__restrict__ vs, int tb, int T,
                                        int Hkv, int hk, int q, int vt0, int vc) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int t = tb + q + 8 * j;
        const bool live = t < T;
        st.vs[j] = live ? vs[(int64_t)t * Hkv + hk] : 0.0f;
        st.p[j] = live && row_live ? prow[t] : 0.0f;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int t = tb + vt0 + 8 * m;
        st.v[m] = t < T ? *reinterpret_cast<const v4i *>(vq + ((int64_t)t * Hkv + hk) * 128 + 16 * vc)
                        : v4i{0, 0, 0, 0};
    }
}

// Byte k of each of four words, as one word (byte m from word m).
__device__ __forceinline__ uint32_t gather_byte(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, int k) {
    const int sh = 8 * k;
    return ((w0 >> sh) & 0xFFu) | (((w1 >> sh) & 0xFFu) << 8) | (((w2 >> sh) & 0xFFu) << 16) |
           (((w3 >> sh) & 0xFFu) << 24);
}

typedef int v16i_pv __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void attn_pv_kernel(const float *__restrict__ p, const int8_t *__restrict__ vq,
                                                      const float *__restrict__ vs, int Mq, int T, int Hq, int Hkv,
                                                      int S, int blocks_per_split, float *__restrict__ out,
                                                      int8_t *__restrict__ pq_out, float *__restrict__ ps_out,
                                                      float *__restrict__ part) {
    __shared__ __attribute__((aligned(16))) int8_t s_pq[32 * kPvLd];
    __shared__ __attribute__((aligned(16))) int8_t s_vt[128 * kPvLd];
    __shared__ float s_ps[32];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int split = blockIdx.x, hk = blockIdx.y, rep = Hq / Hkv, R = rep * Mq;
    const int r0 = blockIdx.z * 32;
    const int B = (T + 127) / 128;
    const int b_begin = split * blocks_per_split, b_end = min(B, b_begin + blocks_per_split);
    // quantisation role
    const int qr = tid >> 3, q = tid & 7;
    const bool row_live = r0 + qr < R;
    const int64_t prow_index = (int64_t)hk * R + min(r0 + qr, R - 1);
    const float *prow = p + prow_index * (int64_t)T;
    // V copy role: tokens vt0 + 8m (m = 0..3) with vt0 = a % 8 + 32 * (a / 8), columns 16*vc ..
    const int a = tid & 31, vc = tid >> 5;
    const int vq0 = a & 7, vj0 = 4 * (a >> 3);
    const int vt0 = vq0 + 8 * vj0;
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;

    PvStage st;
    if (b_begin < b_end) pv_load(st, prow, row_live, vq, vs, b_begin * 128, T, Hkv, hk, q, vt0, vc);
    for (int b = b_begin; b < b_end; ++b) {
        const int tb = b * 128;
        // 1. quantise (p' = fl32(p * vs); zero past T and for rows past R)
        float pp[16];
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            pp[j] = st.p[j] * st.vs[j];
            amax = fmaxf(amax, fabsf(pp[j]));
        }
        {
            int v = __builtin_bit_cast(int, amax);
            v = max(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
            v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
            v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false));  // row_half_mirror
            amax = __builtin_bit_cast(float, v);
        }
        const float ps = amax / 127.0f;
        uint32_t code[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            float c = 0.0f;
            if (ps != 0.0f) c = fminf(fmaxf(rintf(pp[j] / ps), -127.0f), 127.0f);
            code[j >> 2] |= ((uint32_t)(int)c & 0xFFu) << (8 * (j & 3));
        }
        *reinterpret_cast<v4i *>(s_pq + qr * kPvLd + 16 * q) =
            v4i{(int)code[0], (int)code[1], (int)code[2], (int)code[3]};
        if (q == 0) s_ps[qr] = ps;
        if (row_live) {
            if (pq_out) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int t = tb + q + 8 * j;
                    if (t < T) pq_out[prow_index * T + t] = (int8_t)(code[j >> 2] >> (8 * (j & 3)));
                }
            }
            if (ps_out && q == 0) ps_out[prow_index * B + b] = ps;
        }
        // 2. V transposed: column d, positions u = 16*vq0 + vj0 + m (m = 0..3) as one word
#pragma unroll
        for (int w = 0; w < 4; ++w)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int d = 16 * vc + 4 * w + k;
                *reinterpret_cast<uint32_t *>(s_vt + d * kPvLd + 16 * vq0 + vj0) =
                    gather_byte((uint32_t)st.v[0][w], (uint32_t)st.v[1][w], (uint32_t)st.v[2][w],
                                (uint32_t)st.v[3][w], k);
            }
        // the next block's inputs stay in flight during the products
        if (b + 1 < b_end) pv_load(st, prow, row_live, vq, vs, tb + 128, T, Hkv, hk, q, vt0, vc);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        barrier_only();
        // 3. products: lane l -> row l % 32 of the codes, column 32*wave + l % 32 of V
        v16i_pv pi;
#pragma unroll
        for (int i = 0; i < 16; ++i) pi[i] = 0;
#pragma unroll
        for (int ks2 = 0; ks2 < 4; ++ks2) {
            const int u = 32 * ks2 + 16 * (lane >> 5);
            const v4i av = *reinterpret_cast<const v4i *>(s_pq + (lane & 31) * kPvLd + u);
            const v4i bv = *reinterpret_cast<const v4i *>(s_vt + (32 * wave + (lane & 31)) * kPvLd + u);
            pi = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, pi, 0, 0, 0);
        }
        // register i: column 32*wave + l % 32, row 8*(i/4) + 4*(l/32) + i%4
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] += s_ps[8 * (i >> 2) + 4 * (lane >> 5) + (i & 3)] * (float)pi[i];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        barrier_only();
    }

    // register i: row 8*(i/4) + 4*(l/32) + i%4 of the tile, column 32*wave + l % 32
    const int d = 32 * wave + (lane & 31);
    if (S > 1) {
        // this split's 32 x 128 partial, row-major, at (tile * S + split) * 4096; the
        // reduction kernel sums the splits
        float *dst = part + ((int64_t)(blockIdx.y * gridDim.z + blockIdx.z) * S + split) * 4096;
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[(8 * (i >> 2) + 4 * (lane >> 5) + (i & 3)) * 128 + d] = acc[i];
        return;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = r0 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        if (r < R) out[((int64_t)hk * R + r) * 128 + d] = acc[i];
    }
}

// Sum of the PV splits: a workgroup takes 64 cells of a tile's 32 x 128 output; thread
// group g (of 4) sums splits g*SG .. in order, then group 0 adds the four group sums in
// order -- a fixed order, so the result does not depend on scheduling.
__global__ __launch_bounds__(256) void attn_pv_reduce_kernel(const float *__restrict__ part, int S, int R,
                                                             int row_tiles, float *__restrict__ out) {
    __shared__ float s_sum[4][64];
    const int tile = blockIdx.y, hk = tile / row_tiles, r0 = (tile % row_tiles) * 32;
    const int c = blockIdx.x * 64 + (threadIdx.x & 63), g = threadIdx.x >> 6;
    const int SG = (S + 3) / 4;
    const int s0 = g * SG, s1 = min(S, s0 + SG);
    const float *src = part + (int64_t)tile * S * 4096 + c;
    // Up to 16 splits' cells in flight at once, then added in split order: the loads are
    // unconditional (an index past this group's last split reads that split again) so
    // that none waits for the one before it.
    float sum = 0.0f;
    for (int c0 = s0; c0 < s1; c0 += 16) {
        float v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = src[(int64_t)min(c0 + k, s1 - 1) * 4096];
#pragma unroll
        for (int k = 0; k < 16; ++k)
            if (c0 + k < s1) sum += v[k];
    }
    s_sum[g][threadIdx.x & 63] = sum;
    __syncthreads();
    if (g == 0) {
        const int r = r0 + c / 128;
        const float t = ((s_sum[0][threadIdx.x] + s_sum[1][threadIdx.x]) + s_sum[2][threadIdx.x]) + s_sum[3][threadIdx.x];
        if (r < R) out[((int64_t)hk * R + r) * 128 + (c & 127)] = t;
    }
}

}  // namespace

hipError_t launch_kv_quant(const uint16_t *kv, int64_t T, int H, int64_t ld, int8_t *codes, float *scales,
                           hipStream_t s) {
    kv_quant_kernel<<<(unsigned)((T * H + 15) / 16), 256, 0, s>>>(kv, T, H, ld, codes, scales);
    return hipGetLastError();
}

hipError_t launch_attn_qk(const int8_t *qq, const float *qs, const int8_t *kq, const float *ks, float scale, int Mq,
                          int T, int Hq, int Hkv, float *s_out, int32_t *dots, hipStream_t s) {
    const int R = Hq / Hkv * Mq;
    // 32 tokens per wave; four waves per workgroup, or fewer when that leaves fewer than
    // about two workgroups per compute unit (short contexts)
    const int64_t others = (int64_t)Hkv * ((R + 63) / 64);
    int waves = 4;
    while (waves > 1 && (T + 32 * waves - 1) / (32 * waves) * others < 512) waves >>= 1;
    dim3 grid((unsigned)((T + 32 * waves - 1) / (32 * waves)), (unsigned)Hkv, (unsigned)((R + 63) / 64));
    attn_qk_kernel<<<grid, 64 * waves, 0, s>>>(qq, qs, kq, ks, scale, Mq, T, Hq, Hkv, s_out, dots);
    return hipGetLastError();
}

PvPlan attn_pv_plan(int64_t Mq, int64_t T, int64_t Hq, int64_t Hkv) {
    PvPlan pl;
    const int64_t R = Hq / Hkv * Mq;
    const int64_t tiles = Hkv * ((R + 31) / 32);
    const int64_t B = (T + 127) / 128;
    // about 512 workgroups (two per compute unit; 256 and 1024 measured slower): split the
    // token blocks when the row tiles alone give fewer
    int64_t S = tiles >= 512 || B <= 1 ? 1 : std::min<int64_t>(B, (512 + tiles - 1) / tiles);
    const int64_t bps = S > 0 ? (B + S - 1) / std::max<int64_t>(S, 1) : 1;
    S = bps > 0 ? (B + bps - 1) / bps : 1;  // no empty split
    pl.S = (int)std::max<int64_t>(S, 1);
    pl.blocks_per_split = (int)std::max<int64_t>(bps, 1);
    pl.tiles = tiles;
    pl.part_bytes = pl.S > 1 ? (size_t)tiles * pl.S * 4096 * 4 : 0;
    return pl;
}

hipError_t launch_attn_pv(const float *p, const int8_t *vq, const float *vs, int Mq, int T, int Hq, int Hkv,
                          float *out, int8_t *pq_out, float *ps_out, float *part, hipStream_t s) {
    const PvPlan pl = attn_pv_plan(Mq, T, Hq, Hkv);
    const int R = Hq / Hkv * Mq, row_tiles = (R + 31) / 32;
    dim3 grid((unsigned)pl.S, (unsigned)Hkv, (unsigned)row_tiles);
    attn_pv_kernel<<<grid, 256, 0, s>>>(p, vq, vs, Mq, T, Hq, Hkv, pl.S, pl.blocks_per_split, out, pq_out, ps_out,
                                        part);
    if (pl.S > 1) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        attn_pv_reduce_kernel<<<dim3(64, (unsigned)pl.tiles), 256, 0, s>>>(part, pl.S, R, row_tiles, out);
    }
    return hipGetLastError();
}

}  // namespace i8gs
