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
// hk = h / (Hq / Hkv); the dot is exact in int32 (v_mfma_i32_16x16x64_i8, two per 16x16
// tile of queries x tokens), the three scale products are fp32.
//
// PV (INT8 PV): for probabilities p [Hq, Mq, T] and the INT8 V cache, the V scale of
// each token moves onto its probability, p' = fl32(p * vs), and p' is quantised per
// block of 128 tokens with the same codec (ps = max |p'| / 127, pq = clamp(rint(p' / ps)));
// out[h, i, d] = sum_b ps[h, i, b] * sum_{t in b} pq[h, i, t] * vq[t, hk, d], the int32
// block sums exact (MFMA) and folded in fp32 -- the group-scaled INT8 product of the
// linear layer with K = tokens.
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

// QK: a wave computes a 16 x 16 tile (queries i0.., tokens t0..) of one head.
__global__ __launch_bounds__(256) void attn_qk_kernel(const int8_t *__restrict__ qq, const float *__restrict__ qs,
                                                      const int8_t *__restrict__ kq, const float *__restrict__ ks,
                                                      float scale, int Mq, int T, int Hq, int Hkv,
                                                      float *__restrict__ s_out, int32_t *__restrict__ dots) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = blockIdx.z, hk = h / (Hq / Hkv);
    const int i0 = blockIdx.y * 16, t0 = (blockIdx.x * 4 + wave) * 16;
    if (t0 >= T) return;
    const int li = lane & 15, kb = lane >> 4;
    const int qi = min(i0 + li, Mq - 1), kt = min(t0 + li, T - 1);  // rows past the end: never stored
    const int8_t *qrow = qq + ((int64_t)qi * Hq + h) * 128 + 16 * kb;
    const int8_t *krow = kq + ((int64_t)kt * Hkv + hk) * 128 + 16 * kb;
    v4i acc = v4i{0, 0, 0, 0};
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2)
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(*reinterpret_cast<const v4i *>(qrow + 64 * ks2),
                                                    *reinterpret_cast<const v4i *>(krow + 64 * ks2), acc, 0, 0, 0);
    // lane: token t0 + li, queries i0 + 4*kb + r
    const int t = t0 + li;
    if (t >= T) return;
    const float kscale = ks[(int64_t)t * Hkv + hk];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = i0 + 4 * kb + r;
        if (i < Mq) {
            const int64_t o = ((int64_t)h * Mq + i) * T + t;
            s_out[o] = scale * qs[(int64_t)i * Hq + h] * kscale * (float)acc[r];
            if (dots) dots[o] = acc[r];
        }
    }
}

// PV: a workgroup of 4 waves per (head, 16 queries); wave w owns output columns
// 32w .. 32w+31 (two 16-column tiles).  Per block of 128 tokens: quantise p' into LDS
// (16 lanes per query row, 8 tokens each), copy the block's V rows into LDS, then two
// 64-token MFMA steps per tile, B gathered column-wise from the V rows, and the fold.
constexpr int kPvBlock = 128;

__global__ __launch_bounds__(256) void attn_pv_kernel(const float *__restrict__ p, const int8_t *__restrict__ vq,
                                                      const float *__restrict__ vs, int Mq, int T, int Hq, int Hkv,
                                                      float *__restrict__ out, int8_t *__restrict__ pq_out,
                                                      float *__restrict__ ps_out) {
    __shared__ __attribute__((aligned(16))) int8_t s_pq[16 * kPvBlock];
    __shared__ __attribute__((aligned(16))) int8_t s_v[kPvBlock * 128];
    __shared__ float s_ps[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = blockIdx.y, hk = h / (Hq / Hkv);
    const int i0 = blockIdx.x * 16;
    const int B = (T + kPvBlock - 1) / kPvBlock;
    const int li = lane & 15, kb = lane >> 4;
    // quantisation role: query row qr = tid / 16, tokens 8*(tid % 16) .. +7 of the block
    const int qr = tid >> 4, qj = tid & 15;
    const int qi = i0 + qr;
    float acc[2][4];
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[n][r] = 0.0f;

    for (int b = 0; b < B; ++b) {
        const int tb = b * kPvBlock;
        // p' = fl32(p * vs) for this thread's 8 tokens (zero past T or past the queries)
        float pp[8];
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int t = tb + 8 * qj + k;
            pp[k] = (qi < Mq && t < T) ? p[((int64_t)h * Mq + qi) * T + t] * vs[(int64_t)t * Hkv + hk] : 0.0f;
            amax = fmaxf(amax, fabsf(pp[k]));
        }
        amax = row16_max(amax);
        const float ps = amax / 127.0f;
        uint32_t code[2] = {0u, 0u};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            float q = 0.0f;
            if (ps != 0.0f) q = fminf(fmaxf(rintf(pp[k] / ps), -127.0f), 127.0f);
            code[k >> 2] |= ((uint32_t)(int)q & 0xFFu) << (8 * (k & 3));
        }
        *reinterpret_cast<v2i *>(s_pq + qr * kPvBlock + 8 * qj) = v2i{(int)code[0], (int)code[1]};
        if (qj == 0) s_ps[qr] = ps;
        if (qi < Mq) {
            if (pq_out) {
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int t = tb + 8 * qj + k;
                    if (t < T) pq_out[((int64_t)h * Mq + qi) * T + t] = (int8_t)(code[k >> 2] >> (8 * (k & 3)));
                }
            }
            if (ps_out && qj == 0) ps_out[((int64_t)h * Mq + qi) * B + b] = ps;
        }
        // V rows of the block: 128 tokens x 128 bytes, 16 bytes x 4 per thread (zeros past T)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int c = tid + 256 * k;  // 16-byte piece: token c / 8, bytes 16 * (c % 8)
            const int t = tb + (c >> 3);
            const v4i v = t < T ? *reinterpret_cast<const v4i *>(vq + ((int64_t)t * Hkv + hk) * 128 + 16 * (c & 7))
                                : v4i{0, 0, 0, 0};
            *reinterpret_cast<v4i *>(s_v + 16 * c) = v;
        }
        __syncthreads();
        // MFMA: A = pq rows (lane: row li, tokens 64*ks2 + 16*kb ..), B = V column
        // (lane: column 32*wave + 16*n + li, the same 16 tokens), gathered byte by byte
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int d = 32 * wave + 16 * n + li;
            v4i pi = v4i{0, 0, 0, 0};
#pragma unroll
            for (int ks2 = 0; ks2 < 2; ++ks2) {
                const int tk = 64 * ks2 + 16 * kb;
                const v4i a = *reinterpret_cast<const v4i *>(s_pq + li * kPvBlock + tk);
                v4i bv;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    uint32_t word = 0;
#pragma unroll
                    for (int k = 0; k < 4; ++k) word |= (uint32_t)(uint8_t)s_v[(tk + 4 * w + k) * 128 + d] << (8 * k);
                    bv[w] = (int)word;
                }
                pi = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bv, pi, 0, 0, 0);
            }
            // lane: column d, query rows 4*kb + r
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[n][r] += s_ps[4 * kb + r] * (float)pi[r];
        }
        __syncthreads();
    }
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = i0 + 4 * kb + r;
            if (i < Mq) out[((int64_t)h * Mq + i) * 128 + 32 * wave + 16 * n + li] = acc[n][r];
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
    dim3 grid((unsigned)((T + 63) / 64), (unsigned)((Mq + 15) / 16), (unsigned)Hq);
    attn_qk_kernel<<<grid, 256, 0, s>>>(qq, qs, kq, ks, scale, Mq, T, Hq, Hkv, s_out, dots);
    return hipGetLastError();
}

hipError_t launch_attn_pv(const float *p, const int8_t *vq, const float *vs, int Mq, int T, int Hq, int Hkv,
                          float *out, int8_t *pq_out, float *ps_out, hipStream_t s) {
    dim3 grid((unsigned)((Mq + 15) / 16), (unsigned)Hq);
    attn_pv_kernel<<<grid, 256, 0, s>>>(p, vq, vs, Mq, T, Hq, Hkv, out, pq_out, ps_out);
    return hipGetLastError();
}

}  // namespace i8gs
