// Per-token activation quantisation of one bf16 row by one workgroup: the device code
// shared by the standalone quantisation kernel and the decode GEMM's fused prologue.
//
// Flint-DFlash2-GPTQ-INT8-PTQR model card, serving notes: the W8A8 GEMM path quantises
// its bf16 inputs to INT8 on the fly (mode "round"); Qwen3.8-27B W8A8 card, serving
// section, the same.  Per row: a_scale = absmax / 127 (fp32) and
// codes = clamp(rint(x / a_scale), -127, 127), ties to even, with a correctly rounded
// fp32 division (hipcc's default for '/', no fast-math).
//
// The division per element is replaced by a product with inv = 1/a_scale (one correctly
// rounded division per row) wherever that provably gives the same code: r = fl(x * inv)
// and fl(x / a_scale) both lie within 1.5 * 2^-23 * |x / a_scale| <= 2.3e-5 of x / a_scale
// (|x / a_scale| <= 127 + 2^-16), so they round to the same integer unless r is within
// that distance of a half-integer.  Elements with r closer than 2^-15 to a half-integer
// take the exact division; rows whose inv overflows (a subnormal a_scale) take it for
// every element.
#pragma once

#include "internal.h"

namespace i8gs {

__device__ __forceinline__ float absmax8(v4i v, float m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t w = (uint32_t)v[i];
        m = fmaxf(m, fabsf(bf16_bits_to_f32(w & 0xFFFFu)));
        m = fmaxf(m, fabsf(bf16_bits_to_f32(w >> 16)));
    }
    return m;
}

// Quantise 8 bf16 values to 8 int8 codes packed in two dwords.  inv = 1/s, or 0 when
// the row divides exactly (s == 0 gives codes 0 either way).
__device__ __forceinline__ v2i quant8(v4i v, float s, float inv) {
    float x[8], r[8];
    bool exact = inv == 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w = (uint32_t)v[i];
        x[2 * i] = bf16_bits_to_f32(w & 0xFFFFu);
        x[2 * i + 1] = bf16_bits_to_f32(w >> 16);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float p = x[i] * inv;
        r[i] = rintf(p);
        exact |= fabsf(p - r[i]) > 0.5f - 0x1p-15f;  // p - rint(p) is exact
    }
    if (exact && s != 0.0f) {
        // keeps the compiler from computing the divisions ahead of the test
        __asm__ volatile("");
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = rintf(x[i] / s);
    }
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = (uint32_t)(int)fminf(fmaxf(r[i], -127.0f), 127.0f) & 0xFFu;
    v2i out;
    out[0] = (int)(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24));
    out[1] = (int)(b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
    return out;
}

// 1/s when the product path applies (s > 0 and 1/s finite), else 0.
__device__ __forceinline__ float row_inverse(float s) {
    const float inv = 1.0f / s;
    return s > 0.0f && inv <= 3.0e38f ? inv : 0.0f;
}

// Maximum over the 64 lanes of a wave of non-negative floats (compared as their bit
// patterns): DPP steps within each row of 16 lanes -- two quad permutations, then the
// half-row and row mirrors -- and then the four row maxima.
__device__ __forceinline__ float wave_max_nonneg(float m) {
    int v = __builtin_bit_cast(int, m);
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false));  // row_half_mirror
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false));  // row_mirror
    const int r = max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
                      max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
    return __builtin_bit_cast(float, r);
}

// Maximum over the workgroup (TPB threads; red: TPB/64 floats of LDS).
template <int TPB>
__device__ __forceinline__ float block_max(float m, float *red) {
    m = wave_max_nonneg(m);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int w = 1; w < TPB / 64; ++w) m = fmaxf(m, red[w]);
    return m;
}

// One row of K bf16 values (K a multiple of 8) by a workgroup of TPB threads: codes to
// qrow, the scale to *scale_out (thread 0).  NV > 0: each thread keeps its NV 16-byte
// vectors in registers between the reduction and the quantisation (K <= TPB*8*NV), so
// the row is read once; NV = 0: two passes, the second one hitting L2.
template <int NV, int TPB>
__device__ __forceinline__ void quantize_row(const uint16_t *__restrict__ xrow, int K, int8_t *__restrict__ qrow,
                                             float *__restrict__ scale_out, float *red) {
    const int nvec = K >> 3;
    const v4i *row = reinterpret_cast<const v4i *>(xrow);
    v2i *out = reinterpret_cast<v2i *>(qrow);
    float amax = 0.0f;
    if constexpr (NV > 0) {
        v4i v[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int c = threadIdx.x + i * TPB;
            v[i] = c < nvec ? __builtin_nontemporal_load(row + c) : v4i{0, 0, 0, 0};
            amax = absmax8(v[i], amax);
        }
        amax = block_max<TPB>(amax, red);
        const float s = amax / 127.0f;
        const float inv = row_inverse(s);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int c = threadIdx.x + i * TPB;
            if (c < nvec) out[c] = quant8(v[i], s, inv);
        }
        if (threadIdx.x == 0) *scale_out = s;
    } else {
        for (int c = threadIdx.x; c < nvec; c += TPB) amax = absmax8(row[c], amax);
        amax = block_max<TPB>(amax, red);
        const float s = amax / 127.0f;
        const float inv = row_inverse(s);
        for (int c = threadIdx.x; c < nvec; c += TPB) out[c] = quant8(row[c], s, inv);
        if (threadIdx.x == 0) *scale_out = s;
    }
}

}  // namespace i8gs
