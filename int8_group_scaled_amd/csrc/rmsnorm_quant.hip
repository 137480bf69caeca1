// RMS normalisation fused with the per-token INT8 quantisation of its output: the
// producer of the quantised activations of the qkv and gate/up projections.
//
// Qwen3.8-27B-DFlash2-W4A16 model card, bf16-surface table: the norms (input_layernorm,
// post_attention_layernorm) stay bf16 ahead of the quantised linears; qwen38/dflash2
// recipe, numerics: normalisation runs in FP32 keeping the intermediate BF16 casts;
// Flint card, serving notes: the W8A8 path quantises its bf16 inputs per token.  Per
// row of K bf16 values x with weights gamma (bf16 [K]):
//   r      = 1 / sqrt(sum_k x^2 / K + eps)
//   t[k]   = bf16(x[k] * r)          (the normalised value cast to bf16)
//   h[k]   = bf16(gamma[k] * t[k])   (times the weight, cast to bf16; optional output)
//   a_scale = max_k |h| / 127,  qa[k] = clamp(rint(h[k] / a_scale), -127, 127)
// Every step is carried out with each operation correctly rounded in fp64: the sum of
// squares of bf16 values is accumulated as a double-double (TwoSum), which holds it
// exactly here, and rounded once; then one fp64 division, addition, square root,
// reciprocal and product; gamma * t is exact in fp32 (two 8-bit significands), so both
// casts round values that are the exact ones up to fp64 rounding, and the quantisation
// of h is the per-token quantiser's (act_quant.h).
//
// One workgroup per row, the row held in registers (NV 16-byte vectors per thread).
#include "act_quant.h"

#pragma clang fp contract(off)

namespace i8gs {
namespace {

// s + e == a + b exactly (Knuth's TwoSum).
__device__ __forceinline__ void two_sum(double a, double b, double &s, double &e) {
    s = a + b;
    const double bb = s - a;
    e = (a - (s - bb)) + (b - bb);
}

// (hi, lo) += (bh, bl), renormalised.
__device__ __forceinline__ void dd_add(double &hi, double &lo, double bh, double bl) {
    double s, e;
    two_sum(hi, bh, s, e);
    e += lo + bl;
    hi = s + e;
    lo = e - (hi - s);
}

// bf16 bits of a double, rounded to nearest with ties to even (normal bf16 values by
// rounding the significand at bit 45; below 2^-126 to a multiple of 2^-133).
__device__ __forceinline__ uint32_t bf16_rne_f64(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
    const uint64_t mag = u & 0x7FFFFFFFFFFFFFFFull;
    const int e = (int)(mag >> 52) - 1023;
    if (e >= -126) {
        uint64_t m = mag >> 45;  // biased double exponent and the 7 leading mantissa bits
        const uint64_t rem = mag & ((1ull << 45) - 1);
        if (rem > (1ull << 44) || (rem == (1ull << 44) && (m & 1))) m += 1;
        const int be = (int)(m >> 7) - 1023 + 127;
        if (be >= 255) return sign | 0x7F80u;
        return sign | ((uint32_t)be << 7) | (uint32_t)(m & 0x7F);
    }
    const double n = rint(__builtin_bit_cast(double, mag) * 0x1p133);  // subnormal bf16 units
    return sign | (uint32_t)n;
}

// Sum of squares of 8 bf16 values into (hi, lo).
__device__ __forceinline__ void sumsq8(v4i v, double &hi, double &lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w = (uint32_t)v[i];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const double x = (double)bf16_bits_to_f32(j ? (w >> 16) : (w & 0xFFFFu));
            double s, e;
            two_sum(hi, x * x, s, e);  // x * x is exact
            hi = s;
            lo += e;
        }
    }
}

// h for 8 values: bf16(gamma * bf16(x * r)).
__device__ __forceinline__ v4i norm8(v4i xv, v4i gv, double r) {
    v4i out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t o = 0;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t xb = j ? ((uint32_t)xv[i] >> 16) : ((uint32_t)xv[i] & 0xFFFFu);
            const uint32_t gb = j ? ((uint32_t)gv[i] >> 16) : ((uint32_t)gv[i] & 0xFFFFu);
            const uint32_t t = bf16_rne_f64((double)bf16_bits_to_f32(xb) * r);
            const float p = bf16_bits_to_f32(gb) * bf16_bits_to_f32(t);  // exact
            o |= (uint32_t)f32_to_bf16_bits(p) << (16 * j);
        }
        out[i] = (int)o;
    }
    return out;
}

template <int TPB>
__device__ __forceinline__ void block_sum_dd(double &hi, double &lo, double *red_hi, double *red_lo) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const double bh = __shfl_xor(hi, off, 64), bl = __shfl_xor(lo, off, 64);
        dd_add(hi, lo, bh, bl);
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red_hi[wave] = hi;
        red_lo[wave] = lo;
    }
    __syncthreads();
    hi = red_hi[0];
    lo = red_lo[0];
#pragma unroll
    for (int w = 1; w < TPB / 64; ++w) dd_add(hi, lo, red_hi[w], red_lo[w]);
}

template <int NV, int TPB>
__global__ __launch_bounds__(TPB) void rmsnorm_quant_kernel(const uint16_t *__restrict__ x, int64_t ldx,
                                                             const uint16_t *__restrict__ gamma, double eps, int K,
                                                             uint16_t *__restrict__ h, int8_t *__restrict__ qa,
                                                             float *__restrict__ a_scale) {
    __shared__ double red_hi[TPB / 64], red_lo[TPB / 64];
    __shared__ float red[TPB / 64];
    const int m = blockIdx.x;
    const int nvec = K >> 3;
    const v4i *row = reinterpret_cast<const v4i *>(x + (int64_t)m * ldx);
    const v4i *grow = reinterpret_cast<const v4i *>(gamma);
    v4i v[NV], hv[NV];
    double hi = 0.0, lo = 0.0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = threadIdx.x + i * TPB;
        v[i] = c < nvec ? __builtin_nontemporal_load(row + c) : v4i{0, 0, 0, 0};
        sumsq8(v[i], hi, lo);
    }
    block_sum_dd<TPB>(hi, lo, red_hi, red_lo);
    const double ss = hi + lo;
    const double r = 1.0 / sqrt(ss / (double)K + eps);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = threadIdx.x + i * TPB;
        hv[i] = c < nvec ? norm8(v[i], grow[c], r) : v4i{0, 0, 0, 0};
        amax = absmax8(hv[i], amax);
    }
    amax = block_max<TPB>(amax, red);
    const float s = amax / 127.0f;
    const float inv = row_inverse(s);
    v2i *out = reinterpret_cast<v2i *>(qa + (int64_t)m * K);
    v4i *hout = h ? reinterpret_cast<v4i *>(h + (int64_t)m * K) : nullptr;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = threadIdx.x + i * TPB;
        if (c < nvec) {
            out[c] = quant8(hv[i], s, inv);
            if (hout) hout[c] = hv[i];
        }
    }
    if (threadIdx.x == 0) a_scale[m] = s;
}

template <int TPB, int NVMAX>
hipError_t launch_rmsq_tpb(const uint16_t *x, int64_t ldx, const uint16_t *gamma, double eps, int M, int K,
                           uint16_t *h, int8_t *qa, float *a_scale, hipStream_t s) {
    const int per_thread = (K / 8 + TPB - 1) / TPB;
    dim3 grid(M), block(TPB);
    if (per_thread <= 1)
        rmsnorm_quant_kernel<1, TPB><<<grid, block, 0, s>>>(x, ldx, gamma, eps, K, h, qa, a_scale);
    else if (per_thread <= 2)
        rmsnorm_quant_kernel<2, TPB><<<grid, block, 0, s>>>(x, ldx, gamma, eps, K, h, qa, a_scale);
    else if (per_thread <= 3)
        rmsnorm_quant_kernel<3, TPB><<<grid, block, 0, s>>>(x, ldx, gamma, eps, K, h, qa, a_scale);
    else if (NVMAX <= 4 || per_thread <= 4)
        rmsnorm_quant_kernel<4, TPB><<<grid, block, 0, s>>>(x, ldx, gamma, eps, K, h, qa, a_scale);
    else if (per_thread <= 9)
        rmsnorm_quant_kernel<(NVMAX > 4 ? 9 : 4), TPB><<<grid, block, 0, s>>>(x, ldx, gamma, eps, K, h, qa, a_scale);
    else
        rmsnorm_quant_kernel<NVMAX, TPB><<<grid, block, 0, s>>>(x, ldx, gamma, eps, K, h, qa, a_scale);
    return hipGetLastError();
}

}  // namespace

// Rows up to 32768 values take 1024 threads (at most 4 vectors each: more would spill at
// 16 waves per workgroup) when M <= 512; otherwise 256 threads hold up to 13 vectors each.
int rmsnorm_quant_max_k(int64_t M) { return M <= 512 ? 32768 : 256 * 8 * 13; }

hipError_t launch_rmsnorm_quant(const uint16_t *x, int64_t ldx, const uint16_t *gamma, double eps, int M, int K,
                                uint16_t *h, int8_t *qa, float *a_scale, hipStream_t s) {
    if (M <= 512) return launch_rmsq_tpb<1024, 4>(x, ldx, gamma, eps, M, K, h, qa, a_scale, s);
    return launch_rmsq_tpb<256, 13>(x, ldx, gamma, eps, M, K, h, qa, a_scale, s);
}

}  // namespace i8gs
