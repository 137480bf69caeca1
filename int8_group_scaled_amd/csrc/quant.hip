// Dynamic per-token symmetric INT8 activation quantisation.
//
// Flint-DFlash2-GPTQ-INT8-PTQR model card, serving notes: the W8A8 GEMM path
// quantises its bf16 inputs to INT8 on the fly (mode "round"); Qwen3.8-27B W8A8
// card, serving section, the same.  Per row: a_scale = absmax / 127 (fp32) and
// codes = clamp(rint(x / a_scale), -127, 127), ties to even, with a correctly
// rounded fp32 division (hipcc's default for '/', no fast-math).
//
// One workgroup per row: 1024 threads when there are few rows (decode; more waves
// per SIMD hide the latency of the load, the reduction and the fp32 divisions),
// 256 otherwise.  Each thread keeps its NV 16-byte vectors (8 bf16 each) in
// registers between the absmax reduction and the quantise step, so the row is read
// once; rows longer than TPB*8*13 elements take the two-pass variant (NV = 0),
// whose second read hits L2.
#include "internal.h"

namespace i8gs {
namespace {

__device__ __forceinline__ float absmax8(v4i v, float m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t w = (uint32_t)v[i];
        m = fmaxf(m, fabsf(bf16_bits_to_f32(w & 0xFFFFu)));
        m = fmaxf(m, fabsf(bf16_bits_to_f32(w >> 16)));
    }
    return m;
}

__device__ __forceinline__ int quant1(float xv, float s) {
    float r = rintf(xv / s);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

// Quantise 8 bf16 values to 8 int8 codes packed in two dwords.
__device__ __forceinline__ v2i quant8(v4i v, float s) {
    v2i out;
    if (s == 0.0f) {
        out[0] = 0;
        out[1] = 0;
        return out;
    }
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t w = (uint32_t)v[i];
        b[2 * i] = (uint32_t)quant1(bf16_bits_to_f32(w & 0xFFFFu), s) & 0xFFu;
        b[2 * i + 1] = (uint32_t)quant1(bf16_bits_to_f32(w >> 16), s) & 0xFFu;
    }
    out[0] = (int)(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24));
    out[1] = (int)(b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
    return out;
}

template <int TPB>
__device__ __forceinline__ float block_max(float m, float *red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int w = 1; w < TPB / 64; ++w) m = fmaxf(m, red[w]);
    return m;
}

template <int NV, int TPB>
__global__ __launch_bounds__(TPB) void quant_act_kernel(const uint16_t *__restrict__ x, int64_t ldx,
                                                        int K, int8_t *__restrict__ qa,
                                                        float *__restrict__ a_scale) {
    constexpr int kThreads = TPB;
    __shared__ float red[TPB / 64];
    const int m = blockIdx.x;
    const int nvec = K >> 3;
    const v4i *row = reinterpret_cast<const v4i *>(x + (int64_t)m * ldx);
    v2i *out = reinterpret_cast<v2i *>(qa + (int64_t)m * K);
    float amax = 0.0f;
    if constexpr (NV > 0) {
        v4i v[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int c = threadIdx.x + i * kThreads;
            v[i] = c < nvec ? __builtin_nontemporal_load(row + c) : v4i{0, 0, 0, 0};
            amax = absmax8(v[i], amax);
        }
        amax = block_max<TPB>(amax, red);
        const float s = amax / 127.0f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int c = threadIdx.x + i * kThreads;
            if (c < nvec) out[c] = quant8(v[i], s);
        }
        if (threadIdx.x == 0) a_scale[m] = s;
    } else {
        for (int c = threadIdx.x; c < nvec; c += kThreads) amax = absmax8(row[c], amax);
        amax = block_max<TPB>(amax, red);
        const float s = amax / 127.0f;
        for (int c = threadIdx.x; c < nvec; c += kThreads) out[c] = quant8(row[c], s);
        if (threadIdx.x == 0) a_scale[m] = s;
    }
}

template <int TPB>
hipError_t launch_quant_tpb(const uint16_t *x, int64_t ldx, int M, int K, int nvec, int8_t *qa, float *a_scale,
                            hipStream_t s) {
    const int per_thread = (nvec + TPB - 1) / TPB;
    dim3 grid(M), block(TPB);
    if (per_thread <= 1)
        quant_act_kernel<1, TPB><<<grid, block, 0, s>>>(x, ldx, K, qa, a_scale);
    else if (per_thread <= 2)
        quant_act_kernel<2, TPB><<<grid, block, 0, s>>>(x, ldx, K, qa, a_scale);
    else if (per_thread <= 3)
        quant_act_kernel<3, TPB><<<grid, block, 0, s>>>(x, ldx, K, qa, a_scale);
    else if (per_thread <= 4)
        quant_act_kernel<4, TPB><<<grid, block, 0, s>>>(x, ldx, K, qa, a_scale);
    else if (per_thread <= 9)
        quant_act_kernel<9, TPB><<<grid, block, 0, s>>>(x, ldx, K, qa, a_scale);
    else if (per_thread <= 13)
        quant_act_kernel<13, TPB><<<grid, block, 0, s>>>(x, ldx, K, qa, a_scale);
    else
        quant_act_kernel<0, TPB><<<grid, block, 0, s>>>(x, ldx, K, qa, a_scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_act(const uint16_t *x, int64_t ldx, int M, int K, int8_t *qa, float *a_scale,
                            hipStream_t s) {
    const int nvec = K / 8;
    if (M <= 512) return launch_quant_tpb<1024>(x, ldx, M, K, nvec, qa, a_scale, s);
    return launch_quant_tpb<256>(x, ldx, M, K, nvec, qa, a_scale, s);
}

}  // namespace i8gs
