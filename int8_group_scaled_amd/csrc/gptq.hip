// GPTQ unpack / dequantise and round-to-nearest G128 packing.
//
// Qwen3.8-27B-DFlash2-W4A16 model card, dequant-patch table: INT32-packed GPTQ
// weights are unpacked from int32 and scaled per group; Flint INT8 card, format
// table: symmetric, group 128, no g_idx (K in natural order).  Codes are offset
// binary (q + 2^(bits-1)); code j of word [r, n] is k = (32/bits)*r + j, in bits
// [bits*j, bits*j + bits).  The RTN packer follows the W4A16 card's scripts
// (round-to-nearest, no calibration): scale = group absmax / qmax in fp32,
// q = clamp(rint(w / scale)), q = 0 for an all-zero group.
#include "internal.h"

namespace i8gs {
namespace {

// One thread per (word row r, column n): writes the 32/bits codes of that word.
template <int BITS>
__global__ __launch_bounds__(256) void gptq_unpack_kernel(const int32_t *__restrict__ qw,
                                                          const float *__restrict__ ws, int K, int N,
                                                          int8_t *__restrict__ q_out,
                                                          float *__restrict__ w_out) {
    constexpr int PER = 32 / BITS;
    constexpr uint32_t MASK = (1u << BITS) - 1u;
    constexpr int OFF = 1 << (BITS - 1);
    const int nb = (N + 255) >> 8;
    const int n = (int)(blockIdx.x % nb) * 256 + threadIdx.x;
    const int r = (int)(blockIdx.x / nb);
    if (n >= N) return;
    const uint32_t word = (uint32_t)qw[(int64_t)r * N + n];
    const int k0 = r * PER;
    const float s = w_out ? ws[(int64_t)(k0 / kGroup) * N + n] : 0.0f;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int q = (int)((word >> (BITS * j)) & MASK) - OFF;
        const int64_t idx = (int64_t)(k0 + j) * N + n;
        if (q_out) q_out[idx] = (int8_t)q;
        if (w_out) w_out[idx] = s * (float)q;
    }
}

// One thread per (group g, column n); groups of gs consecutive K values.
template <int BITS>
__global__ __launch_bounds__(256) void gptq_rtn_kernel(const float *__restrict__ w, int K, int N, int gs,
                                                       int32_t *__restrict__ qw, float *__restrict__ ws) {
    constexpr int PER = 32 / BITS;
    constexpr float QMAX = BITS == 8 ? 127.0f : 7.0f;
    constexpr float QMIN = BITS == 8 ? -127.0f : -8.0f;
    constexpr int OFF = 1 << (BITS - 1);
    const int nb = (N + 255) >> 8;
    const int n = (int)(blockIdx.x % nb) * 256 + threadIdx.x;
    const int g = (int)(blockIdx.x / nb);
    if (n >= N) return;
    const float *col = w + (int64_t)g * gs * N + n;
    float amax = 0.0f;
    for (int i = 0; i < gs; ++i) amax = fmaxf(amax, fabsf(col[(int64_t)i * N]));
    const float s = amax / QMAX;
    ws[(int64_t)g * N + n] = s;
    for (int wi = 0; wi < gs / PER; ++wi) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            float q = 0.0f;
            if (s != 0.0f) {
                q = rintf(col[(int64_t)(wi * PER + j) * N] / s);
                q = fminf(fmaxf(q, QMIN), QMAX);
            }
            word |= (uint32_t)((int)q + OFF) << (BITS * j);
        }
        qw[((int64_t)g * (gs / PER) + wi) * N + n] = (int32_t)word;
    }
}

}  // namespace

hipError_t launch_gptq_unpack(const int32_t *qw, const float *ws, int bits, int K, int N, int8_t *q_out,
                              float *w_out, hipStream_t s) {
    const int per = 32 / bits;
    dim3 grid((unsigned)(((N + 255) / 256) * (int64_t)(K / per))), block(256);
    if (bits == 8)
        gptq_unpack_kernel<8><<<grid, block, 0, s>>>(qw, ws, K, N, q_out, w_out);
    else
        gptq_unpack_kernel<4><<<grid, block, 0, s>>>(qw, ws, K, N, q_out, w_out);
    return hipGetLastError();
}

hipError_t launch_gptq_rtn(const float *w, int bits, int group, int K, int N, int32_t *qw, float *ws,
                           hipStream_t s) {
    dim3 grid((unsigned)(((N + 255) / 256) * (int64_t)(K / group))), block(256);
    if (bits == 8)
        gptq_rtn_kernel<8><<<grid, block, 0, s>>>(w, K, N, group, qw, ws);
    else
        gptq_rtn_kernel<4><<<grid, block, 0, s>>>(w, K, N, group, qw, ws);
    return hipGetLastError();
}

}  // namespace i8gs
