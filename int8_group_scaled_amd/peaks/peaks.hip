// Achievable-peak microbenchmarks on the running GPU (gfx950): the measured ceilings the
// benchmark reports next to the vendor peaks (8 TB/s HBM, 5.0 POP/s dense INT8 MFMA).
//
//  * i8gs_peak_stream_read: every thread reads its share of a device buffer with
//    16-byte non-temporal loads (a grid-stride loop, many workgroups per CU) and folds
//    the words into one value it writes at the end: HBM read bandwidth when the buffer
//    is much larger than the last-level cache.
//  * i8gs_peak_mfma_i8: every wave runs `iters` rounds of four independent chains of
//    v_mfma_i32_32x32x32_i8 on register operands (no memory traffic) and writes one
//    value: the dense INT8 MFMA rate, 2*32*32*32 ops per instruction.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "i8gs_peaks.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void stream_read_kernel(const v4i *__restrict__ src, size_t nvec,
                                                          int *__restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * 256;
    v4i acc = v4i{0, 0, 0, 0};
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < nvec; i += stride)
        acc ^= __builtin_nontemporal_load(src + i);
    sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

__global__ __launch_bounds__(256) void mfma_i8_kernel(int iters, int seed, int *__restrict__ sink) {
    const v4i a = v4i{seed + (int)threadIdx.x, seed * 3, seed ^ 0x01010101, (int)threadIdx.x};
    const v4i b = v4i{seed * 5, (int)threadIdx.x * 7, seed + 11, seed ^ 0x7F7F7F7F};
    v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
    }
    int r = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) r ^= c0[i] ^ c1[i] ^ c2[i] ^ c3[i];
    sink[(size_t)blockIdx.x * 256 + threadIdx.x] = r;
}

}  // namespace

extern "C" {

int i8gs_peak_stream_read(const void *src, size_t bytes, int *sink, int blocks, void *stream) {
    if (!src || !sink || blocks <= 0 || (reinterpret_cast<uintptr_t>(src) & 15u)) return 1;
    stream_read_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>((const v4i *)src, bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

int i8gs_peak_mfma_i8(int iters, int *sink, int blocks, void *stream) {
    if (!sink || blocks <= 0 || iters <= 0) return 1;
    mfma_i8_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>(iters, 1, sink);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
