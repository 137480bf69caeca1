// Dynamic per-token symmetric INT8 activation quantisation (the row code and its
// citation are in act_quant.h).
//
// One workgroup per row: 1024 threads when there are few rows (decode; more waves
// per SIMD hide the latency of the load, the reduction and the fp32 divisions),
// 256 otherwise.  Each thread keeps its NV 16-byte vectors (8 bf16 each) in
// registers between the absmax reduction and the quantise step, so the row is read
// once; rows longer than TPB*8*13 elements take the two-pass variant (NV = 0),
// whose second read hits L2.
#include "act_quant.h"

namespace i8gs {
namespace {

template <int NV, int TPB>
__global__ __launch_bounds__(TPB) void quant_act_kernel(const uint16_t *__restrict__ x, int64_t ldx,
                                                        int K, int8_t *__restrict__ qa,
                                                        float *__restrict__ a_scale) {
    __shared__ float red[TPB / 64];
    const int m = blockIdx.x;
    quantize_row<NV, TPB>(x + (int64_t)m * ldx, K, qa + (int64_t)m * K, a_scale + m, red);
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
