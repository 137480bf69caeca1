// Internal declarations shared by the HIP translation units of libi8gs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "i8gs.h"

namespace i8gs {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kGroup = 128;

// Records a message for i8gs_last_error() and returns `status`.
int fail(int status, const std::string &msg);
// Clears the thread's last error and returns I8GS_OK.
int ok();
// Checks a HIP call result; on failure records it and returns I8GS_ERR_HIP.
int hip_check(hipError_t e, const char *what);
// Checks that the current device is gfx950 (cached per device).
int check_device();

// Kernel launchers (no validation; callers validate first).
hipError_t launch_quant_act(const uint16_t *x, int64_t ldx, int M, int K, int8_t *qa,
                            float *a_scale, hipStream_t s);
hipError_t launch_rmsnorm_quant(const uint16_t *x, int64_t ldx, const uint16_t *gamma, double eps, int M, int K,
                                uint16_t *h, int8_t *qa, float *a_scale, hipStream_t s);
int rmsnorm_quant_max_k(int64_t M);
hipError_t launch_kv_quant(const uint16_t *kv, int64_t T, int H, int64_t ld, int8_t *codes, float *scales,
                           hipStream_t s);
hipError_t launch_attn_qk(const int8_t *qq, const float *qs, const int8_t *kq, const float *ks, float scale, int Mq,
                          int T, int Hq, int Hkv, float *s_out, int32_t *dots, hipStream_t s);
// PV launch plan: S splits of the token blocks (blocks_per_split each), `tiles` row
// tiles of 32 rows; part_bytes of fp32 partial sums when S > 1.
struct PvPlan {
    int S, blocks_per_split;
    int64_t tiles;
    size_t part_bytes;
};
PvPlan attn_pv_plan(int64_t Mq, int64_t T, int64_t Hq, int64_t Hkv);
hipError_t launch_attn_pv(const float *p, const int8_t *vq, const float *vs, int Mq, int T, int Hq, int Hkv,
                          float *out, int8_t *pq_out, float *ps_out, float *part, hipStream_t s);
hipError_t launch_gptq_unpack(const int32_t *qw, const float *ws, int bits, int K, int N,
                              int8_t *q_out, float *w_out, hipStream_t s);
hipError_t launch_gptq_rtn(const float *w, int bits, int group, int K, int N, int32_t *qw, float *ws,
                           hipStream_t s);

struct W8A8Args {
    const int8_t *qa;
    const float *a_scale;
    const int32_t *qweight;
    const float *w_scale;
    uint16_t *y;
    int64_t ldy;
    int32_t *P;  // non-null: write group partials instead of y
    int M, N, K;
    int kernel;   // I8GS_KERNEL_*
    int workgroups;  // decode kernel workgroups, 0 = automatic
    int *counters;  // split-K arrival counters (kMaxCounters, zero on entry)
    void *ws;       // split-K partial sums
    size_t ws_bytes;
};
size_t w8a8_gemm_workspace(int M, int N, int K, int kernel, int workgroups);
// Whether y (M rows of stride ldy, padded to the kernel's row tiles) is small enough for
// the decode / prefill kernel's 32-bit offsets; an automatic choice falls back to the
// tiled kernel when it is not.
bool decode_y_fits(int64_t M, int64_t ldy);
bool prefill_y_fits(int64_t M, int64_t ldy);
hipError_t launch_w8a8_gemm(const W8A8Args &a, hipStream_t s);
// The 256 x 256-tile prefill kernel (y, or the group partials when a.P is set) and the
// split-K pieces its plan needs.
hipError_t launch_prefill(const W8A8Args &a, hipStream_t s);
size_t prefill_gemm_workspace(int M, int N, int K);

// A validated W8A8 call: what it needs and which kernel family it takes.
struct W8A8Plan {
    bool have_x;         // bf16 x given (quantised first), else qa / a_scale
    bool decode;         // decode kernel (otherwise prefill or tiled)
    size_t quant_bytes;  // quantised activations and row scales (256-byte aligned pieces)
    size_t gemm_bytes;   // split-K pieces the GEMM kernel's plan uses (0 if none)
    int64_t M, N, K;
    int kernel, workgroups;
};
// Argument checks of gemm_w8a8_g128_ex (pure host logic, no HIP call); fills plan.
int w8a8_validate(const void *x, int64_t ldx, const int8_t *qa, const float *a_scale, const int32_t *qweight,
                  const float *w_scale, const void *y, int64_t ldy, int64_t M, int64_t N, int64_t K, int kernel,
                  int decode_workgroups, W8A8Plan *plan);
// Launches the quantisation (when x is given, into `quant`) and the GEMM.  counters:
// kCounterBytes of split-K arrival counters, zero on entry (and on return); gemm_ws:
// room for the split pieces (the prefill kernel runs whole tiles if it is too small).
int w8a8_launch(const W8A8Plan &p, const void *x, int64_t ldx, const int8_t *qa, const float *a_scale,
                const int32_t *qweight, const float *w_scale, void *y, int64_t ldy, char *counters, char *quant,
                char *gemm_ws, size_t gemm_ws_bytes, hipStream_t s);

#define I8GS_TRY(expr)                    \
    do {                                  \
        int _rc = (expr);                 \
        if (_rc != I8GS_OK) return _rc;   \
    } while (0)

struct W4A16Args {
    const uint16_t *x;
    int64_t ldx;
    const int32_t *qweight;
    const float *w_scale;
    uint16_t *y;
    int64_t ldy;
    int M, N, K;
    int *counters;
    void *ws;
    size_t ws_bytes;
    int bits = 4;     // 4 (group 128) or 8 (group 128 or 32)
    int group = 128;
};
size_t w4a16_gemm_workspace(int M, int N, int K);

// Weight-only GEMM (bits 4 or 8, group 32 or 128) by the register-streaming kernel.
struct WoArgs {
    const uint16_t *x;
    int64_t ldx;
    const int32_t *qweight;
    const float *w_scale;
    uint16_t *y;
    int64_t ldy;
    int M, N, K;
    int bits, group;
    int *counters;
    void *ws;
    size_t ws_bytes;
};
size_t wo_gemm_workspace(int M, int N, int K);
hipError_t launch_wo_gemm(const WoArgs &a, hipStream_t s);
// Compute units of the current device (cached per device; 256 if unknown).
int device_cu_count();
hipError_t launch_w4a16_gemm(const W4A16Args &a, hipStream_t s);

// Buffer resource word 3 (raw buffer, gfx9-family format) and cache-policy bits.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kCpolNT = 2;    // non-temporal: streamed data is not reused
constexpr int kCpolSC1 = 16;  // device-coherent (across the XCDs' L2 caches)

// LDS pointer for buffer_load ... lds copies.
#define I8GS_LDS(p) ((__attribute__((address_space(3))) void *)(p))

// Workgroup barrier without the fence of __syncthreads (which would also wait for
// every copy in flight); the compiler keeps memory accesses on their side of it.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// Wait until at most N of this wave's memory operations are outstanding (they
// complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round an fp32 value to bfloat16, nearest with ties to even.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0;  // NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Every GEMM workspace starts with this many bytes of split-K arrival counters.
// The region sits at the same offset whatever the shape, so a caller can reuse one
// zero-filled workspace across calls of different shapes: each call leaves the
// counters it used at zero.
constexpr size_t kCounterBytes = 64 * 1024;
constexpr int kMaxCounters = int(kCounterBytes / sizeof(int));

}  // namespace i8gs
