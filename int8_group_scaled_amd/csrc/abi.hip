// C ABI entry points of libi8gs: argument validation, workspace sizing, dispatch.
// Validation is pure host logic and happens before any HIP call, so a rejected
// call launches nothing and writes nothing.
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

namespace i8gs {

static thread_local std::string g_last_error;

int fail(int status, const std::string &msg) {
    g_last_error = std::string(i8gs_status_string(status)) + ": " + msg;
    return status;
}

int ok() {
    g_last_error.clear();
    return I8GS_OK;
}

int hip_check(hipError_t e, const char *what) {
    if (e == hipSuccess) return I8GS_OK;
    return fail(I8GS_ERR_HIP, std::string(what) + " failed: " + hipGetErrorString(e));
}

int check_device() {
    static std::mutex mu;
    static std::vector<int> verdict;  // per device: 0 unknown, 1 ok, 2 bad
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_check(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(mu);
    if ((int)verdict.size() <= dev) verdict.resize(dev + 1, 0);
    if (verdict[dev] == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_check(e, "hipGetDeviceProperties");
        verdict[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        if (verdict[dev] == 2)
            return fail(I8GS_ERR_UNSUPPORTED_DEVICE,
                        std::string("device is ") + prop.gcnArchName + "; only gfx950 (MI355X) is supported");
    }
    if (verdict[dev] == 2) return fail(I8GS_ERR_UNSUPPORTED_DEVICE, "only gfx950 (MI355X) is supported");
    return I8GS_OK;
}

}  // namespace i8gs

using namespace i8gs;

namespace {

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

std::string fmt(const char *f, long long a, long long b = 0, long long c = 0, long long d = 0) {
    char buf[256];
    snprintf(buf, sizeof buf, f, a, b, c, d);
    return buf;
}

int check_dims(int64_t M, int64_t N, int64_t K, bool need_group) {
    if (M < 0 || N < 0 || K < 0)
        return fail(I8GS_ERR_UNSUPPORTED_SHAPE, fmt("sizes must be >= 0 (M=%lld N=%lld K=%lld)", M, N, K));
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return fail(I8GS_ERR_UNSUPPORTED_SHAPE, "sizes must be below 2^31");
    if (need_group && (K == 0 || K % kGroup != 0))
        return fail(I8GS_ERR_UNSUPPORTED_SHAPE,
                    fmt("K=%lld must be a positive multiple of the 128-wide weight group", K));
    if (N % 8 != 0) return fail(I8GS_ERR_UNSUPPORTED_SHAPE, fmt("N=%lld must be a multiple of 8", N));
    // one layer's 8-bit weights (K*N bytes) and activations (M*K) must stay below 4 GiB
    // (32-bit buffer offsets in the kernels)
    if (K * N >= (int64_t(1) << 32) || M * K >= (int64_t(1) << 32))
        return fail(I8GS_ERR_UNSUPPORTED_SHAPE, "K*N and M*K must be below 2^32");
    return I8GS_OK;
}

int check_ptr(const void *p, const char *name) {
    if (!p) return fail(I8GS_ERR_INVALID_ARG, std::string(name) + " is NULL");
    if (!aligned16(p)) return fail(I8GS_ERR_MISALIGNED, std::string(name) + " is not 16-byte aligned");
    return I8GS_OK;
}

int check_ld(int64_t ld, int64_t dim, const char *name) {
    if (ld < dim || ld % 8 != 0 || ld > kMaxDim)
        return fail(I8GS_ERR_UNSUPPORTED_SHAPE,
                    std::string(name) + fmt("=%lld must be >= %lld and a multiple of 8", ld, dim));
    return I8GS_OK;
}

size_t w8a8_quant_bytes(int64_t M, int64_t K) { return align256(size_t(M) * size_t(K)) + align256(size_t(M) * 4); }

// Which kernel a weight-only call takes: the register-streaming kernel for wide layers at
// few tokens (the vocabulary heads), where each workgroup streams long runs of K, and the
// LDS-staged kernel otherwise (measured faster on the decode layer shapes at 8 and 64
// rows, for 4-bit and 8-bit codes).
bool wo_uses_lds(int bits, int64_t M, int64_t N) {
    (void)bits;
    return !(M <= 16 && N >= 65536);
}

size_t w4_or_wo_workspace(int bits, int64_t M, int64_t N, int64_t K) {
    if (wo_uses_lds(bits, M, N)) return w4a16_gemm_workspace((int)M, (int)N, (int)K);
    return wo_gemm_workspace((int)M, (int)N, (int)K);
}

}  // namespace


namespace i8gs {

int w8a8_validate(const void *x, int64_t ldx, const int8_t *qa, const float *a_scale, const int32_t *qweight,
                  const float *w_scale, const void *y, int64_t ldy, int64_t M, int64_t N, int64_t K, int kernel,
                  int decode_workgroups, W8A8Plan *plan) {
    I8GS_TRY(check_dims(M, N, K, true));
    if (kernel < I8GS_KERNEL_AUTO || kernel > I8GS_KERNEL_TILED)
        return fail(I8GS_ERR_INVALID_ARG, fmt("kernel=%lld is not one of I8GS_KERNEL_*", kernel));
    if (decode_workgroups < 0)
        return fail(I8GS_ERR_INVALID_ARG, fmt("decode_workgroups=%lld must be >= 0", decode_workgroups));
    if (kernel == I8GS_KERNEL_DECODE && M > 64)
        return fail(I8GS_ERR_UNSUPPORTED_SHAPE, fmt("the decode kernel takes M <= 64 (M=%lld)", M));
    const bool have_x = x != nullptr;
    const bool have_q = qa != nullptr || a_scale != nullptr;
    if (have_x == have_q)
        return fail(I8GS_ERR_INVALID_ARG,
                    "pass either x (bf16 activations) or the pre-quantised pair qa/a_scale, not both or neither");
    plan->have_x = have_x;
    plan->M = M;
    plan->N = N;
    plan->K = K;
    plan->kernel = kernel;
    plan->workgroups = decode_workgroups;
    plan->quant_bytes = w8a8_quant_bytes(M, K);
    plan->gemm_bytes = 0;
    plan->decode = false;
    if (M == 0 || N == 0) return I8GS_OK;
    if (have_x) {
        I8GS_TRY(check_ptr(x, "x"));
        I8GS_TRY(check_ld(ldx, K, "ldx"));
    } else {
        I8GS_TRY(check_ptr(qa, "qa"));
        I8GS_TRY(check_ptr(a_scale, "a_scale"));
    }
    I8GS_TRY(check_ptr(qweight, "qweight"));
    I8GS_TRY(check_ptr(w_scale, "w_scale"));
    I8GS_TRY(check_ptr(y, "y"));
    I8GS_TRY(check_ld(ldy, N, "ldy"));
    if (kernel == I8GS_KERNEL_DECODE && !decode_y_fits(M, ldy))
        return fail(I8GS_ERR_UNSUPPORTED_SHAPE,
                    fmt("the decode kernel needs R*ldy*2 < 2^31 bytes of y, R = M rounded up to 32 (M=%lld ldy=%lld)",
                        M, ldy));
    plan->gemm_bytes = w8a8_gemm_workspace((int)M, (int)N, (int)K, kernel, decode_workgroups);
    plan->decode = kernel != I8GS_KERNEL_TILED && M <= 64 && decode_y_fits(M, ldy);
    return I8GS_OK;
}

int w8a8_launch(const W8A8Plan &p, const void *x, int64_t ldx, const int8_t *qa, const float *a_scale,
                const int32_t *qweight, const float *w_scale, void *y, int64_t ldy, char *counters, char *quant,
                char *gemm_ws, size_t gemm_ws_bytes, hipStream_t s) {
    if (p.have_x) {
        int8_t *qa_ws = (int8_t *)quant;
        float *as_ws = (float *)(quant + align256(size_t(p.M) * size_t(p.K)));
        I8GS_TRY(hip_check(launch_quant_act((const uint16_t *)x, ldx, (int)p.M, (int)p.K, qa_ws, as_ws, s),
                           "quant_act_per_token launch"));
        qa = qa_ws;
        a_scale = as_ws;
    }
    const bool pieces = gemm_ws != nullptr && gemm_ws_bytes > 0;
    W8A8Args a{qa, a_scale, qweight, w_scale, (uint16_t *)y, ldy, nullptr, (int)p.M, (int)p.N, (int)p.K, p.kernel,
               p.workgroups, pieces ? (int *)counters : nullptr, pieces ? (void *)gemm_ws : nullptr,
               pieces ? gemm_ws_bytes : 0};
    I8GS_TRY(hip_check(launch_w8a8_gemm(a, s), "gemm_w8a8_g128 launch"));
    return ok();
}

}  // namespace i8gs

extern "C" {

int i8gs_abi_version(void) { return I8GS_ABI_VERSION; }

const char *i8gs_last_error(void) { return g_last_error.c_str(); }

const char *i8gs_status_string(int status) {
    switch (status) {
        case I8GS_OK: return "I8GS_OK";
        case I8GS_ERR_INVALID_ARG: return "I8GS_ERR_INVALID_ARG";
        case I8GS_ERR_UNSUPPORTED_SHAPE: return "I8GS_ERR_UNSUPPORTED_SHAPE";
        case I8GS_ERR_MISALIGNED: return "I8GS_ERR_MISALIGNED";
        case I8GS_ERR_WORKSPACE: return "I8GS_ERR_WORKSPACE";
        case I8GS_ERR_HIP: return "I8GS_ERR_HIP";
        case I8GS_ERR_UNSUPPORTED_DEVICE: return "I8GS_ERR_UNSUPPORTED_DEVICE";
        default: return "I8GS_ERR_UNKNOWN";
    }
}

int quant_act_per_token(const void *x, int64_t ldx, int64_t M, int64_t K, int8_t *qa,
                        float *a_scale, void *stream) {
    if (M < 0 || K < 0 || M > kMaxDim || K > kMaxDim)
        return fail(I8GS_ERR_UNSUPPORTED_SHAPE, fmt("sizes must be in [0, 2^31) (M=%lld K=%lld)", M, K));
    if (K % 8 != 0) return fail(I8GS_ERR_UNSUPPORTED_SHAPE, fmt("K=%lld must be a multiple of 8", K));
    if (M == 0) return ok();
    if (K == 0) return fail(I8GS_ERR_UNSUPPORTED_SHAPE, "K must be positive when M > 0");
    I8GS_TRY(check_ptr(x, "x"));
    I8GS_TRY(check_ptr(qa, "qa"));
    I8GS_TRY(check_ptr(a_scale, "a_scale"));
    I8GS_TRY(check_ld(ldx, K, "ldx"));
    if (int64_t(M) * ldx > (int64_t(1) << 40)) return fail(I8GS_ERR_UNSUPPORTED_SHAPE, "x too large");
    I8GS_TRY(check_device());
    I8GS_TRY(hip_check(launch_quant_act((const uint16_t *)x, ldx, (int)M, (int)K, qa, a_scale,
                                        (hipStream_t)stream),
                       "quant_act_per_token launch"));
    return ok();
}

int rmsnorm_quant_per_token(const void *x, int64_t ldx, const void *gamma, float eps, int64_t M, int64_t K,
                            void *h, int8_t *qa, float *a_scale, void *stream) {
    if (M < 0 || K < 0 || M > kMaxDim || K > kMaxDim)
        return fail(I8GS_ERR_UNSUPPORTED_SHAPE, fmt("sizes must be in [0, 2^31) (M=%lld K=%lld)", M, K));
    if (K % 8 != 0) return fail(I8GS_ERR_UNSUPPORTED_SHAPE, fmt("K=%lld must be a multiple of 8", K));
    if (!(eps > 0.0f) || eps > 3.0e38f) return fail(I8GS_ERR_INVALID_ARG, "eps must be positive and finite");
    if (M == 0) return ok();
    if (K == 0) return fail(I8GS_ERR_UNSUPPORTED_SHAPE, "K must be positive when M > 0");
    if (K > rmsnorm_quant_max_k(M))
        return fail(I8GS_ERR_UNSUPPORTED_SHAPE,
                    fmt("K=%lld exceeds the %lld values a workgroup holds in registers", K, rmsnorm_quant_max_k(M)));
    I8GS_TRY(check_ptr(x, "x"));
    I8GS_TRY(check_ptr(gamma, "gamma"));
    I8GS_TRY(check_ptr(qa, "qa"));
    I8GS_TRY(check_ptr(a_scale, "a_scale"));
    if (h) I8GS_TRY(check_ptr(h, "h"));
    I8GS_TRY(check_ld(ldx, K, "ldx"));
    if (int64_t(M) * ldx > (int64_t(1) << 40)) return fail(I8GS_ERR_UNSUPPORTED_SHAPE, "x too large");
    I8GS_TRY(check_device());
    I8GS_TRY(hip_check(launch_rmsnorm_quant((const uint16_t *)x, ldx, (const uint16_t *)gamma, (double)eps, (int)M,
                                            (int)K, (uint16_t *)h, qa, a_scale, (hipStream_t)stream),
                       "rmsnorm_quant_per_token launch"));
    return ok();
}

size_t i8gs_workspace_bytes_ex(int op, int64_t M, int64_t N, int64_t K, int kernel, int decode_workgroups) {
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return (size_t)-1;
    if (op == I8GS_OP_W8A8) {
        if (kernel < I8GS_KERNEL_AUTO || kernel > I8GS_KERNEL_TILED || decode_workgroups < 0) return (size_t)-1;
        if (M == 0 || N == 0) return 0;
        if (K == 0 || K % kGroup != 0) return (size_t)-1;
        return kCounterBytes + w8a8_quant_bytes(M, K) +
               w8a8_gemm_workspace((int)M, (int)N, (int)K, kernel, decode_workgroups);
    }
    if (op == I8GS_OP_W4A16 || op == I8GS_OP_WEIGHT_ONLY) {
        if (M == 0 || N == 0) return 0;
        if (K == 0 || K % kGroup != 0) return (size_t)-1;
        // I8GS_OP_WEIGHT_ONLY: enough for either bit width
        const size_t part = op == I8GS_OP_W4A16 ? w4_or_wo_workspace(4, M, N, K)
                                                : std::max(w4_or_wo_workspace(4, M, N, K),
                                                           w4_or_wo_workspace(8, M, N, K));
        return part ? kCounterBytes + part : 0;
    }
    return (size_t)-1;
}

size_t i8gs_workspace_bytes(int op, int64_t M, int64_t N, int64_t K) {
    return i8gs_workspace_bytes_ex(op, M, N, K, I8GS_KERNEL_AUTO, 0);
}

int gemm_w8a8_g128_ex(const void *x, int64_t ldx, const int8_t *qa, const float *a_scale,
                      const int32_t *qweight, const float *w_scale, void *y, int64_t ldy, int64_t M,
                      int64_t N, int64_t K, int kernel, int decode_workgroups, void *workspace,
                      size_t workspace_bytes, void *stream) {
    W8A8Plan plan;
    I8GS_TRY(w8a8_validate(x, ldx, qa, a_scale, qweight, w_scale, y, ldy, M, N, K, kernel, decode_workgroups, &plan));
    if (M == 0 || N == 0) return ok();
    const size_t need = kCounterBytes + plan.quant_bytes + plan.gemm_bytes;
    if (plan.have_x || plan.gemm_bytes > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(I8GS_ERR_WORKSPACE, fmt("workspace of %lld bytes needed, %lld given", (long long)need,
                                                 workspace ? (long long)workspace_bytes : 0LL));
        if (!aligned16(workspace)) return fail(I8GS_ERR_MISALIGNED, "workspace is not 16-byte aligned");
    }
    I8GS_TRY(check_device());
    // Workspace layout: counters, the quantised activations (always counted), the split pieces.
    char *wsp = (char *)workspace;
    return w8a8_launch(plan, x, ldx, qa, a_scale, qweight, w_scale, y, ldy, wsp, wsp ? wsp + kCounterBytes : nullptr,
                       wsp ? wsp + kCounterBytes + plan.quant_bytes : nullptr, plan.gemm_bytes, (hipStream_t)stream);
}

int gemm_w8a8_g128(const void *x, int64_t ldx, const int8_t *qa, const float *a_scale,
                   const int32_t *qweight, const float *w_scale, void *y, int64_t ldy, int64_t M,
                   int64_t N, int64_t K, void *workspace, size_t workspace_bytes, void *stream) {
    return gemm_w8a8_g128_ex(x, ldx, qa, a_scale, qweight, w_scale, y, ldy, M, N, K, I8GS_KERNEL_AUTO, 0,
                             workspace, workspace_bytes, stream);
}

int gemm_w8a8_g128_group_partials_ex(const int8_t *qa, const int32_t *qweight, int32_t *P, int64_t M,
                                     int64_t N, int64_t K, int kernel, int decode_workgroups, void *stream) {
    I8GS_TRY(check_dims(M, N, K, true));
    if (kernel < I8GS_KERNEL_AUTO || kernel > I8GS_KERNEL_TILED)
        return fail(I8GS_ERR_INVALID_ARG, fmt("kernel=%lld is not one of I8GS_KERNEL_*", kernel));
    if (decode_workgroups < 0)
        return fail(I8GS_ERR_INVALID_ARG, fmt("decode_workgroups=%lld must be >= 0", decode_workgroups));
    if (kernel == I8GS_KERNEL_DECODE && M > 64)
        return fail(I8GS_ERR_UNSUPPORTED_SHAPE, fmt("the decode kernel takes M <= 64 (M=%lld)", M));
    if (M == 0 || N == 0) return ok();
    I8GS_TRY(check_ptr(qa, "qa"));
    I8GS_TRY(check_ptr(qweight, "qweight"));
    I8GS_TRY(check_ptr(P, "P"));
    I8GS_TRY(check_device());
    // The scale pointers are not read in this mode (their copies have an empty range); they
    // point at valid memory all the same.
    W8A8Args a{qa, (const float *)qa, qweight, (const float *)qweight, nullptr, 0, P, (int)M, (int)N, (int)K, kernel,
               decode_workgroups, nullptr, nullptr, 0};
    I8GS_TRY(hip_check(launch_w8a8_gemm(a, (hipStream_t)stream), "group partials launch"));
    return ok();
}

int gemm_w8a8_g128_group_partials(const int8_t *qa, const int32_t *qweight, int32_t *P,
                                  int64_t M, int64_t N, int64_t K, void *stream) {
    return gemm_w8a8_g128_group_partials_ex(qa, qweight, P, M, N, K, I8GS_KERNEL_AUTO, 0, stream);
}

int gemm_w4a16_g128(const void *x, int64_t ldx, const int32_t *qweight, const float *w_scale,
                    void *y, int64_t ldy, int64_t M, int64_t N, int64_t K, void *workspace,
                    size_t workspace_bytes, void *stream) {
    return gemm_weight_only(x, ldx, qweight, 4, w_scale, 128, y, ldy, M, N, K, workspace, workspace_bytes, stream);
}

int gptq_unpack(const int32_t *qweight, const float *w_scale, int bits, int64_t K, int64_t N,
                int8_t *q_out, float *w_out, void *stream) {
    if (bits != 4 && bits != 8) return fail(I8GS_ERR_INVALID_ARG, fmt("bits=%lld must be 4 or 8", bits));
    I8GS_TRY(check_dims(0, N, K, true));
    if (!q_out && !w_out) return fail(I8GS_ERR_INVALID_ARG, "give q_out, w_out or both");
    if (N == 0) return ok();
    I8GS_TRY(check_ptr(qweight, "qweight"));
    if (q_out) I8GS_TRY(check_ptr(q_out, "q_out"));
    if (w_out) {
        I8GS_TRY(check_ptr(w_out, "w_out"));
        I8GS_TRY(check_ptr(w_scale, "w_scale"));
    }
    I8GS_TRY(check_device());
    I8GS_TRY(hip_check(launch_gptq_unpack(qweight, w_scale, bits, (int)K, (int)N, q_out, w_out,
                                          (hipStream_t)stream),
                       "gptq_unpack launch"));
    return ok();
}

int gptq_quantize_rtn(const float *w, int bits, int64_t K, int64_t N, int32_t *qweight,
                      float *w_scale, void *stream) {
    if (bits != 4 && bits != 8) return fail(I8GS_ERR_INVALID_ARG, fmt("bits=%lld must be 4 or 8", bits));
    I8GS_TRY(check_dims(0, N, K, true));
    if (N == 0) return ok();
    I8GS_TRY(check_ptr(w, "w"));
    I8GS_TRY(check_ptr(qweight, "qweight"));
    I8GS_TRY(check_ptr(w_scale, "w_scale"));
    I8GS_TRY(check_device());
    I8GS_TRY(hip_check(launch_gptq_rtn(w, bits, kGroup, (int)K, (int)N, qweight, w_scale, (hipStream_t)stream),
                       "gptq_quantize_rtn launch"));
    return ok();
}

int gptq_quantize_rtn_group(const float *w, int bits, int group, int64_t K, int64_t N, int32_t *qweight,
                            float *w_scale, void *stream) {
    if (bits != 4 && bits != 8) return fail(I8GS_ERR_INVALID_ARG, fmt("bits=%lld must be 4 or 8", bits));
    if (group != 32 && group != 128) return fail(I8GS_ERR_INVALID_ARG, fmt("group=%lld must be 32 or 128", group));
    I8GS_TRY(check_dims(0, N, K, true));
    if (N == 0) return ok();
    I8GS_TRY(check_ptr(w, "w"));
    I8GS_TRY(check_ptr(qweight, "qweight"));
    I8GS_TRY(check_ptr(w_scale, "w_scale"));
    I8GS_TRY(check_device());
    I8GS_TRY(hip_check(launch_gptq_rtn(w, bits, group, (int)K, (int)N, qweight, w_scale, (hipStream_t)stream),
                       "gptq_quantize_rtn_group launch"));
    return ok();
}

int gemm_weight_only(const void *x, int64_t ldx, const int32_t *qweight, int bits, const float *w_scale, int group,
                     void *y, int64_t ldy, int64_t M, int64_t N, int64_t K, void *workspace,
                     size_t workspace_bytes, void *stream) {
    if (bits != 4 && bits != 8) return fail(I8GS_ERR_INVALID_ARG, fmt("bits=%lld must be 4 or 8", bits));
    if (!(group == 128 || (group == 32 && bits == 8)))
        return fail(I8GS_ERR_INVALID_ARG,
                    fmt("group=%lld with bits=%lld: supported are 4-bit group 128 and 8-bit group 32 or 128", group,
                        bits));
    I8GS_TRY(check_dims(M, N, K, true));
    if (M == 0 || N == 0) return ok();
    I8GS_TRY(check_ptr(x, "x"));
    I8GS_TRY(check_ld(ldx, K, "ldx"));
    I8GS_TRY(check_ptr(qweight, "qweight"));
    I8GS_TRY(check_ptr(w_scale, "w_scale"));
    I8GS_TRY(check_ptr(y, "y"));
    I8GS_TRY(check_ld(ldy, N, "ldy"));
    // a chunk of up to 64 activation rows is addressed with 32-bit byte offsets
    if (((std::min<int64_t>(M, 64) - 1) * ldx + K) * 2 >= (int64_t(1) << 31))
        return fail(I8GS_ERR_UNSUPPORTED_SHAPE,
                    fmt("the weight-only kernel needs (min(M,64)-1)*ldx*2 + K*2 < 2^31 bytes of x (M=%lld ldx=%lld)",
                        M, ldx));
    const size_t part = w4_or_wo_workspace(bits, M, N, K);
    const size_t need = part ? kCounterBytes + part : 0;
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(I8GS_ERR_WORKSPACE, fmt("workspace of %lld bytes needed, %lld given", (long long)need,
                                                 workspace ? (long long)workspace_bytes : 0LL));
        if (!aligned16(workspace)) return fail(I8GS_ERR_MISALIGNED, "workspace is not 16-byte aligned");
    }
    I8GS_TRY(check_device());
    char *wsp = (char *)workspace;
    if (wo_uses_lds(bits, M, N)) {
        // the decode layer shapes: the LDS-staged kernel (faster there)
        W4A16Args a{(const uint16_t *)x, ldx, qweight, w_scale, (uint16_t *)y, ldy, (int)M, (int)N, (int)K,
                    part ? (int *)wsp : nullptr, part ? (void *)(wsp + kCounterBytes) : nullptr, part, bits, group};
        I8GS_TRY(hip_check(launch_w4a16_gemm(a, (hipStream_t)stream), "gemm_weight_only launch"));
        return ok();
    }
    WoArgs a{(const uint16_t *)x, ldx, qweight, w_scale, (uint16_t *)y, ldy, (int)M, (int)N, (int)K, bits, group,
             part ? (int *)wsp : nullptr, part ? (void *)(wsp + kCounterBytes) : nullptr, part};
    I8GS_TRY(hip_check(launch_wo_gemm(a, (hipStream_t)stream), "gemm_weight_only launch"));
    return ok();
}

int kv_quant_int8_block128(const void *kv, int64_t ld, int64_t T, int64_t H, int8_t *codes, float *scales,
                           void *stream) {
    if (T < 0 || H < 0 || T > kMaxDim || H > kMaxDim || ld < 0)
        return fail(I8GS_ERR_UNSUPPORTED_SHAPE, fmt("sizes must be in [0, 2^31) (T=%lld H=%lld)", T, H));
    if (T == 0 || H == 0) return ok();
    if (T * H > kMaxDim) return fail(I8GS_ERR_UNSUPPORTED_SHAPE, "T*H must be below 2^31");
    I8GS_TRY(check_ptr(kv, "kv"));
    I8GS_TRY(check_ptr(codes, "codes"));
    I8GS_TRY(check_ptr(scales, "scales"));
    I8GS_TRY(check_ld(ld, 128 * H, "ld"));
    if (T * ld > (int64_t(1) << 40)) return fail(I8GS_ERR_UNSUPPORTED_SHAPE, "kv too large");
    I8GS_TRY(check_device());
    I8GS_TRY(hip_check(launch_kv_quant((const uint16_t *)kv, T, (int)H, ld, codes, scales, (hipStream_t)stream),
                       "kv_quant_int8_block128 launch"));
    return ok();
}

namespace {
// Shared checks of the attention products: sizes, heads, grid limits.
int check_attn(int64_t Mq, int64_t T, int64_t Hq, int64_t Hkv) {
    if (Mq < 0 || T < 0 || Hq < 0 || Hkv < 0 || Mq > kMaxDim || T > kMaxDim || Hq > kMaxDim || Hkv > kMaxDim)
        return fail(I8GS_ERR_UNSUPPORTED_SHAPE,
                    fmt("sizes must be in [0, 2^31) (Mq=%lld T=%lld Hq=%lld Hkv=%lld)", Mq, T, Hq, Hkv));
    if (Hkv == 0 || Hq % Hkv != 0)
        return fail(I8GS_ERR_UNSUPPORTED_SHAPE, fmt("Hq=%lld must be a multiple of Hkv=%lld > 0", Hq, Hkv));
    if (Hq > 65535) return fail(I8GS_ERR_UNSUPPORTED_SHAPE, "Hq must be at most 65535");
    // rows of one KV head group, (Hq/Hkv) * Mq: 32 per workgroup of the PV kernel's grid
    if (Hkv > 0 && Hq / Hkv * Mq > 32 * 65535)
        return fail(I8GS_ERR_UNSUPPORTED_SHAPE, "(Hq/Hkv)*Mq must be at most 2097120");
    if (Hq * Mq * T > (int64_t(1) << 40)) return fail(I8GS_ERR_UNSUPPORTED_SHAPE, "Hq*Mq*T too large");
    return I8GS_OK;
}
}  // namespace

int attn_qk_int8(const int8_t *qq, const float *qs, const int8_t *kq, const float *ks, float scale, int64_t Mq,
                 int64_t T, int64_t Hq, int64_t Hkv, float *s, int32_t *dots, void *stream) {
    I8GS_TRY(check_attn(Mq, T, Hq, Hkv));
    if (!std::isfinite(scale)) return fail(I8GS_ERR_INVALID_ARG, "scale must be finite");
    if (Mq == 0 || T == 0 || Hq == 0) return ok();
    I8GS_TRY(check_ptr(qq, "qq"));
    I8GS_TRY(check_ptr(qs, "qs"));
    I8GS_TRY(check_ptr(kq, "kq"));
    I8GS_TRY(check_ptr(ks, "ks"));
    I8GS_TRY(check_ptr(s, "s"));
    if (dots) I8GS_TRY(check_ptr(dots, "dots"));
    I8GS_TRY(check_device());
    I8GS_TRY(hip_check(launch_attn_qk(qq, qs, kq, ks, scale, (int)Mq, (int)T, (int)Hq, (int)Hkv, s, dots,
                                      (hipStream_t)stream),
                       "attn_qk_int8 launch"));
    return ok();
}

size_t attn_pv_int8_workspace_bytes(int64_t Mq, int64_t T, int64_t Hq, int64_t Hkv) {
    if (Mq < 0 || T < 0 || Hq < 0 || Hkv <= 0 || Mq > kMaxDim || T > kMaxDim || Hq > kMaxDim || Hq % Hkv != 0)
        return (size_t)-1;
    if (Mq == 0 || Hq == 0) return 0;
    const PvPlan pl = attn_pv_plan(Mq, T, Hq, Hkv);
    return pl.part_bytes ? kCounterBytes + pl.part_bytes : 0;
}

int attn_pv_int8(const float *p, const int8_t *vq, const float *vs, int64_t Mq, int64_t T, int64_t Hq, int64_t Hkv,
                 float *out, int8_t *pq, float *ps, void *workspace, size_t workspace_bytes, void *stream) {
    I8GS_TRY(check_attn(Mq, T, Hq, Hkv));
    if (Mq == 0 || Hq == 0) return ok();
    if (T > 0) {
        I8GS_TRY(check_ptr(p, "p"));
        I8GS_TRY(check_ptr(vq, "vq"));
        I8GS_TRY(check_ptr(vs, "vs"));
    }
    I8GS_TRY(check_ptr(out, "out"));
    if (pq) I8GS_TRY(check_ptr(pq, "pq"));
    if (ps) I8GS_TRY(check_ptr(ps, "ps"));
    const PvPlan pl = attn_pv_plan(Mq, T, Hq, Hkv);
    // the common workspace layout: the (here unused) counter region first, left as it is
    const size_t need = pl.part_bytes ? kCounterBytes + pl.part_bytes : 0;
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(I8GS_ERR_WORKSPACE, fmt("workspace of %lld bytes needed, %lld given", (long long)need,
                                                 workspace ? (long long)workspace_bytes : 0LL));
        if (!aligned16(workspace)) return fail(I8GS_ERR_MISALIGNED, "workspace is not 16-byte aligned");
    }
    I8GS_TRY(check_device());
    I8GS_TRY(hip_check(launch_attn_pv(p, vq, vs, (int)Mq, (int)T, (int)Hq, (int)Hkv, out, pq, ps,
                                      need ? (float *)((char *)workspace + kCounterBytes) : nullptr,
                                      (hipStream_t)stream),
                       "attn_pv_int8 launch"));
    return ok();
}

}  // extern "C"
