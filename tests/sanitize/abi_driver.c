/* Host sanitizer run of the C ABI's argument checks (test infrastructure): every entry
 * point with rejected arguments (each rejection is a host decision, made before any HIP
 * call) and with accepted ones (which then stop at the device check when no GPU is
 * present).  Built with AddressSanitizer and UndefinedBehaviorSanitizer on the host
 * code of the library; device code is not built.  Exit status 0 when every status is
 * as expected. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "i8gs.h"

/* from the HIP runtime (returns 0 on success) */
extern int hipGetDeviceCount(int *count);

static int failures = 0;
#define EXPECT_EQ(got, want)                                                               \
    do {                                                                                   \
        long long g_ = (long long)(got), w_ = (long long)(want);                           \
        if (g_ != w_) {                                                                    \
            fprintf(stderr, "%s:%d: %s = %lld, expected %lld (%s)\n", __FILE__, __LINE__, #got, g_, w_, \
                    i8gs_last_error());                                                    \
            ++failures;                                                                    \
        }                                                                                  \
    } while (0)
/* accepted arguments: anything but a validation error.  Only without a GPU: with one,
 * an accepted call would launch kernels on these host addresses. */
static int have_gpu = 0;
#define EXPECT_VALID(got)                                                                  \
    do {                                                                                   \
        if (have_gpu) break;                                                               \
        int g_ = (got);                                                                    \
        if (g_ != I8GS_OK && g_ != I8GS_ERR_HIP && g_ != I8GS_ERR_UNSUPPORTED_DEVICE) {    \
            fprintf(stderr, "%s:%d: %s = %d (%s)\n", __FILE__, __LINE__, #got, g_, i8gs_last_error()); \
            ++failures;                                                                    \
        }                                                                                  \
        (void)i8gs_status_string(g_);                                                      \
    } while (0)

int main(void) {
    /* 16-byte aligned host memory standing for device buffers: never dereferenced, since
     * nothing reaches a kernel launch without a GPU */
    int ndev = 0;
    have_gpu = hipGetDeviceCount(&ndev) == 0 && ndev > 0;
    char *base = aligned_alloc(256, 1 << 20);
    void *A = base, *MIS = base + 4;
    const size_t BIG = (size_t)1 << 40;
    EXPECT_EQ(i8gs_abi_version(), I8GS_ABI_VERSION);
    for (int s = -1; s < 10; ++s) (void)i8gs_status_string(s);

    /* quantisation and the fused producer */
    EXPECT_EQ(quant_act_per_token(A, 512, 4, 500, A, A, NULL), I8GS_ERR_UNSUPPORTED_SHAPE);
    EXPECT_EQ(quant_act_per_token(MIS, 512, 4, 512, A, A, NULL), I8GS_ERR_MISALIGNED);
    EXPECT_EQ(quant_act_per_token(A, 500, 4, 512, A, A, NULL), I8GS_ERR_UNSUPPORTED_SHAPE);
    EXPECT_EQ(quant_act_per_token(A, 512, 0, 512, A, A, NULL), I8GS_OK);
    EXPECT_VALID(quant_act_per_token(A, 512, 4, 512, A, A, NULL));
    EXPECT_EQ(rmsnorm_quant_per_token(A, 512, A, 0.0f, 4, 512, NULL, A, A, NULL), I8GS_ERR_INVALID_ARG);
    EXPECT_EQ(rmsnorm_quant_per_token(A, 40000, A, 1e-6f, 4, 40000, NULL, A, A, NULL), I8GS_ERR_UNSUPPORTED_SHAPE);
    EXPECT_EQ(rmsnorm_quant_per_token(A, 512, A, 1e-6f, 4, 512, MIS, A, A, NULL), I8GS_ERR_MISALIGNED);
    EXPECT_VALID(rmsnorm_quant_per_token(A, 512, A, 1e-6f, 4, 512, A, A, A, NULL));

    /* workspace queries */
    EXPECT_EQ(i8gs_workspace_bytes(I8GS_OP_W8A8, 64, 6144, 100), (size_t)-1);
    EXPECT_EQ(i8gs_workspace_bytes(7, 64, 6144, 5120), (size_t)-1);
    EXPECT_EQ(i8gs_workspace_bytes_ex(I8GS_OP_W8A8, 64, 6144, 5120, 9, 0), (size_t)-1);
    EXPECT_EQ(i8gs_workspace_bytes(I8GS_OP_W8A8, 0, 6144, 5120), 0);
    size_t ws8 = i8gs_workspace_bytes(I8GS_OP_W8A8, 64, 6144, 5120);
    size_t ws4 = i8gs_workspace_bytes(I8GS_OP_W4A16, 64, 6144, 5120);
    size_t wsw = i8gs_workspace_bytes(I8GS_OP_WEIGHT_ONLY, 8, 248320, 5120);
    size_t wsp = i8gs_workspace_bytes(I8GS_OP_W8A8, 4096, 5120, 17408);
    if (ws8 == (size_t)-1 || ws4 == (size_t)-1 || wsw == (size_t)-1 || wsp == (size_t)-1) ++failures;

    /* W8A8 */
    EXPECT_EQ(gemm_w8a8_g128(A, 5120, NULL, NULL, A, A, A, 6144, 64, 6144, 5000, A, BIG, NULL),
              I8GS_ERR_UNSUPPORTED_SHAPE);
    EXPECT_EQ(gemm_w8a8_g128(A, 5120, A, A, A, A, A, 6144, 64, 6144, 5120, A, BIG, NULL), I8GS_ERR_INVALID_ARG);
    EXPECT_EQ(gemm_w8a8_g128(NULL, 0, NULL, NULL, A, A, A, 6144, 64, 6144, 5120, A, BIG, NULL), I8GS_ERR_INVALID_ARG);
    EXPECT_EQ(gemm_w8a8_g128(A, 5120, NULL, NULL, A, A, A, 6144, 64, 6144, 5120, NULL, 0, NULL), I8GS_ERR_WORKSPACE);
    EXPECT_EQ(gemm_w8a8_g128(A, 5120, NULL, NULL, A, A, MIS, 6144, 64, 6144, 5120, A, BIG, NULL), I8GS_ERR_MISALIGNED);
    EXPECT_EQ(gemm_w8a8_g128(A, 5120, NULL, NULL, A, A, A, 6000, 64, 6144, 5120, A, BIG, NULL),
              I8GS_ERR_UNSUPPORTED_SHAPE);
    EXPECT_EQ(gemm_w8a8_g128_ex(NULL, 0, A, A, A, A, A, 6144, 64, 6144, 5120, 5, 0, A, BIG, NULL),
              I8GS_ERR_INVALID_ARG);
    EXPECT_VALID(gemm_w8a8_g128(A, 5120, NULL, NULL, A, A, A, 6144, 64, 6144, 5120, A, BIG, NULL));
    EXPECT_VALID(gemm_w8a8_g128_ex(NULL, 0, A, A, A, A, A, 5120, 4096, 5120, 17408, I8GS_KERNEL_AUTO, 0, A, BIG,
                                   NULL));
    EXPECT_VALID(gemm_w8a8_g128_ex(NULL, 0, A, A, A, A, A, 5120, 64, 5120, 17408, I8GS_KERNEL_DECODE, 96, A, BIG,
                                   NULL));
    EXPECT_EQ(gemm_w8a8_g128_group_partials(A, A, MIS, 64, 256, 512, NULL), I8GS_ERR_MISALIGNED);
    EXPECT_VALID(gemm_w8a8_g128_group_partials(A, A, A, 64, 256, 512, NULL));
    EXPECT_VALID(gemm_w8a8_g128_group_partials_ex(A, A, A, 300, 256, 512, I8GS_KERNEL_TILED, 0, NULL));
    EXPECT_EQ(gemm_w8a8_g128_noalloc(A, 5120, A, A, A, A, A, 6144, 64, 6144, 5120, NULL), I8GS_ERR_INVALID_ARG);
    EXPECT_VALID(gemm_w8a8_g128_noalloc(A, 5120, NULL, NULL, A, A, A, 6144, 64, 6144, 5120, NULL));
    (void)i8gs_noalloc_scratch_bytes();

    /* weight-only */
    EXPECT_EQ(gemm_w4a16_g128(A, 5120, A, A, A, 6144, 64, 6144, 5120, NULL, 0, NULL), I8GS_ERR_WORKSPACE);
    EXPECT_EQ(gemm_weight_only(A, 5120, A, 5, A, 128, A, 6144, 8, 6144, 5120, A, BIG, NULL), I8GS_ERR_INVALID_ARG);
    EXPECT_EQ(gemm_weight_only(A, 5120, A, 8, A, 64, A, 6144, 8, 6144, 5120, A, BIG, NULL), I8GS_ERR_INVALID_ARG);
    EXPECT_EQ(gemm_weight_only(A, 5120, A, 8, A, 32, A, 6144, 8, 6144, 5100, A, BIG, NULL),
              I8GS_ERR_UNSUPPORTED_SHAPE);
    EXPECT_VALID(gemm_weight_only(A, 5120, A, 8, A, 32, A, 6144, 8, 6144, 5120, A, BIG, NULL));
    EXPECT_VALID(gemm_weight_only(A, 5120, A, 4, A, 128, A, 248320, 1, 248320, 5120, A, BIG, NULL));
    EXPECT_VALID(gemm_w4a16_g128(A, 5120, A, A, A, 6144, 64, 6144, 5120, A, BIG, NULL));

    /* GPTQ utilities */
    EXPECT_EQ(gptq_unpack(A, NULL, 8, 512, 256, NULL, NULL, NULL), I8GS_ERR_INVALID_ARG);
    EXPECT_EQ(gptq_unpack(A, NULL, 6, 512, 256, A, NULL, NULL), I8GS_ERR_INVALID_ARG);
    EXPECT_VALID(gptq_unpack(A, A, 4, 512, 256, A, A, NULL));
    EXPECT_EQ(gptq_quantize_rtn(A, 8, 500, 256, A, A, NULL), I8GS_ERR_UNSUPPORTED_SHAPE);
    EXPECT_VALID(gptq_quantize_rtn(A, 4, 512, 256, A, A, NULL));
    EXPECT_EQ(gptq_quantize_rtn_group(A, 8, 48, 512, 256, A, A, NULL), I8GS_ERR_INVALID_ARG);
    EXPECT_VALID(gptq_quantize_rtn_group(A, 8, 32, 512, 256, A, A, NULL));

    /* KV codec and attention products */
    EXPECT_EQ(kv_quant_int8_block128(A, 100, 4, 1, A, A, NULL), I8GS_ERR_UNSUPPORTED_SHAPE);
    EXPECT_EQ(kv_quant_int8_block128(A, 256, 4, 2, MIS, A, NULL), I8GS_ERR_MISALIGNED);
    EXPECT_VALID(kv_quant_int8_block128(A, 6144, 257, 8, A, A, NULL));
    EXPECT_EQ(attn_qk_int8(A, A, A, A, 0.088f, 4, 16, 6, 4, A, NULL, NULL), I8GS_ERR_UNSUPPORTED_SHAPE);
    EXPECT_EQ(attn_qk_int8(A, A, A, A, 0.088f, 1048560, 1, 64, 1, A, NULL, NULL), I8GS_ERR_UNSUPPORTED_SHAPE);
    EXPECT_VALID(attn_qk_int8(A, A, A, A, 0.088f, 8, 2048, 32, 8, A, A, NULL));
    size_t pvw = attn_pv_int8_workspace_bytes(8, 32768, 32, 8);
    if (pvw == 0 || pvw == (size_t)-1) ++failures;
    EXPECT_EQ(attn_pv_int8_workspace_bytes(8, 100, 6, 4), (size_t)-1);
    EXPECT_EQ(attn_pv_int8(A, A, A, 8, 32768, 32, 8, A, NULL, NULL, A, pvw - 1, NULL), I8GS_ERR_WORKSPACE);
    EXPECT_VALID(attn_pv_int8(A, A, A, 8, 32768, 32, 8, A, A, A, A, pvw, NULL));
    EXPECT_VALID(attn_pv_int8(NULL, NULL, NULL, 3, 0, 4, 1, A, NULL, NULL, NULL, 0, NULL));

    free(base);
    if (failures) {
        fprintf(stderr, "%d expectation(s) failed\n", failures);
        return 1;
    }
    printf("ABI sanitizer run: ok\n");
    return 0;
}
