/* Host sanitizer run of the oracle (test infrastructure): every oracle entry point on
 * small and edge-case inputs, each buffer malloc'ed at exactly the size the function's
 * contract names, so AddressSanitizer reports any access outside it and
 * UndefinedBehaviorSanitizer any overflow, bad shift or misaligned access.  Exit
 * status 0 when every call returns its expected status and the few invariants hold. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_quant_act_per_token(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int8_t *qa, float *a_scale);
int oracle_gptq_unpack(const int32_t *qweight, int bits, int64_t K, int64_t N, int8_t *q_out);
int oracle_gptq_dequant(const int32_t *qweight, const float *w_scale, int bits, int64_t K, int64_t N, float *w_out);
int oracle_gptq_quantize_rtn(const float *w, int bits, int64_t K, int64_t N, int32_t *qweight, float *w_scale);
int oracle_group_partials(const int8_t *qa, const int8_t *q, int64_t M, int64_t N, int64_t K, int32_t *P);
int oracle_gemm_w8a8_g128(const int8_t *qa, const float *a_scale, const int8_t *q, const float *w_scale, int64_t M,
                          int64_t N, int64_t K, const int64_t *rows, int64_t nrows, double *y, double *T);
int oracle_gemm_w4a16_g128(const uint16_t *x, int64_t ldx, const int8_t *q, const float *w_scale, int64_t M, int64_t N,
                           int64_t K, const int64_t *rows, int64_t nrows, double *y, double *T);
void oracle_bf16_from_double_array(const double *v, int64_t n, uint16_t *out);
int oracle_gemm_weight_only(const uint16_t *x, int64_t ldx, const int8_t *q, const float *w_scale, int64_t group,
                            int64_t M, int64_t N, int64_t K, const int64_t *rows, int64_t nrows, double *y, double *T);
int oracle_gptq_quantize_rtn_group(const float *w, int bits, int64_t group, int64_t K, int64_t N, int32_t *qweight,
                                   float *w_scale);
int oracle_rmsnorm_bf16(const uint16_t *x, int64_t ldx, const uint16_t *gamma, double eps, int64_t M, int64_t K,
                        uint16_t *h);
int oracle_attn_qk_int8(const int8_t *qq, const float *qs, const int8_t *kq, const float *ks, double scale, int64_t Mq,
                        int64_t T, int64_t Hq, int64_t Hkv, double *s, int32_t *dots);
int oracle_attn_pv_int8(const float *p, const int8_t *vq, const float *vs, int64_t Mq, int64_t T, int64_t Hq,
                        int64_t Hkv, double *out, double *mag, int8_t *pq_out, float *ps_out);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (uint32_t)(state >> 16);
}
static float next_normal(void) { /* sum of uniforms: enough for test data */
    float s = 0.0f;
    for (int i = 0; i < 4; ++i) s += (float)(next_u32() & 0xFFFF) / 65536.0f;
    return (s - 2.0f) * 1.7f;
}
static uint16_t bf16_of(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) exit(3);
    return p;
}

static int failures = 0;
#define EXPECT(cond)                                                    \
    do {                                                                \
        if (!(cond)) {                                                  \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                 \
        }                                                               \
    } while (0)

static void linear_cases(int64_t M, int64_t K, int64_t N, int64_t ldx) {
    uint16_t *x = xmalloc(sizeof(uint16_t) * (size_t)(M * ldx));
    for (int64_t i = 0; i < M * ldx; ++i) x[i] = bf16_of(next_normal() * ((i % 37) == 0 ? 20.0f : 1.0f));
    if (M > 1) memset(x + ldx, 0, sizeof(uint16_t) * (size_t)ldx); /* an all-zero row */
    int8_t *qa = xmalloc((size_t)(M * K));
    float *as = xmalloc(sizeof(float) * (size_t)M);
    EXPECT(oracle_quant_act_per_token(x, M, K, ldx, qa, as) == 0);
    for (int64_t i = 0; i < M * K; ++i) EXPECT(qa[i] >= -127 && qa[i] <= 127);
    float *w = xmalloc(sizeof(float) * (size_t)(K * N));
    for (int64_t i = 0; i < K * N; ++i) w[i] = next_normal() * 0.02f;
    for (int bits = 4; bits <= 8; bits += 4) {
        const int64_t per = 32 / bits;
        int32_t *qw = xmalloc(sizeof(int32_t) * (size_t)(K / per * N));
        float *ws = xmalloc(sizeof(float) * (size_t)(K / 128 * N));
        EXPECT(oracle_gptq_quantize_rtn(w, bits, K, N, qw, ws) == 0);
        int8_t *q = xmalloc((size_t)(K * N));
        EXPECT(oracle_gptq_unpack(qw, bits, K, N, q) == 0);
        float *wd = xmalloc(sizeof(float) * (size_t)(K * N));
        EXPECT(oracle_gptq_dequant(qw, ws, bits, K, N, wd) == 0);
        int64_t rows[2] = {0, M - 1};
        /* [nrows, N]: M rows, or the 2 sampled rows */
        const int64_t R = M > 2 ? M : 2;
        double *y = xmalloc(sizeof(double) * (size_t)(R * N));
        double *T = xmalloc(sizeof(double) * (size_t)(R * N));
        if (bits == 8) {
            int32_t *P = xmalloc(sizeof(int32_t) * (size_t)(M * (K / 128) * N));
            EXPECT(oracle_group_partials(qa, q, M, N, K, P) == 0);
            free(P);
            EXPECT(oracle_gemm_w8a8_g128(qa, as, q, ws, M, N, K, NULL, 0, y, T) == 0);
            EXPECT(oracle_gemm_w8a8_g128(qa, as, q, ws, M, N, K, rows, 2, y, T) == 0);
        } else {
            EXPECT(oracle_gemm_w4a16_g128(x, ldx, q, ws, M, N, K, NULL, 0, y, T) == 0);
            EXPECT(oracle_gemm_w4a16_g128(x, ldx, q, ws, M, N, K, rows, 2, y, T) == 0);
        }
        uint16_t *yb = xmalloc(sizeof(uint16_t) * (size_t)(M * N));
        oracle_bf16_from_double_array(y, M * N, yb);
        for (int64_t i = 0; i < M * N; ++i) EXPECT(T[i] >= fabs(y[i]) * (1.0 - 1e-12));
        for (int64_t group = 32; group <= 128; group += 96) {
            int32_t *qg = xmalloc(sizeof(int32_t) * (size_t)(K / per * N));
            float *sg = xmalloc(sizeof(float) * (size_t)(K / group * N));
            EXPECT(oracle_gptq_quantize_rtn_group(w, bits, group, K, N, qg, sg) == 0);
            int8_t *qu = xmalloc((size_t)(K * N));
            EXPECT(oracle_gptq_unpack(qg, bits, K, N, qu) == 0);
            EXPECT(oracle_gemm_weight_only(x, ldx, qu, sg, group, M, N, K, NULL, 0, y, T) == 0);
            EXPECT(oracle_gemm_weight_only(x, ldx, qu, sg, group, M, N, K, rows, 2, y, T) == 0);
            free(qg);
            free(sg);
            free(qu);
        }
        EXPECT(oracle_gemm_weight_only(x, ldx, q, ws, 0, M, N, K, NULL, 0, y, T) != 0); /* bad group */
        free(qw);
        free(ws);
        free(q);
        free(wd);
        free(y);
        free(T);
        free(yb);
    }
    uint16_t *gamma = xmalloc(sizeof(uint16_t) * (size_t)K);
    for (int64_t i = 0; i < K; ++i) gamma[i] = bf16_of(1.0f + 0.25f * next_normal());
    uint16_t *h = xmalloc(sizeof(uint16_t) * (size_t)(M * K));
    EXPECT(oracle_rmsnorm_bf16(x, ldx, gamma, 1e-6, M, K, h) == 0);
    EXPECT(oracle_rmsnorm_bf16(x, ldx, gamma, 0.0, M, K, h) != 0); /* eps must be positive */
    free(gamma);
    free(h);
    free(x);
    free(qa);
    free(as);
    free(w);
}

static void attention_case(int64_t Mq, int64_t T, int64_t Hq, int64_t Hkv) {
    const int64_t B = (T + 127) / 128;
    int8_t *qq = xmalloc((size_t)(Mq * Hq * 128));
    float *qs = xmalloc(sizeof(float) * (size_t)(Mq * Hq));
    int8_t *kv = xmalloc((size_t)(T * Hkv * 128));
    float *ks = xmalloc(sizeof(float) * (size_t)(T * Hkv));
    for (int64_t i = 0; i < Mq * Hq * 128; ++i) qq[i] = (int8_t)((int)(next_u32() % 255) - 127);
    for (int64_t i = 0; i < Mq * Hq; ++i) qs[i] = 0.01f + 0.001f * (float)(i % 7);
    for (int64_t i = 0; i < T * Hkv * 128; ++i) kv[i] = (int8_t)((int)(next_u32() % 255) - 127);
    for (int64_t i = 0; i < T * Hkv; ++i) ks[i] = 0.02f + 0.001f * (float)(i % 5);
    double *s = xmalloc(sizeof(double) * (size_t)(Hq * Mq * T));
    int32_t *dots = xmalloc(sizeof(int32_t) * (size_t)(Hq * Mq * T));
    EXPECT(oracle_attn_qk_int8(qq, qs, kv, ks, 0.088, Mq, T, Hq, Hkv, s, dots) == 0);
    EXPECT(oracle_attn_qk_int8(qq, qs, kv, ks, 0.088, Mq, T, Hq, Hkv, s, NULL) == 0);
    float *p = xmalloc(sizeof(float) * (size_t)(Hq * Mq * T));
    for (int64_t r = 0; r < Hq * Mq; ++r) {
        double sum = 0.0;
        for (int64_t t = 0; t < T; ++t) sum += exp(s[r * T + t] - 1.0);
        for (int64_t t = 0; t < T; ++t) p[r * T + t] = (float)(exp(s[r * T + t] - 1.0) / sum);
    }
    if (Hq * Mq > 0 && T > 0) memset(p, 0, sizeof(float) * (size_t)T); /* a zero row: every block scale 0 */
    double *out = xmalloc(sizeof(double) * (size_t)(Hq * Mq * 128));
    double *mag = xmalloc(sizeof(double) * (size_t)(Hq * Mq * 128));
    int8_t *pq = xmalloc((size_t)(Hq * Mq * T));
    float *ps = xmalloc(sizeof(float) * (size_t)(Hq * Mq * B));
    EXPECT(oracle_attn_pv_int8(p, kv, ks, Mq, T, Hq, Hkv, out, mag, pq, ps) == 0);
    EXPECT(oracle_attn_pv_int8(p, kv, ks, Mq, T, Hq, Hkv, out, mag, NULL, NULL) == 0);
    for (int64_t i = 0; i < Hq * Mq * 128; ++i) EXPECT(fabs(out[i]) <= mag[i] * (1.0 + 1e-12));
    EXPECT(oracle_attn_qk_int8(qq, qs, kv, ks, 0.088, Mq, T, 3, 2, s, dots) != 0);  /* Hq % Hkv != 0 */
    EXPECT(oracle_attn_pv_int8(p, kv, ks, Mq, T, 3, 2, out, mag, pq, ps) != 0);
    free(qq); free(qs); free(kv); free(ks); free(s); free(dots); free(p); free(out); free(mag); free(pq); free(ps);
}

int main(void) {
    linear_cases(1, 128, 8, 128);
    linear_cases(3, 256, 24, 264);
    linear_cases(5, 384, 40, 392);
    /* degenerate sizes the contract allows */
    EXPECT(oracle_quant_act_per_token(NULL, 0, 128, 128, NULL, NULL) == 0);
    EXPECT(oracle_group_partials(NULL, NULL, 0, 0, 100, NULL) != 0); /* K % 128 */
    attention_case(3, 77, 4, 1);
    attention_case(2, 300, 4, 2);
    attention_case(1, 1, 1, 1);
    attention_case(4, 0, 2, 2);
    if (failures) {
        fprintf(stderr, "%d expectation(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer run: ok\n");
    return 0;
}
