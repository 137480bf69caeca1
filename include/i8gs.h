/*
 * i8gs.h -- C ABI of the group-scaled INT8 linear layer for AMD MI355X (gfx950).
 *
 * The operation (sources are web pages, cited by title and section):
 *  - "Flint-DFlash2-GPTQ-INT8-PTQR" model card, format table: GPTQ checkpoint
 *    (qweight / qzeros / scales, no g_idx, desc_act false), INT8 weights served
 *    W8A8, group size 128, symmetric; format audit: every matrix uses contiguous
 *    groups of exactly 128 weights; serving notes: the W8A8 GEMM path quantises
 *    its bf16 inputs to INT8 on the fly (rounding mode "round").
 *  - "Qwen3.8-27B GPTQ INT8 W8A8 GS128 PTQR" model card, "Quantization details":
 *    true int8 x int8 compute at every decode and prefill shape, with one weight
 *    scale per 128-wide K block.
 *  - "Qwen3.8-27B-DFlash2-W4A16-g128-sym-GPTQ" model card, property table: the
 *    4-bit weight-only sibling (W4A16, group_size 128, symmetric); dequant-patch
 *    table: INT32-packed GPTQ is unpacked from int32 and scaled per group.
 *  - "Qwen3.5-4B-DFlash-W8A16" model card: RTN weight quantisation with no
 *    calibration data; recovering dense weight rows through the layer itself.
 *
 *  For an activation row x[m, 0..K) (bf16) and packed weights:
 *    a_scale[m] = max_k |x[m,k]| / 127                         (fp32, IEEE division)
 *    qa[m,k]    = clamp(round_half_even(x[m,k] / a_scale[m]), -127, 127)   (int8;
 *                 an all-zero row gives a_scale 0 and codes 0)
 *    q[k,n]     = code(k,n) - 2^(bits-1)      (GPTQ offset binary, bits = 8 or 4)
 *    P[m,g,n]   = sum_{k = 128g}^{128g+127} qa[m,k] * q[k,n]   (exact int32)
 *    y[m,n]     = bf16( a_scale[m] * sum_g w_scale[g,n] * P[m,g,n] )
 *  The group sums are exact; the fold over groups is fp32 in any order, so y is
 *  within one bf16 unit of the exact value plus (K/128 + 2) * 2^-24 times
 *  a_scale[m] * sum_g |w_scale[g,n] * P[m,g,n]|.  Scales are finite with
 *  |w_scale| < 2^100 (the decode kernel folds with w_scale * 2^26).
 *
 * Layouts (all row-major, little-endian):
 *  x        bf16   [M, ldx]        activations (ldx >= K, ldx % 8 == 0)
 *  qa       int8   [M, K]          quantised activations
 *  a_scale  fp32   [M]
 *  qweight  int32  [K / (32/bits), N]  code j of word [r, n] is k = (32/bits)*r + j,
 *                                  stored in bits [bits*j, bits*j + bits) of the word
 *  w_scale  fp32   [K/128, N]      one scale per 128-wide K group per column
 *  y        bf16   [M, ldy]        (ldy >= N, ldy % 8 == 0)
 *  qzeros is not taken: symmetric checkpoints store the constant mid-range code.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or retains memory and never synchronises the stream.
 *    Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) of the
 *    current HIP device.  Calls are reentrant.
 *  - Return value: I8GS_OK or an i8gs_status code.  Every argument is validated
 *    before anything is launched; on a validation error nothing is launched and
 *    nothing is written.  i8gs_last_error() then returns a message (thread-local)
 *    that names the violated rule.  Unsupported requests are rejected explicitly;
 *    there is no fallback path.
 *  - Shapes: K % 128 == 0 and K > 0 for the GEMMs; N % 8 == 0; M >= 0 (M == 0
 *    or N == 0 is a no-op that returns I8GS_OK).  Tensor pointers must be 16-byte
 *    aligned.  Dimensions must be below 2^31, and K*N and M*K below 2^32.  The
 *    W4A16 GEMM also needs (min(M, 64) - 1)*ldx*2 + K*2 < 2^31 (32-bit offsets
 *    within a chunk of activation rows).
 *  - The device must be gfx950 (I8GS_ERR_UNSUPPORTED_DEVICE otherwise).
 */
#ifndef I8GS_H
#define I8GS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define I8GS_ABI_VERSION 1

typedef enum {
    I8GS_OK = 0,
    I8GS_ERR_INVALID_ARG = 1,       /* null pointer, bad enum, x and qa both / neither given */
    I8GS_ERR_UNSUPPORTED_SHAPE = 2, /* K % 128, N % 8, negative or too large sizes, ld < dim */
    I8GS_ERR_MISALIGNED = 3,        /* a tensor pointer is not 16-byte aligned */
    I8GS_ERR_WORKSPACE = 4,         /* workspace missing or smaller than i8gs_workspace_bytes() */
    I8GS_ERR_HIP = 5,               /* a HIP runtime call or kernel launch failed */
    I8GS_ERR_UNSUPPORTED_DEVICE = 6 /* current device is not gfx950 */
} i8gs_status;

/* Operation ids for i8gs_workspace_bytes(). */
#define I8GS_OP_W8A8 0
#define I8GS_OP_W4A16 1
#define I8GS_OP_WEIGHT_ONLY 2 /* gemm_weight_only (enough for any bits / group) */

/* Kernel choice for gemm_w8a8_g128_ex(). */
#define I8GS_KERNEL_AUTO 0   /* decode kernel for M <= 64, the 256x256-tile prefill kernel
                                otherwise; the 128x128 tiled kernel when R*ldy*2 >= 2^31 with
                                R = M rounded up to 32 (M <= 64) or to 256 (M > 64) */
#define I8GS_KERNEL_DECODE 1 /* weight-streaming kernel (M <= 64 and R*ldy*2 < 2^31 only) */
#define I8GS_KERNEL_TILED 2  /* 128x128 LDS-tiled MFMA kernel, any M */

/* ABI version of the loaded library (I8GS_ABI_VERSION at build time). */
int i8gs_abi_version(void);

/* Message describing the last failed call on this thread ("" if none). */
const char *i8gs_last_error(void);

/* Name of a status code, e.g. "I8GS_ERR_UNSUPPORTED_SHAPE". */
const char *i8gs_status_string(int status);

/*
 * Dynamic per-token INT8 activation quantisation (Flint card serving notes;
 * Qwen3.8-27B W8A8 card serving section).  For each of the M rows of x:
 * a_scale[m] = absmax/127 in fp32 and qa[m,:] = clamp(rint(x / a_scale), -127, 127)
 * with a correctly rounded fp32 division and ties to even.
 *   x        device bf16 [M, ldx], K % 8 == 0, ldx >= K, ldx % 8 == 0
 *   qa       device int8 [M, K] (contiguous), output
 *   a_scale  device fp32 [M], output
 * Results are bit-exact (one correct value per element).
 */
int quant_act_per_token(const void *x, int64_t ldx, int64_t M, int64_t K, int8_t *qa,
                        float *a_scale, void *stream);

/*
 * RMS normalisation fused with the per-token INT8 quantisation of its output, the
 * producer of the quantised activations of the qkv and gate/up projections
 * (Qwen3.8-27B-DFlash2-W4A16 card, bf16-surface table: the norms ahead of the quantised
 * linears; qwen38/dflash2 recipe, numerics: FP32 normalisation keeping the intermediate
 * BF16 casts).  For each of the M rows of x:
 *   r = 1 / sqrt(sum_k x^2 / K + eps),  h[k] = bf16(gamma[k] * bf16(x[k] * r)),
 *   a_scale = max |h| / 127,  qa[k] = clamp(rint(h[k] / a_scale), -127, 127)
 * with each step correctly rounded in fp64 (the sum of squares exact), so h, qa and
 * a_scale are bit-exact (one correct value each).
 *   x      device bf16 [M, ldx], K % 8 == 0, ldx >= K, ldx % 8 == 0
 *   gamma  device bf16 [K]
 *   eps    > 0 (e.g. 1e-6)
 *   h      device bf16 [M, K] (contiguous) or NULL: the normalised rows, output
 *   qa     device int8 [M, K] (contiguous), output;  a_scale device fp32 [M], output
 * K is limited to 32768 (M <= 512) or 26624 (larger M): the row stays in registers.
 */
int rmsnorm_quant_per_token(const void *x, int64_t ldx, const void *gamma, float eps, int64_t M, int64_t K,
                            void *h, int8_t *qa, float *a_scale, void *stream);

/*
 * Bytes of workspace gemm_w8a8_g128 (op I8GS_OP_W8A8) or gemm_w4a16_g128
 * (I8GS_OP_W4A16) needs for these sizes.  Layout: a fixed 64 KiB region of
 * split-K arrival counters at offset 0, then (W8A8) the quantised activations used
 * when x is passed (M*K bytes + 4*M, each piece rounded up to 256 bytes; always
 * counted), then the split-K partial sums (decode kernel with K split: T*S fp32
 * pieces of 64 rows by the kernel's chunk width rounded up to 32 columns; prefill
 * kernel, M > 64: the 256 x 256 tiles of a last, partial round of workgroups, as S
 * fp32 pieces each).  Returns 0 when no workspace is needed (W4A16 without a K
 * split) and (size_t)-1 for invalid arguments.
 *
 * Workspace contract: the counter region must be zero when a call starts, and
 * every completed call leaves it zero again, whatever the shape.  Zero-fill a
 * newly allocated workspace once before its first use; after that it can be
 * reused by calls of any shape.  Do not share one workspace between calls that
 * may run concurrently (different streams without ordering).
 */
size_t i8gs_workspace_bytes(int op, int64_t M, int64_t N, int64_t K);

/* Same, for gemm_w8a8_g128_ex() with an explicit kernel / workgroup-count choice. */
size_t i8gs_workspace_bytes_ex(int op, int64_t M, int64_t N, int64_t K, int kernel, int decode_workgroups);

/*
 * W8A8 G128 linear (Qwen3.8-27B W8A8 card "Quantization details"; Flint card
 * format table and serving notes):  y = bf16(a_scale * sum_g w_scale[g] * P_g).
 * Pass EITHER x (bf16 [M, ldx]; it is quantised per token into the workspace
 * first) OR the pre-quantised pair qa (int8 [M, K]) and a_scale (fp32 [M]);
 * the others must be NULL.  qweight is int32 [K/4, N] with 8-bit codes q + 128;
 * w_scale fp32 [K/128, N]; y bf16 [M, ldy].  workspace: device memory of at
 * least i8gs_workspace_bytes(I8GS_OP_W8A8, M, N, K) bytes (may be NULL if that
 * is 0).  Output y is within the tolerance stated at the top of this file.
 */
int gemm_w8a8_g128(const void *x, int64_t ldx, const int8_t *qa, const float *a_scale,
                   const int32_t *qweight, const float *w_scale, void *y, int64_t ldy, int64_t M,
                   int64_t N, int64_t K, void *workspace, size_t workspace_bytes, void *stream);

/*
 * gemm_w8a8_g128 with the kernel chosen by the caller: kernel is one of
 * I8GS_KERNEL_*; decode_workgroups (decode kernel only) is the target number of
 * workgroups, 0 for the automatic choice (one per compute unit).  The decode
 * kernel splits the columns into T tiles of multiples of 8 columns and, for narrow
 * layers, K into S <= 8 parts of whole 128-wide groups (S = ceil(64 * target / N),
 * T = target / S, both clamped to the layer), so it runs T*S workgroups.  Every
 * choice computes the same exact group sums; only the fp32 fold order differs.
 * I8GS_KERNEL_DECODE is rejected when M > 64 or when R*ldy*2 >= 2^31 with R = M
 * rounded up to 32 (32-bit output offsets); I8GS_KERNEL_AUTO takes the 128x128
 * tiled kernel in that case.
 */
int gemm_w8a8_g128_ex(const void *x, int64_t ldx, const int8_t *qa, const float *a_scale,
                      const int32_t *qweight, const float *w_scale, void *y, int64_t ldy, int64_t M,
                      int64_t N, int64_t K, int kernel, int decode_workgroups, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * gemm_w8a8_g128 for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * kernels, launch plan and results as gemm_w8a8_g128 (bit-identical y), but no
 * workspace argument: the split-K counters, the quantised activations (when x is
 * given) and the split-K partial sums live in a static device array of
 * i8gs_noalloc_scratch_bytes() = 16 MiB that the library holds on every GPU it runs
 * on until the process ends.  The call allocates and frees nothing.
 * Limit: 64 KiB + (x given: M*K + 4*M, each rounded up to 256 bytes) + (M <= 64: the
 * decode kernel's split pieces) must fit in 16 MiB, else I8GS_ERR_WORKSPACE and
 * nothing is launched (every decode-sized call of the drafter layers fits; for large
 * M pass qa/a_scale, and the prefill kernel then runs whole tiles when its split
 * pieces do not fit).  The counters are cleared by the first call on each device
 * (on its stream) and every completed call leaves them zero.  All calls on one GPU
 * share its array: calls that may overlap on one GPU (different streams, threads or
 * graphs without ordering) race and must not be issued.
 */
int gemm_w8a8_g128_noalloc(const void *x, int64_t ldx, const int8_t *qa, const float *a_scale,
                           const int32_t *qweight, const float *w_scale, void *y, int64_t ldy, int64_t M,
                           int64_t N, int64_t K, void *stream);

/* Bytes of the static scratch array gemm_w8a8_g128_noalloc uses on each device. */
size_t i8gs_noalloc_scratch_bytes(void);

/*
 * The per-group int32 partials P[m, g, n] = sum_{k in group g} qa[m,k] * q[k,n]
 * of the W8A8 G128 GEMM (Qwen3.8-27B W8A8 card, "Quantization details": int8 x
 * int8 products summed per 128-wide K block), written to P (device int32
 * [M, K/128, N]) instead of being folded.  The call runs the kernel and the launch
 * plan that gemm_w8a8_g128 runs for the same M (the decode kernel for M <= 64 with
 * its column tiles and K splits, the 256 x 256 prefill kernel above, including
 * its K-split last round), in a mode that stores each MFMA chain's group sum --
 * for the decode kernel decoded from its seeded accumulator exactly as its fold
 * decodes it -- where that kernel would fold it.  It checks the integer stage
 * bit-exactly.  Needs no workspace.  Results are bit-exact.
 */
int gemm_w8a8_g128_group_partials(const int8_t *qa, const int32_t *qweight, int32_t *P,
                                  int64_t M, int64_t N, int64_t K, void *stream);

/* Same, with the kernel (I8GS_KERNEL_*) and decode workgroup target chosen as for
 * gemm_w8a8_g128_ex(); I8GS_KERNEL_TILED runs the 128 x 128 tiled kernel.  Every
 * choice writes the same P. */
int gemm_w8a8_g128_group_partials_ex(const int8_t *qa, const int32_t *qweight, int32_t *P, int64_t M,
                                     int64_t N, int64_t K, int kernel, int decode_workgroups, void *stream);

/*
 * W4A16 g128 weight-only linear (Qwen3.8-27B-DFlash2 W4A16 card, property and
 * quantised-layer tables): y[m,n] = bf16( sum_g w_scale[g,n] * sum_{k in g} x[m,k]*q[k,n] )
 * with q = nibble - 8 in [-8, 7].  x bf16 [M, ldx]; qweight int32 [K/8, N] (nibble j of
 * word [r, n] is k = 8r + j); w_scale fp32 [K/128, N]; y bf16 [M, ldy].  Weights are
 * dequantised in registers to exact integer-valued bf16, each group is summed by bf16
 * MFMA in fp32 and then scaled, so y is within one bf16 unit of the exact value plus
 * (K/128 + 130) * 2^-24 * sum_g |w_scale| * sum_k |x*q|.
 * workspace: i8gs_workspace_bytes(I8GS_OP_W4A16, M, N, K) bytes (may be NULL if 0).
 */
int gemm_w4a16_g128(const void *x, int64_t ldx, const int32_t *qweight, const float *w_scale,
                    void *y, int64_t ldy, int64_t M, int64_t N, int64_t K, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * Weight-only group-scaled linear, 4- or 8-bit weights (Qwen3.8-27B-DFlash2 W4A16 card,
 * property table: 4-bit, group 128, symmetric; Qwen3.5-4B-DFlash-W8A16 card: int8
 * weights with bf16 activations, RTN; qwen38/dflash2 recipe, quantisation settings:
 * int8 drafter projections at group 32, int4 / int8 vocabulary heads at group 128):
 *   y[m,n] = bf16( sum_g w_scale[g,n] * sum_{k in g} x[m,k] * q[k,n] ),  g = k / group,
 * q = code - 2^(bits-1).  x bf16 [M, ldx]; qweight int32 [K/(32/bits), N] (code j of word
 * [r, n] is k = (32/bits)*r + j); w_scale fp32 [K/group, N]; y bf16 [M, ldy].
 * (bits, group) is (4, 128), (8, 128) or (8, 32); anything else is I8GS_ERR_INVALID_ARG.
 * Weights are dequantised in registers to exact integer-valued bf16, each group is
 * summed by bf16 MFMA in fp32 and then scaled, so y is within one bf16 unit of the
 * exact value plus (K/group + group + 2) * 2^-24 * sum_g |w_scale| * sum_k |x*q|.
 * Also needs (min(M,64)-1)*ldx*2 + K*2 < 2^31.  workspace:
 * i8gs_workspace_bytes(I8GS_OP_WEIGHT_ONLY, M, N, K) bytes (may be NULL if 0).
 */
int gemm_weight_only(const void *x, int64_t ldx, const int32_t *qweight, int bits, const float *w_scale, int group,
                     void *y, int64_t ldy, int64_t M, int64_t N, int64_t K, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * GPTQ unpack (W4A16 card dequant-patch table, "unpack from int32 plus group
 * scales"; the W8A16 card's identity probe recovers the same dense rows).
 * From qweight int32 [K/(32/bits), N] (bits = 8 or 4) write, for each output that is
 * not NULL:  q_out int8 [K, N] = code - 2^(bits-1);  w_out fp32 [K, N] =
 * fl32(w_scale[k/128, n] * q[k, n]) (w_scale required when w_out is given).
 * At least one output must be given.  Bit-exact.
 */
int gptq_unpack(const int32_t *qweight, const float *w_scale, int bits, int64_t K, int64_t N,
                int8_t *q_out, float *w_out, void *stream);

/*
 * Round-to-nearest G128 symmetric weight quantisation with GPTQ packing (W4A16
 * card scripts: RTN with no calibration data; W8A16 card: pure RTN).  From w fp32
 * [K, N]: w_scale[g, n] = absmax over the group / qmax (fp32; qmax = 127 for 8 bits,
 * 7 for 4 bits), q = clamp(rint(w / w_scale), -127, 127) or (-8, 7) (q = 0 when
 * the group is all zero), written as codes q + 2^(bits-1) into qweight int32
 * [K/(32/bits), N].  K % 128 == 0.  Bit-exact.
 */
int gptq_quantize_rtn(const float *w, int bits, int64_t K, int64_t N, int32_t *qweight,
                      float *w_scale, void *stream);

/* The same with `group` (32 or 128) consecutive K values per scale; w_scale is fp32
 * [K/group, N] (qwen38/dflash2 recipe: group-32 RTN int8 projections).  Bit-exact. */
int gptq_quantize_rtn_group(const float *w, int bits, int group, int64_t K, int64_t N, int32_t *qweight,
                            float *w_scale, void *stream);

/*
 * INT8 block-g128 KV cache codec (Flint-DFlash2-GPTQ-INT8-PTQR model card, serving
 * recipe: the target's and the draft's KV cache dtype "int8_block_g128"; serving notes).
 * One fp32 scale per 128-wide group, i.e. per head vector of one token, with the
 * per-token activation quantiser applied to each such vector:
 *   scales[t, h] = max_d |kv[t, h, d]| / 127 (fp32),
 *   codes[t, h, d] = clamp(rint(kv[t, h, d] / scales[t, h]), -127, 127)   (ties to even)
 *   kv      device bf16, head vector h of token t at kv + t*ld + 128*h (ld >= 128*H,
 *           ld % 8 == 0): a contiguous [T, H, 128] cache, or the K or V slice of a fused
 *           qkv projection output (pointer at the slice, ld = the output's row length)
 *   codes   device int8 [T, H, 128], output;  scales  device fp32 [T, H], output
 * Bit-exact.  The query side of the QK product quantises its head vectors the same way.
 */
int kv_quant_int8_block128(const void *kv, int64_t ld, int64_t T, int64_t H, int8_t *codes, float *scales,
                           void *stream);

/*
 * INT8 QK product on the block-g128 cache (Flint card serving recipe: INT8 DOT
 * attention on the int8_block_g128 KV cache).  For Hq query heads sharing Hkv KV heads
 * (head h reads KV head h / (Hq/Hkv)) and head dimension 128:
 *   dots[h, i, t] = sum_d qq[i, h, d] * kq[t, hk, d]     (exact int32)
 *   s[h, i, t]    = ((scale * qs[i, h]) * ks[t, hk]) * dots[h, i, t]   (fp32, in this order)
 * so s is within 3 * 2^-24 relative of the exact product of the four factors (the
 * int32 dot converts exactly: |dot| <= 128 * 127^2 < 2^24).
 *   qq int8 [Mq, Hq, 128], qs fp32 [Mq, Hq] (the codec's output for the queries)
 *   kq int8 [T, Hkv, 128], ks fp32 [T, Hkv] (the K cache)
 *   scale   finite fp32 (e.g. 1/sqrt(128))
 *   s       fp32 [Hq, Mq, T], output;  dots  int32 [Hq, Mq, T] or NULL, output
 * Hq % Hkv == 0, Hkv > 0, Hq <= 65535, (Hq/Hkv)*Mq <= 2097120, Hq*Mq*T <= 2^40.
 * Empty sizes are a no-op.
 */
int attn_qk_int8(const int8_t *qq, const float *qs, const int8_t *kq, const float *ks, float scale, int64_t Mq,
                 int64_t T, int64_t Hq, int64_t Hkv, float *s, int32_t *dots, void *stream);

/*
 * INT8 PV product on the block-g128 cache (Flint card serving recipe: INT8 PV).  The
 * pages name the INT8 PV product but not how the probabilities are quantised; this
 * moves each token's V scale onto its probability and quantises the result per block
 * of 128 tokens with the activation codec, so the product is the group-scaled INT8
 * product of the linear layer with K = tokens:
 *   p'[h,i,t]  = fl32(p[h,i,t] * vs[t, hk])
 *   ps[h,i,b]  = max_{t in block b} |p'| / 127  (fp32; a last partial block takes its tokens)
 *   pq[h,i,t]  = clamp(rint(p' / ps), -127, 127)  (0 where ps = 0; IEEE division)
 *   out[h,i,d] = sum_b ps[h,i,b] * sum_{t in b} pq[h,i,t] * vq[t, hk, d]
 * The block sums are exact int32; the fold over blocks is fp32 (split over token ranges
 * when there are few rows, the ranges summed in a fixed order), so out is within
 * (B + 2) * 2^-24 * sum_b |ps| * sum_t |pq * vq| of the exact value (B = ceil(T/128))
 * and the same inputs always give the same bits.  pq and ps are bit-exact.
 *   p   fp32 [Hq, Mq, T] (e.g. softmax of the QK scores);  vq int8 [T, Hkv, 128],
 *   vs  fp32 [T, Hkv] (the V cache)
 *   out fp32 [Hq, Mq, 128], output (zeros when T == 0)
 *   pq  int8 [Hq, Mq, T] or NULL;  ps  fp32 [Hq, Mq, B] or NULL (outputs)
 *   workspace  attn_pv_int8_workspace_bytes(Mq, T, Hq, Hkv) bytes (NULL if 0), laid
 *              out as for the GEMMs: the 64 KiB counter region first (not touched
 *              here, so one workspace serves both), then the fp32 sums of the token
 *              ranges, written and read within the call; not shared with a
 *              concurrent call
 * Size limits as for attn_qk_int8.
 */
int attn_pv_int8(const float *p, const int8_t *vq, const float *vs, int64_t Mq, int64_t T, int64_t Hq, int64_t Hkv,
                 float *out, int8_t *pq, float *ps, void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes attn_pv_int8 needs for these sizes (0: none), or (size_t)-1 for
 * invalid sizes. */
size_t attn_pv_int8_workspace_bytes(int64_t Mq, int64_t T, int64_t Hq, int64_t Hkv);

#ifdef __cplusplus
}
#endif

#endif /* I8GS_H */
