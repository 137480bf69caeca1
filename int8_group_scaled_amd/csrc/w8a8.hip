// W8A8 G128 GEMM on gfx950 MFMA.
//
// Qwen3.8-27B GPTQ INT8 W8A8 GS128 PTQR model card, "Quantization details": true
// int8 x int8 compute at every decode and prefill shape with one weight scale per
// 128-wide K block.  Flint INT8 card, format table: GPTQ qweight/scales, symmetric,
// group 128, no g_idx.  For each 128-wide group the int8 products are summed exactly
// in an int32 MFMA accumulator (v_mfma_i32_16x16x64_i8, two per group), converted to
// fp32 and folded with that group's per-column scale; the row scale and the bf16
// rounding are applied once at the end.
//
// MFMA operand layout used here (16x16x64 i8): lane l holds row (l % 16) of A and
// column (l % 16) of B, 16 consecutive K bytes starting at 16 * (l / 16) within a
// 64-wide K step.  A and B use the same K placement, so the product is the plain
// dot product whatever order the hardware walks K in.  The 16x16 int32 result puts
// column (l % 16), rows 4 * (l / 16) + r (r = 0..3) in lane l.
//
// GPTQ codes are offset binary (q + 128); XOR 0x80 per byte turns a code into the
// two's-complement int8 value of q.
//
// Two kernels:
//  * decode (M <= 64): bound by streaming the weights from HBM.  A workgroup owns a
//    tile of 16*F columns and a range of K groups; its W waves split that range,
//    every wave loads its weight fragments straight from HBM into registers (4
//    dword rows of 16 columns per 64-wide K step) and its activation fragments
//    from L2, with one group of loads in flight ahead of the MFMAs.  Waves reduce
//    through LDS in a fixed order.  When the tiles alone cannot fill the GPU, K is
//    also split across S workgroups: each writes an fp32 partial tile to the
//    workspace, and the last of the S to arrive (a per-tile atomic counter) sums the
//    partials in split order and writes y, so results do not depend on timing.
//  * tiled (M > 64): LDS-staged 128x128 tiles, four waves of 64x64.
#include "internal.h"

namespace i8gs {
namespace {

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4i flip(v4i v) {
    return v ^ (int)0x80808080;
}

// ------------------------------------------------------------------ decode kernel

struct DecodePlan {
    int F;       // 16-column fragments per tile
    int W;       // waves per workgroup
    int S;       // K splits across workgroups
    int tiles;   // column tiles
    int blocks;  // launched workgroups (multiple of 8)
};

template <int MT, int F>
struct DecodeFrag {
    v4i a[MT][2];
    v4i b[F][2];
};

template <int MT, int F>
__device__ __forceinline__ void decode_load(DecodeFrag<MT, F> &fr, const int8_t *__restrict__ qa,
                                            const int32_t *__restrict__ qweight, int g, int K, int N,
                                            const int *arow, const int *bcol, int lb) {
#pragma unroll
    for (int f = 0; f < F; ++f) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int32_t *p = qweight + (int64_t)(g * 32 + ks * 16 + lb * 4) * N + bcol[f];
            v4i v;
            v[0] = __builtin_nontemporal_load(p);
            v[1] = __builtin_nontemporal_load(p + N);
            v[2] = __builtin_nontemporal_load(p + 2 * (int64_t)N);
            v[3] = __builtin_nontemporal_load(p + 3 * (int64_t)N);
            fr.b[f][ks] = v;
        }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            fr.a[mt][ks] = *reinterpret_cast<const v4i *>(qa + (int64_t)arow[mt] * K + g * 128 + ks * 64 + lb * 16);
    }
}

template <int MT, int F, int W>
__global__ __launch_bounds__(W * 64) void w8a8_decode_kernel(
    const int8_t *__restrict__ qa, const float *__restrict__ a_scale, const int32_t *__restrict__ qweight,
    const float *__restrict__ w_scale, uint16_t *__restrict__ y, int64_t ldy, int M, int N, int K, int S,
    int tiles, float *__restrict__ part, int *__restrict__ cnt) {
    constexpr int TN = 16 * F;
    constexpr int NACC = F * MT * 4;  // fp32 accumulators per lane
    __shared__ float red[(W > 1 ? W - 1 : 1) * NACC * 64];

    // blockIdx -> (tile, split): consecutive (tile, split) pairs go to the same XCD
    // (workgroups are dispatched round-robin over the 8 XCDs), so the S partials of a
    // tile meet in one L2.
    const int per_xcd = gridDim.x >> 3;
    const int pair = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (pair >= tiles * S) return;
    const int t = pair / S;
    const int s = pair - t * S;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int li = lane & 15, lb = lane >> 4;
    const int n0 = t * TN;
    const int G = K >> 7;
    const int gs0 = (int)((int64_t)s * G / S), gs1 = (int)((int64_t)(s + 1) * G / S);
    const int ng = gs1 - gs0;
    const int g0 = gs0 + (wave * ng) / W, g1 = gs0 + ((wave + 1) * ng) / W;

    int arow[MT], bcol[F];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) arow[mt] = min(mt * 16 + li, M - 1);
#pragma unroll
    for (int f = 0; f < F; ++f) bcol[f] = min(n0 + f * 16 + li, N - 1);

    float acc[F][MT][4];
#pragma unroll
    for (int f = 0; f < F; ++f)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[f][mt][r] = 0.0f;

    if (g0 < g1) {
        DecodeFrag<MT, F> cur, nxt;
        decode_load<MT, F>(nxt, qa, qweight, g0, K, N, arow, bcol, lb);
        for (int g = g0; g < g1; ++g) {
            cur = nxt;
            if (g + 1 < g1) decode_load<MT, F>(nxt, qa, qweight, g + 1, K, N, arow, bcol, lb);
            float sc[F];
#pragma unroll
            for (int f = 0; f < F; ++f) sc[f] = w_scale[(int64_t)g * N + bcol[f]];
#pragma unroll
            for (int f = 0; f < F; ++f) {
                const v4i b0 = flip(cur.b[f][0]);
                const v4i b1 = flip(cur.b[f][1]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    v4i p = mfma_i8(cur.a[mt][0], b0, v4i{0, 0, 0, 0});
                    p = mfma_i8(cur.a[mt][1], b1, p);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[f][mt][r] += sc[f] * (float)p[r];
                }
            }
        }
    }

    // Fixed-order reduction over the waves of the workgroup (wave 0 + 1 + ... in order).
    if constexpr (W > 1) {
        if (wave > 0) {
            float *dst = red + (wave - 1) * NACC * 64;
            int i = 0;
#pragma unroll
            for (int f = 0; f < F; ++f)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r, ++i) dst[i * 64 + lane] = acc[f][mt][r];
        }
        __syncthreads();
        if (wave > 0) return;
#pragma unroll
        for (int w = 1; w < W; ++w) {
            const float *src = red + (w - 1) * NACC * 64;
            int i = 0;
#pragma unroll
            for (int f = 0; f < F; ++f)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r, ++i) acc[f][mt][r] += src[i * 64 + lane];
        }
    }

    if (S > 1) {
        // Publish this split's partial tile, then count arrivals.
        float *mine = part + ((int64_t)t * S + s) * NACC * 64;
        {
            int i = 0;
#pragma unroll
            for (int f = 0; f < F; ++f)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r, ++i) mine[i * 64 + lane] = acc[f][mt][r];
        }
        __threadfence();
        int old = 0;
        if (lane == 0) old = atomicAdd(cnt + t, 1);
        old = __shfl(old, 0, 64);
        if (old != S - 1) return;
        __threadfence();
        // Last arrival: sum the S partials in split order.
        const float *base = part + (int64_t)t * S * NACC * 64;
        int i = 0;
#pragma unroll
        for (int f = 0; f < F; ++f)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r, ++i) {
                    float v = 0.0f;
                    for (int q = 0; q < S; ++q) v += __builtin_nontemporal_load(base + ((int64_t)q * NACC + i) * 64 + lane);
                    acc[f][mt][r] = v;
                }
        if (lane == 0) cnt[t] = 0;  // leave the counter at zero for the next call
    }

    // Epilogue: y = bf16(a_scale[row] * acc).
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = mt * 16 + lb * 4 + r;
            if (row < M) {
                const float as = a_scale[row];
#pragma unroll
                for (int f = 0; f < F; ++f) {
                    const int col = n0 + f * 16 + li;
                    if (col < N) y[(int64_t)row * ldy + col] = f32_to_bf16_bits(as * acc[f][mt][r]);
                }
            }
        }
    }
}

DecodePlan decode_plan(int M, int N, int K, int split_k) {
    (void)M;
    DecodePlan p;
    p.F = 4;
    p.W = 4;
    p.tiles = (N + 16 * p.F - 1) / (16 * p.F);
    const int G = K / kGroup;
    int S = split_k;
    if (S <= 0) {
        // Split K across workgroups until every CU (256) has a workgroup, keeping at
        // least one group per wave.
        S = (256 + p.tiles - 1) / p.tiles;
        if (S * p.W > G) S = G / p.W;
        if (S < 1) S = 1;
    }
    if (S > G) S = G;
    if (p.tiles > kMaxCounters) S = 1;  // counters are per tile
    p.S = S;
    p.blocks = ((p.tiles * p.S + 7) / 8) * 8;
    return p;
}

// Partial-sum bytes after the counter region (0 when K is not split).
size_t decode_workspace(const DecodePlan &p, int M) {
    if (p.S <= 1) return 0;
    const int MT = (M + 15) / 16;
    return align256(size_t(p.tiles) * p.S * p.F * MT * 4 * 64 * sizeof(float));
}

template <int MT>
hipError_t launch_decode_mt(const W8A8Args &a, const DecodePlan &p, hipStream_t st) {
    int *cnt = p.S > 1 ? a.counters : nullptr;
    float *part = p.S > 1 ? (float *)a.ws : nullptr;
    w8a8_decode_kernel<MT, 4, 4><<<p.blocks, 256, 0, st>>>(a.qa, a.a_scale, a.qweight, a.w_scale, a.y, a.ldy,
                                                          a.M, a.N, a.K, p.S, p.tiles, part, cnt);
    return hipGetLastError();
}

// ------------------------------------------------------------------ tiled kernel (M > 64)

constexpr int kTB = 128;       // tile rows and columns
constexpr int kPitch = 144;    // LDS row pitch in bytes (128 + 16)

template <bool PARTIALS>
__global__ __launch_bounds__(256) void w8a8_tiled_kernel(const int8_t *__restrict__ qa,
                                                         const float *__restrict__ a_scale,
                                                         const int32_t *__restrict__ qweight,
                                                         const float *__restrict__ w_scale,
                                                         uint16_t *__restrict__ y, int64_t ldy,
                                                         int32_t *__restrict__ P, int M, int N, int K) {
    constexpr int MT = 4, NT = 4;  // each wave: 64 x 64
    __shared__ __attribute__((aligned(16))) int8_t As[kTB * kPitch];
    __shared__ __attribute__((aligned(16))) int8_t Bs[kTB * kPitch];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lb = lane >> 4;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    const int m0 = blockIdx.y * kTB, n0 = blockIdx.x * kTB;
    const int G = K >> 7;

    float acc[MT][NT][4];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;

    for (int g = 0; g < G; ++g) {
        __syncthreads();
        // A tile: 128 rows x 128 bytes, 16 bytes per thread per step.
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int c = tid + it * 256;
            const int row = c >> 3, c16 = c & 7;
            const int gm = m0 + row;
            v4i v = v4i{0, 0, 0, 0};
            if (gm < M) v = *reinterpret_cast<const v4i *>(qa + (int64_t)gm * K + g * 128 + c16 * 16);
            *reinterpret_cast<v4i *>(As + row * kPitch + c16 * 16) = v;
        }
        // B tile: 32 word rows x 128 columns, transposed into [column][k] bytes.
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int c = tid + it * 256;
            const int rl = c >> 5, cq = c & 31;
            const int gn = n0 + cq * 4;
            v4i v = v4i{0, 0, 0, 0};
            if (gn < N) v = flip(*reinterpret_cast<const v4i *>(qweight + (int64_t)(g * 32 + rl) * N + gn));
#pragma unroll
            for (int i = 0; i < 4; ++i) *reinterpret_cast<int *>(Bs + (cq * 4 + i) * kPitch + rl * 4) = v[i];
        }
        __syncthreads();
        v4i pi[MT][NT];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            v4i af[MT], bf[NT];
#pragma unroll
            for (int i = 0; i < MT; ++i)
                af[i] = *reinterpret_cast<const v4i *>(As + (wm + i * 16 + li) * kPitch + ks * 64 + lb * 16);
#pragma unroll
            for (int j = 0; j < NT; ++j)
                bf[j] = *reinterpret_cast<const v4i *>(Bs + (wn + j * 16 + li) * kPitch + ks * 64 + lb * 16);
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j) pi[i][j] = mfma_i8(af[i], bf[j], ks == 0 ? v4i{0, 0, 0, 0} : pi[i][j]);
        }
        if constexpr (PARTIALS) {
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const int col = n0 + wn + j * 16 + li;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = m0 + wm + i * 16 + lb * 4 + r;
                        if (row < M && col < N) P[((int64_t)row * G + g) * N + col] = pi[i][j][r];
                    }
                }
        } else {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int col = min(n0 + wn + j * 16 + li, N - 1);
                const float sc = w_scale[(int64_t)g * N + col];
#pragma unroll
                for (int i = 0; i < MT; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[i][j][r] += sc * (float)pi[i][j][r];
            }
        }
    }
    if constexpr (!PARTIALS) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm + i * 16 + lb * 4 + r;
                if (row >= M) continue;
                const float as = a_scale[row];
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const int col = n0 + wn + j * 16 + li;
                    if (col < N) y[(int64_t)row * ldy + col] = f32_to_bf16_bits(as * acc[i][j][r]);
                }
            }
    }
}

}  // namespace

static bool use_decode(int M, int kernel) {
    if (kernel == I8GS_KERNEL_DECODE) return true;
    if (kernel == I8GS_KERNEL_TILED) return false;
    return M <= 64;
}

size_t w8a8_gemm_workspace(int M, int N, int K, int kernel, int split_k) {
    if (use_decode(M, kernel)) return decode_workspace(decode_plan(M, N, K, split_k), M);
    return 0;
}

hipError_t launch_w8a8_gemm(const W8A8Args &a, hipStream_t s) {
    if (a.P == nullptr && use_decode(a.M, a.kernel)) {
        const DecodePlan p = decode_plan(a.M, a.N, a.K, a.split_k);
        switch ((a.M + 15) / 16) {
            case 1: return launch_decode_mt<1>(a, p, s);
            case 2: return launch_decode_mt<2>(a, p, s);
            case 3: return launch_decode_mt<3>(a, p, s);
            default: return launch_decode_mt<4>(a, p, s);
        }
    }
    dim3 grid((a.N + kTB - 1) / kTB, (a.M + kTB - 1) / kTB);
    if (a.P)
        w8a8_tiled_kernel<true><<<grid, 256, 0, s>>>(a.qa, nullptr, a.qweight, nullptr, nullptr, 0, a.P, a.M, a.N,
                                                    a.K);
    else
        w8a8_tiled_kernel<false><<<grid, 256, 0, s>>>(a.qa, a.a_scale, a.qweight, a.w_scale, a.y, a.ldy, nullptr,
                                                     a.M, a.N, a.K);
    return hipGetLastError();
}

}  // namespace i8gs
