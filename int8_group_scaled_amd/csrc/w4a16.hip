// W4A16 g128 weight-only GEMM on gfx950 bf16 MFMA.
//
// Qwen3.8-27B-DFlash2-W4A16-g128-sym-GPTQ model card, property table (W4A16,
// group_size 128, symmetric) and quantised-layer table (all attention / MLP
// linears and fc in INT4 g128 sym).  y[m,n] = bf16(sum_g w_scale[g,n] *
// sum_{k in g} x[m,k] * q[k,n]) with q = nibble - 8.
//
// Each nibble is turned into the exact bf16 value of q (an integer in [-8, 7]:
// XOR 8 makes it a two's-complement 4-bit field, a signed bit-field extract and
// an int->float conversion give q exactly, and the top half of that float is its
// bf16 pattern).  One 128-wide group is summed by four v_mfma_f32_16x16x32_bf16
// into a fresh fp32 accumulator (the products are exact in fp32), then scaled by
// that group's per-column scale and added to the running fp32 sum.  Scaling after
// the group keeps the error relative to sum |x*q| rather than to the cancelling
// scaled terms.
//
// MFMA layout (16x16x32 bf16): lane l holds row (l % 16) of A and column (l % 16)
// of B, 8 consecutive K values starting at 8 * (l / 16) within the 32-wide K step;
// with GPTQ's packing those 8 values of one column are exactly one int32 word.
//
// At decode sizes the bf16 activation rows are the larger operand (2 bytes per
// element against half a byte of weight), so a workgroup stages each group's
// activations in LDS once and its W waves, each owning F 16-column fragments,
// all read them; weight words go straight from HBM into registers, one group
// ahead.  K is split across S workgroups when the column tiles alone cannot fill
// the GPU, with the same deterministic last-arrival reduction as the W8A8 path.
// Rows are processed in chunks of 64 (gridDim.y).
#include "internal.h"

namespace i8gs {
namespace {

constexpr int kMC = 64;           // rows per chunk
constexpr int kAPitch = 128 + 8;  // bf16 elements per LDS row (272 bytes)

__device__ __forceinline__ v8bf dequant8(uint32_t w) {
    const uint32_t s = w ^ 0x88888888u;
    uint32_t h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int q = ((int)(s << (28 - 4 * j))) >> 28;  // signed nibble j: code - 8
        h[j] = __float_as_uint((float)q);
    }
    v4i out;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = (int)((h[2 * i] >> 16) | (h[2 * i + 1] & 0xFFFF0000u));
    return __builtin_bit_cast(v8bf, out);
}

__device__ __forceinline__ v4f mfma_bf16(v4i a, v8bf b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), b, c, 0, 0, 0);
}

template <int MT, int F, int W>
__global__ __launch_bounds__(W * 64) void w4a16_decode_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, const int32_t *__restrict__ qweight,
    const float *__restrict__ w_scale, uint16_t *__restrict__ y, int64_t ldy, int M, int N, int K, int S,
    int tiles, float *__restrict__ part, int *__restrict__ cnt) {
    constexpr int TN = 16 * F * W;
    constexpr int ROWS = MT * 16;
    constexpr int CHUNKS = ROWS * 16 / (W * 64);  // 16-byte A pieces per thread per group
    static_assert(CHUNKS >= 1 && CHUNKS * W * 64 == ROWS * 16, "A staging must divide evenly");
    __shared__ __attribute__((aligned(16))) uint16_t As[2][ROWS * kAPitch];

    const int per_xcd = gridDim.x >> 3;
    const int pair = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (pair >= tiles * S) return;
    const int t = pair / S;
    const int s = pair - t * S;
    const int m0 = blockIdx.y * kMC;
    const int mrows = min(M - m0, ROWS);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lb = lane >> 4;
    const int n0 = t * TN + wave * 16 * F;
    const int G = K >> 7;
    const int g0 = (int)((int64_t)s * G / S), g1 = (int)((int64_t)(s + 1) * G / S);

    int bcol[F];
#pragma unroll
    for (int f = 0; f < F; ++f) bcol[f] = min(n0 + f * 16 + li, N - 1);

    // A staging: piece c = tid + i * W*64 covers row c / 16, 16 bytes at (c % 16) * 8 elements.
    const uint16_t *arow_ptr[CHUNKS];
    int aoff[CHUNKS];
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
        const int c = tid + i * W * 64;
        const int row = c >> 4, col = (c & 15) * 8;
        arow_ptr[i] = x + (int64_t)(m0 + min(row, mrows - 1)) * ldx + col;
        aoff[i] = row * kAPitch + col;
    }

    float acc[F][MT][4];
#pragma unroll
    for (int f = 0; f < F; ++f)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[f][mt][r] = 0.0f;

    v4i areg[CHUNKS];
    int wq[F][4];
    if (g0 < g1) {
#pragma unroll
        for (int i = 0; i < CHUNKS; ++i) areg[i] = *reinterpret_cast<const v4i *>(arow_ptr[i] + g0 * 128);
#pragma unroll
        for (int f = 0; f < F; ++f)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                wq[f][ks] = __builtin_nontemporal_load(qweight + (int64_t)(g0 * 16 + ks * 4 + lb) * N + bcol[f]);
    }
    for (int g = g0; g < g1; ++g) {
        const int buf = (g - g0) & 1;
        uint16_t *Ab = As[buf];
#pragma unroll
        for (int i = 0; i < CHUNKS; ++i) *reinterpret_cast<v4i *>(Ab + aoff[i]) = areg[i];
        int wc[F][4];
#pragma unroll
        for (int f = 0; f < F; ++f)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) wc[f][ks] = wq[f][ks];
        if (g + 1 < g1) {
#pragma unroll
            for (int i = 0; i < CHUNKS; ++i) areg[i] = *reinterpret_cast<const v4i *>(arow_ptr[i] + (g + 1) * 128);
#pragma unroll
            for (int f = 0; f < F; ++f)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    wq[f][ks] =
                        __builtin_nontemporal_load(qweight + (int64_t)((g + 1) * 16 + ks * 4 + lb) * N + bcol[f]);
        }
        __syncthreads();
        float sc[F];
#pragma unroll
        for (int f = 0; f < F; ++f) sc[f] = w_scale[(int64_t)g * N + bcol[f]];
        v4f p[F][MT];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            v4i a[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                a[mt] = *reinterpret_cast<const v4i *>(Ab + (mt * 16 + li) * kAPitch + ks * 32 + lb * 8);
#pragma unroll
            for (int f = 0; f < F; ++f) {
                const v8bf b = dequant8((uint32_t)wc[f][ks]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    p[f][mt] = mfma_bf16(a[mt], b, ks == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : p[f][mt]);
            }
        }
#pragma unroll
        for (int f = 0; f < F; ++f)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[f][mt][r] += sc[f] * p[f][mt][r];
    }

    if (S > 1) {
        constexpr int NACC = F * MT * 4;
        const int64_t tile_id = (int64_t)blockIdx.y * tiles + t;
        float *mine = part + ((tile_id * S + s) * W + wave) * NACC * 64;
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
        __syncthreads();
        __shared__ int s_old;
        if (tid == 0) s_old = atomicAdd(cnt + tile_id, 1);
        __syncthreads();
        if (s_old != S - 1) return;
        __threadfence();
        int i = 0;
#pragma unroll
        for (int f = 0; f < F; ++f)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r, ++i) {
                    float v = 0.0f;
                    for (int q = 0; q < S; ++q)
                        v += __builtin_nontemporal_load(part + (((tile_id * S + q) * W + wave) * NACC + i) * 64 + lane);
                    acc[f][mt][r] = v;
                }
        if (tid == 0) cnt[tile_id] = 0;
    }

#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = mt * 16 + lb * 4 + r;
            if (row < mrows) {
#pragma unroll
                for (int f = 0; f < F; ++f) {
                    const int col = n0 + f * 16 + li;
                    if (col < N) y[(int64_t)(m0 + row) * ldy + col] = f32_to_bf16_bits(acc[f][mt][r]);
                }
            }
        }
}

struct W4Plan {
    int MT, F, W, S, tiles, blocks, chunks;
};

W4Plan w4_plan(int M, int N, int K) {
    W4Plan p;
    p.MT = M >= 64 ? 4 : (M + 15) / 16;
    p.F = 2;
    p.W = 4;
    p.chunks = (M + kMC - 1) / kMC;
    const int TN = 16 * p.F * p.W;
    p.tiles = (N + TN - 1) / TN;
    const int G = K / kGroup;
    int S = (256 + p.tiles * p.chunks - 1) / (p.tiles * p.chunks);
    if (S > G) S = G;
    if (S < 1) S = 1;
    if (p.tiles * p.chunks > kMaxCounters) S = 1;
    p.S = S;
    p.blocks = ((p.tiles * p.S + 7) / 8) * 8;
    return p;
}

template <int MT>
hipError_t launch_w4_mt(const W4A16Args &a, const W4Plan &p, hipStream_t st) {
    int *cnt = p.S > 1 ? a.counters : nullptr;
    float *part = p.S > 1 ? (float *)a.ws : nullptr;
    dim3 grid(p.blocks, p.chunks);
    w4a16_decode_kernel<MT, 2, 4><<<grid, 256, 0, st>>>(a.x, a.ldx, a.qweight, a.w_scale, a.y, a.ldy, a.M, a.N,
                                                       a.K, p.S, p.tiles, part, cnt);
    return hipGetLastError();
}

}  // namespace

// Partial-sum bytes after the counter region (0 when K is not split).
size_t w4a16_gemm_workspace(int M, int N, int K) {
    const W4Plan p = w4_plan(M, N, K);
    if (p.S <= 1) return 0;
    return align256(size_t(p.tiles) * p.chunks * p.S * p.W * p.F * p.MT * 4 * 64 * sizeof(float));
}

hipError_t launch_w4a16_gemm(const W4A16Args &a, hipStream_t s) {
    const W4Plan p = w4_plan(a.M, a.N, a.K);
    switch (p.MT) {
        case 1: return launch_w4_mt<1>(a, p, s);
        case 2: return launch_w4_mt<2>(a, p, s);
        case 3: return launch_w4_mt<3>(a, p, s);
        default: return launch_w4_mt<4>(a, p, s);
    }
}

}  // namespace i8gs
