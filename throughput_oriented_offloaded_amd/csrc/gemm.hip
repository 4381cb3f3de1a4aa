// Fused group-wise int4 dequant + fp16 MFMA GEMM for gfx950 (and its fp16-weight twin).
//
//   y[m][n] = fp16( sum_k a[m][k] * What[n][k] + bias[n] (+ residual[m][n]) (ReLU) )
//
// FlexGen computes in fp16 on weights dequantized on the fly inside registers
// (FlexGen guide, "3. Group-Wise 4-Bit Quantization": FP16 compute
// preservation). In a decode step the block's K*b rows form M, so each weight
// tile is fetched from HBM once per step for the whole block (FlexGen guide,
// "2. The Zig-Zag Block Schedule").
//
// gfx950 design:
//  * v_mfma_f32_32x32x16_f16, fp32 accumulation; 256-thread workgroups as a
//    2x2 grid of wavefronts, each owning a (BM/2) x (BN/2) output tile.
//  * The activation tile (BM x 64, one quantization group of K) is staged in
//    LDS, double-buffered, 16-byte chunks XOR-swizzled by row to spread banks.
//  * Weights never touch LDS: the int4 store is pre-tiled so that one 16-byte
//    load per lane brings exactly the 32 nibbles that lane feeds to four MFMA
//    K-steps as its B operand. Dequantization is two packed-fp16 ops per pair:
//    (nibbles | 0x6400) - 1024 gives exact codes, then one v_pk_fma_f16 with
//    (scale, zero) rounds once, so each weight equals fp16(zero + c*scale).
//  * Workgroup ids are remapped so that each XCD (ids round-robin over 8 XCDs)
//    gets a contiguous run of tiles, M fastest: workgroups sharing a weight
//    tile share that XCD's L2.
//  * When the tile grid is too small to fill 256 CUs the K loop is split and
//    fp32 partials are reduced by a second kernel (deterministic order).
#include "common.hpp"

namespace {

constexpr int KG_ELEMS = 64; // K elements per main-loop iteration (one quant group)

struct TileMap {
    int mt, nt, splits, groups_per_split, total;
};

__device__ __forceinline__ int xcd_tile(int b, int total)
{
    // Workgroup b runs on XCD b % 8 as the (b / 8)-th of that XCD; give each XCD a
    // contiguous range of tile ids.
    const int x = b & 7, k = b >> 3, q = total >> 3, r = total & 7;
    return x * q + (x < r ? x : r) + k;
}

__device__ __forceinline__ half8_t dequant_word(uint32_t w, half2_t s2, half2_t z2)
{
    const half2_t bias = {(half_t)1024.0f, (half_t)1024.0f};
    half8_t out;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const uint32_t u = ((w >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
        const half2_t c = __builtin_bit_cast(half2_t, u) - bias; // exact codes
        const half2_t x = __builtin_elementwise_fma(c, s2, z2);  // one rounding
        out[2 * j] = x[0];
        out[2 * j + 1] = x[1];
    }
    return out;
}

template <int BM, int BN, bool INT4>
__global__ void __launch_bounds__(256) k_gemm(GemmArgs g, TileMap tm)
{
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int MB = WM / 32, NB = WN / 32;
    constexpr int A_LOADS = BM * 8 / 256; // 16-byte chunks per thread per group
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * BM * 128];

    const int tile = xcd_tile(blockIdx.x, tm.total);
    if (tile >= tm.total)
        return;
    const int m_tile = tile % tm.mt;
    const int rest = tile / tm.mt;
    const int n_tile = rest % tm.nt;
    const int split = rest / tm.nt;
    const int m0 = m_tile * BM, n0 = n_tile * BN;
    const int KG = g.K / KG_ELEMS;
    const int g0 = split * tm.groups_per_split;
    const int g1 = min(KG, g0 + tm.groups_per_split);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- A tile loader: thread handles chunks c = tid + 256*i (row c/8, chunk c%8)
    uint4_t areg[A_LOADS];
    auto load_a = [&](int grp) {
#pragma unroll
        for (int i = 0; i < A_LOADS; i++) {
            const int c = tid + 256 * i, row = c >> 3, ch = c & 7;
            const int m = m0 + row;
            if (m < g.M)
                areg[i] = *reinterpret_cast<const uint4_t *>(g.a + (int64_t)m * g.lda + grp * KG_ELEMS + ch * 8);
            else
                areg[i] = (uint4_t){0u, 0u, 0u, 0u};
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_LOADS; i++) {
            const int c = tid + 256 * i, row = c >> 3, ch = c & 7;
            *reinterpret_cast<uint4_t *>(smem + buf * BM * 128 + row * 128 + ((ch ^ (row & 7)) << 4)) = areg[i];
        }
    };

    // ---- B (weights) loader
    const int nb_base = (n0 + wn * WN) >> 5; // first 32-column block of this wave
    uint4_t bw[NB];        // int4: 32 nibbles per lane and column block
    uint32_t bp[NB];       // int4: (scale, zero)
    uint4_t bf[NB][4];     // fp16: 4 K-steps x 8 halves per lane and column block
    auto load_b = [&](int grp) {
#pragma unroll
        for (int j = 0; j < NB; j++) {
            const int nb = nb_base + j;
            if constexpr (INT4) {
                if (nb * 32 < g.N) {
                    const int64_t blk = (int64_t)nb * KG + grp;
                    bw[j] = *reinterpret_cast<const uint4_t *>(g.wc + (blk * 64 + lane) * 4);
                    bp[j] = g.wp[blk * 32 + (lane & 31)];
                } else {
                    bw[j] = (uint4_t){0u, 0u, 0u, 0u};
                    bp[j] = 0u;
                }
            } else {
                int n = nb * 32 + (lane & 31);
                n = n < g.N ? n : g.N - 1;
                const uint16_t *p = g.wf + (int64_t)n * g.K + grp * KG_ELEMS + (lane >> 5) * 8;
#pragma unroll
                for (int t = 0; t < 4; t++)
                    bf[j][t] = *reinterpret_cast<const uint4_t *>(p + 16 * t);
            }
        }
    };

    float16_t acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; i++)
#pragma unroll
        for (int j = 0; j < NB; j++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                acc[i][j][r] = 0.0f;

    if (g0 < g1) {
        load_a(g0);
        store_a(0);
        load_b(g0);
        __syncthreads();
    }
    for (int grp = g0; grp < g1; grp++) {
        const int buf = (grp - g0) & 1;
        const bool next = grp + 1 < g1;
        uint4_t bw_cur[NB];
        uint32_t bp_cur[NB];
        uint4_t bf_cur[NB][4];
#pragma unroll
        for (int j = 0; j < NB; j++) {
            if constexpr (INT4) {
                bw_cur[j] = bw[j];
                bp_cur[j] = bp[j];
            } else {
#pragma unroll
                for (int t = 0; t < 4; t++)
                    bf_cur[j][t] = bf[j][t];
            }
        }
        if (next) {
            load_a(grp + 1);
            load_b(grp + 1);
        }
        const uint8_t *abuf = smem + buf * BM * 128;
#pragma unroll
        for (int t = 0; t < 4; t++) {
            half8_t bop[NB];
#pragma unroll
            for (int j = 0; j < NB; j++) {
                if constexpr (INT4) {
                    const half2_t s2 = __builtin_bit_cast(half2_t, (bp_cur[j] & 0xffffu) * 0x10001u);
                    const half2_t z2 = __builtin_bit_cast(half2_t, (bp_cur[j] >> 16) * 0x10001u);
                    bop[j] = dequant_word(bw_cur[j][t], s2, z2);
                } else {
                    bop[j] = __builtin_bit_cast(half8_t, bf_cur[j][t]);
                }
            }
#pragma unroll
            for (int i = 0; i < MB; i++) {
                const int row = wm * WM + i * 32 + (lane & 31);
                const int ch = 2 * t + (lane >> 5);
                const half8_t aop = *reinterpret_cast<const half8_t *>(abuf + row * 128 + ((ch ^ (row & 7)) << 4));
#pragma unroll
                for (int j = 0; j < NB; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop, bop[j], acc[i][j], 0, 0, 0);
            }
        }
        if (next)
            store_a(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds D[i][n] for n = lane%32, i = (r/4)*8 + (lane/32)*4 + r%4
#pragma unroll
    for (int i = 0; i < MB; i++)
#pragma unroll
        for (int j = 0; j < NB; j++) {
            const int col = n0 + wn * WN + j * 32 + (lane & 31);
            if (col >= g.N)
                continue;
            float bias = 0.0f;
            if (tm.splits == 1 && g.bias && g.epi != EPI_NONE)
                bias = h2f(g.bias[col]);
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int row = m0 + wm * WM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (row >= g.M)
                    continue;
                float v = acc[i][j][r];
                if (tm.splits > 1) {
                    g.ws[((int64_t)split * g.M + row) * g.N + col] = v;
                } else {
                    v += bias;
                    if (g.epi == EPI_BIAS_RES)
                        v += h2f(g.residual[(int64_t)row * g.ldc + col]);
                    if (g.epi == EPI_BIAS_RELU)
                        v = fmaxf(v, 0.0f);
                    g.y[(int64_t)row * g.ldc + col] = f2h(v);
                }
            }
        }
}

__global__ void __launch_bounds__(256) k_splitk_reduce(GemmArgs g, int splits)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)g.M * g.N)
        return;
    const int row = (int)(i / g.N), col = (int)(i % g.N);
    float v = 0.0f;
    for (int s = 0; s < splits; s++)
        v += g.ws[(int64_t)s * g.M * g.N + i];
    if (g.bias && g.epi != EPI_NONE)
        v += h2f(g.bias[col]);
    if (g.epi == EPI_BIAS_RES)
        v += h2f(g.residual[(int64_t)row * g.ldc + col]);
    if (g.epi == EPI_BIAS_RELU)
        v = fmaxf(v, 0.0f);
    g.y[(int64_t)row * g.ldc + col] = f2h(v);
}

struct Plan {
    int bm, bn;
    TileMap tm;
};

Plan plan_gemm(int M, int N, int K)
{
    Plan p;
    if (M <= 64) {
        p.bm = 64;
        p.bn = 64;
    } else if (M <= 128) {
        p.bm = 128;
        p.bn = 128;
    } else {
        p.bm = 256;
        p.bn = 128;
    }
    const int KG = K / KG_ELEMS;
    p.tm.mt = (M + p.bm - 1) / p.bm;
    p.tm.nt = (N + p.bn - 1) / p.bn;
    const int tiles = p.tm.mt * p.tm.nt;
    int splits = 1;
    while (tiles * splits < 384 && KG / (splits * 2) >= 8)
        splits *= 2;
    p.tm.groups_per_split = (KG + splits - 1) / splits;
    p.tm.splits = (KG + p.tm.groups_per_split - 1) / p.tm.groups_per_split;
    p.tm.total = tiles * p.tm.splits;
    return p;
}

} // namespace

size_t gemm_workspace_bytes(int M, int N, int K, bool)
{
    const Plan p = plan_gemm(M, N, K);
    return p.tm.splits > 1 ? (size_t)p.tm.splits * M * N * sizeof(float) : 0;
}

hipError_t launch_gemm(const GemmArgs &g, hipStream_t st)
{
    if (g.M <= 0 || g.N <= 0)
        return hipSuccess;
    const bool int4 = g.wc != nullptr;
    Plan p = plan_gemm(g.M, g.N, g.K);
    const size_t need = p.tm.splits > 1 ? (size_t)p.tm.splits * g.M * g.N * sizeof(float) : 0;
    if (need > g.ws_bytes || (need && !g.ws)) {
        // no room for partials: run unsplit
        p.tm.splits = 1;
        p.tm.groups_per_split = g.K / KG_ELEMS;
        p.tm.total = p.tm.mt * p.tm.nt;
    }
    const dim3 grid(p.tm.total), block(256);
#define TOD_GEMM_CASE(BM_, BN_)                                                                      \
    if (p.bm == BM_ && p.bn == BN_) {                                                                \
        if (int4)                                                                                    \
            hipLaunchKernelGGL((k_gemm<BM_, BN_, true>), grid, block, 0, st, g, p.tm);               \
        else                                                                                         \
            hipLaunchKernelGGL((k_gemm<BM_, BN_, false>), grid, block, 0, st, g, p.tm);              \
    }
    TOD_GEMM_CASE(64, 64)
    TOD_GEMM_CASE(128, 128)
    TOD_GEMM_CASE(256, 128)
#undef TOD_GEMM_CASE
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.tm.splits == 1)
        return e;
    const int64_t n = (int64_t)g.M * g.N;
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, g, p.tm.splits);
    return hipGetLastError();
}
