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
// gfx950 design (two kernels, fp32 accumulation in v_mfma_f32_32x32x16_f16):
//  * k_gemm_w4_256 / _192 / _128 (int4 weights; the decode and prefill path
//    above 128 rows): 256-, 192- or 128-row x 256 tiles, eight wavefronts,
//    activations, codes and params fed through a 3-stage LDS ring by
//    direct-to-LDS loads; described at the kernel body (gemm_w4_body).
//    k_gemm_f16_256 is the same body on fp16 weights (LM head, fp16 host
//    tier): the weight tile is staged like the activation tile, in a 2-stage
//    ring.
//    At 128 rows or fewer the same bodies run on 128- or 64-row tiles (int4,
//    two workgroups per CU) and 64-row tiles (fp16).
//    The QKV GEMM can quantize and append the rows' K and V to the int4 KV
//    cache in its epilogue instead of storing them (k_gemm_w4_*a for a decode
//    step, k_gemm_w4_*r for prefill's runs of one sequence's positions).
//  * k_gemm (small GEMMs of 128 rows or fewer that would give the pipelined
//    kernel fewer than 128 workgroups; fp16 weights whose N is not a
//    multiple of 32): 256-thread
//    workgroups as a 2x2 grid of wavefronts, each owning a (BM/2) x (BN/2)
//    output tile; the activation tile (BM x 64, one K-group) is
//    double-buffered in LDS with 16-byte chunks XOR-swizzled by row, and
//    weights go from HBM straight to registers.
//  * The int4 store is pre-tiled so that one 16-byte load brings exactly the
//    32 nibbles a lane feeds to four MFMA K-steps as its B operand.
//  * Dequantization (dequant_word): masked nibbles become exact fp16 codes by
//    one fp8 -> fp16 convert per pair, then one v_pk_fma_f16 with (scale,
//    zero) rounds once, so each weight equals fp16(zero + c*scale).
//  * Workgroup ids are remapped so that each XCD (ids round-robin over 8 XCDs)
//    gets a contiguous run of tiles, ordered in groups of four row tiles
//    (rows fastest, then columns): the workgroups an XCD runs at once share a
//    few activation tiles and a few weight tiles in its L2.
//  * When the tile grid is too small to fill 256 CUs the K loop is split and
//    fp32 partials are reduced by a second kernel (deterministic order).
#include <cstdio>
#include <cstdlib>

#include "common.hpp"

namespace {

constexpr int KG_ELEMS = 64; // K elements per main-loop iteration (one quant group)

struct TileMap {
    int mt, nt, splits, groups_per_split, total;
    int group_m; // row tiles per group of the tile order (tile_coords)
};

__device__ __forceinline__ int xcd_tile(int b, int total)
{
    // Workgroup b runs on XCD b % 8 as the (b / 8)-th of that XCD; give each XCD a
    // contiguous range of tile ids.
    const int x = b & 7, k = b >> 3, q = total >> 3, r = total & 7;
    return x * q + (x < r ? x : r) + k;
}

// Tile id -> (row tile, column tile, K split). Within a split, ids run over groups of
// tm.group_m row tiles: row fastest inside a group, then column, then the next group.
// The workgroups an XCD runs at once (consecutive ids) then share a few activation
// tiles and a few weight tiles in its L2; with every row tile in one group (as in
// decode) this is plain row-fastest order.
__device__ __forceinline__ void tile_coords(int tile, const TileMap &tm, int &m_tile, int &n_tile, int &split)
{
    const int per_split = tm.mt * tm.nt;
    split = tile / per_split;
    const int t = tile - split * per_split;
    const int per_group = tm.group_m * tm.nt;
    const int group = t / per_group, first = group * tm.group_m;
    const int rows = min(tm.mt - first, tm.group_m);
    const int u = t - group * per_group;
    m_tile = first + u % rows;
    n_tile = u / rows;
}

// Eight weights of one tiled word (nibble slots 0,2,4,6 hold e0..e3 and slots
// 1,3,5,7 hold e4..e7, see tiled_word_from_canonical). A byte 0000cccc read as
// fp8 e4m3 is exactly c * 2^-9 (subnormal for c < 8, exponent 1 above), so one
// v_cvt_scalef32_pk_f16_fp8 with scale 2^9 turns two masked bytes into two
// exact fp16 codes; one v_pk_fma_f16 with (scale, zero) then rounds once, so
// each weight equals fp16(zero + c*scale).
__device__ __forceinline__ half8_t dequant_word(uint32_t w, half2_t s2, half2_t z2)
{
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    const half2_t c01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, false);
    const half2_t c23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, true);
    const half2_t c45 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, false);
    const half2_t c67 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, true);
    const half2_t x01 = __builtin_elementwise_fma(c01, s2, z2);
    const half2_t x23 = __builtin_elementwise_fma(c23, s2, z2);
    const half2_t x45 = __builtin_elementwise_fma(c45, s2, z2);
    const half2_t x67 = __builtin_elementwise_fma(c67, s2, z2);
    return (half8_t){x01[0], x01[1], x23[0], x23[1], x45[0], x45[1], x67[0], x67[1]};
}

template <int BM, int BN, bool INT4, int MINW>
__global__ void __launch_bounds__(256, MINW) k_gemm(GemmArgs g, TileMap tm)
{
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int MB = WM / 32, NB = WN / 32;
    constexpr int A_LOADS = BM * 8 / 256; // 16-byte chunks per thread per group
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * BM * 128];

    const int tile = xcd_tile(blockIdx.x, tm.total);
    if (tile >= tm.total)
        return;
    int m_tile, n_tile, split;
    tile_coords(tile, tm, m_tile, n_tile, split);
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

// ---------------------------------------------------------------------------
// Pipelined GEMM (int4 weights, and fp16 weights whose N is a multiple of 32):
// BM x 256 workgroup tiles (BM = 256, 192, 128 or 64, chosen by plan_gemm),
// eight wavefronts as a 2 x 4 grid of BM/2 x 64 wave tiles, fed through an LDS
// ring (S stages) that direct-to-LDS loads (global_load_lds_dwordx4) fill
// S - 1 K-groups ahead of the MFMAs, so the weight stream's HBM latency is
// covered without staging registers. With two waves per SIMD one wave's LDS
// reads and dequantization run while the other's MFMAs issue. Stage
// synchronisation is an explicit vmcnt wait on the wave's own loads plus a
// workgroup barrier.
// ---------------------------------------------------------------------------
// F16: fp16 weights W[N][K] instead of int4 codes. W's tile (BN rows x 64 fp16)
// has the layout of the A tile and the MFMA B fragment is read exactly as an A
// fragment; at 256 rows both tiles need 64 KiB per stage, so that ring has two
// stages (the 64-row tile keeps three).
template <int BM_, bool F16 = false, int S_ = 0> struct W4 {
    static constexpr int BM = BM_, BN = 256, WAVES = 8;
    static constexpr int RB = BM / 2;                   // rows per wave (2 wave rows)
    static constexpr int MB = RB / 32;                  // 32-row blocks per wave
    static constexpr int NB = 2;                        // 32-column blocks per wave (4 wave columns)
    static constexpr int A_BYTES = BM * 128;            // BM rows x 64 fp16, 16-byte chunks swizzled by row
    // int4: per column block 64 lanes x 16 B of codes; fp16: BN rows x 64 fp16 like A
    static constexpr int W_BYTES = F16 ? BN * 128 : (BN / 32) * 1024;
    static constexpr int P_BYTES = F16 ? 0 : (BN / 32) * 256; // per column block: 64 x (scale, zero)
    static constexpr int STAGE = A_BYTES + W_BYTES + P_BYTES;
    static constexpr int S = S_ ? S_ : F16 ? 2 : 3;     // ring stages
    static constexpr int AL = (BM / 8) / WAVES;         // 1 KiB A chunks (8 rows) loaded per wave per stage
    static constexpr int WL = F16 ? (BN / 8) / WAVES : 0; // fp16: 1 KiB W chunks per wave per stage
    // loads per wave per stage: A chunks, W chunks or codes and params
    static constexpr int LPS = AL + (F16 ? WL : 2);
    static_assert(BM % 64 == 0 && (BM / 8) % WAVES == 0, "A chunks split evenly over the waves");
};

typedef __attribute__((address_space(3))) void lds_void;

// LDS position of 16-byte chunk `ch` (0..7) of A-tile row `row`: XOR with a row
// hash that is a bijection on every 8 consecutive rows and, across 16 rows,
// on the even and on the odd rows separately, so that 8- and 16-lane phases of
// a ds_read_b128 (rows r..r+15, one chunk column) touch distinct banks.
__device__ __forceinline__ int a_pos(int row, int ch) { return ch ^ ((row ^ (row >> 3)) & 7); }

// Wait until at most `younger` stages' worth (LPS loads each) of this wave's
// vector-memory loads are outstanding (0 <= younger <= S - 2).
template <int N_>
__device__ __forceinline__ void wait_vmcnt()
{
    // s_waitcnt simm16 on gfx9: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]
    static_assert(N_ < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt((N_ & 15) | ((N_ >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int LPS_, int S_>
__device__ __forceinline__ void wait_vm_loads(int younger)
{
    static_assert(S_ >= 2 && S_ <= 4, "two to four ring stages");
    if (S_ == 4 && younger >= 2)
        wait_vmcnt<(S_ == 4 ? 2 * LPS_ : 0)>();
    else if (S_ >= 3 && younger >= 1)
        wait_vmcnt<(S_ >= 3 ? LPS_ : 0)>();
    else
        wait_vmcnt<0>();
}

// Fused K/V append of the QKV GEMM's epilogue: this lane holds columns gb + c0 .. +15 (a)
// and gb + 32 + c0 .. +15 (b) of one row, fp16 after the bias; its partner (lane ^ 1) holds
// the other 32 columns of the 64-column group gb. Quantized exactly as the KV-append
// kernel does (the same group_quant and code_of on the same fp16 values) and stored in the
// cache's canonical layout. RUNS: rows come in runs of g.kv_rows_per_seq positions of one
// sequence (prefill); otherwise each row is its own sequence (a decode step).
template <bool RUNS>
__device__ __forceinline__ void qkv_append(const GemmArgs &g, int grow, int gb, int c0, half8_t a0, half8_t a1,
                                           half8_t b0, half8_t b1)
{
    float x[32];
#pragma unroll
    for (int e = 0; e < 8; e++) {
        x[e] = (float)a0[e];
        x[8 + e] = (float)a1[e];
        x[16 + e] = (float)b0[e];
        x[24 + e] = (float)b1[e];
    }
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int e = 1; e < 32; e++) {
        mn = fminf(mn, x[e]);
        mx = fmaxf(mx, x[e]);
    }
    mn = fminf(mn, __shfl_xor(mn, 1, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
    const GroupQ q = group_quant(mn, mx);
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 8; e++)
            word |= (uint32_t)code_of(x[8 * k + e], q) << (4 * e); // byte b: elements 2b, 2b + 1
        w[k] = word;
    }
    const int d = g.kv.head_dim, h = g.kv.heads * d;
    const int rel = gb - g.kv_col0, isv = rel >= h ? 1 : 0, within = rel - isv * h;
    const int head = within / d, grp = (within % d) / 64;
    const int seq = RUNS ? grow / g.kv_rows_per_seq : grow, off = RUNS ? grow - seq * g.kv_rows_per_seq : 0;
    const int pos = (g.kv_dpos ? *g.kv_dpos : g.kv_pos0) + off;
    const size_t at = kv_slab(g.kv, g.kv_seq0 + seq, head) * g.kv.cap + pos;
    const size_t cofs = at * (d / 2) + grp * 32 + c0 / 2, pofs = at * (d / 64) + grp;
    const uint32_t param = (uint32_t)q.scale | ((uint32_t)q.zero << 16);
    uint8_t *codes = isv ? g.kv.vc : g.kv.kc;
    *reinterpret_cast<uint2_t *>(codes + cofs) = (uint2_t){w[0], w[1]};
    *reinterpret_cast<uint2_t *>(codes + cofs + 16) = (uint2_t){w[2], w[3]};
    if (c0 == 0)
        (isv ? g.kv.vp : g.kv.kp)[pofs] = param;
    if (g.kv_mirror.kc) { // the same bytes into the pinned host copy of the cache
        uint8_t *mc = isv ? g.kv_mirror.vc : g.kv_mirror.kc;
        *reinterpret_cast<uint2_t *>(mc + cofs) = (uint2_t){w[0], w[1]};
        *reinterpret_cast<uint2_t *>(mc + cofs + 16) = (uint2_t){w[2], w[3]};
        if (c0 == 0)
            (isv ? g.kv_mirror.vp : g.kv_mirror.kp)[pofs] = param;
    }
}

template <int BM_, bool F16, int S_ = 0, int APPEND = 0>
__device__ __forceinline__ void gemm_w4_body(const GemmArgs &g, const TileMap &tm)
{
    using C = W4<BM_, F16, S_>;
    constexpr int BM = C::BM, BN = C::BN, WAVES = C::WAVES, RB = C::RB, MB = C::MB, NB = C::NB;
    constexpr int A_BYTES = C::A_BYTES, W_BYTES = C::W_BYTES, STAGE = C::STAGE, S = C::S, AL = C::AL;
    constexpr int WL = C::WL;
    __shared__ __attribute__((aligned(16))) uint8_t smem[S * STAGE];

    const int tile = xcd_tile(blockIdx.x, tm.total);
    if (tile >= tm.total)
        return;
    int m_tile, n_tile, split;
    tile_coords(tile, tm, m_tile, n_tile, split);
    const int m0 = m_tile * BM, n0 = n_tile * BN;
    const int KG = g.K / KG_ELEMS;
    const int g0 = split * tm.groups_per_split;
    const int g1 = min(KG, g0 + tm.groups_per_split);
    const int nst = g1 - g0;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3; // wave tile: rows wm*128.., column blocks wn*2..

    // Loads of one stage: wave w brings A chunks w, w+8, w+16, w+24 (8 rows
    // each), and the codes and params of column block w. Per-lane byte offsets
    // are fixed for the whole K loop; the per-group part of each address is
    // wave-uniform, so the LDS destinations (m0) are scalar.
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    uint32_t a_off[AL];
#pragma unroll
    for (int i = 0; i < AL; i++) {
        const int row = 8 * (wv + WAVES * i) + (lane >> 3);
        const int ch = a_pos(row, lane & 7); // global chunk landing at LDS position lane & 7
        const int m = min(m0 + row, g.M - 1);
        a_off[i] = (uint32_t)((m - m0) * g.lda + ch * 8) * 2u;
    }
    const int nbw = min((n0 >> 5) + wv, (g.N >> 5) - 1); // clamped: blocks past N feed discarded columns
    const uint8_t *a_tile = reinterpret_cast<const uint8_t *>(g.a + (int64_t)m0 * g.lda);
    const uint8_t *wc8 = reinterpret_cast<const uint8_t *>(g.wc);
    const uint8_t *wp8 = reinterpret_cast<const uint8_t *>(g.wp);
    // fp16 weights: W-tile rows as A-tile rows (clamped: rows past N feed discarded columns)
    uint32_t w_off[WL > 0 ? WL : 1];
    const uint8_t *w_tile = nullptr;
    if constexpr (F16) {
#pragma unroll
        for (int i = 0; i < WL; i++) {
            const int row = 8 * (wv + WAVES * i) + (lane >> 3);
            const int n = min(n0 + row, g.N - 1);
            w_off[i] = (uint32_t)((n - n0) * g.K + a_pos(row, lane & 7) * 8) * 2u;
        }
        w_tile = reinterpret_cast<const uint8_t *>(g.wf + (int64_t)n0 * g.K);
    }

    auto issue = [&](int buf, int grp) {
        uint8_t *base = smem + buf * STAGE;
        const uint8_t *ag = a_tile + grp * (KG_ELEMS * 2);
#pragma unroll
        for (int i = 0; i < AL; i++)
            __builtin_amdgcn_global_load_lds(ag + a_off[i], (lds_void *)(base + (wv + WAVES * i) * 1024), 16, 0, 0);
        if constexpr (F16) {
            const uint8_t *wg = w_tile + grp * (KG_ELEMS * 2);
#pragma unroll
            for (int i = 0; i < WL; i++)
                __builtin_amdgcn_global_load_lds(wg + w_off[i], (lds_void *)(base + A_BYTES + (wv + WAVES * i) * 1024),
                                                 16, 0, 0);
        } else {
            const int64_t blk = (int64_t)nbw * KG + grp;
            __builtin_amdgcn_global_load_lds(wc8 + blk * 1024 + lane * 16, (lds_void *)(base + A_BYTES + wv * 1024),
                                             16, 0, 0);
            __builtin_amdgcn_global_load_lds(wp8 + blk * 128 + (lane & 31) * 4,
                                             (lds_void *)(base + A_BYTES + W_BYTES + wv * 256), 4, 0, 0);
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

#pragma unroll
    for (int s_ = 0; s_ < S - 1; s_++)
        if (s_ < nst)
            issue(s_, g0 + s_);

    // One K-group is four K-steps of 16. In each step the A operands of the next
    // step (LDS) and its B operands are produced before this step's MFMAs.
    const uint8_t *base = smem;
    uint4_t bw[NB];
    half2_t s2[NB], z2[NB];
    half8_t a_cur[MB], b_cur[NB];
    auto a_frag = [&](int i, int t) -> half8_t {
        const int row = wm * RB + i * 32 + (lane & 31);
        return *reinterpret_cast<const half8_t *>(base + row * 128 + (a_pos(row, 2 * t + (lane >> 5)) << 4));
    };
    // B operand of column block j at K-step t: dequantized codes, or the fp16
    // W-tile fragment read like an A fragment
    auto b_frag = [&](int j, int t) -> half8_t {
        if constexpr (F16) {
            const int row = (wn * NB + j) * 32 + (lane & 31);
            return *reinterpret_cast<const half8_t *>(base + A_BYTES + row * 128 +
                                                      (a_pos(row, 2 * t + (lane >> 5)) << 4));
        } else {
            return dequant_word(bw[j][t], s2[j], z2[j]);
        }
    };
    // K-group `it` of this split: its ring stage, its weight words and the operands of step 0
    auto begin_group = [&](int it) {
        base = smem + (it % S) * STAGE;
        if constexpr (!F16) {
#pragma unroll
            for (int j = 0; j < NB; j++) {
                const int cb = wn * NB + j;
                bw[j] = *reinterpret_cast<const uint4_t *>(base + A_BYTES + cb * 1024 + lane * 16);
                const uint32_t bp =
                    *reinterpret_cast<const uint32_t *>(base + A_BYTES + W_BYTES + cb * 256 + (lane & 31) * 4);
                s2[j] = __builtin_bit_cast(half2_t, (bp & 0xffffu) * 0x10001u);
                z2[j] = __builtin_bit_cast(half2_t, (bp >> 16) * 0x10001u);
            }
        }
#pragma unroll
        for (int i = 0; i < MB; i++)
            a_cur[i] = a_frag(i, 0);
#pragma unroll
        for (int j = 0; j < NB; j++)
            b_cur[j] = b_frag(j, 0);
    };
    auto k_step = [&](int t) {
        half8_t a_nxt[MB], b_nxt[NB];
        if (t < 3) {
#pragma unroll
            for (int i = 0; i < MB; i++)
                a_nxt[i] = a_frag(i, t + 1);
            // one workgroup per CU (int4, 192 or 256 rows): keep the next step's A reads ahead of
            // this step's MFMAs; left alone, the compiler sinks each next to its first use
            if constexpr (!F16 && BM >= 192)
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < NB; j++)
                b_nxt[j] = b_frag(j, t + 1);
        }
#pragma unroll
        for (int i = 0; i < MB; i++)
#pragma unroll
            for (int j = 0; j < NB; j++)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_cur[i], b_cur[j], acc[i][j], 0, 0, 0);
        if (t < 3) {
#pragma unroll
            for (int i = 0; i < MB; i++)
                a_cur[i] = a_nxt[i];
#pragma unroll
            for (int j = 0; j < NB; j++)
                b_cur[j] = b_nxt[j];
        }
    };

    for (int it = 0; it < nst; it++) {
        wait_vm_loads<C::LPS, S>(min(S - 2, nst - 1 - it));
        __builtin_amdgcn_s_barrier();
        if (it + S - 1 < nst)
            issue((it + S - 1) % S, g0 + it + S - 1);
        begin_group(it);
#pragma unroll
        for (int t = 0; t < 4; t++)
            k_step(t);
    }

    // Epilogue through LDS: each 32 x 32 accumulator block goes to a per-wave
    // scratch tile in the MFMA lane layout and comes back as 16 consecutive
    // columns of one row per lane, so bias, residual and output move in 32-byte
    // runs. The ring is free once every wave has left the main loop.
    __syncthreads();
    constexpr int SROW = 36; // padded scratch row (floats)
    static_assert(WAVES * 32 * SROW * 4 <= S * STAGE, "scratch fits the ring");
    float *scr = reinterpret_cast<float *>(smem) + wave * 32 * SROW;
    const int lr = lane >> 1, c0 = (lane & 1) * 16;
    // APPEND: the wave's 64 columns are one quantization group of K or V (the QKV
    // output's K and V start at a multiple of 64); column block 0's values wait here
    static_assert(!APPEND || NB == 2, "one 64-column group per wave");
    const bool kv_group = APPEND != 0 && n0 + wn * NB * 32 >= g.kv_col0;
    half8_t hold[APPEND ? MB : 1][2];
#pragma unroll
    for (int j = 0; j < NB; j++) {
        const int gcol = n0 + (wn * NB + j) * 32 + c0;
        const bool colok = gcol < g.N; // N is a multiple of 32 on this path
        float bias[16];
#pragma unroll
        for (int e = 0; e < 16; e++)
            bias[e] = 0.0f;
        if (colok && tm.splits == 1 && g.bias && g.epi != EPI_NONE) {
            const uint4_t b0 = *reinterpret_cast<const uint4_t *>(g.bias + gcol);
            const uint4_t b1 = *reinterpret_cast<const uint4_t *>(g.bias + gcol + 8);
            const half8_t h0 = __builtin_bit_cast(half8_t, b0), h1 = __builtin_bit_cast(half8_t, b1);
#pragma unroll
            for (int e = 0; e < 8; e++) {
                bias[e] = (float)h0[e];
                bias[8 + e] = (float)h1[e];
            }
        }
#pragma unroll
        for (int i = 0; i < MB; i++) {
#pragma unroll
            for (int r = 0; r < 16; r++)
                scr[((r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)) * SROW + (lane & 31)] = acc[i][j][r];
            __builtin_amdgcn_s_waitcnt((7 << 4) | (0 << 8) | 0xc00f); // lgkmcnt(0): scratch written
            __builtin_amdgcn_wave_barrier();
            float v[16];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const float4_t f = *reinterpret_cast<const float4_t *>(scr + lr * SROW + c0 + 4 * q);
                v[4 * q] = f[0];
                v[4 * q + 1] = f[1];
                v[4 * q + 2] = f[2];
                v[4 * q + 3] = f[3];
            }
            __builtin_amdgcn_s_waitcnt((7 << 4) | (0 << 8) | 0xc00f); // lgkmcnt(0): scratch read
            __builtin_amdgcn_wave_barrier();
            const int grow = m0 + wm * RB + i * 32 + lr;
            if (!colok || grow >= g.M)
                continue;
            if (tm.splits > 1) {
                float *dst = g.ws + ((int64_t)split * g.M + grow) * g.N + gcol;
#pragma unroll
                for (int q = 0; q < 4; q++)
                    *reinterpret_cast<float4_t *>(dst + 4 * q) =
                        (float4_t){v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
                continue;
            }
            half8_t res0 = {}, res1 = {};
            if (g.epi == EPI_BIAS_RES) {
                const uint16_t *rp = g.residual + (int64_t)grow * g.ldc + gcol;
                res0 = __builtin_bit_cast(half8_t, *reinterpret_cast<const uint4_t *>(rp));
                res1 = __builtin_bit_cast(half8_t, *reinterpret_cast<const uint4_t *>(rp + 8));
            }
            half8_t o0, o1;
#pragma unroll
            for (int e = 0; e < 16; e++) {
                float x = v[e] + bias[e];
                if (g.epi == EPI_BIAS_RES)
                    x += (float)(e < 8 ? res0[e] : res1[e - 8]);
                if (g.epi == EPI_BIAS_RELU)
                    x = fmaxf(x, 0.0f);
                if (e < 8)
                    o0[e] = (half_t)x;
                else
                    o1[e - 8] = (half_t)x;
            }
            if (kv_group) {
                if (j == 0) {
                    hold[i][0] = o0;
                    hold[i][1] = o1;
                } else {
                    qkv_append<APPEND == 2>(g, grow, n0 + wn * NB * 32, c0, hold[i][0], hold[i][1], o0, o1);
                }
                continue;
            }
            uint16_t *yp = g.y + (int64_t)grow * g.ldc + gcol;
            *reinterpret_cast<uint4_t *>(yp) = __builtin_bit_cast(uint4_t, o0);
            *reinterpret_cast<uint4_t *>(yp + 8) = __builtin_bit_cast(uint4_t, o1);
        }
    }
}

__global__ void __launch_bounds__(512, 1) k_gemm_w4_256(GemmArgs g, TileMap tm) { gemm_w4_body<256, false>(g, tm); }
__global__ void __launch_bounds__(512, 1) k_gemm_w4_192(GemmArgs g, TileMap tm) { gemm_w4_body<192, false>(g, tm); }
__global__ void __launch_bounds__(512, 1) k_gemm_f16_256(GemmArgs g, TileMap tm) { gemm_w4_body<256, true>(g, tm); }
// 128 rows or fewer: short tiles, two workgroups per CU where LDS and registers allow
__global__ void __launch_bounds__(512, 2) k_gemm_w4_128(GemmArgs g, TileMap tm) { gemm_w4_body<128, false>(g, tm); }
__global__ void __launch_bounds__(512, 2) k_gemm_w4_64(GemmArgs g, TileMap tm) { gemm_w4_body<64, false>(g, tm); }
// the QKV GEMM with the K/V append in its epilogue (EPI_QKV_APPEND): a decode step (one
// position per sequence), and prefill (rows in runs of one sequence's positions)
__global__ void __launch_bounds__(512, 1) k_gemm_w4_256a(GemmArgs g, TileMap tm)
{
    gemm_w4_body<256, false, 0, 1>(g, tm);
}
__global__ void __launch_bounds__(512, 1) k_gemm_w4_192a(GemmArgs g, TileMap tm)
{
    gemm_w4_body<192, false, 0, 1>(g, tm);
}
__global__ void __launch_bounds__(512, 2) k_gemm_w4_128a(GemmArgs g, TileMap tm)
{
    gemm_w4_body<128, false, 0, 1>(g, tm);
}
__global__ void __launch_bounds__(512, 2) k_gemm_w4_64a(GemmArgs g, TileMap tm)
{
    gemm_w4_body<64, false, 0, 1>(g, tm);
}
__global__ void __launch_bounds__(512, 1) k_gemm_w4_256r(GemmArgs g, TileMap tm)
{
    gemm_w4_body<256, false, 0, 2>(g, tm);
}
__global__ void __launch_bounds__(512, 1) k_gemm_w4_192r(GemmArgs g, TileMap tm)
{
    gemm_w4_body<192, false, 0, 2>(g, tm);
}
__global__ void __launch_bounds__(512, 2) k_gemm_w4_128r(GemmArgs g, TileMap tm)
{
    gemm_w4_body<128, false, 0, 2>(g, tm);
}
__global__ void __launch_bounds__(512, 2) k_gemm_w4_64r(GemmArgs g, TileMap tm)
{
    gemm_w4_body<64, false, 0, 2>(g, tm);
}
// fp16, 128 rows or fewer: bound by the weight stream, so a third stage in flight pays
__global__ void __launch_bounds__(512, 1) k_gemm_f16_64(GemmArgs g, TileMap tm) { gemm_w4_body<64, true, 3>(g, tm); }

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

// Split-K reduction fused with the LayerNorm of the output rows: one
// 256-thread workgroup per row, thread chunks c = t + 256k of 8 columns. Each
// output is summed over the splits, bias and residual added and rounded
// exactly as in k_splitk_reduce; the fp16 row stays in registers for
// layernorm_row, the same code as the LayerNorm kernel.
// SPLITS > 0: the split count is fixed at compile time and every partial, bias and residual
// word of the thread's chunks is loaded before the first add (a chunk past the row's end reads
// the row's last chunk again and is not used); the sums run in the same split order either way.
template <int K, int SPLITS = 0>
__global__ void __launch_bounds__(256) k_splitk_reduce_ln(GemmArgs g, int splits)
{
    __shared__ float red[8];
    const int row = blockIdx.x, nch = g.N >> 3;
    const int64_t mn = (int64_t)g.M * g.N;
    const bool has_bias = g.bias && g.epi != EPI_NONE, has_res = g.epi == EPI_BIAS_RES;
    constexpr int NS = SPLITS > 0 ? SPLITS : 1;
    float4_t pa[K][NS], pb[K][NS];
    uint4_t bw[K], rw[K];
    if constexpr (SPLITS > 0) {
#pragma unroll
        for (int k = 0; k < K; k++) {
            const int c = min((int)threadIdx.x + 256 * k, nch - 1);
            const int64_t i0 = (int64_t)row * g.N + 8 * c;
#pragma unroll
            for (int sp = 0; sp < SPLITS; sp++) {
                pa[k][sp] = *reinterpret_cast<const float4_t *>(g.ws + sp * mn + i0);
                pb[k][sp] = *reinterpret_cast<const float4_t *>(g.ws + sp * mn + i0 + 4);
            }
            bw[k] = has_bias ? *reinterpret_cast<const uint4_t *>(g.bias + 8 * c) : (uint4_t){0u, 0u, 0u, 0u};
            rw[k] = has_res ? *reinterpret_cast<const uint4_t *>(g.residual + (int64_t)row * g.ldc + 8 * c)
                            : (uint4_t){0u, 0u, 0u, 0u};
        }
    }
    uint4_t v[K];
#pragma unroll
    for (int k = 0; k < K; k++) {
        const int c = threadIdx.x + 256 * k;
        v[k] = (uint4_t){0u, 0u, 0u, 0u};
        if (c >= nch)
            continue;
        const int64_t i0 = (int64_t)row * g.N + 8 * c;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; e++)
            x[e] = 0.0f;
        half8_t bias = {}, res = {};
        if constexpr (SPLITS > 0) {
#pragma unroll
            for (int sp = 0; sp < SPLITS; sp++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    x[e] += pa[k][sp][e];
                    x[4 + e] += pb[k][sp][e];
                }
            bias = __builtin_bit_cast(half8_t, bw[k]);
            res = __builtin_bit_cast(half8_t, rw[k]);
        } else {
            for (int sp = 0; sp < splits; sp++) {
                const float4_t p0 = *reinterpret_cast<const float4_t *>(g.ws + sp * mn + i0);
                const float4_t p1 = *reinterpret_cast<const float4_t *>(g.ws + sp * mn + i0 + 4);
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    x[e] += p0[e];
                    x[4 + e] += p1[e];
                }
            }
            if (has_bias)
                bias = __builtin_bit_cast(half8_t, *reinterpret_cast<const uint4_t *>(g.bias + 8 * c));
            if (has_res)
                res = __builtin_bit_cast(half8_t,
                                         *reinterpret_cast<const uint4_t *>(g.residual + (int64_t)row * g.ldc + 8 * c));
        }
        half8_t o;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            float t = x[e];
            if (has_bias)
                t += (float)bias[e];
            if (has_res)
                t += (float)res[e];
            if (g.epi == EPI_BIAS_RELU)
                t = fmaxf(t, 0.0f);
            o[e] = (half_t)t;
        }
        v[k] = __builtin_bit_cast(uint4_t, o);
        *reinterpret_cast<uint4_t *>(g.y + (int64_t)row * g.ldc + 8 * c) = v[k];
    }
    layernorm_row<K>(v, nch, g.N, g.ln_g, g.ln_b, g.ln_y + (int64_t)row * g.N, red);
}

struct Plan {
    int bm, bn;
    bool pipelined;
    TileMap tm;
};

// Tuning overrides (read once): TOD_GEMM_SPLIT = workgroup count below which the K loop is
// split; TOD_GEMM_BM192 = 0 | 1 pins the pipelined int4 tile height above 128 rows to 256 | 192
// and TOD_GEMM_BIG_BM = 128 | 192 | 256 to any of them; TOD_GEMM_SMALL_BM = 64 | 128 pins it at
// 128 rows or fewer; TOD_GEMM_F16PIPE = 0 keeps fp16
// weights on the register-staged kernel; TOD_GEMM_TILE = "64x64" | "128x128" | "256x128" puts
// every GEMM on it with that tile for M > 64; TOD_GEMM_GROUP_M = row tiles per group of the
// tile order (default 4; a large value gives plain row-fastest order).
struct Tuning {
    int bm = 0, bn = 0, split_fill = -1;
    int bm192 = -1; // pipelined tile height: -1 cost model, 0 always 256, 1 always 192
    bool f16_pipe = true;   // fp16 weights on the pipelined kernel
    int small_bm = 0;       // pin the int4 tile height at 128 rows or fewer (64 or 128)
    int big_bm = 0;         // pin the int4 tile height above 128 rows (128, 192 or 256)
    int group_m = 4;        // row tiles per group of the tile order
    Tuning()
    {
        if (const char *t = getenv("TOD_GEMM_GROUP_M"))
            group_m = atoi(t) >= 1 ? atoi(t) : 4;
        if (const char *t = getenv("TOD_GEMM_SMALL_BM"))
            small_bm = atoi(t) == 64 || atoi(t) == 128 ? atoi(t) : 0;
        if (const char *t = getenv("TOD_GEMM_F16PIPE"))
            f16_pipe = atoi(t) != 0;
        if (const char *t = getenv("TOD_GEMM_BM192"))
            bm192 = atoi(t) > 0 ? 1 : atoi(t) == 0 ? 0 : -1;
        if (const char *t = getenv("TOD_GEMM_BIG_BM"))
            big_bm = atoi(t) == 128 || atoi(t) == 192 || atoi(t) == 256 ? atoi(t) : 0;
        if (const char *t = getenv("TOD_GEMM_TILE")) {
            int a = 0, b = 0;
            if (sscanf(t, "%dx%d", &a, &b) == 2 &&
                ((a == 64 && b == 64) || (a == 128 && b == 128) || (a == 256 && b == 128))) {
                bm = a;
                bn = b;
            }
        }
        if (const char *t = getenv("TOD_GEMM_SPLIT"))
            split_fill = atoi(t);
    }
};

const Tuning &tuning()
{
    static const Tuning t;
    return t;
}

// Tile grid for bm x bn tiles; the K loop is split (powers of two) while the
// workgroups would fill less than `fill` CUs.
Plan split_plan(int M, int N, int K, int bm, int bn, bool pipelined)
{
    const Tuning &tu = tuning();
    Plan p{};
    p.bm = bm;
    p.bn = bn;
    p.pipelined = pipelined;
    const int KG = K / KG_ELEMS;
    p.tm.mt = (M + bm - 1) / bm;
    p.tm.nt = (N + bn - 1) / bn;
    p.tm.group_m = tu.group_m;
    const int tiles = p.tm.mt * p.tm.nt;
    const int fill = tu.split_fill >= 0 ? tu.split_fill : (pipelined ? 160 : 384);
    int splits = 1;
    while (tiles * splits < fill && KG / (splits * 2) >= 8)
        splits *= 2;
    p.tm.groups_per_split = (KG + splits - 1) / splits;
    p.tm.splits = (KG + p.tm.groups_per_split - 1) / p.tm.groups_per_split;
    p.tm.total = tiles * p.tm.splits;
    return p;
}

// Predicted microseconds of a pipelined GEMM plan, used only to rank tile heights (the
// library's cost model prices launches with its own rates). Fitted on MI355X decode GEMMs:
// one K-group of a 256 x 256 tile takes 1.6 us while every CU runs one such workgroup, a
// K-group of a shorter tile takes its share of that times the tile's efficiency loss (128
// rows 1.1, 64 rows 1.5), each wave of resident workgroups (two per CU at 128 rows or fewer)
// adds 25 us of fill and epilogue, and split-K partials are written and read at 7.1 TB/s.
double pipelined_plan_us(const TileMap &tm, int bm, int M, int N)
{
    const double eff = bm <= 64 ? 1.5 : bm <= 128 ? 1.1 : 1.0;
    const int slots = bm <= 128 ? 512 : 256;
    double t = (double)((tm.total + 255) / 256) * tm.groups_per_split * (bm / 256.0) * 1.6 * eff +
               (double)((tm.total + slots - 1) / slots) * 25.0;
    if (tm.splits > 1)
        t += 2.0 * tm.splits * (double)M * N * 4.0 / 7.1e6;
    return t;
}

Plan plan_gemm(int M, int N, int K, bool int4)
{
    Plan p;
    const Tuning &tu = tuning();
    // the pipelined kernel unless fp16 N is not a multiple of 32 (or a tuning override)
    p.pipelined = !tu.bm && (int4 || (tu.f16_pipe && N % 32 == 0));
    if (p.pipelined) {
        // Tile height by predicted time (pipelined_plan_us): 256, 192 or 128 rows above
        // 128 rows, 128 or 64 at 128 rows or fewer; fp16 weights: 256 or 64 rows. Narrow N
        // is split along K instead of shrinking the tile below 256 columns.
        p.bn = 256;
        p.bm = 256;
        int cand[3] = {256, 192, 128};
        int nc = 3;
        if (!int4) {
            cand[0] = M > 128 ? 256 : 64;
            nc = 1;
        } else if (M <= 128) {
            cand[0] = 128;
            cand[1] = 64;
            nc = 2;
            if (tu.small_bm) {
                cand[0] = tu.small_bm;
                nc = 1;
            }
        } else if (tu.big_bm) {
            cand[0] = tu.big_bm;
            nc = 1;
        } else if (tu.bm192 >= 0) {
            cand[0] = tu.bm192 ? 192 : 256;
            nc = 1;
        }
        double best = -1.0;
        int wgs = 0;
        for (int c = 0; c < nc; c++) {
            const int bm = cand[c];
            const Plan q = split_plan(M, N, K, bm, 256, true);
            const double t = pipelined_plan_us(q.tm, bm, M, N);
            if (best < 0.0 || t < best) {
                best = t;
                p.bm = bm;
                wgs = q.tm.total;
            }
        }
        // a small GEMM at 128 rows or fewer whose 256-wide tiles would leave most CUs idle
        // (fewer than 128 workgroups) runs on the register-staged kernel's 64-wide tiles
        if (int4 && M <= 128 && wgs < 128)
            p.pipelined = false;
    }
    if (!p.pipelined) {
        // register-staged kernel: 64 x 64 tiles for a few rows, 128 x 128 above
        p.bm = p.bn = M <= 64 ? 64 : 128;
    }
    if (!p.pipelined && tu.bm && M > 64) {
        p.bm = tu.bm;
        p.bn = tu.bn;
    }
    const Plan q = split_plan(M, N, K, p.bm, p.bn, p.pipelined);
    p.tm = q.tm;
    return p;
}

} // namespace

size_t gemm_workspace_bytes(int M, int N, int K, bool int4)
{
    const Plan p = plan_gemm(M, N, K, int4);
    return p.tm.splits > 1 ? (size_t)p.tm.splits * M * N * sizeof(float) : 0;
}

GemmPlanInfo gemm_plan_info(int M, int N, int K, bool int4)
{
    const Plan p = plan_gemm(M, N, K, int4);
    GemmPlanInfo i;
    i.pipelined = p.pipelined;
    i.bm = p.bm;
    i.bn = p.bn;
    i.splits = p.tm.splits;
    i.groups_per_split = p.tm.groups_per_split;
    i.workgroups = p.tm.total;
    return i;
}

hipError_t launch_gemm(const GemmArgs &g, hipStream_t st)
{
    if (g.M <= 0 || g.N <= 0)
        return hipSuccess;
    if (g.ln_y && (g.ldc != g.N || g.N % 8 || g.N > 16384 || !g.ln_g || !g.ln_b))
        return hipErrorInvalidValue; // LayerNorm of the output needs dense rows of at most 16384
    const bool int4 = g.wc != nullptr;
    Plan p = plan_gemm(g.M, g.N, g.K, int4);
    const size_t need = p.tm.splits > 1 ? (size_t)p.tm.splits * g.M * g.N * sizeof(float) : 0;
    if (need > g.ws_bytes || (need && !g.ws)) {
        // no room for partials: run unsplit
        p.tm.splits = 1;
        p.tm.groups_per_split = g.K / KG_ELEMS;
        p.tm.total = p.tm.mt * p.tm.nt;
    }
    const dim3 grid(p.tm.total), block(256);
    const dim3 wg8(64 * W4<256>::WAVES); // every pipelined kernel runs eight wavefronts
    if (g.epi == EPI_QKV_APPEND) {
        // only where the caller checked the plan: int4 weights, pipelined, K loop not split
        if (!int4 || !p.pipelined || p.tm.splits != 1 || g.kv_col0 % 64 || g.kv.head_dim % 64)
            return hipErrorInvalidValue;
        const bool runs = g.kv_rows_per_seq > 1;
        if (p.bm == 64)
            hipLaunchKernelGGL(runs ? k_gemm_w4_64r : k_gemm_w4_64a, grid, wg8, 0, st, g, p.tm);
        else if (p.bm == 128)
            hipLaunchKernelGGL(runs ? k_gemm_w4_128r : k_gemm_w4_128a, grid, wg8, 0, st, g, p.tm);
        else if (p.bm == 192)
            hipLaunchKernelGGL(runs ? k_gemm_w4_192r : k_gemm_w4_192a, grid, wg8, 0, st, g, p.tm);
        else
            hipLaunchKernelGGL(runs ? k_gemm_w4_256r : k_gemm_w4_256a, grid, wg8, 0, st, g, p.tm);
        return hipGetLastError();
    }
    if (p.pipelined && !int4 && p.bm == 64)
        hipLaunchKernelGGL(k_gemm_f16_64, grid, wg8, 0, st, g, p.tm);
    else if (p.pipelined && !int4)
        hipLaunchKernelGGL(k_gemm_f16_256, grid, wg8, 0, st, g, p.tm);
    else if (p.pipelined && p.bm == 64)
        hipLaunchKernelGGL(k_gemm_w4_64, grid, wg8, 0, st, g, p.tm);
    else if (p.pipelined && p.bm == 128)
        hipLaunchKernelGGL(k_gemm_w4_128, grid, wg8, 0, st, g, p.tm);
    else if (p.pipelined && p.bm == 192)
        hipLaunchKernelGGL(k_gemm_w4_192, grid, wg8, 0, st, g, p.tm);
    else if (p.pipelined)
        hipLaunchKernelGGL(k_gemm_w4_256, grid, wg8, 0, st, g, p.tm);
    else {
#define TOD_GEMM_CASE(BM_, BN_, MINW_)                                                               \
    if (p.bm == BM_ && p.bn == BN_) {                                                                \
        if (int4)                                                                                    \
            hipLaunchKernelGGL((k_gemm<BM_, BN_, true, MINW_>), grid, block, 0, st, g, p.tm);        \
        else                                                                                         \
            hipLaunchKernelGGL((k_gemm<BM_, BN_, false, MINW_>), grid, block, 0, st, g, p.tm);       \
    }
    TOD_GEMM_CASE(64, 64, 1)
    TOD_GEMM_CASE(128, 128, 1)
    TOD_GEMM_CASE(256, 128, 2)
#undef TOD_GEMM_CASE
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (p.tm.splits == 1)
        return g.ln_y ? launch_layernorm(g.y, g.M, g.N, g.ln_g, g.ln_b, g.ln_y, st) : hipSuccess;
    if (g.ln_y) {
        const dim3 grid((unsigned)g.M), block(256);
        const int chunks = layernorm_chunks(g.N), sp = p.tm.splits;
        if (chunks <= 1)
            hipLaunchKernelGGL(k_splitk_reduce_ln<1>, grid, block, 0, st, g, sp);
        else if (chunks <= 2)
            hipLaunchKernelGGL(k_splitk_reduce_ln<2>, grid, block, 0, st, g, sp);
        else if (chunks <= 4 && sp == 2)
            hipLaunchKernelGGL((k_splitk_reduce_ln<4, 2>), grid, block, 0, st, g, sp);
        else if (chunks <= 4 && sp == 4)
            hipLaunchKernelGGL((k_splitk_reduce_ln<4, 4>), grid, block, 0, st, g, sp);
        else if (chunks <= 4)
            hipLaunchKernelGGL(k_splitk_reduce_ln<4>, grid, block, 0, st, g, sp);
        else
            hipLaunchKernelGGL(k_splitk_reduce_ln<8>, grid, block, 0, st, g, sp);
        return hipGetLastError();
    }
    const int64_t n = (int64_t)g.M * g.N;
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, g, p.tm.splits);
    return hipGetLastError();
}
