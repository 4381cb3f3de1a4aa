// Shared device helpers and internal launcher declarations of libtod (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t uint4_t __attribute__((ext_vector_type(4)));
typedef uint32_t uint2_t __attribute__((ext_vector_type(2)));

#define TOD_WAVE 64

__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(half_t, b); }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (half_t)f); }

// Wave-wide reductions over 64 lanes (xor butterfly).
__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_min(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v = fminf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o, 64);
    return v;
}

// Cross-lane moves without LDS traffic. DPP quad permutations and row
// rotations stay inside a 16-lane row; ds_swizzle exchanges across rows within
// each half of the wave; lane ^ 32 goes through ds_bpermute.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_XOR1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int DPP_ROR4 = 0x124;    // row_ror:4
constexpr int DPP_ROR8 = 0x128;    // row_ror:8
constexpr int DPP_HMIRROR = 0x141; // row_half_mirror: lane i of each 8 reads lane 7 - i
__device__ __forceinline__ float swizzle_xor16(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}
__device__ __forceinline__ float shfl_xor32(float v) { return __shfl_xor(v, 32, 64); }

struct OpAdd {
    __device__ float operator()(float a, float b) const { return a + b; }
};
struct OpMax {
    __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct OpMin {
    __device__ float operator()(float a, float b) const { return fminf(a, b); }
};

// Combine over the lanes of each aligned group of 8 (all 8 lanes end with the result).
template <class Op>
__device__ __forceinline__ float reduce8(float v, Op op)
{
    v = op(v, dpp_move<DPP_XOR1>(v));
    v = op(v, dpp_move<DPP_XOR2>(v));
    return op(v, dpp_move<DPP_HMIRROR>(v));
}

// Combine over the lanes that share lane % L (L = 1, 2 or 4), i.e. across the
// 64 / L slots of a wave whose lanes are grouped L at a time.
template <int L, class Op>
__device__ __forceinline__ float reduce_slots(float v, Op op)
{
    static_assert(L == 1 || L == 2 || L == 4, "L");
    if constexpr (L == 1)
        v = op(v, dpp_move<DPP_XOR1>(v));
    if constexpr (L <= 2)
        v = op(v, dpp_move<DPP_XOR2>(v));
    v = op(v, dpp_move<DPP_ROR4>(v));
    v = op(v, dpp_move<DPP_ROR8>(v));
    v = op(v, swizzle_xor16(v));
    return op(v, shfl_xor32(v));
}

// Combine within each aligned group of L lanes (L = 1, 2 or 4).
template <int L, class Op>
__device__ __forceinline__ float reduce_group(float v, Op op)
{
    if constexpr (L >= 2)
        v = op(v, dpp_move<DPP_XOR1>(v));
    if constexpr (L >= 4)
        v = op(v, dpp_move<DPP_XOR2>(v));
    return v;
}

// int4 packing inside the GEMM's tiled weight layout: a 32-bit word carries 8
// consecutive reduction-axis elements e0..e7; the low nibbles of its four
// bytes hold e0, e1, e2, e3 and the high nibbles e4, e5, e6, e7 (nibble slot p
// holds e_(p/2) for even p and e_(4+p/2) for odd p). Masking the low (or
// shifted high) nibbles leaves bytes whose pairs (bytes 0,1 and 2,3) are the
// ordered element pairs the MFMA operand needs.
__device__ __forceinline__ int tiled_slot(int e) { return e < 4 ? 2 * e : 2 * (e - 4) + 1; }

__device__ __forceinline__ uint32_t tiled_word_from_canonical(uint32_t c)
{
    // canonical: nibble p holds element p
    uint32_t r = 0;
#pragma unroll
    for (int e = 0; e < 8; e++)
        r |= ((c >> (4 * e)) & 15u) << (4 * tiled_slot(e));
    return r;
}
__device__ __forceinline__ uint32_t canonical_word_from_tiled(uint32_t t)
{
    uint32_t r = 0;
#pragma unroll
    for (int e = 0; e < 8; e++)
        r |= ((t >> (4 * tiled_slot(e))) & 15u) << (4 * e);
    return r;
}

// LayerNorm of one row held by one 256-thread workgroup: thread t holds the
// 16-byte chunks c = t + 256k (k < K) of the row's nch = h/8 chunks (zeros
// past nch). fp32 statistics in two passes over the registers (mean, then the
// biased variance of x - mean): DPP reductions within each wavefront, then the
// four wavefront sums added in a fixed order through LDS (`red`, 8 floats);
// eps 1e-5, one rounding to fp16. Shared by the LayerNorm kernel and the
// split-K reduction that fuses it, so both give identical bits.
template <int K>
__device__ __forceinline__ void layernorm_row(const uint4_t (&v)[K], int nch, int h, const uint16_t *__restrict__ g,
                                              const uint16_t *__restrict__ b, uint16_t *__restrict__ yrow, float *red)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < K; k++) {
        const half8_t hv = __builtin_bit_cast(half8_t, v[k]);
#pragma unroll
        for (int e = 0; e < 8; e++)
            s += (float)hv[e];
    }
    s = reduce_slots<1>(s, OpAdd());
    if (lane == 0)
        red[wave] = s;
    __syncthreads();
    const float mu = (((red[0] + red[1]) + red[2]) + red[3]) / (float)h;
    float q = 0.0f;
#pragma unroll
    for (int k = 0; k < K; k++) {
        if (tid + 256 * k < nch) {
            const half8_t hv = __builtin_bit_cast(half8_t, v[k]);
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const float c = (float)hv[e] - mu;
                q += c * c;
            }
        }
    }
    q = reduce_slots<1>(q, OpAdd());
    if (lane == 0)
        red[4 + wave] = q;
    __syncthreads();
    const float var = (((red[4] + red[5]) + red[6]) + red[7]) / (float)h;
    const float rs = 1.0f / sqrtf(var + 1e-5f);
#pragma unroll
    for (int k = 0; k < K; k++) {
        const int c = tid + 256 * k;
        if (c < nch) {
            const half8_t hv = __builtin_bit_cast(half8_t, v[k]);
            const half8_t gv = __builtin_bit_cast(half8_t, *reinterpret_cast<const uint4_t *>(g + 8 * c));
            const half8_t bv = __builtin_bit_cast(half8_t, *reinterpret_cast<const uint4_t *>(b + 8 * c));
            half8_t o;
#pragma unroll
            for (int e = 0; e < 8; e++)
                o[e] = (half_t)(((float)hv[e] - mu) * rs * (float)gv[e] + (float)bv[e]);
            *reinterpret_cast<uint4_t *>(yrow + 8 * c) = __builtin_bit_cast(uint4_t, o);
        }
    }
}

// 16-byte chunks per thread for a row of h fp16 values (h % 8 == 0, h <= 16384)
inline int layernorm_chunks(int h) { return (h / 8 + 255) / 256; }

// ---------------------------------------------------------------------------
// KV cache view (one layer): for each (sequence, head) "slab" of `cap`
// positions (cap % 64 == 0):
//   K codes  : [cap][d/2]  canonical bytes (byte b holds elements 2b in the
//              low nibble and 2b+1 in the high nibble)
//   K params : [cap][d/64] x uint32 (scale in the low half, zero in the high)
//   V codes  : [cap][d/2]  canonical bytes
//   V params : [cap][d/64] x uint32
// Slab (s, h) starts at index (s * heads + h) in units of the per-slab sizes.
// ---------------------------------------------------------------------------
struct KvView {
    uint8_t *kc;
    uint32_t *kp;
    uint8_t *vc;
    uint32_t *vp;
    int heads, head_dim, cap;
};

__device__ __forceinline__ size_t kv_slab(const KvView &v, int seq, int head) { return (size_t)seq * v.heads + head; }

// ---------------------------------------------------------------------------
// The int4 group quantizer (FlexGen guide, "3. Group-Wise 4-Bit Quantization
// for Weights and KV Cache"): per group, zero = min, scale = fp16(fp32(max -
// min) / 15), code = nearest grid point with ties to the larger code. Shared
// by the quantize and KV-append kernels and the QKV GEMM's fused append, so
// every path produces the same bytes.
// ---------------------------------------------------------------------------
// Parameters of one group from its minimum and maximum.
struct GroupQ {
    float mn, sf, rcp;
    uint16_t scale, zero;
};

__device__ __forceinline__ GroupQ group_quant(float mn, float mx)
{
#pragma clang fp contract(off)
    // -0 and +0 are one value: a zero minimum is stored as +0, a zero range gives scale +0
    if (mn == 0.0f)
        mn = fabsf(mn);
    if (mx == 0.0f)
        mx = fabsf(mx);
    const float range = mx - mn;
    const float s32 = range / 15.0f; // correctly rounded division
    const half_t s16 = (half_t)s32;  // round to nearest even
    GroupQ g;
    g.mn = mn;
    g.sf = (float)s16;
    g.rcp = g.sf != 0.0f ? __builtin_amdgcn_rcpf(g.sf) : 0.0f; // estimate only
    g.scale = __builtin_bit_cast(uint16_t, s16);
    g.zero = f2h(mn); // exact: mn is one of the fp16 inputs
    return g;
}

// Code of x: the number of k in 0..14 with fl32(x - mn) >= (k + 1/2) * scale.
// In exact arithmetic that count is clamp(floor(d/scale + 1/2), 0, 15) with
// d = fl32(x - mn) >= 0. The estimate from the approximate reciprocal is off
// by at most one (d/scale <= 15.01 and the relative error is below 2^-21), and
// one exact threshold test in each direction settles it: the thresholds are
// exact in fp32 (an fp16 scale times a 5-bit multiple of 1/2).
__device__ __forceinline__ int code_of(float x, const GroupQ &g)
{
#pragma clang fp contract(off)
    const float d = x - g.mn;
    int c = (int)(d * g.rcp + 0.5f);
    c = c < 0 ? 0 : (c > 15 ? 15 : c);
    c += (c < 15 && d >= ((float)c + 0.5f) * g.sf) ? 1 : 0;
    c -= (c > 0 && d < ((float)c - 0.5f) * g.sf) ? 1 : 0;
    return g.sf == 0.0f ? 0 : c;
}

// Rows of activations feeding the KV and attention kernels: row r belongs to
// sequence seq0 + r / rows_per_seq at position pos0 + r % rows_per_seq.
struct RowMap {
    int seq0, rows_per_seq, pos0;
    const int *dpos; // if non-null, pos0 is read from device memory (captured decode steps)
};

// EPI_QKV_APPEND: EPI_BIAS, and the output's K and V columns are quantized into the KV
// cache instead of being stored (the fields after ln_y in GemmArgs)
enum Epilogue { EPI_BIAS = 0, EPI_BIAS_RES = 1, EPI_BIAS_RELU = 2, EPI_NONE = 3, EPI_QKV_APPEND = 4 };

// ---------------------------------------------------------------------------
// Launchers (host side), defined next to their kernels.
// ---------------------------------------------------------------------------
hipError_t launch_quantize_groupwise(const uint16_t *x, int64_t n, uint8_t *codes, uint16_t *scale, uint16_t *zero,
                                     hipStream_t st);
hipError_t launch_dequantize_groupwise(const uint8_t *codes, const uint16_t *scale, const uint16_t *zero, int64_t n,
                                       uint16_t *out, hipStream_t st);
// canonical int4 W[N][K] -> tiled GEMM layout (codes [N/32][K/64][64][16 B], params [N/32][K/64][32] u32)
hipError_t launch_repack_w4(const uint8_t *codes, const uint16_t *scale, const uint16_t *zero, int N, int K,
                            uint32_t *tcodes, uint32_t *tparams, hipStream_t st);
hipError_t launch_unpack_w4(const uint32_t *tcodes, const uint32_t *tparams, int N, int K, uint8_t *codes,
                            uint16_t *scale, uint16_t *zero, hipStream_t st);
// Where the K/V vector of (row r, head) starts, in elements:
//   (r / rows_per_seq) * seq_stride + (r % rows_per_seq) * pos_stride + head * head_stride
struct SrcMap {
    int64_t seq_stride, pos_stride, head_stride;
};
// quantize + store the K and V vectors of `rows` rows into the cache (and, when
// mirror is given, the same bytes into that second cache of the same shape)
hipError_t launch_kv_append(const uint16_t *k, const uint16_t *v, SrcMap src, int rows, RowMap map, KvView kv,
                            hipStream_t st, const KvView *mirror = nullptr);
hipError_t launch_kv_export(KvView kv, int seq, int head, int t0, int t1, uint8_t *kc, uint16_t *ks, uint16_t *kz,
                            uint8_t *vc, uint16_t *vs, uint16_t *vz, hipStream_t st);
// decode attention: each of `rows` rows is one sequence (seq0 + r) attending positions 0..ctx-1
// ctx = *dctx + 1 when dctx is non-null (the position of the step, read on the device)
hipError_t launch_attn_decode(const uint16_t *q, int64_t q_stride, uint16_t *out, int64_t out_stride, int rows,
                              int seq0, int ctx, const int *dctx, KvView kv, hipStream_t st);
// causal prefill attention: `n_seq` sequences starting at seq0, `len` positions each, from position 0
hipError_t launch_attn_prefill(const uint16_t *q, int64_t q_stride, uint16_t *out, int64_t out_stride, int n_seq,
                               int seq0, int len, KvView kv, hipStream_t st);

struct GemmArgs {
    const uint16_t *a;   // [M][lda] fp16
    int64_t lda;
    const uint32_t *wc;  // int4 tiled codes (int4 path)
    const uint32_t *wp;  // int4 tiled params
    const uint16_t *wf;  // fp16 weights [N][K] (fp16 path)
    const uint16_t *bias;     // [N] or null
    const uint16_t *residual; // [M][ldc] or null (may alias y)
    uint16_t *y;              // [M][ldc]
    int64_t ldc;
    int M, N, K;
    int epi;
    float *ws;       // split-K workspace (fp32 [splits][M][N]) or null
    size_t ws_bytes;
    // optional LayerNorm of the output rows (ldc == N): ln_y [M][N] = LN(y) with
    // gamma ln_g, beta ln_b; fused into the split-K reduction when there is one
    const uint16_t *ln_g, *ln_b;
    uint16_t *ln_y;
    // EPI_QKV_APPEND (int4 weights on the pipelined kernel, K loop not split): output
    // columns [kv_col0, kv_col0 + h) are K and the next h are V. Rows come in runs of
    // kv_rows_per_seq consecutive positions of one sequence (1 in a decode step, the prompt
    // length in prefill; 0 counts as 1): row r's K and V are quantized in groups of 64 and
    // stored at position (*kv_dpos, or kv_pos0 when null) + r % kv_rows_per_seq of sequence
    // kv_seq0 + r / kv_rows_per_seq in kv, and in kv_mirror too when its kc is set; only the
    // columns before kv_col0 (the query) are written to y.
    KvView kv, kv_mirror;
    const int *kv_dpos;
    int kv_pos0, kv_seq0, kv_col0, kv_rows_per_seq;
};
hipError_t launch_gemm(const GemmArgs &g, hipStream_t st);
size_t gemm_workspace_bytes(int M, int N, int K, bool int4);
// The tile plan launch_gemm uses for this shape (with the workspace it asks for):
// the pipelined kernel or the register-staged one, tile, K splits, K-groups
// of 64 per workgroup and workgroups launched.
struct GemmPlanInfo {
    bool pipelined;
    int bm, bn, splits, groups_per_split, workgroups;
};
GemmPlanInfo gemm_plan_info(int M, int N, int K, bool int4);

hipError_t launch_layernorm(const uint16_t *x, int rows, int h, const uint16_t *g, const uint16_t *b, uint16_t *y,
                            hipStream_t st);
// h[r] = fp16(E[ids[r]] + P[pos + 2]), pos = pos0 + r % rows_per_seq
// pos0 = *dpos when dpos is non-null
hipError_t launch_embed(const int32_t *ids, int rows, int rows_per_seq, int pos0, const int *dpos, const uint16_t *tok,
                        int vocab, const uint16_t *posemb, int h, uint16_t *out, hipStream_t st);
// *p = v; and *p += 1 (a captured decode step advances its own position)
hipError_t launch_set_int(int *p, int v, hipStream_t st);
hipError_t launch_increment_int(int *p, hipStream_t st);
// ids[r] = argmax over fp16 logits [rows][V], lowest index on ties
hipError_t launch_argmax(const uint16_t *logits, int rows, int V, int32_t *ids, hipStream_t st);
// dst[r][i] = src[r * src_step + i], i < h (e.g. the last prompt position of each sequence)
hipError_t launch_gather_rows(const uint16_t *src, int64_t src_step, int rows, int h, uint16_t *dst, hipStream_t st);
