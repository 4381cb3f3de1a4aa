// Attention over the group-wise int4 KV cache on gfx950.
//
// FlexGen keeps the KV cache 4-bit and computes attention in fp16 on values
// dequantized on the fly (FlexGen guide, "3. Group-Wise 4-Bit Quantization for
// Weights and KV Cache"). Every cached position, the current one included,
// is read back dequantized: the step's K/V are quantized before attention.
//
// Decode (one query per (sequence, head)) is HBM-bound: it streams d/2 code
// bytes plus 4 bytes of (scale, zero) per group per position for K and for V.
// One wavefront per (sequence, head) walks the context in chunks of 64
// positions with its own online softmax (details at k_attn_decode); nothing
// is shared between wavefronts, so there are no workgroup barriers. K and V
// codes share the canonical per-position layout.
// Prefill (causal, all prompt positions) uses a tiled MFMA variant: 128 queries
// per workgroup, K/V tiles of 64 positions dequantized into LDS, online softmax.
#include <cstdlib>

#include "common.hpp"

namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));

// Exact codes of bytes 0,1 (HI = false) or 2,3 (HI = true) of a word whose
// bytes each hold one 4-bit code: the byte read as fp8 e4m3 is c * 2^-9.
template <bool HI> __device__ __forceinline__ half2_t code_pair(uint32_t nibbles)
{
    const half2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(nibbles, 512.0f, HI);
    return c;
}

__device__ __forceinline__ half2_t splat_half(uint32_t bits)
{
    const half_t h = __builtin_bit_cast(half_t, (uint16_t)bits);
    return (half2_t){h, h};
}

// The eight cache values fp16(c_e * scale + zero), rounded once, of a code word whose nibble e
// holds dim e: exact code pairs (e0,e2) (e4,e6) from the low nibbles, (e1,e3) (e5,e7) from the
// high ones, then one packed FMA per pair.
__device__ __forceinline__ half8_t dequant8(uint32_t w, half2_t s2, half2_t z2)
{
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    const half2_t x02 = __builtin_elementwise_fma(code_pair<false>(lo), s2, z2);
    const half2_t x46 = __builtin_elementwise_fma(code_pair<true>(lo), s2, z2);
    const half2_t x13 = __builtin_elementwise_fma(code_pair<false>(hi), s2, z2);
    const half2_t x57 = __builtin_elementwise_fma(code_pair<true>(hi), s2, z2);
    return (half8_t){x02[0], x13[0], x02[1], x13[1], x46[0], x57[0], x46[1], x57[1]};
}

// One chunk of 64 positions as seen by one lane: L = d/32 lanes share a
// position, each holding 16 code bytes (32 dims) of K and of V and the
// (scale, zero) word of its group, for positions slot + (64/L)*j. Lanes past
// the context load the last position again (always in bounds); their
// weights are masked to zero.
template <int L>
struct KvChunk {
    uint4_t k[L], v[L];
    uint32_t kp[L], vp[L];
};

template <int D>
__device__ __forceinline__ void load_chunk(KvChunk<D / 32> &c, int c0, int slot, uint32_t pc, int ctx,
                                           const uint8_t *kc, const uint8_t *vc, const uint8_t *kp, const uint8_t *vp)
{
    constexpr int L = D / 32, PPI = 64 / L, CB = D / 2, G = D / 64;
#pragma unroll
    for (int j = 0; j < L; j++) {
        const uint32_t t = (uint32_t)min(c0 + slot + PPI * j, ctx - 1);
        const uint32_t cofs = t * CB + pc * 16, pofs = (t * G + (pc >> 1)) * 4;
        c.k[j] = __builtin_nontemporal_load(reinterpret_cast<const uint4_t *>(kc + cofs));
        c.v[j] = __builtin_nontemporal_load(reinterpret_cast<const uint4_t *>(vc + cofs));
        c.kp[j] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(kp + pofs));
        c.vp[j] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(vp + pofs));
    }
}

// State of one wavefront's online softmax; acc holds the lane's 32 dims.
struct SoftmaxState {
    float acc[32];
    float m_run, lsum, zsum;
};

// Scores of a chunk and its weighted values.
//  * K: each code word (dims e0..e7, two per byte) is split into its low and
//    high nibbles (one byte each); read as fp8 e4m3 a byte 0000cccc is
//    c * 2^-9, so a scaled fp8 -> fp16 conversion gives the code pairs
//    (e0,e2) (e4,e6) (e1,e3) (e5,e7) exactly, and one packed FMA gives the
//    fp16 key fp16(c * scale + zero), rounded once, i.e. the dequantized cache
//    entry itself; v_dot2 against the matching query pairs sums q.k in fp32.
//  * V: the codes are decoded exactly the same way and feed fp32 accumulators
//    through mixed-precision FMA, acc_e += (p * scale) * c; the zero term is
//    added once at the end from the running sum of p * zero. So V enters as
//    the exact value zero + c * scale (never rounded to fp16), and each
//    accumulator carries only the code part of the weighted sum.
// R < L: only the first R rounds of PPI positions (the rest of the chunk lies past the context,
// so those positions would contribute exact zeros).
template <int D, int R = D / 32>
__device__ __forceinline__ void attend_chunk(const KvChunk<D / 32> &c, int c0, int slot, int ctx,
                                             const half2_t (&qa)[8], const half2_t (&qb)[8], SoftmaxState &st)
{
    constexpr int L = D / 32, PPI = 64 / L;
    static_assert(R >= 1 && R <= L, "rounds of a chunk");
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    float sc[R];
    float mloc = -INFINITY;
#pragma unroll
    for (int j = 0; j < R; j++) {
        const half2_t s2 = splat_half(c.kp[j] & 0xffffu), z2 = splat_half(c.kp[j] >> 16);
        float da = 0.0f, db = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; w++) {
            const uint32_t x = c.k[j][w], lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
            const half2_t k02 = __builtin_elementwise_fma(code_pair<false>(lo), s2, z2);
            const half2_t k46 = __builtin_elementwise_fma(code_pair<true>(lo), s2, z2);
            const half2_t k13 = __builtin_elementwise_fma(code_pair<false>(hi), s2, z2);
            const half2_t k57 = __builtin_elementwise_fma(code_pair<true>(hi), s2, z2);
            da = __builtin_amdgcn_fdot2(qa[2 * w], k02, da, false);
            db = __builtin_amdgcn_fdot2(qb[2 * w], k13, db, false);
            da = __builtin_amdgcn_fdot2(qa[2 * w + 1], k46, da, false);
            db = __builtin_amdgcn_fdot2(qb[2 * w + 1], k57, db, false);
        }
        const float score = reduce_group<L>(da + db, OpAdd()) * inv_sqrt_d;
        sc[j] = c0 + slot + PPI * j < ctx ? score : -INFINITY;
        mloc = fmaxf(mloc, sc[j]);
    }
    mloc = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                         __builtin_bit_cast(int, reduce_slots<L>(mloc, OpMax())))); // wave-uniform
    if (mloc > st.m_run) {
        const float corr = __expf(st.m_run - mloc); // 0 while nothing has been seen
#pragma unroll
        for (int e = 0; e < 32; e++)
            st.acc[e] *= corr;
        st.lsum *= corr;
        st.zsum *= corr;
        st.m_run = mloc;
    }
#pragma unroll
    for (int j = 0; j < R; j++) {
        const bool live = c0 + slot + PPI * j < ctx;
        const float p = __expf(sc[j] - st.m_run); // 0 past the context
        const float ps = live ? p * h2f((uint16_t)(c.vp[j] & 0xffffu)) : 0.0f;
        st.lsum += p;
        st.zsum += live ? p * h2f((uint16_t)(c.vp[j] >> 16)) : 0.0f;
#pragma unroll
        for (int w = 0; w < 4; w++) {
            const uint32_t x = c.v[j][w], lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
            const half2_t c02 = code_pair<false>(lo), c46 = code_pair<true>(lo);
            const half2_t c13 = code_pair<false>(hi), c57 = code_pair<true>(hi);
            float *acc = st.acc + 8 * w;
            acc[0] = fmaf(ps, (float)c02[0], acc[0]);
            acc[2] = fmaf(ps, (float)c02[1], acc[2]);
            acc[4] = fmaf(ps, (float)c46[0], acc[4]);
            acc[6] = fmaf(ps, (float)c46[1], acc[6]);
            acc[1] = fmaf(ps, (float)c13[0], acc[1]);
            acc[3] = fmaf(ps, (float)c13[1], acc[3]);
            acc[5] = fmaf(ps, (float)c57[0], acc[5]);
            acc[7] = fmaf(ps, (float)c57[1], acc[7]);
        }
    }
}

// Decode attention of one query per (sequence, head) over cached positions
// 0..ctx-1: one wavefront per (sequence, head), four per workgroup. L = d/32
// lanes share a position (32 dims each), so one 16-byte load per lane covers
// 64/L consecutive positions of K (or V) as one contiguous line. The next
// chunk's loads are issued before the current chunk's arithmetic (two
// register buffers), the softmax maximum and sums use DPP/swizzle reductions
// within the wave, and the final cross-lane sum runs once per (sequence, head)
// as a reduce-scatter: each lane ends with its share of the output dims.
template <int D>
__global__ void __launch_bounds__(256) k_attn_decode(const uint16_t *__restrict__ q, int64_t q_stride,
                                                     uint16_t *__restrict__ out, int64_t out_stride, int rows,
                                                     int seq0, int ctx, const int *__restrict__ dctx, KvView kv)
{
    if (dctx)
        ctx = *dctx + 1;
    constexpr int L = D / 32, CB = D / 2, G = D / 64;
    const int lane = threadIdx.x & 63;
    const int item = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    if (item >= rows * kv.heads)
        return; // whole wavefront
    const int row = item / kv.heads, head = item - row * kv.heads;
    const int pc = lane % L, slot = lane / L;
    const size_t slab = kv_slab(kv, seq0 + row, head);
    // per-wave bases (scalar), per-lane 32-bit offsets
    const uint8_t *kc = kv.kc + slab * kv.cap * CB;
    const uint8_t *vc = kv.vc + slab * kv.cap * CB;
    const uint8_t *kp = reinterpret_cast<const uint8_t *>(kv.kp + slab * kv.cap * G);
    const uint8_t *vp = reinterpret_cast<const uint8_t *>(kv.vp + slab * kv.cap * G);

    // query dims pc*32 .. pc*32+31, paired to match the decoded key pairs
    const uint16_t *qp = q + (int64_t)row * q_stride + (int64_t)head * D + pc * 32;
    half2_t qa[8], qb[8];
#pragma unroll
    for (int w = 0; w < 4; w++) {
        const half8_t h = __builtin_bit_cast(half8_t, *reinterpret_cast<const uint4_t *>(qp + 8 * w));
        qa[2 * w] = (half2_t){h[0], h[2]};
        qa[2 * w + 1] = (half2_t){h[4], h[6]};
        qb[2 * w] = (half2_t){h[1], h[3]};
        qb[2 * w + 1] = (half2_t){h[5], h[7]};
    }

    SoftmaxState st;
#pragma unroll
    for (int e = 0; e < 32; e++)
        st.acc[e] = 0.0f;
    st.m_run = -INFINITY;
    st.lsum = st.zsum = 0.0f;

    // chunks in pairs through two register buffers (loads of a position past
    // the context are clamped to its last position: cache hits); the last
    // chunk runs only its rounds that hold live positions
    KvChunk<L> ca, cb;
    const int nchunks = (ctx + 63) / 64;
    int c0 = 0, i = 0;
    load_chunk<D>(ca, 0, slot, pc, ctx, kc, vc, kp, vp);
    for (; i + 2 < nchunks; i += 2, c0 += 128) {
        load_chunk<D>(cb, c0 + 64, slot, pc, ctx, kc, vc, kp, vp);
        attend_chunk<D>(ca, c0, slot, ctx, qa, qb, st);
        load_chunk<D>(ca, c0 + 128, slot, pc, ctx, kc, vc, kp, vp);
        attend_chunk<D>(cb, c0 + 64, slot, ctx, qa, qb, st);
    }
    if (nchunks - i == 2) {
        load_chunk<D>(cb, c0 + 64, slot, pc, ctx, kc, vc, kp, vp);
        attend_chunk<D>(ca, c0, slot, ctx, qa, qb, st);
        c0 += 64;
        ca = cb;
    }
    const int rounds = (ctx - c0 + 64 / L - 1) / (64 / L); // 1 .. L, wave-uniform
    if (rounds >= L)
        attend_chunk<D, L>(ca, c0, slot, ctx, qa, qb, st);
    else if (rounds == 1)
        attend_chunk<D, 1>(ca, c0, slot, ctx, qa, qb, st);
    else if (L > 2 && rounds == 2)
        attend_chunk<D, (L > 2 ? 2 : 1)>(ca, c0, slot, ctx, qa, qb, st);
    else
        attend_chunk<D, (L > 3 ? 3 : 1)>(ca, c0, slot, ctx, qa, qb, st);

    // add the zero term, sum over the wave's positions: the denominator on every lane; the 32
    // dims of each lane group as a butterfly reduce-scatter over the 64/L slots (slot bit k: the
    // lanes L << k apart; each step keeps the half of the dims that bit selects), so each lane ends
    // with 32 / (64/L) consecutive dims of its block, summed slot pair by slot pair
    const float den = reduce_slots<L>(st.lsum, OpAdd());
    constexpr int NSLOT = 64 / L, KEEP = 32 / NSLOT, STEPS = L == 4 ? 4 : 5; // log2(NSLOT)
    typedef float f32x32_t __attribute__((ext_vector_type(32))); // a vector: the selects below pick values
    f32x32_t o;
#pragma unroll
    for (int e = 0; e < 32; e++)
        o[e] = st.acc[e] + st.zsum;
    int e0 = 0;
#pragma unroll
    for (int k = 0; k < STEPS; k++) {
        const int half = 16 >> k;
        const bool hi = (slot >> k) & 1;
#pragma unroll
        for (int i = 0; i < half; i++) {
            const float lo_v = o[i], hi_v = o[i + half];
            const float send = hi ? lo_v : hi_v;
            const float keep = hi ? hi_v : lo_v;
            o[i] = keep + __shfl_xor(send, L << k, 64);
        }
        e0 += hi ? half : 0;
    }
    const float inv = 1.0f / den;
    uint16_t *op = out + (int64_t)row * out_stride + (int64_t)head * D + pc * 32 + e0;
    if constexpr (KEEP == 2)
        *reinterpret_cast<uint32_t *>(op) = (uint32_t)f2h(o[0] * inv) | ((uint32_t)f2h(o[1] * inv) << 16);
    else
        *op = f2h(o[0] * inv);
}

// ---------------------------------------------------------------------------
// Prefill: QT tiles of 64 queries of one (sequence, head) per workgroup (two by
// default), causal, on MFMA.
//
// Wavefronts take 16 queries each, four per query tile. Per tile of 64 keys, K
// is dequantized once for the whole workgroup into LDS row-major and V
// transposed (fp16 values, each rounded once, as the cache defines them); a
// wavefront whose queries all precede the tile only joins its barriers.
// Scores are computed transposed, S^T = K . Q^T, with
// v_mfma_f32_16x16x32_f16: lane l ends up with keys 4*(l/16)+i (i < 4) of
// each 16-key block for query l % 16. Those registers are directly the B
// operand of O^T += V^T . P^T once the reduction index (keys) is permuted the
// same way on both operands: within a 32-key step lane group g holds keys
// 4g..4g+3 of the first 16-key block and 4g..4g+3 of the second, and reads
// the matching V^T columns. Softmax is online per query (max and sum across
// the four lanes of a query by lane shuffles); P, scaled by 2^12 so that both
// parts stay normal fp16 numbers, is split into an fp16 high part and an fp16
// remainder, each through its own MFMA, so the weights keep fp32-level
// precision; the scale comes off exactly at the end. Accumulation is fp32.
// ---------------------------------------------------------------------------
template <int D, int QT>
__global__ void __launch_bounds__(256 * QT) k_attn_prefill(const uint16_t *__restrict__ q, int64_t q_stride,
                                                           uint16_t *__restrict__ out, int64_t out_stride, int seq0,
                                                           int len, KvView kv)
{
    constexpr int CB = D / 2, G = D / 64;
    constexpr int KS = D / 32;      // 32-dim MFMA steps of the score product
    constexpr int DB = D / 16;      // 16-dim output blocks
    constexpr int KP = D + 8;       // K row pitch (halves)
    constexpr int VP = 64 + 8;      // V^T row pitch (halves)
    constexpr int WPR = CB / 4;     // 32-bit code words per position
    constexpr int PPT = 64 * WPR / (256 * QT); // positions per thread in the dequantization
    static_assert(PPT == 1 || PPT == 2 || PPT == 4, "d = 64 or 128, one or two query tiles");
    __shared__ __attribute__((aligned(16))) half_t sk[64 * KP];
    __shared__ __attribute__((aligned(16))) half_t svt[D * VP];

    // workgroup: QT consecutive query tiles of one (sequence, head); wave w takes queries 16 (w % 4) ..
    // of tile QT * (workgroup's tile pair) + w / 4 and all its waves share each dequantized key tile
    const int qtiles = (len + 63) / 64, groups = (qtiles + QT - 1) / QT;
    const int qg = blockIdx.x % groups;
    const int sh = blockIdx.x / groups;
    const int head = sh % kv.heads, s = sh / kv.heads;
    const size_t slab = kv_slab(kv, seq0 + s, head);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, g = lane >> 4;
    const int qt = qg * QT + (wave >> 2);       // this wave's query tile (may be past the last one)
    const int qpos = qt * 64 + (wave & 3) * 16 + col; // this lane's query
    const bool qlive = qpos < len;

    // Q^T fragments (B operand): dims 32k + 8g .. +8 of query qpos (zeros past len)
    half8_t qf[KS];
    {
        const uint16_t *qp = q + ((int64_t)s * len + (qlive ? qpos : 0)) * q_stride + (int64_t)head * D;
#pragma unroll
        for (int k = 0; k < KS; k++) {
            const uint4_t w = qlive ? *reinterpret_cast<const uint4_t *>(qp + 32 * k + 8 * g) : (uint4_t){0, 0, 0, 0};
            qf[k] = __builtin_bit_cast(half8_t, w);
        }
    }
    const float scale = 1.0f / sqrtf((float)D);
    float4_t acc[DB];
#pragma unroll
    for (int e = 0; e < DB; e++)
        acc[e] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, l_part = 0.0f; // l_part: this lane's share of the query's sum

    const int last_key = min(len, (qg * QT + QT - 1) * 64 + 64); // the workgroup's last key
    const int my_last = qt < qtiles ? min(len, qt * 64 + 64) : 0;  // this wave's last key
    for (int k0 = 0; k0 < last_key; k0 += 64) {
        __syncthreads();
        // dequantize keys k0..k0+63: thread (word wd, positions p0..p0+PPT-1) takes code word wd (dims
        // 8wd..8wd+7) of PPT consecutive positions, of K and of V; K rows go to LDS as 16-byte runs
        // and each dim of V^T as one run of PPT keys
        {
            const int wd = tid % WPR, p0 = (tid / WPR) * PPT;
            half8_t vh[PPT];
#pragma unroll
            for (int i = 0; i < PPT; i++) {
                const int pos = k0 + p0 + i;
                half8_t kh = {};
                vh[i] = (half8_t){};
                if (pos < len) {
                    const size_t at = slab * kv.cap + pos;
                    const uint32_t kw = *reinterpret_cast<const uint32_t *>(kv.kc + at * CB + 4 * wd);
                    const uint32_t vw = *reinterpret_cast<const uint32_t *>(kv.vc + at * CB + 4 * wd);
                    const uint32_t kpw = kv.kp[at * G + wd / 8], vpw = kv.vp[at * G + wd / 8];
                    kh = dequant8(kw, splat_half(kpw & 0xffffu), splat_half(kpw >> 16));
                    vh[i] = dequant8(vw, splat_half(vpw & 0xffffu), splat_half(vpw >> 16));
                }
                *reinterpret_cast<half8_t *>(&sk[(p0 + i) * KP + 8 * wd]) = kh;
            }
#pragma unroll
            for (int e = 0; e < 8; e++) {
                half_t *dst = &svt[(8 * wd + e) * VP + p0];
                if constexpr (PPT == 4)
                    *reinterpret_cast<half4_t *>(dst) = (half4_t){vh[0][e], vh[1][e], vh[2][e], vh[3][e]};
                else if constexpr (PPT == 2)
                    *reinterpret_cast<half2_t *>(dst) = (half2_t){vh[0][e], vh[1][e]};
                else
                    *dst = vh[0][e];
            }
        }
        __syncthreads();
        if (k0 >= my_last) // keys past this wave's queries (wave-uniform); the barriers above still run
            continue;

        // S^T for the four 16-key blocks: lane holds keys k0 + 16b + 4g + i for query qpos
        float sc[4][4];
        float tmax = -INFINITY;
#pragma unroll
        for (int b = 0; b < 4; b++) {
            float4_t c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int k = 0; k < KS; k++) {
                const half8_t kf = *reinterpret_cast<const half8_t *>(&sk[(16 * b + col) * KP + 32 * k + 8 * g]);
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[k], c, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int kpos = k0 + 16 * b + 4 * g + i;
                sc[b][i] = (kpos <= qpos && kpos < len) ? c[i] * scale : -INFINITY;
                tmax = fmaxf(tmax, sc[b][i]);
            }
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float m_new = fmaxf(m_run, tmax);
        const float corr = m_new == -INFINITY ? 1.0f : __expf(m_run - m_new);
        m_run = m_new;
        l_part *= corr;
#pragma unroll
        for (int e = 0; e < DB; e++)
            acc[e] *= corr;

        // P^T operands per 32-key step t: blocks 2t and 2t+1, split into fp16 high and low parts
#pragma unroll
        for (int t = 0; t < 2; t++) {
            half8_t ph, pl;
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const float sv = sc[2 * t + j / 4][j % 4];
                const float p = sv == -INFINITY ? 0.0f : __expf(sv - m_new);
                l_part += p;
                const float ps = p * 4096.0f; // exact
                const half_t hi = (half_t)ps;
                ph[j] = hi;
                pl[j] = (half_t)(ps - (float)hi);
            }
#pragma unroll
            for (int e = 0; e < DB; e++) {
                const half_t *vr = &svt[(16 * e + col) * VP + 32 * t + 4 * g];
                const uint2 v0 = *reinterpret_cast<const uint2 *>(vr);
                const uint2 v1 = *reinterpret_cast<const uint2 *>(vr + 16);
                const half8_t vf = __builtin_bit_cast(half8_t, (uint4_t){v0.x, v0.y, v1.x, v1.y});
                acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, ph, acc[e], 0, 0, 0);
                acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pl, acc[e], 0, 0, 0);
            }
        }
    }
    float l_sum = l_part + __shfl_xor(l_part, 16, 64);
    l_sum += __shfl_xor(l_sum, 32, 64);
    if (qlive) {
        const float inv = 1.0f / l_sum * (1.0f / 4096.0f); // the P scale, exactly
        uint16_t *op = out + ((int64_t)s * len + qpos) * out_stride + (int64_t)head * D;
#pragma unroll
        for (int e = 0; e < DB; e++) { // O^T rows 16e + 4g + i of this query
            uint2 w;
            w.x = (uint32_t)f2h(acc[e][0] * inv) | ((uint32_t)f2h(acc[e][1] * inv) << 16);
            w.y = (uint32_t)f2h(acc[e][2] * inv) | ((uint32_t)f2h(acc[e][3] * inv) << 16);
            *reinterpret_cast<uint2 *>(op + 16 * e + 4 * g) = w;
        }
    }
}

} // namespace

hipError_t launch_attn_decode(const uint16_t *q, int64_t q_stride, uint16_t *out, int64_t out_stride, int rows,
                              int seq0, int ctx, const int *dctx, KvView kv, hipStream_t st)
{
    if (rows == 0)
        return hipSuccess;
    const dim3 grid((unsigned)(((int64_t)rows * kv.heads + 3) / 4)), block(256);
    if (kv.head_dim == 128)
        hipLaunchKernelGGL(k_attn_decode<128>, grid, block, 0, st, q, q_stride, out, out_stride, rows, seq0, ctx,
                           dctx, kv);
    else if (kv.head_dim == 64)
        hipLaunchKernelGGL(k_attn_decode<64>, grid, block, 0, st, q, q_stride, out, out_stride, rows, seq0, ctx,
                           dctx, kv);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_attn_prefill(const uint16_t *q, int64_t q_stride, uint16_t *out, int64_t out_stride, int n_seq,
                               int seq0, int len, KvView kv, hipStream_t st)
{
    if (n_seq == 0 || len == 0)
        return hipSuccess;
    static const int qt_per_wg = [] {
        const char *t = getenv("TOD_PREFILL_QT"); // query tiles per workgroup: 1 or 2
        return t && atoi(t) == 1 ? 1 : 2;
    }();
    if (kv.head_dim != 128 && kv.head_dim != 64)
        return hipErrorInvalidValue;
    const int qtiles = (len + 63) / 64, groups = (qtiles + qt_per_wg - 1) / qt_per_wg;
    const dim3 grid((unsigned)n_seq * kv.heads * groups), block(256 * qt_per_wg);
    if (kv.head_dim == 128 && qt_per_wg == 2)
        hipLaunchKernelGGL((k_attn_prefill<128, 2>), grid, block, 0, st, q, q_stride, out, out_stride, seq0, len, kv);
    else if (kv.head_dim == 128)
        hipLaunchKernelGGL((k_attn_prefill<128, 1>), grid, block, 0, st, q, q_stride, out, out_stride, seq0, len, kv);
    else if (qt_per_wg == 2)
        hipLaunchKernelGGL((k_attn_prefill<64, 2>), grid, block, 0, st, q, q_stride, out, out_stride, seq0, len, kv);
    else
        hipLaunchKernelGGL((k_attn_prefill<64, 1>), grid, block, 0, st, q, q_stride, out, out_stride, seq0, len, kv);
    return hipGetLastError();
}
