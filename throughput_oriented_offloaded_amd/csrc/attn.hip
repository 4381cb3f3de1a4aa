// Attention over the group-wise int4 KV cache on gfx950.
//
// FlexGen keeps the KV cache 4-bit and computes attention in fp16 on values
// dequantized on the fly (FlexGen guide, "3. Group-Wise 4-Bit Quantization for
// Weights and KV Cache"). Every cached position, the current one included,
// is read back dequantized: the step's K/V are quantized before attention.
//
// Decode (one query per (sequence, head)) is HBM-bound: it streams d/2 code
// bytes plus 4 bytes of (scale, zero) per group per position for K and for V.
// One 256-thread workgroup per (sequence, head) walks the context in chunks
// of 256 positions with an online softmax (details at k_attn_decode). K codes
// sit in a position-chunked layout so that the 64 lanes of a wave read 64
// positions' 16-byte pieces as one contiguous 1 KiB line; V codes stay in the
// canonical per-position layout, read 16 bytes per lane.
// Prefill (causal, all prompt positions) uses a tiled variant: 64 queries per
// workgroup, K/V tiles of 64 positions dequantized into LDS, online softmax.
#include "common.hpp"

namespace {

// Block-wide reductions over the 4 wavefronts of a 256-thread workgroup.
__device__ __forceinline__ float block_max(float v, float *red)
{
    v = wave_max(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ float block_sum(float v, float *red)
{
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

// Codes c_j and c_{j+4} of a canonical word, centred (c - 8, exact) as an fp16 pair:
// (nibble | 0x6400) is the fp16 value 1024 + c, and 1024 + c - 1032 is exact.
__device__ __forceinline__ half2_t centred_pair(uint32_t w, int j)
{
    const half2_t bias = {(half_t)1032.0f, (half_t)1032.0f};
    return __builtin_bit_cast(half2_t, ((w >> (4 * j)) & 0x000F000Fu) | 0x64006400u) - bias;
}

// Decode attention of one query per (sequence, head) over cached positions
// 0..ctx-1, in chunks of 256 positions with an online softmax:
//  * all global loads of a chunk (the K codes and (scale, zero) of the
//    thread's position, and 16-byte slices of 256/ (d/32) positions' V codes)
//    are issued before any of its arithmetic, so each thread keeps ~13
//    independent loads in flight;
//  * scores: with centred codes, q.khat = scale * sum(q * (c - 8)) +
//    (zero + 8 * scale) * sum(q), the first sum by v_dot2_f32_f16;
//  * values: each thread owns 32 dims of (d/32)-strided positions and
//    accumulates (p * scale) * c in fp32 plus p * zero per group; the partial
//    sums are reduced across lanes with shuffles and across waves in LDS.
template <int D>
__global__ void __launch_bounds__(256) k_attn_decode(const uint16_t *__restrict__ q, int64_t q_stride,
                                                     uint16_t *__restrict__ out, int64_t out_stride, int seq0,
                                                     int ctx, KvView kv)
{
    constexpr int CB = D / 2;          // code bytes per position
    constexpr int PIECES = CB / 16;    // 16-byte pieces per position
    constexpr int G = D / 64;          // groups per head vector
    constexpr int VQ = PIECES;         // threads per position in the value pass
    constexpr int VTOK = 256 / VQ;     // positions per value iteration
    constexpr int VIT = 256 / VTOK;    // value iterations per chunk of 256 positions
    __shared__ float sp[256];
    __shared__ float red[4];
    __shared__ float part[4 * D];

    const int row = blockIdx.x / kv.heads, head = blockIdx.x % kv.heads;
    const int seq = seq0 + row;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t slab = kv_slab(kv, seq, head);
    const uint8_t *kc = kv.kc + slab * kv.cap * CB;
    const uint32_t *kp = kv.kp + slab * kv.cap * G;
    const uint8_t *vc = kv.vc + slab * kv.cap * CB;
    const uint32_t *vp = kv.vp + slab * kv.cap * G;

    // query in registers, paired (j, j + 4) within each word of 8 to match centred_pair
    const uint16_t *qp = q + (int64_t)row * q_stride + (int64_t)head * D;
    half2_t qv[D / 2];
    float qsum[G];
#pragma unroll
    for (int gi = 0; gi < G; gi++)
        qsum[gi] = 0.0f;
#pragma unroll
    for (int w = 0; w < D / 8; w++) {
        const half8_t h = __builtin_bit_cast(half8_t, *reinterpret_cast<const uint4_t *>(qp + 8 * w));
#pragma unroll
        for (int j = 0; j < 4; j++) {
            qv[4 * w + j] = (half2_t){h[j], h[j + 4]};
            qsum[w / 8] += (float)h[j] + (float)h[j + 4];
        }
    }
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);

    const int vq = tid % VQ;             // which 16-byte slice (32 dims) of a position
    const int vgrp = (vq * 32) / 64;     // its group
    float acc[32];
#pragma unroll
    for (int e = 0; e < 32; e++)
        acc[e] = 0.0f;
    float zacc = 0.0f, lsum = 0.0f, m_run = -INFINITY;

    for (int c0 = 0; c0 < ctx; c0 += 256) {
        // ---- issue every load of the chunk
        const int t = c0 + tid;
        const bool tk = t < ctx;
        uint4_t kr[PIECES];
        uint32_t kpar[G];
        const uint8_t *kb = kc + ((size_t)(t >> 6) * PIECES * 64 + (t & 63)) * 16;
#pragma unroll
        for (int pc = 0; pc < PIECES; pc++)
            kr[pc] = tk ? *reinterpret_cast<const uint4_t *>(kb + (size_t)pc * 64 * 16) : (uint4_t){0u, 0u, 0u, 0u};
#pragma unroll
        for (int gi = 0; gi < G; gi++)
            kpar[gi] = tk ? kp[(size_t)t * G + gi] : 0u;
        uint4_t vr[VIT];
        uint32_t vpar[VIT];
#pragma unroll
        for (int j = 0; j < VIT; j++) {
            const int tv = c0 + tid / VQ + VTOK * j;
            const bool ok = tv < ctx;
            vr[j] = ok ? *reinterpret_cast<const uint4_t *>(vc + (size_t)tv * CB + vq * 16) : (uint4_t){0u, 0u, 0u, 0u};
            vpar[j] = ok ? vp[(size_t)tv * G + vgrp] : 0u;
        }

        // ---- scores of this chunk
        float score = -INFINITY;
        if (tk) {
            score = 0.0f;
#pragma unroll
            for (int gi = 0; gi < G; gi++) {
                float dot = 0.0f;
#pragma unroll
                for (int pc = 0; pc < 2; pc++) {
#pragma unroll
                    for (int w = 0; w < 4; w++) {
                        const int qw = (2 * gi + pc) * 4 + w;
#pragma unroll
                        for (int j = 0; j < 4; j++)
                            dot = __builtin_amdgcn_fdot2(qv[4 * qw + j], centred_pair(kr[2 * gi + pc][w], j), dot,
                                                         false);
                    }
                }
                const float s = h2f((uint16_t)(kpar[gi] & 0xffff)), z = h2f((uint16_t)(kpar[gi] >> 16));
                score += s * dot + (z + 8.0f * s) * qsum[gi];
            }
            score *= inv_sqrt_d;
        }
        const float m_new = fmaxf(m_run, block_max(score, red));
        const float corr = __expf(m_run - m_new); // 0 on the first chunk
        const float p = tk ? __expf(score - m_new) : 0.0f;
        sp[tid] = p;
        lsum = lsum * corr + p;
        zacc *= corr;
#pragma unroll
        for (int e = 0; e < 32; e++)
            acc[e] *= corr;
        m_run = m_new;
        __syncthreads();

        // ---- values of this chunk: canonical bytes, byte b = elements 2b (low) and 2b+1 (high)
#pragma unroll
        for (int j = 0; j < VIT; j++) {
            const float pr = sp[tid / VQ + VTOK * j];
            const float ps = pr * h2f((uint16_t)(vpar[j] & 0xffff));
            zacc += pr * h2f((uint16_t)(vpar[j] >> 16));
#pragma unroll
            for (int w = 0; w < 4; w++) {
                const uint32_t lo = vr[j][w] & 0x0F0F0F0Fu, hi = (vr[j][w] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
                for (int b = 0; b < 4; b++) {
                    acc[8 * w + 2 * b] += ps * (float)((lo >> (8 * b)) & 0xffu);
                    acc[8 * w + 2 * b + 1] += ps * (float)((hi >> (8 * b)) & 0xffu);
                }
            }
        }
        __syncthreads(); // sp is rewritten by the next chunk
    }

    // ---- reduce: lanes sharing vq (lane % VQ) within the wave, then the 4 waves in LDS
    const float den = block_sum(lsum, red);
#pragma unroll
    for (int e = 0; e < 32; e++) {
        float v = acc[e] + zacc;
#pragma unroll
        for (int o = VQ; o < 64; o <<= 1)
            v += __shfl_xor(v, o, 64);
        acc[e] = v;
    }
    if (lane < VQ) {
#pragma unroll
        for (int e = 0; e < 32; e++)
            part[wave * D + lane * 32 + e] = acc[e];
    }
    __syncthreads();
    if (tid < D) {
        const float o = (part[tid] + part[D + tid]) + (part[2 * D + tid] + part[3 * D + tid]);
        out[(int64_t)row * out_stride + (int64_t)head * D + tid] = f2h(o / den);
    }
}

// ---------------------------------------------------------------------------
// Prefill: 64 queries x (sequence, head) per workgroup, causal.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) k_attn_prefill(const uint16_t *__restrict__ q, int64_t q_stride,
                                                      uint16_t *__restrict__ out, int64_t out_stride, int seq0,
                                                      int len, KvView kv)
{
    constexpr int CB = D / 2, PIECES = CB / 16, G = D / 64;
    constexpr int DP = D + 2; // padded LDS row (halves)
    constexpr int DPV = 32;   // dims per thread in the PV product
    __shared__ half_t sq[64 * DP];
    __shared__ half_t sk[64 * DP];
    __shared__ half_t sv[64 * DP];
    __shared__ float sp[64 * 65];

    const int qtiles = (len + 63) / 64;
    const int qt = blockIdx.x % qtiles;
    const int sh = blockIdx.x / qtiles;
    const int head = sh % kv.heads, s = sh / kv.heads;
    const int seq = seq0 + s;
    const int tid = threadIdx.x;
    const int q0 = qt * 64;
    const size_t slab = kv_slab(kv, seq, head);

    // load Q tile (rows beyond len are zero)
    for (int i = tid; i < 64 * D; i += 256) {
        const int r = i / D, dd = i % D;
        const int pos = q0 + r;
        sq[r * DP + dd] = pos < len ? __builtin_bit_cast(half_t, q[((int64_t)s * len + pos) * q_stride +
                                                                   (int64_t)head * D + dd])
                                    : (half_t)0.0f;
    }
    const int myq = tid >> 2, sub = tid & 3; // 4 threads per query
    const int qpos = q0 + myq;
    float m_run = -INFINITY, l_run = 0.0f;
    float o[DPV * D / 128];
    constexpr int NO = DPV * D / 128; // D=128: 32 dims per thread; D=64: 16
#pragma unroll
    for (int e = 0; e < NO; e++)
        o[e] = 0.0f;
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    const int last_key = min(len, q0 + 64); // keys [0, last_key)
    for (int k0 = 0; k0 < last_key; k0 += 64) {
        __syncthreads();
        // dequantize K and V tiles (positions k0..k0+63) into LDS
        for (int i = tid; i < 64 * CB; i += 256) {
            const int r = i / CB, byte = i % CB, pos = k0 + r;
            half_t k_lo = (half_t)0.0f, k_hi = (half_t)0.0f, v_lo = (half_t)0.0f, v_hi = (half_t)0.0f;
            if (pos < len) {
                const int piece = byte >> 4, off = byte & 15, gi = byte / 32;
                const uint8_t kb =
                    kv.kc[slab * kv.cap * CB + (((size_t)(pos >> 6) * PIECES + piece) * 64 + (pos & 63)) * 16 + off];
                const uint8_t vb = kv.vc[(slab * kv.cap + pos) * CB + byte];
                const uint32_t kp = kv.kp[(slab * kv.cap + pos) * G + gi];
                const uint32_t vp = kv.vp[(slab * kv.cap + pos) * G + gi];
                const half_t ks = __builtin_bit_cast(half_t, (uint16_t)(kp & 0xffff));
                const half_t kz = __builtin_bit_cast(half_t, (uint16_t)(kp >> 16));
                const half_t vs = __builtin_bit_cast(half_t, (uint16_t)(vp & 0xffff));
                const half_t vz = __builtin_bit_cast(half_t, (uint16_t)(vp >> 16));
                k_lo = __builtin_fmaf16((half_t)(float)(kb & 15), ks, kz);
                k_hi = __builtin_fmaf16((half_t)(float)(kb >> 4), ks, kz);
                v_lo = __builtin_fmaf16((half_t)(float)(vb & 15), vs, vz);
                v_hi = __builtin_fmaf16((half_t)(float)(vb >> 4), vs, vz);
            }
            sk[r * DP + 2 * byte] = k_lo;
            sk[r * DP + 2 * byte + 1] = k_hi;
            sv[r * DP + 2 * byte] = v_lo;
            sv[r * DP + 2 * byte + 1] = v_hi;
        }
        __syncthreads();
        // scores for keys k0 + sub + 4*i
        float sc[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int kr = sub + 4 * i;
            const int kpos = k0 + kr;
            float acc = 0.0f;
            for (int dd = 0; dd < D; dd += 2) {
                const half2_t a = *reinterpret_cast<const half2_t *>(&sq[myq * DP + dd]);
                const half2_t b = *reinterpret_cast<const half2_t *>(&sk[kr * DP + dd]);
                acc = __builtin_amdgcn_fdot2(a, b, acc, false);
            }
            acc *= inv_sqrt_d;
            sc[i] = (kpos <= qpos && kpos < len) ? acc : -INFINITY;
            tmax = fmaxf(tmax, sc[i]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 1, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 2, 64));
        const float m_new = fmaxf(m_run, tmax);
        const float corr = m_new == -INFINITY ? 1.0f : __expf(m_run - m_new);
        float psum = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const float p = sc[i] == -INFINITY ? 0.0f : __expf(sc[i] - m_new);
            sp[myq * 65 + sub + 4 * i] = p;
            psum += p;
        }
        psum += __shfl_xor(psum, 1, 64);
        psum += __shfl_xor(psum, 2, 64);
        l_run = l_run * corr + psum;
        m_run = m_new;
#pragma unroll
        for (int e = 0; e < NO; e++)
            o[e] *= corr;
        __syncthreads();
        // o[q][d] += sum_k p[q][k] v[k][d], dims sub*NO .. +NO
        for (int kr = 0; kr < 64; kr++) {
            const float p = sp[myq * 65 + kr];
#pragma unroll
            for (int e = 0; e < NO; e += 2) {
                const half2_t v2 = *reinterpret_cast<const half2_t *>(&sv[kr * DP + sub * NO + e]);
                o[e] += p * (float)v2[0];
                o[e + 1] += p * (float)v2[1];
            }
        }
    }
    if (qpos < len) {
        const float inv = 1.0f / l_run;
        uint16_t *op = out + ((int64_t)s * len + qpos) * out_stride + (int64_t)head * D + sub * NO;
#pragma unroll
        for (int e = 0; e < NO; e++)
            op[e] = f2h(o[e] * inv);
    }
}

} // namespace

hipError_t launch_attn_decode(const uint16_t *q, int64_t q_stride, uint16_t *out, int64_t out_stride, int rows,
                              int seq0, int ctx, KvView kv, hipStream_t st)
{
    if (rows == 0)
        return hipSuccess;
    const dim3 grid((unsigned)rows * kv.heads), block(256);
    if (kv.head_dim == 128)
        hipLaunchKernelGGL(k_attn_decode<128>, grid, block, 0, st, q, q_stride, out, out_stride, seq0, ctx, kv);
    else if (kv.head_dim == 64)
        hipLaunchKernelGGL(k_attn_decode<64>, grid, block, 0, st, q, q_stride, out, out_stride, seq0, ctx, kv);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_attn_prefill(const uint16_t *q, int64_t q_stride, uint16_t *out, int64_t out_stride, int n_seq,
                               int seq0, int len, KvView kv, hipStream_t st)
{
    if (n_seq == 0 || len == 0)
        return hipSuccess;
    const int qtiles = (len + 63) / 64;
    const dim3 grid((unsigned)n_seq * kv.heads * qtiles), block(256);
    if (kv.head_dim == 128)
        hipLaunchKernelGGL(k_attn_prefill<128>, grid, block, 0, st, q, q_stride, out, out_stride, seq0, len, kv);
    else if (kv.head_dim == 64)
        hipLaunchKernelGGL(k_attn_prefill<64>, grid, block, 0, st, q, q_stride, out, out_stride, seq0, len, kv);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}
