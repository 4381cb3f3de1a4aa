// Group-wise asymmetric int4 quantization on gfx950: weight quantization at
// load time, the per-step KV-cache quantize+append, layout repacking and the
// canonical exports.
//
// Quantizer (FlexGen guide, "3. Group-Wise 4-Bit Quantization for Weights and
// KV Cache": contiguous groups, 16-bit to 4-bit, dequantized on the fly):
// per group of 64, zero = min, scale = fp16(fp32(max - min) / 15), and the code
// of x is the nearest grid point zero + c*scale with ties to the larger code.
// One wavefront handles one group: lane i holds element i, min/max come from
// xor-butterfly shuffles, each lane estimates its code from a division and
// settles it with exact threshold comparisons (c + 1/2) * scale, which are
// exact in fp32, so the codes are independent of how the estimate rounds.
#include "common.hpp"

namespace {

#pragma clang fp contract(off)

struct QuantLane {
    uint16_t scale, zero;
    int code;
};

// One wavefront per group: lane i holds element i.
__device__ __forceinline__ QuantLane quantize_lane(float x)
{
    const GroupQ g = group_quant(wave_min(x), wave_max(x));
    QuantLane q;
    q.scale = g.scale;
    q.zero = g.zero;
    q.code = code_of(x, g);
    return q;
}

// Pack the wave's 64 codes two per byte (even element in the low nibble);
// returns the byte for even lanes.
__device__ __forceinline__ uint8_t pack_pair(int code)
{
    const int hi = __shfl_down(code, 1, 64);
    return (uint8_t)(code | (hi << 4));
}

__global__ void __launch_bounds__(256) k_quantize_groupwise(const uint16_t *__restrict__ x, int64_t ngroups,
                                                            uint8_t *__restrict__ codes, uint16_t *__restrict__ scale,
                                                            uint16_t *__restrict__ zero)
{
    const int lane = threadIdx.x & 63;
    const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (g >= ngroups)
        return; // whole wave exits together
    const QuantLane q = quantize_lane(h2f(x[g * 64 + lane]));
    const uint8_t b = pack_pair(q.code);
    if ((lane & 1) == 0)
        codes[g * 32 + (lane >> 1)] = b;
    if (lane == 0) {
        scale[g] = q.scale;
        zero[g] = q.zero;
    }
}

__global__ void __launch_bounds__(256) k_dequantize_groupwise(const uint8_t *__restrict__ codes,
                                                              const uint16_t *__restrict__ scale,
                                                              const uint16_t *__restrict__ zero, int64_t nbytes,
                                                              uint16_t *__restrict__ out)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= nbytes)
        return;
    const uint8_t b = codes[t];
    const int64_t g = t / 32;
    const half_t s = __builtin_bit_cast(half_t, scale[g]);
    const half_t z = __builtin_bit_cast(half_t, zero[g]);
    // one rounding: fp16 fma of (code, scale, zero)
    const half_t lo = __builtin_fmaf16((half_t)(float)(b & 15), s, z);
    const half_t hi = __builtin_fmaf16((half_t)(float)(b >> 4), s, z);
    out[2 * t] = __builtin_bit_cast(uint16_t, lo);
    out[2 * t + 1] = __builtin_bit_cast(uint16_t, hi);
}

// tiled word index w -> (nb, g, lane, t); canonical word = n * (K/8) + g*8 + 2t + hk
__global__ void __launch_bounds__(256) k_repack_w4(const uint32_t *__restrict__ ccodes,
                                                   const uint16_t *__restrict__ scale,
                                                   const uint16_t *__restrict__ zero, int N, int K,
                                                   uint32_t *__restrict__ tcodes, uint32_t *__restrict__ tparams)
{
    const int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int KG = K / 64;
    const int64_t nwords = (int64_t)N * K / 8;
    if (w >= nwords)
        return;
    const int t = (int)(w & 3);
    const int lane = (int)((w >> 2) & 63);
    const int64_t blk = w >> 8; // (nb * KG + g)
    const int g = (int)(blk % KG);
    const int nb = (int)(blk / KG);
    const int n = nb * 32 + (lane & 31);
    const int hk = lane >> 5;
    tcodes[w] = tiled_word_from_canonical(ccodes[(int64_t)n * (K / 8) + g * 8 + 2 * t + hk]);
    if (t == 0 && hk == 0)
        tparams[blk * 32 + (lane & 31)] =
            (uint32_t)scale[(int64_t)n * KG + g] | ((uint32_t)zero[(int64_t)n * KG + g] << 16);
}

__global__ void __launch_bounds__(256) k_unpack_w4(const uint32_t *__restrict__ tcodes,
                                                   const uint32_t *__restrict__ tparams, int N, int K,
                                                   uint32_t *__restrict__ ccodes, uint16_t *__restrict__ scale,
                                                   uint16_t *__restrict__ zero)
{
    const int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int KG = K / 64;
    const int64_t nwords = (int64_t)N * K / 8;
    if (w >= nwords)
        return;
    const int t = (int)(w & 3);
    const int lane = (int)((w >> 2) & 63);
    const int64_t blk = w >> 8;
    const int g = (int)(blk % KG);
    const int nb = (int)(blk / KG);
    const int n = nb * 32 + (lane & 31);
    const int hk = lane >> 5;
    ccodes[(int64_t)n * (K / 8) + g * 8 + 2 * t + hk] = canonical_word_from_tiled(tcodes[w]);
    if (t == 0 && hk == 0) {
        const uint32_t p = tparams[blk * 32 + (lane & 31)];
        scale[(int64_t)n * KG + g] = (uint16_t)(p & 0xffff);
        zero[(int64_t)n * KG + g] = (uint16_t)(p >> 16);
    }
}

// Eight lanes per (row, head, group, K or V), eight consecutive elements per
// lane: one 16-byte load, min/max over the group by DPP, and one 32-bit store
// of the lane's four code bytes into the canonical per-position layout.
__global__ void __launch_bounds__(256) k_kv_append(const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
                                                   SrcMap src_map, int rows, RowMap map, KvView kv, KvView mirror)
{
    const int G = kv.head_dim / 64;
    const int64_t item = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 3;
    const int part = threadIdx.x & 7;
    const int64_t total = (int64_t)rows * kv.heads * G * 2;
    if (item >= total)
        return; // all eight lanes of an item leave together
    const int isv = (int)(item & 1);
    int64_t rest = item >> 1;
    const int g = (int)(rest % G);
    rest /= G;
    const int head = (int)(rest % kv.heads);
    const int row = (int)(rest / kv.heads);
    const int seq = map.seq0 + row / map.rows_per_seq;
    const int pos = (map.dpos ? *map.dpos : map.pos0) + row % map.rows_per_seq;
    const uint16_t *src = (isv ? v : k) + (int64_t)(row / map.rows_per_seq) * src_map.seq_stride +
                          (int64_t)(row % map.rows_per_seq) * src_map.pos_stride +
                          (int64_t)head * src_map.head_stride + g * 64 + part * 8;
    const half8_t h = __builtin_bit_cast(half8_t, *reinterpret_cast<const uint4_t *>(src));
    float x[8];
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; e++) {
        x[e] = (float)h[e];
        mn = fminf(mn, x[e]);
        mx = fmaxf(mx, x[e]);
    }
    const GroupQ q = group_quant(reduce8(mn, OpMin()), reduce8(mx, OpMax()));
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; e++)
        word |= (uint32_t)code_of(x[e], q) << (4 * e);
    const size_t at = kv_slab(kv, seq, head) * kv.cap + pos;
    const int cb = kv.head_dim / 2; // code bytes per position
    const uint32_t param = (uint32_t)q.scale | ((uint32_t)q.zero << 16);
    uint8_t *codes = isv ? kv.vc : kv.kc;
    *reinterpret_cast<uint32_t *>(codes + at * cb + g * 32 + part * 4) = word;
    if (part == 0) {
        uint32_t *pp = isv ? kv.vp : kv.kp;
        pp[at * G + g] = param;
    }
    if (mirror.kc) { // the same bytes into a second cache of the same shape (pinned host memory)
        uint8_t *mc = isv ? mirror.vc : mirror.kc;
        *reinterpret_cast<uint32_t *>(mc + at * cb + g * 32 + part * 4) = word;
        if (part == 0)
            (isv ? mirror.vp : mirror.kp)[at * G + g] = param;
    }
}

__global__ void k_kv_export(KvView kv, int seq, int head, int t0, int n, uint8_t *__restrict__ kc,
                            uint16_t *__restrict__ ks, uint16_t *__restrict__ kz, uint8_t *__restrict__ vc,
                            uint16_t *__restrict__ vs, uint16_t *__restrict__ vz)
{
    const int cb = kv.head_dim / 2, G = kv.head_dim / 64;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)n * cb)
        return;
    const int t = (int)(i / cb), byte = (int)(i % cb), pos = t0 + t;
    const size_t slab = kv_slab(kv, seq, head);
    kc[i] = kv.kc[(slab * kv.cap + pos) * cb + byte];
    vc[i] = kv.vc[(slab * kv.cap + pos) * cb + byte];
    if (byte < G) {
        const uint32_t a = kv.kp[(slab * kv.cap + pos) * G + byte];
        const uint32_t b = kv.vp[(slab * kv.cap + pos) * G + byte];
        ks[t * G + byte] = (uint16_t)(a & 0xffff);
        kz[t * G + byte] = (uint16_t)(a >> 16);
        vs[t * G + byte] = (uint16_t)(b & 0xffff);
        vz[t * G + byte] = (uint16_t)(b >> 16);
    }
}

inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

} // namespace

hipError_t launch_quantize_groupwise(const uint16_t *x, int64_t n, uint8_t *codes, uint16_t *scale, uint16_t *zero,
                                     hipStream_t st)
{
    const int64_t ng = n / 64;
    if (ng == 0)
        return hipSuccess;
    // grid.x is limited to 2^31-1 blocks: 4 groups per block covers n < 2^39
    hipLaunchKernelGGL(k_quantize_groupwise, dim3(blocks_for(ng, 4)), dim3(256), 0, st, x, ng, codes, scale, zero);
    return hipGetLastError();
}

hipError_t launch_dequantize_groupwise(const uint8_t *codes, const uint16_t *scale, const uint16_t *zero, int64_t n,
                                       uint16_t *out, hipStream_t st)
{
    if (n == 0)
        return hipSuccess;
    hipLaunchKernelGGL(k_dequantize_groupwise, dim3(blocks_for(n / 2, 256)), dim3(256), 0, st, codes, scale, zero,
                       n / 2, out);
    return hipGetLastError();
}

hipError_t launch_repack_w4(const uint8_t *codes, const uint16_t *scale, const uint16_t *zero, int N, int K,
                            uint32_t *tcodes, uint32_t *tparams, hipStream_t st)
{
    const int64_t nwords = (int64_t)N * K / 8;
    hipLaunchKernelGGL(k_repack_w4, dim3(blocks_for(nwords, 256)), dim3(256), 0, st,
                       reinterpret_cast<const uint32_t *>(codes), scale, zero, N, K, tcodes, tparams);
    return hipGetLastError();
}

hipError_t launch_unpack_w4(const uint32_t *tcodes, const uint32_t *tparams, int N, int K, uint8_t *codes,
                            uint16_t *scale, uint16_t *zero, hipStream_t st)
{
    const int64_t nwords = (int64_t)N * K / 8;
    hipLaunchKernelGGL(k_unpack_w4, dim3(blocks_for(nwords, 256)), dim3(256), 0, st, tcodes, tparams, N, K,
                       reinterpret_cast<uint32_t *>(codes), scale, zero);
    return hipGetLastError();
}

hipError_t launch_kv_append(const uint16_t *k, const uint16_t *v, SrcMap src, int rows, RowMap map, KvView kv,
                            hipStream_t st, const KvView *mirror)
{
    const int64_t items = (int64_t)rows * kv.heads * (kv.head_dim / 64) * 2;
    if (items == 0)
        return hipSuccess;
    KvView mv{};
    if (mirror)
        mv = *mirror;
    hipLaunchKernelGGL(k_kv_append, dim3(blocks_for(items, 32)), dim3(256), 0, st, k, v, src, rows, map, kv, mv);
    return hipGetLastError();
}

hipError_t launch_kv_export(KvView kv, int seq, int head, int t0, int t1, uint8_t *kc, uint16_t *ks, uint16_t *kz,
                            uint8_t *vc, uint16_t *vs, uint16_t *vz, hipStream_t st)
{
    const int n = t1 - t0;
    const int64_t items = (int64_t)n * (kv.head_dim / 2);
    if (items == 0)
        return hipSuccess;
    hipLaunchKernelGGL(k_kv_export, dim3(blocks_for(items, 256)), dim3(256), 0, st, kv, seq, head, t0, n, kc, ks, kz,
                       vc, vs, vz);
    return hipGetLastError();
}
