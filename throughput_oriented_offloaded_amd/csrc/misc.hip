// Row-wise kernels of the decode step on gfx950: pre-LN LayerNorm, token +
// learned-position embedding (OPT keeps two offset rows in its position
// table), greedy argmax over fp16 logits, and a row gather.
#include "common.hpp"

namespace {

// One 256-thread workgroup per row: the row is read once with 16-byte loads
// and held in registers as fp16 (up to 8 * 256 * K elements); the statistics
// and the output are layernorm_row's.
template <int K>
__global__ void __launch_bounds__(256) k_layernorm(const uint16_t *__restrict__ x, int rows, int h,
                                                   const uint16_t *__restrict__ g, const uint16_t *__restrict__ b,
                                                   uint16_t *__restrict__ y)
{
    __shared__ float red[8];
    const int row = blockIdx.x, nch = h >> 3;
    const uint16_t *xr = x + (int64_t)row * h;
    uint4_t v[K];
#pragma unroll
    for (int k = 0; k < K; k++) {
        const int c = threadIdx.x + 256 * k;
        v[k] = c < nch ? *reinterpret_cast<const uint4_t *>(xr + 8 * c) : (uint4_t){0u, 0u, 0u, 0u};
    }
    layernorm_row<K>(v, nch, h, g, b, y + (int64_t)row * h, red);
}

// The sum of two fp16 values rounded to fp32 and then to fp16 equals its
// direct rounding to fp16 (fp32 carries more than 2*11+1 bits), so this is
// exactly fp16(E[id] + P[pos + 2]). Ids outside [0, vocab) are clamped into it
// (they are outside the contract; clamping keeps every read in bounds).
__global__ void __launch_bounds__(256) k_embed(const int32_t *__restrict__ ids, int rows, int rows_per_seq, int pos0,
                                               const int *__restrict__ dpos, const uint16_t *__restrict__ tok,
                                               int vocab, const uint16_t *__restrict__ posemb, int h,
                                               uint16_t *__restrict__ out)
{
    if (dpos)
        pos0 = *dpos;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)rows * h)
        return;
    const int r = (int)(i / h), c = (int)(i % h);
    const int pos = pos0 + r % rows_per_seq;
    const int id = min(max(ids[r], 0), vocab - 1);
    out[i] = f2h(h2f(tok[(int64_t)id * h + c]) + h2f(posemb[(int64_t)(pos + 2) * h + c]));
}

__device__ __forceinline__ void better(float &bv, int &bi, float v, int i)
{
    if (v > bv || (v == bv && i < bi)) {
        bv = v;
        bi = i;
    }
}

// One workgroup per row: 16-byte loads when rows are 16-byte aligned (V a
// multiple of 8), element loads otherwise; then DPP/shuffle reductions within
// each wave and LDS across the four waves. Ties go to the lowest index.
__global__ void __launch_bounds__(256) k_argmax(const uint16_t *__restrict__ logits, int V, int32_t *__restrict__ ids)
{
    __shared__ float sv[4];
    __shared__ int si[4];
    const int64_t r = blockIdx.x;
    const uint16_t *lr = logits + r * V;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    if ((V & 7) == 0) {
        const int nch = V >> 3;
        for (int c = threadIdx.x; c < nch; c += 256) {
            const half8_t hv = __builtin_bit_cast(half8_t, *reinterpret_cast<const uint4_t *>(lr + 8 * c));
#pragma unroll
            for (int e = 0; e < 8; e++)
                better(bv, bi, (float)hv[e], 8 * c + e);
        }
    } else {
        for (int i = threadIdx.x; i < V; i += 256)
            better(bv, bi, h2f(lr[i]), i);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        better(bv, bi, ov, oi);
    }
    if ((threadIdx.x & 63) == 0) {
        sv[threadIdx.x >> 6] = bv;
        si[threadIdx.x >> 6] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < 4; w++)
            better(bv, bi, sv[w], si[w]);
        ids[r] = bi;
    }
}

__global__ void __launch_bounds__(256) k_gather_rows(const uint16_t *__restrict__ src, int64_t step, int rows, int h,
                                                     uint16_t *__restrict__ dst)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)rows * h)
        return;
    const int64_t r = i / h, c = i % h;
    dst[i] = src[r * step + c];
}

__global__ void k_set_int(int *p, int v) { *p = v; }
__global__ void k_increment_int(int *p) { *p += 1; }

} // namespace

hipError_t launch_set_int(int *p, int v, hipStream_t st)
{
    hipLaunchKernelGGL(k_set_int, dim3(1), dim3(1), 0, st, p, v);
    return hipGetLastError();
}

hipError_t launch_increment_int(int *p, hipStream_t st)
{
    hipLaunchKernelGGL(k_increment_int, dim3(1), dim3(1), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_layernorm(const uint16_t *x, int rows, int h, const uint16_t *g, const uint16_t *b, uint16_t *y,
                            hipStream_t st)
{
    if (rows == 0)
        return hipSuccess;
    // h is a multiple of 64 (checked at init), so rows are 16-byte aligned
    const dim3 grid((unsigned)rows), block(256);
    const int chunks = layernorm_chunks(h);
    if (chunks <= 1)
        hipLaunchKernelGGL(k_layernorm<1>, grid, block, 0, st, x, rows, h, g, b, y);
    else if (chunks <= 2)
        hipLaunchKernelGGL(k_layernorm<2>, grid, block, 0, st, x, rows, h, g, b, y);
    else if (chunks <= 4)
        hipLaunchKernelGGL(k_layernorm<4>, grid, block, 0, st, x, rows, h, g, b, y);
    else if (chunks <= 8)
        hipLaunchKernelGGL(k_layernorm<8>, grid, block, 0, st, x, rows, h, g, b, y);
    else
        return hipErrorInvalidValue; // hidden > 16384
    return hipGetLastError();
}

hipError_t launch_embed(const int32_t *ids, int rows, int rows_per_seq, int pos0, const int *dpos, const uint16_t *tok,
                        int vocab, const uint16_t *posemb, int h, uint16_t *out, hipStream_t st)
{
    const int64_t n = (int64_t)rows * h;
    if (n == 0)
        return hipSuccess;
    hipLaunchKernelGGL(k_embed, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, ids, rows, rows_per_seq, pos0,
                       dpos, tok, vocab, posemb, h, out);
    return hipGetLastError();
}

hipError_t launch_argmax(const uint16_t *logits, int rows, int V, int32_t *ids, hipStream_t st)
{
    if (rows == 0)
        return hipSuccess;
    hipLaunchKernelGGL(k_argmax, dim3(rows), dim3(256), 0, st, logits, V, ids);
    return hipGetLastError();
}

hipError_t launch_gather_rows(const uint16_t *src, int64_t src_step, int rows, int h, uint16_t *dst, hipStream_t st)
{
    const int64_t n = (int64_t)rows * h;
    if (n == 0)
        return hipSuccess;
    hipLaunchKernelGGL(k_gather_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src, src_step, rows, h, dst);
    return hipGetLastError();
}
