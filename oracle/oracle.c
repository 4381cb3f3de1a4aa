/*
 * oracle.c -- plain, slow CPU oracle for throughput-oriented, block-scheduled
 * int4 decode of an OPT-shaped decoder stack (FlexGen).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path links, loads or calls
 * this file; only the test suite, the smoke check and the benchmark's CPU
 * baseline do. It shares no code, header or table with the GPU library.
 *
 * What it computes, and where the pages say so:
 *   - group-wise 4-bit quantization of weights and of the KV cache, with
 *     on-the-fly dequantization and fp16 compute
 *       (FlexGen guide, "3. Group-Wise 4-Bit Quantization for Weights and KV Cache";
 *        FlexLLMGen page, "The interesting bit" and "Key highlights");
 *   - the zig-zag block schedule: a layer's weights are loaded once and used
 *     for every micro-batch of the block before the next layer
 *       (FlexGen guide, "2. The Zig-Zag Block Schedule");
 *   - the row-by-row schedule it replaces, which reloads every layer for every
 *     token of every batch
 *       (FlexGen guide, "1. Row-by-Row Execution (Token-by-Token Reloading)");
 *   - the OPT decoder layer and greedy generation (OPT models are the pages'
 *     workload: FlexGen guide, "The Problem"; FlexLLMGen page, "What it does").
 * The pages give no formulas for the quantizer, the layer or the rounding;
 * the readings taken (min/max asymmetric quantizer, ties to the larger code,
 * pre-LN OPT layer, quantize-then-attend) are listed in the design notes.
 *
 * Number handling: fp16 values are converted exactly; every result stored as
 * fp16 is rounded once, to nearest-even, with subnormals kept. Sums and dot
 * products accumulate in double. Built with -ffp-contract=off (no fused ops)
 * and without -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* fp16 <-> double (IEEE 754 binary16)                                       */
/* ------------------------------------------------------------------------ */

double o_half_to_double(uint16_t h)
{
    const int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);
    return s ? -v : v;
}

/* Round a double to the nearest binary16 value, ties to even. */
uint16_t o_double_to_half(double x)
{
    const uint16_t s = signbit(x) ? 0x8000u : 0u;
    const double a = fabs(x);
    if (isnan(x))
        return 0x7e00u;
    if (a >= 65520.0) /* at or above the midpoint between 65504 and 2^16 */
        return (uint16_t)(s | 0x7c00u);
    if (a < 0x1p-14) {
        /* subnormal grid: multiples of 2^-24; 1024 * 2^-24 is the smallest normal */
        const double q = rint(a * 0x1p24);
        return (uint16_t)(s | (uint16_t)q);
    }
    int e;
    frexp(a, &e);               /* 2^(e-1) <= a < 2^e */
    const int E = e - 1;        /* -14 <= E <= 15 */
    const double q = rint(ldexp(a, 10 - E)); /* 1024 <= q <= 2048 */
    return (uint16_t)(s | (uint16_t)(((E + 15) << 10) + ((int)q - 1024)));
}

void o_half_to_double_array(const uint16_t *h, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = o_half_to_double(h[i]);
}

void o_double_to_half_array(const double *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = o_double_to_half(x[i]);
}

/* ------------------------------------------------------------------------ */
/* Group-wise asymmetric 4-bit quantizer                                     */
/* ------------------------------------------------------------------------ */

/*
 * Quantize one group of g fp16 values (FlexGen guide, "3. Group-Wise 4-Bit
 * Quantization": small contiguous groups, 16-bit to 4-bit).
 *   zero  = the group minimum (stored as fp16, exactly; a zero minimum is +0)
 *   scale = fp16_rn(fl32(fl32(max - min) / 15))
 *   code  = nearest of the 16 grid points min + c * scale, ties to the larger
 *           code, decided by exact comparisons:
 *           c = #{k in 0..14 : fl32(x - min) >= (k + 1/2) * scale}
 *           (each (k + 1/2) * scale is exact in fp32); all codes 0 if scale == 0.
 *   packing: byte t holds element 2t in its low nibble, 2t+1 in its high nibble.
 * Returns -1 on a non-finite input (out of contract).
 */
static int quantize_group(const uint16_t *x, int g, uint8_t *codes, uint16_t *scale, uint16_t *zero)
{
    float mn = 0.0f, mx = 0.0f;
    for (int i = 0; i < g; i++) {
        const double v = o_half_to_double(x[i]);
        if (!isfinite(v))
            return -1;
        const float f = (float)v;
        if (i == 0 || f < mn)
            mn = f;
        if (i == 0 || f > mx)
            mx = f;
    }
    /* -0 and +0 are the same value: a zero minimum is stored as +0 and a zero
     * range gives scale +0 */
    if (mn == 0.0f)
        mn = fabsf(mn);
    if (mx == 0.0f)
        mx = fabsf(mx);
    const float range = mx - mn;
    const float s32 = range / 15.0f;
    const uint16_t s16 = o_double_to_half((double)s32);
    const float sf = (float)o_half_to_double(s16);
    *zero = o_double_to_half((double)mn);
    *scale = s16;
    for (int t = 0; t < g / 2; t++) {
        int c[2];
        for (int u = 0; u < 2; u++) {
            c[u] = 0;
            if (sf != 0.0f) {
                const float d = (float)o_half_to_double(x[2 * t + u]) - mn;
                for (int k = 0; k < 15; k++)
                    if (d >= ((float)k + 0.5f) * sf)
                        c[u]++;
            }
        }
        codes[t] = (uint8_t)(c[0] | (c[1] << 4));
    }
    return 0;
}

int o_quantize_groupwise(const uint16_t *x, int64_t n, int group, uint8_t *codes,
                         uint16_t *scale, uint16_t *zero)
{
    if (group <= 0 || group % 2 || n < 0 || n % group)
        return -1;
    const int64_t ng = n / group;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t j = 0; j < ng; j++)
        bad |= quantize_group(x + j * group, group, codes + j * (group / 2), scale + j, zero + j) != 0;
    return bad ? -1 : 0;
}

/* Dequantized value of code c: fp16_rn(zero + c * scale), the exact value rounded once. */
static inline double dequant(int c, uint16_t scale, uint16_t zero)
{
    return o_half_to_double(o_double_to_half(o_half_to_double(zero) + (double)c * o_half_to_double(scale)));
}

static inline int code_at(const uint8_t *codes, int64_t i)
{
    return (codes[i >> 1] >> ((i & 1) * 4)) & 15;
}

int o_dequantize_groupwise(const uint8_t *codes, const uint16_t *scale, const uint16_t *zero,
                           int64_t n, int group, uint16_t *out)
{
    if (group <= 0 || group % 2 || n < 0 || n % group)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = o_double_to_half(dequant(code_at(codes, i), scale[i / group], zero[i / group]));
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Layer pieces                                                             */
/* ------------------------------------------------------------------------ */

/*
 * Accumulation precision. The oracle accumulates in double. For calibration
 * only, o_set_fp32_accumulation(1) rounds every running sum (dot products,
 * LayerNorm statistics, softmax sums) to fp32 after each addition, the
 * precision a GPU accumulator carries: comparing the two settings measures how
 * far a correct fp32-accumulating implementation may drift from the fp64 one.
 */
static int g_acc32 = 0;

void o_set_fp32_accumulation(int on) { g_acc32 = on != 0; }

static inline double acc_add(double acc, double term)
{
    const double r = acc + term;
    return g_acc32 ? (double)(float)r : r;
}

/*
 * Value of a cached V element in attention. The pages compute attention in
 * fp16 on dequantized values, so by default each V element is the fp16 value
 * fp16_rn(zero + c * scale). With o_set_exact_v(1) it is instead the exact
 * real zero + c * scale (never rounded): the same attention with that one
 * rounding left out. Both readings give one result up to half an fp16 ulp of
 * the largest |v| (the output is a weighted mean of the values); the second
 * one isolates what accumulation order and precision alone change.
 */
static int g_exact_v = 0;

void o_set_exact_v(int on) { g_exact_v = on != 0; }

static inline double v_value(int c, uint16_t scale, uint16_t zero)
{
    return g_exact_v ? o_half_to_double(zero) + (double)c * o_half_to_double(scale) : dequant(c, scale, zero);
}

/* LayerNorm over h features: biased variance, eps 1e-5, one rounding. */
void o_layernorm(const uint16_t *x, int64_t rows, int h, const uint16_t *gain,
                 const uint16_t *shift, uint16_t *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        const uint16_t *xr = x + r * h;
        double mu = 0.0, var = 0.0;
        for (int i = 0; i < h; i++)
            mu = acc_add(mu, o_half_to_double(xr[i]));
        mu /= h;
        for (int i = 0; i < h; i++) {
            const double c = o_half_to_double(xr[i]) - mu;
            var = acc_add(var, c * c);
        }
        var /= h;
        const double sd = sqrt(var + 1e-5);
        for (int i = 0; i < h; i++)
            y[r * h + i] = o_double_to_half((o_half_to_double(xr[i]) - mu) / sd * o_half_to_double(gain[i])
                                            + o_half_to_double(shift[i]));
    }
}

/*
 * y[m][o] = fp16_rn(sum_k a[m][k] * w[o][k] + bias[o] (+ residual[m][o])),
 * with ReLU applied before the rounding when relu != 0.
 * w holds exact dequantized weights (fp16 values as float).
 */
static void linear_rows(const uint16_t *a, int64_t rows, int in, int out, const float *w,
                        const uint16_t *bias, const uint16_t *residual, int relu, uint16_t *y)
{
    double *ad = malloc(sizeof(double) * (size_t)rows * in);
    for (int64_t i = 0; i < rows * in; i++)
        ad[i] = o_half_to_double(a[i]);
#pragma omp parallel for schedule(static) collapse(2)
    for (int64_t m = 0; m < rows; m++)
        for (int o = 0; o < out; o++) {
            const double *am = ad + m * in;
            const float *wo = w + (int64_t)o * in;
            double acc = 0.0;
            for (int k = 0; k < in; k++)
                acc = acc_add(acc, am[k] * (double)wo[k]);
            if (bias)
                acc = acc_add(acc, o_half_to_double(bias[o]));
            if (residual)
                acc = acc_add(acc, o_half_to_double(residual[m * out + o]));
            if (relu && acc < 0.0)
                acc = 0.0;
            y[m * out + o] = o_double_to_half(acc);
        }
    free(ad);
}

/* Linear layer over int4 group-quantized weights W[out][in] (groups along in). */
int o_linear_w4(const uint16_t *a, int64_t rows, int in, int out, const uint8_t *codes,
                const uint16_t *scale, const uint16_t *zero, int group, const uint16_t *bias,
                const uint16_t *residual, int relu, uint16_t *y)
{
    if (in % group)
        return -1;
    float *w = malloc(sizeof(float) * (size_t)out * in);
    if (!w)
        return -2;
    const int64_t n = (int64_t)out * in;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        w[i] = (float)dequant(code_at(codes, i), scale[i / group], zero[i / group]);
    linear_rows(a, rows, in, out, w, bias, residual, relu, y);
    free(w);
    return 0;
}

/* Linear layer over fp16 weights W[out][in]. */
int o_linear_f16(const uint16_t *a, int64_t rows, int in, int out, const uint16_t *wt,
                 const uint16_t *bias, const uint16_t *residual, int relu, uint16_t *y)
{
    float *w = malloc(sizeof(float) * (size_t)out * in);
    if (!w)
        return -2;
    const int64_t n = (int64_t)out * in;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        w[i] = (float)o_half_to_double(wt[i]);
    linear_rows(a, rows, in, out, w, bias, residual, relu, y);
    free(w);
    return 0;
}

/*
 * Attention of one query over cached positions 0..T-1 of one head, all keys
 * and values dequantized (the cache is int4; compute on fp16 values):
 *   score_t = (sum_i q_i * k_t,i) / sqrt(d),  w_t = exp(score_t - max_t score)
 *   out_i   = fp16_rn(sum_t w_t * v_t,i / sum_t w_t)
 * (v_t,i as chosen by o_set_exact_v: the fp16 dequantized value by default).
 * Cache layout for the head: codes [T][d/2], scale/zero [T][d/group].
 */
void o_attend(int d, int group, int T, const uint16_t *q, const uint8_t *kc, const uint16_t *ks,
              const uint16_t *kz, const uint8_t *vc, const uint16_t *vs, const uint16_t *vz, uint16_t *out)
{
    const int ng = d / group;
    double *score = malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    double mx = -INFINITY;
    for (int t = 0; t < T; t++) {
        double acc = 0.0;
        for (int i = 0; i < d; i++)
            acc = acc_add(acc, o_half_to_double(q[i]) *
                                   dequant(code_at(kc + (int64_t)t * (d / 2), i), ks[(int64_t)t * ng + i / group],
                                           kz[(int64_t)t * ng + i / group]));
        score[t] = acc / sqrt((double)d);
        if (score[t] > mx)
            mx = score[t];
    }
    double den = 0.0;
    for (int t = 0; t < T; t++) {
        score[t] = exp(score[t] - mx);
        den = acc_add(den, score[t]);
    }
    for (int i = 0; i < d; i++) {
        double acc = 0.0;
        for (int t = 0; t < T; t++)
            acc = acc_add(acc, score[t] * v_value(code_at(vc + (int64_t)t * (d / 2), i),
                                                  vs[(int64_t)t * ng + i / group], vz[(int64_t)t * ng + i / group]));
        out[i] = o_double_to_half(acc / den);
    }
    free(score);
}

/* ------------------------------------------------------------------------ */
/* Layer weights, KV cache, layer forward                                   */
/* ------------------------------------------------------------------------ */

typedef struct {
    int hidden, n_heads, head_dim, ffn, vocab, max_pos, group;
} o_dims;

enum { W_Q, W_K, W_V, W_O, W_FC1, W_FC2, N_MATS };

typedef struct {
    o_dims dm;
    uint16_t *ln1_g, *ln1_b, *ln2_g, *ln2_b;
    uint16_t *bias[N_MATS];
    int rows[N_MATS], cols[N_MATS];
    uint8_t *codes[N_MATS];
    uint16_t *scale[N_MATS], *zero[N_MATS];
    float *w[N_MATS]; /* exact dequantized values */
} o_layer;

static uint16_t *dup16(const uint16_t *p, int64_t n)
{
    uint16_t *q = malloc(sizeof(uint16_t) * (size_t)n);
    memcpy(q, p, sizeof(uint16_t) * (size_t)n);
    return q;
}

void o_layer_free(o_layer *L)
{
    if (!L)
        return;
    free(L->ln1_g); free(L->ln1_b); free(L->ln2_g); free(L->ln2_b);
    for (int m = 0; m < N_MATS; m++) {
        free(L->bias[m]); free(L->codes[m]); free(L->scale[m]); free(L->zero[m]); free(L->w[m]);
    }
    free(L);
}

/*
 * Build one layer from its 16 fp16 tensors, in this order:
 * ln1 gain, ln1 shift, Wq, bq, Wk, bk, Wv, bv, Wo, bo, ln2 gain, ln2 shift,
 * W1, b1, W2, b2 (matrices row-major [out][in]). With int4_weights the six
 * matrices are quantized by this file's quantizer (the weight tier kept in
 * GPU memory); otherwise they stay fp16 (the tier streamed from host memory,
 * FlexGen guide, "1. Three-Tier Storage Hierarchy"). The rest stays fp16.
 */
o_layer *o_layer_new(const o_dims *dm, const uint16_t *const *t, int int4_weights)
{
    const int h = dm->hidden, f = dm->ffn, G = dm->group;
    o_layer *L = calloc(1, sizeof(o_layer));
    L->dm = *dm;
    L->ln1_g = dup16(t[0], h); L->ln1_b = dup16(t[1], h);
    L->ln2_g = dup16(t[10], h); L->ln2_b = dup16(t[11], h);
    const int src[N_MATS] = {2, 4, 6, 8, 12, 14};
    const int rows[N_MATS] = {h, h, h, h, f, h};
    const int cols[N_MATS] = {h, h, h, h, h, f};
    for (int m = 0; m < N_MATS; m++) {
        const int64_t n = (int64_t)rows[m] * cols[m];
        L->rows[m] = rows[m];
        L->cols[m] = cols[m];
        L->bias[m] = dup16(t[src[m] + 1], rows[m]);
        if (!int4_weights) {
            float *w = malloc(sizeof(float) * (size_t)n);
            const uint16_t *x = t[src[m]];
            if (!w) {
                o_layer_free(L);
                return NULL;
            }
#pragma omp parallel for schedule(static)
            for (int64_t i = 0; i < n; i++)
                w[i] = (float)o_half_to_double(x[i]);
            L->w[m] = w;
            continue;
        }
        L->codes[m] = malloc((size_t)n / 2);
        L->scale[m] = malloc(sizeof(uint16_t) * (size_t)(n / G));
        L->zero[m] = malloc(sizeof(uint16_t) * (size_t)(n / G));
        L->w[m] = malloc(sizeof(float) * (size_t)n);
        if (!L->codes[m] || !L->w[m] ||
            o_quantize_groupwise(t[src[m]], n, G, L->codes[m], L->scale[m], L->zero[m]) != 0) {
            o_layer_free(L);
            return NULL;
        }
        uint8_t *cd = L->codes[m];
        uint16_t *sc = L->scale[m], *zr = L->zero[m];
        float *w = L->w[m];
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < n; i++)
            w[i] = (float)dequant(code_at(cd, i), sc[i / G], zr[i / G]);
    }
    return L;
}

int o_layer_export(const o_layer *L, int which, uint8_t *codes, uint16_t *scale, uint16_t *zero)
{
    if (which < 0 || which >= N_MATS || !L->codes[which])
        return -1;
    const int64_t n = (int64_t)L->rows[which] * L->cols[which];
    memcpy(codes, L->codes[which], (size_t)n / 2);
    memcpy(scale, L->scale[which], sizeof(uint16_t) * (size_t)(n / L->dm.group));
    memcpy(zero, L->zero[which], sizeof(uint16_t) * (size_t)(n / L->dm.group));
    return 0;
}

/* int4 KV cache of one layer for one sequence: per head, positions 0..cap-1. */
typedef struct {
    o_dims dm;
    int cap;
    uint8_t *kc, *vc;          /* [H][cap][d/2] */
    uint16_t *ks, *kz, *vs, *vz; /* [H][cap][d/group] */
} o_kv;

o_kv *o_kv_new(const o_dims *dm, int cap)
{
    const int H = dm->n_heads, d = dm->head_dim, ng = d / dm->group;
    o_kv *c = calloc(1, sizeof(o_kv));
    c->dm = *dm;
    c->cap = cap;
    c->kc = calloc((size_t)H * cap * (d / 2), 1);
    c->vc = calloc((size_t)H * cap * (d / 2), 1);
    c->ks = calloc((size_t)H * cap * ng, 2);
    c->kz = calloc((size_t)H * cap * ng, 2);
    c->vs = calloc((size_t)H * cap * ng, 2);
    c->vz = calloc((size_t)H * cap * ng, 2);
    return c;
}

void o_kv_free(o_kv *c)
{
    if (!c)
        return;
    free(c->kc); free(c->vc); free(c->ks); free(c->kz); free(c->vs); free(c->vz);
    free(c);
}

/* Quantize and store the K and V vectors ([n][H*d] fp16) of positions pos0..pos0+n-1. */
int o_kv_store(o_kv *c, int pos0, int n, const uint16_t *k, const uint16_t *v)
{
    const int H = c->dm.n_heads, d = c->dm.head_dim, G = c->dm.group, ng = d / G;
    if (pos0 < 0 || pos0 + n > c->cap)
        return -4;
    int bad = 0;
#pragma omp parallel for schedule(static) collapse(2) reduction(| : bad)
    for (int t = 0; t < n; t++)
        for (int hd = 0; hd < H; hd++) {
            const int64_t slot = (int64_t)hd * c->cap + pos0 + t;
            const int64_t src = (int64_t)t * H * d + (int64_t)hd * d;
            for (int g = 0; g < ng; g++) {
                bad |= quantize_group(k + src + g * G, G, c->kc + slot * (d / 2) + g * (G / 2), c->ks + slot * ng + g,
                                      c->kz + slot * ng + g) != 0;
                bad |= quantize_group(v + src + g * G, G, c->vc + slot * (d / 2) + g * (G / 2), c->vs + slot * ng + g,
                                      c->vz + slot * ng + g) != 0;
            }
        }
    return bad ? -1 : 0;
}

int o_kv_export(const o_kv *c, int head, int t0, int t1, uint8_t *kc, uint16_t *ks, uint16_t *kz,
                uint8_t *vc, uint16_t *vs, uint16_t *vz)
{
    const int d = c->dm.head_dim, ng = d / c->dm.group;
    if (head < 0 || head >= c->dm.n_heads || t0 < 0 || t1 > c->cap || t0 > t1)
        return -1;
    const int64_t base = (int64_t)head * c->cap + t0, n = t1 - t0;
    memcpy(kc, c->kc + base * (d / 2), (size_t)(n * (d / 2)));
    memcpy(vc, c->vc + base * (d / 2), (size_t)(n * (d / 2)));
    memcpy(ks, c->ks + base * ng, sizeof(uint16_t) * (size_t)(n * ng));
    memcpy(kz, c->kz + base * ng, sizeof(uint16_t) * (size_t)(n * ng));
    memcpy(vs, c->vs + base * ng, sizeof(uint16_t) * (size_t)(n * ng));
    memcpy(vz, c->vz + base * ng, sizeof(uint16_t) * (size_t)(n * ng));
    return 0;
}

/* Store positions [t0, t1) of one head from the canonical per-position format
 * (the inverse of o_kv_export): codes [t1-t0][d/2], params [t1-t0][d/group]. */
int o_kv_load(o_kv *c, int head, int t0, int t1, const uint8_t *kc, const uint16_t *ks, const uint16_t *kz,
              const uint8_t *vc, const uint16_t *vs, const uint16_t *vz)
{
    const int d = c->dm.head_dim, ng = d / c->dm.group;
    if (head < 0 || head >= c->dm.n_heads || t0 < 0 || t1 > c->cap || t0 > t1)
        return -1;
    const int64_t base = (int64_t)head * c->cap + t0, n = t1 - t0;
    memcpy(c->kc + base * (d / 2), kc, (size_t)(n * (d / 2)));
    memcpy(c->vc + base * (d / 2), vc, (size_t)(n * (d / 2)));
    memcpy(c->ks + base * ng, ks, sizeof(uint16_t) * (size_t)(n * ng));
    memcpy(c->kz + base * ng, kz, sizeof(uint16_t) * (size_t)(n * ng));
    memcpy(c->vs + base * ng, vs, sizeof(uint16_t) * (size_t)(n * ng));
    memcpy(c->vz + base * ng, vz, sizeof(uint16_t) * (size_t)(n * ng));
    return 0;
}

/*
 * The layer of o_layer_forward for positions pos0..pos0+n-1 of one sequence,
 * except that the K/V cache is taken as given: positions 0..pos0+n-1 must
 * already hold codes (o_kv_load). The layer's own k and v for these positions
 * (fp16 [n][h], before quantization) go to k_out / v_out (nullable) and are
 * not stored. With a cache that o_layer_forward itself filled this equals
 * o_layer_forward; with another implementation's cache it checks that
 * implementation's layer on the inputs it actually saw.
 */
int o_layer_forward_given_kv(const o_layer *L, const o_kv *c, int pos0, int n, uint16_t *hidden, uint16_t *k_out,
                             uint16_t *v_out)
{
    const int h = L->dm.hidden, H = L->dm.n_heads, d = L->dm.head_dim, f = L->dm.ffn, G = L->dm.group;
    if (pos0 < 0 || pos0 + n > c->cap || n <= 0)
        return -4;
    uint16_t *a = malloc(sizeof(uint16_t) * (size_t)n * h);
    uint16_t *q = malloc(sizeof(uint16_t) * (size_t)n * h);
    uint16_t *k = malloc(sizeof(uint16_t) * (size_t)n * h);
    uint16_t *v = malloc(sizeof(uint16_t) * (size_t)n * h);
    uint16_t *o = malloc(sizeof(uint16_t) * (size_t)n * h);
    uint16_t *u = malloc(sizeof(uint16_t) * (size_t)n * f);
    o_layernorm(hidden, n, h, L->ln1_g, L->ln1_b, a);
    linear_rows(a, n, h, h, L->w[W_Q], L->bias[W_Q], NULL, 0, q);
    linear_rows(a, n, h, h, L->w[W_K], L->bias[W_K], NULL, 0, k);
    linear_rows(a, n, h, h, L->w[W_V], L->bias[W_V], NULL, 0, v);
    if (k_out)
        memcpy(k_out, k, sizeof(uint16_t) * (size_t)n * h);
    if (v_out)
        memcpy(v_out, v, sizeof(uint16_t) * (size_t)n * h);
    const int ng = d / G;
#pragma omp parallel for schedule(dynamic) collapse(2)
    for (int t = 0; t < n; t++)
        for (int hd = 0; hd < H; hd++) {
            const int64_t base = (int64_t)hd * c->cap;
            o_attend(d, G, pos0 + t + 1, q + (int64_t)t * h + (int64_t)hd * d, c->kc + base * (d / 2),
                     c->ks + base * ng, c->kz + base * ng, c->vc + base * (d / 2), c->vs + base * ng,
                     c->vz + base * ng, o + (int64_t)t * h + (int64_t)hd * d);
        }
    linear_rows(o, n, h, h, L->w[W_O], L->bias[W_O], hidden, 0, hidden);
    o_layernorm(hidden, n, h, L->ln2_g, L->ln2_b, a);
    linear_rows(a, n, h, f, L->w[W_FC1], L->bias[W_FC1], NULL, 1, u);
    linear_rows(u, n, f, h, L->w[W_FC2], L->bias[W_FC2], hidden, 0, hidden);
    free(a); free(q); free(k); free(v); free(o); free(u);
    return 0;
}

/*
 * One pre-LN OPT decoder layer for n consecutive positions pos0..pos0+n-1 of
 * one sequence; hidden [n][h] is updated in place.
 *   a = LN1(h); q,k,v = Linear(a); quantize k, v into the cache;
 *   attention of each position p over cached 0..p (dequantized);
 *   h = Linear_o(attn) + h; b = LN2(h); h = Linear2(ReLU(Linear1(b))) + h.
 * All of the step's K/V are quantized before any of its attention, so a prompt
 * processed in one call equals the same prompt fed one position at a time.
 */
int o_layer_forward(const o_layer *L, o_kv *c, int pos0, int n, uint16_t *hidden)
{
    const int h = L->dm.hidden, H = L->dm.n_heads, d = L->dm.head_dim, f = L->dm.ffn, G = L->dm.group;
    if (pos0 < 0 || pos0 + n > c->cap || n <= 0)
        return -4;
    uint16_t *a = malloc(sizeof(uint16_t) * (size_t)n * h);
    uint16_t *q = malloc(sizeof(uint16_t) * (size_t)n * h);
    uint16_t *k = malloc(sizeof(uint16_t) * (size_t)n * h);
    uint16_t *v = malloc(sizeof(uint16_t) * (size_t)n * h);
    uint16_t *o = malloc(sizeof(uint16_t) * (size_t)n * h);
    uint16_t *u = malloc(sizeof(uint16_t) * (size_t)n * f);
    int rc = 0;
    o_layernorm(hidden, n, h, L->ln1_g, L->ln1_b, a);
    linear_rows(a, n, h, h, L->w[W_Q], L->bias[W_Q], NULL, 0, q);
    linear_rows(a, n, h, h, L->w[W_K], L->bias[W_K], NULL, 0, k);
    linear_rows(a, n, h, h, L->w[W_V], L->bias[W_V], NULL, 0, v);
    rc = o_kv_store(c, pos0, n, k, v);
    if (rc == 0) {
        const int ng = d / G;
#pragma omp parallel for schedule(dynamic) collapse(2)
        for (int t = 0; t < n; t++)
            for (int hd = 0; hd < H; hd++) {
                const int64_t base = (int64_t)hd * c->cap;
                o_attend(d, G, pos0 + t + 1, q + (int64_t)t * h + (int64_t)hd * d, c->kc + base * (d / 2),
                         c->ks + base * ng, c->kz + base * ng, c->vc + base * (d / 2), c->vs + base * ng,
                         c->vz + base * ng, o + (int64_t)t * h + (int64_t)hd * d);
            }
        linear_rows(o, n, h, h, L->w[W_O], L->bias[W_O], hidden, 0, hidden);
        o_layernorm(hidden, n, h, L->ln2_g, L->ln2_b, a);
        linear_rows(a, n, h, f, L->w[W_FC1], L->bias[W_FC1], NULL, 1, u);
        linear_rows(u, n, f, h, L->w[W_FC2], L->bias[W_FC2], hidden, 0, hidden);
    }
    free(a); free(q); free(k); free(v); free(o); free(u);
    return rc;
}

/* Token + learned position embedding: fp16_rn(E[id] + P[pos + 2]) (OPT keeps two offset rows). */
int o_embed(const o_dims *dm, const uint16_t *tok_emb, const uint16_t *pos_emb, const int32_t *ids,
            const int32_t *pos, int n, uint16_t *out)
{
    const int h = dm->hidden;
    for (int t = 0; t < n; t++) {
        if (ids[t] < 0 || ids[t] >= dm->vocab || pos[t] < 0 || pos[t] >= dm->max_pos)
            return -1;
        for (int i = 0; i < h; i++)
            out[(int64_t)t * h + i] = o_double_to_half(o_half_to_double(tok_emb[(int64_t)ids[t] * h + i]) +
                                                       o_half_to_double(pos_emb[(int64_t)(pos[t] + 2) * h + i]));
    }
    return 0;
}

/*
 * Final LayerNorm, tied-embedding logits fp16_rn(z . E[v]) and the greedy
 * pick: the largest fp16 logit, lowest index on ties.
 */
void o_head(const o_dims *dm, const uint16_t *lnf_g, const uint16_t *lnf_b, const uint16_t *tok_emb,
            const uint16_t *hidden, int n, uint16_t *logits, int32_t *next)
{
    const int h = dm->hidden, V = dm->vocab;
    uint16_t *z = malloc(sizeof(uint16_t) * (size_t)n * h);
    uint16_t *lg = logits ? logits : malloc(sizeof(uint16_t) * (size_t)n * V);
    o_layernorm(hidden, n, h, lnf_g, lnf_b, z);
    o_linear_f16(z, n, h, V, tok_emb, NULL, NULL, 0, lg);
    for (int t = 0; t < n; t++) {
        int best = 0;
        double bv = o_half_to_double(lg[(int64_t)t * V]);
        for (int j = 1; j < V; j++) {
            const double x = o_half_to_double(lg[(int64_t)t * V + j]);
            if (x > bv) {
                bv = x;
                best = j;
            }
        }
        if (next)
            next[t] = best;
    }
    if (!logits)
        free(lg);
    free(z);
}

/* ------------------------------------------------------------------------ */
/* Generation under the two schedules                                       */
/* ------------------------------------------------------------------------ */

enum { SCHED_ROW_BY_ROW = 0, SCHED_ZIGZAG = 1, SCHED_ZIGZAG_ALTERNATE = 2 };

/*
 * Greedy generation of g tokens for n_seq = K * b sequences with prompts
 * [n_seq][s]: step 0 runs the prompt (positions 0..s-1) and yields token 1;
 * step j >= 1 feeds token j at position s + j - 1 and yields token j + 1.
 * Batch k holds rows k*b .. k*b + b - 1.
 *
 * schedule SCHED_ROW_BY_ROW: for each batch, for each step, for each layer
 *   -- a layer is loaded for every (batch, step), K*g*L loads;
 * schedule SCHED_ZIGZAG(_ALTERNATE): for each step, for each layer, load the
 *   layer once and run every batch of the block through it (batch order
 *   reversed on odd layers for the alternate form) -- g*L loads.
 * forced ([n_seq][g-1], nullable) replaces the model's own pick as the input
 * of each decode step (teacher forcing). tokens [n_seq][g]; logits
 * [g][n_seq][V] (nullable); *loads counts layer loads.
 */
typedef struct {
    const o_dims *dm;
    int n_layers, n_seq, s, g;
    o_layer *const *layers;
    const uint16_t *tok_emb, *pos_emb, *lnf_g, *lnf_b;
    const int32_t *prompts, *forced;
    int32_t *tokens, *cur, *pos;
    uint16_t *logits, *hid, *last;
    o_kv **kv;
} gen_ctx;

/* Embedding of step j for rows r0..r1-1. */
static int gen_embed(gen_ctx *c, int r0, int r1, int j)
{
    const int h = c->dm->hidden, s = c->s;
    int rc = 0;
    for (int r = r0; r < r1; r++) {
        uint16_t *hr = c->hid + (int64_t)r * s * h;
        if (j == 0) {
            for (int t = 0; t < s; t++)
                c->pos[t] = t;
            rc |= o_embed(c->dm, c->tok_emb, c->pos_emb, c->prompts + (int64_t)r * s, c->pos, s, hr);
        } else {
            c->pos[0] = s + j - 1;
            rc |= o_embed(c->dm, c->tok_emb, c->pos_emb, c->cur + r, c->pos, 1, hr);
        }
    }
    return rc;
}

/* Layer l of step j for rows r0..r1-1. */
static int gen_layer(gen_ctx *c, int l, int r0, int r1, int j)
{
    const int h = c->dm->hidden, s = c->s;
    int rc = 0;
    for (int r = r0; r < r1 && !rc; r++)
        rc = o_layer_forward(c->layers[l], c->kv[(int64_t)r * c->n_layers + l], j == 0 ? 0 : s + j - 1,
                             j == 0 ? s : 1, c->hid + (int64_t)r * s * h);
    return rc;
}

/* Head of step j for rows r0..r1-1: the step's last position gives the next token. */
static void gen_head(gen_ctx *c, int r0, int r1, int j)
{
    const int h = c->dm->hidden, s = c->s, g = c->g, V = c->dm->vocab, n = r1 - r0;
    const int last = j == 0 ? s - 1 : 0;
    for (int r = r0; r < r1; r++)
        memcpy(c->last + (int64_t)(r - r0) * h, c->hid + ((int64_t)r * s + last) * h, sizeof(uint16_t) * (size_t)h);
    int32_t *nx = malloc(sizeof(int32_t) * (size_t)n);
    o_head(c->dm, c->lnf_g, c->lnf_b, c->tok_emb, c->last, n,
           c->logits ? c->logits + ((int64_t)j * c->n_seq + r0) * V : NULL, nx);
    for (int r = r0; r < r1; r++) {
        c->tokens[(int64_t)r * g + j] = nx[r - r0];
        c->cur[r] = c->forced && j + 1 < g ? c->forced[(int64_t)r * (g - 1) + j] : nx[r - r0];
    }
    free(nx);
}

int o_generate(const o_dims *dm, int n_layers, o_layer *const *layers, const uint16_t *tok_emb,
               const uint16_t *pos_emb, const uint16_t *lnf_g, const uint16_t *lnf_b, int n_seq, int K,
               int s, int g, const int32_t *prompts, int schedule, const int32_t *forced, int32_t *tokens,
               uint16_t *logits, int64_t *loads)
{
    const int h = dm->hidden;
    if (K <= 0 || n_seq <= 0 || n_seq % K || s <= 0 || g <= 0 || s + g - 1 > dm->max_pos)
        return -1;
    const int b = n_seq / K, cap = s + g - 1;
    gen_ctx c = {dm, n_layers, n_seq, s, g, layers, tok_emb, pos_emb, lnf_g, lnf_b, prompts, forced, tokens,
                 NULL, NULL, logits, NULL, NULL, NULL};
    c.kv = calloc((size_t)n_seq * n_layers, sizeof(o_kv *));
    for (int64_t i = 0; i < (int64_t)n_seq * n_layers; i++)
        c.kv[i] = o_kv_new(dm, cap);
    c.hid = malloc(sizeof(uint16_t) * (size_t)n_seq * s * h);
    c.last = malloc(sizeof(uint16_t) * (size_t)n_seq * h);
    c.cur = malloc(sizeof(int32_t) * (size_t)n_seq);
    c.pos = malloc(sizeof(int32_t) * (size_t)s);
    int rc = 0;
    *loads = 0;
    if (schedule == SCHED_ROW_BY_ROW) {
        for (int k = 0; k < K && !rc; k++)
            for (int j = 0; j < g && !rc; j++) {
                rc |= gen_embed(&c, k * b, k * b + b, j);
                for (int l = 0; l < n_layers && !rc; l++) {
                    (*loads)++; /* this batch's pass over the model reloads layer l */
                    rc |= gen_layer(&c, l, k * b, k * b + b, j);
                }
                if (!rc)
                    gen_head(&c, k * b, k * b + b, j);
            }
    } else if (schedule == SCHED_ZIGZAG || schedule == SCHED_ZIGZAG_ALTERNATE) {
        for (int j = 0; j < g && !rc; j++) {
            rc |= gen_embed(&c, 0, n_seq, j);
            for (int l = 0; l < n_layers && !rc; l++) {
                (*loads)++; /* layer l is loaded once and reused by every batch of the block */
                const int reverse = schedule == SCHED_ZIGZAG_ALTERNATE && (l & 1);
                for (int kk = 0; kk < K && !rc; kk++) {
                    const int k = reverse ? K - 1 - kk : kk;
                    rc |= gen_layer(&c, l, k * b, k * b + b, j);
                }
            }
            if (!rc)
                gen_head(&c, 0, n_seq, j);
        }
    } else {
        rc = -1;
    }
    for (int64_t i = 0; i < (int64_t)n_seq * n_layers; i++)
        o_kv_free(c.kv[i]);
    free(c.kv); free(c.hid); free(c.last); free(c.cur); free(c.pos);
    return rc;
}
