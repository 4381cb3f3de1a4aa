// Runtime and C ABI of libtod: model state, the zig-zag block driver, the
// pinned-host weight tier streamed over a copy stream, and test/bench hooks.
//
// Schedule (FlexGen guide, "2. The Zig-Zag Block Schedule"): a pass over the
// stack visits each layer once; while a layer's weights are resident every
// batch of the block runs through it before the next layer. In a decode step
// the block's K*b rows form the M dimension of each fused int4 GEMM, so the
// weights are read once per (step, layer); attention and the KV append are
// per sequence. Prefill runs the K batches through each layer one after
// another (M = b * prompt_len per GEMM).
//
// Host tier (FlexGen guide, "1. Three-Tier Storage Hierarchy"; TightLLM
// abstract, static overlap of transfer and compute): fp16 weights live in
// pinned host memory; a copy stream brings layer l+1 into one of two HBM
// slots while the compute stream works on layer l; events order slot reuse.
#include <atomic>
#include <cerrno>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include <fcntl.h>
#include <unistd.h>

#include "../../include/tod.h"
#include "api.hpp"
#include "common.hpp"

namespace {
thread_local char g_err[512];
} // namespace

int fail(int code, const char *fmt, ...)
{
    char buf[sizeof g_err]; // the arguments may point into g_err itself
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    memcpy(g_err, buf, sizeof g_err);
    return code;
}

namespace {

#define HIPCHK(expr)                                                                          \
    do {                                                                                      \
        hipError_t e_ = (expr);                                                               \
        if (e_ != hipSuccess)                                                                 \
            return fail(TOD_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_));              \
    } while (0)

inline hipStream_t S(void *p) { return reinterpret_cast<hipStream_t>(p); }

enum { MAT_QKV = 0, MAT_O, MAT_FC1, MAT_FC2, N_GEMM_MATS };

struct LayerStore {
    uint32_t *wc[N_GEMM_MATS] = {};   // int4 tiled codes
    uint32_t *wp[N_GEMM_MATS] = {};   // int4 tiled (scale, zero)
    uint16_t *bias[N_GEMM_MATS] = {}; // device fp16
    uint16_t *ln1_g = nullptr, *ln1_b = nullptr, *ln2_g = nullptr, *ln2_b = nullptr;
    uint8_t *host = nullptr;          // host tiers: pinned image of the layer's matrices
    uint8_t *dev = nullptr;           // host tiers, resident layers: that image kept in HBM
    bool loaded = false;
};

} // namespace

struct tod_model {
    tod_model_config cfg{};
    tod_run_config run{};
    int M = 0;      // rows per block (K * b)
    int cap = 0;    // KV positions per (sequence, head), multiple of 64
    int n_out[N_GEMM_MATS] = {}, n_in[N_GEMM_MATS] = {};
    // host tiers: byte offsets of each matrix's image in a layer (fp16 values, or
    // tiled int4 codes followed by their tiled params) and the layer's size
    int64_t mat_off[N_GEMM_MATS] = {}, par_off[N_GEMM_MATS] = {};
    int64_t layer_bytes = 0;
    bool streamed = false, int4 = true; // weights streamed from host; int4 GEMMs
    int hbm_layers = 0;                // host tiers: leading layers whose image stays in HBM
    int host_layers = 0;               // host tiers: streamed layers with their own pinned image
    std::vector<LayerStore> layers;
    uint16_t *tok_emb = nullptr, *pos_emb = nullptr, *lnf_g = nullptr, *lnf_b = nullptr;
    bool glob_loaded = false;
    std::vector<KvView> kv; // [block * L + layer]
    std::vector<void *> dev_allocs;
    std::vector<void *> host_allocs;
    // activations
    uint16_t *hid = nullptr, *act = nullptr, *qkv = nullptr, *att = nullptr, *ffn = nullptr, *last = nullptr,
             *logits = nullptr;
    int32_t *ids = nullptr;
    float *ws = nullptr;
    size_t ws_bytes = 0;
    // decode steps quantize and append K/V in the QKV GEMM's epilogue (its plan allows
    // it: int4 weights on the pipelined kernel, K loop not split; TOD_QKV_APPEND=0: never)
    bool qkv_append = false;
    // load-time staging
    uint16_t *stage = nullptr;
    uint8_t *stage_codes = nullptr;
    uint16_t *stage_scale = nullptr, *stage_zero = nullptr;
    // host tier streaming
    uint8_t *slot[2] = {};
    hipStream_t copy = nullptr;
    hipEvent_t ev_loaded[2] = {}, ev_free[2] = {};
    bool prefetched = false; // slot 0 holds, or is being filled with, the first streamed layer
    // host KV tier: the last kv_host layers keep their caches in pinned host memory; a
    // step copies a layer's cached positions into one of two HBM slots, and the append
    // writes each new position into the slot and through to the host cache
    int kv_host = 0;
    KvView kvslot[2] = {};
    hipEvent_t ev_kv_loaded[2] = {}, ev_kv_free[2] = {};
    // disk tier: the streamed layers' images live in a file; an I/O stream reads each
    // into one of two pinned staging buffers, from which the copy stream moves it into the
    // HBM slot. Direct I/O cannot target pinned buffers, so reads go through the page
    // cache, and every image is dropped from it after each write and read.
    bool on_disk = false;
    int fd = -1;
    int64_t image_stride = 0; // layer_bytes rounded up to the 4 KiB I/O alignment
    uint8_t *staging[2] = {};
    hipStream_t io = nullptr;
    hipEvent_t ev_staged[2] = {}, ev_staging_free[2] = {};
    std::atomic<int> io_errno{0};
    std::vector<int> prefilled, decoded;
    // captured decode steps (HBM tier): one graph per block, replayed on gstream;
    // the step reads its position from gpos and its token ids from gids (the
    // argmax writes the next ids back there) and advances gpos itself
    bool graphs_on = true;
    int *gpos = nullptr;
    int32_t *gids = nullptr;
    hipStream_t gstream = nullptr;
    hipEvent_t gev_in = nullptr, gev_out = nullptr;
    std::vector<hipGraphExec_t> gexec; // [block], null until captured
    std::vector<int> gfail;            // [block], capture failed: stay eager
    // kernel timing (profile_kernels / profile_read)
    unsigned prof_mask = 0;
    std::vector<hipEvent_t> ev_pool;
    struct Pending {
        int kind;
        hipEvent_t a, b;
    };
    std::vector<Pending> pend;
    double prof_ms[TOD_K_COUNT] = {};
    int64_t prof_n[TOD_K_COUNT] = {};
    // test taps (set_layer_tap): per phase (0 prefill, 1 decode) and layer, a range of the
    // pass's hidden rows copied out before and after the layer
    struct Tap {
        int64_t row0 = 0, n = 0;
        uint16_t *in = nullptr, *out = nullptr;
    };
    std::vector<Tap> taps[2];
    int n_decode_taps = 0;
};

struct tod_attn_cache {
    KvView kv{};
    int batch = 0;
    std::vector<void *> allocs;
};

namespace {

int dev_alloc(tod_model *m, void **p, size_t bytes)
{
    if (bytes == 0) {
        *p = nullptr;
        return TOD_OK;
    }
    hipError_t e = hipMalloc(p, bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(TOD_ENOMEM, "hipMalloc(%zu bytes) failed: %s", bytes, hipGetErrorString(e));
    }
    m->dev_allocs.push_back(*p);
    return TOD_OK;
}

#define ALLOC(ptr, bytes)                                                   \
    do {                                                                    \
        int rc_ = dev_alloc(m, reinterpret_cast<void **>(&(ptr)), (bytes)); \
        if (rc_)                                                            \
            return rc_;                                                     \
    } while (0)

KvView make_kv_view(uint8_t *kc, uint32_t *kp, uint8_t *vc, uint32_t *vp, int heads, int d, int cap)
{
    KvView v;
    v.kc = kc;
    v.kp = kp;
    v.vc = vc;
    v.vp = vp;
    v.heads = heads;
    v.head_dim = d;
    v.cap = cap;
    return v;
}

// bytes of one KV array set for n_slabs (sequence, head) slabs
size_t kv_bytes(size_t n_slabs, int d, int cap, size_t *kc_b, size_t *kp_b)
{
    *kc_b = n_slabs * cap * (size_t)(d / 2);
    *kp_b = n_slabs * cap * (size_t)(d / 64) * 4;
    return 2 * (*kc_b + *kp_b);
}

hipEvent_t pooled_event(tod_model *m)
{
    if (!m->ev_pool.empty()) {
        hipEvent_t e = m->ev_pool.back();
        m->ev_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    return e;
}

// Brackets the launches issued in its lifetime with events when `kind` is profiled.
struct ProfScope {
    tod_model *m;
    int kind;
    hipStream_t st;
    hipEvent_t a = nullptr;
    ProfScope(tod_model *m_, int kind_, hipStream_t st_) : m(m_), kind(kind_), st(st_)
    {
        if (m->prof_mask & (1u << kind)) {
            a = pooled_event(m);
            if (a && hipEventRecord(a, st) != hipSuccess) {
                (void)hipGetLastError();
                m->ev_pool.push_back(a);
                a = nullptr;
            }
        }
    }
    // Never throws: the event lists have room reserved by profile_kernels, and an event that
    // cannot be kept is destroyed instead (its launch then goes untimed).
    ~ProfScope()
    {
        if (!a)
            return;
        hipEvent_t b = pooled_event(m);
        const bool recorded = b && hipEventRecord(b, st) == hipSuccess;
        if (!recorded)
            (void)hipGetLastError();
        try {
            if (recorded) {
                m->pend.push_back({kind, a, b});
                return;
            }
            m->ev_pool.push_back(a);
            a = nullptr;
            if (b)
                m->ev_pool.push_back(b);
        } catch (...) {
            if (a)
                (void)hipEventDestroy(a);
            if (b)
                (void)hipEventDestroy(b);
        }
    }
};

// Weights of matrix `mat` of layer L: HBM int4, or the layer's image in a
// streamed slot (fp16 values, or tiled int4 codes and params).
void weights_of(const tod_model *m, const LayerStore &L, int mat, const uint8_t *slot, GemmArgs &g)
{
    if (!slot) {
        g.wc = L.wc[mat];
        g.wp = L.wp[mat];
    } else if (m->int4) {
        g.wc = reinterpret_cast<const uint32_t *>(slot + m->mat_off[mat]);
        g.wp = reinterpret_cast<const uint32_t *>(slot + m->par_off[mat]);
    } else {
        g.wf = reinterpret_cast<const uint16_t *>(slot + m->mat_off[mat]);
    }
}

// ln_g/ln_b (nullable): also write LayerNorm(y) into m->act, fused into the
// GEMM's split-K reduction when it has one.
// kv (nullable, EPI_QKV_APPEND): the cache the QKV GEMM appends the rows' K/V to, with its
// host mirror: rows in runs of per_seq positions (*dpos, or pos0 when null, onwards) of
// sequences seq0, seq0 + 1, ...
int run_gemm(tod_model *m, const uint16_t *a, int rows, int mat, const LayerStore &L, const uint8_t *slot,
             uint16_t *y, int64_t ldc, int epi, hipStream_t st, const uint16_t *ln_g = nullptr,
             const uint16_t *ln_b = nullptr, const KvView *kv = nullptr, const KvView *kv_mirror = nullptr,
             int seq0 = 0, int pos0 = 0, const int *dpos = nullptr, int per_seq = 1)
{
    GemmArgs g{};
    g.a = a;
    g.lda = m->n_in[mat];
    weights_of(m, L, mat, slot, g);
    g.bias = L.bias[mat];
    g.residual = epi == EPI_BIAS_RES ? y : nullptr;
    g.y = y;
    g.ldc = ldc;
    g.M = rows;
    g.N = m->n_out[mat];
    g.K = m->n_in[mat];
    g.epi = epi;
    g.ws = m->ws;
    g.ws_bytes = m->ws_bytes;
    if (ln_g) {
        g.ln_g = ln_g;
        g.ln_b = ln_b;
        g.ln_y = m->act;
    }
    if (kv) {
        g.kv = *kv;
        if (kv_mirror)
            g.kv_mirror = *kv_mirror;
        g.kv_dpos = dpos;
        g.kv_pos0 = pos0;
        g.kv_seq0 = seq0;
        g.kv_col0 = m->cfg.hidden; // q, then k, then v
        g.kv_rows_per_seq = per_seq;
    }
    ProfScope ps(m, TOD_K_GEMM_QKV + mat, st);
    HIPCHK(launch_gemm(g, st));
    return TOD_OK;
}

// The QKV GEMM over `rows` rows can append K/V in its epilogue: int4 weights on the
// pipelined kernel with the K loop not split.
bool qkv_append_plan(const tod_model *m, int rows)
{
    const GemmPlanInfo qp = gemm_plan_info(rows, m->n_out[MAT_QKV], m->n_in[MAT_QKV], m->int4);
    return m->int4 && qp.pipelined && qp.splits == 1;
}

// One decoder layer for `rows` rows whose hidden states start at `h`.
// decode: rows = M sequences at position pos; prefill: rows = b * s (b sequences
// starting at seq0, positions 0..s-1). act_ready: m->act already holds LN1(h)
// (written by the previous layer's fc2); next_g/next_b (nullable): the fc2
// GEMM also writes that LayerNorm of the new h into m->act for the next layer
// (or the head). LN2 comes out of the out-projection GEMM the same way.
int layer_pass(tod_model *m, int l, const KvView &kv, uint16_t *h, int rows, bool prefill_mode, int seq0, int s,
               int pos, const int *dpos, const uint8_t *wslot, hipStream_t st, bool act_ready = false,
               const uint16_t *next_g = nullptr, const uint16_t *next_b = nullptr, const KvView *kv_mirror = nullptr)
{
    const int hd = m->cfg.hidden, f = m->cfg.ffn;
    const LayerStore &L = m->layers[l];
    int rc;
    if (!act_ready) {
        ProfScope ps(m, TOD_K_LAYERNORM, st);
        HIPCHK(launch_layernorm(h, rows, hd, L.ln1_g, L.ln1_b, m->act, st));
    }
    // K/V appended by the QKV GEMM itself (prefill: where its plan for these rows allows)
    const bool fused = m->qkv_append && (!prefill_mode || qkv_append_plan(m, rows));
    if (fused) {
        if ((rc = run_gemm(m, m->act, rows, MAT_QKV, L, wslot, m->qkv, 3 * hd, EPI_QKV_APPEND, st, nullptr, nullptr,
                           &kv, kv_mirror, seq0, prefill_mode ? 0 : pos, prefill_mode ? nullptr : dpos,
                           prefill_mode ? s : 1)))
            return rc;
    } else if ((rc = run_gemm(m, m->act, rows, MAT_QKV, L, wslot, m->qkv, 3 * hd, EPI_BIAS, st))) {
        return rc;
    }
    SrcMap src;
    RowMap map;
    if (prefill_mode) {
        src = {(int64_t)s * 3 * hd, 3 * hd, m->cfg.head_dim};
        map = {seq0, s, 0, nullptr};
    } else {
        src = {3 * hd, 0, m->cfg.head_dim};
        map = {seq0, 1, pos, dpos};
    }
    if (!fused) {
        ProfScope ps(m, TOD_K_KV_APPEND, st);
        HIPCHK(launch_kv_append(m->qkv + hd, m->qkv + 2 * hd, src, rows, map, kv, st, kv_mirror));
    }
    {
        ProfScope ps(m, TOD_K_ATTN, st);
        if (prefill_mode)
            HIPCHK(launch_attn_prefill(m->qkv, 3 * hd, m->att, hd, rows / s, seq0, s, kv, st));
        else
            HIPCHK(launch_attn_decode(m->qkv, 3 * hd, m->att, hd, rows, seq0, pos + 1, dpos, kv, st));
    }
    if ((rc = run_gemm(m, m->att, rows, MAT_O, L, wslot, h, hd, EPI_BIAS_RES, st, L.ln2_g, L.ln2_b)))
        return rc;
    if ((rc = run_gemm(m, m->act, rows, MAT_FC1, L, wslot, m->ffn, f, EPI_BIAS_RELU, st)))
        return rc;
    if ((rc = run_gemm(m, m->ffn, rows, MAT_FC2, L, wslot, h, hd, EPI_BIAS_RES, st, next_g, next_b)))
        return rc;
    return TOD_OK;
}

// Test taps: copy the tapped rows that lie among the `rows` hidden rows at h (global rows
// r0 .. r0 + rows - 1 of the pass) into the tap's `in` buffer (before the layer) or its
// `out` buffer (after it), on the pass's stream.
int tap_copy(tod_model *m, int phase, int l, const uint16_t *h, int64_t r0, int64_t rows, bool after,
             hipStream_t st)
{
    if (m->taps[phase].empty())
        return TOD_OK;
    const tod_model::Tap &t = m->taps[phase][l];
    uint16_t *dst = after ? t.out : t.in;
    const int64_t lo = t.row0 > r0 ? t.row0 : r0, hi = t.row0 + t.n < r0 + rows ? t.row0 + t.n : r0 + rows;
    if (t.n <= 0 || !dst || lo >= hi)
        return TOD_OK;
    const int64_t hd = m->cfg.hidden;
    HIPCHK(hipMemcpyAsync(dst + (lo - t.row0) * hd, h + (lo - r0) * hd, (size_t)((hi - lo) * hd) * 2,
                          hipMemcpyDeviceToDevice, st));
    return TOD_OK;
}

// Host tiers: the layer whose pinned image streamed layer l copies. Streamed
// layers past the first host_layers reuse theirs, in turn.
int image_layer(const tod_model *m, int l)
{
    const int R = m->hbm_layers;
    return l < R + m->host_layers ? l : R + (l - R) % m->host_layers;
}

// Disk tier: one read of a layer image into a staging buffer, run on the I/O
// stream by the HIP runtime's callback thread.
struct ImageRead {
    tod_model *m;
    int sl;
    int64_t offset;
};

void read_image(void *arg)
{
    ImageRead *job = static_cast<ImageRead *>(arg);
    tod_model *m = job->m;
    uint8_t *dst = m->staging[job->sl];
    int64_t done = 0;
    while (done < m->image_stride) {
        const ssize_t n = pread(m->fd, dst + done, (size_t)(m->image_stride - done), job->offset + done);
        if (n < 0 && errno == EINTR)
            continue;
        if (n <= 0) {
            int expected = 0;
            m->io_errno.compare_exchange_strong(expected, n < 0 ? errno : EIO);
            break;
        }
        done += n;
    }
    (void)posix_fadvise(m->fd, job->offset, m->image_stride, POSIX_FADV_DONTNEED);
    delete job;
}

// Byte offset of layer l's image in the weight file (images of the streamed layers that
// own one, packed from the first streamed layer on).
int64_t image_offset(const tod_model *m, int l)
{
    return (int64_t)(image_layer(m, l) - m->hbm_layers) * m->image_stride;
}

// Host tiers: enqueue the copy of streamed layer l into its slot (streamed
// layers alternate between the two) on the copy stream; on the disk tier the
// image is first read into the slot's staging buffer on the I/O stream.
int stream_layer(tod_model *m, int l)
{
    const int sl = (l - m->hbm_layers) & 1;
    if (m->on_disk) {
        // stage on the I/O stream once the previous copy out of this staging buffer is done
        HIPCHK(hipStreamWaitEvent(m->io, m->ev_staging_free[sl], 0));
        ImageRead *job = new (std::nothrow) ImageRead{m, sl, image_offset(m, l)};
        if (!job)
            return fail(TOD_ENOMEM, "no memory for an image read");
        const hipError_t e = hipLaunchHostFunc(m->io, read_image, job);
        if (e != hipSuccess) {
            delete job;
            HIPCHK(e);
        }
        HIPCHK(hipEventRecord(m->ev_staged[sl], m->io));
        HIPCHK(hipStreamWaitEvent(m->copy, m->ev_free[sl], 0));
        HIPCHK(hipStreamWaitEvent(m->copy, m->ev_staged[sl], 0));
        HIPCHK(hipMemcpyAsync(m->slot[sl], m->staging[sl], (size_t)m->layer_bytes, hipMemcpyHostToDevice, m->copy));
        HIPCHK(hipEventRecord(m->ev_staging_free[sl], m->copy));
        HIPCHK(hipEventRecord(m->ev_loaded[sl], m->copy));
        return TOD_OK;
    }
    HIPCHK(hipStreamWaitEvent(m->copy, m->ev_free[sl], 0));
    HIPCHK(hipMemcpyAsync(m->slot[sl], m->layers[image_layer(m, l)].host, (size_t)m->layer_bytes,
                          hipMemcpyHostToDevice, m->copy));
    HIPCHK(hipEventRecord(m->ev_loaded[sl], m->copy));
    return TOD_OK;
}

// Host KV tier: enqueue the copy of positions [0, npos) of layer l's host cache
// (block `block`) into its HBM slot on the copy stream (host-KV layers alternate
// between the two slots), after the slot's previous user has finished.
int stream_kv(tod_model *m, int block, int l, int npos)
{
    const int sl = (l - (m->cfg.n_layers - m->kv_host)) & 1;
    HIPCHK(hipStreamWaitEvent(m->copy, m->ev_kv_free[sl], 0));
    if (npos > 0) {
        const KvView &src = m->kv[(size_t)block * m->cfg.n_layers + l];
        const KvView &dst = m->kvslot[sl];
        const size_t slabs = (size_t)m->M * m->cfg.n_heads, cb = (size_t)m->cfg.head_dim / 2,
                     pb = (size_t)m->cfg.head_dim / 64 * 4, cap = (size_t)m->cap;
        // per slab the first npos positions of each array: one 2D copy per array
        HIPCHK(hipMemcpy2DAsync(dst.kc, cap * cb, src.kc, cap * cb, npos * cb, slabs, hipMemcpyHostToDevice, m->copy));
        HIPCHK(hipMemcpy2DAsync(dst.vc, cap * cb, src.vc, cap * cb, npos * cb, slabs, hipMemcpyHostToDevice, m->copy));
        HIPCHK(hipMemcpy2DAsync(dst.kp, cap * pb, src.kp, cap * pb, npos * pb, slabs, hipMemcpyHostToDevice, m->copy));
        HIPCHK(hipMemcpy2DAsync(dst.vp, cap * pb, src.vp, cap * pb, npos * pb, slabs, hipMemcpyHostToDevice, m->copy));
    }
    HIPCHK(hipEventRecord(m->ev_kv_loaded[sl], m->copy));
    return TOD_OK;
}

// One pass over all layers of block `block`. `body(l, wslot, kv, mirror)` runs
// layer l for every batch of the block against the KV cache `kv` (mirror: the
// host cache the appended positions are also written to, or null). Host-KV
// layers get an HBM slot holding their first kv_npos cached positions.
template <class F>
int stack_pass(tod_model *m, hipStream_t st, int block, int kv_npos, F body)
{
    // layers below R run from HBM (the int4 store, or a host tier's resident
    // image); the others stream. The first streamed layer's copy is issued at
    // the end of the previous pass (layer images never change during passes),
    // so it overlaps that pass's tail, the head and this pass's resident layers.
    const int L = m->cfg.n_layers, R = m->streamed ? m->hbm_layers : L;
    const int KH = L - m->kv_host; // first layer whose KV cache lives on the host
    int rc;
    if (R < L && !m->prefetched && (rc = stream_layer(m, R)))
        return rc;
    m->prefetched = false;
    if (KH == 0 && L > 0 && (rc = stream_kv(m, block, 0, kv_npos)))
        return rc;
    for (int l = 0; l < L; l++) {
        const uint8_t *wslot = l < R ? m->layers[l].dev : nullptr;
        const int sl = (l - R) & 1;
        if (l >= R) {
            if (l + 1 < L && (rc = stream_layer(m, l + 1)))
                return rc;
            HIPCHK(hipStreamWaitEvent(st, m->ev_loaded[sl], 0));
            wslot = m->slot[sl];
        }
        if (l + 1 < L && l + 1 >= KH && (rc = stream_kv(m, block, l + 1, kv_npos)))
            return rc;
        const KvView *kv = &m->kv[(size_t)block * L + l];
        const KvView *mirror = nullptr;
        const int ks = (l - KH) & 1;
        if (l >= KH) {
            HIPCHK(hipStreamWaitEvent(st, m->ev_kv_loaded[ks], 0));
            mirror = kv;
            kv = &m->kvslot[ks];
        }
        if ((rc = body(l, wslot, *kv, mirror)))
            return rc;
        if (l >= R)
            HIPCHK(hipEventRecord(m->ev_free[sl], st));
        if (l >= KH)
            HIPCHK(hipEventRecord(m->ev_kv_free[ks], st));
    }
    if (R < L) { // the next pass's first copy, ordered after this pass's use of its slot
        if ((rc = stream_layer(m, R)))
            return rc;
        m->prefetched = true;
    }
    return TOD_OK;
}

int check_ready(tod_model *m, int block)
{
    if (!m)
        return fail(TOD_EINVAL, "null model");
    if (block < 0 || block >= m->run.n_blocks)
        return fail(TOD_ESTATE, "block %d out of range [0, %d)", block, m->run.n_blocks);
    if (!m->glob_loaded)
        return fail(TOD_ESTATE, "global weights not set");
    if (const int e = m->io_errno.load())
        return fail(TOD_EHIP, "a weight file read failed: %s", strerror(e));
    for (int l = 0; l < m->cfg.n_layers; l++)
        if (!m->layers[l].loaded)
            return fail(TOD_ESTATE, "layer %d weights not set", l);
    return TOD_OK;
}

// LM head on `rows` final hidden rows: LN_f, tied-embedding logits, argmax.
// act_ready: m->act already holds LN_f of the rows (fused into the last fc2).
int head_pass(tod_model *m, const uint16_t *hrows, int rows, uint16_t *logits, int32_t *next, hipStream_t st,
              bool act_ready = false)
{
    const int hd = m->cfg.hidden, V = m->cfg.vocab;
    if (!act_ready) {
        ProfScope ps(m, TOD_K_LAYERNORM, st);
        HIPCHK(launch_layernorm(hrows, rows, hd, m->lnf_g, m->lnf_b, m->act, st));
    }
    GemmArgs g{};
    g.a = m->act;
    g.lda = hd;
    g.wf = m->tok_emb;
    g.y = logits;
    g.ldc = V;
    g.M = rows;
    g.N = V;
    g.K = hd;
    g.epi = EPI_NONE;
    g.ws = m->ws;
    g.ws_bytes = m->ws_bytes;
    {
        ProfScope ps(m, TOD_K_LM_HEAD, st);
        HIPCHK(launch_gemm(g, st));
    }
    {
        ProfScope ps(m, TOD_K_ARGMAX, st);
        HIPCHK(launch_argmax(logits, rows, V, next, st));
    }
    return TOD_OK;
}

} // namespace

// The rules init_model applies to its configurations (estimate_decode applies them too).
int check_config(const tod_model_config *cfg, const tod_run_config *run)
{
    if (!cfg || !run)
        return fail(TOD_EINVAL, "null config");
    const tod_model_config &c = *cfg;
    const tod_run_config &r = *run;
    if (c.n_layers <= 0 || c.hidden <= 0 || c.n_heads <= 0 || c.head_dim <= 0 || c.ffn <= 0 || c.vocab <= 0 ||
        c.max_pos <= 0)
        return fail(TOD_EINVAL, "model config fields must be positive");
    if (c.hidden != c.n_heads * c.head_dim)
        return fail(TOD_EINVAL, "hidden (%d) != n_heads * head_dim (%d)", c.hidden, c.n_heads * c.head_dim);
    if (c.head_dim % 64 || c.hidden % 64 || c.ffn % 64 || (c.head_dim != 64 && c.head_dim != 128))
        return fail(TOD_EINVAL, "head_dim must be 64 or 128; hidden and ffn multiples of 64");
    if (c.hidden > 16384)
        return fail(TOD_EINVAL, "hidden (%d) above 16384", c.hidden);
    if (r.group != TOD_GROUP)
        return fail(TOD_EINVAL, "group must be 64 (got %d)", r.group);
    if (r.gpu_batch <= 0 || r.batches_per_block <= 0 || r.prompt_len <= 0 || r.gen_len <= 0 || r.n_blocks <= 0)
        return fail(TOD_EINVAL, "run config fields must be positive");
    if (r.n_blocks > TOD_MAX_BLOCKS)
        return fail(TOD_EINVAL, "n_blocks (%d) above %d", r.n_blocks, TOD_MAX_BLOCKS);
    if (r.weight_tier != TOD_W_HBM_INT4 && r.weight_tier != TOD_W_HOST_FP16_STREAM &&
        r.weight_tier != TOD_W_HOST_INT4_STREAM)
        return fail(TOD_EINVAL, "unknown weight tier %d", r.weight_tier);
    if ((int64_t)r.prompt_len + r.gen_len - 1 > c.max_pos)
        return fail(TOD_EINVAL, "prompt_len + gen_len - 1 exceeds max_pos");
    if ((int64_t)r.gpu_batch * r.batches_per_block > (1 << 24) || (int64_t)r.gpu_batch * r.prompt_len > (1 << 24))
        return fail(TOD_EINVAL, "gpu_batch * batches_per_block and gpu_batch * prompt_len must be at most 2^24");
    const bool host = r.weight_tier != TOD_W_HBM_INT4;
    if (r.host_layers < 0 || (r.host_layers && !host))
        return fail(TOD_EINVAL, "host_layers (%d) applies to the host tiers only and must be >= 0", r.host_layers);
    if (r.hbm_layers < 0 || r.hbm_layers > c.n_layers || (r.hbm_layers && !host))
        return fail(TOD_EINVAL, "hbm_layers (%d) applies to the host tiers only and must be in [0, n_layers]",
                    r.hbm_layers);
    if (r.kv_host_layers < 0 || r.kv_host_layers > c.n_layers)
        return fail(TOD_EINVAL, "kv_host_layers (%d) must be in [0, n_layers]", r.kv_host_layers);
    if (r.weights_on_disk != 0 && r.weights_on_disk != 1)
        return fail(TOD_EINVAL, "weights_on_disk must be 0 or 1 (got %d)", r.weights_on_disk);
    if (r.weights_on_disk && !host)
        return fail(TOD_EINVAL, "weights_on_disk applies to the host tiers only");
    return TOD_OK;
}

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

const char *last_error(void) { return g_err; }

int free_model(tod_model *m)
{
    return guard("free_model", [&]() -> int {
        if (!m)
            return TOD_OK;
        (void)hipDeviceSynchronize();
        for (void *p : m->dev_allocs)
            (void)hipFree(p);
        for (void *p : m->host_allocs)
            (void)hipHostFree(p);
        for (int i = 0; i < 2; i++) {
            if (m->ev_loaded[i])
                (void)hipEventDestroy(m->ev_loaded[i]);
            if (m->ev_free[i])
                (void)hipEventDestroy(m->ev_free[i]);
            if (m->ev_kv_loaded[i])
                (void)hipEventDestroy(m->ev_kv_loaded[i]);
            if (m->ev_kv_free[i])
                (void)hipEventDestroy(m->ev_kv_free[i]);
            if (m->ev_staged[i])
                (void)hipEventDestroy(m->ev_staged[i]);
            if (m->ev_staging_free[i])
                (void)hipEventDestroy(m->ev_staging_free[i]);
        }
        if (m->copy)
            (void)hipStreamDestroy(m->copy);
        if (m->io)
            (void)hipStreamDestroy(m->io);
        if (m->fd >= 0)
            (void)close(m->fd);
        for (hipGraphExec_t e : m->gexec)
            if (e)
                (void)hipGraphExecDestroy(e);
        if (m->gstream)
            (void)hipStreamDestroy(m->gstream);
        if (m->gev_in)
            (void)hipEventDestroy(m->gev_in);
        if (m->gev_out)
            (void)hipEventDestroy(m->gev_out);
        for (auto &p : m->pend) {
            (void)hipEventDestroy(p.a);
            (void)hipEventDestroy(p.b);
        }
        for (hipEvent_t e : m->ev_pool)
            (void)hipEventDestroy(e);
        delete m;
        return TOD_OK;
    });
}

static int init_model_impl(const tod_model_config *cfg, const tod_run_config *run, tod_model *m)
{
    const tod_model_config &c = *cfg;
    const tod_run_config &r = *run; // checked by init_model
    m->cfg = c;
    m->run = r;
    m->M = r.gpu_batch * r.batches_per_block;
    m->cap = (r.prompt_len + r.gen_len - 1 + 63) / 64 * 64;
    const int h = c.hidden, f = c.ffn, L = c.n_layers;
    m->n_out[MAT_QKV] = 3 * h; m->n_in[MAT_QKV] = h;
    m->n_out[MAT_O] = h;       m->n_in[MAT_O] = h;
    m->n_out[MAT_FC1] = f;     m->n_in[MAT_FC1] = h;
    m->n_out[MAT_FC2] = h;     m->n_in[MAT_FC2] = f;
    m->streamed = r.weight_tier != TOD_W_HBM_INT4;
    m->int4 = r.weight_tier != TOD_W_HOST_FP16_STREAM;
    // a layer's image on the host tiers: the four GEMM matrices back to back,
    // fp16 values, or tiled int4 codes each followed by its tiled params
    int64_t off = 0;
    for (int mat = 0; mat < N_GEMM_MATS; mat++) {
        const int64_t n = (int64_t)m->n_out[mat] * m->n_in[mat];
        m->mat_off[mat] = off;
        if (m->int4) {
            m->par_off[mat] = off + n / 2;
            off += n / 2 + n / 16;
        } else {
            off += n * 2;
        }
    }
    m->layer_bytes = off;
    m->layers.resize(L);
    const bool host = m->streamed;
    m->hbm_layers = host ? r.hbm_layers : 0;
    m->kv_host = r.kv_host_layers;
    m->on_disk = r.weights_on_disk != 0;
    m->image_stride = (m->layer_bytes + 4095) / 4096 * 4096;
    const int n_streamed = host ? L - m->hbm_layers : 0;
    m->host_layers = r.host_layers > 0 && r.host_layers < n_streamed ? r.host_layers : n_streamed;

    // weights
    for (int l = 0; l < L; l++) {
        LayerStore &S_ = m->layers[l];
        for (int mat = 0; mat < N_GEMM_MATS; mat++) {
            const int64_t n = (int64_t)m->n_out[mat] * m->n_in[mat];
            if (!host) {
                ALLOC(S_.wc[mat], (size_t)n / 2);
                ALLOC(S_.wp[mat], (size_t)n / 64 * 4);
            }
            ALLOC(S_.bias[mat], (size_t)m->n_out[mat] * 2);
        }
        ALLOC(S_.ln1_g, (size_t)h * 2);
        ALLOC(S_.ln1_b, (size_t)h * 2);
        ALLOC(S_.ln2_g, (size_t)h * 2);
        ALLOC(S_.ln2_b, (size_t)h * 2);
        if (host && l < m->hbm_layers)
            ALLOC(S_.dev, (size_t)m->layer_bytes);
        if (host && !m->on_disk && l >= m->hbm_layers && l < m->hbm_layers + m->host_layers) {
            void *p = nullptr;
            hipError_t e = hipHostMalloc(&p, (size_t)m->layer_bytes, hipHostMallocDefault);
            if (e != hipSuccess) {
                (void)hipGetLastError();
                return fail(TOD_ENOMEM, "hipHostMalloc(%lld bytes) for layer %d failed: %s",
                            (long long)m->layer_bytes, l, hipGetErrorString(e));
            }
            m->host_allocs.push_back(p);
            S_.host = static_cast<uint8_t *>(p);
        }
    }
    ALLOC(m->tok_emb, (size_t)c.vocab * h * 2);
    ALLOC(m->pos_emb, (size_t)(c.max_pos + 2) * h * 2);
    ALLOC(m->lnf_g, (size_t)h * 2);
    ALLOC(m->lnf_b, (size_t)h * 2);

    // KV caches: per block and layer
    const size_t slabs = (size_t)m->M * c.n_heads;
    size_t kc_b, kp_b;
    kv_bytes(slabs, c.head_dim, m->cap, &kc_b, &kp_b);
    m->kv.resize((size_t)r.n_blocks * L);
    for (int b = 0; b < r.n_blocks; b++)
        for (int l = 0; l < L; l++) {
            uint8_t *kc, *vc;
            uint32_t *kp, *vp;
            if (l >= L - m->kv_host) {
                // host KV tier: pinned and coherent, so the append kernel's stores through to it
                // are visible to the later copies into the HBM slot
                void *p = nullptr;
                const size_t bytes = 2 * (kc_b + kp_b);
                hipError_t e = hipHostMalloc(&p, bytes, hipHostMallocCoherent);
                if (e != hipSuccess) {
                    (void)hipGetLastError();
                    return fail(TOD_ENOMEM, "hipHostMalloc(%zu bytes) for the KV cache of layer %d failed: %s", bytes,
                                l, hipGetErrorString(e));
                }
                m->host_allocs.push_back(p);
                uint8_t *base = static_cast<uint8_t *>(p);
                kc = base;
                vc = base + kc_b;
                kp = reinterpret_cast<uint32_t *>(base + 2 * kc_b);
                vp = reinterpret_cast<uint32_t *>(base + 2 * kc_b + kp_b);
            } else {
                ALLOC(kc, kc_b);
                ALLOC(vc, kc_b);
                ALLOC(kp, kp_b);
                ALLOC(vp, kp_b);
            }
            m->kv[(size_t)b * L + l] = make_kv_view(kc, kp, vc, vp, c.n_heads, c.head_dim, m->cap);
        }
    if (m->kv_host > 0) // two HBM slots of one block-layer each
        for (int i = 0; i < 2; i++) {
            uint8_t *kc, *vc;
            uint32_t *kp, *vp;
            ALLOC(kc, kc_b);
            ALLOC(vc, kc_b);
            ALLOC(kp, kp_b);
            ALLOC(vp, kp_b);
            m->kvslot[i] = make_kv_view(kc, kp, vc, vp, c.n_heads, c.head_dim, m->cap);
        }

    // activations: prefill processes one batch (b * s rows) per layer call; the
    // block's prefill hidden states are kept for all K batches
    const int64_t prow = (int64_t)r.gpu_batch * r.prompt_len;
    const int64_t arow = prow > m->M ? prow : m->M;
    ALLOC(m->hid, (size_t)m->M * r.prompt_len * h * 2);
    ALLOC(m->act, (size_t)arow * h * 2);
    ALLOC(m->qkv, (size_t)arow * 3 * h * 2);
    ALLOC(m->att, (size_t)arow * h * 2);
    ALLOC(m->ffn, (size_t)arow * f * 2);
    ALLOC(m->last, (size_t)m->M * h * 2);
    ALLOC(m->logits, (size_t)m->M * c.vocab * 2);
    ALLOC(m->ids, (size_t)m->M * 4);
    size_t ws = 0;
    const int rows_list[2] = {m->M, (int)prow};
    for (int ri = 0; ri < 2; ri++)
        for (int mat = 0; mat < N_GEMM_MATS; mat++) {
            const size_t b = gemm_workspace_bytes(rows_list[ri], m->n_out[mat], m->n_in[mat], m->int4);
            ws = b > ws ? b : ws;
        }
    {
        const size_t b = gemm_workspace_bytes(m->M, c.vocab, h, false);
        ws = b > ws ? b : ws;
    }
    m->ws_bytes = ws;
    {
        const GemmPlanInfo qp = gemm_plan_info(m->M, m->n_out[MAT_QKV], m->n_in[MAT_QKV], m->int4);
        const char *t = getenv("TOD_QKV_APPEND");
        m->qkv_append = m->int4 && qp.pipelined && qp.splits == 1 && h % 64 == 0 && c.head_dim % 64 == 0 &&
                        !(t && atoi(t) == 0);
    }
    ALLOC(m->ws, ws);

    if (host && n_streamed > 0) {
        ALLOC(m->slot[0], (size_t)m->layer_bytes);
        ALLOC(m->slot[1], (size_t)m->layer_bytes);
    }
    if (host || m->kv_host > 0) { // the copy stream and the events that order slot reuse
        HIPCHK(hipStreamCreateWithFlags(&m->copy, hipStreamNonBlocking));
        for (int i = 0; i < 2; i++) {
            HIPCHK(hipEventCreateWithFlags(&m->ev_loaded[i], hipEventDisableTiming));
            HIPCHK(hipEventCreateWithFlags(&m->ev_free[i], hipEventDisableTiming));
            HIPCHK(hipEventCreateWithFlags(&m->ev_kv_loaded[i], hipEventDisableTiming));
            HIPCHK(hipEventCreateWithFlags(&m->ev_kv_free[i], hipEventDisableTiming));
        }
    }
    if (m->on_disk) { // two pinned staging images, the I/O stream and its events
        for (int i = 0; i < 2; i++) {
            void *p = nullptr;
            hipError_t e = hipHostMalloc(&p, (size_t)m->image_stride, hipHostMallocDefault);
            if (e != hipSuccess) {
                (void)hipGetLastError();
                return fail(TOD_ENOMEM, "hipHostMalloc(%lld bytes) for a staging image failed: %s",
                            (long long)m->image_stride, hipGetErrorString(e));
            }
            m->host_allocs.push_back(p);
            m->staging[i] = static_cast<uint8_t *>(p);
            HIPCHK(hipEventCreateWithFlags(&m->ev_staged[i], hipEventDisableTiming));
            HIPCHK(hipEventCreateWithFlags(&m->ev_staging_free[i], hipEventDisableTiming));
        }
        HIPCHK(hipStreamCreateWithFlags(&m->io, hipStreamNonBlocking));
    }
    if (m->int4) { // quantization staging for the HBM and int4 host tiers
        const int64_t big = (int64_t)(f > 3 * h ? f : 3 * h) * h;
        ALLOC(m->stage, (size_t)big * 2);
        ALLOC(m->stage_codes, (size_t)big / 2);
        ALLOC(m->stage_scale, (size_t)big / 64 * 2);
        ALLOC(m->stage_zero, (size_t)big / 64 * 2);
    }
    m->prefilled.assign(r.n_blocks, 0);
    m->decoded.assign(r.n_blocks, 0);
    m->gexec.assign(r.n_blocks, nullptr);
    m->gfail.assign(r.n_blocks, 0);
    if (!host) {
        ALLOC(m->gpos, sizeof(int));
        ALLOC(m->gids, (size_t)m->M * 4);
        HIPCHK(hipStreamCreateWithFlags(&m->gstream, hipStreamNonBlocking));
        HIPCHK(hipEventCreateWithFlags(&m->gev_in, hipEventDisableTiming));
        HIPCHK(hipEventCreateWithFlags(&m->gev_out, hipEventDisableTiming));
    }
    return TOD_OK;
}

int init_model(const tod_model_config *cfg, const tod_run_config *run, void *stream, tod_model **out)
{
    return guard("init_model", [&]() -> int {
        (void)stream;
        if (!out)
            return fail(TOD_EINVAL, "null out pointer");
        *out = nullptr;
        if (int rc = check_config(cfg, run)) // before any allocation or device call
            return rc;
        tod_model *m = new (std::nothrow) tod_model();
        if (!m)
            return fail(TOD_ENOMEM, "no memory for the model");
        const int rc = init_model_impl(cfg, run, m);
        if (rc) {
            char msg[sizeof g_err];
            memcpy(msg, g_err, sizeof msg);
            free_model(m);
            memcpy(g_err, msg, sizeof msg);
            return rc;
        }
        *out = m;
        return TOD_OK;
    });
}

int set_global_weights(tod_model *m, const uint16_t *tok, const uint16_t *pos, const uint16_t *g, const uint16_t *b)
{
    return guard("set_global_weights", [&]() -> int {
        if (!m || !tok || !pos || !g || !b)
            return fail(TOD_EINVAL, "null argument");
        const int h = m->cfg.hidden;
        HIPCHK(hipMemcpy(m->tok_emb, tok, (size_t)m->cfg.vocab * h * 2, hipMemcpyHostToDevice));
        HIPCHK(hipMemcpy(m->pos_emb, pos, (size_t)(m->cfg.max_pos + 2) * h * 2, hipMemcpyHostToDevice));
        HIPCHK(hipMemcpy(m->lnf_g, g, (size_t)h * 2, hipMemcpyHostToDevice));
        HIPCHK(hipMemcpy(m->lnf_b, b, (size_t)h * 2, hipMemcpyHostToDevice));
        m->glob_loaded = true;
        return TOD_OK;
    });
}

// Disk tier: synchronous whole-image transfers between staging buffer 0 and the file;
// written images are synced and dropped from the page cache.
static int image_io(tod_model *m, int layer, bool write)
{
    uint8_t *buf = m->staging[0];
    const int64_t off = image_offset(m, layer);
    int64_t done = 0;
    while (done < m->image_stride) {
        const ssize_t n = write ? pwrite(m->fd, buf + done, (size_t)(m->image_stride - done), off + done)
                                : pread(m->fd, buf + done, (size_t)(m->image_stride - done), off + done);
        if (n < 0 && errno == EINTR)
            continue;
        if (n <= 0)
            return fail(TOD_EHIP, "weight file %s of layer %d failed: %s", write ? "write" : "read", layer,
                        n < 0 ? strerror(errno) : "short transfer");
        done += n;
    }
    if (write && fdatasync(m->fd) != 0)
        return fail(TOD_EHIP, "weight file sync failed: %s", strerror(errno));
    (void)posix_fadvise(m->fd, off, m->image_stride, POSIX_FADV_DONTNEED); // keep it out of RAM
    return TOD_OK;
}

int set_weight_file(tod_model *m, const char *path)
{
    return guard("set_weight_file", [&]() -> int {
        if (!m || !path)
            return fail(TOD_EINVAL, "null argument");
        if (!m->on_disk)
            return fail(TOD_ESTATE, "the model was not created with weights_on_disk");
        if (m->fd >= 0)
            return fail(TOD_ESTATE, "the weight file is already set");
        for (const LayerStore &L : m->layers)
            if (L.loaded)
                return fail(TOD_ESTATE, "set_weight_file must come before set_layer_weights");
        const int fd = open(path, O_RDWR | O_CREAT | O_TRUNC, 0600);
        if (fd < 0)
            return fail(TOD_EINVAL, "cannot open %s: %s", path, strerror(errno));
        m->fd = fd;
        return TOD_OK;
    });
}

int set_layer_weights(tod_model *m, int layer, const uint16_t *const *t)
{
    return guard("set_layer_weights", [&]() -> int {
        if (!m || !t)
            return fail(TOD_EINVAL, "null argument");
        if (layer < 0 || layer >= m->cfg.n_layers)
            return fail(TOD_EINVAL, "layer %d out of range", layer);
        if (m->on_disk && m->fd < 0)
            return fail(TOD_ESTATE, "set_weight_file must come before set_layer_weights");
        for (int i = 0; i < TOD_LAYER_TENSORS; i++)
            if (!t[i])
                return fail(TOD_EINVAL, "tensor %d of layer %d is null", i, layer);
        LayerStore &L = m->layers[layer];
        const int h = m->cfg.hidden, f = m->cfg.ffn;
        const size_t hb = (size_t)h * 2;
        HIPCHK(hipMemcpy(L.ln1_g, t[TOD_LN1_G], hb, hipMemcpyHostToDevice));
        HIPCHK(hipMemcpy(L.ln1_b, t[TOD_LN1_B], hb, hipMemcpyHostToDevice));
        HIPCHK(hipMemcpy(L.ln2_g, t[TOD_LN2_G], hb, hipMemcpyHostToDevice));
        HIPCHK(hipMemcpy(L.ln2_b, t[TOD_LN2_B], hb, hipMemcpyHostToDevice));
        HIPCHK(hipMemcpy(L.bias[MAT_QKV], t[TOD_Q_B], hb, hipMemcpyHostToDevice));
        HIPCHK(hipMemcpy(L.bias[MAT_QKV] + h, t[TOD_K_B], hb, hipMemcpyHostToDevice));
        HIPCHK(hipMemcpy(L.bias[MAT_QKV] + 2 * h, t[TOD_V_B], hb, hipMemcpyHostToDevice));
        HIPCHK(hipMemcpy(L.bias[MAT_O], t[TOD_O_B], hb, hipMemcpyHostToDevice));
        HIPCHK(hipMemcpy(L.bias[MAT_FC1], t[TOD_FC1_B], (size_t)f * 2, hipMemcpyHostToDevice));
        HIPCHK(hipMemcpy(L.bias[MAT_FC2], t[TOD_FC2_B], hb, hipMemcpyHostToDevice));
        // the six matrices: (source tensor, gemm matrix, row offset inside it, rows, cols)
        struct Part {
            int tensor, mat, row0, rows, cols;
        } parts[6] = {{TOD_Q_W, MAT_QKV, 0, h, h},   {TOD_K_W, MAT_QKV, h, h, h}, {TOD_V_W, MAT_QKV, 2 * h, h, h},
                      {TOD_O_W, MAT_O, 0, h, h},     {TOD_FC1_W, MAT_FC1, 0, f, h}, {TOD_FC2_W, MAT_FC2, 0, h, f}};
        const bool resident = m->streamed && layer < m->hbm_layers;
        if (m->streamed) { // slot 0 serves as scratch below and an image may change: drop the prefetch
            HIPCHK(hipDeviceSynchronize());
            m->prefetched = false;
        }
        if (m->streamed && !resident && image_layer(m, layer) != layer) {
            // this streamed layer reuses the pinned image of an earlier one
        } else if (!m->int4) {
            uint8_t *image = m->on_disk ? m->staging[0] : L.host; // the disk tier stages, then writes
            for (const Part &p : parts) {
                const int64_t off = m->mat_off[p.mat] + ((int64_t)p.row0 * p.cols) * 2;
                const size_t bytes = (size_t)p.rows * p.cols * 2;
                if (resident)
                    HIPCHK(hipMemcpy(L.dev + off, t[p.tensor], bytes, hipMemcpyHostToDevice));
                else
                    memcpy(image + off, t[p.tensor], bytes);
            }
            int rc;
            if (m->on_disk && !resident && (rc = image_io(m, layer, true)))
                return rc;
        } else {
            // quantize in HBM; on the int4 host tier a resident layer's image is
            // built in place, a streamed one's in slot 0 (idle outside a pass) and
            // then copied to its pinned buffer
            const uint8_t *image = !m->streamed ? nullptr : resident ? L.dev : m->slot[0];
            HIPCHK(hipDeviceSynchronize());
            for (const Part &p : parts) {
                const int64_t n = (int64_t)p.rows * p.cols;
                const int KG = p.cols / 64;
                HIPCHK(hipMemcpy(m->stage, t[p.tensor], (size_t)n * 2, hipMemcpyHostToDevice));
                HIPCHK(launch_quantize_groupwise(m->stage, n, m->stage_codes, m->stage_scale, m->stage_zero, nullptr));
                const int64_t nb0 = p.row0 / 32;
                GemmArgs dst{};
                weights_of(m, L, p.mat, image, dst);
                HIPCHK(launch_repack_w4(m->stage_codes, m->stage_scale, m->stage_zero, p.rows, p.cols,
                                        const_cast<uint32_t *>(dst.wc) + nb0 * KG * 256,
                                        const_cast<uint32_t *>(dst.wp) + nb0 * KG * 32, nullptr));
            }
            HIPCHK(hipDeviceSynchronize());
            if (m->streamed && !resident) {
                HIPCHK(hipMemcpy(m->on_disk ? m->staging[0] : L.host, m->slot[0], (size_t)m->layer_bytes,
                                 hipMemcpyDeviceToHost));
                int rc;
                if (m->on_disk && (rc = image_io(m, layer, true)))
                    return rc;
            }
        }
        L.loaded = true;
        return TOD_OK;
    });
}

int prefill(tod_model *m, int block, const int32_t *d_ids, int32_t *d_next, uint16_t *d_logits, void *stream)
{
    return guard("prefill", [&]() -> int {
        int rc = check_ready(m, block);
        if (rc)
            return rc;
        if (!d_ids || !d_next)
            return fail(TOD_EINVAL, "null ids");
        const hipStream_t st = S(stream);
        const int b = m->run.gpu_batch, K = m->run.batches_per_block, s = m->run.prompt_len, h = m->cfg.hidden;
        const int64_t brow = (int64_t)b * s; // rows of one batch
        for (int k = 0; k < K; k++) {
            ProfScope ps(m, TOD_K_EMBED, st);
            HIPCHK(launch_embed(d_ids + k * brow, (int)brow, s, 0, nullptr, m->tok_emb, m->cfg.vocab, m->pos_emb, h,
                                    m->hid + k * brow * h, st));
        }
        auto layer = [&](int l, const uint8_t *wslot, const KvView &kv, const KvView *mirror) -> int {
            for (int kk = 0; kk < K; kk++) {
                const int k = (l & 1) ? K - 1 - kk : kk; // zig-zag: alternate the batch order per layer
                uint16_t *hk = m->hid + k * brow * h;
                int r = tap_copy(m, 0, l, hk, k * brow, brow, false, st);
                if (!r)
                    r = layer_pass(m, l, kv, hk, (int)brow, true, k * b, s, 0, nullptr, wslot, st, false, nullptr,
                                   nullptr, mirror);
                if (!r)
                    r = tap_copy(m, 0, l, hk, k * brow, brow, true, st);
                if (r)
                    return r;
            }
            return TOD_OK;
        };
        rc = stack_pass(m, st, block, 0, layer);
        if (rc)
            return rc;
        HIPCHK(launch_gather_rows(m->hid + (int64_t)(s - 1) * h, (int64_t)s * h, m->M, h, m->last, st));
        if ((rc = head_pass(m, m->last, m->M, d_logits ? d_logits : m->logits, d_next, st)))
            return rc;
        m->prefilled[block] = 1;
        m->decoded[block] = 0;
        return TOD_OK;
    });
}

// One decode step of a block: embed the ids at `pos`, every layer, head and argmax
// into `out`. With dpos set (captured steps), the position is read from device
// memory and advanced by the step itself.
static int decode_step(tod_model *m, int block, const int32_t *in, int pos, const int *dpos, uint16_t *logits,
                       int32_t *out, hipStream_t st)
{
    const int Mr = m->M, h = m->cfg.hidden, L = m->cfg.n_layers;
    {
        ProfScope ps(m, TOD_K_EMBED, st);
        HIPCHK(launch_embed(in, Mr, 1, pos, dpos, m->tok_emb, m->cfg.vocab, m->pos_emb, h, m->hid, st));
    }
    // all M rows pass each layer together, so every LayerNorm after the first
    // comes out of the GEMM before it (the last one is the head's LN_f)
    // host-KV layers load the pos positions cached before this step (the graph path,
    // whose position lives on the device, is not taken when there are any)
    auto layer = [&](int l, const uint8_t *wslot, const KvView &kv, const KvView *mirror) -> int {
        const bool last = l + 1 == L;
        const uint16_t *ng = last ? m->lnf_g : m->layers[l + 1].ln1_g;
        const uint16_t *nb = last ? m->lnf_b : m->layers[l + 1].ln1_b;
        int r = tap_copy(m, 1, l, m->hid, 0, Mr, false, st);
        if (!r)
            r = layer_pass(m, l, kv, m->hid, Mr, false, 0, 1, pos, dpos, wslot, st, l > 0, ng, nb, mirror);
        if (!r)
            r = tap_copy(m, 1, l, m->hid, 0, Mr, true, st);
        return r;
    };
    int rc = stack_pass(m, st, block, pos, layer);
    if (rc)
        return rc;
    if ((rc = head_pass(m, m->hid, Mr, logits, out, st, true)))
        return rc;
    if (dpos)
        HIPCHK(launch_increment_int(const_cast<int *>(dpos), st));
    return TOD_OK;
}

// Capture one decode step of `block` into a graph (kernels only: no memsets,
// copies or events inside). Returns false if capture is not possible here.
static bool capture_step(tod_model *m, int block)
{
    hipGraph_t graph = nullptr;
    if (hipStreamBeginCapture(m->gstream, hipStreamCaptureModeThreadLocal) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    const int rc = decode_step(m, block, m->gids, 0, m->gpos, m->logits, m->gids, m->gstream);
    const hipError_t e = hipStreamEndCapture(m->gstream, &graph);
    if (rc || e != hipSuccess || !graph) {
        (void)hipGetLastError();
        if (graph)
            (void)hipGraphDestroy(graph);
        return false;
    }
    hipGraphExec_t exec = nullptr;
    const hipError_t ei = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (ei != hipSuccess || !exec) {
        (void)hipGetLastError();
        return false;
    }
    m->gexec[block] = exec;
    return true;
}

int decode_block(tod_model *m, int block, int n_steps, const int32_t *d_ids_in, int32_t *d_ids_out,
                 uint16_t *d_logits, void *stream)
{
    return guard("decode_block", [&]() -> int {
        int rc = check_ready(m, block);
        if (rc)
            return rc;
        if (!d_ids_in || !d_ids_out || n_steps < 0)
            return fail(TOD_EINVAL, "bad decode arguments");
        if (!m->prefilled[block])
            return fail(TOD_ESTATE, "decode_block before prefill on block %d", block);
        if (m->decoded[block] + n_steps > m->run.gen_len - 1)
            return fail(TOD_ESTATE, "decode would exceed gen_len - 1 = %d steps (done %d, asked %d)",
                        m->run.gen_len - 1, m->decoded[block], n_steps);
        const hipStream_t st = S(stream);
        const int Mr = m->M, V = m->cfg.vocab;
        const bool graph = n_steps > 0 && m->graphs_on && !m->prof_mask && !m->n_decode_taps && m->gstream &&
                           m->run.weight_tier == TOD_W_HBM_INT4 && m->kv_host == 0 && !m->gfail[block] &&
                           (m->gexec[block] || capture_step(m, block) || (m->gfail[block] = 1, false));
        if (graph) {
            // replay on the model's stream, ordered after and before the caller's
            HIPCHK(hipEventRecord(m->gev_in, st));
            HIPCHK(hipStreamWaitEvent(m->gstream, m->gev_in, 0));
            HIPCHK(hipMemcpyAsync(m->gids, d_ids_in, (size_t)Mr * 4, hipMemcpyDeviceToDevice, m->gstream));
            HIPCHK(launch_set_int(m->gpos, m->run.prompt_len + m->decoded[block], m->gstream));
            for (int j = 0; j < n_steps; j++) {
                HIPCHK(hipGraphLaunch(m->gexec[block], m->gstream));
                HIPCHK(hipMemcpyAsync(d_ids_out + (int64_t)j * Mr, m->gids, (size_t)Mr * 4, hipMemcpyDeviceToDevice,
                                      m->gstream));
                if (d_logits)
                    HIPCHK(hipMemcpyAsync(d_logits + (int64_t)j * Mr * V, m->logits, (size_t)Mr * V * 2,
                                          hipMemcpyDeviceToDevice, m->gstream));
                m->decoded[block]++;
            }
            HIPCHK(hipEventRecord(m->gev_out, m->gstream));
            HIPCHK(hipStreamWaitEvent(st, m->gev_out, 0));
            return TOD_OK;
        }
        for (int j = 0; j < n_steps; j++) {
            const int pos = m->run.prompt_len + m->decoded[block];
            const int32_t *in = j == 0 ? d_ids_in : d_ids_out + (int64_t)(j - 1) * Mr;
            uint16_t *lg = d_logits ? d_logits + (int64_t)j * Mr * V : m->logits;
            if ((rc = decode_step(m, block, in, pos, nullptr, lg, d_ids_out + (int64_t)j * Mr, st)))
                return rc;
            m->decoded[block]++;
        }
        return TOD_OK;
    });
}

int set_decode_graph(tod_model *m, int enable)
{
    return guard("set_decode_graph", [&]() -> int {
        if (!m)
            return fail(TOD_EINVAL, "null model");
        m->graphs_on = enable != 0;
        return TOD_OK;
    });
}

int set_layer_tap(tod_model *m, int phase, int layer, int64_t row0, int64_t n_rows, uint16_t *d_in,
                  uint16_t *d_out)
{
    return guard("set_layer_tap", [&]() -> int {
        if (!m)
            return fail(TOD_EINVAL, "null model");
        if (phase != 0 && phase != 1)
            return fail(TOD_EINVAL, "phase must be 0 (prefill) or 1 (decode), got %d", phase);
        if (layer < 0 || layer >= m->cfg.n_layers)
            return fail(TOD_EINVAL, "layer %d out of range", layer);
        const int64_t limit = phase == 0 ? (int64_t)m->M * m->run.prompt_len : (int64_t)m->M;
        if (n_rows < 0 || row0 < 0 || row0 + n_rows > limit)
            return fail(TOD_EINVAL, "tap rows [%lld, %lld) outside the pass's %lld rows", (long long)row0,
                        (long long)(row0 + n_rows), (long long)limit);
        if (n_rows > 0 && !d_in && !d_out)
            return fail(TOD_EINVAL, "a tap needs d_in or d_out");
        std::vector<tod_model::Tap> &taps = m->taps[phase];
        if (taps.empty())
            taps.resize(m->cfg.n_layers);
        tod_model::Tap &t = taps[layer];
        if (phase == 1)
            m->n_decode_taps += (n_rows > 0) - (t.n > 0);
        t.row0 = row0;
        t.n = n_rows;
        t.in = d_in;
        t.out = d_out;
        return TOD_OK;
    });
}

int set_decode_position(tod_model *m, int block, int steps)
{
    return guard("set_decode_position", [&]() -> int {
        if (!m)
            return fail(TOD_EINVAL, "null model");
        if (block < 0 || block >= m->run.n_blocks)
            return fail(TOD_ESTATE, "block %d out of range", block);
        if (!m->prefilled[block])
            return fail(TOD_ESTATE, "block %d has not been prefilled", block);
        if (steps < 0 || steps > m->run.gen_len - 1)
            return fail(TOD_EINVAL, "steps %d outside [0, %d]", steps, m->run.gen_len - 1);
        m->decoded[block] = steps;
        return TOD_OK;
    });
}

int quantize_groupwise(const uint16_t *d_x, int64_t n, int group, uint8_t *d_codes, uint16_t *d_scale,
                       uint16_t *d_zero, void *stream)
{
    return guard("quantize_groupwise", [&]() -> int {
        if (group != TOD_GROUP)
            return fail(TOD_EINVAL, "group must be 64 (got %d)", group);
        if (n < 0 || n % group)
            return fail(TOD_EINVAL, "n (%lld) must be a non-negative multiple of %d", (long long)n, group);
        if (n && (!d_x || !d_codes || !d_scale || !d_zero))
            return fail(TOD_EINVAL, "null pointer");
        HIPCHK(launch_quantize_groupwise(d_x, n, d_codes, d_scale, d_zero, S(stream)));
        return TOD_OK;
    });
}

int dequantize_groupwise(const uint8_t *d_codes, const uint16_t *d_scale, const uint16_t *d_zero, int64_t n,
                         int group, uint16_t *d_out, void *stream)
{
    return guard("dequantize_groupwise", [&]() -> int {
        if (group != TOD_GROUP)
            return fail(TOD_EINVAL, "group must be 64 (got %d)", group);
        if (n < 0 || n % group)
            return fail(TOD_EINVAL, "n must be a non-negative multiple of 64");
        if (n && (!d_codes || !d_scale || !d_zero || !d_out))
            return fail(TOD_EINVAL, "null pointer");
        HIPCHK(launch_dequantize_groupwise(d_codes, d_scale, d_zero, n, d_out, S(stream)));
        return TOD_OK;
    });
}

int export_weight(tod_model *m, int layer, int which, uint8_t *d_codes, uint16_t *d_scale, uint16_t *d_zero,
                  void *stream)
{
    return guard("export_weight", [&]() -> int {
        if (!m || !d_codes || !d_scale || !d_zero)
            return fail(TOD_EINVAL, "null argument");
        if (layer < 0 || layer >= m->cfg.n_layers || which < TOD_MAT_Q || which > TOD_MAT_FC2)
            return fail(TOD_EINVAL, "layer or matrix id out of range");
        if (!m->int4)
            return fail(TOD_ESTATE, "the fp16 host tier keeps fp16 weights");
        if (!m->layers[layer].loaded)
            return fail(TOD_ESTATE, "layer %d weights not set", layer);
        const uint8_t *slot = nullptr;
        if (m->streamed && layer < m->hbm_layers) {
            slot = m->layers[layer].dev;
        } else if (m->streamed) { // bring the layer's pinned image into slot 0 (idle outside a pass)
            const int src = image_layer(m, layer);
            if (!m->layers[src].loaded)
                return fail(TOD_ESTATE, "layer %d (whose image layer %d streams) weights not set", src, layer);
            HIPCHK(hipDeviceSynchronize());
            m->prefetched = false; // slot 0 is overwritten here
            int rc;
            if (m->on_disk && (rc = image_io(m, layer, false)))
                return rc;
            HIPCHK(hipMemcpy(m->slot[0], m->on_disk ? m->staging[0] : m->layers[src].host, (size_t)m->layer_bytes,
                             hipMemcpyHostToDevice));
            slot = m->slot[0];
        }
        const int h = m->cfg.hidden, f = m->cfg.ffn;
        int mat, row0 = 0, rows = h, cols = h;
        switch (which) {
        case TOD_MAT_Q: mat = MAT_QKV; break;
        case TOD_MAT_K: mat = MAT_QKV; row0 = h; break;
        case TOD_MAT_V: mat = MAT_QKV; row0 = 2 * h; break;
        case TOD_MAT_O: mat = MAT_O; break;
        case TOD_MAT_FC1: mat = MAT_FC1; rows = f; break;
        default: mat = MAT_FC2; cols = f; break;
        }
        const int KG = cols / 64;
        const int64_t nb0 = row0 / 32;
        GemmArgs src{};
        weights_of(m, m->layers[layer], mat, slot, src);
        HIPCHK(launch_unpack_w4(src.wc + nb0 * KG * 256, src.wp + nb0 * KG * 32, rows, cols, d_codes, d_scale, d_zero,
                                S(stream)));
        return TOD_OK;
    });
}

int export_kv(tod_model *m, int layer, int block, int row, int head, int t0, int t1, uint8_t *d_kc, uint16_t *d_ks,
              uint16_t *d_kz, uint8_t *d_vc, uint16_t *d_vs, uint16_t *d_vz, void *stream)
{
    return guard("export_kv", [&]() -> int {
        if (!m || !d_kc || !d_ks || !d_kz || !d_vc || !d_vs || !d_vz)
            return fail(TOD_EINVAL, "null argument");
        if (layer < 0 || layer >= m->cfg.n_layers || block < 0 || block >= m->run.n_blocks || row < 0 || row >= m->M ||
            head < 0 || head >= m->cfg.n_heads || t0 < 0 || t1 > m->cap || t0 > t1)
            return fail(TOD_EINVAL, "export_kv index out of range");
        HIPCHK(launch_kv_export(m->kv[(size_t)block * m->cfg.n_layers + layer], row, head, t0, t1, d_kc, d_ks, d_kz,
                                d_vc, d_vs, d_vz, S(stream)));
        return TOD_OK;
    });
}

// Argument rules of the linear entry points (no device work).
static int check_linear(const uint16_t *d_a, int64_t rows, int in, int out, const uint8_t *d_codes,
                        const uint16_t *d_scale, const uint16_t *d_zero, const uint16_t *d_w,
                        const uint16_t *d_residual, int relu, const uint16_t *d_y)
{
    if (!d_a || !d_y || rows < 0 || rows > 0x7fffffff || in <= 0 || out <= 0)
        return fail(TOD_EINVAL, "bad linear arguments");
    if (in % 64)
        return fail(TOD_EINVAL, "in (%d) must be a multiple of 64", in);
    const bool int4 = d_codes != nullptr;
    if (int4 && (out % 32 || !d_scale || !d_zero))
        return fail(TOD_EINVAL, "int4 linear needs out %% 32 == 0 and scale/zero");
    if (!int4 && !d_w)
        return fail(TOD_EINVAL, "null weights");
    if (relu && d_residual)
        return fail(TOD_EINVAL, "relu with residual is not an epilogue of this library");
    return TOD_OK;
}

// The GEMM of a linear call, given device memory for the repacked int4 weights (tc, tp; int4
// only) and for the split-K partials (ws, gemm_workspace_bytes of the shape).
static int run_linear(const uint16_t *d_a, int64_t rows, int in, int out, const uint8_t *d_codes,
                      const uint16_t *d_scale, const uint16_t *d_zero, const uint16_t *d_w, const uint16_t *d_bias,
                      const uint16_t *d_residual, int relu, uint16_t *d_y, uint32_t *tc, uint32_t *tp, float *ws,
                      hipStream_t st)
{
    GemmArgs g{};
    g.a = d_a;
    g.lda = in;
    if (d_codes) {
        hipError_t e = launch_repack_w4(d_codes, d_scale, d_zero, out, in, tc, tp, st);
        if (e != hipSuccess)
            return fail(TOD_EHIP, "repack failed: %s", hipGetErrorString(e));
        g.wc = tc;
        g.wp = tp;
    } else {
        g.wf = d_w;
    }
    g.bias = d_bias;
    g.residual = d_residual;
    g.y = d_y;
    g.ldc = out;
    g.M = (int)rows;
    g.N = out;
    g.K = in;
    g.epi = relu ? EPI_BIAS_RELU : (d_residual ? EPI_BIAS_RES : (d_bias ? EPI_BIAS : EPI_NONE));
    g.ws_bytes = gemm_workspace_bytes((int)rows, out, in, d_codes != nullptr);
    g.ws = ws;
    hipError_t e = launch_gemm(g, st);
    if (e != hipSuccess)
        return fail(TOD_EHIP, "gemm failed: %s", hipGetErrorString(e));
    return TOD_OK;
}

static int linear_common(const uint16_t *d_a, int64_t rows, int in, int out, const uint8_t *d_codes,
                         const uint16_t *d_scale, const uint16_t *d_zero, const uint16_t *d_w, const uint16_t *d_bias,
                         const uint16_t *d_residual, int relu, uint16_t *d_y, void *stream)
{
    int rc = check_linear(d_a, rows, in, out, d_codes, d_scale, d_zero, d_w, d_residual, relu, d_y);
    if (rc)
        return rc;
    const hipStream_t st = S(stream);
    std::vector<void *> tmp;
    auto cleanup = [&]() {
        (void)hipStreamSynchronize(st);
        for (void *p : tmp)
            (void)hipFree(p);
    };
    auto talloc = [&](size_t bytes) -> void * {
        void *p = nullptr;
        if (bytes && hipMalloc(&p, bytes) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        tmp.push_back(p);
        return p;
    };
    uint32_t *tc = nullptr, *tp = nullptr;
    if (d_codes) {
        const int64_t n = (int64_t)out * in;
        tc = static_cast<uint32_t *>(talloc((size_t)n / 2));
        tp = static_cast<uint32_t *>(talloc((size_t)n / 64 * 4));
        if (!tc || !tp) {
            cleanup();
            return fail(TOD_ENOMEM, "no memory for the repacked weights");
        }
    }
    const size_t ws_bytes = gemm_workspace_bytes((int)rows, out, in, d_codes != nullptr);
    float *ws = static_cast<float *>(talloc(ws_bytes));
    if (ws_bytes && !ws) {
        cleanup();
        return fail(TOD_ENOMEM, "no memory for the split-K workspace");
    }
    rc = run_linear(d_a, rows, in, out, d_codes, d_scale, d_zero, d_w, d_bias, d_residual, relu, d_y, tc, tp, ws, st);
    cleanup();
    return rc;
}

// Scratch of linear_w4_noalloc: the repacked weights and split-K partials of one call, so that
// the call allocates nothing. In host code `scratch` names a host-side stand-in, not a device
// address: host code uses only the address scratch_base() looked up for the current device.
constexpr size_t kNoallocBytes = TOD_LINEAR_NOALLOC_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kNoallocBytes];

// The current device's address of `scratch`: looked up on the device's first call, then kept.
static int scratch_base(uint8_t **out)
{
    static std::atomic<uint8_t *> addr[kMaxDevices];
    int dev = -1;
    HIPCHK(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(TOD_EINVAL, "device %d beyond the %d this library tracks", dev, kMaxDevices);
    uint8_t *p = addr[dev].load();
    if (!p) {
        void *q = nullptr;
        HIPCHK(hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)));
        p = static_cast<uint8_t *>(q);
        addr[dev].store(p);
    }
    *out = p;
    return TOD_OK;
}

static size_t round256(size_t b) { return (b + 255) / 256 * 256; }

int linear_w4(const uint16_t *d_a, int64_t rows, int in, int out, const uint8_t *d_codes, const uint16_t *d_scale,
              const uint16_t *d_zero, const uint16_t *d_bias, const uint16_t *d_residual, int relu, uint16_t *d_y,
              void *stream)
{
    return guard("linear_w4", [&]() -> int {
        if (!d_codes)
            return fail(TOD_EINVAL, "null codes");
        return linear_common(d_a, rows, in, out, d_codes, d_scale, d_zero, nullptr, d_bias, d_residual, relu, d_y,
                             stream);
    });
}

int linear_w4_noalloc(const uint16_t *d_a, int64_t rows, int in, int out, const uint8_t *d_codes,
                      const uint16_t *d_scale, const uint16_t *d_zero, const uint16_t *d_bias,
                      const uint16_t *d_residual, int relu, uint16_t *d_y, void *stream)
{
    return guard("linear_w4_noalloc", [&]() -> int {
        if (!d_codes)
            return fail(TOD_EINVAL, "null codes");
        int rc = check_linear(d_a, rows, in, out, d_codes, d_scale, d_zero, nullptr, d_residual, relu, d_y);
        if (rc)
            return rc;
        const size_t n = (size_t)out * in;
        const size_t codes_b = round256(n / 2), params_b = round256(n / 64 * 4);
        const size_t ws_b = gemm_workspace_bytes((int)rows, out, in, true);
        if (codes_b + params_b + ws_b > kNoallocBytes)
            return fail(TOD_EINVAL,
                        "linear_w4_noalloc: %d x %d weights at %lld rows need %zu bytes of scratch, above its %zu",
                        out, in, (long long)rows, codes_b + params_b + ws_b, kNoallocBytes);
        uint8_t *base = nullptr;
        if ((rc = scratch_base(&base)))
            return rc;
        uint32_t *tc = reinterpret_cast<uint32_t *>(base);
        uint32_t *tp = reinterpret_cast<uint32_t *>(base + codes_b);
        float *ws = ws_b ? reinterpret_cast<float *>(base + codes_b + params_b) : nullptr;
        return run_linear(d_a, rows, in, out, d_codes, d_scale, d_zero, nullptr, d_bias, d_residual, relu, d_y, tc, tp,
                          ws, S(stream));
    });
}

int linear_f16(const uint16_t *d_a, int64_t rows, int in, int out, const uint16_t *d_w, const uint16_t *d_bias,
               const uint16_t *d_residual, int relu, uint16_t *d_y, void *stream)
{
    return guard("linear_f16", [&]() -> int {
        return linear_common(d_a, rows, in, out, nullptr, nullptr, nullptr, d_w, d_bias, d_residual, relu, d_y, stream);
    });
}

int profile_kernels(tod_model *m, unsigned mask)
{
    return guard("profile_kernels", [&]() -> int {
        if (!m)
            return fail(TOD_EINVAL, "null model");
        double ms;
        int64_t n;
        int rc = profile_read(m, 0, &ms, &n); // drain pending events
        if (rc)
            return rc;
        m->prof_mask = mask;
        if (mask) { // room for the launches of a few decode steps, so timing rarely grows the lists
            m->pend.reserve(1 << 14);
            m->ev_pool.reserve(1 << 15);
        }
        for (int k = 0; k < TOD_K_COUNT; k++) {
            m->prof_ms[k] = 0.0;
            m->prof_n[k] = 0;
        }
        return TOD_OK;
    });
}

int profile_read(tod_model *m, int kind, double *total_ms, int64_t *launches)
{
    return guard("profile_read", [&]() -> int {
        if (!m || !total_ms || !launches || kind < 0 || kind >= TOD_K_COUNT)
            return fail(TOD_EINVAL, "bad profile_read arguments");
        for (auto &p : m->pend) {
            HIPCHK(hipEventSynchronize(p.b));
            float ms = 0.0f;
            HIPCHK(hipEventElapsedTime(&ms, p.a, p.b));
            m->prof_ms[p.kind] += ms;
            m->prof_n[p.kind]++;
            m->ev_pool.push_back(p.a);
            m->ev_pool.push_back(p.b);
        }
        m->pend.clear();
        *total_ms = m->prof_ms[kind];
        *launches = m->prof_n[kind];
        return TOD_OK;
    });
}

inline bool misaligned16(const void *p) { return ((uintptr_t)p & 15u) != 0; }

int attn_cache_create(int batch, int heads, int head_dim, int cap, tod_attn_cache **out)
{
    return guard("attn_cache_create", [&]() -> int {
        if (!out)
            return fail(TOD_EINVAL, "null out pointer");
        *out = nullptr;
        if (batch <= 0 || heads <= 0 || cap <= 0 || (head_dim != 64 && head_dim != 128))
            return fail(TOD_EINVAL, "bad attention cache shape");
        tod_attn_cache *c = new (std::nothrow) tod_attn_cache();
        if (!c)
            return fail(TOD_ENOMEM, "no memory for the attention cache");
        const int capp = (cap + 63) / 64 * 64;
        size_t kc_b, kp_b;
        kv_bytes((size_t)batch * heads, head_dim, capp, &kc_b, &kp_b);
        void *p[4] = {};
        const size_t sz[4] = {kc_b, kp_b, kc_b, kp_b};
        for (int i = 0; i < 4; i++) {
            if (hipMalloc(&p[i], sz[i]) != hipSuccess) {
                (void)hipGetLastError();
                for (void *q : c->allocs)
                    (void)hipFree(q);
                delete c;
                return fail(TOD_ENOMEM, "hipMalloc of %zu bytes for the attention cache failed", sz[i]);
            }
            c->allocs.push_back(p[i]);
        }
        c->kv = make_kv_view(static_cast<uint8_t *>(p[0]), static_cast<uint32_t *>(p[1]), static_cast<uint8_t *>(p[2]),
                             static_cast<uint32_t *>(p[3]), heads, head_dim, capp);
        c->batch = batch;
        *out = c;
        return TOD_OK;
    });
}

int attn_cache_fill(tod_attn_cache *c, const uint16_t *d_k, const uint16_t *d_v, int t0, int n, void *stream)
{
    return guard("attn_cache_fill", [&]() -> int {
        if (!c || !d_k || !d_v || t0 < 0 || n < 0 || t0 + n > c->kv.cap)
            return fail(TOD_EINVAL, "bad attention cache fill");
        if (misaligned16(d_k) || misaligned16(d_v))
            return fail(TOD_EINVAL, "K/V buffers must be 16-byte aligned");
        // time-major input [n][batch][heads][d]: row r = (sequence r / n, position t0 + r % n)
        const int d = c->kv.head_dim, H = c->kv.heads;
        const SrcMap src = {(int64_t)H * d, (int64_t)c->batch * H * d, d};
        const RowMap map = {0, n, t0, nullptr};
        HIPCHK(launch_kv_append(d_k, d_v, src, c->batch * n, map, c->kv, S(stream)));
        return TOD_OK;
    });
}

int attn_decode_step(tod_attn_cache *c, int pos, const uint16_t *d_q, const uint16_t *d_k_new,
                     const uint16_t *d_v_new, uint16_t *d_out, void *stream)
{
    return guard("attn_decode_step", [&]() -> int {
        if (!c || !d_q || !d_k_new || !d_v_new || !d_out)
            return fail(TOD_EINVAL, "null argument");
        if (pos < 0 || pos >= c->kv.cap)
            return fail(TOD_ESTATE, "position %d outside the cache (capacity %d)", pos, c->kv.cap);
        if (misaligned16(d_q) || misaligned16(d_k_new) || misaligned16(d_v_new) || misaligned16(d_out))
            return fail(TOD_EINVAL, "q, k, v and out buffers must be 16-byte aligned");
        const int d = c->kv.head_dim, H = c->kv.heads;
        const SrcMap src = {(int64_t)H * d, 0, d};
        const RowMap map = {0, 1, pos, nullptr};
        HIPCHK(launch_kv_append(d_k_new, d_v_new, src, c->batch, map, c->kv, S(stream)));
        HIPCHK(launch_attn_decode(d_q, (int64_t)H * d, d_out, (int64_t)H * d, c->batch, 0, pos + 1, nullptr, c->kv,
                                  S(stream)));
        return TOD_OK;
    });
}

int attn_cache_export(tod_attn_cache *c, int seq, int head, int t0, int t1, uint8_t *d_kc, uint16_t *d_ks,
                      uint16_t *d_kz, uint8_t *d_vc, uint16_t *d_vs, uint16_t *d_vz, void *stream)
{
    return guard("attn_cache_export", [&]() -> int {
        if (!c || !d_kc || !d_ks || !d_kz || !d_vc || !d_vs || !d_vz)
            return fail(TOD_EINVAL, "null argument");
        if (seq < 0 || seq >= c->batch || head < 0 || head >= c->kv.heads || t0 < 0 || t1 > c->kv.cap || t0 > t1)
            return fail(TOD_EINVAL, "export index out of range");
        HIPCHK(launch_kv_export(c->kv, seq, head, t0, t1, d_kc, d_ks, d_kz, d_vc, d_vs, d_vz, S(stream)));
        return TOD_OK;
    });
}

int attn_cache_free(tod_attn_cache *c)
{
    return guard("attn_cache_free", [&]() -> int {
        if (!c)
            return TOD_OK;
        (void)hipDeviceSynchronize();
        for (void *p : c->allocs)
            (void)hipFree(p);
        delete c;
        return TOD_OK;
    });
}

} // extern "C"
