// Cost model and placement search for block decode (host code only).
//
// The FlexGen guide's cost simulator ("Implementation: Simulating FlexGen's
// Zig-Zag Block Scheduling in Python") prices a generation step as the time to
// move the weights over PCIe; the FlexLLMGen overview ("A 175B-parameter model
// on one GPU, if you can wait": what it does; caveats) places tensors across
// the memory hierarchy with a policy that is tuned by hand through flags, an
// automatic optimiser being future work. Here the step is priced from the
// measured rates of the library's kernels and of the host link, and the search
// enumerates the run-configuration choices the library offers (weight tier,
// resident layers, GPU batch and batches per block) under the device and
// pinned-host capacities.
//
// Step model at the average decode context c = prompt_len + gen_len / 2:
//  * each GEMM is priced on the tile plan the library launches for it. The
//    pipelined kernel (int4 weights; fp16 weights of N a multiple of 32) runs
//    its workgroups in waves of one per CU; a wave costs its K-groups per
//    workgroup times the time of one K-group (the steady int4 or fp16 rate,
//    scaled by the tile's rows, and for 128- and 64-row int4 tiles by their
//    efficiency loss of 1.1 and 1.5; those sit two per CU and share one fixed
//    cost per pair) plus a fixed
//    cost for pipeline fill and epilogue, and a split K loop adds its fp32
//    partials, written once and read once at the streaming rate; no GEMM is
//    faster than its weight bytes at the streaming rate plus the fixed cost
//    (the fp16 LM head at a few rows is bound there). Fitted to the
//    measured decode GEMMs at 512 rows (OPT-30B) and 256 rows (OPT-6.7B), this
//    is within 8% on each of them (profiles/cost_model_measurements.txt), where
//    one flat rate misses the 256-row GEMMs by up to 2x (their K loops split 4
//    to 16 ways). The
//    register-staged kernel (small GEMMs of 128 rows or fewer; fp16 weights of
//    N not a multiple of 32) costs its own fixed time plus its weight bytes
//    and its flops at that kernel's effective rates (it reads weights at well
//    under HBM bandwidth). Every kernel costs at least one launch floor;
//  * decode attention moves M * heads * (c * (d + d/8) + 4d) bytes at the
//    attention rate; the KV append reads 4d and writes d + d/8 bytes per
//    (row, head); one LayerNorm per step (the others are fused); the LM head is
//    an fp16 GEMM plus the logits' write and the argmax's read;
//  * on the host tiers the L - R streamed layers each copy one layer image at
//    the link rate while the GPU computes; the first streamed copies (at most
//    two, one per slot) overlap the R resident layers, which leaves the link
//    idle for max(0, R * t_layer - min(2, L - R) * t_copy), so the step takes
//    max(compute, link + idle);
//  * each of the last kv_host layers (host KV tier) also copies its ctx - 1
//    cached positions and writes its appended one through, M * heads * ctx *
//    (d + d/8) bytes, over the same link. When no weights stream, the first
//    two host-KV copies (one per slot) can start as soon as the previous pass
//    frees their slots and overlap the L - kv_host layers before them; the
//    link idles for max(0, (L - kv_host) * t_layer - min(2, kv_host) * t_kv);
//  * with the images on disk, a streamed layer's copy takes the longer of its
//    disk read and its link copy (the two overlap across layers).
// The footprint mirrors init_model's allocations. The search takes, for each
// candidate, the fewest host-KV layers that make it fit.
#include <cmath>

#include "api.hpp"
#include "common.hpp"
#include "tod.h"

namespace {

struct Shape {
    double L, h, H, d, f, V, P;
};

double weights_per_layer(const Shape &s) { return 4.0 * s.h * s.h + 2.0 * s.h * s.f; }

double image_bytes(const Shape &s, int tier)
{
    return weights_per_layer(s) * (tier == TOD_W_HOST_FP16_STREAM ? 2.0 : 0.5625);
}

// Device and pinned-host bytes init_model allocates for this configuration.
void footprint(const tod_model_config *c, const tod_run_config *r, double *hbm, double *host, double *wsb,
               double *disk_b)
{
    const Shape s{(double)c->n_layers, (double)c->hidden, (double)c->n_heads, (double)c->head_dim,
                  (double)c->ffn, (double)c->vocab, (double)c->max_pos};
    const int tier = r->weight_tier;
    const bool streamed = tier != TOD_W_HBM_INT4, int4 = tier != TOD_W_HOST_FP16_STREAM;
    const double M = (double)r->gpu_batch * r->batches_per_block;
    const double L = s.L, h = s.h, f = s.f;
    const int R = streamed ? r->hbm_layers : 0;
    const int S = streamed ? c->n_layers - R : 0;
    const int P = r->host_layers > 0 && r->host_layers < S ? r->host_layers : S;
    const double img = image_bytes(s, tier);
    double dev = 0.0;
    // weights: int4 store (tier 0) or resident images and two slots; biases and LayerNorm vectors
    dev += streamed ? R * img + (S > 0 ? 2.0 * img : 0.0) : L * image_bytes(s, TOD_W_HBM_INT4);
    dev += L * ((5.0 * h + f) * 2.0 + 4.0 * h * 2.0);
    dev += s.V * h * 2.0 + (s.P + 2.0) * h * 2.0 + 2.0 * h * 2.0;
    // KV cache: per block, layer and (row, head) slab, codes and params of K and V; the
    // host KV tier keeps its layers' caches pinned and two HBM slots of one block-layer
    const double cap = std::ceil((r->prompt_len + r->gen_len - 1) / 64.0) * 64.0;
    const double slabs = M * s.H;
    const double kv_layer = 2.0 * (slabs * cap * s.d / 2.0 + slabs * cap * (s.d / 64.0) * 4.0);
    const int KVH = r->kv_host_layers;
    dev += r->n_blocks * (L - KVH) * kv_layer + (KVH > 0 ? 2.0 * kv_layer : 0.0);
    // activations
    const double prow = (double)r->gpu_batch * r->prompt_len, arow = prow > M ? prow : M;
    dev += M * r->prompt_len * h * 2.0 + arow * (h + 3.0 * h + h + f) * 2.0 + M * h * 2.0 + M * s.V * 2.0 +
           M * 4.0;
    // split-K workspace
    const int mats[4][2] = {{3 * c->hidden, c->hidden}, {c->hidden, c->hidden}, {c->ffn, c->hidden},
                            {c->hidden, c->ffn}};
    size_t ws = gemm_workspace_bytes((int)M, c->vocab, c->hidden, false);
    for (int rows : {(int)M, (int)prow})
        for (const auto &mk : mats) {
            const size_t b = gemm_workspace_bytes(rows, mk[0], mk[1], int4);
            ws = b > ws ? b : ws;
        }
    dev += (double)ws;
    *wsb = (double)ws;
    // quantization staging (int4 tiers) and the decode-graph buffers (tier 0)
    if (int4) {
        const double big = (f > 3.0 * h ? f : 3.0 * h) * h;
        dev += big * 2.0 + big / 2.0 + 2.0 * (big / 64.0 * 2.0);
    }
    if (!streamed)
        dev += 4.0 + M * 4.0;
    *hbm = dev;
    // pinned: the owned images (or, with the images on disk, two staging images) and host caches
    const double stride = std::ceil(img / 4096.0) * 4096.0;
    const bool on_disk = streamed && r->weights_on_disk;
    *host = (streamed ? (on_disk ? 2.0 * stride : P * img) : 0.0) + r->n_blocks * (double)KVH * kv_layer;
    *disk_b = on_disk ? P * stride : 0.0;
}

// Bytes of one block-layer's KV cache (codes and params of K and V).
double kv_layer_bytes(const tod_model_config *c, const tod_run_config *r)
{
    const double cap = std::ceil((r->prompt_len + r->gen_len - 1) / 64.0) * 64.0;
    const double slabs = (double)r->gpu_batch * r->batches_per_block * c->n_heads;
    return slabs * cap * (c->head_dim + c->head_dim / 8.0);
}

double kernel_time(double work_s, const tod_hw *hw)
{
    return work_s > hw->launch_us * 1e-6 ? work_s : hw->launch_us * 1e-6;
}

constexpr double kCUs = 256.0; // MI355X compute units; one pipelined GEMM workgroup each

// One GEMM of M rows, N outputs and K inputs on the tile plan launch_gemm takes.
double gemm_time(int M, int N, int K, bool int4, const tod_hw *hw)
{
    const GemmPlanInfo p = gemm_plan_info(M, N, K, int4);
    const double mem = hw->mem_gbs * 1e9;
    double t;
    const double wb = (double)N * K * (int4 ? 0.5625 : 2.0);
    if (p.pipelined) {
        const double rate = (int4 ? hw->int4_tflops : hw->fp16_tflops) * 1e12;
        const double t_group = kCUs * 2.0 * 256.0 * 256.0 * 64.0 / rate;
        // shorter int4 tiles lose some efficiency per flop and sit two per CU
        const double eff = !int4 ? 1.0 : p.bm <= 64 ? 1.5 : p.bm <= 128 ? 1.1 : 1.0;
        const double slots = int4 && p.bm <= 128 ? 2.0 * kCUs : kCUs;
        t = std::ceil(p.workgroups / kCUs) * p.groups_per_split * (p.bm / 256.0) * eff * t_group +
            std::ceil(p.workgroups / slots) * hw->gemm_wg_us * 1e-6;
        const double t_read = wb / mem + hw->gemm_wg_us * 1e-6; // few rows: the weight stream
        t = t > t_read ? t : t_read;
        if (p.splits > 1)
            t += 2.0 * p.splits * (double)M * N * 4.0 / mem;
    } else {
        const double flop = 2.0 * M * (double)N * K;
        t = hw->staged_us * 1e-6 + wb / (hw->staged_gbs * 1e9) + flop / (hw->staged_tflops * 1e12);
    }
    return kernel_time(t, hw);
}

void step_model(const tod_model_config *c, const tod_run_config *r, const tod_hw *hw, tod_estimate *e)
{
    const Shape s{(double)c->n_layers, (double)c->hidden, (double)c->n_heads, (double)c->head_dim,
                  (double)c->ffn, (double)c->vocab, (double)c->max_pos};
    const int tier = r->weight_tier;
    const bool streamed = tier != TOD_W_HBM_INT4;
    const double M = (double)r->gpu_batch * r->batches_per_block;
    const double h = s.h, f = s.f, d = s.d;
    const double wbpe = tier == TOD_W_HOST_FP16_STREAM ? 2.0 : 0.5625; // weight bytes per element
    const double mem = hw->mem_gbs * 1e9;
    const double ctx = r->prompt_len + r->gen_len / 2.0;
    // one layer
    const int Mi = r->gpu_batch * r->batches_per_block, hi = c->hidden, fi = c->ffn;
    const int nk[4][2] = {{3 * hi, hi}, {hi, hi}, {fi, hi}, {hi, fi}};
    double t_layer = 0.0;
    for (const auto &g : nk)
        t_layer += gemm_time(Mi, g[0], g[1], tier != TOD_W_HOST_FP16_STREAM, hw);
    const double kvpos = d + d / 8.0; // K and V codes and params per (head, position)
    t_layer += kernel_time(M * s.H * (ctx * kvpos + 4.0 * d) / (hw->attn_gbs * 1e9), hw);
    t_layer += kernel_time(M * s.H * (4.0 * d + kvpos) / mem, hw);
    // head: embedding, the first LayerNorm, LM head GEMM, argmax
    double t_head = kernel_time(M * h * 2.0 * 2.0 / mem, hw) + kernel_time(M * h * 4.0 / mem, hw);
    t_head += gemm_time(Mi, c->vocab, hi, false, hw);
    t_head += kernel_time(M * s.V * 2.0 / mem, hw);
    const double t_comp = s.L * t_layer + t_head;
    double t_link = 0.0, idle = 0.0;
    int S = 0;
    if (streamed) {
        const int R = r->hbm_layers;
        S = c->n_layers - R;
        const double img = weights_per_layer(s) * wbpe;
        const double t_link_img = img / (hw->link_gbs * 1e9);
        // from disk, reads and link copies of consecutive layers overlap: the slower sets the pace
        const double t_copy = r->weights_on_disk && img / (hw->disk_gbs * 1e9) > t_link_img
                                  ? img / (hw->disk_gbs * 1e9)
                                  : t_link_img;
        t_link = S * t_copy;
        if (S > 0) {
            const double overlap = (S < 2 ? S : 2) * t_copy;
            idle = R * t_layer > overlap ? R * t_layer - overlap : 0.0;
        }
    }
    const int KVH = r->kv_host_layers;
    if (KVH > 0) {
        // ctx - 1 cached positions loaded and the new one written through, per host-KV layer
        const double t_kv = M * s.H * ctx * kvpos / (hw->link_gbs * 1e9);
        t_link += KVH * t_kv;
        if (S == 0) { // the first two host-KV copies (one per slot) overlap the layers before them
            const double front = (c->n_layers - KVH) * t_layer, overlap = (KVH < 2 ? KVH : 2) * t_kv;
            idle = front > overlap ? front - overlap : 0.0;
        }
    }
    e->compute_s = t_comp;
    e->link_s = t_link;
    e->step_s = t_link > 0.0 && t_link + idle > t_comp ? t_link + idle : t_comp;
    e->tokens_per_s = M / e->step_s;
}

} // namespace

void default_hw(tod_hw *hw)
{
    if (!hw)
        return;
    hw->attn_gbs = 6100.0;    // decode attention, int4 cache, OPT-30B shape
    hw->mem_gbs = 7100.0;     // streaming reads with nontemporal 16-byte loads
    hw->link_gbs = 57.2;      // one pinned -> HBM copy of a layer image
    hw->int4_tflops = 1260.0; // pipelined int4 GEMMs, steady rate with every CU busy (fitted)
    hw->fp16_tflops = 1300.0; // pipelined fp16-weight GEMMs (LM head), steady rate (fitted)
    hw->launch_us = 4.0;      // per kernel inside a replayed decode graph
    hw->hbm_bytes = 280e9;    // device memory a model may use
    hw->host_bytes = 270e9;   // pinned host memory a process may hold
    hw->disk_gbs = 7.4;       // reads of the weight file (one image per read)
    hw->disk_bytes = 80e9;    // free space for the weight file
    hw->gemm_wg_us = 20.0;    // fixed cost per wave of pipelined GEMM workgroups (fitted)
    hw->staged_tflops = 1700.0; // register-staged GEMM (<= 128 rows): flops, fitted
    hw->staged_gbs = 3230.0;   // register-staged GEMM: weight bytes, fitted
    hw->staged_us = 10.0;      // register-staged GEMM: fixed time (OPT-125m GEMMs at 8 rows)
}

int estimate_decode(const tod_model_config *cfg, const tod_run_config *run, const tod_hw *hw, tod_estimate *out)
{
    return guard("estimate_decode", [&]() -> int {
        if (!out || !hw)
            return fail(TOD_EINVAL, "null argument");
        if (int rc = check_config(cfg, run))
            return rc;
        if (!(hw->attn_gbs > 0.0 && hw->mem_gbs > 0.0 && hw->link_gbs > 0.0 && hw->int4_tflops > 0.0 &&
              hw->fp16_tflops > 0.0 && hw->launch_us >= 0.0 && hw->disk_gbs > 0.0 && hw->gemm_wg_us >= 0.0 &&
              hw->staged_tflops > 0.0 && hw->staged_gbs > 0.0 && hw->staged_us >= 0.0))
            return fail(TOD_EINVAL, "hardware rates must be positive and fixed costs non-negative");
        step_model(cfg, run, hw, out);
        footprint(cfg, run, &out->hbm_bytes, &out->host_bytes, &out->workspace_bytes, &out->disk_bytes);
        out->fits = out->hbm_bytes <= hw->hbm_bytes && out->host_bytes <= hw->host_bytes &&
                    out->disk_bytes <= hw->disk_bytes;
        return TOD_OK;
    });
}

int estimate_gemm(int64_t rows, int out, int in, int int4, const tod_hw *hw, double *seconds)
{
    return guard("estimate_gemm", [&]() -> int {
        if (!hw || !seconds)
            return fail(TOD_EINVAL, "null argument");
        if (rows <= 0 || rows > (1 << 24) || out <= 0 || in <= 0 || in % 64 || (int4 && out % 32))
            return fail(TOD_EINVAL, "bad GEMM shape %lld x %d x %d", (long long)rows, out, in);
        if (!(hw->mem_gbs > 0.0 && hw->int4_tflops > 0.0 && hw->fp16_tflops > 0.0 && hw->launch_us >= 0.0 &&
              hw->gemm_wg_us >= 0.0 && hw->staged_tflops > 0.0 && hw->staged_gbs > 0.0 && hw->staged_us >= 0.0))
            return fail(TOD_EINVAL, "hardware rates must be positive and fixed costs non-negative");
        *seconds = gemm_time((int)rows, out, in, int4 != 0, hw);
        return TOD_OK;
    });
}

int plan_decode(const tod_model_config *cfg, int prompt_len, int gen_len, int max_rows, const tod_hw *hw,
                tod_run_config *best, tod_estimate *est)
{
    return guard("plan_decode", [&]() -> int {
        if (!cfg || !hw || !best || !est || prompt_len <= 0 || gen_len <= 0 || max_rows <= 0)
            return fail(TOD_EINVAL, "bad plan_decode arguments");
        bool found = false;
        tod_estimate cur{};
        const int64_t row_cap = 1 << 24; // init_model's limit on block rows and on prefill rows
        if (max_rows > row_cap)
            max_rows = (int)row_cap;
        int b_top = 1;
        while (b_top * 2 <= max_rows)
            b_top *= 2;
        for (int tier = TOD_W_HBM_INT4; tier <= TOD_W_HOST_INT4_STREAM; tier++)
            for (int disk = 0; disk <= (tier == TOD_W_HBM_INT4 ? 0 : 1); disk++)
            for (int b = b_top; b >= 1; b /= 2)
                for (int K = 1; b * K <= max_rows && (int64_t)b * prompt_len <= row_cap; K *= 2) {
                    const int r_max = tier == TOD_W_HBM_INT4 ? 0 : cfg->n_layers;
                    for (int R = 0; R <= r_max; R++) {
                        tod_run_config r{};
                        r.gpu_batch = b;
                        r.batches_per_block = K;
                        r.prompt_len = prompt_len;
                        r.gen_len = gen_len;
                        r.group = 64;
                        r.weight_tier = tier;
                        r.n_blocks = 1;
                        r.host_layers = 0;
                        r.hbm_layers = R;
                        r.kv_host_layers = 0;
                        r.weights_on_disk = disk;
                        int rc = estimate_decode(cfg, &r, hw, &cur);
                        if (rc)
                            return rc;
                        if (cur.hbm_bytes > hw->hbm_bytes) {
                            // the fewest host-KV layers that bring the device footprint within the
                            // capacity: each moves one layer's cache out, the first also adds two
                            // slots. Counted without the split-K workspace, then raised while the
                            // workspace still keeps it from fitting.
                            const double kv_layer = kv_layer_bytes(cfg, &r);
                            const double need = std::ceil((cur.hbm_bytes - cur.workspace_bytes + 2.0 * kv_layer -
                                                           hw->hbm_bytes) / kv_layer);
                            if (need > cfg->n_layers)
                                continue;
                            r.kv_host_layers = need < 1.0 ? 1 : (int)need;
                            if ((rc = estimate_decode(cfg, &r, hw, &cur)))
                                return rc;
                            while (cur.hbm_bytes > hw->hbm_bytes && r.kv_host_layers < cfg->n_layers) {
                                r.kv_host_layers++;
                                if ((rc = estimate_decode(cfg, &r, hw, &cur)))
                                    return rc;
                            }
                        }
                        // strictly better only: ties keep the earlier (lower tier, pinned before disk,
                        // larger b, then smaller K, R)
                        if (cur.fits && (!found || cur.tokens_per_s > est->tokens_per_s)) {
                            *best = r;
                            *est = cur;
                            found = true;
                        }
                    }
                }
        return found ? TOD_OK : fail(TOD_ENOMEM, "no configuration fits the capacities");
    });
}
