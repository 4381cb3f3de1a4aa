/*
 * tod.h -- C ABI of the MI355X (gfx950) block-scheduled int4 decode library.
 *
 * The library runs the throughput-oriented generation loop of FlexGen on one
 * GPU: greedy decode of an OPT-shaped decoder stack for a block of K GPU
 * batches, with
 *   - the zig-zag block schedule: each layer's weights are read once per
 *     decode step and used for every batch of the block
 *       (FlexGen guide, "2. The Zig-Zag Block Schedule");
 *   - group-wise 4-bit weights and a group-wise 4-bit KV cache, dequantized
 *     on the fly for fp16 compute
 *       (FlexGen guide, "3. Group-Wise 4-Bit Quantization for Weights and KV Cache");
 *   - optionally, weights (fp16 or the int4 image) held in pinned host memory
 *     or in a file on disk and streamed into HBM layer by layer, overlapped
 *     with compute, with a chosen number of leading layers kept resident, and
 *     the KV caches of trailing layers in pinned host memory
 *       (FlexGen guide, "1. Three-Tier Storage Hierarchy"; TightLLM abstract,
 *        on overlapping transfer with computation);
 *   - a cost model of the decode step and a search over these placements.
 *
 * Conventions for every entry point:
 *   - Return 0 on success, a negative TOD_E* code on error; never abort and
 *     never throw: a host allocation that fails inside the library (a C++
 *     exception) is caught at the entry point and returned as TOD_ENOMEM.
 *     last_error() returns a message for the calling thread's last failing
 *     call.
 *   - Pointers named d_* are caller-owned device (HBM) memory; h_* are
 *     caller-owned host memory. Sizes are element counts unless stated.
 *   - fp16 tensors are passed as uint16_t bit patterns (IEEE binary16).
 *   - stream is a hipStream_t passed as void*; NULL is the null stream.
 *     Calls that take a stream are asynchronous on it; init_model,
 *     set_global_weights, set_layer_weights and free_model synchronize.
 *   - A kernel fault surfaces as TOD_EHIP at the next synchronizing call.
 *   - One model (or attention cache) handle is used by one thread at a time;
 *     distinct handles are independent. Besides the per-thread error message
 *     the library keeps no global state (tuning variables are read once).
 *
 * Group-wise int4 format (canonical, as exchanged through this ABI): a tensor
 * of n elements is cut into n/64 contiguous groups. Per group: zero = group
 * minimum (fp16), scale = fp16(fp32(max - min) / 15), code c in [0, 15] =
 * nearest grid point zero + c*scale with ties to the larger code; element
 * value zero + c*scale rounded once to fp16. Codes are packed two per byte,
 * element 2t in the low nibble of byte t. Weight matrices W[out][in] are
 * grouped along `in`; K and V vectors along the head dimension.
 */
#ifndef TOD_H
#define TOD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif
/* the library is built with hidden visibility: these declarations are its only exports */
#pragma GCC visibility push(default)

#define TOD_OK 0
#define TOD_EINVAL (-1) /* bad argument: null pointer, shape or size mismatch, group != 64 */
#define TOD_ENOMEM (-2) /* device or pinned host allocation failed */
#define TOD_EHIP (-3)   /* HIP runtime error; the message carries hipGetErrorString */
#define TOD_ESTATE (-4) /* call out of order: decode before prefill, context full, block out of range */

#define TOD_GROUP 64
#define TOD_MAX_BLOCKS 4096 /* most blocks (each with its own KV cache) one model holds */

/* Where a model's six decoder matrices per layer live. */
#define TOD_W_HBM_INT4 0         /* int4 group-64 in HBM, quantized at load */
#define TOD_W_HOST_FP16_STREAM 1 /* fp16 in pinned host memory, streamed per layer into a 2-slot HBM buffer */
#define TOD_W_HOST_INT4_STREAM 2 /* int4 group-64 (tiled codes + params) in pinned host memory, streamed per layer */

/* Order of the 16 per-layer tensors passed to set_layer_weights. */
enum {
    TOD_LN1_G = 0, TOD_LN1_B, TOD_Q_W, TOD_Q_B, TOD_K_W, TOD_K_B, TOD_V_W, TOD_V_B,
    TOD_O_W, TOD_O_B, TOD_LN2_G, TOD_LN2_B, TOD_FC1_W, TOD_FC1_B, TOD_FC2_W, TOD_FC2_B,
    TOD_LAYER_TENSORS
};

/* Matrix ids for export_weight. */
enum { TOD_MAT_Q = 0, TOD_MAT_K, TOD_MAT_V, TOD_MAT_O, TOD_MAT_FC1, TOD_MAT_FC2 };

typedef struct tod_model tod_model;

/* OPT decoder stack shape. hidden = n_heads * head_dim; head_dim is 64 or
 * 128; hidden % 64 == 0 and hidden <= 16384; ffn % 64 == 0; max_pos = rows of
 * the position table minus the two offset rows. */
typedef struct {
    int32_t n_layers, hidden, n_heads, head_dim, ffn, vocab, max_pos;
} tod_model_config;

/* One block = batches_per_block (K) GPU batches of gpu_batch sequences each;
 * its K*gpu_batch rows are row k*gpu_batch + i for batch k. Every sequence
 * has prompt_len prompt tokens and at most gen_len generated tokens, so the
 * KV cache holds prompt_len + gen_len - 1 positions. n_blocks blocks (1 ..
 * TOD_MAX_BLOCKS) are resident at once (each has its own KV cache). group
 * must be 64.
 * hbm_layers (host tiers only; 0..n_layers, default 0): layers 0..hbm_layers-1
 * keep their weight image (the bytes a streamed layer would copy) resident in
 * HBM and never cross the host link; the remaining layers stream. This is the
 * placement choice the FlexLLMGen overview ("A 175B-parameter model on one
 * GPU, if you can wait": what it does; caveats, the manual placement flags)
 * leaves to the user: what share of the weights sits on the GPU versus host
 * memory. Results are identical for every hbm_layers.
 * host_layers (host tiers only; 0 = every streamed layer): pinned host memory
 * is kept for the six matrices of the first host_layers streamed layers only,
 * and a later streamed layer l streams those of layer
 * hbm_layers + (l - hbm_layers) % host_layers (its vectors stay its own). This
 * exists to measure stacks whose weights exceed the host's memory: copy sizes,
 * streams and overlap are those of distinct layers.
 * kv_host_layers (0..n_layers, default 0; any weight tier): the KV caches of
 * the last kv_host_layers layers live in pinned host memory (FlexGen guide,
 * "1. Three-Tier Storage Hierarchy": the cache spills to CPU memory). Each
 * pass copies such a layer's cached positions into one of two HBM slots on a
 * copy stream while the previous layers compute; the append writes each new
 * position into the slot and through to the host cache, and attention reads
 * the slot. Results are identical for every kv_host_layers; decode steps are
 * then launched one by one (no decode graph).
 * weights_on_disk (host tiers only; 0 or 1): the streamed layers' images live
 * in a file named by set_weight_file instead of pinned memory (FlexGen guide,
 * "1. Three-Tier Storage Hierarchy": the disk tier below CPU memory). */
typedef struct {
    int32_t gpu_batch, batches_per_block, prompt_len, gen_len, group, weight_tier, n_blocks;
    int32_t host_layers;
    int32_t hbm_layers;
    int32_t kv_host_layers;
    int32_t weights_on_disk;
} tod_run_config;

/*
 * set_weight_file: for a model created with run.weights_on_disk, create (or
 * truncate) the file at `path` that holds the streamed layers' images; call it
 * once, before set_layer_weights. set_layer_weights then writes each image
 * that a streamed layer owns (see host_layers) to the file, 4 KiB-aligned, and
 * every pass reads it back into one of two pinned staging buffers on an I/O
 * stream, from which the copy stream moves it into the HBM slot; reads of one
 * layer overlap the copy of the previous one. Direct I/O cannot target pinned
 * memory, so the reads are buffered, and each image is dropped from the page
 * cache after it is written and after every read: each pass reads the disk.
 * Results are identical to the pinned tiers. A failed read makes the next prefill / decode_block return TOD_EHIP
 * (the outputs of the pass it happened in are undefined). The library keeps
 * the file open until free_model and never deletes it.
 * Errors: TOD_EINVAL (null argument, cannot open), TOD_ESTATE (not a disk-tier
 * model, file already set, or weights already set).
 */
int set_weight_file(tod_model *m, const char *path);

/*
 * init_model: allocate a model (weights store, KV caches, activation buffers).
 * Weights are supplied afterwards with set_global_weights / set_layer_weights.
 * FlexGen guide, "2. The Zig-Zag Block Schedule" (a block of K micro-batches
 * shares each weight load) and "1. Three-Tier Storage Hierarchy" (weight tier).
 * Errors: TOD_EINVAL on an invalid shape (also when gpu_batch *
 * batches_per_block or gpu_batch * prompt_len exceeds 2^24 rows), found before
 * any allocation or device call; TOD_ENOMEM if HBM or pinned host memory runs
 * out, TOD_EHIP otherwise. *out is NULL on error.
 */
int init_model(const tod_model_config *cfg, const tod_run_config *run, void *stream, tod_model **out);

/*
 * set_global_weights: copy the fp16 token embedding h_tok_emb [vocab][hidden]
 * (also the tied LM head), the position table h_pos_emb [max_pos + 2][hidden]
 * (OPT's two offset rows first) and the final LayerNorm gain/shift [hidden]
 * into HBM. Host buffers may be freed on return.
 */
int set_global_weights(tod_model *m, const uint16_t *h_tok_emb, const uint16_t *h_pos_emb,
                       const uint16_t *h_lnf_g, const uint16_t *h_lnf_b);

/*
 * set_layer_weights: supply layer `layer`'s 16 fp16 host tensors in TOD_*
 * order (matrices row-major [out][in]: q, k, v, o [hidden][hidden], fc1
 * [ffn][hidden], fc2 [hidden][ffn]; vectors [out] or [hidden]).
 * TOD_W_HBM_INT4: the six matrices are copied to HBM and quantized there to
 * int4 group-64 (FlexGen guide, "3. Group-Wise 4-Bit Quantization"); host
 * buffers may be freed on return.
 * TOD_W_HOST_FP16_STREAM: the matrices are copied into the library's pinned
 * host tier and streamed to HBM on every pass over the layer.
 * TOD_W_HOST_INT4_STREAM: the matrices are quantized in HBM as for
 * TOD_W_HBM_INT4 and their tiled int4 image (0.5625 byte per weight) is kept
 * in pinned host memory and streamed on every pass: the packed 4-bit weights
 * cross the host link instead of fp16 (FlexGen guide, "3. Group-Wise 4-Bit
 * Quantization", transfer of packed 4-bit data over PCIe); results are
 * identical to TOD_W_HBM_INT4.
 * On both host tiers, streamed layers that reuse an earlier layer's pinned
 * image (run.host_layers) do not read their matrices, only their vectors.
 */
int set_layer_weights(tod_model *m, int layer, const uint16_t *const *h_tensors);

/*
 * prefill: run the prompts of block `block` (d_ids int32 [K*b][prompt_len])
 * through the stack in the zig-zag order (per layer, batch by batch), storing
 * every prompt position's K/V into the int4 cache, and write each row's first
 * generated token to d_next int32 [K*b]. d_logits (nullable) receives the fp16
 * logits of the last prompt position, [K*b][vocab].
 * Resets the block's decode position. FlexGen guide, "2. The Zig-Zag Block
 * Schedule"; FlexLLMGen page, "Key highlights" (generate API).
 * Errors: TOD_EINVAL, TOD_ESTATE (weights missing, block out of range).
 */
int prefill(tod_model *m, int block, const int32_t *d_ids, int32_t *d_next, uint16_t *d_logits, void *stream);

/*
 * decode_block: run n_steps greedy decode steps for all K*b rows of block
 * `block`. Step t feeds d_ids_in [K*b] (t = 0) or the previous step's picks,
 * at position prompt_len + (decode steps already run since prefill), appends that
 * position's quantized K/V, and writes the picks to d_ids_out int32
 * [n_steps][K*b]; d_logits (nullable) receives fp16 [n_steps][K*b][vocab].
 * Within a step every layer's weights are read from HBM (or streamed from a
 * host tier) once for the whole block: the block's rows form the M dimension
 * of each fused int4 GEMM (FlexGen guide, "2. The Zig-Zag Block Schedule";
 * comparison table, "Weight Reuse per Load").
 * Errors: TOD_ESTATE before prefill or when the KV cache would overflow.
 */
int decode_block(tod_model *m, int block, int n_steps, const int32_t *d_ids_in, int32_t *d_ids_out,
                 uint16_t *d_logits, void *stream);

/*
 * set_decode_position: set how many decode steps block `block` has completed
 * since its prefill (0 <= steps <= gen_len - 1); later decode steps overwrite
 * the cache from that position on. Lets a caller replay decode steps.
 */
int set_decode_position(tod_model *m, int block, int steps);

/*
 * set_decode_graph: with enable != 0 (the default) decode_block on the HBM
 * tier captures one decode step of each block into a HIP graph at its first
 * use and replays it per step on a stream of the model's own, ordered after
 * the caller's stream and before its later work; the step reads its position
 * and token ids from device memory, so one graph serves every step. Outputs
 * are identical to the step-by-step launches, which run instead when enable is
 * 0, on the host tiers, while profile_kernels is active, or if capture fails.
 */
int set_decode_graph(tod_model *m, int enable);

/*
 * quantize_groupwise: group-wise int4 quantization of d_x fp16 [n] into the
 * canonical format above: d_codes uint8 [n/2], d_scale fp16 [n/group],
 * d_zero fp16 [n/group]. n % group == 0, group == 64. Non-finite inputs are
 * outside the contract (codes undefined, no error).
 * FlexGen guide, "3. Group-Wise 4-Bit Quantization for Weights and KV Cache".
 */
int quantize_groupwise(const uint16_t *d_x, int64_t n, int group, uint8_t *d_codes, uint16_t *d_scale,
                       uint16_t *d_zero, void *stream);

/* dequantize_groupwise: d_out fp16 [n] = fp16(zero + code * scale) from the canonical format. */
int dequantize_groupwise(const uint8_t *d_codes, const uint16_t *d_scale, const uint16_t *d_zero, int64_t n,
                         int group, uint16_t *d_out, void *stream);

/* free_model: synchronize, release every allocation of m. NULL is accepted. */
int free_model(tod_model *m);

/* last_error: message of the calling thread's last failing call ("" if none). */
const char *last_error(void);

/* ------------------------------------------------------------------------ */
/* Inspection and unit entry points (used by tests and the benchmark).      */
/* ------------------------------------------------------------------------ */

/* Kernel classes timed by profile_kernels / profile_read. */
enum {
    TOD_K_GEMM_QKV = 0, TOD_K_GEMM_O, TOD_K_GEMM_FC1, TOD_K_GEMM_FC2, TOD_K_ATTN, TOD_K_KV_APPEND,
    TOD_K_LAYERNORM, TOD_K_LM_HEAD, TOD_K_ARGMAX, TOD_K_EMBED, TOD_K_COUNT
};

/*
 * profile_kernels: from now on, bracket every launch of the kernel classes
 * whose bit (1 << TOD_K_*) is set in `mask` with HIP events on the stream it
 * is launched on (prefill and decode_block); mask 0 stops. Resets the totals.
 * profile_read: wait for the recorded events and return the summed duration
 * (ms) and the number of launches of class `kind` since profile_kernels.
 */
int profile_kernels(tod_model *m, unsigned mask);
int profile_read(tod_model *m, int kind, double *total_ms, int64_t *launches);

/*
 * export_weight: copy layer `layer`'s matrix `which` (TOD_MAT_*) back out of
 * the int4 store in the canonical format (device buffers: codes [out*in/2],
 * scale and zero [out*in/64]). On the int4 host tier a streamed layer's
 * pinned image (see run.host_layers) is read back through an idle streaming
 * slot, after a device synchronize. TOD_ESTATE for the fp16 host tier.
 */
int export_weight(tod_model *m, int layer, int which, uint8_t *d_codes, uint16_t *d_scale, uint16_t *d_zero,
                  void *stream);

/*
 * set_layer_tap: test hook that exposes one layer's input and output. From the
 * next prefill (phase 0) or decode_block (phase 1) on, every pass of that phase
 * over layer `layer` copies hidden rows [row0, row0 + n_rows) of the pass into
 * d_in (before the layer) and d_out (after it), each fp16 [n_rows][hidden]
 * device memory owned by the caller and kept alive while the tap is set (either
 * may be NULL). The hidden rows are the residual stream between layers (before
 * the layer's own LayerNorm): in decode row r is row r of the block; in
 * prefill row r is position r % prompt_len of block row r / prompt_len. The
 * copies run on the pass's stream. n_rows == 0 removes the tap. While any
 * decode tap is set decode steps are launched one by one (no decode graph).
 * Used to check a layer against a reference given exactly the inputs it saw
 * (FlexGen guide, "3. Group-Wise 4-Bit Quantization": the layer computes in
 * fp16 on dequantized weights and cache). Errors: TOD_EINVAL (phase not 0/1,
 * layer out of range, rows outside the pass, n_rows > 0 with both buffers NULL).
 */
int set_layer_tap(tod_model *m, int phase, int layer, int64_t row0, int64_t n_rows, uint16_t *d_in,
                  uint16_t *d_out);

/*
 * export_kv: copy positions [t0, t1) of (layer, block, row, head) out of the
 * KV cache in the canonical per-position format (device buffers): K codes
 * [t1-t0][head_dim/2], K scale/zero [t1-t0][head_dim/64], same for V.
 */
int export_kv(tod_model *m, int layer, int block, int row, int head, int t0, int t1, uint8_t *d_kc,
              uint16_t *d_ks, uint16_t *d_kz, uint8_t *d_vc, uint16_t *d_vs, uint16_t *d_vz, void *stream);

/*
 * linear_w4: y [rows][out] = fp16(a [rows][in] . What^T + bias [+ residual]
 * [, ReLU]) with W given in the canonical int4 format (device). The library
 * repacks W into its GEMM layout in scratch memory it owns, then runs the same
 * fused dequant+MFMA GEMM as the decode path. relu: 0/1. bias and residual
 * are nullable. Used to test the GEMM at full shapes. Synchronizes stream
 * before returning (the scratch memory is freed). Errors, all before any
 * device work: TOD_EINVAL for a null a, y, codes (scale, zero) or d_w, rows
 * outside [0, 2^31), in not a positive multiple of 64, out <= 0, an int4 out
 * not a multiple of 32, or relu with a residual; TOD_ENOMEM when the scratch
 * memory cannot be allocated.
 */
int linear_w4(const uint16_t *d_a, int64_t rows, int in, int out, const uint8_t *d_codes, const uint16_t *d_scale,
              const uint16_t *d_zero, const uint16_t *d_bias, const uint16_t *d_residual, int relu, uint16_t *d_y,
              void *stream);

/*
 * linear_w4_noalloc: linear_w4 for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments, kernels and results as linear_w4, but the
 * repacked weights and the split-K partials live in a fixed scratch array of
 * TOD_LINEAR_NOALLOC_BYTES that each device holds from its first call until
 * the process ends; the call allocates and frees nothing and does not
 * synchronize (it is asynchronous on stream). A call needs out*in/2 and
 * out*in/16 bytes (each rounded up to 256) plus the GEMM's split-K partials
 * (0, or splits * rows * out * 4 bytes); a call that needs more fails with
 * TOD_EINVAL before any device work. Every call on a device shares that
 * device's scratch: calls on one stream are ordered, but calls that overlap on
 * one device (other streams or threads) race and their outputs are undefined.
 * The scratch keeps the last call's contents; no call reads what it did not
 * write first, so nothing needs clearing. Errors: as linear_w4, plus the
 * scratch limit above.
 */
#define TOD_LINEAR_NOALLOC_BYTES ((size_t)192 << 20)
int linear_w4_noalloc(const uint16_t *d_a, int64_t rows, int in, int out, const uint8_t *d_codes,
                      const uint16_t *d_scale, const uint16_t *d_zero, const uint16_t *d_bias,
                      const uint16_t *d_residual, int relu, uint16_t *d_y, void *stream);

/* linear_f16: as linear_w4 with fp16 weights d_w [out][in] (the LM head's and the fp16 host tier's GEMM). */
int linear_f16(const uint16_t *d_a, int64_t rows, int in, int out, const uint16_t *d_w, const uint16_t *d_bias,
               const uint16_t *d_residual, int relu, uint16_t *d_y, void *stream);

/*
 * Isolated decode attention over an int4 KV cache (one query per sequence).
 * attn_cache_create allocates a cache for batch x heads sequences of up to
 * cap positions with head_dim 64 or 128 and returns a handle (TOD_EINVAL for
 * other shapes). Every fp16 buffer passed to fill/step must be 16-byte aligned
 * (TOD_EINVAL otherwise).
 * attn_cache_fill quantizes and stores fp16 d_k, d_v [n][batch][heads][head_dim]
 * (position-major) at positions [t0, t0+n). attn_decode_step quantizes and appends the new
 * d_k_new, d_v_new [batch][heads][head_dim] at position pos, then writes
 * d_out [batch][heads][head_dim] = attention of d_q [batch][heads][head_dim]
 * over positions 0..pos (FlexGen guide, "3. Group-Wise 4-Bit Quantization"
 * for the dynamic KV cache). attn_cache_export reads a position range of one
 * (sequence, head) back in the canonical format, as export_kv.
 */
typedef struct tod_attn_cache tod_attn_cache;
int attn_cache_create(int batch, int heads, int head_dim, int cap, tod_attn_cache **out);
int attn_cache_fill(tod_attn_cache *c, const uint16_t *d_k, const uint16_t *d_v, int t0, int n, void *stream);
int attn_decode_step(tod_attn_cache *c, int pos, const uint16_t *d_q, const uint16_t *d_k_new,
                     const uint16_t *d_v_new, uint16_t *d_out, void *stream);
int attn_cache_export(tod_attn_cache *c, int seq, int head, int t0, int t1, uint8_t *d_kc, uint16_t *d_ks,
                      uint16_t *d_kz, uint8_t *d_vc, uint16_t *d_vs, uint16_t *d_vz, void *stream);
int attn_cache_free(tod_attn_cache *c);

/*
 * Cost model and placement search (host computation only; no device calls).
 * The FlexGen guide's simulator ("Implementation: Simulating FlexGen's Zig-Zag
 * Block Scheduling in Python") prices a step by the weight bytes moved over
 * PCIe; the FlexLLMGen overview ("A 175B-parameter model on one GPU, if you
 * can wait": caveats) tunes placement by hand, an automatic policy optimiser
 * being future work. Here a decode step is priced from measured rates:
 *
 * tod_hw: attn_gbs = decode-attention read rate, mem_gbs = streaming rate of
 * the other row-wise kernels and weight reads, link_gbs = pinned -> HBM copy
 * rate (GB/s); int4_tflops / fp16_tflops = steady rates of the pipelined GEMM
 * on int4 / fp16 weights while every CU holds one of its
 * workgroups, and gemm_wg_us = the fixed time each wave of its workgroups adds
 * (pipeline fill, epilogue); staged_us / staged_gbs / staged_tflops = the
 * register-staged GEMM's fixed time, effective weight-read rate and flop rate
 * (small GEMMs of 128 rows or fewer, fp16 weights whose N is not a multiple
 * of 32); launch_us = floor per kernel;
 * hbm_bytes / host_bytes =
 * capacities the model may use; disk_gbs / disk_bytes = read rate and free
 * space of the weight file's disk. default_hw fills the figures measured on
 * MI355X for this library.
 *
 * estimate_decode prices one decode step of the block `run` describes at the
 * average decode context (prompt_len + gen_len / 2): per layer, each GEMM runs
 * the library's own tile plan: a pipelined GEMM takes ceil(workgroups / 256)
 * waves of (K-groups per workgroup * tile rows / 256 * t_g + gemm_wg_us),
 * where t_g = 256 * 2 * 256 * 256 * 64 / (int4_tflops or fp16_tflops) is one
 * K-group of a full 256 x 256 tile on every CU, at least weight bytes /
 * mem_gbs + gemm_wg_us, plus, when its K loop is split, its fp32 partials
 * written and read back at mem_gbs; a
 * register-staged GEMM takes staged_us + weight bytes / staged_gbs + flops /
 * staged_tflops (each GEMM at least launch_us),
 * attention M * heads * (ctx * (d + d/8) + 4d) bytes / attn_gbs, the KV append
 * M * heads * (4d + d + d/8) bytes / mem_gbs; plus embedding, one LayerNorm, the
 * fp16 LM head and the argmax. On the host tiers the L - hbm_layers streamed
 * layers each copy one layer image (weights x 2 B fp16, or x 0.5625 B int4) at
 * link_gbs while the GPU computes; the resident layers run while at most two
 * copies (one per slot) are in flight, so step = max(compute, link + idle),
 * idle = max(0, hbm_layers * t_layer - min(2, streamed) * t_copy). Each
 * host-KV layer (run.kv_host_layers) adds M * heads * ctx * (d + d/8) bytes of
 * copies to the link (its cached positions in, the new one written through);
 * with no streamed weights the idle term is max(0, (L - kv_host) * t_layer -
 * min(2, kv_host) * t_kv). With run.weights_on_disk a streamed layer's copy
 * takes max(image / link_gbs, image / disk_gbs) (disk reads and link copies of
 * consecutive layers overlap), the pinned memory is two staging images and
 * disk_bytes the file. out also
 * gets the device and pinned-host bytes init_model would allocate (the device
 * figure includes workspace_bytes, the GEMMs' split-K partials), and fits =
 * both within the capacities. Errors: TOD_EINVAL on a null pointer, a run
 * configuration init_model would reject, a non-positive rate or a negative
 * gemm_wg_us.
 *
 * plan_decode searches weight tier (0, 1, 2), GPU batch b and batches per
 * block K (powers of two, b * K <= max_rows, b * K and b * prompt_len at
 * most 2^24 as init_model requires) and, on the host tiers,
 * hbm_layers (0..n_layers), for the most decode tokens per second among the
 * configurations that fit; ties keep the earliest in the order lower tier,
 * larger b, smaller K, smaller hbm_layers (decode cost depends on b * K only;
 * b sets prefill's batch of b * prompt_len rows, so the largest b that fits
 * is kept). A candidate whose device footprint exceeds the capacity gets the
 * fewest host-KV layers (run.kv_host_layers) that make it fit, if any. Host
 * tiers are tried with pinned images first and then with images on disk
 * (run.weights_on_disk), within disk_bytes. *best is a complete run
 * configuration (group 64, one block, host_layers 0) and *est its estimate.
 * TOD_EINVAL for null pointers, non-positive lengths or max_rows, or a model
 * configuration or prompt_len + gen_len that init_model would reject;
 * TOD_ENOMEM if nothing fits.
 */
typedef struct {
    double attn_gbs, mem_gbs, link_gbs, int4_tflops, fp16_tflops, launch_us, hbm_bytes, host_bytes, disk_gbs,
        disk_bytes, gemm_wg_us, staged_tflops, staged_gbs, staged_us;
} tod_hw;
typedef struct {
    double step_s, tokens_per_s, compute_s, link_s, hbm_bytes, host_bytes, workspace_bytes, disk_bytes;
    int32_t fits;
} tod_estimate;
void default_hw(tod_hw *hw);
int estimate_decode(const tod_model_config *cfg, const tod_run_config *run, const tod_hw *hw, tod_estimate *out);
/* estimate_gemm: the seconds estimate_decode charges one GEMM of rows x out x in (int4 != 0: int4
 * weights, else fp16), on the tile plan the library launches for that shape. TOD_EINVAL for a shape
 * the GEMM does not take (in % 64, int4 out % 32, rows outside [1, 2^24]) or invalid rates. */
int estimate_gemm(int64_t rows, int out, int in, int int4, const tod_hw *hw, double *seconds);
int plan_decode(const tod_model_config *cfg, int prompt_len, int gen_len, int max_rows, const tod_hw *hw,
                tod_run_config *best, tod_estimate *est);

#pragma GCC visibility pop
#ifdef __cplusplus
}
#endif

#endif /* TOD_H */
