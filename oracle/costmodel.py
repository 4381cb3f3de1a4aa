"""Closed-form I/O cost model of offloaded generation (plain Python).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``.

Two models are given:

* ``p1_naive`` / ``p1_zigzag`` restate the toy simulator of the FlexGen guide
  ("Implementation: Simulating FlexGen's Zig-Zag Block Scheduling in Python",
  Steps 1-3): transfer time = output tokens x model GB / PCIe GB/s and
  throughput = batch x tokens / transfer time. As printed, both schedules use
  that same formula and differ only in the batch they are given (4 against
  128), and the micro-batch count is not used; the printed result is
  1.83 against 58.51 tokens/s, a ratio of 32.0.
* ``weight_bytes`` counts layer loads the way the zig-zag block schedule
  defines them (FlexGen guide, "2. The Zig-Zag Block Schedule", and the
  comparison table's "Weight Reuse per Load" row): with K micro-batches per
  block, row-by-row execution streams the model once per micro-batch per
  token, the zig-zag schedule once per token for the whole block, so
  row-by-row moves K times the bytes.

A third part, ``decode_step`` / ``footprint`` / ``plan``, prices one decode
step of the block schedule from measured rates, and searches the run
configurations for the most tokens per second under memory capacities. It
extends the simulator's "time = bytes moved / link rate" with the roofline
terms of the step (GEMM flops, KV-cache reads) and with the placement choices
that the FlexLLMGen overview ("A 175B-parameter model on one GPU, if you can
wait": caveats) leaves to manual flags. It is written from those terms alone
and knows nothing of how any implementation tiles its GEMMs: a GEMM costs the
larger of its flops at the GEMM rate and its weight bytes at the streaming
rate, plus one fixed cost. With free compute and an all-streamed fp16 model it
reduces to the simulator's formula (pinned against the printed figures). The
device footprint here leaves out an implementation's GEMM workspace.
"""
from __future__ import annotations

import math

PCIE_GB_S = 16.0  # simulator's PCIe constant (guide, Step 1)


def p1_naive(batch: int, output_tokens: int, model_gb: float = 35.0, pcie_gb_s: float = PCIE_GB_S) -> float:
    io_s = output_tokens * model_gb / pcie_gb_s
    return batch * output_tokens / io_s


def p1_zigzag(batch: int, output_tokens: int, micro_batches: int = 4, model_gb: float = 35.0,
              pcie_gb_s: float = PCIE_GB_S) -> float:
    del micro_batches  # unused by the printed simulator
    io_s = output_tokens * model_gb / pcie_gb_s
    return batch * output_tokens / io_s


def weight_bytes(model_bytes: float, tokens: int, micro_batches: int, schedule: str) -> float:
    """Weight bytes moved to generate ``tokens`` tokens for a block of ``micro_batches`` batches."""
    if schedule == "row_by_row":
        return model_bytes * tokens * micro_batches
    if schedule == "zigzag":
        return model_bytes * tokens
    raise ValueError(schedule)


def throughput(model_bytes: float, link_bytes_s: float, tokens: int, batch: int, micro_batches: int,
               schedule: str) -> float:
    """Tokens/s when the link is the only cost: block of ``micro_batches`` batches of ``batch`` rows."""
    t = weight_bytes(model_bytes, tokens, micro_batches, schedule) / link_bytes_s
    return batch * micro_batches * tokens / t


# ---------------------------------------------------------------------------
# decode step model, footprint and configuration search
# ---------------------------------------------------------------------------

TIER_HBM_INT4, TIER_HOST_FP16, TIER_HOST_INT4 = 0, 1, 2


def _layer_weights(shape) -> float:
    """Elements of the four GEMM matrices of a layer: qkv 3h x h, out h x h, fc1 f x h, fc2 h x f."""
    h, f = float(shape.hidden), float(shape.ffn)
    return 3 * h * h + h * h + f * h + h * f


def _bytes_per_weight(tier: int) -> float:
    # fp16 on the fp16 host tier; otherwise a 4-bit code plus a (scale, zero) fp16 pair per 64 weights
    return 2.0 if tier == TIER_HOST_FP16 else 0.5 + 4.0 / 64


def _kernel(seconds: float, hw: dict) -> float:
    return max(seconds, hw["launch_us"] * 1e-6)


ROW_CAP = 1 << 24  # most rows of a block and of one prefill batch


def gemm_time(rows: int, n_out: int, n_in: int, int4: bool, hw: dict) -> float:
    """Seconds for one GEMM of rows x n_out x n_in: the larger of its flops 2 * rows * n_out * n_in
    at the GEMM rate (int4 or fp16 weights) and its weight bytes (0.5625 or 2 per weight) at the
    streaming rate, plus the fixed cost of one GEMM (gemm_wg_us), and at least one launch."""
    rate = (hw["int4_tflops"] if int4 else hw["fp16_tflops"]) * 1e12
    weight_bytes_ = n_out * n_in * (0.5 + 4.0 / 64 if int4 else 2.0)
    seconds = max(2.0 * rows * n_out * n_in / rate, weight_bytes_ / (hw["mem_gbs"] * 1e9))
    return _kernel(seconds + hw["gemm_wg_us"] * 1e-6, hw)


def decode_step(shape, run: dict, hw: dict) -> dict:
    """Seconds per decode step at the average decode context, and tokens/s."""
    tier = run.get("weight_tier", TIER_HBM_INT4)
    rows = run["gpu_batch"] * run["batches_per_block"]
    h, f, d, heads, vocab = shape.hidden, shape.ffn, shape.head_dim, shape.n_heads, shape.vocab
    mem = hw["mem_gbs"] * 1e9
    context = run["prompt_len"] + run["gen_len"] / 2.0

    layer = 0.0
    for n_out, n_in in ((3 * h, h), (h, h), (f, h), (h, f)):
        layer += gemm_time(rows, n_out, n_in, tier != TIER_HOST_FP16, hw)
    per_position = 2 * (d / 2 + 4 * (d / 64))          # K and V: codes + (scale, zero) per group
    attention_bytes = rows * heads * (context * per_position + 4 * d)   # cache, plus q and out in fp16
    layer += _kernel(attention_bytes / (hw["attn_gbs"] * 1e9), hw)
    layer += _kernel(rows * heads * (2 * 2 * d + per_position) / mem, hw)  # append: read k, v; write codes

    head = _kernel(rows * h * 4.0 / mem, hw)            # embedding: two table rows in, one row out
    head += _kernel(rows * h * 4.0 / mem, hw)           # the first layer's LayerNorm
    head += gemm_time(rows, vocab, h, False, hw)            # LM head: fp16 tied embedding
    head += _kernel(rows * vocab * 2.0 / mem, hw)       # argmax over the fp16 logits
    compute = shape.n_layers * layer + head

    link = 0.0
    idle = 0.0
    streamed = 0
    if tier != TIER_HBM_INT4:
        resident = run.get("hbm_layers", 0)
        streamed = shape.n_layers - resident
        image = _layer_weights(shape) * _bytes_per_weight(tier)
        copy = image / (hw["link_gbs"] * 1e9)
        if run.get("weights_on_disk", 0):
            # reads from the file and copies over the link overlap across layers
            copy = max(copy, image / (hw["disk_gbs"] * 1e9))
        link = streamed * copy
        if streamed > 0:
            # the resident layers run while at most two copies (one per slot) are in flight
            idle = max(0.0, resident * layer - min(2, streamed) * copy)
    kv_host = run.get("kv_host_layers", 0)
    if kv_host > 0:
        # per host-KV layer: context - 1 cached positions in, the appended one written through
        kv_copy = rows * heads * context * per_position / (hw["link_gbs"] * 1e9)
        link += kv_host * kv_copy
        if streamed == 0:
            # the first two host-KV copies (one per slot) overlap the layers in front of them
            idle = max(0.0, (shape.n_layers - kv_host) * layer - min(2, kv_host) * kv_copy)
    step = max(compute, link + idle) if link > 0 else compute
    return {"step_s": step, "tokens_per_s": rows / step, "compute_s": compute, "link_s": link}


def footprint(shape, run: dict) -> tuple:
    """(device bytes without the split-K workspace, pinned host bytes) of a run configuration."""
    tier = run.get("weight_tier", TIER_HBM_INT4)
    rows = run["gpu_batch"] * run["batches_per_block"]
    h, f, d, heads, vocab, L = shape.hidden, shape.ffn, shape.head_dim, shape.n_heads, shape.vocab, shape.n_layers
    image = _layer_weights(shape) * _bytes_per_weight(tier)
    device = 0.0
    if tier == TIER_HBM_INT4:
        device += L * image
        streamed = 0
    else:
        resident = run.get("hbm_layers", 0)
        streamed = L - resident
        device += resident * image + (2 * image if streamed else 0)
    device += L * 2.0 * ((3 * h + h + f + h) + 4 * h)   # biases and LayerNorm vectors, fp16
    device += 2.0 * h * (vocab + shape.max_pos + 2 + 2)  # token and position tables, final LayerNorm
    capacity = -(-(run["prompt_len"] + run["gen_len"] - 1) // 64) * 64
    per_slab_position = 2 * (d / 2 + 4 * (d / 64))
    cache = rows * heads * capacity * per_slab_position   # one block-layer
    kv_host = run.get("kv_host_layers", 0)
    device += run.get("n_blocks", 1) * (L - kv_host) * cache + (2 * cache if kv_host else 0)
    prefill_rows = run["gpu_batch"] * run["prompt_len"]
    work_rows = max(prefill_rows, rows)
    device += 2.0 * (rows * run["prompt_len"] * h         # block hidden states during prefill
                     + work_rows * (h + 3 * h + h + f)     # LayerNorm out, qkv, attention out, fc1 out
                     + rows * h + rows * vocab)            # last-position rows, logits
    device += 4.0 * rows                                   # token ids
    if tier != TIER_HOST_FP16:                             # quantization staging
        largest = max(f, 3 * h) * h
        device += largest * 2 + largest / 2 + 2 * (largest / 64 * 2)
    if tier == TIER_HBM_INT4:                              # decode-graph position and ids
        device += 4 + 4.0 * rows
    pinned = 0
    if tier != TIER_HBM_INT4:
        if run.get("weights_on_disk", 0):
            pinned = 2 * _aligned_image(image)   # two staging buffers; the images are in the file
        else:
            pinned = _owned_images(run, streamed) * image
    pinned += run.get("n_blocks", 1) * kv_host * cache
    return device, float(pinned)


def _aligned_image(image: float) -> float:
    return math.ceil(image / 4096) * 4096


def _owned_images(run: dict, streamed: int) -> int:
    held = run.get("host_layers", 0)
    return held if 0 < held < streamed else streamed


def disk_bytes(shape, run: dict) -> float:
    """Bytes of the weight file: the streamed layers' own images, each 4 KiB-aligned."""
    tier = run.get("weight_tier", TIER_HBM_INT4)
    if tier == TIER_HBM_INT4 or not run.get("weights_on_disk", 0):
        return 0.0
    streamed = shape.n_layers - run.get("hbm_layers", 0)
    return _owned_images(run, streamed) * _aligned_image(_layer_weights(shape) * _bytes_per_weight(tier))


def _cache_bytes(shape, run: dict) -> float:
    """One block-layer's KV cache: every (row, head) slab's capacity of K and V codes and params."""
    capacity = -(-(run["prompt_len"] + run["gen_len"] - 1) // 64) * 64
    rows = run["gpu_batch"] * run["batches_per_block"]
    d = shape.head_dim
    return rows * shape.n_heads * capacity * 2 * (d / 2 + 4 * (d / 64))


def plan(shape, prompt_len: int, gen_len: int, max_rows: int, hw: dict):
    """Most decode tokens/s over tier, GPU batch b, batches per block K (powers of two, b * K <= max_rows,
    b * K and b * prompt_len at most ROW_CAP)
    and resident layers, among configurations whose footprint fits hw's capacities. Ties keep the first
    found in the order: tier ascending (pinned images before images on disk), b descending, K
    ascending, resident layers ascending (the step
    depends on b * K only, and the largest b gives prefill its largest batches). Returns (run, estimate)
    or None."""
    best = None
    max_rows = min(max_rows, ROW_CAP)
    top = 1
    while top * 2 <= max_rows:
        top *= 2
    for tier, on_disk in ((TIER_HBM_INT4, 0), (TIER_HOST_FP16, 0), (TIER_HOST_FP16, 1), (TIER_HOST_INT4, 0),
                          (TIER_HOST_INT4, 1)):
        b = top
        while b >= 1:
            k = 1
            while b * k <= max_rows and b * prompt_len <= ROW_CAP:
                for resident in range(0, (shape.n_layers if tier != TIER_HBM_INT4 else 0) + 1):
                    run = dict(gpu_batch=b, batches_per_block=k, prompt_len=prompt_len, gen_len=gen_len,
                               group=64, weight_tier=tier, n_blocks=1, host_layers=0, hbm_layers=resident,
                               kv_host_layers=0, weights_on_disk=on_disk)
                    device, pinned = footprint(shape, run)
                    if device > hw["hbm_bytes"]:
                        # move the fewest layers' caches to the host that make it fit (the first
                        # one also adds two device slots)
                        cache = _cache_bytes(shape, run)
                        need = math.ceil((device + 2 * cache - hw["hbm_bytes"]) / cache)
                        if need > shape.n_layers:
                            continue
                        run["kv_host_layers"] = max(1, need)
                        device, pinned = footprint(shape, run)
                    if (device > hw["hbm_bytes"] or pinned > hw["host_bytes"]
                            or disk_bytes(shape, run) > hw["disk_bytes"]):
                        continue
                    est = decode_step(shape, run, hw)
                    if best is None or est["tokens_per_s"] > best[1]["tokens_per_s"]:
                        best = (run, est)
                k *= 2
            b //= 2
    return best
