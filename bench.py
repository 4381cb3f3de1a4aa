#!/usr/bin/env python3
"""Decode throughput of block-scheduled int4 OPT decode on one MI355X.

Workload (default): OPT-30B-shaped stack (48 layers, hidden 7168, 56 heads of
128, FFN 28672, vocab 50272), random N(0, 0.02) fp16 weights quantized to
int4 group-64 in HBM, int4 group-64 KV cache, GPU batch 64 x 8 batches per
block (512 rows), uniform random prompts of 512 tokens, 32 generated tokens.

A step is one decode step of the whole block through the whole stack: embed,
48 x (LN, fused int4 QKV GEMM, KV quantize+append, int4-KV attention, out
GEMM, LN, FC1, FC2), final LN, LM head, greedy argmax. The timed region
replays decode steps 1..31 (contexts 513..543) after one prefill; the KV
cache and weights are resident in HBM when it starts.

Prints one JSON line. `value` is decode tokens/s = rows * steps / time.
`roofline` reports the kernel class with the largest share of the step,
timed with HIP events on the library's stream over a second pass of the
same steps (launched one by one; the timed region replays captured graphs),
and beside it (`step_achieved`, `step_frac`) the whole step's algorithmic
HBM bytes over the step time. `cpu_baseline` times the CPU oracle on a
bounded sample (one layer and one decode step for every row of the block,
plus the LM head for those rows) and extrapolates to the stack.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "generated tokens/sec (1 GPU), OPT-30B shape int4 W+KV; % of HBM roofline"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
BPE_INT4 = 0.5 + 4.0 / 64.0   # bytes per int4 element incl. fp16 scale + zero per 64


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kv_bytes_per_position(shape):
    """K and V of one (sequence, position, layer): codes + (scale, zero) per 64."""
    return 2 * shape.hidden * BPE_INT4


def step_bytes(shape, rows, context):
    """Algorithmic HBM bytes of one decode step at a given attended context."""
    L, h, f, V = shape.n_layers, shape.hidden, shape.ffn, shape.vocab
    w = L * (4 * h * h + 2 * f * h) * BPE_INT4          # int4 weights, once per step for the whole block
    lm = V * h * 2                                       # tied fp16 LM head
    kv_read = rows * L * kv_bytes_per_position(shape) * context
    kv_write = rows * L * kv_bytes_per_position(shape)
    logits = rows * V * 2
    return w + lm + kv_read + kv_write + logits


def gemm_shapes(shape, rows):
    h, f = shape.hidden, shape.ffn
    return {"gemm_qkv": (rows, 3 * h, h), "gemm_o": (rows, h, h), "gemm_fc1": (rows, f, h),
            "gemm_fc2": (rows, h, f), "lm_head": (rows, shape.vocab, h)}


def build_model(tod, synth, w, log_every=8, kv_host_layers=0):
    shape = w.shape
    run = dict(gpu_batch=w.gpu_batch, batches_per_block=w.batches_per_block, prompt_len=w.prompt_len,
               gen_len=w.gen_len, weight_tier=w.weight_tier, kv_host_layers=kv_host_layers)
    m = tod.Model(shape, run)
    g = synth.global_weights(shape)
    m.set_global_weights(g["tok_emb"], g["pos_emb"], g["lnf_g"], g["lnf_b"])
    del g
    for l in range(shape.n_layers):
        m.set_layer_weights(l, synth.layer_weights(shape, l))
        if (l + 1) % log_every == 0 or l + 1 == shape.n_layers:
            log(f"weights: {l + 1}/{shape.n_layers} layers loaded")
    return m


def measure_h2d(torch, nbytes, reps=3):
    """Pinned host -> HBM copy rate (GB/s) for one copy of nbytes on a side stream."""
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        dst.copy_(src, non_blocking=True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            dst.copy_(src, non_blocking=True)
        e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return nbytes / (ms * 1e-3) / 1e9


def measure_disk_read(path, image_bytes, n_images):
    """GB/s of reads of the weight file's images, one image per read as the library issues them,
    no copy to the device: the better of direct (O_DIRECT) reads and buffered reads whose pages are
    dropped from the page cache afterwards (the library's method). Returns (best, direct, buffered)."""
    import mmap
    stride = -(-image_bytes // 4096) * 4096
    buf = mmap.mmap(-1, stride)  # page-aligned, as O_DIRECT needs
    rates = []
    for flags in (getattr(os, "O_DIRECT", 0), 0):
        fd = os.open(path, os.O_RDONLY | flags)
        try:
            for i in range(n_images):  # start cold
                os.posix_fadvise(fd, i * stride, stride, os.POSIX_FADV_DONTNEED)
            t0 = time.perf_counter()
            for i in range(n_images):
                done = 0
                while done < stride:
                    n = os.preadv(fd, [memoryview(buf)[done:]], i * stride + done)
                    if n <= 0:
                        raise OSError("short read of the weight file")
                    done += n
                os.posix_fadvise(fd, i * stride, stride, os.POSIX_FADV_DONTNEED)
            rates.append(n_images * image_bytes / (time.perf_counter() - t0) / 1e9)
        finally:
            os.close(fd)
    buf.close()
    return max(rates), rates[0], rates[1]


def cost_model_check(tod, shape, run, measured_ms):
    """The library's cost model (estimate_decode, default measured rates) for this run beside the
    measured step time."""
    est = tod.estimate_decode(shape, run)
    return {"predicted_ms_per_step": est["step_s"] * 1e3,
            "measured_over_predicted": measured_ms / (est["step_s"] * 1e3),
            "predicted_hbm_gb": est["hbm_bytes"] / 1e9, "predicted_host_gb": est["host_bytes"] / 1e9}


def host_tier_bench(args, w, tod, synth, torch):
    """Decode with weights streamed per layer from pinned host memory: fp16
    (weight tier 1) or the tiled int4 image (tier 2, 0.5625 byte per weight).

    The step is bound by the host link (every streamed layer's matrices cross
    it once per step), so the report is tokens/s and link GB/s against a
    measured pinned -> HBM copy of the same size. --hbm-layers R keeps the
    first R layers' images resident in HBM (they never cross the link); of the
    streamed layers only --host-layers distinct ones keep pinned matrices (the
    others stream those in turn), so the stack fits host memory, and resident
    layers other than layer 0 are given layer 0's matrices with their own
    vectors (values do not change the work). The prompt is shortened
    (--prompt-len, default 16) because prefill at 512 tokens would take minutes
    of fp16 GEMMs, and a link-bound step does not depend on the attended
    context."""
    import dataclasses
    w = dataclasses.replace(w, prompt_len=args.prompt_len or 16)
    shape, M = w.shape, w.rows
    L, h, f = shape.n_layers, shape.hidden, shape.ffn
    R = min(max(args.hbm_layers, 0), L)
    P = min(args.host_layers, L - R)
    on_disk = bool(args.weight_file)
    run = dict(gpu_batch=w.gpu_batch, batches_per_block=w.batches_per_block, prompt_len=w.prompt_len,
               gen_len=w.gen_len, weight_tier=w.weight_tier, host_layers=P, hbm_layers=R,
               weights_on_disk=int(on_disk))
    t_setup = time.perf_counter()
    m = tod.Model(shape, run, weight_file=args.weight_file or None)
    g = synth.global_weights(shape)
    m.set_global_weights(g["tok_emb"], g["pos_emb"], g["lnf_g"], g["lnf_b"])
    del g
    mats = ("q_w", "k_w", "v_w", "o_w", "fc1_w", "fc2_w")
    shared = None
    for l in range(L):
        if l == 0 or R <= l < R + P:
            t = synth.layer_weights(shape, l)
            if shared is None:
                shared = {n: t[n] for n in mats}  # placeholders for layers that reuse a copy
        else:
            t = {n: synth.draw_tensor(shape, n, l) for n in synth.LAYER_TENSORS if n not in mats}
            t.update(shared)
        m.set_layer_weights(l, t)
        del t
        if (l + 1) % 8 == 0 or l + 1 == L:
            log(f"weights: {l + 1}/{L} layers set ({R} resident in HBM, {P} with pinned matrices)")
    del shared
    prompts = torch.from_numpy(synth.prompt_ids(M, w.prompt_len, shape.vocab)).cuda()
    first = torch.empty(M, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    log(f"setup {time.perf_counter() - t_setup:.1f} s")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    tod.prefill(m.handle, 0, prompts, first)
    e1.record()
    torch.cuda.synchronize()
    prefill_s = e0.elapsed_time(e1) / 1e3
    log(f"prefill {prefill_s:.2f} s")
    out = torch.empty((w.gen_len - 1, M), dtype=torch.int32, device="cuda")
    steps, warm = args.steps, args.warmup
    if warm:
        tod.decode_block(m.handle, 0, warm, first, out[:warm])
    torch.cuda.synchronize()
    log(f"warm-up {warm} step(s) done")
    ids = out[warm - 1] if warm else first
    t0 = time.perf_counter()
    tod.decode_block(m.handle, 0, steps, ids, out[warm:warm + steps])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    m.close()
    del m
    torch.cuda.empty_cache()
    int4 = w.weight_tier == 2
    layer_weights = 4 * h * h + 2 * f * h
    layer_bytes = layer_weights // 2 + layer_weights // 16 if int4 else layer_weights * 2
    link_gbs = (L - R) * layer_bytes * steps / elapsed / 1e9
    log("measuring pinned -> HBM copy rate ...")
    h2d = measure_h2d(torch, layer_bytes)
    disk = disk_direct = disk_buffered = None
    if on_disk:
        log("measuring direct reads of the weight file ...")
        disk, disk_direct, disk_buffered = measure_disk_read(args.weight_file, layer_bytes, P)
        os.remove(args.weight_file)
    return {
        "metric": f"generated tokens/sec (1 GPU), OPT-175B shape {'int4' if int4 else 'fp16'} weights streamed "
                  "from pinned host; % of measured host-link bandwidth",
        "value": M * steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": elapsed * 1e3 / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4-f16" if int4 else "f16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}-shaped {'int4' if int4 else 'fp16'} host-streamed block decode",
                   "layers": L, "hidden": h,
                   "heads": shape.n_heads, "head_dim": shape.head_dim, "ffn": f, "vocab": shape.vocab,
                   "gpu_batch": w.gpu_batch, "batches_per_block": w.batches_per_block, "rows": M,
                   "prompt_len": w.prompt_len, "gen_len": w.gen_len, "hbm_layers": R, "host_layers_pinned": P,
                   "weights": ("int4 group-64 (tiled codes + fp16 scale/zero)" if int4 else "fp16")
                   + (" in a file on disk, read into 2 pinned staging buffers" if on_disk else
                      " in pinned host memory") + ", 2 HBM layer slots, copies on a side stream"},
        "roofline": ({"bound": "link", "achieved": link_gbs, "peak": h2d, "unit": "GB/s", "frac": link_gbs / h2d,
                      "traffic": None, "kernel": "hipMemcpyAsync pinned -> HBM (one layer per copy)"}
                     if not on_disk else
                     {"bound": "disk", "achieved": link_gbs, "peak": min(disk, h2d), "unit": "GB/s",
                      "frac": link_gbs / min(disk, h2d), "traffic": None,
                      "kernel": "pread -> pinned staging -> hipMemcpyAsync -> HBM, one layer per read"}),
        "disk_read_measured_gbs": disk,
        "disk_read_direct_gbs": disk_direct if on_disk else None,
        "disk_read_buffered_gbs": disk_buffered if on_disk else None,
        "link_bytes_per_step": (L - R) * layer_bytes,
        "h2d_measured_gbs": h2d,
        "prefill_s": prefill_s,
        "cost_model": cost_model_check(tod, shape, run, elapsed * 1e3 / steps),
    }


def attention_bench(args, tod, synth, torch):
    """The isolated decode-attention + KV-quantize workload: batch x heads
    sequences with `context` cached int4 positions; each step quantizes and
    appends one new K/V per sequence and attends over everything cached.
    Inputs come from torch's seeded device generator, N(0, 1) fp16 (same
    shapes and distribution as the parity tests' host-generated data)."""
    W = synth.ATTN_WORKLOAD
    B, H, d, T = W["batch"], W["heads"], W["head_dim"], W["context"]
    steps, warm = args.steps, args.warmup
    c = tod.attn_cache_create(B, H, d, T + warm + steps)
    gen = torch.Generator(device="cuda").manual_seed(2)
    for t0 in range(0, T, 128):
        n = min(128, T - t0)
        k = torch.randn((n, B, H, d), generator=gen, device="cuda", dtype=torch.float16)
        v = torch.randn((n, B, H, d), generator=gen, device="cuda", dtype=torch.float16)
        tod.attn_cache_fill(c, k, v, t0)
        del k, v
    q = [torch.randn((B, H, d), generator=gen, device="cuda", dtype=torch.float16) for _ in range(3 * (warm + steps))]
    out = torch.empty((B, H, d), dtype=torch.float16, device="cuda")
    for i in range(warm):
        tod.attn_decode_step(c, T + i, q[3 * i], q[3 * i + 1], q[3 * i + 2], out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(warm, warm + steps):
        tod.attn_decode_step(c, T + i, q[3 * i], q[3 * i + 1], q[3 * i + 2], out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    tod.attn_cache_free(c)
    G = d // 64
    per_pos = 2 * (d // 2 + 4 * G)                 # K and V codes + (scale, zero) per group
    ctx_avg = T + warm + (steps + 1) / 2.0          # attended positions, averaged over the timed steps
    kv_read = B * H * per_pos * ctx_avg
    other = B * H * d * 2 * 4 + B * H * per_pos     # q, k_new, v_new, out (fp16) + the appended codes
    gbs = (kv_read + other) / (ms * 1e-3) / 1e9
    return {
        "metric": "decode attention + KV quantize step over an int4 cache (1 GPU); % of HBM roofline",
        "value": ms, "unit": "ms/step", "n_gpus": 1, "steps": steps, "warmup": warm, "ms_per_step": ms,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "isolated decode attention + KV append", "batch": B, "heads": H, "head_dim": d,
                   "cached_context": T, "context_avg": ctx_avg},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None, "kernel": "k_kv_append + k_attn_decode<128>"},
    }


def cpu_model():
    """The host CPU's model name (first processor entry of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, rows=None, passes=1):
    """The oracle on one layer x one decode step of the whole block (every row, at the average
    decode context) plus the LM head for those rows (about 30 s on a 16-core host); extrapolated
    to the whole stack as rows / (layers x t_layer + t_lm)."""
    import numpy as np

    import oracle
    import synth
    shape = w.shape
    rows = rows or w.rows
    ctx = w.prompt_len + (w.gen_len - 1) // 2          # average attended context - 1 cached positions
    layer = oracle.Layer(shape, synth.layer_weights(shape, 0))
    glob = synth.global_weights(shape)
    caches = []
    for r in range(rows):
        c = oracle.KVCache(shape, ctx + 1)
        k = synth.normal_f16(4096 + r, 0, (ctx, shape.hidden), 0.0, 1.0)
        v = synth.normal_f16(4096 + r, 1, (ctx, shape.hidden), 0.0, 1.0)
        c.store(0, k, v)
        caches.append(c)
    hid = synth.normal_f16(8191, 0, (rows, shape.hidden), 0.0, 1.0)
    t0 = time.perf_counter()
    for _ in range(passes):  # each pass rewrites the same cache position
        for r in range(rows):
            layer.forward(caches[r], ctx, hid[r:r + 1])
    t_layer = (time.perf_counter() - t0) / passes
    t0 = time.perf_counter()
    for _ in range(passes):
        oracle.head(shape, glob["lnf_g"], glob["lnf_b"], glob["tok_emb"], hid)
    t_lm = (time.perf_counter() - t0) / passes
    del caches
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    tps = rows / (shape.n_layers * t_layer + t_lm)
    return {"value": tps, "unit": "tokens/s", "cores": cores, "cpu": cpu_model(), "kind": "oracle",
            "sample": (f"1 of {shape.n_layers} layers x 1 decode step x all {rows} sequences of the block at context "
                       f"{ctx + 1} ({t_layer:.2f} s) + LM head for {rows} rows ({t_lm:.2f} s), {passes} timed "
                       f"pass(es); extrapolated as {rows} / ({shape.n_layers} * t_layer + t_lm)")}


# HBM traffic of the dominant kernel, measured separately with rocprofv3 counters
# (FETCH_SIZE and WRITE_SIZE per dispatch, scaled by the same counters on a plain
# copy of known size) and kept with the profiles as the ratio of measured to
# algorithmic bytes; a run reports that ratio times its own algorithmic bytes per
# launch. It is reported only while the kernel's sources are unchanged since the
# counters were taken.
TRAFFIC_FILES = {"k_attn_decode<128>": ("profiles/k_attn_decode_opt30b_counters.txt",
                                        ("throughput_oriented_offloaded_amd/csrc/attn.hip",
                                         "throughput_oriented_offloaded_amd/csrc/common.hpp"))}


def source_digest(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, algorithmic_bytes):
    """Measured HBM bytes per launch (the recorded ratio times this run's algorithmic bytes), or None
    if the summary is absent or its kernel sources have changed since."""
    if kernel not in TRAFFIC_FILES:
        return None
    summary, sources = TRAFFIC_FILES[kernel]
    try:
        with open(os.path.join(ROOT, summary)) as f:
            fields = dict(line.split(":", 1) for line in f if line.startswith(("traffic_ratio:", "source_sha256:")))
    except OSError:
        return None
    if fields.get("source_sha256", "").strip() != source_digest(sources):
        return None
    try:
        return float(fields["traffic_ratio"]) * algorithmic_bytes
    except (KeyError, ValueError):
        return None


def copy_probe(mib):
    """A plain device copy of known size, for calibrating the HBM byte counters."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.bitwise_not(src, out=dst)  # one elementwise kernel: reads n bytes, writes n bytes
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)


def blas_probe():
    """fp16 GEMMs of the vendor library (torch.mm, hipBLASLt on ROCm) at the OPT-30B decode shapes and on
    two large ones: a measured practical ceiling for the int4 GEMMs' rate on this part. Context only: the
    library never calls it."""
    import torch
    torch.manual_seed(0)
    for m, n, k in ((512, 21504, 7168), (512, 7168, 7168), (512, 28672, 7168), (512, 7168, 28672),
                    (512, 50272, 7168), (8192, 8192, 8192), (32768, 28672, 7168)):
        a = torch.randn(m, k, device="cuda", dtype=torch.float16)
        wt = (torch.randn(n, k, device="cuda", dtype=torch.float16) * 0.02).t().contiguous()
        reps = 50 if m * n * k < 1e12 else 10
        for _ in range(5):
            torch.mm(a, wt)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.mm(a, wt)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        print(json.dumps({"blas_probe": "torch.mm fp16", "m": m, "n": n, "k": k, "us": us,
                          "tflops": 2 * m * n * k / us / 1e6}), flush=True)
        del a, wt
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed decode steps (default 31; fp16 host tier 2, int4 host tier 6)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed decode steps first (default 2; host tiers 1)")
    ap.add_argument("--workload", default="opt-30b",
                    help="opt-125m | opt-6.7b | opt-30b (default) | opt-175b (fp16 host tier) | "
                         "opt-175b-int4 (int4 host tier) | attention")
    ap.add_argument("--cpu-baseline", choices=("on", "off"), default="on")
    ap.add_argument("--prompt-len", type=int, default=0, help="host tiers only: prompt length (default 16)")
    ap.add_argument("--kv-host-layers", type=int, default=0,
                    help="HBM-weight workloads: trailing layers whose KV cache lives in pinned host memory "
                         "(default 0; not the headline configuration)")
    ap.add_argument("--weight-file", default="",
                    help="host tiers only: keep the streamed images in this file (created or truncated; buffered "
                         "reads, each image dropped from the page cache after use)")
    ap.add_argument("--hbm-layers", type=int, default=0,
                    help="host tiers only: leading layers whose weights stay resident in HBM (default 0)")
    ap.add_argument("--host-layers", type=int, default=8,
                    help="host tiers only: layers with their own pinned matrices (default 8)")
    ap.add_argument("--progress", action="store_true",
                    help="one decode step per call with a log line each (long profiler runs); not for the metric")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    ap.add_argument("--blas-probe", action="store_true",
                    help="only time the vendor library's fp16 GEMMs at the decode shapes (a ceiling) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (see the design notes on "
              "sharding); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.blas_probe:
        blas_probe()
        return

    import synth
    import throughput_oriented_offloaded_amd as tod

    if args.workload == "attention":
        args.steps = args.steps or 16
        args.warmup = 2 if args.warmup is None else args.warmup
        print(json.dumps(attention_bench(args, tod, synth, torch)), flush=True)
        return
    w = synth.WORKLOADS[args.workload]
    if args.steps is None:
        args.steps = {1: 2, 2: 6}.get(w.weight_tier, 31)
    if args.warmup is None:
        args.warmup = 1 if w.weight_tier else 2
    if w.weight_tier:
        print(json.dumps(host_tier_bench(args, w, tod, synth, torch)), flush=True)
        return
    shape, M = w.shape, w.rows
    torch.cuda.set_device(0)
    t_setup = time.perf_counter()
    m = build_model(tod, synth, w, kv_host_layers=args.kv_host_layers)
    prompts = torch.from_numpy(synth.prompt_ids(M, w.prompt_len, shape.vocab)).cuda()
    first = torch.empty(M, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    log(f"setup {time.perf_counter() - t_setup:.1f} s")

    # prefill (its own timed region, reported beside the decode metric)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    tod.prefill(m.handle, 0, prompts, first)
    e1.record()
    torch.cuda.synchronize()
    prefill_s = e0.elapsed_time(e1) / 1e3
    log(f"prefill {prefill_s:.2f} s")

    max_steps = w.gen_len - 1
    out = torch.empty((max_steps, M), dtype=torch.int32, device="cuda")

    def run_steps(n):
        """n decode steps, replaying steps 1..gen_len-1 from the prefill state."""
        done = 0
        state = run_steps.state
        while done < n:
            if state["decoded"] == max_steps:
                tod.set_decode_position(m.handle, 0, 0)
                state["decoded"], state["ids"] = 0, first
            k = min(n - done, max_steps - state["decoded"])
            if args.progress:
                k = 1  # one step per call, so every step can report
            tod.decode_block(m.handle, 0, k, state["ids"], out[state["decoded"]:state["decoded"] + k])
            state["ids"] = out[state["decoded"] + k - 1]
            state["decoded"] += k
            done += k
            if args.progress:
                torch.cuda.synchronize()
                log(f"{run_steps.label}: {done}/{n} decode steps")
            run_steps.contexts.extend(range(w.prompt_len + state["decoded"] - k + 1,
                                            w.prompt_len + state["decoded"] + 1))
    run_steps.state = {"decoded": 0, "ids": first}
    run_steps.contexts = []
    run_steps.label = "timed pass"

    def restart():
        tod.set_decode_position(m.handle, 0, 0)
        run_steps.state = {"decoded": 0, "ids": first}
        run_steps.contexts = []

    # warm-up (captures the decode step's graph), then the timed region: the
    # default path, replayed graphs, nothing else on the stream
    run_steps(args.warmup)
    torch.cuda.synchronize()
    restart()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(args.steps)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    contexts = list(run_steps.contexts)

    # per-kernel averages: the same steps again, each launch bracketed by HIP
    # events on the library's stream (step-by-step launches while timing)
    restart()
    run_steps.label = "profiled pass"
    kinds = ("gemm_qkv", "gemm_o", "gemm_fc1", "gemm_fc2", "attn", "kv_append", "layernorm", "lm_head",
             "argmax", "embed")
    tod.profile_kernels(m.handle, kinds)
    torch.cuda.synchronize()
    tp = time.perf_counter()
    run_steps(args.steps)
    torch.cuda.synchronize()
    elapsed_prof = time.perf_counter() - tp
    prof = {k: tod.profile_read(m.handle, k) for k in kinds}
    tod.profile_kernels(m.handle, ())

    ms_per_step = elapsed * 1e3 / args.steps
    value = M * args.steps / elapsed
    ctx_avg = sum(contexts) / len(contexts)
    bytes_avg = sum(step_bytes(shape, M, c) for c in contexts) / len(contexts)
    hbm_frac = bytes_avg / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9)

    # per-kernel-class achieved rates over the profiled pass
    kernels = {}
    shapes = gemm_shapes(shape, M)
    for k, (ms, n) in prof.items():
        if n == 0:
            continue
        entry = {"launches": n, "avg_us": ms * 1e3 / n, "share": ms / (elapsed_prof * 1e3)}
        if k in shapes:
            r, nn, kk = shapes[k]
            tflops = 2.0 * r * nn * kk * n / (ms * 1e-3) / 1e12
            entry.update(bound="mfma", achieved_tflops=tflops, frac=tflops / MFMA_F16_PEAK_TFLOPS)
        elif k == "attn":
            # per launch (one layer): K and V of every cached position of every row, plus q and the output
            total = sum((M * kv_bytes_per_position(shape) * c + 2 * M * shape.hidden * 2) * shape.n_layers
                        for c in contexts)
            gbs = total / (ms * 1e-3) / 1e9
            entry.update(bound="hbm", achieved_gbs=gbs, frac=gbs / HBM_PEAK_GBS, bytes_per_launch=total / n)
        kernels[k] = entry
    dom = max((k for k in kernels if "frac" in kernels[k]), key=lambda k: kernels[k]["share"])
    d = kernels[dom]
    if d["bound"] == "hbm":
        kname = f"k_attn_decode<{shape.head_dim}>"
        roof = {"bound": "hbm", "achieved": d["achieved_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": d["frac"],
                "traffic": measured_traffic(kname, d["bytes_per_launch"]) if w.name == "opt-30b" else None,
                "kernel": kname}
    else:
        roof = {"bound": "mfma", "achieved": d["achieved_tflops"], "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": d["frac"], "traffic": None, "kernel": f"k_gemm ({dom})"}
    # the whole step against HBM: algorithmic bytes of a step (weights once, the LM head, every cached
    # K/V read, the appends and the logits) over the step time
    roof.update(step_achieved=bytes_avg / (ms_per_step * 1e-3) / 1e9, step_frac=hbm_frac,
                step_unit="GB/s of algorithmic step bytes")

    result = {
        "metric": METRIC.replace("OPT-30B", "OPT-" + w.name[4:].replace("b", "B")),
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}-shaped int4 W+KV block decode", "layers": shape.n_layers,
                   "hidden": shape.hidden, "heads": shape.n_heads, "head_dim": shape.head_dim, "ffn": shape.ffn,
                   "vocab": shape.vocab, "gpu_batch": w.gpu_batch, "batches_per_block": w.batches_per_block,
                   "rows": M, "prompt_len": w.prompt_len, "gen_len": w.gen_len, "context_avg": ctx_avg,
                   "weights": "int4 g64 in HBM" if w.weight_tier == 0 else "fp16 streamed from pinned host",
                   "kv_host_layers": args.kv_host_layers},
        "roofline": roof,
        "hbm_frac_step": hbm_frac,
        "algorithmic_gb_per_step": bytes_avg / 1e9,
        "ms_per_step_step_launches": elapsed_prof * 1e3 / args.steps,
        "prefill_s": prefill_s,
        "e2e_tokens_per_s": M * w.gen_len / (prefill_s + (w.gen_len - 1) * ms_per_step * 1e-3),
        "kernels": kernels,
        "cost_model": cost_model_check(tod, shape, dict(gpu_batch=w.gpu_batch, batches_per_block=w.batches_per_block,
                                                        prompt_len=w.prompt_len, gen_len=w.gen_len,
                                                        kv_host_layers=args.kv_host_layers),
                                       ms_per_step),
    }
    m.close()
    del m
    torch.cuda.empty_cache()
    if args.cpu_baseline == "on":
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
