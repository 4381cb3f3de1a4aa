"""Pins of the closed-form cost model against the FlexGen guide's printed simulator output."""
import math
import os

import pytest

from oracle import costmodel

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "p1_simulator.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            vals[k] = float(v)
    return vals


def test_printed_simulator_values():
    g = _golden()
    naive = costmodel.p1_naive(4, 64)
    flex = costmodel.p1_zigzag(128, 64, micro_batches=8)
    assert round(naive, 2) == g["naive_tokens_per_s"]
    assert round(flex, 2) == g["flexgen_tokens_per_s"]
    assert round(flex / naive, 1) == g["multiplier"]
    # the printed ratio is just the ratio of batch sizes
    assert flex / naive == pytest.approx(128 / 4)


def test_load_counting_model():
    W = 35e9
    assert costmodel.weight_bytes(W, 64, 8, "row_by_row") == 8 * costmodel.weight_bytes(W, 64, 8, "zigzag")
    t_rr = costmodel.throughput(W, 16e9, 64, 16, 8, "row_by_row")
    t_zz = costmodel.throughput(W, 16e9, 64, 16, 8, "zigzag")
    assert t_zz / t_rr == pytest.approx(8.0)
    with pytest.raises(ValueError):
        costmodel.weight_bytes(W, 1, 1, "column")


def test_int4_compression_ratio():
    """4 bits per value plus an fp16 scale and an fp16 zero per 64 values: 16 / 4.5 = 3.56x, not 4x."""
    bits_per_value = 4 + (16 + 16) / 64
    assert 16 / bits_per_value == pytest.approx(3.5556, abs=1e-4)


# ---------------------------------------------------------------------------
# the decode step model: pins against the simulator and closed forms
# ---------------------------------------------------------------------------

class _Shape:
    def __init__(self, n_layers, hidden, n_heads, head_dim, ffn, vocab, max_pos=2048):
        self.n_layers, self.hidden, self.n_heads, self.head_dim = n_layers, hidden, n_heads, head_dim
        self.ffn, self.vocab, self.max_pos = ffn, vocab, max_pos


FREE = dict(attn_gbs=1e12, mem_gbs=1e12, link_gbs=16.0, int4_tflops=1e12, fp16_tflops=1e12, launch_us=0.0,
            hbm_bytes=1e15, host_bytes=1e15, disk_gbs=1e12, disk_bytes=1e15, gemm_wg_us=0.0, staged_tflops=1e12,
            staged_gbs=1e12, staged_us=0.0)
MI355X = dict(attn_gbs=6250.0, mem_gbs=7100.0, link_gbs=57.2, int4_tflops=1340.0, fp16_tflops=1400.0,
              launch_us=4.0, hbm_bytes=280e9, host_bytes=270e9, disk_gbs=7.4, disk_bytes=80e9, gemm_wg_us=25.0,
              staged_tflops=1700.0, staged_gbs=3230.0, staged_us=10.0)


def test_free_compute_reduces_to_the_printed_simulator():
    """Compute that costs nothing and an all-streamed fp16 model of exactly 35 GB (35 layers of
    hidden 5000 and ffn 40000: 10^9 fp16 bytes each) over a 16 GB/s link: the step is the
    simulator's transfer time, so 4 and 128 rows give its printed 1.83 and 58.51 tokens/s."""
    g = _golden()
    shape = _Shape(35, 5000, 40, 125, 40000, 1000)
    for rows, key in ((4, "naive_tokens_per_s"), (128, "flexgen_tokens_per_s")):
        run = dict(gpu_batch=rows, batches_per_block=1, prompt_len=16, gen_len=8, weight_tier=1)
        est = costmodel.decode_step(shape, run, FREE)
        assert est["link_s"] == pytest.approx(35e9 / 16e9, rel=1e-12)
        assert round(est["tokens_per_s"], 2) == g[key]


def test_resident_tier_has_no_link_and_a_fully_resident_host_tier_matches_it():
    shape = _Shape(8, 1024, 16, 64, 4096, 5000)
    base = dict(gpu_batch=8, batches_per_block=4, prompt_len=64, gen_len=16)
    t0 = costmodel.decode_step(shape, dict(base, weight_tier=0), MI355X)
    assert t0["link_s"] == 0.0 and t0["step_s"] == t0["compute_s"]
    t2 = costmodel.decode_step(shape, dict(base, weight_tier=2, hbm_layers=8), MI355X)
    assert t2["link_s"] == 0.0 and t2["step_s"] == t0["step_s"]


def test_link_bound_step_is_the_copy_time_and_shrinks_with_resident_layers():
    """OPT-175B shape, int4 streamed: each streamed layer moves its image once per step."""
    shape = _Shape(96, 12288, 96, 128, 49152, 50272)
    image = (4 * 12288 ** 2 + 2 * 12288 * 49152) * (0.5 + 4 / 64)
    run = dict(gpu_batch=32, batches_per_block=8, prompt_len=16, gen_len=32, weight_tier=2)
    prev = None
    for resident in range(0, 97, 8):
        est = costmodel.decode_step(shape, dict(run, hbm_layers=resident), MI355X)
        assert est["link_s"] == pytest.approx((96 - resident) * image / 57.2e9, rel=1e-12)
        if resident == 0:
            assert est["step_s"] == pytest.approx(est["link_s"], rel=1e-12)
        if prev is not None:
            assert est["step_s"] <= prev
        prev = est["step_s"]


def test_footprint_terms():
    """Adding 64 cache positions adds exactly one 64-position slab per (layer, row, head) for K and V;
    one more resident layer adds one layer image; pinned memory holds the streamed images."""
    shape = _Shape(6, 2048, 16, 128, 8192, 5000)
    run = dict(gpu_batch=16, batches_per_block=4, prompt_len=100, gen_len=10, weight_tier=2, hbm_layers=2)
    d0, p0 = costmodel.footprint(shape, run)
    d1, _ = costmodel.footprint(shape, dict(run, gen_len=run["gen_len"] + 64))
    assert d1 - d0 == 6 * 64 * 16 * 64 * (128 + 128 / 8)
    d2, p2 = costmodel.footprint(shape, dict(run, hbm_layers=3))
    image = (4 * 2048 ** 2 + 2 * 2048 * 8192) * 0.5625
    assert d2 - d0 == pytest.approx(image, rel=1e-12)
    assert p0 == pytest.approx(4 * image, rel=1e-12) and p2 == pytest.approx(3 * image, rel=1e-12)
    _, p3 = costmodel.footprint(shape, dict(run, host_layers=1))
    assert p3 == pytest.approx(image, rel=1e-12)


def test_images_on_disk():
    """With the images in a file, the slower of the disk read and the link copy paces each streamed
    layer; pinned memory is two staging images and the file holds the owned images, 4 KiB-aligned."""
    shape = _Shape(96, 12288, 96, 128, 49152, 50272)
    image = (4 * 12288 ** 2 + 2 * 12288 * 49152) * (0.5 + 4 / 64)
    run = dict(gpu_batch=32, batches_per_block=8, prompt_len=16, gen_len=32, weight_tier=2, hbm_layers=16,
               host_layers=8, weights_on_disk=1)
    est = costmodel.decode_step(shape, run, MI355X)
    assert est["link_s"] == pytest.approx(80 * image / 7.4e9, rel=1e-12)
    fast_disk = dict(MI355X, disk_gbs=1e6)
    assert costmodel.decode_step(shape, run, fast_disk)["link_s"] == pytest.approx(80 * image / 57.2e9, rel=1e-12)
    aligned = -(-image // 4096) * 4096
    assert costmodel.footprint(shape, run)[1] == pytest.approx(2 * aligned, rel=1e-12)
    assert costmodel.disk_bytes(shape, run) == pytest.approx(8 * aligned, rel=1e-12)
    assert costmodel.disk_bytes(shape, dict(run, weights_on_disk=0)) == 0.0


def test_gemm_is_the_larger_of_its_flops_and_its_weight_stream():
    """Closed forms of one GEMM: compute-bound at many rows (flops / rate + the fixed cost), bound by
    its weight bytes at few rows (bytes / streaming rate + the fixed cost), and the crossover row
    count where the two terms are equal: rows* = rate x bytes-per-weight / (2 x streaming rate)."""
    hw = dict(MI355X, launch_us=0.0)
    n, k = 28672, 7168
    assert costmodel.gemm_time(4096, n, k, True, hw) == pytest.approx(2 * 4096 * n * k / 1340e12 + 25e-6, rel=1e-12)
    assert costmodel.gemm_time(8, n, k, True, hw) == pytest.approx(n * k * 0.5625 / 7100e9 + 25e-6, rel=1e-12)
    cross = 1340e12 * 0.5625 / (2 * 7100e9)
    lo, hi = math.floor(cross), math.ceil(cross)
    assert costmodel.gemm_time(lo, n, k, True, hw) == pytest.approx(n * k * 0.5625 / 7100e9 + 25e-6, rel=1e-12)
    assert costmodel.gemm_time(hi, n, k, True, hw) == pytest.approx(2 * hi * n * k / 1340e12 + 25e-6, rel=1e-12)


def test_fp16_weights_use_their_own_rate_and_bytes():
    hw = dict(MI355X, launch_us=0.0, gemm_wg_us=0.0)
    assert costmodel.gemm_time(512, 50272, 7168, False, hw) == pytest.approx(2 * 512 * 50272 * 7168 / 1400e12,
                                                                              rel=1e-12)
    assert costmodel.gemm_time(8, 50272, 7168, False, hw) == pytest.approx(50272 * 7168 * 2.0 / 7100e9, rel=1e-12)


def test_every_kernel_costs_at_least_a_launch():
    hw = dict(FREE, launch_us=4.0)
    assert costmodel.gemm_time(1, 64, 64, True, hw) == pytest.approx(4e-6, rel=1e-12)
    shape = _Shape(2, 64, 1, 64, 256, 100)
    run = dict(gpu_batch=1, batches_per_block=1, prompt_len=4, gen_len=2)
    # per layer: 4 GEMMs, attention, KV append; head: embedding, LayerNorm, LM head, argmax
    assert costmodel.decode_step(shape, run, hw)["step_s"] == pytest.approx((2 * 6 + 4) * 4e-6, rel=1e-12)
