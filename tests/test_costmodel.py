"""Pins of the closed-form cost model against the FlexGen guide's printed simulator output."""
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


def test_gemm_plan_splits_and_tile_heights():
    """The planner rule at the decode shapes: QKV of OPT-30B fills one wave with 192-row tiles,
    fc1 with 256-row ones and fc2 splits their 56 tiles' K four ways; the out-projection takes
    112 tiles of 128 rows split twice (half the partials of 256-row tiles split four ways); at
    256 rows the OPT-6.7B GEMMs take 128-row tiles split 2 or 8 ways; at 128 rows or fewer int4
    GEMMs take 128- or 64-row tiles, fp16 ones 64-row tiles."""
    p = costmodel.gemm_plan(512, 21504, 7168, True)
    assert (p["tile_rows"], p["splits"], p["workgroups"]) == (192, 1, 252)
    p = costmodel.gemm_plan(512, 28672, 7168, True)
    assert (p["tile_rows"], p["splits"], p["workgroups"], p["groups_per_split"]) == (256, 1, 224, 112)
    p = costmodel.gemm_plan(512, 7168, 28672, True)
    assert (p["tile_rows"], p["splits"], p["workgroups"], p["groups_per_split"]) == (256, 4, 224, 112)
    p = costmodel.gemm_plan(512, 7168, 7168, True)
    assert (p["tile_rows"], p["splits"], p["workgroups"], p["groups_per_split"]) == (128, 2, 224, 56)
    assert [(p["tile_rows"], p["splits"]) for p in (costmodel.gemm_plan(256, n, k, True) for n, k in
            ((12288, 4096), (4096, 4096), (16384, 4096), (4096, 16384)))] == [(128, 2), (128, 8), (128, 2), (128, 8)]
    p = costmodel.gemm_plan(128, 4096, 4096, True)
    assert (p["tile_rows"], p["splits"], p["workgroups"]) == (64, 8, 256)
    # OPT-125m's GEMMs at 8 rows would give 3 to 12 workgroups: register-staged
    assert all(costmodel.gemm_plan(8, n, k, True) is None for n, k in ((2304, 768), (768, 768), (3072, 768),
                                                                        (768, 3072)))
    assert [costmodel.gemm_plan(r, 28672, 7168, True)["tile_rows"] for r in (8, 64, 128)] == [64, 64, 128]
    p = costmodel.gemm_plan(8, 50272, 7168, False)
    assert (p["tile_rows"], p["splits"], p["workgroups"]) == (64, 1, 197)
    p = costmodel.gemm_plan(512, 50272, 7168, False)  # the fp16 LM head: 256-row tiles, two waves
    assert (p["tile_rows"], p["splits"], p["workgroups"]) == (256, 1, 394)
    assert costmodel.gemm_plan(512, 50200, 7168, False) is None  # N not a multiple of 32


def test_gemm_in_whole_waves_of_full_tiles_runs_at_the_steady_rate():
    """With no fixed cost, a GEMM whose 256 x 256 tiles fill whole waves of 256 workgroups, unsplit,
    takes exactly its flops over the steady int4 rate (one and two waves)."""
    hw = dict(MI355X, gemm_wg_us=0.0, launch_us=0.0)
    for rows in (512, 1024):
        t = costmodel.gemm_time(rows, 32768, 4096, True, hw)
        assert t == pytest.approx(2.0 * rows * 32768 * 4096 / 1340e12, rel=1e-12)


def test_gemm_fixed_cost_counts_once_per_wave():
    hw = dict(MI355X, int4_tflops=1e30, mem_gbs=1e30, launch_us=0.0, gemm_wg_us=25.0)
    assert costmodel.gemm_time(512, 32768, 4096, True, hw) == pytest.approx(25e-6, rel=1e-9)
    assert costmodel.gemm_time(1024, 32768, 4096, True, hw) == pytest.approx(50e-6, rel=1e-9)


def test_split_gemm_pays_its_partials_twice():
    """With free compute and no fixed cost, a GEMM costs its weight stream, and a GEMM whose K loop
    is split also its fp32 partials (splits x rows x N) written once and read once, all at the
    streaming rate."""
    hw = dict(MI355X, int4_tflops=1e30, launch_us=0.0, gemm_wg_us=0.0)
    weights = 7168 * 28672 * 0.5625 / 7100e9  # fc2 of OPT-30B at 512 rows: K split four ways
    assert costmodel.gemm_time(512, 7168, 28672, True, hw) == pytest.approx(
        weights + 2 * 4 * 512 * 7168 * 4 / 7100e9, rel=1e-12)
    assert costmodel.gemm_time(512, 28672, 7168, True, hw) == pytest.approx(weights, rel=1e-12)


def test_register_staged_gemm_limits():
    """fp16 weights whose N is not a multiple of 32: with free flops and no fixed cost a GEMM is its
    weight bytes at the kernel's read rate; each added row adds exactly its flops."""
    hw = dict(MI355X, launch_us=0.0, staged_us=0.0, staged_tflops=1e30)
    assert costmodel.gemm_plan(128, 4004, 4096, False) is None
    assert costmodel.gemm_time(128, 4004, 4096, False, hw) == pytest.approx(4004 * 4096 * 2.0 / 3230e9, rel=1e-12)
    hw = dict(MI355X, launch_us=0.0)
    step = costmodel.gemm_time(65, 4004, 4096, False, hw) - costmodel.gemm_time(64, 4004, 4096, False, hw)
    assert step == pytest.approx(2.0 * 4004 * 4096 / 1700e12, rel=1e-9)


def test_pipelined_gemm_is_no_faster_than_its_weight_stream():
    """With free flops, the fp16 LM head of OPT-30B at 8 rows (one wave, unsplit) costs its weights
    read once at the streaming rate plus the fixed cost."""
    hw = dict(MI355X, launch_us=0.0, fp16_tflops=1e30)
    assert costmodel.gemm_time(8, 50272, 7168, False, hw) == pytest.approx(50272 * 7168 * 2.0 / 7100e9 + 25e-6,
                                                                           rel=1e-12)


def test_fp16_gemm_in_whole_waves_runs_at_the_fp16_steady_rate():
    hw = dict(MI355X, gemm_wg_us=0.0, launch_us=0.0)
    assert costmodel.gemm_time(512, 32768, 4096, False, hw) == pytest.approx(2.0 * 512 * 32768 * 4096 / 1400e12,
                                                                             rel=1e-12)
