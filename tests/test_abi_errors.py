"""Argument checks of the C entry points, called through the C ABI without a GPU.

Every check exercised here runs before the library touches the device (the
header promises TOD_EINVAL for these arguments), so the calls return on a
machine with no GPU. Fake non-null addresses stand in for device buffers that
a rejected call never reads.
"""
import ctypes
import os

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EINVAL, ENOMEM = -1, -2
FAKE = 0x100000  # 16-byte aligned, never dereferenced by a rejected call
NULL = None


@pytest.fixture(scope="module")
def lib():
    from throughput_oriented_offloaded_amd import _lib
    return _lib.lib()


def _err(lib):
    return lib.last_error().decode()


def test_group_wise_quantization_arguments(lib):
    q, d = lib.quantize_groupwise, lib.dequantize_groupwise
    assert q(FAKE, 128, 32, FAKE, FAKE, FAKE, NULL) == EINVAL and "group" in _err(lib)
    assert q(FAKE, 100, 64, FAKE, FAKE, FAKE, NULL) == EINVAL and "multiple" in _err(lib)
    assert q(FAKE, -64, 64, FAKE, FAKE, FAKE, NULL) == EINVAL
    for i in range(4):
        ptrs = [FAKE] * 4
        ptrs[i] = NULL
        assert q(ptrs[0], 64, 64, ptrs[1], ptrs[2], ptrs[3], NULL) == EINVAL and "null" in _err(lib)
        assert d(ptrs[0], ptrs[1], ptrs[2], 64, 64, ptrs[3], NULL) == EINVAL and "null" in _err(lib)
    assert d(FAKE, FAKE, FAKE, 64, 128, FAKE, NULL) == EINVAL and "group" in _err(lib)
    assert d(FAKE, FAKE, FAKE, 65, 64, FAKE, NULL) == EINVAL


@pytest.mark.parametrize("case,rows,inp,out,codes,scale,zero,residual,relu", [
    ("null a", 8, 64, 32, FAKE, FAKE, FAKE, NULL, 0),
    ("negative rows", -1, 64, 32, FAKE, FAKE, FAKE, NULL, 0),
    ("rows above 2^31 - 1", 1 << 31, 64, 32, FAKE, FAKE, FAKE, NULL, 0),
    ("in not a multiple of 64", 8, 96, 32, FAKE, FAKE, FAKE, NULL, 0),
    ("in zero", 8, 0, 32, FAKE, FAKE, FAKE, NULL, 0),
    ("out zero", 8, 64, 0, FAKE, FAKE, FAKE, NULL, 0),
    ("int4 out not a multiple of 32", 8, 64, 48, FAKE, FAKE, FAKE, NULL, 0),
    ("null scale", 8, 64, 32, FAKE, NULL, FAKE, NULL, 0),
    ("null zero", 8, 64, 32, FAKE, FAKE, NULL, NULL, 0),
    ("null codes", 8, 64, 32, NULL, FAKE, FAKE, NULL, 0),
    ("relu with residual", 8, 64, 32, FAKE, FAKE, FAKE, FAKE, 1),
])
def test_linear_w4_arguments(lib, case, rows, inp, out, codes, scale, zero, residual, relu):
    a = NULL if case == "null a" else FAKE
    rc = lib.linear_w4(a, rows, inp, out, codes, scale, zero, NULL, residual, relu, FAKE, NULL)
    assert rc == EINVAL, (case, _err(lib))


def test_linear_f16_arguments(lib):
    assert lib.linear_f16(FAKE, 8, 64, 40, NULL, NULL, NULL, 0, FAKE, NULL) == EINVAL
    assert "weights" in _err(lib)
    assert lib.linear_f16(FAKE, 8, 64, 40, FAKE, NULL, NULL, 0, NULL, NULL) == EINVAL  # null y
    assert lib.linear_f16(FAKE, 8, 64, 40, FAKE, NULL, FAKE, 1, FAKE, NULL) == EINVAL
    assert "relu" in _err(lib)


def test_attention_cache_arguments(lib):
    out = ctypes.c_void_p(FAKE)
    for batch, heads, d, cap in ((0, 4, 64, 64), (2, 0, 64, 64), (2, 4, 96, 64), (2, 4, 64, 0)):
        out.value = FAKE
        assert lib.attn_cache_create(batch, heads, d, cap, ctypes.byref(out)) == EINVAL
        assert out.value is None  # *out is cleared on error
    assert lib.attn_cache_create(2, 4, 64, 64, NULL) == EINVAL
    assert lib.attn_cache_fill(NULL, FAKE, FAKE, 0, 1, NULL) == EINVAL
    assert lib.attn_decode_step(NULL, 0, FAKE, FAKE, FAKE, FAKE, NULL) == EINVAL
    assert lib.attn_cache_export(NULL, 0, 0, 0, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == EINVAL
    assert lib.attn_cache_free(NULL) == 0


def test_null_model_handle(lib):
    """Every call that takes a model handle rejects a null one; freeing null is a no-op."""
    ptrs = (ctypes.c_void_p * 16)(*([FAKE] * 16))
    ms, n = ctypes.c_double(), ctypes.c_int64()
    calls = {
        "set_global_weights": lambda: lib.set_global_weights(NULL, FAKE, FAKE, FAKE, FAKE),
        "set_layer_weights": lambda: lib.set_layer_weights(NULL, 0, ptrs),
        "set_weight_file": lambda: lib.set_weight_file(NULL, b"/nonexistent"),
        "prefill": lambda: lib.prefill(NULL, 0, FAKE, FAKE, NULL, NULL),
        "decode_block": lambda: lib.decode_block(NULL, 0, 1, FAKE, FAKE, NULL, NULL),
        "set_decode_position": lambda: lib.set_decode_position(NULL, 0, 0),
        "set_decode_graph": lambda: lib.set_decode_graph(NULL, 1),
        "export_weight": lambda: lib.export_weight(NULL, 0, 0, FAKE, FAKE, FAKE, NULL),
        "export_kv": lambda: lib.export_kv(NULL, 0, 0, 0, 0, 0, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL),
        "profile_kernels": lambda: lib.profile_kernels(NULL, 1),
        "profile_read": lambda: lib.profile_read(NULL, 0, ctypes.byref(ms), ctypes.byref(n)),
    }
    for name, call in calls.items():
        assert call() == EINVAL, name
    assert lib.free_model(NULL) == 0


OK_RUN = dict(gpu_batch=2, batches_per_block=1, prompt_len=4, gen_len=3)
BAD_CONFIGS = [  # (what, model-shape changes, run changes)
    ("group 32", {}, dict(group=32)),
    ("zero gpu_batch", {}, dict(gpu_batch=0)),
    ("zero blocks", {}, dict(n_blocks=0)),
    ("blocks above TOD_MAX_BLOCKS", {}, dict(n_blocks=4097)),
    ("unknown tier", {}, dict(weight_tier=7)),
    ("past max_pos", {}, dict(gen_len=4000)),
    ("resident layers on the HBM tier", {}, dict(hbm_layers=1)),
    ("held layers on the HBM tier", {}, dict(host_layers=1)),
    ("too many resident layers", {}, dict(weight_tier=2, hbm_layers=2)),
    ("too many host-KV layers", {}, dict(kv_host_layers=2)),
    ("negative host-KV layers", {}, dict(kv_host_layers=-1)),
    ("disk on the HBM tier", {}, dict(weights_on_disk=1)),
    ("disk flag 2", {}, dict(weight_tier=2, weights_on_disk=2)),
    ("block rows above 2^24", {}, dict(gpu_batch=1 << 13, batches_per_block=1 << 12)),
    ("prefill rows above 2^24", {}, dict(gpu_batch=1 << 14, prompt_len=2044)),
    ("hidden != heads * head_dim", dict(n_heads=6), {}),
    ("head_dim 96", dict(hidden=768, n_heads=8, head_dim=96), {}),
    ("ffn not a multiple of 64", dict(ffn=3000), {}),
    ("hidden above 16384", dict(hidden=16448, n_heads=257, head_dim=64), {}),
    ("zero max_pos", dict(max_pos=0), {}),
    ("zero vocab", dict(vocab=0), {}),
]


@pytest.mark.parametrize("what,shape_changes,run_changes", BAD_CONFIGS, ids=[c[0] for c in BAD_CONFIGS])
def test_init_model_and_estimate_reject_the_same_configurations(lib, what, shape_changes, run_changes):
    """init_model rejects each invalid configuration with TOD_EINVAL before any allocation or device
    call (so it returns here, with no GPU), and estimate_decode rejects it with the same message."""
    from throughput_oriented_offloaded_amd import _lib
    shape = synth.OPT_125M.replace(n_layers=1, **shape_changes)
    mc, rc = _lib._model_config(shape), _lib._run_config(dict(OK_RUN, **run_changes))
    h = ctypes.c_void_p(FAKE)
    assert lib.init_model(ctypes.byref(mc), ctypes.byref(rc), NULL, ctypes.byref(h)) == EINVAL, what
    assert h.value is None
    msg = _err(lib)
    assert msg
    lib.quantize_groupwise(FAKE, 64, 32, FAKE, FAKE, FAKE, NULL)  # leave a different message behind
    hw, est = _lib.HW(**_lib.default_hw()), _lib.Estimate()
    assert lib.estimate_decode(ctypes.byref(mc), ctypes.byref(rc), ctypes.byref(hw), ctypes.byref(est)) == EINVAL
    assert _err(lib) == msg


def test_valid_configuration_passes_the_checks(lib):
    """The base configuration of the cases above is one estimate_decode accepts."""
    from throughput_oriented_offloaded_amd import _lib
    est = _lib.estimate_decode(synth.OPT_125M.replace(n_layers=1), OK_RUN)
    assert est["tokens_per_s"] > 0


def test_estimate_and_plan_null_and_rate_arguments(lib):
    from throughput_oriented_offloaded_amd import _lib
    mc, rc = _lib._model_config(synth.OPT_125M), _lib._run_config(OK_RUN)
    hw, est, best = _lib.HW(**_lib.default_hw()), _lib.Estimate(), _lib.RunConfig()
    assert lib.estimate_decode(ctypes.byref(mc), ctypes.byref(rc), ctypes.byref(hw), NULL) == EINVAL
    assert lib.estimate_decode(NULL, ctypes.byref(rc), ctypes.byref(hw), ctypes.byref(est)) == EINVAL
    for field in ("attn_gbs", "mem_gbs", "link_gbs", "int4_tflops", "fp16_tflops", "disk_gbs", "staged_tflops",
                  "staged_gbs"):
        bad = _lib.HW(**dict(_lib.default_hw(), **{field: 0.0}))
        assert lib.estimate_decode(ctypes.byref(mc), ctypes.byref(rc), ctypes.byref(bad),
                                   ctypes.byref(est)) == EINVAL, field
        assert "rates" in _err(lib)
    for field in ("launch_us", "gemm_wg_us", "staged_us"):
        bad = _lib.HW(**dict(_lib.default_hw(), **{field: -1.0}))
        assert lib.estimate_decode(ctypes.byref(mc), ctypes.byref(rc), ctypes.byref(bad),
                                   ctypes.byref(est)) == EINVAL, field
    for prompt, gen, rows in ((0, 8, 8), (32, 0, 8), (32, 8, 0), (2048, 2, 8)):
        assert lib.plan_decode(ctypes.byref(mc), prompt, gen, rows, ctypes.byref(hw), ctypes.byref(best),
                               ctypes.byref(est)) == EINVAL, (prompt, gen, rows)
    tiny = _lib.HW(**dict(_lib.default_hw(), hbm_bytes=1e6))
    assert lib.plan_decode(ctypes.byref(mc), 32, 8, 8, ctypes.byref(tiny), ctypes.byref(best),
                           ctypes.byref(est)) == ENOMEM
    assert "fits" in _err(lib)


def test_plan_keeps_within_the_row_limits():
    """With room for anything, the search stops at the library's row limits: b * K and b * prompt_len
    at most 2^24 (init_model rejects more), the same choice as the oracle's search (GEMMs made free,
    where the two step models agree exactly)."""
    from oracle import costmodel
    from throughput_oriented_offloaded_amd import _lib
    shape = synth.OPT_125M.replace(n_layers=2)
    hw = dict(_lib.default_hw(), hbm_bytes=1e18, host_bytes=1e18, disk_bytes=1e18, int4_tflops=1e30,
              fp16_tflops=1e30, staged_tflops=1e30, staged_gbs=1e30, staged_us=0.0, gemm_wg_us=0.0, mem_gbs=1e30)
    run, est = _lib.plan_decode(shape, 2048, 1, 1 << 15, hw)
    assert run["gpu_batch"] * 2048 <= 1 << 24 and run["gpu_batch"] * run["batches_per_block"] <= 1 << 15
    ref_run, ref_est = costmodel.plan(shape, 2048, 1, 1 << 15, hw)
    assert (run["gpu_batch"], run["batches_per_block"], run["weight_tier"]) == \
        (ref_run["gpu_batch"], ref_run["batches_per_block"], ref_run["weight_tier"])
    assert est["tokens_per_s"] == pytest.approx(ref_est["tokens_per_s"], rel=1e-12)
    _lib.estimate_decode(shape, run, hw)  # a configuration the checks accept
