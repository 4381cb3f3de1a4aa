"""The library's cost model and placement search (C ABI, host code only) against the oracle's.

Both price a decode step from the same measured rates (oracle/costmodel.py
writes the definition out term by term); the oracle's device footprint
leaves out the split-K workspace, which the library reports separately.
The search cases are ones where that omission cannot change the winner;
where it can, the library's choice is checked to fit and to be within 1%
of the oracle's optimum.
"""
import itertools

import pytest

import synth
from oracle import costmodel

SHAPES = ("opt-125m", "opt-6.7b", "opt-30b", "opt-175b")


def _lib():
    import throughput_oriented_offloaded_amd as tod
    return tod


@pytest.mark.parametrize("name", SHAPES)
def test_estimate_matches_oracle(name):
    tod = _lib()
    hw = tod.default_hw()
    shape = synth.WORKLOADS[name].shape
    L = shape.n_layers
    for tier, (b, k), resident, (s, g), held, kv_host, on_disk in itertools.product(
            (0, 1, 2), ((1, 1), (4, 2), (64, 8), (32, 8)), (0, 1, L // 2, L), ((16, 32), (512, 32), (100, 7)),
            (0, 3), (0, 1, L), (0, 1)):
        if tier == 0 and (resident or held or on_disk):
            continue
        run = dict(gpu_batch=b, batches_per_block=k, prompt_len=s, gen_len=g, weight_tier=tier,
                   hbm_layers=resident, host_layers=held, kv_host_layers=kv_host, weights_on_disk=on_disk)
        got = tod.estimate_decode(shape, run, hw)
        ref = costmodel.decode_step(shape, run, hw)
        for key in ("step_s", "tokens_per_s", "compute_s", "link_s"):
            assert got[key] == pytest.approx(ref[key], rel=1e-12, abs=0.0), (run, key)
        device, pinned = costmodel.footprint(shape, run)
        assert got["hbm_bytes"] - got["workspace_bytes"] == pytest.approx(device, rel=1e-12), run
        assert got["host_bytes"] == pytest.approx(pinned, rel=1e-12), run
        assert got["disk_bytes"] == pytest.approx(costmodel.disk_bytes(shape, run), rel=1e-12), run
        assert 0 <= got["workspace_bytes"] < 1e9
        assert got["fits"] == (got["hbm_bytes"] <= hw["hbm_bytes"] and got["host_bytes"] <= hw["host_bytes"] and
                               got["disk_bytes"] <= hw["disk_bytes"])


PLAN_CASES = [  # shape, prompt, gen, max rows, device GB, pinned GB
    ("opt-30b", 512, 32, 512, 280, 270),
    ("opt-175b", 512, 32, 256, 280, 270),
    ("opt-175b", 512, 32, 256, 150, 270),
    ("opt-6.7b", 512, 32, 1024, 40, 270),
    ("opt-30b", 2000, 32, 8, 20, 270),
    ("opt-30b", 2000, 32, 64, 90, 270),
    ("opt-175b", 512, 32, 256, 60, 270),     # int4 weights do not fit: streamed, every cache on the host
    ("opt-175b", 512, 32, 256, 90, 270),
    ("opt-175b", 2000, 32, 64, 60, 270),     # long prompts: some caches stay in HBM
    ("opt-175b", 2000, 32, 64, 100, 270),
    ("opt-175b", 512, 32, 256, 60, 20),      # little pinned memory: the streamed images go to disk
]


@pytest.mark.parametrize("name,prompt_len,gen_len,max_rows,hbm_gb,host_gb", PLAN_CASES)
def test_plan_matches_oracle(name, prompt_len, gen_len, max_rows, hbm_gb, host_gb):
    """Same configuration and tokens/s as the oracle's search. In these cases no candidate that
    could win sits within the library's split-K workspace of the device capacity (which the
    oracle leaves out); see the next test for cases that do."""
    tod = _lib()
    shape = synth.WORKLOADS[name].shape
    hw = dict(tod.default_hw(), hbm_bytes=hbm_gb * 1e9, host_bytes=host_gb * 1e9)
    run, est = tod.plan_decode(shape, prompt_len, gen_len, max_rows, hw)
    ref_run, ref_est = costmodel.plan(shape, prompt_len, gen_len, max_rows, hw)
    for key in ("gpu_batch", "batches_per_block", "weight_tier", "hbm_layers", "host_layers", "prompt_len",
                "gen_len", "group", "n_blocks", "kv_host_layers", "weights_on_disk"):
        assert run[key] == ref_run[key], (key, run, ref_run)
    assert est["tokens_per_s"] == pytest.approx(ref_est["tokens_per_s"], rel=1e-12)
    assert est["fits"] == 1
    print(f"{name} prompt {prompt_len} rows <= {max_rows} hbm {hbm_gb} GB host {host_gb} GB -> tier "
          f"{run['weight_tier']} b {run['gpu_batch']} K {run['batches_per_block']} resident {run['hbm_layers']} "
          f"host-KV layers {run['kv_host_layers']} on disk {run['weights_on_disk']}: "
          f"{est['tokens_per_s']:.1f} tokens/s")


@pytest.mark.parametrize("name,prompt_len,gen_len,max_rows,hbm_gb,host_gb", [
    ("opt-175b", 512, 32, 256, 80, 270), ("opt-175b", 512, 32, 256, 80, 30), ("opt-175b", 512, 32, 256, 100, 270)])
def test_plan_near_capacity_boundaries(name, prompt_len, gen_len, max_rows, hbm_gb, host_gb):
    """Where the split-K workspace decides a fit, the library may pick an adjacent configuration
    (a smaller GPU batch, one more host-KV layer): it must fit by its own footprint and be within 1%
    of the oracle's optimum."""
    tod = _lib()
    shape = synth.WORKLOADS[name].shape
    hw = dict(tod.default_hw(), hbm_bytes=hbm_gb * 1e9, host_bytes=host_gb * 1e9)
    run, est = tod.plan_decode(shape, prompt_len, gen_len, max_rows, hw)
    _, ref_est = costmodel.plan(shape, prompt_len, gen_len, max_rows, hw)
    again = tod.estimate_decode(shape, run, hw)
    assert again["fits"] == 1 and again["hbm_bytes"] <= hw["hbm_bytes"]
    assert est["tokens_per_s"] == pytest.approx(ref_est["tokens_per_s"], rel=1e-2)
    assert est["tokens_per_s"] <= ref_est["tokens_per_s"] * (1 + 1e-12)


def test_errors():
    tod = _lib()
    shape = synth.WORKLOADS["opt-125m"].shape
    ok = dict(gpu_batch=4, batches_per_block=2, prompt_len=32, gen_len=8)
    for bad in (dict(ok, gpu_batch=0), dict(ok, weight_tier=3), dict(ok, hbm_layers=2),
                dict(ok, weight_tier=2, hbm_layers=13)):
        with pytest.raises(tod.TodError):
            tod.estimate_decode(shape, bad)
    with pytest.raises(tod.TodError):
        tod.estimate_decode(shape, ok, dict(tod.default_hw(), link_gbs=0.0))
    with pytest.raises(tod.TodError):  # nothing fits in 1 MB
        tod.plan_decode(shape, 32, 8, 8, dict(tod.default_hw(), hbm_bytes=1e6))
