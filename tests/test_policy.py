"""The library's cost model and placement search (C ABI, host code only) against the oracle's.

Both price a decode step from the same measured rates (oracle/costmodel.py
writes the definition out term by term); the oracle's device footprint
leaves out the split-K workspace, which the library reports separately.
The search cases keep the device capacity at least 256 MB away from every
candidate's footprint, so that omission cannot change a fit decision.
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
    for tier, (b, k), resident, (s, g), held in itertools.product(
            (0, 1, 2), ((1, 1), (4, 2), (64, 8), (32, 8)), (0, 1, L // 2, L), ((16, 32), (512, 32), (100, 7)),
            (0, 3)):
        if tier == 0 and (resident or held):
            continue
        run = dict(gpu_batch=b, batches_per_block=k, prompt_len=s, gen_len=g, weight_tier=tier,
                   hbm_layers=resident, host_layers=held)
        got = tod.estimate_decode(shape, run, hw)
        ref = costmodel.decode_step(shape, run, hw)
        for key in ("step_s", "tokens_per_s", "compute_s", "link_s"):
            assert got[key] == pytest.approx(ref[key], rel=1e-12, abs=0.0), (run, key)
        device, pinned = costmodel.footprint(shape, run)
        assert got["hbm_bytes"] - got["workspace_bytes"] == pytest.approx(device, rel=1e-12), run
        assert got["host_bytes"] == pytest.approx(pinned, rel=1e-12), run
        assert 0 <= got["workspace_bytes"] < 1e9
        assert got["fits"] == (got["hbm_bytes"] <= hw["hbm_bytes"] and got["host_bytes"] <= hw["host_bytes"])


def _capacity_away_from_footprints(shape, prompt_len, gen_len, max_rows, target, margin=256e6):
    """A device capacity near `target` with no candidate footprint within `margin` of it."""
    fps = []
    top = 1
    while top * 2 <= max_rows:
        top *= 2
    for tier in (0, 1, 2):
        b = top
        while b >= 1:
            k = 1
            while b * k <= max_rows:
                for r in range(0, (shape.n_layers if tier else 0) + 1):
                    run = dict(gpu_batch=b, batches_per_block=k, prompt_len=prompt_len, gen_len=gen_len,
                               weight_tier=tier, hbm_layers=r)
                    fps.append(costmodel.footprint(shape, run)[0])
                k *= 2
            b //= 2
    cap = target
    while any(abs(f - cap) < margin for f in fps):
        cap += margin / 4
    return cap


@pytest.mark.parametrize("name,prompt_len,gen_len,max_rows,hbm_target,host", [
    ("opt-30b", 512, 32, 512, 280e9, 270e9),
    ("opt-175b", 512, 32, 256, 280e9, 270e9),
    ("opt-175b", 512, 32, 256, 80e9, 270e9),    # int4 weights alone do not fit: streaming wins
    ("opt-175b", 512, 32, 256, 80e9, 30e9),     # little pinned memory: more layers stay resident
    ("opt-6.7b", 512, 32, 1024, 40e9, 270e9),
])
def test_plan_matches_oracle(name, prompt_len, gen_len, max_rows, hbm_target, host):
    tod = _lib()
    shape = synth.WORKLOADS[name].shape
    hw = dict(tod.default_hw(), host_bytes=host)
    hw["hbm_bytes"] = _capacity_away_from_footprints(shape, prompt_len, gen_len, max_rows, hbm_target)
    run, est = tod.plan_decode(shape, prompt_len, gen_len, max_rows, hw)
    ref_run, ref_est = costmodel.plan(shape, prompt_len, gen_len, max_rows, hw)
    for key in ("gpu_batch", "batches_per_block", "weight_tier", "hbm_layers", "host_layers", "prompt_len",
                "gen_len", "group", "n_blocks"):
        assert run[key] == ref_run[key], (key, run, ref_run)
    assert est["tokens_per_s"] == pytest.approx(ref_est["tokens_per_s"], rel=1e-12)
    assert est["fits"] == 1
    print(f"{name} hbm {hw['hbm_bytes'] / 1e9:.1f} GB host {host / 1e9:.0f} GB -> tier {run['weight_tier']} "
          f"b {run['gpu_batch']} K {run['batches_per_block']} resident {run['hbm_layers']}: "
          f"{est['tokens_per_s']:.1f} tokens/s")


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
