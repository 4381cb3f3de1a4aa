"""The seeded input generators: determinism, slicing and distribution."""
import numpy as np

import synth


def test_deterministic_and_sliceable():
    a = synth.normal_f16(0, 7, 10000)
    b = synth.normal_f16(0, 7, 10000)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    c = synth.normal_f16(0, 7, 3000, offset=5000)
    assert np.array_equal(a[5000:8000].view(np.uint16), c.view(np.uint16))
    d = synth.normal_f16(0, 8, 10000)
    assert not np.array_equal(a.view(np.uint16), d.view(np.uint16))


def test_normal_moments():
    x = synth.normal_f16(0, 3, 2_000_000, 0.0, 0.02).astype(np.float64)
    assert abs(x.mean()) < 1e-4
    assert abs(x.std() - 0.02) < 2e-4
    assert np.abs(x).max() < 0.02 * 4.4
    y = synth.normal_f16(5, 3, 1_000_000, 1.0, 0.02).astype(np.float64)
    assert abs(y.mean() - 1.0) < 1e-4


def test_uniform_ids_range():
    ids = synth.uniform_ids(1, 0, 1_000_000, 50272)
    assert ids.min() >= 0 and ids.max() < 50272
    counts = np.bincount(ids // 5027, minlength=11)[:10]
    assert counts.min() > 0.95 * counts.mean()


def test_weight_init_variants():
    shape = synth.ModelShape(1, 64, 1, 64, 256, vocab=100, max_pos=16)
    p = synth.layer_weights(shape, 0, variant="plain")
    assert (p["q_b"] == 0).all() and (p["ln1_g"] == 1).all() and (p["ln1_b"] == 0).all()
    f = synth.layer_weights(shape, 0, variant="full")
    assert f["q_b"].std() > 0.01 and abs(f["ln1_g"].astype(np.float64).mean() - 1) < 0.01
    assert np.array_equal(p["q_w"].view(np.uint16), f["q_w"].view(np.uint16))
