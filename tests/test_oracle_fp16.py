"""Pins of the oracle's own fp16 conversion against numpy's IEEE binary16."""
import numpy as np

import oracle


def test_half_to_double_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.half_to_double(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_half_roundtrip_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    finite = np.isfinite(vals) | np.isinf(vals)
    back = oracle.double_to_half(vals[finite])
    assert np.array_equal(back, bits[finite])


def test_double_to_half_matches_numpy_rne():
    with np.errstate(over="ignore"):
        _check_rne()


def _check_rne():
    rng = np.random.default_rng(0)
    h = np.arange(0, 0x7c00, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    nxt = np.nextafter(h.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    mid = (h + nxt) / 2.0                       # exact ties between neighbours
    cases = [mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf),
             rng.standard_normal(200000) * 0.02, rng.standard_normal(200000) * 1e3,
             rng.uniform(-1e-7, 1e-7, 200000), np.exp(rng.uniform(-20, 11.1, 200000)),
             np.array([65504.0, 65519.99, 65520.0, 65536.0, 1e30, 2.0 ** -25, 2.0 ** -24, 3 * 2.0 ** -26,
                       0.0, -0.0, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25])]
    x = np.concatenate(cases)
    x = np.concatenate([x, -x])
    ours = oracle.double_to_half(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)
