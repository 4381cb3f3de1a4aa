"""Pins of the oracle's group-wise 4-bit quantizer.

The pages fix only "group-wise, 16-bit to 4-bit, small contiguous groups"
(FlexGen guide, "3. Group-Wise 4-Bit Quantization"). The oracle's reading is
min/max asymmetric with 15 steps; these tests pin it by means other than its
own code: a closed-form error bound, a 16-candidate brute-force search, exact
special cases and a numpy decode of the packed nibbles.
"""
import numpy as np
import pytest

import oracle
from tests.quant_cases import adversarial_groups

G = 64


def _unpack(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.size * 2, dtype=np.int64)
    out[0::2] = codes & 15
    out[1::2] = codes >> 4
    return out


def _brute_force(x16):
    """Nearest grid index by exhaustive search over the 16 codes (ties to the larger)."""
    x = x16.reshape(-1, G).astype(np.float32)
    mn = x.min(axis=1, keepdims=True)
    mx = x.max(axis=1, keepdims=True)
    s32 = ((mx - mn).astype(np.float32) / np.float32(15.0)).astype(np.float32)
    s16 = s32.astype(np.float16)
    d = (x - mn).astype(np.float32).astype(np.float64)           # fl32(x - min)
    grid = np.arange(16, dtype=np.float64)[None, None, :] * s16.astype(np.float64)[:, :, None]
    dist = np.abs(d[:, :, None] - grid)
    # ties to the larger code: search from the top
    best = 15 - np.argmin(dist[:, :, ::-1], axis=2)
    best[(s16 == 0).reshape(-1)] = 0
    return best.reshape(-1), s16.reshape(-1), mn.astype(np.float16).reshape(-1)


@pytest.mark.parametrize("sigma", [0.02, 1.0, 300.0])
def test_brute_force_normal(sigma):
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(64 * 4000) * sigma).astype(np.float16)
    codes, scale, zero = oracle.quantize_groupwise(x)
    bc, bs, bz = _brute_force(x)
    assert np.array_equal(_unpack(codes), bc)
    assert np.array_equal(scale.view(np.uint16), bs.view(np.uint16))
    assert np.array_equal(zero.view(np.uint16), (bz + np.float16(0)).view(np.uint16))


def test_brute_force_adversarial():
    x = adversarial_groups()
    codes, scale, zero = oracle.quantize_groupwise(x)
    bc, bs, bz = _brute_force(x)
    assert np.array_equal(_unpack(codes), bc)
    assert np.array_equal(scale.view(np.uint16), bs.view(np.uint16))
    # a zero minimum is stored as +0
    assert np.array_equal(zero.view(np.uint16), (bz + np.float16(0)).view(np.uint16))


@pytest.mark.parametrize("sigma", [0.02, 1.0])
def test_roundtrip_error_bound(sigma):
    """|x - xhat| <= scale/2 + ulp16(xhat)/2 (+ ulp32(x - min)/2 if that difference was rounded)."""
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(64 * 8000) * sigma).astype(np.float16)
    codes, scale, zero = oracle.quantize_groupwise(x)
    xh = oracle.dequantize_groupwise(codes, scale, zero).astype(np.float64)
    s = np.repeat(scale.astype(np.float64), G)
    mn = np.repeat(zero.astype(np.float64), G)
    xd = x.astype(np.float64)
    normal = s >= 2.0 ** -14
    d_exact = xd - mn
    d32 = d_exact.astype(np.float32).astype(np.float64)
    slack = np.where(d32 != d_exact, np.spacing(np.abs(d32).astype(np.float32)).astype(np.float64) / 2, 0.0)
    bound = s / 2 + np.spacing(np.abs(xh).astype(np.float16)).astype(np.float64) / 2 + slack
    err = np.abs(xd - xh)
    assert np.all(err[normal] <= bound[normal])
    assert normal.mean() > 0.99


def test_min_and_max_codes():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(64 * 2000) * 0.02).astype(np.float16).reshape(-1, G)
    codes, scale, zero = oracle.quantize_groupwise(x)
    c = _unpack(codes).reshape(-1, G)
    xh = oracle.dequantize_groupwise(codes, scale, zero).reshape(-1, G)
    rows = np.arange(x.shape[0])
    imin = np.argmin(x, axis=1)
    imax = np.argmax(x, axis=1)
    assert np.all(c[rows, imin] == 0)
    assert np.array_equal(xh[rows, imin].view(np.uint16), x[rows, imin].view(np.uint16))
    assert np.all(c[rows, imax] == 15)


def test_counting_group_packs_exactly():
    """x_i = i mod 16: scale 1, codes i mod 16, bytes 0x10 0x32 ... 0xFE, zero error."""
    x = (np.arange(G) % 16).astype(np.float16)
    codes, scale, zero = oracle.quantize_groupwise(x)
    assert float(scale[0]) == 1.0 and float(zero[0]) == 0.0
    assert list(codes[:8]) == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    assert np.array_equal(codes, np.tile(codes[:8], 4))
    assert np.array_equal(oracle.dequantize_groupwise(codes, scale, zero), x)


def test_constant_group_is_all_zero_codes():
    for v in (0.0, -0.0, 1.5, -65504.0, 6e-8):
        x = np.full(G, v, dtype=np.float16)
        codes, scale, zero = oracle.quantize_groupwise(x)
        assert not codes.any() and float(scale[0]) == 0.0
        assert np.array_equal(oracle.dequantize_groupwise(codes, scale, zero).astype(np.float64),
                              np.full(G, float(np.float16(v)) + 0.0))


def test_exact_ties_round_to_larger_code():
    s = 2.0 ** -6
    mn = -0.25
    k = np.arange(15)
    vals = np.concatenate([[mn, mn + 15 * s], mn + (k + 0.5) * s])
    x = np.concatenate([vals, np.full(G - vals.size, mn)]).astype(np.float16)
    assert np.array_equal(x.astype(np.float64)[:vals.size], vals)  # all exact in fp16
    codes, scale, zero = oracle.quantize_groupwise(x)
    c = _unpack(codes)
    assert float(scale[0]) == s
    assert list(c[2:17]) == list(k + 1)


def test_on_grid_weights_dequantize_exactly():
    """A group built as min + c * s (s a power of two) quantizes back to c with no error."""
    rng = np.random.default_rng(4)
    c = rng.integers(0, 16, size=(500, G))
    c[:, 0], c[:, 1] = 0, 15
    s = 2.0 ** rng.integers(-12, -6, size=(500, 1))
    mn = -rng.integers(0, 200, size=(500, 1)) * s
    x = (mn + c * s).astype(np.float16)
    assert np.array_equal(x.astype(np.float64), mn + c * s)
    codes, scale, zero = oracle.quantize_groupwise(x)
    assert np.array_equal(_unpack(codes), c.reshape(-1))
    assert np.array_equal(oracle.dequantize_groupwise(codes, scale, zero), x.reshape(-1))


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.quantize_groupwise(np.full(G, np.inf, dtype=np.float16))
    with pytest.raises(ValueError):
        oracle.quantize_groupwise(np.zeros(G + 2, dtype=np.float16))
