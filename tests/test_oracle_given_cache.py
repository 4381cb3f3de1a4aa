"""Pins of the oracle entries used for teacher-forced layer checks, and of its two switches.

* ``KVCache.load`` is the inverse of ``KVCache.export``.
* ``Layer.forward_given_kv`` on a cache that ``Layer.forward`` filled gives
  ``Layer.forward``'s output bit for bit (an invariant tying it to the pinned
  layer), and its k/v quantize to the stored codes.
* ``exact_v`` (attention on exact real dequantized V values): closed forms
  (one cached position returns that value rounded once; identical keys return
  the exact rational mean of the values rounded once), the special case where
  every value is on the fp16 grid (both readings agree bit for bit), and the
  bound between the two readings (half an fp16 ulp of the largest value).
* ``fp32_accumulation``: a closed-form cancellation (2^24 + 1 - 2^24 is 0 in
  fp32, 1 in fp64); sums whose partial sums are exact in fp32 agree with the
  fp64 oracle; and numpy float32 sequential-sum references of a linear layer,
  a LayerNorm and an attention, written from the switch's definition (every
  running sum rounded to fp32 after each addition; terms in float64).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

G = 64


def _shape(h=128, heads=2, d=64, f=256):
    return synth.ModelShape(n_layers=1, hidden=h, n_heads=heads, head_dim=d, ffn=f, vocab=300, max_pos=128)


def _bits(x):
    return np.asarray(x).view(np.uint16)


def test_kv_load_is_the_inverse_of_export():
    shape = _shape()
    rng = np.random.default_rng(21)
    T = 11
    src = oracle.KVCache(shape, T)
    src.store(0, rng.standard_normal((T, 128)).astype(np.float16), rng.standard_normal((T, 128)).astype(np.float16))
    dst = oracle.KVCache(shape, T)
    for hd in range(shape.n_heads):
        dst.load(hd, 0, *src.export(hd, 0, T))
    for hd in range(shape.n_heads):
        for a, b in zip(src.export(hd, 0, T), dst.export(hd, 0, T)):
            assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
    with pytest.raises(ValueError):
        dst.load(shape.n_heads, 0, *src.export(0, 0, T))


def test_forward_given_the_oracles_own_cache_equals_forward():
    shape = _shape()
    tw = synth.layer_weights(shape, 0, variant="full")
    layer = oracle.Layer(shape, tw)
    rng = np.random.default_rng(22)
    T = 9
    hid = rng.standard_normal((T, 128)).astype(np.float16)
    own = oracle.KVCache(shape, T)
    full = layer.forward(own, 0, hid)
    given = oracle.KVCache(shape, T)
    for hd in range(shape.n_heads):
        given.load(hd, 0, *own.export(hd, 0, T))
    out, k, v = layer.forward_given_kv(given, 0, hid)
    assert np.array_equal(_bits(out), _bits(full))
    for t in (0, 4, T - 1):  # one position at a time, against the cached prefix
        one, _, _ = layer.forward_given_kv(given, t, hid[t:t + 1])
        assert np.array_equal(_bits(one), _bits(full[t:t + 1]))
    # the returned k and v are what the cache quantized
    requant = oracle.KVCache(shape, T)
    requant.store(0, k, v)
    for hd in range(shape.n_heads):
        for a, b in zip(own.export(hd, 0, T), requant.export(hd, 0, T)):
            assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
    # the given cache is read, never written
    for hd in range(shape.n_heads):
        for a, b in zip(own.export(hd, 0, T), given.export(hd, 0, T)):
            assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))


def _cache(k, v):
    kc, ks, kz = oracle.quantize_groupwise(k)
    vc, vs, vz = oracle.quantize_groupwise(v)
    T, d = k.shape
    return (kc.reshape(T, d // 2), ks.reshape(T, d // G), kz.reshape(T, d // G),
            vc.reshape(T, d // 2), vs.reshape(T, d // G), vz.reshape(T, d // G))


def _exact_values(vc, vs, vz):
    """Exact rationals zero + c * scale of every cached V element, [T][d]."""
    T = vc.shape[0]
    d = vc.shape[1] * 2
    out = []
    for t in range(T):
        row = []
        for i in range(d):
            c = (int(vc[t, i // 2]) >> (4 * (i & 1))) & 15
            row.append(Fraction(float(vz[t, i // G])) + c * Fraction(float(vs[t, i // G])))
        out.append(row)
    return out


def test_exact_v_single_position_is_the_value_rounded_once():
    rng = np.random.default_rng(23)
    q = rng.standard_normal(128).astype(np.float16)
    k = rng.standard_normal((1, 128)).astype(np.float16)
    v = rng.standard_normal((1, 128)).astype(np.float16)
    cache = _cache(k, v)
    exact = _exact_values(*cache[3:])[0]
    ref = np.array([float(x) for x in exact]).astype(np.float16)  # one rounding of each exact value
    with oracle.exact_v():
        out = oracle.attend(q, *cache)
    assert np.array_equal(_bits(out), _bits(ref))
    assert np.array_equal(_bits(oracle.attend(q, *cache)), _bits(ref))  # the rounded reading agrees here


def test_exact_v_identical_keys_give_the_exact_mean():
    """Identical keys weigh every position by exactly 1: the output is the exact rational mean
    of the exact values, rounded once (float() of a Fraction rounds correctly)."""
    rng = np.random.default_rng(24)
    T = 23
    q = rng.standard_normal(128).astype(np.float16)
    k = np.tile(rng.standard_normal((1, 128)).astype(np.float16), (T, 1))
    v = rng.standard_normal((T, 128)).astype(np.float16)
    cache = _cache(k, v)
    vals = _exact_values(*cache[3:])
    ref = np.array([float(sum(vals[t][i] for t in range(T)) / T) for i in range(128)]).astype(np.float16)
    with oracle.exact_v():
        out = oracle.attend(q, *cache)
    assert np.array_equal(_bits(out), _bits(ref))


def test_exact_v_on_grid_values_agree_with_the_rounded_reading():
    """V groups whose grid points zero + c * scale are all fp16 values: rounding them changes
    nothing, so both readings give identical bits on random queries and keys."""
    rng = np.random.default_rng(25)
    T, d = 40, 128
    c = rng.integers(0, 16, size=(T * d // G, G))
    c[:, 0], c[:, 1] = 0, 15
    s = 2.0 ** rng.integers(-8, -3, size=(T * d // G, 1))
    mn = -rng.integers(0, 64, size=(T * d // G, 1)) * s
    v = (mn + c * s).astype(np.float16).reshape(T, d)
    q = rng.standard_normal(d).astype(np.float16)
    k = rng.standard_normal((T, d)).astype(np.float16)
    cache = _cache(k, v)
    with oracle.exact_v():
        a = oracle.attend(q, *cache)
    assert np.array_equal(_bits(a), _bits(oracle.attend(q, *cache)))


def test_exact_v_differs_by_at_most_half_an_ulp_of_the_largest_value():
    rng = np.random.default_rng(26)
    T, d = 300, 128
    q = (rng.standard_normal(d) * 2).astype(np.float16)
    k = rng.standard_normal((T, d)).astype(np.float16)
    v = rng.standard_normal((T, d)).astype(np.float16)
    cache = _cache(k, v)
    rounded = oracle.attend(q, *cache).astype(np.float64)
    with oracle.exact_v():
        exact = oracle.attend(q, *cache).astype(np.float64)
    vmax = np.abs(oracle.dequantize_groupwise(cache[3].reshape(-1), cache[4].reshape(-1),
                                              cache[5].reshape(-1)).astype(np.float64)).max()
    half_ulp_v = np.spacing(np.float16(vmax)).astype(np.float64) / 2
    out_ulp = np.spacing(np.maximum(np.abs(rounded), np.abs(exact)).astype(np.float16)).astype(np.float64)
    assert (np.abs(rounded - exact) <= half_ulp_v + out_ulp).all()
    assert not np.array_equal(rounded, exact)  # on random data the readings do differ somewhere


# ---------------------------------------------------------------------------- fp32 accumulation

def test_fp32_accumulation_closed_form_cancellation():
    """Products 2^24, 1, -2^24 in that order: the fp32 running sum rounds 2^24 + 1 to 2^24 (a tie,
    to even) and ends at 0; the fp64 oracle keeps the 1."""
    a = np.zeros((1, 64), np.float16)
    w = np.zeros((1, 64), np.float16)
    a[0, :3] = [4096, 1, 4096]
    w[0, :3] = [4096, 1, -4096]
    assert float(oracle.linear_f16(a, w)[0, 0]) == 1.0
    with oracle.fp32_accumulation():
        assert float(oracle.linear_f16(a, w)[0, 0]) == 0.0
    assert float(oracle.linear_f16(a, w)[0, 0]) == 1.0  # the switch is restored


def test_fp32_accumulation_is_exact_where_every_partial_sum_is():
    """Small integers (every partial sum below 2^24) give identical bits with and without the switch,
    for a linear layer, a LayerNorm and an attention with identical keys."""
    rng = np.random.default_rng(27)
    a = rng.integers(-8, 9, size=(5, 256)).astype(np.float16)
    w = rng.integers(-8, 9, size=(64, 256)).astype(np.float16)
    g = np.ones(256, np.float16)
    b = np.zeros(256, np.float16)
    ref_lin, ref_ln = oracle.linear_f16(a, w), oracle.layernorm(a, g, b)
    k = np.tile(rng.integers(-3, 4, size=(1, 128)).astype(np.float16), (16, 1))
    v = rng.integers(-7, 8, size=(16, 128)).astype(np.float16)
    q = rng.integers(-3, 4, size=128).astype(np.float16)
    ref_att = oracle.attend(q, *_cache(k, v))
    with oracle.fp32_accumulation():
        assert np.array_equal(_bits(oracle.linear_f16(a, w)), _bits(ref_lin))
        assert np.array_equal(_bits(oracle.layernorm(a, g, b)), _bits(ref_ln))
        assert np.array_equal(_bits(oracle.attend(q, *_cache(k, v))), _bits(ref_att))


def _f32_sum(terms):
    """Running sum with the running value rounded to fp32 after every addition (terms float64)."""
    acc = np.float32(0.0)
    for t in terms:
        acc = np.float32(np.float64(acc) + np.float64(t))
    return np.float64(acc)


def test_fp32_accumulation_linear_matches_sequential_float32_sums():
    rng = np.random.default_rng(28)
    a = (rng.standard_normal((3, 512)) * 8).astype(np.float16)
    w = (rng.standard_normal((16, 512)) * 8).astype(np.float16)
    # products +2^24 first and -2^24 last: while the running sum sits near 2^24 fp32 keeps only
    # even integers, so the two settings differ visibly
    a[:, 0], a[:, -1] = 4096, 4096
    w[:, 0], w[:, -1] = 4096, -4096
    bias = rng.standard_normal(16).astype(np.float16)
    res = rng.standard_normal((3, 16)).astype(np.float16)
    with oracle.fp32_accumulation():
        got = oracle.linear_f16(a, w, bias=bias, residual=res)
    ref = np.empty((3, 16))
    for m in range(3):
        for o in range(16):
            terms = list(a[m].astype(np.float64) * w[o].astype(np.float64)) + [float(bias[o]), float(res[m, o])]
            ref[m, o] = _f32_sum(terms)
    assert np.array_equal(_bits(got), _bits(ref.astype(np.float16)))
    assert not np.array_equal(_bits(got), _bits(oracle.linear_f16(a, w, bias=bias, residual=res)))


def test_fp32_accumulation_layernorm_matches_sequential_float32_sums():
    rng = np.random.default_rng(29)
    h = 1024
    x = (rng.standard_normal((4, h)) * 3 + 200).astype(np.float16)  # a large mean: the sums lose bits
    g = (1 + rng.standard_normal(h) * 0.5).astype(np.float16)
    b = (rng.standard_normal(h) * 0.5).astype(np.float16)
    with oracle.fp32_accumulation():
        got = oracle.layernorm(x, g, b)
    ref = np.empty((4, h))
    for r in range(4):
        xr = x[r].astype(np.float64)
        mu = _f32_sum(xr) / h
        var = _f32_sum((xr - mu) ** 2) / h
        ref[r] = (xr - mu) / np.sqrt(var + 1e-5) * g.astype(np.float64) + b.astype(np.float64)
    assert np.array_equal(_bits(got), _bits(ref.astype(np.float16)))


def test_fp32_accumulation_attention_matches_sequential_float32_sums():
    rng = np.random.default_rng(30)
    T, d = 150, 128
    q = (rng.standard_normal(d) * 2).astype(np.float16)
    k = rng.standard_normal((T, d)).astype(np.float16)
    v = (rng.standard_normal((T, d)) * 4).astype(np.float16)
    cache = _cache(k, v)
    with oracle.fp32_accumulation():
        got = oracle.attend(q, *cache).astype(np.float64)
    kh = oracle.dequantize_groupwise(cache[0].reshape(-1), cache[1].reshape(-1),
                                     cache[2].reshape(-1)).astype(np.float64).reshape(T, d)
    vh = oracle.dequantize_groupwise(cache[3].reshape(-1), cache[4].reshape(-1),
                                     cache[5].reshape(-1)).astype(np.float64).reshape(T, d)
    qd = q.astype(np.float64)
    score = np.array([_f32_sum(qd * kh[t]) / np.sqrt(d) for t in range(T)])
    wgt = np.exp(score - score.max())
    den = _f32_sum(wgt)
    ref = np.array([_f32_sum(wgt * vh[:, i]) / den for i in range(d)]).astype(np.float16).astype(np.float64)
    ulp = np.spacing(np.maximum(np.abs(got), np.abs(ref)).astype(np.float16)).astype(np.float64)
    assert (np.abs(got - ref) <= ulp).all()  # numpy's exp and the C library's may differ in the last bit
    assert (got == ref).mean() > 0.99
