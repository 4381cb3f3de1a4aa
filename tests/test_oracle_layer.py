"""Pins of the oracle's layer arithmetic against float64 library routines.

LayerNorm against torch.nn.functional.layer_norm, linear layers against
matrix products, attention against closed-form special cases and a brute-force
float64 softmax attention, and a whole tiny single-head decoder layer against
a float64 PyTorch reference assembled from the same dequantized tensors.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.test_oracle_quant import _brute_force

G = 64


def _f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def _ulps(a, b):
    """Distance in fp16 ulps between two fp16 arrays of the same sign pattern."""
    a = np.asarray(a, dtype=np.float16).astype(np.float64)
    b = np.asarray(b, dtype=np.float16).astype(np.float64)
    sp = np.spacing(np.maximum(np.abs(a), np.abs(b)).astype(np.float16)).astype(np.float64)
    return np.abs(a - b) / sp


def _dequant_np(x16):
    """Independent numpy quantize+dequantize (brute-force codes) of groups of 64."""
    c, s, mn = _brute_force(np.ascontiguousarray(x16).reshape(-1))
    s = np.repeat(s.astype(np.float64), G)
    mn = np.repeat(mn.astype(np.float64) + 0.0, G)
    return _f16(mn + c * s).reshape(np.shape(x16))


def test_layernorm_matches_torch():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((37, 768)) * 0.5 + 0.1).astype(np.float16)
    g = (1 + rng.standard_normal(768) * 0.02).astype(np.float16)
    b = (rng.standard_normal(768) * 0.02).astype(np.float16)
    ours = oracle.layernorm(x, g, b)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x.astype(np.float64)), (768,),
                                         torch.from_numpy(g.astype(np.float64)),
                                         torch.from_numpy(b.astype(np.float64)), eps=1e-5).numpy()
    assert _ulps(ours, _f16(ref)).max() <= 1
    assert (ours == _f16(ref)).mean() > 0.999


def test_linear_on_grid_weights_equals_fp16_matmul():
    """With on-grid weights dequantization is exact, so the int4 linear is an fp16 matmul."""
    rng = np.random.default_rng(6)
    n_out, k = 96, 256
    c = rng.integers(0, 16, size=(n_out * k // G, G))
    c[:, 0], c[:, 1] = 0, 15   # every group spans the full grid
    s = 2.0 ** rng.integers(-10, -6, size=(n_out * k // G, 1))
    mn = -rng.integers(0, 64, size=(n_out * k // G, 1)) * s
    w = _f16(mn + c * s).reshape(n_out, k)
    a = (rng.standard_normal((13, k))).astype(np.float16)
    bias = (rng.standard_normal(n_out) * 0.1).astype(np.float16)
    res = (rng.standard_normal((13, n_out))).astype(np.float16)
    codes, scale, zero = oracle.quantize_groupwise(w)
    assert np.array_equal(oracle.dequantize_groupwise(codes, scale, zero).reshape(n_out, k), w)
    ours = oracle.linear_w4(a, codes, scale, zero, n_out, bias=bias, residual=res)
    ref = torch.matmul(torch.from_numpy(a.astype(np.float64)), torch.from_numpy(w.astype(np.float64)).T).numpy()
    ref = ref + bias.astype(np.float64) + res.astype(np.float64)
    assert _ulps(ours, _f16(ref)).max() <= 1
    relu = oracle.linear_w4(a, codes, scale, zero, n_out, bias=bias, relu=True)
    ref_relu = np.maximum(torch.matmul(torch.from_numpy(a.astype(np.float64)),
                                       torch.from_numpy(w.astype(np.float64)).T).numpy() + bias.astype(np.float64), 0)
    assert _ulps(relu, _f16(ref_relu)).max() <= 1
    assert (relu.astype(np.float64) >= 0).all()


def test_linear_w4_matches_matmul_of_dequantized_weights():
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((80, 192)) * 0.02).astype(np.float16)
    a = rng.standard_normal((9, 192)).astype(np.float16)
    codes, scale, zero = oracle.quantize_groupwise(w)
    ours = oracle.linear_w4(a, codes, scale, zero, 80)
    wh = _dequant_np(w)
    ref = a.astype(np.float64) @ wh.astype(np.float64).T
    assert _ulps(ours, _f16(ref)).max() <= 1
    f16 = oracle.linear_f16(a, w)
    assert _ulps(f16, _f16(a.astype(np.float64) @ w.astype(np.float64).T)).max() <= 1


def _cache_from(k, v):
    kc, ks, kz = oracle.quantize_groupwise(k)
    vc, vs, vz = oracle.quantize_groupwise(v)
    T, d = k.shape
    return (kc.reshape(T, d // 2), ks.reshape(T, d // G), kz.reshape(T, d // G),
            vc.reshape(T, d // 2), vs.reshape(T, d // G), vz.reshape(T, d // G))


def test_attention_context_one_returns_value():
    rng = np.random.default_rng(8)
    q = rng.standard_normal(128).astype(np.float16)
    k = rng.standard_normal((1, 128)).astype(np.float16)
    v = rng.standard_normal((1, 128)).astype(np.float16)
    out = oracle.attend(q, *_cache_from(k, v))
    assert np.array_equal(out, _dequant_np(v).reshape(-1))


def test_attention_identical_keys_average_values():
    rng = np.random.default_rng(9)
    T = 37
    q = rng.standard_normal(128).astype(np.float16)
    k = np.tile(rng.standard_normal((1, 128)).astype(np.float16), (T, 1))
    v = rng.standard_normal((T, 128)).astype(np.float16)
    out = oracle.attend(q, *_cache_from(k, v))
    ref = _dequant_np(v).astype(np.float64).mean(axis=0)
    assert _ulps(out, _f16(ref)).max() <= 1


def test_attention_matches_float64_softmax():
    rng = np.random.default_rng(10)
    T, d = 200, 128
    q = rng.standard_normal(d).astype(np.float16)
    k = rng.standard_normal((T, d)).astype(np.float16)
    v = rng.standard_normal((T, d)).astype(np.float16)
    out = oracle.attend(q, *_cache_from(k, v))
    kh, vh = _dequant_np(k).astype(np.float64), _dequant_np(v).astype(np.float64)
    p = torch.softmax(torch.from_numpy(kh @ q.astype(np.float64) / np.sqrt(d)), dim=0).numpy()
    assert _ulps(out, _f16(p @ vh)).max() <= 1


def _tiny_shape():
    return synth.ModelShape(n_layers=1, hidden=64, n_heads=1, head_dim=64, ffn=256, vocab=300, max_pos=64)


def _torch_reference_layer(tw, hid, n_pos):
    """float64 single-head pre-LN layer with the oracle's rounding points, built from
    torch layer_norm/matmul/softmax and brute-force quantized K/V."""
    def ln(x, g, b):
        return _f16(torch.nn.functional.layer_norm(torch.from_numpy(x.astype(np.float64)), (x.shape[-1],),
                                                   torch.from_numpy(g.astype(np.float64)),
                                                   torch.from_numpy(b.astype(np.float64)), eps=1e-5).numpy())

    def lin(x, name, relu=False, res=None):
        w = _dequant_np(tw[name + "_w"]).astype(np.float64)
        y = x.astype(np.float64) @ w.T + tw[name + "_b"].astype(np.float64)
        if res is not None:
            y = y + res.astype(np.float64)
        if relu:
            y = np.maximum(y, 0)
        return _f16(y)

    a = ln(hid, tw["ln1_g"], tw["ln1_b"])
    q, k, v = lin(a, "q"), lin(a, "k"), lin(a, "v")
    kh, vh = _dequant_np(k).astype(np.float64), _dequant_np(v).astype(np.float64)
    scores = (q.astype(np.float64) @ kh.T) / np.sqrt(64)
    mask = np.tril(np.ones((n_pos, n_pos), dtype=bool))
    scores = np.where(mask, scores, -np.inf)
    p = torch.softmax(torch.from_numpy(scores), dim=1).numpy()
    o = _f16(p @ vh)
    h1 = lin(o, "o", res=hid)
    b2 = ln(h1, tw["ln2_g"], tw["ln2_b"])
    u = lin(b2, "fc1", relu=True)
    return lin(u, "fc2", res=h1)


def test_tiny_single_head_layer_matches_torch_reference():
    shape = _tiny_shape()
    tw = synth.layer_weights(shape, 0, variant="full")
    # larger weights than N(0, 0.02) so that attention is far from uniform
    for n in ("q_w", "k_w"):
        tw[n] = (tw[n].astype(np.float64) * 25).astype(np.float16)
    rng = np.random.default_rng(11)
    T = 12
    hid = rng.standard_normal((T, 64)).astype(np.float16)
    layer = oracle.Layer(shape, tw)
    cache = oracle.KVCache(shape, T)
    ours = layer.forward(cache, 0, hid)
    ref = _torch_reference_layer(tw, hid, T)
    assert _ulps(ours, ref).max() <= 2
    assert (ours == ref).mean() > 0.99


def test_prefill_equals_incremental_positions():
    """Quantize-then-attend: one call over T positions equals T one-position calls, bitwise."""
    shape = synth.ModelShape(n_layers=1, hidden=128, n_heads=2, head_dim=64, ffn=256, vocab=300, max_pos=64)
    tw = synth.layer_weights(shape, 0, variant="full")
    rng = np.random.default_rng(12)
    T = 9
    hid = rng.standard_normal((T, 128)).astype(np.float16)
    layer = oracle.Layer(shape, tw)
    c1, c2 = oracle.KVCache(shape, T), oracle.KVCache(shape, T)
    full = layer.forward(c1, 0, hid)
    inc = np.concatenate([layer.forward(c2, t, hid[t:t + 1]) for t in range(T)])
    assert np.array_equal(full.view(np.uint16), inc.view(np.uint16))
    for hd in range(2):
        for a, b in zip(c1.export(hd, 0, T), c2.export(hd, 0, T)):
            assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))


def test_embed_and_head():
    shape = _tiny_shape()
    glob = synth.global_weights(shape, variant="full")
    ids = np.array([0, 5, 299], dtype=np.int32)
    pos = np.array([0, 3, 63], dtype=np.int32)
    e = oracle.embed(shape, glob["tok_emb"], glob["pos_emb"], ids, pos)
    ref = _f16(glob["tok_emb"][ids].astype(np.float64) + glob["pos_emb"][pos + 2].astype(np.float64))
    assert np.array_equal(e.view(np.uint16), ref.view(np.uint16))
    logits, nxt = oracle.head(shape, glob["lnf_g"], glob["lnf_b"], glob["tok_emb"], e)
    z = oracle.layernorm(e, glob["lnf_g"], glob["lnf_b"])
    ref_logits = _f16(z.astype(np.float64) @ glob["tok_emb"].astype(np.float64).T)
    assert _ulps(logits, ref_logits).max() <= 1
    assert np.array_equal(nxt, np.argmax(logits.astype(np.float64), axis=1))
    with pytest.raises(ValueError):
        oracle.embed(shape, glob["tok_emb"], glob["pos_emb"], np.array([300], np.int32), np.array([0], np.int32))


def test_argmax_ties_pick_lowest_index():
    shape = synth.ModelShape(n_layers=1, hidden=64, n_heads=1, head_dim=64, ffn=256, vocab=8, max_pos=8)
    emb = np.zeros((8, 64), dtype=np.float16)
    emb[3, 0] = emb[5, 0] = 1.0   # rows 3 and 5 give the same, largest logit
    hid = np.zeros((1, 64), dtype=np.float16)
    hid[0, 0] = 1.0
    g = np.ones(64, dtype=np.float16)
    b = np.zeros(64, dtype=np.float16)
    logits, nxt = oracle.head(shape, g, b, emb, hid)
    assert logits[0, 3] == logits[0, 5] and logits[0, 3] == logits[0].max()
    assert nxt[0] == 3
