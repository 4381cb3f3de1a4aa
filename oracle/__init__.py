"""CPU oracle for block-scheduled int4 decode (ctypes front end of ``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product package. It shares no code
with the GPU library; the two meet only in the seeded inputs from ``synth``.

Arrays are numpy; fp16 tensors are passed as ``np.float16`` (or their
``uint16`` bit views). Every function here is argument marshalling around the
plain C implementation, except the few helpers marked as plain Python.
"""
from __future__ import annotations

import ctypes
import functools
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

SCHED_ROW_BY_ROW = 0
SCHED_ZIGZAG = 1
SCHED_ZIGZAG_ALTERNATE = 2
MATRICES = ("q", "k", "v", "o", "fc1", "fc2")


def build() -> str:
    """Compile the oracle (gcc, -O2 -ffp-contract=off, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-o", _SO + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)
    return _SO


class Dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int), ("n_heads", ctypes.c_int), ("head_dim", ctypes.c_int),
                ("ffn", ctypes.c_int), ("vocab", ctypes.c_int), ("max_pos", ctypes.c_int),
                ("group", ctypes.c_int)]


@functools.lru_cache(maxsize=None)
def _lib() -> ctypes.CDLL:
    if not os.path.exists(_SO):
        build()
    L = ctypes.CDLL(_SO)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sig = {
        "o_half_to_double": ([ctypes.c_uint16], ctypes.c_double),
        "o_double_to_half": ([ctypes.c_double], ctypes.c_uint16),
        "o_half_to_double_array": ([vp, vp, i64], None),
        "o_double_to_half_array": ([vp, vp, i64], None),
        "o_quantize_groupwise": ([vp, i64, i32, vp, vp, vp], i32),
        "o_dequantize_groupwise": ([vp, vp, vp, i64, i32, vp], i32),
        "o_layernorm": ([vp, i64, i32, vp, vp, vp], None),
        "o_linear_w4": ([vp, i64, i32, i32, vp, vp, vp, i32, vp, vp, i32, vp], i32),
        "o_linear_f16": ([vp, i64, i32, i32, vp, vp, vp, i32, vp], i32),
        "o_attend": ([i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp], None),
        "o_layer_new": ([vp, vp, i32], vp),
        "o_layer_free": ([vp], None),
        "o_layer_export": ([vp, i32, vp, vp, vp], i32),
        "o_kv_new": ([vp, i32], vp),
        "o_kv_free": ([vp], None),
        "o_kv_store": ([vp, i32, i32, vp, vp], i32),
        "o_kv_export": ([vp, i32, i32, i32, vp, vp, vp, vp, vp, vp], i32),
        "o_layer_forward": ([vp, vp, i32, i32, vp], i32),
        "o_embed": ([vp, vp, vp, vp, vp, i32, vp], i32),
        "o_head": ([vp, vp, vp, vp, vp, i32, vp, vp], None),
        "o_generate": ([vp, i32, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, i32, vp, vp, vp, vp], i32),
        "o_set_fp32_accumulation": ([i32], None),
        "o_set_exact_v": ([i32], None),
        "o_kv_load": ([vp, i32, i32, i32, vp, vp, vp, vp, vp, vp], i32),
        "o_layer_forward_given_kv": ([vp, vp, i32, i32, vp, vp, vp], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _h(a) -> np.ndarray:
    """fp16 bit pattern view (uint16) of an fp16 array."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    assert a.dtype == np.uint16
    return a


def dims_of(shape, group: int = 64) -> Dims:
    return Dims(shape.hidden, shape.n_heads, shape.head_dim, shape.ffn, shape.vocab, shape.max_pos, group)


class fp32_accumulation:
    """Context manager: run the oracle with every running sum rounded to fp32 (calibration
    of how far a correct fp32-accumulating implementation drifts from the fp64 oracle)."""

    def __enter__(self):
        _lib().o_set_fp32_accumulation(1)
        return self

    def __exit__(self, *exc):
        _lib().o_set_fp32_accumulation(0)
        return False


class exact_v:
    """Context manager: attention reads each cached V element as the exact real zero + c * scale
    instead of its fp16 rounding (the same attention with that one rounding left out)."""

    def __enter__(self):
        _lib().o_set_exact_v(1)
        return self

    def __exit__(self, *exc):
        _lib().o_set_exact_v(0)
        return False


# ---------------------------------------------------------------------------- fp16

def half_to_double(h: np.ndarray) -> np.ndarray:
    h = _h(h)
    out = np.empty(h.shape, dtype=np.float64)
    _lib().o_half_to_double_array(_p(h), _p(out), h.size)
    return out


def double_to_half(x: np.ndarray) -> np.ndarray:
    """fp16 bit patterns (uint16) of x rounded to nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _lib().o_double_to_half_array(_p(x), _p(out), x.size)
    return out


# ---------------------------------------------------------------------------- quantizer

def quantize_groupwise(x, group: int = 64):
    """codes u8 [n/2] (low nibble = even element), scale and zero fp16 [n/group]."""
    x = _h(x).reshape(-1)
    n = x.size
    codes = np.empty(n // 2, dtype=np.uint8)
    scale = np.empty(n // group, dtype=np.uint16)
    zero = np.empty(n // group, dtype=np.uint16)
    rc = _lib().o_quantize_groupwise(_p(x), n, group, _p(codes), _p(scale), _p(zero))
    if rc != 0:
        raise ValueError(f"oracle quantize_groupwise failed ({rc})")
    return codes, scale.view(np.float16), zero.view(np.float16)


def dequantize_groupwise(codes, scale, zero, group: int = 64) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1)
    scale, zero = _h(scale).reshape(-1), _h(zero).reshape(-1)
    n = codes.size * 2
    out = np.empty(n, dtype=np.uint16)
    rc = _lib().o_dequantize_groupwise(_p(codes), _p(scale), _p(zero), n, group, _p(out))
    if rc != 0:
        raise ValueError(f"oracle dequantize_groupwise failed ({rc})")
    return out.view(np.float16)


# ---------------------------------------------------------------------------- layer pieces

def layernorm(x, gain, shift) -> np.ndarray:
    x = _h(x)
    h = x.shape[-1]
    rows = x.size // h
    y = np.empty(x.shape, dtype=np.uint16)
    _lib().o_layernorm(_p(x), rows, h, _p(_h(gain)), _p(_h(shift)), _p(y))
    return y.view(np.float16)


def linear_w4(a, codes, scale, zero, out_features: int, bias=None, residual=None, relu=False,
              group: int = 64) -> np.ndarray:
    a = _h(a)
    rows, k = a.shape
    y = np.empty((rows, out_features), dtype=np.uint16)
    rc = _lib().o_linear_w4(_p(a), rows, k, out_features, _p(np.ascontiguousarray(codes, dtype=np.uint8)),
                            _p(_h(scale)), _p(_h(zero)), group, _p(_h(bias)) if bias is not None else None,
                            _p(_h(residual)) if residual is not None else None, int(relu), _p(y))
    if rc != 0:
        raise ValueError(f"oracle linear_w4 failed ({rc})")
    return y.view(np.float16)


def linear_f16(a, w, bias=None, residual=None, relu=False) -> np.ndarray:
    a, w = _h(a), _h(w)
    rows, k = a.shape
    n = w.shape[0]
    y = np.empty((rows, n), dtype=np.uint16)
    rc = _lib().o_linear_f16(_p(a), rows, k, n, _p(w), _p(_h(bias)) if bias is not None else None,
                             _p(_h(residual)) if residual is not None else None, int(relu), _p(y))
    if rc != 0:
        raise ValueError(f"oracle linear_f16 failed ({rc})")
    return y.view(np.float16)


def attend(q, kc, ks, kz, vc, vs, vz, group: int = 64) -> np.ndarray:
    """One query of one head over T cached int4 positions: codes [T][d/2], params [T][d/group]."""
    q = _h(q).reshape(-1)
    d = q.size
    T = int(np.asarray(kc).shape[0])
    out = np.empty(d, dtype=np.uint16)
    arr = [np.ascontiguousarray(kc, dtype=np.uint8), _h(ks), _h(kz), np.ascontiguousarray(vc, dtype=np.uint8),
           _h(vs), _h(vz)]
    _lib().o_attend(d, group, T, _p(q), *[_p(x) for x in arr], _p(out))
    return out.view(np.float16)


def embed(shape, tok_emb, pos_emb, ids, pos) -> np.ndarray:
    dm = dims_of(shape)
    ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
    pos = np.ascontiguousarray(pos, dtype=np.int32).reshape(-1)
    out = np.empty((ids.size, shape.hidden), dtype=np.uint16)
    rc = _lib().o_embed(ctypes.byref(dm), _p(_h(tok_emb)), _p(_h(pos_emb)), _p(ids), _p(pos), ids.size, _p(out))
    if rc != 0:
        raise ValueError("oracle embed: id or position out of range")
    return out.view(np.float16)


def head(shape, lnf_g, lnf_b, tok_emb, hidden):
    """(logits fp16 [n][V], greedy ids [n])."""
    dm = dims_of(shape)
    hidden = _h(hidden).reshape(-1, shape.hidden)
    n = hidden.shape[0]
    logits = np.empty((n, shape.vocab), dtype=np.uint16)
    nxt = np.empty(n, dtype=np.int32)
    _lib().o_head(ctypes.byref(dm), _p(_h(lnf_g)), _p(_h(lnf_b)), _p(_h(tok_emb)), _p(hidden), n, _p(logits),
                  _p(nxt))
    return logits.view(np.float16), nxt


# ---------------------------------------------------------------------------- layers and cache

class Layer:
    """One decoder layer built from its 16 fp16 tensors (dict keyed by synth.LAYER_TENSORS).

    int4_weights=False keeps the six matrices in fp16 (the host-streamed weight tier)."""

    ORDER = ("ln1_g", "ln1_b", "q_w", "q_b", "k_w", "k_b", "v_w", "v_b",
             "o_w", "o_b", "ln2_g", "ln2_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b")

    def __init__(self, shape, tensors: dict, group: int = 64, int4_weights: bool = True):
        self.shape = shape
        self.dims = dims_of(shape, group)
        keep = [_h(tensors[n]) for n in self.ORDER]
        ptrs = (ctypes.c_void_p * 16)(*[_p(t) for t in keep])
        self._ptr = _lib().o_layer_new(ctypes.byref(self.dims), ptrs, int(int4_weights))
        if not self._ptr:
            raise ValueError("oracle layer construction failed")

    def export(self, which: str):
        """Canonical (codes, scale, zero) of matrix ``which`` in q, k, v, o, fc1, fc2."""
        m = MATRICES.index(which)
        h, f = self.shape.hidden, self.shape.ffn
        rows, cols = {"fc1": (f, h), "fc2": (h, f)}.get(which, (h, h))
        n = rows * cols
        codes = np.empty(n // 2, dtype=np.uint8)
        scale = np.empty(n // self.dims.group, dtype=np.uint16)
        zero = np.empty(n // self.dims.group, dtype=np.uint16)
        _lib().o_layer_export(self._ptr, m, _p(codes), _p(scale), _p(zero))
        return codes, scale.view(np.float16), zero.view(np.float16)

    def forward(self, cache: "KVCache", pos0: int, hidden: np.ndarray) -> np.ndarray:
        hid = np.array(_h(hidden), dtype=np.uint16, copy=True).reshape(-1, self.shape.hidden)
        rc = _lib().o_layer_forward(self._ptr, cache._ptr, pos0, hid.shape[0], _p(hid))
        if rc != 0:
            raise ValueError(f"oracle layer forward failed ({rc})")
        return hid.view(np.float16)

    def forward_given_kv(self, cache: "KVCache", pos0: int, hidden: np.ndarray):
        """The layer at positions pos0.. against the cache as given (positions 0..pos0+n-1
        already loaded): (hidden out fp16 [n][h], the layer's own k and v fp16 [n][h])."""
        hid = np.array(_h(hidden), dtype=np.uint16, copy=True).reshape(-1, self.shape.hidden)
        k = np.empty_like(hid)
        v = np.empty_like(hid)
        rc = _lib().o_layer_forward_given_kv(self._ptr, cache._ptr, pos0, hid.shape[0], _p(hid), _p(k), _p(v))
        if rc != 0:
            raise ValueError(f"oracle layer forward (given cache) failed ({rc})")
        return hid.view(np.float16), k.view(np.float16), v.view(np.float16)

    def close(self):
        if self._ptr:
            _lib().o_layer_free(self._ptr)
            self._ptr = None

    def __del__(self):
        self.close()


class KVCache:
    """int4 KV cache of one layer for one sequence, positions 0..cap-1."""

    def __init__(self, shape, cap: int, group: int = 64):
        self.shape = shape
        self.cap = cap
        self.dims = dims_of(shape, group)
        self._ptr = _lib().o_kv_new(ctypes.byref(self.dims), cap)

    def store(self, pos0: int, k, v):
        k = _h(k).reshape(-1, self.shape.hidden)
        v = _h(v).reshape(-1, self.shape.hidden)
        rc = _lib().o_kv_store(self._ptr, pos0, k.shape[0], _p(k), _p(v))
        if rc != 0:
            raise ValueError(f"oracle kv store failed ({rc})")

    def export(self, head: int, t0: int, t1: int):
        d, G = self.shape.head_dim, self.dims.group
        n = t1 - t0
        kc = np.empty((n, d // 2), np.uint8); vc = np.empty((n, d // 2), np.uint8)
        ks, kz, vs, vz = (np.empty((n, d // G), np.uint16) for _ in range(4))
        rc = _lib().o_kv_export(self._ptr, head, t0, t1, _p(kc), _p(ks), _p(kz), _p(vc), _p(vs), _p(vz))
        if rc != 0:
            raise ValueError("oracle kv export: bad range")
        return kc, ks.view(np.float16), kz.view(np.float16), vc, vs.view(np.float16), vz.view(np.float16)

    def load(self, head: int, t0: int, kc, ks, kz, vc, vs, vz):
        """Store positions t0.. of one head from the canonical format (inverse of export)."""
        kc = np.ascontiguousarray(kc, dtype=np.uint8)
        vc = np.ascontiguousarray(vc, dtype=np.uint8)
        n = kc.shape[0]
        arr = [_h(np.ascontiguousarray(x)) for x in (ks, kz, vs, vz)]
        rc = _lib().o_kv_load(self._ptr, head, t0, t0 + n, _p(kc), _p(arr[0]), _p(arr[1]), _p(vc), _p(arr[2]),
                              _p(arr[3]))
        if rc != 0:
            raise ValueError("oracle kv load: bad range")

    def close(self):
        if self._ptr:
            _lib().o_kv_free(self._ptr)
            self._ptr = None

    def __del__(self):
        self.close()


def generate(shape, layers, glob: dict, prompts, gen_len: int, batches_per_block: int,
             schedule: int = SCHED_ZIGZAG, forced=None, want_logits: bool = True):
    """Greedy generation; returns (tokens [n][g], logits [g][n][V] or None, layer loads)."""
    dm = dims_of(shape, layers[0].dims.group)
    prompts = np.ascontiguousarray(prompts, dtype=np.int32)
    n, s = prompts.shape
    g = gen_len
    lp = (ctypes.c_void_p * len(layers))(*[l._ptr for l in layers])
    tokens = np.empty((n, g), dtype=np.int32)
    logits = np.empty((g, n, shape.vocab), dtype=np.uint16) if want_logits else None
    fz = np.ascontiguousarray(forced, dtype=np.int32) if forced is not None else None
    loads = ctypes.c_int64(0)
    rc = _lib().o_generate(ctypes.byref(dm), len(layers), lp, _p(_h(glob["tok_emb"])), _p(_h(glob["pos_emb"])),
                           _p(_h(glob["lnf_g"])), _p(_h(glob["lnf_b"])), n, batches_per_block, s, g,
                           _p(prompts), schedule, _p(fz), _p(tokens), _p(logits), ctypes.byref(loads))
    if rc != 0:
        raise ValueError(f"oracle generate failed ({rc})")
    return tokens, (logits.view(np.float16) if logits is not None else None), loads.value


def teacher_forced_logits(shape, layer_source, glob: dict, ids: np.ndarray, first: int,
                          group: int = 64, int4_weights: bool = True, progress=None):
    """Logits of one sequence at positions first..T-1 given all its T input ids.

    Runs the whole sequence through one layer at a time (``layer_source(l)``
    returns that layer's tensors), so only one layer's weights are held; by the
    quantize-then-attend construction this equals prefill of ids[:first+1]
    followed by teacher-forced decode steps. Returns (logits fp16 [T-first][V],
    greedy ids)."""
    ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
    T = ids.size
    hid = embed(shape, glob["tok_emb"], glob["pos_emb"], ids, np.arange(T, dtype=np.int32))
    for l in range(shape.n_layers):
        layer = Layer(shape, layer_source(l), group, int4_weights)
        cache = KVCache(shape, T, group)
        hid = layer.forward(cache, 0, hid)
        layer.close()
        cache.close()
        if progress:
            progress(l)
    return head(shape, glob["lnf_g"], glob["lnf_b"], glob["tok_emb"], hid[first:])
