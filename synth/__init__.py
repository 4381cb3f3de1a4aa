"""Seeded synthetic workloads for the block-scheduled int4 decode path.

This package is the one piece shared by the CPU oracle's tests and the GPU
path's tests and bench: it draws inputs, and holds none of the method's
arithmetic (no quantizer, no layer math, no fp16 rounding of results).

* Random numbers are SplitMix64 outputs addressed by (seed, tensor id, index)
  (see ``synth.c``), so a tensor or any slice of it is reproducible alone.
* Normal fp16 values use inverse-transform sampling on a 65536-quantile grid:
  the top 16 bits of a draw index a table of fp16(mu + sigma * Phi^-1(p)).
  Tails are cut at |z| = 4.32 (probability 1.5e-5 per draw).
* Token ids are uniform over [0, vocab) by multiply-shift.

Workload shapes follow the OPT family that the FlexGen pages run (OPT-125m ...
OPT-175B; FlexGen guide, "The Problem"; FlexLLMGen page, "What it does").
Seeds: weights 0, prompt ids 1, isolated-attention tensors 2, its per-step new
K/V and query 3 + step.
"""
from __future__ import annotations

import ctypes
import dataclasses
import functools
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_SO = os.path.join(_HERE, "libsynth.so")

SEED_WEIGHTS = 0
SEED_PROMPTS = 1
SEED_ATTN = 2


def build() -> str:
    """Compile ``libsynth.so`` with gcc (OpenMP) and return its path."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", _SO + ".tmp", _SRC]
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)
    return _SO


@functools.lru_cache(maxsize=None)
def _lib() -> ctypes.CDLL:
    if not os.path.exists(_SO):
        build()
    lib = ctypes.CDLL(_SO)
    u64, i64, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
    lib.synth_draw.argtypes = [u64, u64, u64]
    lib.synth_draw.restype = u64
    lib.synth_table16.argtypes = [u64, u64, vp, vp, i64, i64]
    lib.synth_table16.restype = None
    lib.synth_uniform_ids.argtypes = [u64, u64, vp, i64, i64, ctypes.c_uint32]
    lib.synth_uniform_ids.restype = None
    lib.synth_fill16.argtypes = [vp, i64, ctypes.c_uint16]
    lib.synth_fill16.restype = None
    return lib


def draw(seed: int, tensor: int, index: int) -> int:
    """Raw 64-bit draw ``index`` of stream (seed, tensor)."""
    return int(_lib().synth_draw(seed, tensor, index))


@functools.lru_cache(maxsize=None)
def normal_table(mu: float, sigma: float) -> np.ndarray:
    """fp16 bit patterns of mu + sigma * Phi^-1((j + 0.5) / 65536), j = 0..65535."""
    from scipy.special import ndtri

    p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
    v = mu + sigma * ndtri(p)
    t = np.ascontiguousarray(v.astype(np.float16).view(np.uint16))
    t.setflags(write=False)
    return t


def normal_f16(seed: int, tensor: int, shape, mu: float = 0.0, sigma: float = 0.02,
               offset: int = 0, out: np.ndarray | None = None) -> np.ndarray:
    """Draw ``prod(shape)`` fp16 values ~ N(mu, sigma) from stream (seed, tensor).

    ``offset`` selects the first element index, so slices of a large tensor can
    be drawn alone. ``out`` may be any C-contiguous 2-byte buffer (e.g. a numpy
    view of pinned host memory)."""
    shape = tuple(shape) if not isinstance(shape, int) else (shape,)
    n = int(np.prod(shape, dtype=np.int64))
    if out is None:
        out = np.empty(shape, dtype=np.float16)
    assert out.flags["C_CONTIGUOUS"] and out.itemsize == 2 and out.size == n
    tab = normal_table(float(mu), float(sigma))
    _lib().synth_table16(seed, tensor, tab.ctypes.data, out.ctypes.data, n, offset)
    return out


def constant_f16(shape, value: float, out: np.ndarray | None = None) -> np.ndarray:
    shape = tuple(shape) if not isinstance(shape, int) else (shape,)
    if out is None:
        out = np.empty(shape, dtype=np.float16)
    bits = int(np.array([value], dtype=np.float16).view(np.uint16)[0])
    _lib().synth_fill16(out.ctypes.data, out.size, bits)
    return out


def uniform_ids(seed: int, tensor: int, shape, vocab: int, offset: int = 0) -> np.ndarray:
    """int32 ids uniform over [0, vocab) from stream (seed, tensor)."""
    shape = tuple(shape) if not isinstance(shape, int) else (shape,)
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(shape, dtype=np.int32)
    _lib().synth_uniform_ids(seed, tensor, out.ctypes.data, n, offset, vocab)
    return out


# --------------------------------------------------------------------------
# Workload shapes
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class ModelShape:
    n_layers: int
    hidden: int
    n_heads: int
    head_dim: int
    ffn: int
    vocab: int = 50272
    max_pos: int = 2048

    def replace(self, **kw) -> "ModelShape":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: ModelShape
    gpu_batch: int
    batches_per_block: int
    prompt_len: int
    gen_len: int
    weight_tier: int = 0   # 0: int4 weights resident in HBM; 1: fp16 / 2: int4 weights streamed from pinned host memory

    @property
    def rows(self) -> int:
        return self.gpu_batch * self.batches_per_block

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


OPT_125M = ModelShape(12, 768, 12, 64, 3072)
OPT_6_7B = ModelShape(32, 4096, 32, 128, 16384)
OPT_30B = ModelShape(48, 7168, 56, 128, 28672)
OPT_175B = ModelShape(96, 12288, 96, 128, 49152)

WORKLOADS = {
    "opt-125m": Workload("opt-125m", OPT_125M, 4, 2, 32, 8),
    "opt-6.7b": Workload("opt-6.7b", OPT_6_7B, 64, 4, 512, 32),
    "opt-30b": Workload("opt-30b", OPT_30B, 64, 8, 512, 32),
    "opt-175b": Workload("opt-175b", OPT_175B, 32, 8, 512, 32, weight_tier=1),
    "opt-175b-int4": Workload("opt-175b-int4", OPT_175B, 32, 8, 512, 32, weight_tier=2),
}

# Isolated decode attention + KV quantize workload.
ATTN_WORKLOAD = dict(batch=256, heads=96, head_dim=128, context=2048)

# --------------------------------------------------------------------------
# OPT-shaped weights
# --------------------------------------------------------------------------

LAYER_TENSORS = ("ln1_g", "ln1_b", "q_w", "q_b", "k_w", "k_b", "v_w", "v_b",
                 "o_w", "o_b", "ln2_g", "ln2_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b")

TENSOR_TOK_EMB = 0
TENSOR_POS_EMB = 1


def layer_tensor_id(layer: int, t: int) -> int:
    return 2 + 16 * layer + t


def final_ln_tensor_ids(shape: ModelShape):
    return 2 + 16 * shape.n_layers, 3 + 16 * shape.n_layers


def layer_tensor_shapes(shape: ModelShape):
    h, f = shape.hidden, shape.ffn
    return {"ln1_g": (h,), "ln1_b": (h,), "q_w": (h, h), "q_b": (h,), "k_w": (h, h), "k_b": (h,),
            "v_w": (h, h), "v_b": (h,), "o_w": (h, h), "o_b": (h,), "ln2_g": (h,), "ln2_b": (h,),
            "fc1_w": (f, h), "fc1_b": (f,), "fc2_w": (h, f), "fc2_b": (h,)}


def _init_kind(name: str) -> str:
    if name.endswith("_w"):
        return "matrix"
    if name.endswith("_g"):
        return "gain"
    return "bias"


def draw_tensor(shape: ModelShape, name: str, layer: int | None, seed: int = SEED_WEIGHTS,
                variant: str = "plain", out: np.ndarray | None = None) -> np.ndarray:
    """One weight tensor of the OPT-shaped stack.

    variant "plain": matrices and embeddings N(0, 0.02), biases 0, LN gain 1, LN shift 0.
    variant "full":  additionally biases and LN shifts N(0, 0.02), LN gains 1 + N(0, 0.02),
                     so that every bias and LN parameter path carries non-trivial values."""
    if layer is None:
        tid = {"tok_emb": TENSOR_TOK_EMB, "pos_emb": TENSOR_POS_EMB,
               "lnf_g": final_ln_tensor_ids(shape)[0], "lnf_b": final_ln_tensor_ids(shape)[1]}[name]
        shp = {"tok_emb": (shape.vocab, shape.hidden), "pos_emb": (shape.max_pos + 2, shape.hidden),
               "lnf_g": (shape.hidden,), "lnf_b": (shape.hidden,)}[name]
        kind = {"tok_emb": "matrix", "pos_emb": "matrix", "lnf_g": "gain", "lnf_b": "bias"}[name]
    else:
        tid = layer_tensor_id(layer, LAYER_TENSORS.index(name))
        shp = layer_tensor_shapes(shape)[name]
        kind = _init_kind(name)
    if kind == "matrix":
        return normal_f16(seed, tid, shp, 0.0, 0.02, out=out)
    if variant == "plain":
        return constant_f16(shp, 1.0 if kind == "gain" else 0.0, out=out)
    if variant == "full":
        return normal_f16(seed, tid, shp, 1.0 if kind == "gain" else 0.0, 0.02, out=out)
    raise ValueError(f"unknown init variant {variant!r}")


def layer_weights(shape: ModelShape, layer: int, seed: int = SEED_WEIGHTS,
                  variant: str = "plain") -> dict:
    return {n: draw_tensor(shape, n, layer, seed, variant) for n in LAYER_TENSORS}


def global_weights(shape: ModelShape, seed: int = SEED_WEIGHTS, variant: str = "plain") -> dict:
    return {n: draw_tensor(shape, n, None, seed, variant) for n in ("tok_emb", "pos_emb", "lnf_g", "lnf_b")}


def prompt_ids(n_seq: int, prompt_len: int, vocab: int, seed: int = SEED_PROMPTS) -> np.ndarray:
    """Prompt token ids [n_seq][prompt_len], uniform over the vocabulary."""
    return uniform_ids(seed, 0, (n_seq, prompt_len), vocab)


def attn_cache_chunk(batch: int, heads: int, head_dim: int, t0: int, t1: int):
    """Cached K and V of positions t0..t1-1 of the isolated attention workload, N(0, 1),
    position-major [t1-t0][batch][heads][head_dim] (so position chunks are contiguous draws)."""
    per = batch * heads * head_dim
    k = normal_f16(SEED_ATTN, 1, (t1 - t0, batch, heads, head_dim), 0.0, 1.0, offset=t0 * per)
    v = normal_f16(SEED_ATTN, 2, (t1 - t0, batch, heads, head_dim), 0.0, 1.0, offset=t0 * per)
    return k, v


def attn_step_tensors(step: int, batch: int, heads: int, head_dim: int):
    """New K, new V and the query of decode step ``step`` of the isolated attention workload."""
    s = 3 + step
    k = normal_f16(s, 0, (batch, heads, head_dim), 0.0, 1.0)
    v = normal_f16(s, 1, (batch, heads, head_dim), 0.0, 1.0)
    q = normal_f16(s, 2, (batch, heads, head_dim), 0.0, 1.0)
    return k, v, q
