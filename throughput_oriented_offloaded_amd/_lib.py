"""ctypes binding of libtod (include/tod.h): argument marshalling only.

Device buffers are torch tensors on the GPU (their data pointers are passed
through); host weights are numpy arrays. Every computation runs in the HIP
library; if ``libtod.so`` is missing this module raises instead of computing
anything on the CPU.
"""
from __future__ import annotations

import ctypes
import functools
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtod.so")

TOD_OK, TOD_EINVAL, TOD_ENOMEM, TOD_EHIP, TOD_ESTATE = 0, -1, -2, -3, -4
TOD_W_HBM_INT4, TOD_W_HOST_FP16_STREAM, TOD_W_HOST_INT4_STREAM = 0, 1, 2
MATRICES = ("q", "k", "v", "o", "fc1", "fc2")
LAYER_TENSORS = ("ln1_g", "ln1_b", "q_w", "q_b", "k_w", "k_b", "v_w", "v_b",
                 "o_w", "o_b", "ln2_g", "ln2_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b")

EXPORTED = ("init_model", "set_global_weights", "set_layer_weights", "prefill", "decode_block",
            "set_decode_position", "set_decode_graph", "quantize_groupwise", "dequantize_groupwise", "free_model",
            "last_error",
            "export_weight", "export_kv", "linear_w4", "linear_f16", "attn_cache_create", "attn_cache_fill",
            "attn_decode_step", "attn_cache_export", "attn_cache_free", "profile_kernels", "profile_read",
            "default_hw", "estimate_decode", "plan_decode", "set_weight_file", "set_layer_tap",
            "linear_w4_noalloc", "estimate_gemm")
KERNEL_KINDS = ("gemm_qkv", "gemm_o", "gemm_fc1", "gemm_fc2", "attn", "kv_append", "layernorm", "lm_head",
                "argmax", "embed")


class TodError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed ({code}): {msg}")
        self.code = code


class ModelConfig(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("max_pos", ctypes.c_int32)]


class RunConfig(ctypes.Structure):
    _fields_ = [("gpu_batch", ctypes.c_int32), ("batches_per_block", ctypes.c_int32),
                ("prompt_len", ctypes.c_int32), ("gen_len", ctypes.c_int32), ("group", ctypes.c_int32),
                ("weight_tier", ctypes.c_int32), ("n_blocks", ctypes.c_int32), ("host_layers", ctypes.c_int32),
                ("hbm_layers", ctypes.c_int32), ("kv_host_layers", ctypes.c_int32),
                ("weights_on_disk", ctypes.c_int32)]


class HW(ctypes.Structure):
    _fields_ = [(n, ctypes.c_double) for n in ("attn_gbs", "mem_gbs", "link_gbs", "int4_tflops", "fp16_tflops",
                                                 "launch_us", "hbm_bytes", "host_bytes", "disk_gbs", "disk_bytes",
                                                 "gemm_wg_us", "staged_tflops", "staged_gbs", "staged_us")]


class Estimate(ctypes.Structure):
    _fields_ = [(n, ctypes.c_double) for n in ("step_s", "tokens_per_s", "compute_s", "link_s", "hbm_bytes",
                                                 "host_bytes", "workspace_bytes", "disk_bytes")]
    _fields_ += [("fits", ctypes.c_int32)]


@functools.lru_cache(maxsize=None)
def lib() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(python -m throughput_oriented_offloaded_amd.build)")
    # torch ships its own HIP runtime under the same soname as ROCm's; load it first so that this
    # library binds to the runtime torch uses (two runtimes in one process do not share a device)
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    sig = {
        "init_model": [vp, vp, vp, vp],
        "set_global_weights": [vp, vp, vp, vp, vp],
        "set_layer_weights": [vp, i32, vp],
        "prefill": [vp, i32, vp, vp, vp, vp],
        "decode_block": [vp, i32, i32, vp, vp, vp, vp],
        "set_decode_position": [vp, i32, i32],
        "set_decode_graph": [vp, i32],
        "quantize_groupwise": [vp, i64, i32, vp, vp, vp, vp],
        "dequantize_groupwise": [vp, vp, vp, i64, i32, vp, vp],
        "free_model": [vp],
        "export_weight": [vp, i32, i32, vp, vp, vp, vp],
        "export_kv": [vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp],
        "linear_w4": [vp, i64, i32, i32, vp, vp, vp, vp, vp, i32, vp, vp],
        "linear_f16": [vp, i64, i32, i32, vp, vp, vp, i32, vp, vp],
        "linear_w4_noalloc": [vp, i64, i32, i32, vp, vp, vp, vp, vp, i32, vp, vp],
        "attn_cache_create": [i32, i32, i32, i32, vp],
        "attn_cache_fill": [vp, vp, vp, i32, i32, vp],
        "attn_decode_step": [vp, i32, vp, vp, vp, vp, vp],
        "attn_cache_export": [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp],
        "attn_cache_free": [vp],
        "profile_kernels": [vp, ctypes.c_uint],
        "profile_read": [vp, i32, vp, vp],
        "estimate_decode": [vp, vp, vp, vp],
        "plan_decode": [vp, i32, i32, i32, vp, vp, vp],
        "estimate_gemm": [i64, i32, i32, i32, vp, vp],
        "set_weight_file": [vp, ctypes.c_char_p],
        "set_layer_tap": [vp, i32, i32, i64, i64, vp, vp],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.last_error.argtypes = []
    L.last_error.restype = ctypes.c_char_p
    L.default_hw.argtypes = [vp]
    L.default_hw.restype = None
    return L


def _check(fn: str, rc: int):
    if rc != TOD_OK:
        raise TodError(fn, rc, lib().last_error().decode(errors="replace"))


def _ptr(t):
    """Device pointer of a torch tensor (or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to libtod must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _host16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    if a.dtype != np.uint16:
        raise ValueError("host weights must be fp16")
    return a


# ---------------------------------------------------------------------------- model

def init_model(cfg, run, stream=None) -> ctypes.c_void_p:
    """cfg: synth.ModelShape-like (n_layers, hidden, n_heads, head_dim, ffn, vocab, max_pos);
    run: dict with gpu_batch, batches_per_block, prompt_len, gen_len, and optional group, weight_tier,
    n_blocks, host_layers, hbm_layers, kv_host_layers, weights_on_disk."""
    mc, rc_ = _model_config(cfg), _run_config(run)
    h = ctypes.c_void_p()
    _check("init_model", lib().init_model(ctypes.byref(mc), ctypes.byref(rc_), _stream(stream), ctypes.byref(h)))
    return h


def set_global_weights(m, tok_emb: np.ndarray, pos_emb: np.ndarray, lnf_g: np.ndarray, lnf_b: np.ndarray):
    arrs = [_host16(x) for x in (tok_emb, pos_emb, lnf_g, lnf_b)]
    _check("set_global_weights", lib().set_global_weights(m, *[a.ctypes.data for a in arrs]))


def set_weight_file(m, path: str):
    _check("set_weight_file", lib().set_weight_file(m, os.fsencode(path)))


def set_layer_weights(m, layer: int, tensors):
    """tensors: dict keyed by LAYER_TENSORS or a sequence in that order (fp16 numpy)."""
    if isinstance(tensors, dict):
        tensors = [tensors[n] for n in LAYER_TENSORS]
    arrs = [_host16(x) for x in tensors]
    ptrs = (ctypes.c_void_p * 16)(*[a.ctypes.data for a in arrs])
    _check("set_layer_weights", lib().set_layer_weights(m, layer, ptrs))


def prefill(m, block: int, ids, next_ids, logits=None, stream=None):
    _check("prefill", lib().prefill(m, block, _ptr(ids), _ptr(next_ids), _ptr(logits), _stream(stream)))


def decode_block(m, block: int, n_steps: int, ids_in, ids_out, logits=None, stream=None):
    _check("decode_block", lib().decode_block(m, block, n_steps, _ptr(ids_in), _ptr(ids_out), _ptr(logits),
                                              _stream(stream)))


def set_decode_position(m, block: int, steps: int):
    _check("set_decode_position", lib().set_decode_position(m, block, steps))


def set_decode_graph(m, enable: bool):
    _check("set_decode_graph", lib().set_decode_graph(m, int(bool(enable))))


def set_layer_tap(m, phase: str, layer: int, row0: int = 0, n_rows: int = 0, t_in=None, t_out=None):
    """phase "prefill" or "decode"; n_rows 0 removes the tap."""
    ph = {"prefill": 0, "decode": 1}[phase]
    _check("set_layer_tap", lib().set_layer_tap(m, ph, layer, row0, n_rows, _ptr(t_in), _ptr(t_out)))


def free_model(m):
    _check("free_model", lib().free_model(m))


def last_error() -> str:
    return lib().last_error().decode(errors="replace")


def export_weight(m, layer: int, which: str, codes, scale, zero, stream=None):
    _check("export_weight", lib().export_weight(m, layer, MATRICES.index(which), _ptr(codes), _ptr(scale),
                                                _ptr(zero), _stream(stream)))


def export_kv(m, layer: int, block: int, row: int, head: int, t0: int, t1: int, kc, ks, kz, vc, vs, vz,
              stream=None):
    _check("export_kv", lib().export_kv(m, layer, block, row, head, t0, t1, _ptr(kc), _ptr(ks), _ptr(kz),
                                        _ptr(vc), _ptr(vs), _ptr(vz), _stream(stream)))


# ---------------------------------------------------------------------------- kernels

def quantize_groupwise(x, codes, scale, zero, group: int = 64, stream=None):
    _check("quantize_groupwise", lib().quantize_groupwise(_ptr(x), x.numel(), group, _ptr(codes), _ptr(scale),
                                                          _ptr(zero), _stream(stream)))


def dequantize_groupwise(codes, scale, zero, n: int, out, group: int = 64, stream=None):
    _check("dequantize_groupwise", lib().dequantize_groupwise(_ptr(codes), _ptr(scale), _ptr(zero), n, group,
                                                              _ptr(out), _stream(stream)))


def linear_w4(a, codes, scale, zero, out_features: int, y, bias=None, residual=None, relu=False, stream=None):
    rows, k = a.shape
    _check("linear_w4", lib().linear_w4(_ptr(a), rows, k, out_features, _ptr(codes), _ptr(scale), _ptr(zero),
                                        _ptr(bias), _ptr(residual), int(relu), _ptr(y), _stream(stream)))


def linear_w4_noalloc(a, codes, scale, zero, out_features: int, y, bias=None, residual=None, relu=False,
                      stream=None):
    rows, k = a.shape
    _check("linear_w4_noalloc", lib().linear_w4_noalloc(_ptr(a), rows, k, out_features, _ptr(codes), _ptr(scale),
                                                        _ptr(zero), _ptr(bias), _ptr(residual), int(relu), _ptr(y),
                                                        _stream(stream)))


def linear_f16(a, w, y, bias=None, residual=None, relu=False, stream=None):
    rows, k = a.shape
    _check("linear_f16", lib().linear_f16(_ptr(a), rows, k, w.shape[0], _ptr(w), _ptr(bias), _ptr(residual),
                                          int(relu), _ptr(y), _stream(stream)))


def attn_cache_create(batch: int, heads: int, head_dim: int, cap: int):
    h = ctypes.c_void_p()
    _check("attn_cache_create", lib().attn_cache_create(batch, heads, head_dim, cap, ctypes.byref(h)))
    return h


def attn_cache_fill(c, k, v, t0: int, stream=None):
    """k, v: fp16 device tensors [n][batch][heads][head_dim] for positions t0..t0+n-1."""
    n = k.shape[0]
    _check("attn_cache_fill", lib().attn_cache_fill(c, _ptr(k), _ptr(v), t0, n, _stream(stream)))


def attn_decode_step(c, pos: int, q, k_new, v_new, out, stream=None):
    _check("attn_decode_step", lib().attn_decode_step(c, pos, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out),
                                                      _stream(stream)))


def attn_cache_export(c, seq: int, head: int, t0: int, t1: int, kc, ks, kz, vc, vs, vz, stream=None):
    _check("attn_cache_export", lib().attn_cache_export(c, seq, head, t0, t1, _ptr(kc), _ptr(ks), _ptr(kz),
                                                        _ptr(vc), _ptr(vs), _ptr(vz), _stream(stream)))


def attn_cache_free(c):
    _check("attn_cache_free", lib().attn_cache_free(c))


def profile_kernels(m, kinds=()):
    """Time every launch of the given kernel classes (names in KERNEL_KINDS) with HIP events."""
    mask = 0
    for k in kinds:
        mask |= 1 << KERNEL_KINDS.index(k)
    _check("profile_kernels", lib().profile_kernels(m, mask))


def profile_read(m, kind: str):
    """(total ms, launches) of a profiled kernel class since profile_kernels."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check("profile_read", lib().profile_read(m, KERNEL_KINDS.index(kind), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


# ---------------------------------------------------------------------------- cost model

def _struct_dict(st) -> dict:
    return {n: getattr(st, n) for n, _ in st._fields_}


def default_hw() -> dict:
    """The library's measured MI355X rates and capacities (see tod.h, default_hw)."""
    hw = HW()
    lib().default_hw(ctypes.byref(hw))
    return _struct_dict(hw)


def _model_config(cfg) -> ModelConfig:
    return ModelConfig(cfg.n_layers, cfg.hidden, cfg.n_heads, cfg.head_dim, cfg.ffn, cfg.vocab, cfg.max_pos)


def _run_config(run: dict) -> RunConfig:
    return RunConfig(run["gpu_batch"], run["batches_per_block"], run["prompt_len"], run["gen_len"],
                     run.get("group", 64), run.get("weight_tier", 0), run.get("n_blocks", 1),
                     run.get("host_layers", 0), run.get("hbm_layers", 0), run.get("kv_host_layers", 0),
                     run.get("weights_on_disk", 0))


def estimate_decode(cfg, run: dict, hw: dict | None = None) -> dict:
    """Predicted decode step (seconds, tokens/s) and footprint of a run configuration."""
    h = HW(**(hw or default_hw()))
    est = Estimate()
    mc, rc_ = _model_config(cfg), _run_config(run)
    _check("estimate_decode", lib().estimate_decode(ctypes.byref(mc), ctypes.byref(rc_), ctypes.byref(h),
                                                    ctypes.byref(est)))
    return _struct_dict(est)


def estimate_gemm(rows: int, out_features: int, in_features: int, int4: bool, hw: dict | None = None) -> float:
    """Seconds the cost model charges one GEMM of this shape."""
    h = HW(**(hw or default_hw()))
    t = ctypes.c_double()
    _check("estimate_gemm", lib().estimate_gemm(rows, out_features, in_features, int(int4), ctypes.byref(h),
                                                ctypes.byref(t)))
    return t.value


def plan_decode(cfg, prompt_len: int, gen_len: int, max_rows: int, hw: dict | None = None):
    """Best run configuration (dict) for decode tokens/s under the capacities, and its estimate."""
    h = HW(**(hw or default_hw()))
    best, est = RunConfig(), Estimate()
    mc = _model_config(cfg)
    _check("plan_decode", lib().plan_decode(ctypes.byref(mc), prompt_len, gen_len, max_rows, ctypes.byref(h),
                                            ctypes.byref(best), ctypes.byref(est)))
    return _struct_dict(best), _struct_dict(est)
