"""Block-scheduled int4 decode of OPT-shaped stacks on MI355X (gfx950).

The compute path is the HIP library ``libtod.so`` behind the C ABI in
``include/tod.h``; this package is a thin ctypes binding (``_lib``) plus a
``Model`` convenience wrapper. PyTorch is used only to own device memory and
streams.
"""
from __future__ import annotations

from . import _lib
from ._lib import (TOD_W_HBM_INT4, TOD_W_HOST_FP16_STREAM, TOD_W_HOST_INT4_STREAM, attn_cache_create,
                   attn_cache_export, attn_cache_fill, attn_cache_free, attn_decode_step, decode_block, default_hw,
                   dequantize_groupwise, estimate_decode, estimate_gemm, export_kv, export_weight, free_model,
                   init_model, last_error, linear_f16, linear_w4, linear_w4_noalloc, plan_decode, prefill,
                   profile_kernels, profile_read, quantize_groupwise, set_decode_graph, set_decode_position,
                   set_global_weights, set_layer_tap, set_layer_weights, set_weight_file, TodError)

__all__ = ["Model", "TodError", "init_model", "set_global_weights", "set_layer_weights", "prefill", "decode_block",
           "set_decode_position", "set_decode_graph", "quantize_groupwise", "dequantize_groupwise", "free_model",
           "last_error", "export_weight", "export_kv", "linear_w4", "linear_w4_noalloc", "linear_f16",
           "attn_cache_create", "attn_cache_fill", "attn_decode_step", "attn_cache_export", "attn_cache_free",
           "profile_kernels", "profile_read", "default_hw", "estimate_decode", "estimate_gemm", "plan_decode",
           "set_weight_file", "set_layer_tap", "TOD_W_HBM_INT4", "TOD_W_HOST_FP16_STREAM", "TOD_W_HOST_INT4_STREAM"]


class Model:
    """One model instance on the current GPU.

    shape: object with n_layers, hidden, n_heads, head_dim, ffn, vocab, max_pos.
    run:   dict with gpu_batch, batches_per_block, prompt_len, gen_len,
           optional weight_tier (0 int4 in HBM, 1 fp16 or 2 int4 streamed from pinned host),
           n_blocks, host_layers, hbm_layers, kv_host_layers and weights_on_disk.
    weight_file: path of the image file when run["weights_on_disk"] is set.
    """

    def __init__(self, shape, run: dict, weight_file: str | None = None):
        self.shape = shape
        self.run = dict(run)
        self.rows = run["gpu_batch"] * run["batches_per_block"]
        self.handle = init_model(shape, self.run)
        if weight_file is not None:
            set_weight_file(self.handle, weight_file)

    def set_global_weights(self, tok_emb, pos_emb, lnf_g, lnf_b):
        set_global_weights(self.handle, tok_emb, pos_emb, lnf_g, lnf_b)

    def set_layer_weights(self, layer: int, tensors):
        set_layer_weights(self.handle, layer, tensors)

    def generate(self, prompt_ids, max_new_tokens: int, block: int = 0, return_logits: bool = False):
        """Greedy generation: prefill, then ``max_new_tokens - 1`` decode steps.

        prompt_ids: int32 device tensor [rows][prompt_len]. Returns int32 tokens
        [rows][max_new_tokens] (and fp16 logits [max_new_tokens][rows][vocab])."""
        import torch

        dev = prompt_ids.device
        first = torch.empty(self.rows, dtype=torch.int32, device=dev)
        steps = max_new_tokens - 1
        out = torch.empty((max(steps, 1), self.rows), dtype=torch.int32, device=dev)
        logits = (torch.empty((max_new_tokens, self.rows, self.shape.vocab), dtype=torch.float16, device=dev)
                  if return_logits else None)
        prefill(self.handle, block, prompt_ids, first, logits[0] if return_logits else None)
        if steps > 0:
            decode_block(self.handle, block, steps, first, out, logits[1:] if return_logits else None)
        tokens = torch.cat([first[:, None], out[:steps].T], dim=1) if steps > 0 else first[:, None]
        return (tokens, logits) if return_logits else tokens

    def close(self):
        if self.handle is not None and self.handle.value:
            free_model(self.handle)
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
