"""Shared helpers of the GPU parity tests (device tensors, comparisons, tie-aware greedy rule)."""
import numpy as np
import pytest


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return torch


def to_dev(a: np.ndarray, torch):
    """numpy (fp16 / uint8 / int32) -> device tensor with the same bits."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.float16).cuda()
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.float16).cuda()
    return torch.from_numpy(a.copy()).cuda()


def to_np16(t) -> np.ndarray:
    """device fp16 tensor -> numpy fp16 with the same bits."""
    return t.detach().contiguous().view(dtype=__import__("torch").int16).cpu().numpy().view(np.float16)


def ulps(a, b, floor: float = 2.0 ** -7):
    """|a - b| in fp16 ulps of max(|a|, |b|, floor): values near zero are judged on the
    absolute scale of `floor` (fp32 and fp64 sums of O(1) terms differ there by ~1e-6)."""
    a = np.asarray(a, dtype=np.float16).astype(np.float64)
    b = np.asarray(b, dtype=np.float16).astype(np.float64)
    mag = np.maximum(np.maximum(np.abs(a), np.abs(b)), floor)
    sp = np.spacing(mag.astype(np.float16)).astype(np.float64)
    return np.abs(a - b) / sp


def tie_aware_greedy(oracle_logits: np.ndarray, gpu_pick: np.ndarray, tau: float = 2e-2):
    """(exact, tie, fail) counts: a GPU pick that differs from the oracle's argmax passes
    only if its oracle logit is within tau of the oracle's best."""
    o = oracle_logits.astype(np.float64)
    best = np.argmax(o, axis=-1)
    exact = gpu_pick == best
    gap = np.take_along_axis(o, best[..., None], -1)[..., 0] - np.take_along_axis(o, gpu_pick[..., None], -1)[..., 0]
    tie = (~exact) & (gap <= tau)
    fail = (~exact) & (gap > tau)
    return int(exact.sum()), int(tie.sum()), int(fail.sum())
