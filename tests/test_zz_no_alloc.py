"""linear_w4_noalloc (the entry point that allocates nothing) against linear_w4.

Both run the same repack and GEMM kernels on the same plan, so their outputs
must be identical bit for bit. Two calls in a row go through the shared
scratch: the first at the OPT-30B fc2 decode shape (512 rows, K split four
ways, so the split-K partials live in the scratch too), the second smaller
(ragged rows and columns, K split eight ways), so stale contents of the
first call must not leak into the second. Calls that need more scratch than
it holds are rejected before any device work, also without a GPU.
"""
import ctypes

import numpy as np
import pytest

import synth
from tests.gpu_util import to_dev, torch_cuda

NULL = None
FAKE = 0x1000  # never dereferenced: every case below fails its checks before device work


def _lib():
    from throughput_oriented_offloaded_amd import _lib
    return _lib.lib()


def test_noalloc_rejects_calls_beyond_its_scratch_without_device_work():
    lib = _lib()
    # 32768 x 16384 int4 weights need 256 MiB + 32 MiB of repacked codes and params: over 192 MiB
    rc = lib.linear_w4_noalloc(FAKE, 1, 16384, 32768, FAKE, FAKE, FAKE, NULL, NULL, 0, FAKE, NULL)
    assert rc == -1
    assert b"scratch" in lib.last_error()
    for args in ((NULL, 1, 64, 32, FAKE, FAKE, FAKE), (FAKE, 1, 64, 32, NULL, FAKE, FAKE),
                 (FAKE, 1, 63, 32, FAKE, FAKE, FAKE), (FAKE, 1, 64, 48, FAKE, FAKE, FAKE),
                 (FAKE, -1, 64, 32, FAKE, FAKE, FAKE)):
        assert lib.linear_w4_noalloc(*args, NULL, NULL, 0, FAKE, NULL) == -1, args
    assert lib.linear_w4_noalloc(FAKE, 1, 64, 32, FAKE, FAKE, FAKE, NULL, FAKE, 1, FAKE, NULL) == -1  # relu+res


def _weights(torch, tod, n, k, seed):
    w = synth.normal_f16(seed, 0, (n, k), 0.0, 0.02)
    wd = to_dev(w.reshape(-1), torch)
    codes = torch.empty(n * k // 2, dtype=torch.uint8, device="cuda")
    scale = torch.empty(n * k // 64, dtype=torch.float16, device="cuda")
    zero = torch.empty(n * k // 64, dtype=torch.float16, device="cuda")
    tod.quantize_groupwise(wd, codes, scale, zero)
    return codes, scale, zero


@pytest.mark.gpu
def test_noalloc_matches_linear_w4_on_two_calls():
    torch = torch_cuda()
    import throughput_oriented_offloaded_amd as tod
    outs = []
    for rows, k, n, epi, seed in ((512, 28672, 7168, "res", 71), (257, 4096, 2080, "relu", 72)):
        print(f"linear_w4_noalloc rows={rows} in={k} out={n} {epi}", flush=True)
        codes, scale, zero = _weights(torch, tod, n, k, seed)
        a = to_dev(synth.normal_f16(seed, 1, (rows, k), 0.0, 1.0), torch)
        bias = to_dev(synth.normal_f16(seed, 2, (n,), 0.0, 0.1), torch)
        res = to_dev(synth.normal_f16(seed, 3, (rows, n), 0.0, 1.0), torch) if epi == "res" else None
        ref = torch.empty((rows, n), dtype=torch.float16, device="cuda")
        got = torch.full((rows, n), float("nan"), dtype=torch.float16, device="cuda")
        tod.linear_w4(a, codes, scale, zero, n, ref, bias=bias, residual=res, relu=epi == "relu")
        tod.linear_w4_noalloc(a, codes, scale, zero, n, got, bias=bias, residual=res, relu=epi == "relu")
        torch.cuda.synchronize()
        same = torch.equal(got.view(torch.int16), ref.view(torch.int16))
        print(f"  identical bits: {same}", flush=True)
        assert same
        outs.append(got)
    # a call beyond the scratch fails cleanly on a GPU too, and leaves the device usable
    with pytest.raises(tod.TodError):
        tod.linear_w4_noalloc(torch.zeros((1, 16384), dtype=torch.float16, device="cuda"),
                              torch.zeros(32768 * 16384 // 2, dtype=torch.uint8, device="cuda"),
                              torch.zeros(32768 * 16384 // 64, dtype=torch.float16, device="cuda"),
                              torch.zeros(32768 * 16384 // 64, dtype=torch.float16, device="cuda"), 32768,
                              torch.empty((1, 32768), dtype=torch.float16, device="cuda"))
    torch.cuda.synchronize()
    assert np.isfinite(outs[-1].float().cpu().numpy()).all()
