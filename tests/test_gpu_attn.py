"""GPU decode attention over the int4 KV cache and the per-step KV quantize+append.

Cache codes, scales and zeros must equal the oracle's quantizer bit for bit.
Attention outputs: the oracle attends over dequantized values rounded to fp16
(zero + c*scale, one rounding each). The GPU kernel dequantizes K the same
way (packed fp16 FMA, one rounding), so its scores differ from the oracle's
only by fp32 summation; for V it uses the factored form scale * sum(p*c) +
zero * sum(p) in fp32, which never rounds the dequantized value. That
differs from the oracle's weighted mean by at most half an fp16 ulp of the
largest |v|, and each side rounds its output to fp16 once, so the
per-element bar is
    |o_gpu - o_oracle| <= ulp16(max|v|)/2 + ulp16(max(|o_gpu|, |o_oracle|)) + 1e-5
(the last term for fp32 sums and exp), and the mean error must stay well
below it. That bound is loose by construction, so the outputs are also held
to the oracle's exact-V reading (the same attention on the exact values
zero + c*scale, the one rounding the GPU leaves out): there only fp32
accumulation, the fp32 exp and the output rounding differ, and every element
must be within 1 fp16 ulp (judged on an absolute floor of 2^-7 near zero),
with a mean under 0.05 ulp (measured: at most 1 ulp, mean 0.012 ulp and 97.5%
bit-equal at 2051 positions); a V accumulation that lost a few bits fails
that, as the earlier offset form (acc += p*s*(1024 + c)) did at 700 and 2051
positions. Contexts straddle the kernel's 64-position chunks and its pairs of
chunks; a scaled query gives sharply peaked softmax weights.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import to_dev, to_np16, torch_cuda, ulps

pytestmark = pytest.mark.gpu


def _oracle_cache(kseq, vseq):
    """kseq, vseq: [T][d] fp16 of one (sequence, head) -> the oracle's int4 cache arrays."""
    T, d = kseq.shape
    kc, ks, kz = oracle.quantize_groupwise(np.ascontiguousarray(kseq))
    vc, vs, vz = oracle.quantize_groupwise(np.ascontiguousarray(vseq))
    G = d // 64
    return (kc.reshape(T, d // 2), ks.reshape(T, G), kz.reshape(T, G), vc.reshape(T, d // 2), vs.reshape(T, G),
            vz.reshape(T, G))


def _spacing16(x):
    return np.spacing(np.abs(np.asarray(x, dtype=np.float64)).astype(np.float16)).astype(np.float64)


EXACT_V_MAX_ULP = 1
EXACT_V_MEAN_ULP = 0.05


def _check_attention(got, q, ref_cache, label, stats=None):
    """got: the GPU's fp16 output of one (sequence, head); q its query; ref_cache the oracle's
    int4 cache arrays. Checks both readings (see the module docstring); stats collects the
    exact-V ulp errors for a summary line."""
    ref = oracle.attend(q, *ref_cache)
    with oracle.exact_v():
        ref_x = oracle.attend(q, *ref_cache)
    vh = oracle.dequantize_groupwise(ref_cache[3], ref_cache[4], ref_cache[5]).astype(np.float64)
    big = np.maximum(np.abs(got.astype(np.float64)), np.abs(ref.astype(np.float64)))
    tol = 0.5 * _spacing16(np.abs(vh).max()) + _spacing16(big) + 1e-5
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    assert np.all(err <= tol), f"{label}: max err {err.max():.3g} (bound {tol.min():.3g}..{tol.max():.3g})"
    assert err.mean() <= 0.25 * tol.mean(), f"{label}: mean err {err.mean():.3g}"
    u = ulps(got, ref_x)
    if stats is not None:
        stats.append(u)
    assert u.max() <= EXACT_V_MAX_ULP, f"{label}: {u.max():.0f} ulp from the exact-V reading"
    assert u.mean() <= EXACT_V_MEAN_ULP, f"{label}: mean {u.mean():.3f} ulp from the exact-V reading"


def _summary(label, stats):
    u = np.concatenate([x.reshape(-1) for x in stats])
    print(f"{label}: vs exact-V reading max {u.max():.0f} ulp, mean {u.mean():.4f} ulp, "
          f"{np.mean(u == 0):.4f} equal", flush=True)


def _export(tod, torch, c, b, h, T, d):
    G = d // 64
    kc = torch.empty((T, d // 2), dtype=torch.uint8, device="cuda")
    vc = torch.empty((T, d // 2), dtype=torch.uint8, device="cuda")
    ks, kz, vs, vz = (torch.empty((T, G), dtype=torch.float16, device="cuda") for _ in range(4))
    tod.attn_cache_export(c, b, h, 0, T, kc, ks, kz, vc, vs, vz)
    torch.cuda.synchronize()
    return (kc.cpu().numpy(), to_np16(ks), to_np16(kz), vc.cpu().numpy(), to_np16(vs), to_np16(vz))


@pytest.mark.parametrize("B,H,d,T,qsig", [(3, 2, 128, 0, 1.0), (3, 2, 128, 63, 1.0), (2, 3, 128, 64, 1.0),
                                          (2, 2, 128, 127, 1.0), (1, 3, 128, 128, 1.0), (2, 2, 128, 200, 1.0),
                                          (4, 2, 64, 65, 1.0), (2, 2, 64, 191, 1.0), (1, 1, 64, 1, 1.0),
                                          (2, 1, 128, 700, 1.0), (2, 2, 128, 300, 6.0), (2, 2, 64, 130, 6.0)])
def test_decode_step_matches_oracle(B, H, d, T, qsig):
    """qsig scales the query: 6.0 gives peaked softmax weights (a few positions dominate)."""
    torch = torch_cuda()
    import throughput_oriented_offloaded_amd as tod
    print(f"attention B={B} H={H} d={d} cached={T} qsig={qsig}", flush=True)
    seed = 100 + B * 13 + H * 7 + d + T
    k = synth.normal_f16(seed, 1, (T, B, H, d), 0.0, 1.0)
    v = synth.normal_f16(seed, 2, (T, B, H, d), 0.0, 1.0)
    q = synth.normal_f16(seed, 3, (B, H, d), 0.0, qsig)
    kn = synth.normal_f16(seed, 4, (B, H, d), 0.0, 1.0)
    vn = synth.normal_f16(seed, 5, (B, H, d), 0.0, 1.0)
    c = tod.attn_cache_create(B, H, d, T + 1)
    try:
        if T:
            tod.attn_cache_fill(c, to_dev(k, torch), to_dev(v, torch), 0)
        out = torch.empty((B, H, d), dtype=torch.float16, device="cuda")
        tod.attn_decode_step(c, T, to_dev(q, torch), to_dev(kn, torch), to_dev(vn, torch), out)
        torch.cuda.synchronize()
        got = to_np16(out)
        stats = []
        for b in range(B):
            for h in range(H):
                ks = np.concatenate([k[:, b, h, :], kn[None, b, h, :]])
                vs = np.concatenate([v[:, b, h, :], vn[None, b, h, :]])
                ref_cache = _oracle_cache(ks, vs)
                gpu_cache = _export(tod, torch, c, b, h, T + 1, d)
                for x, y in zip(gpu_cache, ref_cache):
                    assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8))
                _check_attention(got[b, h], q[b, h], ref_cache, f"(b={b}, h={h})", stats)
        _summary(f"B={B} H={H} d={d} cached={T} qsig={qsig}", stats)
    finally:
        tod.attn_cache_free(c)


def test_decode_attention_full_size():
    """Isolated attention workload at full size: batch 256, 96 heads, d 128, 2048 cached
    positions; 3 decode steps appended; sampled (sequence, head) pairs against the oracle."""
    torch = torch_cuda()
    import throughput_oriented_offloaded_amd as tod
    W = synth.ATTN_WORKLOAD
    B, H, d, T = W["batch"], W["heads"], W["head_dim"], W["context"]
    steps = 3
    pairs = [(0, 0), (0, 95), (1, 7), (127, 48), (200, 3), (255, 95)]
    hist_k = {p: [] for p in pairs}
    hist_v = {p: [] for p in pairs}
    c = tod.attn_cache_create(B, H, d, T + steps)
    try:
        chunk = 128
        for t0 in range(0, T, chunk):
            k, v = synth.attn_cache_chunk(B, H, d, t0, t0 + chunk)
            for (b, h) in pairs:
                hist_k[(b, h)].append(k[:, b, h, :].copy())
                hist_v[(b, h)].append(v[:, b, h, :].copy())
            tod.attn_cache_fill(c, to_dev(k, torch), to_dev(v, torch), t0)
            del k, v
        print("filled 2048 positions", flush=True)
        out = torch.empty((B, H, d), dtype=torch.float16, device="cuda")
        for st in range(steps):
            kn, vn, q = synth.attn_step_tensors(st, B, H, d)
            tod.attn_decode_step(c, T + st, to_dev(q, torch), to_dev(kn, torch), to_dev(vn, torch), out)
            for (b, h) in pairs:
                hist_k[(b, h)].append(kn[None, b, h, :])
                hist_v[(b, h)].append(vn[None, b, h, :])
        torch.cuda.synchronize()
        got = to_np16(out)
        stats = []
        for (b, h) in pairs:
            ks = np.concatenate(hist_k[(b, h)])
            vs = np.concatenate(hist_v[(b, h)])
            ref_cache = _oracle_cache(ks, vs)
            gpu_cache = _export(tod, torch, c, b, h, T + steps, d)
            for x, y in zip(gpu_cache, ref_cache):
                assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8))
            _check_attention(got[b, h], q[b, h], ref_cache, f"(b={b}, h={h})", stats)
        _summary("full size", stats)
    finally:
        tod.attn_cache_free(c)


def test_attention_bad_position_is_an_error():
    torch = torch_cuda()
    import throughput_oriented_offloaded_amd as tod
    c = tod.attn_cache_create(1, 1, 64, 64)
    try:
        x = torch.zeros((1, 1, 64), dtype=torch.float16, device="cuda")
        with pytest.raises(tod.TodError):
            tod.attn_decode_step(c, 64, x, x, x, x)
    finally:
        tod.attn_cache_free(c)


def test_attention_misaligned_buffers_are_an_error():
    torch = torch_cuda()
    import throughput_oriented_offloaded_amd as tod
    c = tod.attn_cache_create(1, 1, 64, 64)
    try:
        buf = torch.zeros(72, dtype=torch.float16, device="cuda")
        x = buf[:64].view(1, 1, 64)
        bad = buf[1:65].view(1, 1, 64)  # 2 bytes off a 16-byte boundary
        with pytest.raises(tod.TodError):
            tod.attn_decode_step(c, 0, bad, x, x, x)
        with pytest.raises(tod.TodError):
            tod.attn_cache_fill(c, bad.view(1, 1, 1, 64), x.view(1, 1, 1, 64), 0)
        tod.attn_decode_step(c, 0, x, x, x, x)  # aligned buffers still work
        torch.cuda.synchronize()
    finally:
        tod.attn_cache_free(c)
