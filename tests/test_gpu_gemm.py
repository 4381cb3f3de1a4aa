"""GPU fused int4 dequant + MFMA GEMM parity against the oracle's linear layers.

Both sides start from the same fp16 weights: the GPU quantizes them with its
own kernel (bit-exact to the oracle's, tested separately), the oracle with its
own quantizer. Outputs are fp16; fp32 (GPU) against fp64 (oracle)
accumulation may move a result across an fp16 rounding boundary, so the bar
is at most 1 fp16 ulp per element (2 where a split-K sum adds a rounding).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import to_dev, to_np16, torch_cuda, ulps

pytestmark = pytest.mark.gpu


def _gpu_codes(w16, torch):
    import throughput_oriented_offloaded_amd as tod
    wd = to_dev(w16.reshape(-1), torch)
    n = w16.size
    codes = torch.empty(n // 2, dtype=torch.uint8, device="cuda")
    scale = torch.empty(n // 64, dtype=torch.float16, device="cuda")
    zero = torch.empty(n // 64, dtype=torch.float16, device="cuda")
    tod.quantize_groupwise(wd, codes, scale, zero)
    return codes, scale, zero


CASES = [  # rows, in, out, epilogue
    (1, 64, 32, "bias"), (13, 192, 96, "res"), (64, 768, 2304, "relu"), (100, 768, 768, "none"),
    (129, 256, 160, "res"), (300, 1024, 256, "bias"), (512, 3072, 768, "res"), (37, 4096, 64, "relu"),
    # pipelined kernel with ragged M and N tiles, split along K
    (300, 1280, 480, "relu"), (640, 2048, 1056, "res"), (257, 4096, 288, "bias"),
    # pipelined kernel, one wave of tiles: 192-row tiles (QKV-like width; ragged M and N)
    (512, 512, 21504, "bias"), (450, 768, 20384, "res"),
    # 256-row tiles, where 192-row ones would need a second wave (fc1-like width; ragged M and N)
    (500, 512, 28640, "relu"),
    # more than four row tiles, where tile ids run in groups of four row tiles: two whole groups;
    # a ragged last group of three (and ragged N); the same with the K loop split eight ways
    (2000, 512, 1056, "res"), (2600, 768, 800, "relu"), (2600, 4096, 256, "bias"),
]


@pytest.mark.parametrize("rows,k,n,epi", CASES)
def test_linear_w4_matches_oracle(rows, k, n, epi):
    torch = torch_cuda()
    import throughput_oriented_offloaded_amd as tod
    print(f"linear_w4 rows={rows} in={k} out={n} {epi}", flush=True)
    seed = rows * 7 + k + n
    w = synth.normal_f16(seed, 0, (n, k), 0.0, 0.02)
    a = synth.normal_f16(seed, 1, (rows, k), 0.0, 1.0)
    bias = synth.normal_f16(seed, 2, (n,), 0.0, 0.1) if epi != "none" else None
    res = synth.normal_f16(seed, 3, (rows, n), 0.0, 1.0) if epi == "res" else None
    codes, scale, zero = _gpu_codes(w, torch)
    y = torch.empty((rows, n), dtype=torch.float16, device="cuda")
    tod.linear_w4(to_dev(a, torch), codes, scale, zero, n, y, bias=to_dev(bias, torch) if bias is not None else None,
                  residual=to_dev(res, torch) if res is not None else None, relu=epi == "relu")
    torch.cuda.synchronize()
    oc, os_, oz = oracle.quantize_groupwise(w)
    ref = oracle.linear_w4(a, oc, os_, oz, n, bias=bias, residual=res, relu=epi == "relu")
    u = ulps(to_np16(y), ref)
    assert u.max() <= 2, f"max {u.max()} ulp"
    assert (u == 0).mean() > 0.99


SHORT_CASES = [  # rows, in, out, epilogue: 128 rows or fewer on the pipelined kernel's 64- and 128-row tiles
    (8, 2048, 32768, "relu"), (64, 1024, 20480, "bias"), (100, 2048, 16384, "res"), (128, 1024, 32768, "none"),
    (37, 4096, 16384, "res"), (128, 7168, 7168, "bias"),
]


@pytest.mark.parametrize("rows,k,n,epi", SHORT_CASES)
def test_linear_w4_short_tiles(rows, k, n, epi):
    """Few rows and wide N: 64- or 128-row tiles (ragged M at 37 and 100 rows), with and without a
    split K loop; the oracle checks the first, middle and last rows."""
    torch = torch_cuda()
    import throughput_oriented_offloaded_amd as tod
    print(f"linear_w4 short rows={rows} in={k} out={n} {epi}", flush=True)
    seed = rows * 13 + k + n
    w = synth.normal_f16(seed, 0, (n, k), 0.0, 0.02)
    a = synth.normal_f16(seed, 1, (rows, k), 0.0, 1.0)
    bias = synth.normal_f16(seed, 2, (n,), 0.0, 0.1) if epi != "none" else None
    res = synth.normal_f16(seed, 3, (rows, n), 0.0, 1.0) if epi == "res" else None
    codes, scale, zero = _gpu_codes(w, torch)
    y = torch.empty((rows, n), dtype=torch.float16, device="cuda")
    tod.linear_w4(to_dev(a, torch), codes, scale, zero, n, y, bias=to_dev(bias, torch) if bias is not None else None,
                  residual=to_dev(res, torch) if res is not None else None, relu=epi == "relu")
    torch.cuda.synchronize()
    sample = np.unique(np.array([0, rows // 2, rows - 1]))
    oc, os_, oz = oracle.quantize_groupwise(w)
    ref = oracle.linear_w4(a[sample], oc, os_, oz, n, bias=bias, residual=res[sample] if res is not None else None,
                           relu=epi == "relu")
    u = ulps(to_np16(y)[sample], ref)
    assert u.max() <= 2, f"max {u.max()} ulp"
    assert (u == 0).mean() > 0.99


def test_linear_residual_in_place():
    """The decode path adds the residual into the same buffer it writes."""
    torch = torch_cuda()
    import throughput_oriented_offloaded_amd as tod
    rows, k, n = 70, 512, 512
    w = synth.normal_f16(5, 0, (n, k), 0.0, 0.02)
    a = synth.normal_f16(5, 1, (rows, k), 0.0, 1.0)
    h = synth.normal_f16(5, 2, (rows, n), 0.0, 1.0)
    codes, scale, zero = _gpu_codes(w, torch)
    hd = to_dev(h, torch)
    tod.linear_w4(to_dev(a, torch), codes, scale, zero, n, hd, residual=hd)
    torch.cuda.synchronize()
    oc, os_, oz = oracle.quantize_groupwise(w)
    ref = oracle.linear_w4(a, oc, os_, oz, n, residual=h)
    assert ulps(to_np16(hd), ref).max() <= 2


F16_CASES = [  # rows, in, out, epilogue: above 128 rows with out % 32 == 0 the pipelined kernel runs
    (129, 256, 160, "res"), (300, 1280, 480, "relu"), (257, 4096, 288, "bias"), (640, 2048, 1056, "res"),
    (512, 3072, 768, "none"), (300, 512, 200, "bias"), (100, 768, 768, "res"),
]


@pytest.mark.parametrize("rows,k,n,epi", F16_CASES)
def test_linear_f16_matches_oracle(rows, k, n, epi):
    """fp16-weight GEMM with ragged M and N tiles, split K and every epilogue; out = 200 is not a
    multiple of 32 and 100 rows stay at 128 or fewer, so those take the register-staged kernel."""
    torch = torch_cuda()
    import throughput_oriented_offloaded_amd as tod
    print(f"linear_f16 rows={rows} in={k} out={n} {epi}", flush=True)
    seed = rows * 11 + k + n
    w = synth.normal_f16(seed, 0, (n, k), 0.0, 0.02)
    a = synth.normal_f16(seed, 1, (rows, k), 0.0, 1.0)
    bias = synth.normal_f16(seed, 2, (n,), 0.0, 0.1) if epi != "none" else None
    res = synth.normal_f16(seed, 3, (rows, n), 0.0, 1.0) if epi == "res" else None
    y = torch.empty((rows, n), dtype=torch.float16, device="cuda")
    tod.linear_f16(to_dev(a, torch), to_dev(w, torch), y, bias=to_dev(bias, torch) if bias is not None else None,
                   residual=to_dev(res, torch) if res is not None else None, relu=epi == "relu")
    torch.cuda.synchronize()
    ref = oracle.linear_f16(a, w, bias=bias, residual=res, relu=epi == "relu")
    u = ulps(to_np16(y), ref)
    assert u.max() <= 2, f"max {u.max()} ulp"
    assert (u == 0).mean() > 0.99


@pytest.mark.parametrize("rows", [8, 100, 512])
def test_lm_head_fp16_ragged_vocab(rows):
    """fp16 weights with N = 50272 (not a multiple of the tile), as in the tied LM head."""
    torch = torch_cuda()
    import throughput_oriented_offloaded_amd as tod
    k, n = 768, 50272
    w = synth.normal_f16(21, 0, (n, k), 0.0, 0.02)
    a = synth.normal_f16(21, 1, (rows, k), 0.0, 1.0)
    y = torch.empty((rows, n), dtype=torch.float16, device="cuda")
    tod.linear_f16(to_dev(a, torch), to_dev(w, torch), y)
    torch.cuda.synchronize()
    sample = np.unique(np.array([0, rows // 2, rows - 1]))
    ref = oracle.linear_f16(a[sample], w)
    u = ulps(to_np16(y)[sample], ref)
    assert u.max() <= 2 and (u == 0).mean() > 0.99


@pytest.mark.parametrize("name", ["q_w", "o_w", "fc1_w", "fc2_w"])
def test_full_size_opt30b_decode_gemms(name):
    """OPT-30B decode GEMMs at the block's M = 512 rows, checked on sampled rows.

    QKV uses the [3h][h] shape the decode step launches (q, k, v stacked)."""
    torch = torch_cuda()
    import throughput_oriented_offloaded_amd as tod
    shape = synth.OPT_30B
    print(f"OPT-30B {name} at M=512", flush=True)
    if name == "q_w":
        w = np.concatenate([synth.draw_tensor(shape, t, 0) for t in ("q_w", "k_w", "v_w")])
    else:
        w = synth.draw_tensor(shape, name, 0)
    n, k = w.shape
    rows = 512
    a = synth.normal_f16(31, 0, (rows, k), 0.0, 1.0)
    res = synth.normal_f16(31, 1, (rows, n), 0.0, 1.0) if name in ("o_w", "fc2_w") else None
    bias = synth.normal_f16(31, 2, (n,), 0.0, 0.02)
    codes, scale, zero = _gpu_codes(w, torch)
    y = torch.empty((rows, n), dtype=torch.float16, device="cuda")
    tod.linear_w4(to_dev(a, torch), codes, scale, zero, n, y, bias=to_dev(bias, torch),
                  residual=to_dev(res, torch) if res is not None else None, relu=name == "fc1_w")
    torch.cuda.synchronize()
    sample = np.array([0, 1, 255, 256, 511])
    oc, os_, oz = oracle.quantize_groupwise(w)
    ref = oracle.linear_w4(a[sample], oc, os_, oz, n, bias=bias,
                           residual=res[sample] if res is not None else None, relu=name == "fc1_w")
    u = ulps(to_np16(y)[sample], ref)
    assert u.max() <= 2, f"max {u.max()} ulp"
    assert (u == 0).mean() > 0.99


def test_split_k_is_repeatable():
    """Split-K partials are reduced in a fixed order, so repeated launches give identical bits."""
    torch = torch_cuda()
    import throughput_oriented_offloaded_amd as tod
    rows, k, n = 512, 3072, 768
    a = synth.normal_f16(41, 1, (rows, k), 0.0, 1.0)
    w = synth.normal_f16(41, 2, (n, k), 0.0, 0.02)
    codes, scale, zero = _gpu_codes(w, torch)
    ad = to_dev(a, torch)
    outs = []
    for _ in range(4):
        y = torch.empty((rows, n), dtype=torch.float16, device="cuda")
        tod.linear_w4(ad, codes, scale, zero, n, y)
        torch.cuda.synchronize()
        outs.append(to_np16(y))
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint16), outs[0].view(np.uint16))

