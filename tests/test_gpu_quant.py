"""GPU quantizer parity: bit-exact codes, scales and zeros against the oracle."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import to_dev, torch_cuda
from tests.quant_cases import adversarial_groups

pytestmark = pytest.mark.gpu


def _gpu_quant(x16):
    torch = torch_cuda()
    import throughput_oriented_offloaded_amd as tod
    n = x16.size
    xd = to_dev(x16.reshape(-1), torch)
    codes = torch.empty(n // 2, dtype=torch.uint8, device="cuda")
    scale = torch.empty(n // 64, dtype=torch.float16, device="cuda")
    zero = torch.empty(n // 64, dtype=torch.float16, device="cuda")
    tod.quantize_groupwise(xd, codes, scale, zero)
    torch.cuda.synchronize()
    return (codes.cpu().numpy(), scale.view(torch.int16).cpu().numpy().view(np.uint16),
            zero.view(torch.int16).cpu().numpy().view(np.uint16))


def _assert_bit_exact(x16):
    gc, gs, gz = _gpu_quant(x16)
    oc, os_, oz = oracle.quantize_groupwise(x16)
    assert np.array_equal(gs, os_.view(np.uint16)), "scales differ"
    assert np.array_equal(gz, oz.view(np.uint16)), "zeros differ"
    assert np.array_equal(gc, oc), f"codes differ at {np.count_nonzero(gc != oc)} bytes"


@pytest.mark.parametrize("sigma", [0.02, 1.0])
def test_quantize_normal_bit_exact(sigma):
    print(f"quantize N(0,{sigma}) 64 x 50003 groups", flush=True)
    _assert_bit_exact(synth.normal_f16(11, 0, 64 * 50003, 0.0, sigma))


def test_quantize_adversarial_bit_exact():
    _assert_bit_exact(adversarial_groups())


def test_quantize_one_group_and_empty():
    _assert_bit_exact(synth.normal_f16(12, 0, 64))
    torch = torch_cuda()
    import throughput_oriented_offloaded_amd as tod
    e = torch.empty(0, dtype=torch.float16, device="cuda")
    tod.quantize_groupwise(e, torch.empty(0, dtype=torch.uint8, device="cuda"), e, e)
    with pytest.raises(tod.TodError):
        tod.quantize_groupwise(torch.empty(96, dtype=torch.float16, device="cuda"),
                               torch.empty(48, dtype=torch.uint8, device="cuda"), e, e)


def test_dequantize_matches_oracle():
    torch = torch_cuda()
    import throughput_oriented_offloaded_amd as tod
    x = synth.normal_f16(13, 0, 64 * 4099, 0.0, 0.02)
    oc, os_, oz = oracle.quantize_groupwise(x)
    out = torch.empty(x.size, dtype=torch.float16, device="cuda")
    tod.dequantize_groupwise(to_dev(oc, torch), to_dev(os_, torch), to_dev(oz, torch), x.size, out)
    torch.cuda.synchronize()
    ref = oracle.dequantize_groupwise(oc, os_, oz)
    assert np.array_equal(out.view(torch.int16).cpu().numpy(), ref.view(np.int16))


def test_quantize_full_size_opt30b_fc1():
    """The largest int4 matrix of the OPT-30B shape: fc1 [28672][7168], 205 M elements."""
    print("quantize OPT-30B fc1 28672x7168", flush=True)
    x = synth.draw_tensor(synth.OPT_30B, "fc1_w", 0)
    _assert_bit_exact(x)
