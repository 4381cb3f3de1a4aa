"""Pins of the closed-form cost model against the FlexGen guide's printed simulator output."""
import os

import pytest

from oracle import costmodel

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "p1_simulator.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            vals[k] = float(v)
    return vals


def test_printed_simulator_values():
    g = _golden()
    naive = costmodel.p1_naive(4, 64)
    flex = costmodel.p1_zigzag(128, 64, micro_batches=8)
    assert round(naive, 2) == g["naive_tokens_per_s"]
    assert round(flex, 2) == g["flexgen_tokens_per_s"]
    assert round(flex / naive, 1) == g["multiplier"]
    # the printed ratio is just the ratio of batch sizes
    assert flex / naive == pytest.approx(128 / 4)


def test_load_counting_model():
    W = 35e9
    assert costmodel.weight_bytes(W, 64, 8, "row_by_row") == 8 * costmodel.weight_bytes(W, 64, 8, "zigzag")
    t_rr = costmodel.throughput(W, 16e9, 64, 16, 8, "row_by_row")
    t_zz = costmodel.throughput(W, 16e9, 64, 16, 8, "zigzag")
    assert t_zz / t_rr == pytest.approx(8.0)
    with pytest.raises(ValueError):
        costmodel.weight_bytes(W, 1, 1, "column")


def test_int4_compression_ratio():
    """4 bits per value plus an fp16 scale and an fp16 zero per 64 values: 16 / 4.5 = 3.56x, not 4x."""
    bits_per_value = 4 + (16 + 16) / 64
    assert 16 / bits_per_value == pytest.approx(3.5556, abs=1e-4)
