"""Closed-form I/O cost model of offloaded generation (plain Python).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``.

Two models are given:

* ``p1_naive`` / ``p1_zigzag`` restate the toy simulator of the FlexGen guide
  ("Implementation: Simulating FlexGen's Zig-Zag Block Scheduling in Python",
  Steps 1-3): transfer time = output tokens x model GB / PCIe GB/s and
  throughput = batch x tokens / transfer time. As printed, both schedules use
  that same formula and differ only in the batch they are given (4 against
  128), and the micro-batch count is not used; the printed result is
  1.83 against 58.51 tokens/s, a ratio of 32.0.
* ``weight_bytes`` counts layer loads the way the zig-zag block schedule
  defines them (FlexGen guide, "2. The Zig-Zag Block Schedule", and the
  comparison table's "Weight Reuse per Load" row): with K micro-batches per
  block, row-by-row execution streams the model once per micro-batch per
  token, the zig-zag schedule once per token for the whole block, so
  row-by-row moves K times the bytes.
"""
from __future__ import annotations

PCIE_GB_S = 16.0  # simulator's PCIe constant (guide, Step 1)


def p1_naive(batch: int, output_tokens: int, model_gb: float = 35.0, pcie_gb_s: float = PCIE_GB_S) -> float:
    io_s = output_tokens * model_gb / pcie_gb_s
    return batch * output_tokens / io_s


def p1_zigzag(batch: int, output_tokens: int, micro_batches: int = 4, model_gb: float = 35.0,
              pcie_gb_s: float = PCIE_GB_S) -> float:
    del micro_batches  # unused by the printed simulator
    io_s = output_tokens * model_gb / pcie_gb_s
    return batch * output_tokens / io_s


def weight_bytes(model_bytes: float, tokens: int, micro_batches: int, schedule: str) -> float:
    """Weight bytes moved to generate ``tokens`` tokens for a block of ``micro_batches`` batches."""
    if schedule == "row_by_row":
        return model_bytes * tokens * micro_batches
    if schedule == "zigzag":
        return model_bytes * tokens
    raise ValueError(schedule)


def throughput(model_bytes: float, link_bytes_s: float, tokens: int, batch: int, micro_batches: int,
               schedule: str) -> float:
    """Tokens/s when the link is the only cost: block of ``micro_batches`` batches of ``batch`` rows."""
    t = weight_bytes(model_bytes, tokens, micro_batches, schedule) / link_bytes_s
    return batch * micro_batches * tokens / t
