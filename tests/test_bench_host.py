"""Host-side logic of bench.py (no GPU): the algorithmic byte counts behind the roofline
figures, the staleness rule for recorded HBM traffic, and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_kv_position_bytes_are_codes_plus_group_parameters():
    """One position of K and V at hidden 7168: 2 x (7168 / 2 code bytes + 7168 / 64 groups x 4 bytes)."""
    shape = synth.WORKLOADS["opt-30b"].shape
    assert bench.kv_bytes_per_position(shape) == 2 * (7168 // 2 + (7168 // 64) * 4)


def test_step_bytes_structure():
    """Rows and context enter only through the cache and the logits: with no rows a step reads the
    int4 weights and the fp16 LM head once; each further attended position adds one K/V position per
    row and layer; each further row adds its cache, its new K/V and its logits."""
    shape = synth.WORKLOADS["opt-30b"].shape
    L, h, f, V = shape.n_layers, shape.hidden, shape.ffn, shape.vocab
    weights = L * (4 * h * h + 2 * f * h) * 0.5625 + V * h * 2
    assert bench.step_bytes(shape, 0, 500) == pytest.approx(weights, rel=1e-12)
    per_pos = bench.kv_bytes_per_position(shape)
    d_ctx = bench.step_bytes(shape, 512, 501) - bench.step_bytes(shape, 512, 500)
    assert d_ctx == pytest.approx(512 * L * per_pos, rel=1e-12)
    d_row = bench.step_bytes(shape, 513, 500) - bench.step_bytes(shape, 512, 500)
    assert d_row == pytest.approx(L * per_pos * 501 + V * 2, rel=1e-12)
    # the benchmark's step at its average context is ~121 GB
    assert 120e9 < bench.step_bytes(shape, 512, 523.5) < 122e9


def test_recorded_traffic_is_reported_only_for_unchanged_sources(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel v1\n")
    summary = tmp_path / "counters.txt"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_FILES", {"k": ("counters.txt", ("kernel.hip",))})
    digest = bench.source_digest(["kernel.hip"])
    summary.write_text(f"header\ntraffic_ratio: 1.25\nsource_sha256: {digest}\n")
    assert bench.measured_traffic("k", 2e9) == pytest.approx(2.5e9)
    assert bench.measured_traffic("other kernel", 2e9) is None
    src.write_text("// kernel v2\n")
    assert bench.measured_traffic("k", 2e9) is None      # sources changed since the counters
    os.remove(summary)
    assert bench.measured_traffic("k", 2e9) is None      # no summary


def test_recorded_attention_traffic_summary_is_well_formed():
    """The committed counter summary carries a ratio near 1 (no re-reads) and a source digest."""
    path, _ = bench.TRAFFIC_FILES["k_attn_decode<128>"]
    with open(os.path.join(ROOT, path)) as f:
        fields = dict(line.split(":", 1) for line in f if line.startswith(("traffic_ratio:", "source_sha256:")))
    assert 1.0 <= float(fields["traffic_ratio"]) < 1.05
    assert len(fields["source_sha256"].strip()) == 64


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
