"""Teacher-forced per-layer parity at full width and full depth.

The GPU runs a whole workload (prefill of every prompt, then one decode step)
with taps on a few layers: the residual-stream rows entering and leaving each
tapped layer are copied out (``set_layer_tap``), and the int4 KV cache the
layer attended over is read back (``export_kv``). The oracle then recomputes
each tapped layer on exactly those inputs: the GPU's input rows and the
GPU's cache (``Layer.forward_given_kv``), so an element-wise bar applies at
any depth. Everything the oracle computes comes from its own weights
(quantized by its own quantizer) and its own arithmetic; the GPU supplies
only the inputs of the function under test.

Checked per tapped layer:
  * decode: the first and last rows of the block at the new position;
  * prefill: sampled positions of the block's last sequence, spanning the
    64-query tiles of the MFMA prefill attention and the causal mask across
    tiles;
  * the int4 codes of the new K/V (the oracle quantizes its own k, v).
Bars (the readings are in the design notes):
  * against the oracle's exact-V reading (attention on zero + c * scale, not
    rounded; the only rounding the GPU's attention leaves out): every
    element within 2 fp16 ulps;
  * against the pages' reading (each V element rounded to fp16 first): the
    two readings differ by up to half an ulp of the largest cached value,
    which the later GEMMs carry forward, so that comparison is reported and
    held to the bound the exact-V difference implies (printed);
  * K/V codes: bit-exact except where the fp16 k or v itself differs by an
    ulp. The quantizer is discontinuous: one ulp on a group's largest or
    smallest value changes its scale and can move every code of the group, up
    to 36 of the 8064 bytes of a position at OPT-30B width. So each checked
    set of positions must agree with the oracle's codes at least as well as
    the fp32-accumulating oracle's codes do on the same inputs, less one
    group's bytes, and never below 0.99 (agreement of both is reported).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import to_dev, to_np16, torch_cuda

pytestmark = pytest.mark.gpu

# (workload, layers: decode count, tapped layers, weight variant, weight tier)
CASES = {
    # the benchmark's own configuration: 48 layers, 512 rows, prompt 512, its plain weights
    "opt-30b": dict(workload="opt-30b", n_layers=None, taps=(0, 23, 47), variant="plain"),
    # OPT-6.7B shape at full depth, full weights (biases and LayerNorm parameters drawn)
    "opt-6.7b": dict(workload="opt-6.7b", n_layers=None, taps=(0, 15, 31), variant="full"),
    # OPT-175B width on its own tier (fp16 weights streamed from pinned host memory), 4 layers
    "opt-175b": dict(workload="opt-175b", n_layers=4, taps=(0, 3), variant="full"),
}
PREFILL_POSITIONS = (0, 1, 63, 64, 65, 127, 200, 383, 447, 448, 510, 511)
ROW_ULP_MAX = 2.0       # every element within 2 fp16 ulps of its row's largest value
MEAN_ABS_FACTOR = 2.0   # mean error at most twice the fp32-accumulating oracle's drift


def _export_cache(tod, torch, m, layer, row, shape, T):
    """The GPU's int4 cache of (layer, block 0, row) for positions 0..T-1, every head,
    as an oracle KVCache, plus the codes of the last position per head."""
    d = shape.head_dim
    cache = oracle.KVCache(shape, T)
    kc = torch.empty((T, d // 2), dtype=torch.uint8, device="cuda")
    vc = torch.empty_like(kc)
    ks, kz, vs, vz = (torch.empty((T, d // 64), dtype=torch.float16, device="cuda") for _ in range(4))
    last = []
    for head in range(shape.n_heads):
        tod.export_kv(m.handle, layer, 0, row, head, 0, T, kc, ks, kz, vc, vs, vz)
        torch.cuda.synchronize()
        arr = (kc.cpu().numpy(), to_np16(ks), to_np16(kz), vc.cpu().numpy(), to_np16(vs), to_np16(vz))
        cache.load(head, 0, *arr)
        last.append(arr)
    return cache, last


def _code_agreement(shape, gpu_arrays, k, v, positions):
    """Fraction of K/V code and parameter bytes equal between the GPU cache at `positions` and the
    oracle's quantization of its own k, v rows (one row per position)."""
    T = len(positions)
    own = oracle.KVCache(shape, T)
    own.store(0, k, v)
    agree = total = 0
    for head, arr in enumerate(gpu_arrays):
        ref = own.export(head, 0, T)
        for x, y in zip(arr, ref):
            x = np.asarray(x)[list(positions)].view(np.uint8)
            y = np.asarray(y).view(np.uint8)
            agree += int((x == y).sum())
            total += x.size
    return agree / total


def _oracle_code_agreement(shape, k_a, v_a, k_b, v_b):
    """Fraction of K/V code and parameter bytes equal between the oracle's quantization of two
    sets of k, v rows (one row per position)."""
    T = k_a.shape[0]
    ca, cb = oracle.KVCache(shape, T), oracle.KVCache(shape, T)
    ca.store(0, k_a, v_a)
    cb.store(0, k_b, v_b)
    agree = total = 0
    for head in range(shape.n_heads):
        for x, y in zip(ca.export(head, 0, T), cb.export(head, 0, T)):
            x, y = np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8)
            agree += int((x == y).sum())
            total += x.size
    ca.close()
    cb.close()
    return agree / total


def _row_ulps(got, ref):
    """|got - ref| in fp16 ulps of each row's largest |ref|: the scale at which the layer's sums
    are carried (a row's small elements come out of sums of terms of that size)."""
    g, r = got.astype(np.float64), ref.astype(np.float64)
    scale = np.spacing(np.abs(r).max(axis=-1, keepdims=True).astype(np.float16)).astype(np.float64)
    return np.abs(g - r) / scale


class Stats:
    """Errors of the GPU and of the fp32-accumulating oracle against the fp64 oracle (exact-V)."""

    def __init__(self):
        self.gpu, self.fp32, self.gpu_abs, self.fp32_abs = [], [], [], []

    def add(self, label, got, ref_x, ref_rounded, ref32):
        g, f = _row_ulps(got, ref_x), _row_ulps(ref32, ref_x)
        ga = np.abs(got.astype(np.float64) - ref_x.astype(np.float64))
        fa = np.abs(ref32.astype(np.float64) - ref_x.astype(np.float64))
        self.gpu.append(g.reshape(-1))
        self.fp32.append(f.reshape(-1))
        self.gpu_abs.append(ga.reshape(-1))
        self.fp32_abs.append(fa.reshape(-1))
        ur = _row_ulps(got, ref_rounded)
        print(f"{label}: GPU vs oracle (exact-V) max {g.max():.2f} / mean {g.mean():.4f} row-ulp, "
              f"{np.mean(ga == 0):.4f} equal, max-abs {ga.max():.3g} | fp32 oracle max {f.max():.2f} / mean "
              f"{f.mean():.4f} row-ulp, {np.mean(fa == 0):.4f} equal | GPU vs rounded-V max {ur.max():.2f} row-ulp",
              flush=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(CASES))
def test_teacher_forced_layers(name):
    torch = torch_cuda()
    import throughput_oriented_offloaded_amd as tod
    case = CASES[name]
    w = synth.WORKLOADS[case["workload"]]
    shape = w.shape if case["n_layers"] is None else w.shape.replace(n_layers=case["n_layers"])
    M, s, h = w.rows, w.prompt_len, shape.hidden
    tier = w.weight_tier
    run = dict(gpu_batch=w.gpu_batch, batches_per_block=w.batches_per_block, prompt_len=s, gen_len=w.gen_len,
               weight_tier=tier)
    print(f"{name}: {shape.n_layers} layers, {M} rows, prompt {s}, tier {tier}, taps {case['taps']}", flush=True)
    m = tod.Model(shape, run)
    glob = synth.global_weights(shape, variant=case["variant"])
    m.set_global_weights(glob["tok_emb"], glob["pos_emb"], glob["lnf_g"], glob["lnf_b"])
    for l in range(shape.n_layers):
        m.set_layer_weights(l, synth.layer_weights(shape, l, variant=case["variant"]))
    pseq = M - 1  # the last sequence of the block's last batch
    bufs = {}
    for l in case["taps"]:
        bufs[l] = [torch.empty((n, h), dtype=torch.float16, device="cuda") for n in (s, s, M, M)]
        tod.set_layer_tap(m.handle, "prefill", l, pseq * s, s, bufs[l][0], bufs[l][1])
        tod.set_layer_tap(m.handle, "decode", l, 0, M, bufs[l][2], bufs[l][3])
    prompts = synth.prompt_ids(M, s, shape.vocab)
    first = torch.empty(M, dtype=torch.int32, device="cuda")
    tod.prefill(m.handle, 0, to_dev(prompts, torch), first)
    out = torch.empty((1, M), dtype=torch.int32, device="cuda")
    tod.decode_block(m.handle, 0, 1, first, out)
    torch.cuda.synchronize()
    print("GPU prefill + 1 decode step done", flush=True)
    st = Stats()
    code_rates = []

    def refs(layer, cache, pos, rows):
        """(fp64 pages' reading, fp64 exact-V, fp32-accumulating exact-V, k, v, and the
        fp32-accumulating oracle's k, v) of one layer."""
        r, k, v = layer.forward_given_kv(cache, pos, rows)
        with oracle.exact_v():
            rx, _, _ = layer.forward_given_kv(cache, pos, rows)
            with oracle.fp32_accumulation():
                r32, k32, v32 = layer.forward_given_kv(cache, pos, rows)
        return r, rx, r32, k, v, k32, v32

    for l in case["taps"]:
        pin, pout, din, dout = (to_np16(b) for b in bufs[l])
        layer = oracle.Layer(shape, synth.layer_weights(shape, l, variant=case["variant"]), int4_weights=tier != 1)
        for row in (0, M - 1):
            cache, arrays = _export_cache(tod, torch, m, l, row, shape, s + 1)
            r, rx, r32, k, v, k32, v32 = refs(layer, cache, s, din[row:row + 1])
            st.add(f"layer {l} decode row {row}", dout[row:row + 1], rx, r, r32)
            code_rates.append((_code_agreement(shape, arrays, k, v, [s]), _oracle_code_agreement(shape, k, v, k32, v32)))
            print(f"layer {l} decode row {row}: new-position K/V byte agreement {code_rates[-1][0]:.5f} "
                  f"(fp32-accumulating oracle {code_rates[-1][1]:.5f})", flush=True)
            if row == pseq:
                parts = [refs(layer, cache, t, pin[t:t + 1]) for t in PREFILL_POSITIONS]
                got = np.concatenate([pout[t:t + 1] for t in PREFILL_POSITIONS])
                st.add(f"layer {l} prefill row {row} positions {PREFILL_POSITIONS}", got,
                       np.concatenate([x[1] for x in parts]), np.concatenate([x[0] for x in parts]),
                       np.concatenate([x[2] for x in parts]))
                k64, v64 = np.concatenate([x[3] for x in parts]), np.concatenate([x[4] for x in parts])
                k32, v32 = np.concatenate([x[5] for x in parts]), np.concatenate([x[6] for x in parts])
                code_rates.append((_code_agreement(shape, arrays, k64, v64, PREFILL_POSITIONS),
                                   _oracle_code_agreement(shape, k64, v64, k32, v32)))
                print(f"layer {l} prefill row {row}: K/V byte agreement {code_rates[-1][0]:.5f} "
                      f"(fp32-accumulating oracle {code_rates[-1][1]:.5f})", flush=True)
            cache.close()
        layer.close()
    m.close()
    g, f = np.concatenate(st.gpu), np.concatenate(st.fp32)
    ga, fa = np.concatenate(st.gpu_abs), np.concatenate(st.fp32_abs)
    print(f"{name}: GPU max {g.max():.2f} row-ulp, mean-abs {ga.mean():.4g}; fp32 oracle max {f.max():.2f} "
          f"row-ulp, mean-abs {fa.mean():.4g}; K/V agreement min {min(c[0] for c in code_rates):.5f} "
          f"(fp32-accumulating oracle min {min(c[1] for c in code_rates):.5f})", flush=True)
    assert g.max() <= ROW_ULP_MAX
    assert ga.mean() <= MEAN_ABS_FACTOR * fa.mean()
    group_bytes = (32 + 4) / (2 * shape.hidden * (0.5 + 4 / 64))  # one group of K or V over a position's bytes
    for gpu_rate, fp32_rate in code_rates:
        assert gpu_rate >= max(0.99, min(0.999, fp32_rate) - group_bytes), (gpu_rate, fp32_rate)
