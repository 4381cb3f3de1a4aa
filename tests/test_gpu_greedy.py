"""Greedy decoding at full depth: the benchmark's model and block against a stored oracle run.

The GPU runs the OPT-30B-shaped decode workload as the benchmark does (48
layers, the plain weight draw, 64 sequences x 8 batches = 512 rows, int4
weights and KV cache in HBM) with a 16-token prompt and 8 generated tokens.
Rows 0 and 511, the first and the last sequence of the zig-zag block, are
compared with the oracle's greedy generation of the same two prompts, stored
in tests/golden/opt30b_greedy.npz by tests/golden/make_opt30b_greedy.py. That
script calls only the oracle; holding all 48 oracle layers takes ~135 GB of
host memory, so the run is stored rather than repeated here.

The two rows are fed the oracle's own tokens (teacher-forced; the other 510
rows follow their own picks), so every step compares the same history.

What the stored run shows about this stack: at 48 layers a correct
implementation that accumulates in fp32 (the oracle with every running sum
rounded to fp32, fed the same tokens) already differs from the fp64 oracle by
0.58-0.80 max-abs and ~0.12 mean-abs on logits of magnitude ~7, and its argmax
differs in 5 of the 16 steps: the int4 KV quantizer is discontinuous, and a
random-weight stack amplifies a one-ulp difference layer after layer. So the
stated logit bar (max-abs 2e-2 / mean-abs 2e-3) and identical ids cannot hold
here for any fp32 implementation; the element-wise check at this depth is the
per-layer teacher-forced test (tests/test_gpu_layers.py). This test holds the
GPU to the fp32 implementation's drift:
  * logits: max-abs <= 2 x and mean-abs <= 1.5 x the fp32-accumulating
    oracle's drift from the fp64 oracle on the same tokens (stored per step);
  * greedy ids: equal to the oracle's, or with an oracle logit within that
    max-abs bar of the oracle's best (tie-aware); the count of identical ids
    is printed next to the fp32-accumulating oracle's own count.
"""
import os

import numpy as np
import pytest

import synth
from tests.gpu_util import to_dev, to_np16, torch_cuda

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "opt30b_greedy.npz")


def test_opt30b_full_depth_teacher_forced_against_the_oracle():
    torch = torch_cuda()
    import throughput_oriented_offloaded_amd as tod
    ref = np.load(GOLDEN)
    w = synth.WORKLOADS["opt-30b"]
    shape = w.shape
    rows = [int(r) for r in ref["rows"]]
    P, G = int(ref["prompt_len"]), int(ref["gen_len"])
    prompts = synth.prompt_ids(w.rows, P, shape.vocab)
    assert np.array_equal(prompts[rows], ref["prompts"]), "the stored run was made from another prompt draw"
    ot, ol = ref["tokens"], ref["logits"]                  # [rows][G], [rows][G][V]
    drift_max, drift_mean = ref["fp32_drift_max"], ref["fp32_drift_mean"]
    print(f"opt-30b shape, {shape.n_layers} layers, {w.rows} rows, prompt {P}, {G} tokens; rows {rows}", flush=True)

    run = dict(gpu_batch=w.gpu_batch, batches_per_block=w.batches_per_block, prompt_len=P, gen_len=G)
    m = tod.Model(shape, run)
    g = synth.global_weights(shape)
    m.set_global_weights(g["tok_emb"], g["pos_emb"], g["lnf_g"], g["lnf_b"])
    for l in range(shape.n_layers):
        m.set_layer_weights(l, synth.layer_weights(shape, l))
    M, V = w.rows, shape.vocab
    picks = torch.empty((G, M), dtype=torch.int32, device="cuda")
    logits = torch.empty((G, M, V), dtype=torch.float16, device="cuda")
    tod.prefill(m.handle, 0, to_dev(prompts, torch), picks[0], logits[0])
    forced = torch.from_numpy(np.ascontiguousarray(ot)).cuda()
    ids = torch.empty((G, M), dtype=torch.int32, device="cuda")
    for j in range(1, G):
        ids[j].copy_(picks[j - 1])
        ids[j, rows] = forced[:, j - 1]   # the oracle's token of the previous step
        tod.decode_block(m.handle, 0, 1, ids[j], picks[j:j + 1], logits[j:j + 1])
    torch.cuda.synchronize()
    gp = picks.cpu().numpy()[:, rows].T                    # [rows][G]
    gl = np.stack([to_np16(logits[:, r]) for r in rows])   # [rows][G][V]
    m.close()

    for i, row in enumerate(rows):
        d = np.abs(gl[i].astype(np.float64) - ol[i].astype(np.float64))
        max_bar = 2.0 * float(drift_max[i].max())
        mean_bar = 1.5 * float(drift_mean[i].mean())
        same, ties = 0, 0
        for j in range(G):
            best, pick = int(ot[i, j]), int(gp[i, j])
            gap = float(ol[i, j, best]) - float(ol[i, j, pick])
            print(f"row {row} step {j}: GPU {pick} oracle {best} (oracle gap {gap:.4g}); logits max-abs "
                  f"{d[j].max():.4g} mean-abs {d[j].mean():.4g}; fp32-oracle drift {drift_max[i, j]:.4g} / "
                  f"{drift_mean[i, j]:.4g}", flush=True)
            if pick == best:
                same += 1
            else:
                assert gap <= max_bar, (row, j, pick, best, gap, max_bar)
                ties += 1
        own32 = int((ref["tokens_fp32"][i] == ot[i]).sum())
        print(f"row {row}: greedy ids identical at {same} of {G} steps ({ties} within the bar; the fp32-accumulating "
              f"oracle: {own32} of {G}); logits max-abs {d.max():.4g} (stated 2e-2, bar {max_bar:.4g}) mean-abs "
              f"{d.mean():.4g} (stated 2e-3, bar {mean_bar:.4g})", flush=True)
        assert d.max() <= max_bar
        assert d.mean() <= mean_bar
