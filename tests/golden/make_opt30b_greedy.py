"""Write opt30b_greedy.npz and opt30b_greedy.txt: the oracle's greedy generation at full
depth for two sequences of the OPT-30B-shaped decode workload.

The workload is the benchmark's model (48 layers, hidden 7168, 56 heads, the plain
weight draw) and block (64 sequences x 8 batches = 512 rows), with a 16-token prompt
and 8 generated tokens. The sequences are rows 0 and 511 of the block's prompt draw
(synth.prompt_ids(512, 16, vocab)): the first and the last sequence of the zig-zag
block. Each sequence is computed alone; in the oracle's arithmetic a sequence's
results do not depend on the other sequences of its block (the zig-zag and
row-by-row orders give identical outputs).

Runs the oracle only (oracle.Layer, oracle.head, oracle.embed), twice:
  * its default reading, fp64 sums, V cached values rounded to fp16 before the
    weighted sum: tokens and every logit are stored;
  * the same with every running sum rounded to fp32 (oracle.fp32_accumulation),
    fed the first run's tokens: its own argmax per step and the max-abs and
    mean-abs difference of its logits from the first run's (the drift of a
    correct fp32-accumulating implementation on the same inputs) are stored.
The first run is free-running: each generated token is the argmax (lowest index
on ties) of the previous position's logits.

All 48 layers are held at once (about 2.8 GB each, 135 GB in all), so this needs a
host with about 150 GB of memory; about 6 minutes on 16 cores:

    python tests/golden/make_opt30b_greedy.py [output directory]
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
import oracle  # noqa: E402
import synth  # noqa: E402

WORKLOAD = "opt-30b"
PROMPT_LEN = 16
GEN_LEN = 8
ROWS = (0, 511)


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def generate(shape, layers, glob, prompt, forced=None):
    """Greedy generation of one sequence: (argmax tokens [GEN_LEN], logits fp16 [GEN_LEN][V]). With
    `forced`, position prompt_len + i is fed forced[i] instead of the argmax of step i."""
    caches = [oracle.KVCache(shape, PROMPT_LEN + GEN_LEN) for _ in layers]
    tokens, logits = [], []
    ids, pos = np.asarray(prompt, dtype=np.int32), 0
    for step in range(GEN_LEN):
        positions = np.arange(pos, pos + ids.size, dtype=np.int32)
        hid = oracle.embed(shape, glob["tok_emb"], glob["pos_emb"], ids, positions)
        for layer, cache in zip(layers, caches):
            hid = layer.forward(cache, pos, hid)
        lg, nxt = oracle.head(shape, glob["lnf_g"], glob["lnf_b"], glob["tok_emb"], hid[-1:])
        tokens.append(int(nxt[0]))
        logits.append(lg[0].copy())
        pos += ids.size
        ids = np.array([tokens[-1] if forced is None else forced[step]], dtype=np.int32)
        log(f"  step {step}: token {tokens[-1]}")
    for c in caches:
        c.close()
    return np.array(tokens, dtype=np.int32), np.stack(logits)


def main():
    out_dir = sys.argv[1] if len(sys.argv) > 1 else HERE
    w = synth.WORKLOADS[WORKLOAD]
    shape = w.shape
    prompts = synth.prompt_ids(w.rows, PROMPT_LEN, shape.vocab)[list(ROWS)]
    glob = synth.global_weights(shape)
    layers = []
    for l in range(shape.n_layers):
        layers.append(oracle.Layer(shape, synth.layer_weights(shape, l)))
        log(f"layer {l} built")
    tok64, log64, tok32, drift_max, drift_mean = [], [], [], [], []
    for row, prompt in zip(ROWS, prompts):
        log(f"row {row}, fp64 sums")
        t, lg = generate(shape, layers, glob, prompt)
        log(f"row {row}, fp32 sums")
        with oracle.fp32_accumulation():
            t32, lg32 = generate(shape, layers, glob, prompt, forced=t)
        d = np.abs(lg32.astype(np.float64) - lg.astype(np.float64))
        tok64.append(t)
        log64.append(lg)
        tok32.append(t32)
        drift_max.append(d.max(axis=-1))
        drift_mean.append(d.mean(axis=-1))
    for layer in layers:
        layer.close()
    res = dict(rows=np.array(ROWS, dtype=np.int32), prompt_len=np.int32(PROMPT_LEN), gen_len=np.int32(GEN_LEN),
               prompts=prompts.astype(np.int32), tokens=np.stack(tok64), logits=np.stack(log64),
               tokens_fp32=np.stack(tok32), fp32_drift_max=np.stack(drift_max), fp32_drift_mean=np.stack(drift_mean))
    np.savez_compressed(os.path.join(out_dir, "opt30b_greedy.npz"), **res)
    with open(os.path.join(out_dir, "opt30b_greedy.txt"), "w") as f:
        f.write(f"Oracle greedy generation, {WORKLOAD} shape, {shape.n_layers} layers, plain weights, prompt "
                f"{PROMPT_LEN}, {GEN_LEN} tokens, rows {ROWS} of the {w.rows}-row block (tests/golden/"
                f"make_opt30b_greedy.py)\n")
        for i, row in enumerate(ROWS):
            f.write(f"row {row} prompt {prompts[i].tolist()}\n")
            f.write(f"row {row} tokens (fp64 sums) {res['tokens'][i].tolist()}\n")
            f.write(f"row {row} tokens (fp32 sums) {res['tokens_fp32'][i].tolist()}\n")
            f.write(f"row {row} fp32 drift max-abs per step {np.round(res['fp32_drift_max'][i], 4).tolist()}\n")
            f.write(f"row {row} fp32 drift mean-abs per step {np.round(res['fp32_drift_mean'][i], 5).tolist()}\n")
            lg = res["logits"][i].astype(np.float64)
            top2 = np.sort(lg, axis=-1)[:, -2:]
            f.write(f"row {row} top-1 minus top-2 logit per step {np.round(top2[:, 1] - top2[:, 0], 4).tolist()}\n")
            f.write(f"row {row} max |logit| per step {np.round(np.abs(lg).max(axis=-1), 3).tolist()}\n")
    log("written")


if __name__ == "__main__":
    main()
