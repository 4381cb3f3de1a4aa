"""Write fullsize_kv_calibration.txt: how closely a correct fp32-accumulating
implementation reproduces the fp64 oracle's int4 K/V codes of layers 0 and 1
for the last sequence of the OPT-30B-shaped benchmark block (512-token prompt).

Runs the oracle only (fp64, then with every running sum rounded to fp32 via
oracle.fp32_accumulation) over the prompt's 512 positions of layers 0 and 1,
and compares the exported codes, scales and zeros of heads 0, 28 and 55 byte by
byte. Takes about 15 minutes on 8 cores:

    python tests/golden/calibrate_fullsize_kv.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
import oracle  # noqa: E402
import synth  # noqa: E402


def kv_caches(shape, glob, ids, fp32):
    T = ids.size
    hid = oracle.embed(shape, glob["tok_emb"], glob["pos_emb"], ids, np.arange(T, dtype=np.int32))
    caches = []
    for layer in (0, 1):
        lo = oracle.Layer(shape, synth.layer_weights(shape, layer))
        c = oracle.KVCache(shape, T)
        if fp32:
            with oracle.fp32_accumulation():
                hid = lo.forward(c, 0, hid)
        else:
            hid = lo.forward(c, 0, hid)
        caches.append(c)
        del lo
    return caches


def main():
    w = synth.WORKLOADS["opt-30b"]
    shape, M, s = w.shape, w.rows, w.prompt_len
    glob = synth.global_weights(shape)
    row = M - 1
    ids = synth.prompt_ids(M, s, shape.vocab)[row].astype(np.int32)
    ref, f32 = kv_caches(shape, glob, ids, False), kv_caches(shape, glob, ids, True)
    heads = (0, shape.n_heads // 2, shape.n_heads - 1)
    lines = ["# fp64 oracle vs fp32-accumulating oracle: int4 K/V byte agreement (codes, scales, zeros)",
             f"# workload opt-30b, row {row}, positions 0..{s - 1}, heads {heads}; written by calibrate_fullsize_kv.py"]
    for layer in (0, 1):
        agree = total = 0
        for head in heads:
            for x, y in zip(ref[layer].export(head, 0, s), f32[layer].export(head, 0, s)):
                x, y = np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8)
                agree += int((x == y).sum())
                total += x.size
        lines.append(f"layer{layer}_fp32_agreement: {agree / total:.6f}")
    with open(os.path.join(HERE, "fullsize_kv_calibration.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
