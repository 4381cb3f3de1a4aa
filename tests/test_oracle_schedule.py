"""Pins of the oracle's schedules and generation loop.

The zig-zag block schedule changes only the order in which (step, layer,
batch) work runs and how often a layer is loaded (FlexGen guide, "2. The
Zig-Zag Block Schedule" and the comparison table's "Weight Reuse per Load"
row); sequences never interact, so every order must give the same bits.
"""
import numpy as np
import pytest

import oracle
import synth

SHAPE = synth.ModelShape(n_layers=3, hidden=128, n_heads=2, head_dim=64, ffn=256, vocab=500, max_pos=64)


@pytest.fixture(scope="module")
def model():
    layers = [oracle.Layer(SHAPE, synth.layer_weights(SHAPE, l, variant="full")) for l in range(SHAPE.n_layers)]
    glob = synth.global_weights(SHAPE, variant="full")
    return layers, glob


def _run(model, prompts, g, K, schedule, forced=None):
    layers, glob = model
    return oracle.generate(SHAPE, layers, glob, prompts, g, K, schedule, forced=forced)


def test_zigzag_equals_row_by_row_bitwise(model):
    K, b, s, g = 3, 2, 7, 5
    prompts = synth.prompt_ids(K * b, s, SHAPE.vocab)
    t0, l0, n0 = _run(model, prompts, g, K, oracle.SCHED_ROW_BY_ROW)
    t1, l1, n1 = _run(model, prompts, g, K, oracle.SCHED_ZIGZAG)
    t2, l2, n2 = _run(model, prompts, g, K, oracle.SCHED_ZIGZAG_ALTERNATE)
    assert np.array_equal(t0, t1) and np.array_equal(t0, t2)
    assert np.array_equal(l0.view(np.uint16), l1.view(np.uint16))
    assert np.array_equal(l0.view(np.uint16), l2.view(np.uint16))
    # weight reuse: row-by-row loads every layer once per (batch, step), zig-zag once per step
    assert n0 == K * g * SHAPE.n_layers
    assert n1 == n2 == g * SHAPE.n_layers
    assert n0 == K * n1


def test_tokens_are_greedy_picks_of_logits(model):
    K, b, s, g = 2, 2, 5, 4
    prompts = synth.prompt_ids(K * b, s, SHAPE.vocab)
    toks, logits, _ = _run(model, prompts, g, K, oracle.SCHED_ZIGZAG)
    for j in range(g):
        lj = logits[j].astype(np.float64)
        assert np.array_equal(toks[:, j], np.argmax(lj, axis=1))


def test_batch_permutation_invariance(model):
    K, b, s, g = 3, 2, 6, 3
    prompts = synth.prompt_ids(K * b, s, SHAPE.vocab)
    perm = np.array([4, 5, 0, 1, 2, 3])        # rotate whole batches
    t0, l0, _ = _run(model, prompts, g, K, oracle.SCHED_ZIGZAG)
    t1, l1, _ = _run(model, prompts[perm], g, K, oracle.SCHED_ZIGZAG)
    assert np.array_equal(t0[perm], t1)
    assert np.array_equal(l0[:, perm].view(np.uint16), l1.view(np.uint16))


def test_teacher_forcing_with_own_tokens_is_identity(model):
    K, b, s, g = 1, 3, 6, 4
    prompts = synth.prompt_ids(K * b, s, SHAPE.vocab)
    t0, l0, _ = _run(model, prompts, g, K, oracle.SCHED_ZIGZAG)
    t1, l1, _ = _run(model, prompts, g, K, oracle.SCHED_ZIGZAG, forced=t0[:, :g - 1])
    assert np.array_equal(t0, t1) and np.array_equal(l0.view(np.uint16), l1.view(np.uint16))


def test_incremental_decode_equals_one_pass_over_the_sequence(model):
    """Prefill + teacher-forced decode equals one pass over all positions (layer-streamed)."""
    layers, glob = model
    K, b, s, g = 1, 2, 6, 4
    prompts = synth.prompt_ids(K * b, s, SHAPE.vocab)
    toks, logits, _ = _run(model, prompts, g, K, oracle.SCHED_ZIGZAG)
    for r in range(b):
        ids = np.concatenate([prompts[r], toks[r, :g - 1]])
        lg, nx = oracle.teacher_forced_logits(
            SHAPE, lambda l: synth.layer_weights(SHAPE, l, variant="full"), glob, ids, s - 1)
        assert np.array_equal(lg.view(np.uint16), logits[:, r].view(np.uint16))
        assert np.array_equal(nx, toks[r])


def test_bad_arguments_rejected(model):
    prompts = synth.prompt_ids(4, 5, SHAPE.vocab)
    with pytest.raises(ValueError):
        _run(model, prompts, 3, 3, oracle.SCHED_ZIGZAG)          # 4 rows not divisible into 3 batches
    with pytest.raises(ValueError):
        _run(model, prompts, 70, 2, oracle.SCHED_ZIGZAG)         # beyond the position table
