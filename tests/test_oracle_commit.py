"""Pins for the commit rule and the block-diffusion loop.

Expected outcomes are worked out by hand from the rule as the pages state it
(threshold 0.9 plus at least one per step, ties to the smaller position,
forced completion on the last step, committed positions never change) and the
worked example of Module 12, sec. 6.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _c(conf, masked=None, tau=0.9, quota=1, step=0, max_steps=32):
    conf = np.asarray(conf, dtype=np.float32)
    l = conf.size
    masked = np.ones(l, bool) if masked is None else np.asarray(masked, bool)
    canvas = np.where(masked, -1, 7)
    arg = np.arange(100, 100 + l)
    c, m, s, n = oracle.commit(conf, arg, canvas, masked, tau, quota, step, max_steps)
    opened = sorted(np.flatnonzero(masked & ~m).tolist())
    return opened, c, m, s, n


def test_threshold_commits_all_above():
    opened, c, m, s, n = _c([0.95, 0.2, 0.92, 0.1])
    assert opened == [0, 2] and n == 2 and s == 1
    assert c[0] == 100 and c[2] == 102 and c[1] == -1 and c[3] == -1


def test_quota_one_when_none_above_ties_to_lower_position():
    opened, *_ = _c([0.3, 0.5, 0.5, 0.1])
    assert opened == [1]


def test_threshold_is_strict():
    opened, *_ = _c(np.array([0.9, 0.9, 0.1], dtype=np.float32), tau=np.float32(0.9))
    assert opened == [0]        # neither is above 0.9: quota 1, tie -> position 0


def test_only_masked_positions_are_candidates():
    opened, c, *_ = _c([0.99, 0.2, 0.6, 0.1], masked=[False, True, True, True])
    assert opened == [2] and c[0] == 7


def test_quota_larger_than_masked_count():
    opened, *_ = _c([0.1, 0.2, 0.3], masked=[True, False, True], quota=5)
    assert opened == [0, 2]


def test_forced_completion_on_last_step():
    opened, _, m, s, n = _c([0.1, 0.2, 0.3, 0.4], step=15, max_steps=16)
    assert opened == [0, 1, 2, 3] and not m.any() and s == 16


def test_finished_row_is_frozen():
    opened, c, m, s, n = _c([0.99, 0.99], masked=[False, False], step=3)
    assert opened == [] and n == 0 and s == 3


def test_reveal_schedule_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "reveal_schedule.json")))
    assert oracle.linear_mask_schedule(g["length"], g["steps"]) == tuple(g["schedule"])
    # more steps than positions: some calls open nothing
    # ceil(2*3/4)=2, ceil(2*2/4)=1, ceil(2*1/4)=1, 0
    assert oracle.linear_mask_schedule(2, 4) == (2, 2, 1, 1, 0)
    with pytest.raises(ValueError):
        oracle.linear_mask_schedule(0, 3)


def _stub_predictor(peaks, vocab=6, mask_id=0):
    """Logits that do not depend on the input: position j prefers token tok_j with
    a strength peaks[j], so its confidence grows with peaks[j]."""
    peaks = np.asarray(peaks, dtype=np.float64)
    l = peaks.size
    tok = 1 + (np.arange(l) % (vocab - 1))

    def predict(tokens, step):
        logits = np.zeros((l, vocab))
        logits[np.arange(l), tok] = peaks
        logits[:, mask_id] = -np.inf
        return logits
    return predict, tok


def test_fixed_schedule_sampler_opens_by_confidence():
    # Eight positions, four calls, two openings per call (worked example A).
    # Strengths: position -> peak; ranking by confidence is the ranking of peaks:
    # 5 (4.0) > 1 (3.0) > 6 = 2 (2.5, tie -> 2 first) > 0 (2.0) > 7 (1.5) > 3 = 4 (1.0).
    peaks = [2.0, 3.0, 2.5, 1.0, 1.0, 4.0, 2.5, 1.5]
    predict, tok = _stub_predictor(peaks, mask_id=0)
    tokens, trace = oracle.sample_fixed_schedule(predict, 8, 4, mask_id=0)
    assert [t[0] for t in trace] == [(1, 5), (2, 6), (0, 7), (3, 4)]
    np.testing.assert_array_equal(tokens, tok)


def _run_block(conf_fn, l, tau, quota, max_steps):
    """Drive the commit rule over one block with a stub confidence source."""
    canvas = np.full(l, -1)
    masked = np.ones(l, bool)
    step = 0
    history = []
    while masked.any():
        conf, arg = conf_fn(canvas, masked, step)
        canvas_new, masked_new, step, n = oracle.commit(conf, arg, canvas, masked, tau,
                                                        quota, step, max_steps)
        # committed positions never change, the masked count strictly decreases
        assert (canvas_new[~masked] == canvas[~masked]).all()
        assert not (masked_new & ~masked).any()
        assert masked_new.sum() < masked.sum()
        history.append(sorted(np.flatnonzero(masked & ~masked_new).tolist()))
        canvas, masked = canvas_new, masked_new
    return canvas, step, history


def test_threshold_one_quota_one_takes_block_length_steps_in_confidence_order():
    g = np.random.default_rng(0)
    conf = g.random(16).astype(np.float32) * 0.99
    arg = np.arange(16) + 1
    canvas, steps, hist = _run_block(lambda c, m, s: (conf, arg), 16, 1.0, 1, 16)
    assert steps == 16
    assert [h[0] for h in hist] == list(np.argsort(-conf, kind="stable"))


def test_all_confident_commits_whole_block_in_one_step():
    conf = np.full(32, 0.97, dtype=np.float32)
    canvas, steps, hist = _run_block(lambda c, m, s: (conf, np.arange(32) + 1), 32, 0.9, 1, 32)
    assert steps == 1 and hist == [list(range(32))]


def test_forced_completion_when_block_longer_than_step_budget():
    conf = np.linspace(0.1, 0.5, 32).astype(np.float32)
    canvas, steps, hist = _run_block(lambda c, m, s: (conf, np.arange(32) + 1), 32, 0.9, 1, 16)
    assert steps == 16
    assert [len(h) for h in hist] == [1] * 15 + [17]


def test_block_diffusion_threshold_one_takes_exactly_block_length_steps():
    shape = synth.TINY
    w = synth.model_weights(shape, seed=0)
    prompt = synth.prompt(shape, 1, 32, seed=0)[0]
    out, st, cache = oracle.generate_block_diffusion(w, shape, prompt, 32, 16, 16,
                                                     tau=1.0, quota=1)
    assert st.steps_per_block == [16, 16]
    assert st.denoise_nfe == 32 and st.post_block_nfe == 2
    assert st.tokens_per_denoise_forward == 1.0
    assert out.shape == (32,) and (out != shape.mask_id).all()
    assert cache.length == 64


def test_block_diffusion_threshold_fires_with_confident_head():
    shape = synth.TINY
    w = synth.model_weights(shape, seed=0, lm_head_gain=60.0)
    prompt = synth.prompt(shape, 1, 32, seed=0)[0]
    out, st, cache = oracle.generate_block_diffusion(w, shape, prompt, 32, 16, 16, tau=0.9)
    assert st.denoise_nfe < 32                 # some steps commit more than one token
    assert st.accepted_tokens == 32
    # The cache after the run equals a causal prefill of prompt + generated tokens.
    ref, _ = oracle.prefill(w, shape, np.concatenate([prompt, out]))
    np.testing.assert_allclose(cache.k[1], ref.k[1], rtol=1e-11, atol=1e-12)


def test_commit_batch_rows_are_independent():
    conf, arg = synth.confidences(4, 8, 50, seed=1, ties=True)
    canvas = np.full((4, 8), -1)
    masked = np.ones((4, 8), bool)
    masked[2, ::2] = False
    steps = np.array([0, 3, 5, 7])
    c, m, s, n, left = oracle.commit_batch(conf, arg, canvas, masked, 0.9, 1, steps, 8)
    for r in range(4):
        c1, m1, s1, n1 = oracle.commit(conf[r], arg[r], canvas[r], masked[r], 0.9, 1,
                                       steps[r], 8)
        np.testing.assert_array_equal(c[r], c1)
        assert s[r] == s1 and n[r] == n1 and left[r] == m1.sum()
    assert left[3] == 0                         # row 3 was on its last allowed step
