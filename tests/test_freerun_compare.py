"""The end-to-end comparison helpers on the CPU: fed the oracle's own decode
they pass, and a planted mistake in the "device" side (a flipped token, also
at the last clear step, a position committed out of confidence order, a
remasked position, a clearly confident position left masked, a missed quota, an
incomplete last step) fails them.  Hand-built logits check that each kind of
near decision (threshold, selection boundary, token) is flagged as ambiguous.
The decode cases are the ones the GPU free-running tests use."""
import numpy as np
import pytest

import synth
from freerun import check_trajectory_step, compare_until_ambiguity, first_ambiguous, oracle_run

TINY = synth.TINY

# (head gain, weight seed, prompt seed): the oracle commits each block whole in
# one step with every decision clear of the margins (5e-2, widened to twice what
# bf16 storage alone moves each quantity), so the whole decode is compared,
# block 2 reading the cache appended after block 1.  With fewer confident
# positions there is no clear case: at random init the canvas positions'
# confidences are nearly equal, so the oracle's own selection is within the
# margin of another one already at the first step (searched over 6 weight x 16
# prompt seeds at gains 40-200).
CLEAR = [(60.0, 0, 9), (60.0, 1, 0), (60.0, 0, 12)]


def decode(gain, wseed, pseed, n_blocks=2, Lb=16, max_steps=16):
    w = synth.model_weights(TINY, seed=wseed, lm_head_gain=gain)
    prompt = synth.prompt(TINY, 1, 32, seed=pseed)[0]
    return w, prompt, oracle_run(w, TINY, prompt, n_blocks, Lb, max_steps, 0.9)


@pytest.mark.parametrize("case", CLEAR)
def test_clear_cases_compare_whole_blocks_and_catch_a_flipped_token(case):
    _, _, steps = decode(*case)
    canv = [s.canvas_after.copy() for s in steps]
    stop, blocks = compare_until_ambiguity(steps, canv)
    assert stop == len(steps) and blocks == 2
    # flip one committed token of the first block in the "device" copy
    i = 0
    j = int(np.flatnonzero(~steps[i].masked_after)[0])
    bad = [c.copy() for c in canv]
    bad[i][j] = (bad[i][j] + 1) % TINY.vocab or 1
    with pytest.raises(AssertionError):
        compare_until_ambiguity(steps, bad)
    # a device that stops early fails too
    with pytest.raises(AssertionError):
        compare_until_ambiguity(steps, canv[:-1])


@pytest.mark.parametrize("gain,min_exact", [(1.0, 8), (20.0, 28)])
def test_trajectory_check_accepts_the_oracle(gain, min_exact):
    # unit gain is config 1 itself: logits spread ~0.2 and the canvas positions'
    # confidences agree to ~1e-2 in log space, so the oracle's own selection is
    # ambiguous at once and only about a quarter of its tokens have a clear margin
    _, _, steps = decode(gain, 0, 0)
    assert first_ambiguous(steps) < 3
    exact = sum(check_trajectory_step(s.logits, s.canvas_before, s.masked_before, s.canvas_after, s.masked_after,
                                      0.9, 1, s.last, TINY.mask_id) for s in steps)
    assert exact >= min_exact


def test_trajectory_check_catches_planted_mistakes():
    from oracle import confidence
    _, _, steps = decode(20.0, 0, 0)
    flipped = moved = remasked = 0
    for s in steps:
        com = np.flatnonzero(s.masked_before & ~s.masked_after)
        conf, arg = confidence(s.logits)
        fin = np.isfinite(s.logits[0])
        run = lambda c, m: check_trajectory_step(s.logits, s.canvas_before, s.masked_before, c, m, 0.9, 1, s.last,
                                                 TINY.mask_id)
        for j in com:
            top2 = np.sort(s.logits[j][fin])[-2:]
            if top2[1] - top2[0] > 0.2:
                c = s.canvas_after.copy()
                c[j] = int(np.argsort(s.logits[j])[-2])      # the runner-up token
                with pytest.raises(AssertionError):
                    run(c, s.masked_after)
                flipped += 1
        left = np.flatnonzero(s.masked_after)
        if len(com) == 1 and len(left):
            j = int(com[0])
            k = int(left[np.argmin(conf[left])])
            if np.log(conf[j]) - np.log(conf[k]) > 0.06:
                c, m = s.canvas_after.copy(), s.masked_after.copy()
                c[j], m[j] = TINY.mask_id, True
                c[k], m[k] = arg[k], False
                with pytest.raises(AssertionError):
                    run(c, m)
                moved += 1
        kept = np.flatnonzero(~s.masked_before)
        if len(kept):
            c, m = s.canvas_after.copy(), s.masked_after.copy()
            c[kept[0]], m[kept[0]] = TINY.mask_id, True
            with pytest.raises(AssertionError):
                run(c, m)
            remasked += 1
        if len(left) > 1:                                    # two commits where the quota allows one
            c, m = s.canvas_after.copy(), s.masked_after.copy()
            k = int(left[np.argmax(conf[left])])
            if conf[k] < 0.9 - 0.05:
                c[k], m[k] = arg[k], False
                with pytest.raises(AssertionError):
                    run(c, m)
    assert flipped >= 10 and moved >= 5 and remasked >= 20


def _logits(rows):
    """[L, 8] logits, id 0 the mask (-inf); each row (top, second, rest): token 1
    scores top, token 2 second, tokens 3-7 rest."""
    out = np.full((len(rows), 8), -np.inf)
    for i, (top, second, rest) in enumerate(rows):
        out[i, 1], out[i, 2], out[i, 3:] = top, second, rest
    return out


def test_step_ambiguity_flags_each_kind_of_near_decision():
    from freerun import step_ambiguity
    from oracle import confidence
    clear = (10.0, 0.0, 0.0)                     # conf 0.9997, top-2 gap 10
    # a masked position 0.03 from the threshold (conf 0.93: top logit 4.38 above six others)
    lo = _logits([clear, (4.88, 0.5, 0.5), (0.0, -1.0, -1.0)])
    conf, _ = confidence(lo)
    assert abs(conf[1] - 0.93) < 0.01
    assert step_ambiguity(lo, conf, np.array([1, 1, 1], bool), [0], 1, 0.9, False) == ["threshold"]
    # the selection boundary: the committed position and the first one left 0.02 apart in
    # log-confidence, far from the threshold and from the least confident position
    lo = _logits([(1.02, 0.0, 0.0), (1.0, 0.0, 0.0), (0.0, 0.0, 0.0)])
    conf, _ = confidence(lo)
    assert step_ambiguity(lo, conf, np.array([1, 1, 1], bool), [0], 1, 0.9, False) == ["selection"]
    # a committed token whose top two logits are 0.03 apart
    lo = _logits([(10.0, 9.97, 0.0), clear, (0.0, -1.0, -1.0)])
    conf, _ = confidence(lo)
    assert step_ambiguity(lo, conf, np.array([1, 0, 1], bool), [0], 1, 0.9, True) == ["token"]
    # all three clear: nothing flagged
    lo = _logits([clear, (0.0, -1.0, -1.0), (-0.5, -1.0, -1.0)])
    conf, _ = confidence(lo)
    assert step_ambiguity(lo, conf, np.array([1, 1, 1], bool), [0], 1, 0.9, False) == []


def test_trajectory_check_rule_violations():
    # four masked positions: 0 and 1 clearly above the threshold, 2 and 3 far below
    lo = _logits([(10.0, 0.0, 0.0), (9.0, 0.0, 0.0), (0.5, 0.0, 0.0), (0.0, -0.5, -0.5)])
    M = TINY.mask_id
    canvas, masked = np.full(4, M), np.ones(4, bool)
    run = lambda c, m, last=False: check_trajectory_step(lo, canvas, masked, np.array(c), np.array(m, bool), 0.9,
                                                         1, last, M)
    assert run([1, 1, M, M], [0, 0, 1, 1]) == 2                  # the threshold set: allowed
    with pytest.raises(AssertionError, match="clearly above the threshold"):
        run([1, M, M, M], [0, 1, 1, 1])                           # quota met, position 1 left behind
    with pytest.raises(AssertionError, match="quota"):
        run([M, M, M, M], [1, 1, 1, 1])                           # nothing committed
    assert run([1, 1, 1, 1], [0, 0, 0, 0], last=True) == 4       # last step: everything (4 clear tokens)
    with pytest.raises(AssertionError, match="every remaining mask"):
        run([1, 1, 1, M], [0, 0, 0, 1], last=True)                # last step leaving one masked


@pytest.mark.parametrize("case", CLEAR[:1])
def test_compare_checks_the_last_clear_step(case):
    _, _, steps = decode(*case)
    canv = [s.canvas_after.copy() for s in steps]
    stop, _ = compare_until_ambiguity(steps, canv)
    i = stop - 1
    j = int(np.flatnonzero(~steps[i].masked_after)[-1])
    canv[i][j] = (canv[i][j] + 1) % TINY.vocab or 1
    with pytest.raises(AssertionError):
        compare_until_ambiguity(steps, canv)
