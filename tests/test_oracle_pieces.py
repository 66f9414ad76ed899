"""Pins for the oracle's building blocks: closed forms and hand-computed values.

Nothing here re-types the oracle's formula: every expected value is either a
number worked out by hand (written next to it), a property that any correct
implementation has (norm preservation, relative-position invariance), or a
special case that reduces to something simpler (one visible key, equal scores).
"""
import math

import numpy as np
import pytest

import oracle


# ---------------------------------------------------------------- RMSNorm ----

def test_rms_norm_hand_values():
    # mean(x^2) of [1,2,3,4] is 30/4 = 7.5, sqrt(7.5) = 2.7386127875258306
    y = oracle.rms_norm(np.array([1.0, 2.0, 3.0, 4.0]), np.ones(4), 0.0)
    np.testing.assert_allclose(y, [0.3651483716701107, 0.7302967433402214,
                                   1.0954451150103321, 1.4605934866804429], rtol=1e-14)


def test_rms_norm_eps_inside_sqrt_and_gain():
    # x = 1e-3 everywhere: 1e-3 / sqrt(1e-6 + 1e-5) = 0.30151134457776363
    y = oracle.rms_norm(np.full(4, 1e-3), np.ones(4), 1e-5)
    np.testing.assert_allclose(y, 0.30151134457776363, rtol=1e-13)
    # per-channel gains multiply the normalised value
    y = oracle.rms_norm(np.array([3.0, 4.0]), np.array([2.0, -1.0]), 0.0)
    # rms = sqrt(12.5) = 3.5355339059327378
    np.testing.assert_allclose(y, [2 * 3 / 3.5355339059327378, -4 / 3.5355339059327378])


def test_silu_values():
    np.testing.assert_allclose(oracle.silu(np.array([0.0, 1.0, -1.0, 40.0])),
                               [0.0, 0.7310585786300049, -0.2689414213699951, 40.0],
                               rtol=1e-12)


# ------------------------------------------------------------------- RoPE ----

def test_rope_rotate_half_pairing_hand_values():
    # hd = 4, base 10000: frequencies [1, 10000^-0.5 = 0.01]; pairs (0,2) and (1,3).
    p = 3.0
    e = np.eye(4)[:, None, :]                   # four unit vectors, T = 1
    out = oracle.rope(e, np.array([p]), 10000.0)[:, 0, :]
    np.testing.assert_allclose(out[0], [math.cos(p), 0, math.sin(p), 0], atol=1e-15)
    np.testing.assert_allclose(out[1], [0, math.cos(0.01 * p), 0, math.sin(0.01 * p)],
                               atol=1e-15)
    np.testing.assert_allclose(out[2], [-math.sin(p), 0, math.cos(p), 0], atol=1e-15)
    np.testing.assert_allclose(out[3], [0, -math.sin(0.01 * p), 0, math.cos(0.01 * p)],
                               atol=1e-15)


def test_rope_identity_norm_and_relative_position():
    g = np.random.default_rng(0)
    q = g.standard_normal((1, 32))
    k = g.standard_normal((1, 32))
    np.testing.assert_allclose(oracle.rope(q, np.array([0]), 1e4), q, atol=0)
    for base in (1e4, 1e6):
        for m, n in [(5, 2), (100, 37), (4000, 4095)]:
            qm = oracle.rope(q, np.array([m]), base)
            kn = oracle.rope(k, np.array([n]), base)
            assert np.isclose(np.linalg.norm(qm), np.linalg.norm(q), rtol=1e-13)
            rel = oracle.rope(q, np.array([m - n]), base) if m >= n else None
            if rel is not None:
                assert np.isclose((qm * kn).sum(), (rel * k).sum(), rtol=1e-9, atol=1e-11)


# -------------------------------------------------------------- attention ----

def test_attend_two_keys_hand_value():
    # hd = 2: score of key 0 is 1/sqrt(2), key 1 is 0.
    # p0 = e^0.70710678 / (e^0.70710678 + 1) = 0.6697615493266569
    q = np.array([[[1.0, 0.0]]])
    k = np.array([[[1.0, 0.0], [0.0, 0.0]]])
    v = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    o = oracle.attend(q, k, v, np.ones((1, 2), bool))
    np.testing.assert_allclose(o[0, 0], [0.6697615493266569, 0.3302384506733431], rtol=1e-13)


def test_attend_single_visible_key_and_uniform_scores():
    g = np.random.default_rng(1)
    q = g.standard_normal((2, 3, 8))
    k = g.standard_normal((2, 5, 8))
    v = g.standard_normal((2, 5, 8))
    allowed = np.zeros((3, 5), bool)
    allowed[0, 2] = allowed[1, 4] = allowed[2, 0] = True
    o = oracle.attend(q, k, v, allowed)
    np.testing.assert_allclose(o[:, 0], v[:, 2])
    np.testing.assert_allclose(o[:, 1], v[:, 4])
    np.testing.assert_allclose(o[:, 2], v[:, 0])
    # zero queries: equal scores, so each output is the plain mean of the visible values
    causal = np.tril(np.ones((5, 5), bool))
    o = oracle.attend(np.zeros((2, 5, 8)), k, v, causal)
    for t in range(5):
        np.testing.assert_allclose(o[:, t], v[:, : t + 1].mean(axis=1), rtol=1e-13)


def test_attend_gqa_head_to_group_mapping():
    # 4 query heads, 2 KV heads; KV head g holds constant value g+1.
    # Heads 0,1 must read KV head 0 and heads 2,3 KV head 1.
    k = np.zeros((2, 3, 4))
    v = np.stack([np.full((3, 4), 1.0), np.full((3, 4), 2.0)])
    q = np.random.default_rng(2).standard_normal((4, 2, 4))
    o = oracle.attend(q, k, v, np.ones((2, 3), bool))
    np.testing.assert_allclose(o[:2], 1.0)
    np.testing.assert_allclose(o[2:], 2.0)


def test_attend_gqa_equals_mha_with_repeated_kv():
    g = np.random.default_rng(3)
    q = g.standard_normal((4, 6, 8))
    k = g.standard_normal((2, 6, 8))
    v = g.standard_normal((2, 6, 8))
    mask = np.tril(np.ones((6, 6), bool))
    o1 = oracle.attend(q, k, v, mask)
    o2 = oracle.attend(q, np.repeat(k, 2, axis=0), np.repeat(v, 2, axis=0), mask)
    np.testing.assert_allclose(o1, o2, rtol=1e-14)


# ------------------------------------------------------------- confidence ----

def test_confidence_hand_values_and_mask_exclusion():
    # vocab 3, mask id 0: logits (-inf, ln 3, 0) -> probabilities (0, 3/4, 1/4)
    conf, arg = oracle.confidence(np.array([[-np.inf, math.log(3.0), 0.0]]))
    assert arg[0] == 1
    np.testing.assert_allclose(conf[0], 0.75, rtol=1e-15)


def test_confidence_equal_logits_lowest_id():
    # V = 5 with the mask (id 0) excluded: four equal logits -> conf 1/4, argmax 1
    conf, arg = oracle.confidence(np.array([[-np.inf, 2.0, 2.0, 2.0, 2.0]]))
    assert arg[0] == 1 and conf[0] == 0.25
    conf, arg = oracle.confidence(np.array([[0.0, 5.0, 7.0, 7.0]]))
    assert arg[0] == 2


def test_confidence_rejects_nan():
    with pytest.raises(ValueError):
        oracle.confidence(np.array([[0.0, np.nan]]))
    with pytest.raises(ValueError):
        oracle.confidence(np.array([[0.0, np.inf]]))


def test_attend_refuses_a_query_that_sees_no_key():
    # softmax over no visible key is 0/0: the oracle refuses it instead of returning NaN
    q = np.ones((1, 2, 4))
    k = v = np.ones((1, 3, 4))
    allowed = np.array([[True, False, False], [False, False, False]])
    with pytest.raises(ValueError):
        oracle.attend(q, k, v, allowed)
