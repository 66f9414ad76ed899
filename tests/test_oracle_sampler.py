"""Pins of the oracle's sampler variants: entropy, the bounded and entropy-bound
commit rules, the per-step cap and adaptive stopping (MLX guide, sec. 5.2 and
5.5; DiffusionGemma docs, Schedulers and adaptive stopping)."""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_entropy_closed_forms():
    V = 10
    lg = np.zeros((1, V))
    lg[0, 3] = -np.inf                                   # the mask id
    assert oracle.entropy(lg)[0] == pytest.approx(math.log(V - 1), rel=1e-12)
    for d in (0.0, 0.7, 3.0):                            # two-way split: binary entropy
        p = 1.0 / (1.0 + math.exp(-d))
        want = -p * math.log(p) - (1 - p) * math.log(1 - p)
        assert oracle.entropy([[d, 0.0, -np.inf]])[0] == pytest.approx(want, rel=1e-12)
    assert oracle.entropy([[60.0, 0.0, 0.0, 0.0]])[0] < 1e-20  # one dominant logit
    with pytest.raises(ValueError):
        oracle.entropy([[0.0, np.nan]])


def test_entropy_of_a_shifted_row_is_unchanged():
    rng = np.random.default_rng(0)
    lg = rng.normal(size=(5, 40))
    np.testing.assert_allclose(oracle.entropy(lg), oracle.entropy(lg + 123.0), rtol=1e-12)


def _golden():
    return json.load(open(os.path.join(GOLDEN, "sampler_rules.json")))


@pytest.mark.parametrize("case", _golden()["cases"], ids=lambda c: c["name"][:40])
def test_commit_rule_golden(case):
    conf = np.asarray(case["conf"], dtype=np.float32)
    L = len(conf)
    arg = np.arange(100, 100 + L)
    canvas = np.zeros(L, dtype=np.int64)
    masked = np.ones(L, dtype=bool)
    kw = dict(rule=case["rule"], max_transfer=case["max_transfer"])
    if "entropy" in case:
        kw.update(entropy=np.asarray(case["entropy"], dtype=np.float32), entropy_bound=case["entropy_bound"])
    c, m, s, n = oracle.commit_rule(conf, arg, canvas, masked, case["tau"], case["quota"], case["step"],
                                    case["max_steps"], **kw)
    opened = np.flatnonzero(~m).tolist()
    assert opened == case["committed"]
    assert n == len(opened) and s == case["step"] + 1
    np.testing.assert_array_equal(c[opened], arg[opened])


def test_adaptive_stop_golden():
    g = _golden()["adaptive_stop"]
    prev = np.full(3, -1)
    stable = 0
    masked = np.ones(3, dtype=bool)
    for t, (a, e) in enumerate(zip(g["argmax"], g["entropy"])):
        stop, stable = oracle.adaptive_stop(a, prev, masked, np.asarray(e, np.float32), stable,
                                            g["stability_steps"], g["stop_entropy"])
        assert (stop, stable) == (g["stop"][t], g["stable"][t])
        prev = np.asarray(a)
        if t == len(g["argmax"]) - 1:
            hi, _ = oracle.adaptive_stop(a, prev, masked, np.asarray(g["high_entropy"], np.float32),
                                         g["stable"][t - 1], g["stability_steps"], g["stop_entropy"])
            assert not hi
    # a changed argmax resets the count
    _, st = oracle.adaptive_stop([7, 8, 1], np.array([7, 8, 9]), masked, np.zeros(3, np.float32), 5, 2, 0.005)
    assert st == 0


def test_native_rule_equals_commit():
    rng = np.random.default_rng(1)
    for trial in range(300):
        L = int(rng.integers(1, 10))
        conf = rng.choice([0.1, 0.5, 0.9, 0.95, 1.0], size=L).astype(np.float32)
        arg = rng.integers(0, 50, size=L)
        masked = rng.random(L) < 0.7
        canvas = np.where(masked, -1, rng.integers(0, 50, size=L))
        tau, quota, step = float(rng.choice([0.5, 0.9, 1.0])), int(rng.integers(1, 4)), int(rng.integers(0, 4))
        a = oracle.commit(conf, arg, canvas, masked, tau, quota, step, 4)
        b = oracle.commit_rule(conf, arg, canvas, masked, tau, quota, step, 4, rule="threshold")
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)


def test_rules_brute_force_properties():
    rng = np.random.default_rng(2)
    for trial in range(400):
        L = int(rng.integers(1, 9))
        conf = rng.choice([0.1, 0.3, 0.46, 0.5, 0.62, 0.8, 0.9, 0.97], size=L).astype(np.float32)
        ent = rng.choice([0.0, 0.01, 0.02, 0.05, 0.2], size=L).astype(np.float32)
        masked = rng.random(L) < 0.8
        arg = np.arange(L) + 10
        quota, cap = int(rng.integers(1, 3)), int(rng.integers(0, 3))
        idx = np.flatnonzero(masked)
        for rule in oracle.RULES:
            _, m, _, n = oracle.commit_rule(conf, arg, np.zeros(L, int), masked, 0.9, quota, 0, 8, rule=rule,
                                            entropy=ent, entropy_bound=0.04, max_transfer=cap)
            chosen = set(np.flatnonzero(masked & ~m).tolist())
            assert n == len(chosen) and chosen <= set(idx.tolist())
            if idx.size == 0:
                assert n == 0
                continue
            if rule == "entropy":
                key = lambda j: (float(ent[j]), j)
                A, tot = [], np.float32(0)
                for j in sorted(idx, key=key):
                    tot = np.float32(tot + ent[j])
                    if tot > np.float32(0.04):
                        break
                    A.append(j)
            else:
                key = lambda j: (-float(conf[j]), j)
                if rule == "threshold":
                    A = [j for j in idx if conf[j] > np.float32(0.9)]
                else:
                    A = [j for j in idx if conf[j] >= np.float32(0.9) or
                         (conf[j] >= np.float32(0.45) and conf[j] >= np.float32(1) - np.float32(2) / np.float32(j + 2))]
            want = max(len(A), min(quota, idx.size))
            if cap:
                want = min(want, cap)
            assert n == want
            # the chosen set is the best-ranked among the qualifying positions, then the rest
            order = sorted(idx, key=key)
            pool = sorted(A, key=key) + [j for j in order if j not in A]
            if len(A) >= min(quota, idx.size):
                assert chosen == set(sorted(A, key=key)[:want])
            else:
                assert chosen == set(pool[:want])


def test_bound_rule_reaches_the_global_threshold():
    # MLX guide, sec. 5.2: under the bounded sampler a token qualifies when its
    # confidence reaches the global threshold (0.9), or is not below min_threshold
    # (0.45) and not below the position threshold 1 - 2 / (pos + 2).  Positions 21
    # and 22 hold exactly 0.9 where the position threshold is above it (0.913,
    # 0.917), so they qualify through the global threshold alone, and both open
    # although the quota is 1; every other position (0.3) is below min_threshold.
    L = 24
    conf = np.full(L, 0.3, np.float32)
    conf[21] = conf[22] = np.float32(0.9)
    canvas = np.zeros(L, np.int64)
    argmax = np.arange(L) + 100
    c, m, s, n = oracle.commit_rule(conf, argmax, canvas, np.ones(L, bool), 0.9, 1, 0, 32, rule="bound")
    assert n == 2 and np.flatnonzero(~m).tolist() == [21, 22]
    assert c[21] == 121 and c[22] == 122 and s == 1


def test_max_transfer_keeps_the_best_ranked_of_the_chosen():
    # Bounded sampler, quota 2, at most 1 per step.  Position 0 (0.5) qualifies
    # through its position threshold (1 - 2/2 = 0, and 0.5 >= 0.45); position 5
    # (0.6) does not (1 - 2/7 = 0.714) and joins through the quota.  The cap keeps
    # the best-ranked of the two by (-conf, position): position 5, although the
    # qualifying set listed position 0 first.
    L = 8
    conf = np.full(L, 0.1, np.float32)
    conf[0], conf[5] = 0.5, 0.6
    canvas = np.zeros(L, np.int64)
    argmax = np.arange(L) + 100
    c, m, s, n = oracle.commit_rule(conf, argmax, canvas, np.ones(L, bool), 0.9, 2, 0, 32, rule="bound",
                                    max_transfer=1)
    assert n == 1 and np.flatnonzero(~m).tolist() == [5] and c[5] == 105
