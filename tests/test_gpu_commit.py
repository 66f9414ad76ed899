"""Commit/remask kernel vs the oracle's commit rule: bit-exact when fed the same
confidences and candidates (ragged masks, ties, per-row thresholds and quotas,
forced completion, frozen rows), and the sampler variants of dlm_commit_ex
(bounded confidence, entropy bound, per-step cap, adaptive stopping) vs the
oracle's commit_ex on the same float32 confidences and entropies."""
import ctypes as C

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import announce, f32, host, i32, p, stream, sync, u8
from masked_block_diffusion_denoise_amd import _lib as L

pytestmark = pytest.mark.gpu


def run_both(conf, arg, canvas, masked, tau, quota, steps, max_steps):
    B, Lb = conf.shape
    tc, ta, tcan, tm = f32(conf), i32(arg), i32(canvas), u8(masked)
    ttau, tq, ts = f32(tau), i32(quota), i32(steps)
    tn, tl = i32(np.zeros(B)), i32(np.zeros(B))
    L.call("dlm_commit", p(tc), p(ta), p(tcan), p(tm), B, Lb, p(ttau), p(tq), p(ts), max_steps, p(tn), p(tl),
           stream())
    sync()
    want = oracle.commit_batch(conf, arg, canvas, masked.astype(bool), tau, quota, steps, max_steps)
    got = (host(tcan), host(tm).astype(bool), host(ts), host(tn), host(tl))
    for g, w, name in zip(got, want, ["canvas", "masked", "steps", "n_committed", "n_left"]):
        np.testing.assert_array_equal(g, np.asarray(w).astype(g.dtype), err_msg=name)


@pytest.mark.parametrize("B,Lb,ties,seed", [(37, 32, False, 0), (37, 32, True, 1), (5, 64, True, 2),
                                            (9, 16, False, 3), (1, 1, False, 4), (64, 7, True, 5)])
def test_commit_bit_exact(B, Lb, ties, seed):
    announce(f"commit B={B} L={Lb} ties={ties}")
    g = np.random.default_rng(seed)
    conf, arg = synth.confidences(B, Lb, 1000, seed=seed, ties=ties)
    masked = (g.random((B, Lb)) < 0.6).astype(np.uint8)
    masked[0] = 0                                      # a frozen row
    canvas = np.where(masked, 0, g.integers(1, 1000, (B, Lb))).astype(np.int32)
    tau = np.where(g.random(B) < 0.5, 0.9, g.choice([0.0, 0.5, 1.0, 2.0], B)).astype(np.float32)
    quota = g.integers(0, 4, B).astype(np.int32)
    max_steps = 8
    steps = g.integers(0, max_steps, B).astype(np.int32)   # some rows on their last step
    run_both(conf, arg, canvas, masked, tau, quota, steps, max_steps)


def test_commit_threshold_boundary_and_full_block():
    announce("commit boundary")
    B, Lb = 3, 32
    conf = np.full((B, Lb), np.float32(0.9))
    conf[1] = np.nextafter(np.float32(0.9), np.float32(1.0))   # just above
    conf[2, :5] = 0.99
    arg = np.tile(np.arange(1, Lb + 1, dtype=np.int32), (B, 1))
    masked = np.ones((B, Lb), np.uint8)
    canvas = np.zeros((B, Lb), np.int32)
    run_both(conf, arg, canvas, masked, np.full(B, 0.9, np.float32), np.ones(B, np.int32),
             np.zeros(B, np.int32), 32)


def test_commit_loop_matches_oracle_loop():
    """Drive whole blocks: repeated commits on the device equal the oracle's sequence."""
    announce("commit loop")
    B, Lb, max_steps = 6, 32, 16
    g = np.random.default_rng(9)
    conf_all = g.random((max_steps, B, Lb)).astype(np.float32)
    conf_all[:, 1] *= 0.5
    conf_all[3:, 2] = 0.95
    arg = g.integers(1, 500, (B, Lb)).astype(np.int32)
    tc, ta = f32(conf_all[0]), i32(arg)
    tcan, tm = i32(np.zeros((B, Lb))), u8(np.ones((B, Lb)))
    ttau, tq, ts = f32(np.full(B, 0.9)), i32(np.ones(B)), i32(np.zeros(B))
    tn, tl = i32(np.zeros(B)), i32(np.zeros(B))
    canvas = np.zeros((B, Lb), np.int32)
    masked = np.ones((B, Lb), bool)
    steps = np.zeros(B, np.int32)
    for s in range(max_steps):
        tc.copy_(f32(conf_all[s]))
        L.call("dlm_commit", p(tc), p(ta), p(tcan), p(tm), B, Lb, p(ttau), p(tq), p(ts), max_steps, p(tn),
               p(tl), stream())
        canvas, masked, steps, n, left = oracle.commit_batch(conf_all[s], arg, canvas, masked, 0.9, 1, steps,
                                                             max_steps)
    sync()
    np.testing.assert_array_equal(host(tcan), canvas)
    assert not host(tm).any() and not masked.any()
    np.testing.assert_array_equal(host(ts), steps)


# ------------------------------------------------------- sampler variants ----
RULE_IDS = {"threshold": L.RULE_THRESHOLD, "bound": L.RULE_BOUND, "entropy": L.RULE_ENTROPY}


def run_ex(conf, arg, ent, canvas, masked, tau, quota, steps, max_steps, rule, cap=0, ebound=0.1, stab=0,
           stop_ent=0.005, prev=None, stable=None, dev=None):
    """One dlm_commit_ex call and the oracle's commit_ex per row; compares every
    output.  ``dev`` carries device buffers across calls (adaptive stopping)."""
    B, Lb = conf.shape
    d = dev if dev is not None else {}
    if not d:
        d.update(can=i32(canvas), m=u8(masked), s=i32(steps), n=i32(np.zeros(B)), l=i32(np.zeros(B)))
        if stab:
            d.update(prev=i32(prev), stable=i32(stable))
    o = L.CommitOpts(rule=RULE_IDS[rule], min_threshold=0.45, scaling=2.0, entropy_bound=ebound, max_transfer=cap,
                     stability_steps=stab, stop_entropy=stop_ent,
                     prev_argmax=d["prev"].data_ptr() if stab else None,
                     stable=d["stable"].data_ptr() if stab else None)
    # device copies held in names until the call has finished (a temporary's
    # memory could be reused before the kernel reads it)
    tc, ta, te, ttau, tq = f32(conf), i32(arg), f32(ent), f32(tau), i32(quota)
    L.call("dlm_commit_ex", p(tc), p(ta), p(te), p(d["can"]), p(d["m"]), B, Lb, p(ttau), p(tq),
           p(d["s"]), max_steps, C.byref(o), p(d["n"]), p(d["l"]), stream())
    sync()
    want_c, want_m, want_s, want_n, want_p, want_st = [], [], [], [], [], []
    for r in range(B):
        c, m, s, n, pa, st = oracle.commit_ex(conf[r], arg[r], canvas[r], masked[r].astype(bool), tau[r], quota[r],
                                              int(steps[r]), max_steps, entropy=ent[r],
                                              prev_argmax=None if prev is None else prev[r],
                                              stable=0 if stable is None else int(stable[r]), stability_steps=stab,
                                              stop_entropy=stop_ent, rule=rule, entropy_bound=ebound,
                                              max_transfer=cap)
        want_c.append(c), want_m.append(m), want_s.append(s), want_n.append(n), want_p.append(pa), want_st.append(st)
    got = {"canvas": host(d["can"]), "masked": host(d["m"]).astype(bool), "steps": host(d["s"]),
           "n_committed": host(d["n"]), "n_left": host(d["l"])}
    want = {"canvas": np.array(want_c), "masked": np.array(want_m), "steps": np.array(want_s),
            "n_committed": np.array(want_n), "n_left": np.array(want_m).sum(1)}
    if stab:
        got.update(prev=host(d["prev"]), stable=host(d["stable"]))
        want.update(prev=np.array(want_p), stable=np.array(want_st))
    for k in want:
        np.testing.assert_array_equal(got[k], want[k].astype(got[k].dtype), err_msg=k)
    return want


def variant_inputs(B, Lb, seed, ties):
    g = np.random.default_rng(seed)
    conf, arg = synth.confidences(B, Lb, 1000, seed=seed, ties=ties)
    # some confidences exactly at a position's float32 bound threshold, or the floor
    thr = np.float32(1.0) - np.float32(2.0) / (np.arange(Lb, dtype=np.float32) + np.float32(2.0))
    at = g.random((B, Lb)) < 0.15
    conf = np.where(at, np.maximum(thr, np.float32(0.45))[None, :], conf).astype(np.float32)
    ent = g.choice(np.array([0.0, 0.01, 0.02, 0.05, 0.1, 0.3, 1.5], np.float32), size=(B, Lb))
    masked = (g.random((B, Lb)) < 0.7).astype(np.uint8)
    masked[0] = 0                                       # a frozen row
    canvas = np.where(masked, 0, g.integers(1, 1000, (B, Lb))).astype(np.int32)
    tau = np.where(g.random(B) < 0.6, 0.9, g.choice([0.5, 1.0], B)).astype(np.float32)
    quota = g.integers(0, 4, B).astype(np.int32)
    steps = g.integers(0, 8, B).astype(np.int32)        # some rows on their last allowed step
    return conf, arg, ent, canvas, masked, tau, quota, steps


@pytest.mark.parametrize("rule", ["threshold", "bound", "entropy"])
@pytest.mark.parametrize("cap", [0, 2])
@pytest.mark.parametrize("B,Lb,ties,seed", [(37, 32, True, 11), (5, 64, False, 12), (16, 9, True, 13)])
def test_commit_variants_bit_exact(rule, cap, B, Lb, ties, seed):
    announce(f"commit {rule} cap={cap} B={B} L={Lb}")
    conf, arg, ent, canvas, masked, tau, quota, steps = variant_inputs(B, Lb, seed, ties)
    run_ex(conf, arg, ent, canvas, masked, tau, quota, steps, 8, rule, cap=cap, ebound=0.1)


def test_commit_ex_threshold_equals_commit():
    announce("commit_ex native == commit")
    conf, arg, ent, canvas, masked, tau, quota, steps = variant_inputs(37, 32, 21, True)
    want = run_ex(conf, arg, ent, canvas, masked, tau, quota, steps, 8, "threshold")
    run_both(conf, arg, canvas, masked, tau, quota, steps, 8)
    c, m, s, n, left = oracle.commit_batch(conf, arg, canvas, masked.astype(bool), tau, quota, steps, 8)
    np.testing.assert_array_equal(want["canvas"], c)
    np.testing.assert_array_equal(want["n_committed"], n)


@pytest.mark.parametrize("rule", ["threshold", "entropy"])
def test_commit_adaptive_stopping_sequence(rule):
    """Whole blocks with adaptive stopping: the state buffers and every commit
    follow the oracle step by step; rows whose argmax settles with low entropy
    stop early."""
    announce(f"commit adaptive stopping {rule}")
    B, Lb, max_steps = 12, 32, 16
    g = np.random.default_rng(31)
    canvas = np.zeros((B, Lb), np.int32)
    masked = np.ones((B, Lb), np.uint8)
    masked[0] = 0                                       # frozen from the start
    steps = np.zeros(B, np.int32)
    prev = np.full((B, Lb), -1, np.int32)
    stable = np.zeros(B, np.int32)
    tau, quota = np.full(B, 0.9, np.float32), np.ones(B, np.int32)
    arg = g.integers(1, 900, (B, Lb)).astype(np.int32)
    dev = {}
    done_at = np.full(B, -1)
    for s in range(max_steps):
        conf = (g.random((B, Lb)) * 0.8).astype(np.float32)
        ent = g.choice(np.array([0.0005, 0.001, 0.004, 0.02], np.float32), size=(B, Lb))
        ent[: B // 2] = np.float32(0.001)               # half the rows are confident enough to stop
        changed = g.random((B, Lb)) < (0.5 if s < 3 else 0.02)
        arg = np.where(changed, g.integers(1, 900, (B, Lb)), arg).astype(np.int32)
        want = run_ex(conf, arg, ent, canvas, masked, tau, quota, steps, max_steps, rule, ebound=0.01, stab=2,
                      prev=prev, stable=stable, dev=dev)
        canvas, masked = want["canvas"], want["masked"].astype(np.uint8)
        steps, prev, stable = want["steps"], want["prev"], want["stable"]
        done_at[(done_at < 0) & ~masked.any(axis=1)] = s
        if not masked.any():
            break
    assert not masked.any()
    # the low-entropy rows settle after step 3 and stop two stable steps later
    assert (done_at[1:B // 2] < max_steps - 1).all(), done_at
