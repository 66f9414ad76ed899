"""Commit/remask kernel vs the oracle's commit rule: bit-exact when fed the same
confidences and candidates (ragged masks, ties, per-row thresholds and quotas,
forced completion, frozen rows)."""
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
