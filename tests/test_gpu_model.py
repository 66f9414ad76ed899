"""Whole denoising path through the C ABI vs the oracle.

* Tiny model (2 layers, d=128, vocab 1024): prefill cache, teacher-forced
  denoise steps (conf within 1e-2, logits within 2e-2 relative RMS, argmax equal
  where the top-1 margin exceeds 5e-2), commit bit-exact on the oracle's
  (conf, argmax), append cache equal to the oracle's.
* Free-running block diffusion with a confident head: committed tokens equal the
  oracle's up to the first decision the oracle itself takes within 5e-2.
* One decoder layer at 8B-class shapes with the 131072-vocab head over a 4096-key
  N(0,1) prefix, batch 1 and 32 (sampled rows at 32).
"""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import announce, f32, host, i32, p, rel_rms, stream, sync, u8
from masked_block_diffusion_denoise_amd import _lib as L
from masked_block_diffusion_denoise_amd import runtime as R

pytestmark = pytest.mark.gpu

TINY = synth.TINY


def make(shape, w):
    return R.DlmModel.from_arrays(R.ModelConfig.of(shape), w)


def cache_close(sess, cache, b, upto, tol=1e-2):
    kl = host(sess.kv.k_logical().float())
    vl = host(sess.kv.v_logical().float())
    for l in range(cache.shape.n_layers):
        assert rel_rms(kl[l, b, :, :upto], cache.k[l][:, :upto]) < tol, ("k", l)
        assert rel_rms(vl[l, b, :, :upto], cache.v[l][:, :upto]) < tol, ("v", l)


def check_step(conf_g, arg_g, logits_g, logits_o, masked):
    conf_o, arg_o = oracle.confidence(logits_o)
    mk = np.flatnonzero(masked)
    assert np.abs(conf_g[mk] - conf_o[mk]).max() < 1e-2
    fin = np.isfinite(logits_o[0])
    for j in mk:
        assert rel_rms(logits_g[j][fin], logits_o[j][fin]) < 2e-2
        top2 = np.sort(logits_o[j][fin])[-2:]
        if top2[1] - top2[0] > 5e-2:
            assert arg_g[j] == arg_o[j]
    return conf_o, arg_o


def test_tiny_prefill_cache_and_last_token():
    announce("tiny prefill")
    w = synth.model_weights(TINY, seed=0, lm_head_gain=20.0)
    m = make(TINY, w)
    B, T = 2, 40
    prompt = synth.prompt(TINY, B, T, seed=1)
    sess = R.Session(m, B, 128, 16)
    tp = i32(prompt)
    last_a = i32(np.zeros(B))
    last_c = f32(np.zeros(B))
    # a workspace for 32-row passes forces two prefill passes (32 + 8 positions)
    ws, n = sess.ws.get(m.workspace_bytes(B * 32, T))
    L.call("dlm_prefill", m.handle, C.byref(sess.kv.c), p(tp), B, T, p(sess.prefix), p(last_a), p(last_c),
           p(sess.flags), ws, n, stream())
    sync()
    assert (host(sess.prefix) == T).all()
    for b in range(B):
        cache, x = oracle.prefill(w, TINY, prompt[b])
        cache_close(sess, cache, b, T)
        lg = oracle.head_logits(w, TINY, x[-1:])
        c, a = oracle.confidence(lg)
        assert abs(host(last_c)[b] - c[0]) < 1e-2
        top2 = np.sort(lg[0][np.isfinite(lg[0])])[-2:]
        if top2[1] - top2[0] > 5e-2:
            assert host(last_a)[b] == a[0]
    assert (host(sess.flags) == 0).all()


@pytest.mark.parametrize("gain,tau", [(1.0, 0.9), (60.0, 0.9)])
def test_tiny_teacher_forced_blocks(gain, tau):
    announce(f"tiny teacher-forced gain={gain}")
    w = synth.model_weights(TINY, seed=0, lm_head_gain=gain)
    m = make(TINY, w)
    prompt = synth.prompt(TINY, 1, 32, seed=0)
    Lb, max_steps = 16, 16
    sess = R.Session(m, 1, 128, Lb)
    sess.prefill(i32(prompt))
    cache, _ = oracle.prefill(w, TINY, prompt[0])
    logits = torch.zeros(Lb, TINY.vocab, dtype=torch.float32, device="cuda")
    tau_t, q_t = f32([tau]), i32([1])
    for blk in range(2):
        canvas = np.full(Lb, TINY.mask_id, np.int64)
        masked = np.ones(Lb, bool)
        step = 0
        while masked.any():
            lo = oracle.denoise_logits(w, TINY, cache, canvas)
            sess.canvas.copy_(i32(canvas[None]))
            sess.masked.copy_(u8(masked[None]))
            sess.denoise_step(logits)
            sync()
            conf_o, arg_o = check_step(host(sess.conf)[0], host(sess.argmax)[0], host(logits), lo, masked)
            # commit on the device fed with the oracle's confidences: bit-exact
            sess.conf.copy_(f32(conf_o[None]))
            sess.argmax.copy_(i32(arg_o[None]))
            sess.steps.fill_(step)
            sess.commit(tau_t, q_t, max_steps)
            canvas, masked, step, n = oracle.commit(conf_o.astype(np.float32), arg_o, canvas, masked, tau, 1,
                                                    step, max_steps)
            sync()
            np.testing.assert_array_equal(host(sess.canvas)[0], canvas)
            np.testing.assert_array_equal(host(sess.masked)[0].astype(bool), masked)
            assert host(sess.steps)[0] == step and host(sess.n_committed)[0] == n
        if gain == 1.0:
            assert step == Lb                    # no confidence reaches 0.9: one commit per step
        sess.append_block()
        oracle.append_block(w, TINY, cache, canvas)
        sync()
        assert host(sess.prefix)[0] == cache.length
        cache_close(sess, cache, 0, cache.length)
    assert (host(sess.flags) == 0).all()


def test_tiny_free_running_matches_until_first_ambiguity():
    announce("tiny free-running")
    gain, tau, Lb, max_steps = 60.0, 0.9, 16, 16
    w = synth.model_weights(TINY, seed=0, lm_head_gain=gain)
    m = make(TINY, w)
    prompt = synth.prompt(TINY, 1, 32, seed=0)
    sess = R.Session(m, 1, 128, Lb)
    out_g, st_g = sess.generate(i32(prompt), 32, max_steps, tau, 1)
    out_o, st_o, cache = oracle.generate_block_diffusion(w, TINY, prompt[0], 32, Lb, max_steps, tau, 1,
                                                         keep_trace=True)
    got = host(out_g)[0]
    if not np.array_equal(got, out_o):
        # locate the first step whose decision the oracle takes with less than 5e-2 to spare
        cache2, _ = oracle.prefill(w, TINY, prompt[0])
        ambiguous = False
        for blk in range(2):
            canvas = np.full(Lb, TINY.mask_id, np.int64)
            masked = np.ones(Lb, bool)
            step = 0
            while masked.any() and not ambiguous:
                lo = oracle.denoise_logits(w, TINY, cache2, canvas)
                conf, arg = oracle.confidence(lo)
                mk = np.flatnonzero(masked)
                lc = np.sort(np.log(conf[mk]))[::-1]
                srt = np.sort(lo[mk], axis=1)
                if (np.abs(conf[mk] - tau).min() < 5e-2 or (len(lc) > 1 and np.min(-np.diff(lc)) < 5e-2)
                        or (srt[:, -1] - srt[:, -2]).min() < 5e-2):
                    ambiguous = True
                canvas, masked, step, _ = oracle.commit(conf, arg, canvas, masked, tau, 1, step, max_steps)
            if ambiguous:
                break
            oracle.append_block(w, TINY, cache2, canvas)
        assert ambiguous, (got, out_o)
    assert st_g.denoise_nfe < 32 and st_o.denoise_nfe < 32


@pytest.fixture(scope="module")
def layer8b():
    announce("generating one 8B-class layer")
    shape = synth.LAYER_8B
    w = synth.model_weights(shape, seed=0)
    return shape, w, make(shape, w)


@pytest.mark.parametrize("B,rows", [(1, [0]), (32, [0, 13, 31])])
def test_layer8b_denoise_step(layer8b, B, rows):
    announce(f"8B layer denoise B={B}")
    shape, w, m = layer8b
    P, Lb = 4096, 32
    k, v = synth.kv_prefix(shape, B, P, seed=3)
    canvas, masked = synth.ragged_canvas(shape, B, Lb, seed=3)
    sess = R.Session(m, B, P + Lb + 64, Lb)
    sess.kv.write(0, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    sess.prefix.fill_(P)
    sess.max_prefix = P
    sess.canvas.copy_(i32(canvas))
    sess.masked.copy_(u8(masked))
    logits = torch.zeros(B * Lb, shape.vocab, dtype=torch.float32, device="cuda") if B == 1 else None
    sess.denoise_step(logits)
    sync()
    conf_g, arg_g = host(sess.conf), host(sess.argmax)
    lg_all = host(logits).reshape(B, Lb, -1) if logits is not None else None
    for b in rows:
        cache = oracle.KVCache(shape)
        cache.k[0] = k[b].astype(np.float64)
        cache.v[0] = v[b].astype(np.float64)
        lo = oracle.denoise_logits(w, shape, cache, canvas[b])
        conf_o, arg_o = oracle.confidence(lo)
        mk = np.flatnonzero(masked[b])
        assert np.abs(conf_g[b, mk] - conf_o[mk]).max() < 1e-2
        for j in mk:
            top2 = np.sort(lo[j][np.isfinite(lo[j])])[-2:]
            if top2[1] - top2[0] > 5e-2:
                assert arg_g[b, j] == arg_o[j], (b, j)
            if lg_all is not None:
                fin = np.isfinite(lo[j])
                assert rel_rms(lg_all[b, j][fin], lo[j][fin]) < 2e-2
    assert (host(sess.flags) == 0).all()


def test_layer8b_append_block_batch1(layer8b):
    # batch 1 runs the K-split projections whose partial sums fold into RoPE + KV
    # write and into the residual add + norm: the appended keys/values and the
    # causal next-token predictions must match the oracle's causal pass
    announce("8B layer append B=1")
    shape, w, m = layer8b
    B, P, Lb = 1, 4096, 32
    k, v = synth.kv_prefix(shape, B, P, seed=5)
    block = synth.prompt(shape, B, Lb, seed=5)
    sess = R.Session(m, B, P + Lb + 64, Lb)
    sess.kv.write(0, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    sess.prefix.fill_(P)
    sess.max_prefix = P
    sess.canvas.copy_(i32(block))
    arg = torch.zeros(B, Lb, dtype=torch.int32, device="cuda")
    conf = torch.zeros(B, Lb, dtype=torch.float32, device="cuda")
    sess.append_block(arg, conf)
    sync()
    cache = oracle.KVCache(shape)
    cache.k[0] = k[0].astype(np.float64)
    cache.v[0] = v[0].astype(np.float64)
    x = oracle.append_block(w, shape, cache, block[0])
    kg = host(sess.kv.k_logical()[0, 0, :, P:P + Lb].float())
    vg = host(sess.kv.v_logical()[0, 0, :, P:P + Lb].float())
    assert rel_rms(kg, cache.k[0][:, P:P + Lb]) < 1e-2
    assert rel_rms(vg, cache.v[0][:, P:P + Lb]) < 1e-2
    assert int(host(sess.prefix)[0]) == P + Lb
    lo = oracle.head_logits(w, shape, x)
    conf_o, arg_o = oracle.confidence(lo)
    assert np.abs(host(conf)[0] - conf_o).max() < 1e-2
    for j in range(Lb):
        top2 = np.sort(lo[j][np.isfinite(lo[j])])[-2:]
        if top2[1] - top2[0] > 5e-2:
            assert host(arg)[0, j] == arg_o[j], j


# Two layers wide enough (d 1024) that the batch-1 projections split over K:
# the partial sums fold into RoPE + KV write and into the residual add + the
# next RMSNorm (after the output projection and after the down projection,
# which normalises for the next layer).
WIDE2 = synth.ModelShape(n_layers=2, d_model=1024, n_heads=8, n_kv_heads=2, head_dim=128, d_ffn=2048,
                         vocab=2048, mask_id=0, rope_base=1.0e6)


def test_two_wide_layers_split_reductions_prefill_denoise_append():
    announce("two wide layers: K-split reductions fused")
    shape = WIDE2
    # head gain 2: logit spread ~1.3 as for the 8B-class head at unit gain (a
    # larger gain pushes confidences near 1, where the bf16 logit error alone
    # moves them by ~1e-2)
    w = synth.model_weights(shape, seed=4, lm_head_gain=2.0)
    m = make(shape, w)
    T, Lb = 40, 32
    prompt = synth.prompt(shape, 1, T, seed=6)
    sess = R.Session(m, 1, 128, Lb)
    sess.prefill(i32(prompt))
    cache, _ = oracle.prefill(w, shape, prompt[0])
    sync()
    for layer in range(shape.n_layers):
        kg = host(sess.kv.k_logical()[layer, 0, :, :T].float())
        vg = host(sess.kv.v_logical()[layer, 0, :, :T].float())
        assert rel_rms(kg, cache.k[layer][:, :T]) < 1e-2, layer
        assert rel_rms(vg, cache.v[layer][:, :T]) < 1e-2, layer

    canvas, masked = synth.ragged_canvas(shape, 1, Lb, seed=6)
    sess.canvas.copy_(i32(canvas))
    sess.masked.copy_(u8(masked))
    logits = torch.zeros(Lb, shape.vocab, dtype=torch.float32, device="cuda")
    sess.denoise_step(logits)
    sync()
    lo = oracle.denoise_logits(w, shape, cache, canvas[0])
    conf_o, arg_o = oracle.confidence(lo)
    lg = host(logits)
    mk = np.flatnonzero(masked[0])
    assert np.abs(host(sess.conf)[0, mk] - conf_o[mk]).max() < 1e-2
    for j in mk:
        fin = np.isfinite(lo[j])
        assert rel_rms(lg[j][fin], lo[j][fin]) < 2e-2, j
        top2 = np.sort(lo[j][fin])[-2:]
        if top2[1] - top2[0] > 5e-2:
            assert host(sess.argmax)[0, j] == arg_o[j], j

    block = synth.prompt(shape, 1, Lb, seed=7)
    arg = torch.zeros(1, Lb, dtype=torch.int32, device="cuda")
    conf = torch.zeros(1, Lb, dtype=torch.float32, device="cuda")
    sess.append(i32(block), arg, conf)
    x = oracle.append_block(w, shape, cache, block[0])
    sync()
    for layer in range(shape.n_layers):
        kg = host(sess.kv.k_logical()[layer, 0, :, T:T + Lb].float())
        vg = host(sess.kv.v_logical()[layer, 0, :, T:T + Lb].float())
        assert rel_rms(kg, cache.k[layer][:, T:T + Lb]) < 1e-2, layer
        assert rel_rms(vg, cache.v[layer][:, T:T + Lb]) < 1e-2, layer
    lo = oracle.head_logits(w, shape, x)
    conf_o, arg_o = oracle.confidence(lo)
    assert np.abs(host(conf)[0] - conf_o).max() < 1e-2
    for j in range(Lb):
        top2 = np.sort(lo[j][np.isfinite(lo[j])])[-2:]
        if top2[1] - top2[0] > 5e-2:
            assert host(arg)[0, j] == arg_o[j], j
    assert (host(sess.flags) == 0).all()


def check_step_first_order(conf_g, arg_g, logits_g, logits_o, masked):
    """check_step for a large head gain, which scales the logits and so their
    absolute error: logits within 2e-2 relative RMS as always; the argmax equal
    wherever the top-1 margin exceeds both 5e-2 and twice the row's largest
    logit error (below that, the error alone can reorder the two); the
    confidence within its first-order change under the measured logit error,
    d ln p_max / d l_k = [k = top] - p_k, so |d conf| ~ conf |d_top - sum_k p_k d_k|
    (twice that plus 1e-3)."""
    conf_o, arg_o = oracle.confidence(logits_o)
    fin = np.isfinite(logits_o[0])
    for j in np.flatnonzero(masked):
        l, g = logits_o[j][fin], logits_g[j][fin]
        assert rel_rms(g, l) < 2e-2
        d = g - l
        top2 = np.sort(l)[-2:]
        if top2[1] - top2[0] > max(5e-2, 2.0 * np.abs(d).max()):
            assert arg_g[j] == arg_o[j]
        pr = np.exp(l - l.max())
        pr /= pr.sum()
        bar = 2.0 * conf_o[j] * abs(d[np.argmax(l)] - np.sum(pr * d)) + 1e-3
        assert abs(conf_g[j] - conf_o[j]) <= bar, (j, conf_g[j], conf_o[j], bar)
    return conf_o, arg_o


def entropy_bar(lg_g, lo):
    """First-order bound on the entropy error from the logit error of each row:
    dH/dl_k = -p_k (l_k - mean_p l), so |dH| ~ |sum_k p_k (l_k - lbar) d_k|;
    twice that plus 1e-3 nats covers the second order and fp32 rounding."""
    fin = np.isfinite(lo)
    out = np.empty(len(lo))
    for j in range(len(lo)):
        l, d = lo[j][fin[j]], (lg_g[j][fin[j]] - lo[j][fin[j]])
        p = np.exp(l - l.max())
        p /= p.sum()
        out[j] = 2.0 * abs(np.sum(p * (l - np.sum(p * l)) * d)) + 1e-3
    return out


@pytest.mark.parametrize("sampler", [dict(rule="entropy", entropy_bound=0.5), dict(rule="bound"),
                                     dict(rule="threshold", max_transfer=2),
                                     dict(rule="threshold", stability_steps=2, stop_entropy=0.5)],
                         ids=["entropy", "bound", "cap2", "adaptive-stop"])
def test_tiny_teacher_forced_samplers(sampler):
    """Sampler variants through whole blocks: the device's entropies against the
    oracle's, and dlm_commit_ex fed the oracle's confidences and entropies
    bit-exact with the oracle's commit_ex (adaptive-stopping state included)."""
    announce(f"tiny teacher-forced sampler {sampler}")
    w = synth.model_weights(TINY, seed=0, lm_head_gain=60.0)
    m = make(TINY, w)
    prompt = synth.prompt(TINY, 1, 32, seed=0)
    Lb, max_steps, tau = 16, 16, 0.9
    sess = R.Session(m, 1, 128, Lb)
    sess.prefill(i32(prompt))
    cache, _ = oracle.prefill(w, TINY, prompt[0])
    logits = torch.zeros(Lb, TINY.vocab, dtype=torch.float32, device="cuda")
    ent_g = torch.zeros(1, Lb, dtype=torch.float32, device="cuda")
    smp = R.Sampler(**sampler)
    tau_t, q_t = f32([tau]), i32([1])
    steps_seen = []
    for blk in range(2):
        sess.begin_block()
        canvas = np.full(Lb, TINY.mask_id, np.int64)
        masked = np.ones(Lb, bool)
        step, prev, stable = 0, np.full(Lb, -1), 0
        while masked.any():
            lo = oracle.denoise_logits(w, TINY, cache, canvas)
            sess.canvas.copy_(i32(canvas[None]))
            sess.masked.copy_(u8(masked[None]))
            sess.denoise_step(logits, ent_g)
            sync()
            lg = host(logits)
            conf_o, arg_o = check_step_first_order(host(sess.conf)[0], host(sess.argmax)[0], lg, lo, masked)
            ent_o = oracle.entropy(lo)
            mk = np.flatnonzero(masked)
            bar = entropy_bar(lg[mk], lo[mk])
            assert (np.abs(host(ent_g)[0][mk] - ent_o[mk]) <= bar).all(), (host(ent_g)[0][mk], ent_o[mk], bar)
            # commit on the device fed with the oracle's values: bit-exact
            c32, e32 = conf_o.astype(np.float32), ent_o.astype(np.float32)
            sess.conf.copy_(f32(c32[None]))
            sess.argmax.copy_(i32(arg_o[None]))
            ent_g.copy_(f32(e32[None]))
            sess.steps.fill_(step)
            sess.commit_ex(tau_t, q_t, max_steps, smp, ent_g)
            canvas, masked, step, n, prev, stable = oracle.commit_ex(
                c32, arg_o, canvas, masked, tau, 1, step, max_steps, entropy=e32, prev_argmax=prev,
                stable=stable, **sampler)
            sync()
            np.testing.assert_array_equal(host(sess.canvas)[0], canvas)
            np.testing.assert_array_equal(host(sess.masked)[0].astype(bool), masked)
            assert host(sess.steps)[0] == step and host(sess.n_committed)[0] == n
            if smp.stability_steps:
                np.testing.assert_array_equal(host(sess.prev_argmax)[0], prev)
                assert host(sess.stable)[0] == stable
        steps_seen.append(step)
        sess.append_block()
        oracle.append_block(w, TINY, cache, canvas)
        sync()
        cache_close(sess, cache, 0, cache.length)
    if sampler.get("max_transfer"):
        assert max(steps_seen) >= Lb // 2                   # at most 2 per step: at least 8 steps a block


def test_tiny_anchor_blocks():
    """Anchor layout on the device: each block's first token is the causal
    argmax after everything before it (the oracle's, wherever its top-1 margin
    is clear), it is never reopened, and a block takes at most L - 1 steps."""
    announce("tiny anchor blocks")
    w = synth.model_weights(TINY, seed=0, lm_head_gain=20.0)
    m = make(TINY, w)
    prompt = synth.prompt(TINY, 1, 32, seed=2)
    Lb, max_steps, n_blocks = 16, 16, 3
    sess = R.Session(m, 1, 128, Lb)
    out, st = sess.generate(i32(prompt), n_blocks * Lb, max_steps, 0.9, 1, anchor=True)
    toks = host(out)[0]
    assert all(s <= Lb - 1 for s in st.steps_per_block), st.steps_per_block
    assert st.accepted_tokens == n_blocks * (Lb - 1)      # the anchors are not denoised
    checked = 0
    for k in range(n_blocks):
        before = np.concatenate([prompt[0], toks[:k * Lb]])
        _, x = oracle.prefill(w, TINY, before)
        lo = oracle.head_logits(w, TINY, x[-1:])[0]
        top2 = np.sort(lo[np.isfinite(lo)])[-2:]
        if top2[1] - top2[0] > 5e-2:
            assert toks[k * Lb] == int(np.argmax(lo)), k
            checked += 1
    assert checked >= 2
    assert (toks != TINY.mask_id).all()


@pytest.mark.parametrize("K,anchor,rule", [(4, False, None), (3, True, None), (5, False, "entropy")])
def test_tiny_graph_replay_equals_eager(K, anchor, rule):
    """The block loop replaying a captured graph of K steps (eager fills and host
    reads between the replays) produces exactly the eager loop's tokens and step
    counts, block after block."""
    announce(f"tiny graph replay K={K} anchor={anchor} rule={rule}")
    w = synth.model_weights(TINY, seed=0, lm_head_gain=60.0)
    m = make(TINY, w)
    prompt = synth.prompt(TINY, 2, 32, seed=7)
    Lb, max_steps = 16, 16
    smp = R.Sampler(rule=rule, entropy_bound=0.5) if rule else None
    runs = []
    for gs in (0, K):
        sess = R.Session(m, 2, 128, Lb)
        out, st = sess.generate(i32(prompt), 3 * Lb, max_steps, 0.9, 1, sampler=smp, anchor=anchor, graph_steps=gs)
        sync()
        runs.append((host(out), st.steps_per_block, st.accepted_tokens, host(sess.prefix)))
    (o0, s0, a0, p0), (o1, s1, a1, p1) = runs
    np.testing.assert_array_equal(o1, o0)
    assert s1 == s0 and a1 == a0
    np.testing.assert_array_equal(p1, p0)
    assert (o0 != TINY.mask_id).all()
