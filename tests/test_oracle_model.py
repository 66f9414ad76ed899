"""Pins for the oracle's decoder stack: structural special cases and cache invariants."""
import dataclasses

import numpy as np

import oracle
import synth

TINY = synth.TINY


def _zero_out_projections(w):
    w = {**w, "layers": [dict(l) for l in w["layers"]]}
    for l in w["layers"]:
        l["wo"] = np.zeros_like(l["wo"])
        l["wd"] = np.zeros_like(l["wd"])
    return w


def test_zero_output_projections_leave_the_embedding():
    # With every attention and FFN output projection zero, each residual
    # update is zero and the stream is the embedding row, in either mask mode.
    w = _zero_out_projections(synth.model_weights(TINY, seed=5))
    tok = np.array([3, 17, 900, 4])
    for mode in ("causal", "block"):
        x = oracle.forward(w, TINY, tok, None, mode=mode)
        np.testing.assert_array_equal(x, w["embed"][tok].astype(np.float64))


def _identity_attention_model(seed=0):
    """One layer, MHA (G = H), zero queries/keys, value and output projections = identity.

    Scores are all zero, so attention averages the visible value rows, and the
    values are the normalised inputs: x_t -> x_t + mean_{s visible} n_s, where
    n_s = x_s / sqrt(|x_s|^2 / d + eps).  The FFN is switched off (wd = 0).
    """
    shape = dataclasses.replace(TINY, n_layers=1, n_kv_heads=TINY.n_heads)
    w = synth.model_weights(shape, seed=seed)
    d = shape.d_model
    l = w["layers"][0]
    l["wq"] = np.zeros_like(l["wq"])
    l["wk"] = np.zeros_like(l["wk"])
    l["wv"] = np.eye(d, dtype=np.float32)
    l["wo"] = np.eye(d, dtype=np.float32)
    l["wd"] = np.zeros_like(l["wd"])
    return shape, w


def _normalised(e, eps):
    d = e.shape[-1]
    return e / np.sqrt(np.linalg.norm(e, axis=-1, keepdims=True) ** 2 / d + eps)


def test_mask_modes_by_uniform_attention():
    shape, w = _identity_attention_model()
    tok = np.array([5, 9, 11, 200, 7])
    e = w["embed"][tok].astype(np.float64)
    n = _normalised(e, shape.rms_eps)
    xc = oracle.forward(w, shape, tok, None, mode="causal")
    xb = oracle.forward(w, shape, tok, None, mode="block")
    for t in range(len(tok)):
        np.testing.assert_allclose(xc[t], e[t] + n[: t + 1].mean(axis=0), rtol=1e-12)
        np.testing.assert_allclose(xb[t], e[t] + n.mean(axis=0), rtol=1e-12)


def test_block_denoise_sees_prefix_and_whole_canvas_but_prefix_is_cached():
    # Prefix of 4 tokens (causal, cached), canvas of 3: every canvas row is the
    # mean over all 7 normalised rows -- canvas queries see the full prefix and
    # every canvas position, masked or not.
    shape, w = _identity_attention_model(seed=1)
    prefix = np.array([1, 2, 3, 4])
    canvas = np.array([shape.mask_id, 8, shape.mask_id])
    cache = oracle.KVCache(shape)
    oracle.forward(w, shape, prefix, cache, mode="causal", write_cache=True)
    assert cache.length == 4
    x = oracle.forward(w, shape, canvas, cache, mode="block")
    assert cache.length == 4                       # the denoise pass does not write
    e = w["embed"][np.concatenate([prefix, canvas])].astype(np.float64)
    n = _normalised(e, shape.rms_eps)
    for j in range(3):
        np.testing.assert_allclose(x[j], e[4 + j] + n.mean(axis=0), rtol=1e-12)


def test_cached_denoise_equals_recompute_with_explicit_block_mask():
    w = synth.model_weights(TINY, seed=2)
    prompt = synth.prompt(TINY, 1, 11, seed=2)[0]
    canvas = np.array([TINY.mask_id] * 5 + [77, TINY.mask_id, 901])
    cache, _ = oracle.prefill(w, TINY, prompt)
    got = oracle.denoise_logits(w, TINY, cache, canvas)
    # From scratch over [prompt; canvas] with an explicit mask: prompt rows causal,
    # canvas rows see everything, prompt rows never see the canvas.
    p, l = len(prompt), len(canvas)
    mask = np.zeros((p + l, p + l), bool)
    mask[:p, :p] = np.tril(np.ones((p, p), bool))
    mask[p:, :] = True
    x = oracle.forward(w, TINY, np.concatenate([prompt, canvas]), None, mode=mask)
    want = oracle.head_logits(w, TINY, x[p:])
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


def test_append_keeps_cache_equal_to_causal_prefill_of_everything():
    w = synth.model_weights(TINY, seed=3)
    prompt = synth.prompt(TINY, 1, 9, seed=3)[0]
    blocks = [np.array([5, 6, 7, 8]), np.array([100, 3, 2, 1])]
    cache, _ = oracle.prefill(w, TINY, prompt)
    for blk in blocks:
        oracle.append_block(w, TINY, cache, blk)
    ref, _ = oracle.prefill(w, TINY, np.concatenate([prompt] + blocks))
    for li in range(TINY.n_layers):
        np.testing.assert_allclose(cache.k[li], ref.k[li], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(cache.v[li], ref.v[li], rtol=1e-12, atol=1e-13)


def test_mask_token_is_never_predicted():
    # Make the mask id's head row the best match for every hidden state.
    w = synth.model_weights(TINY, seed=4)
    w["lm_head"] = w["lm_head"].copy()
    w["lm_head"][TINY.mask_id] = 50.0
    logits = oracle.head_logits(w, TINY, np.ones((3, TINY.d_model)))
    conf, arg = oracle.confidence(logits)
    assert (arg != TINY.mask_id).all()
    assert np.isneginf(logits[:, TINY.mask_id]).all()


def test_greedy_ar_with_cache_equals_recompute():
    w = synth.model_weights(TINY, seed=6, lm_head_gain=20.0)
    prompt = synth.prompt(TINY, 1, 7, seed=6)[0]
    a = oracle.generate_ar(w, TINY, prompt, 6)
    b = oracle.generate_ar_recompute(w, TINY, prompt, 6)
    np.testing.assert_array_equal(a, b)
