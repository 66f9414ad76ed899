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


def test_head_logits_apply_the_final_norm_hand_values():
    # x = [3, 4]: mean square 12.5, so the normalised row is [3, 4] / 3.5355339 =
    # [0.8485281, 1.1313708] (eps 1e-5 moves the 7th digit); head rows [1, 0],
    # [0, 1], [1, 1] read it out, and the final-norm gains scale it per column.
    shape = dataclasses.replace(TINY, d_model=2, vocab=4, mask_id=0)
    head = np.array([[7.0, 7.0], [1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    lo = oracle.head_logits({"final_norm": np.array([1.0, 1.0]), "lm_head": head}, shape, np.array([[3.0, 4.0]]))
    assert np.isneginf(lo[0, 0])
    np.testing.assert_allclose(lo[0, 1:], [0.8485281, 1.1313708, 1.9798990], atol=2e-6)
    lo = oracle.head_logits({"final_norm": np.array([2.0, 0.5]), "lm_head": head}, shape, np.array([[3.0, 4.0]]))
    np.testing.assert_allclose(lo[0, 1:], [1.6970563, 0.5656854, 2.2627417], atol=2e-6)
    # scaling the residual row leaves the logits unchanged (the norm removes it)
    lo2 = oracle.head_logits({"final_norm": np.array([2.0, 0.5]), "lm_head": head}, shape, np.array([[30.0, 40.0]]))
    np.testing.assert_allclose(lo2, lo, atol=1e-6)


def test_greedy_ar_with_cache_equals_recompute():
    w = synth.model_weights(TINY, seed=6, lm_head_gain=20.0)
    prompt = synth.prompt(TINY, 1, 7, seed=6)[0]
    a = oracle.generate_ar(w, TINY, prompt, 6)
    b = oracle.generate_ar_recompute(w, TINY, prompt, 6)
    np.testing.assert_array_equal(a, b)


def test_swiglu_ffn_by_hand():
    # One layer with its attention switched off (wo = 0) and an FFN that reads
    # one gate row and one up row.  The embedding row is (3, 4, 0, ..., 0) in
    # d = 128, the FFN norm gains are 0.5 (the attention norm's stay 1, so using
    # the wrong norm shows), gate row 0 = 0.2 e_0, up row 0 = 0.2 e_1, and the
    # down projection writes their product to dimension 5.  By hand:
    #   rstd = 1 / sqrt(25/128 + 1e-5)          = 2.2626838
    #   normalised input = (3, 4) * rstd * 0.5  = (3.3940257, 4.5253676)
    #   gate = 0.2 * 3.3940257 = 0.67880513,  up = 0.2 * 4.5253676 = 0.90507351
    #   sigmoid(gate) = 1 / (1 + e^-0.67880513) = 0.66347196
    #   silu(gate) * up = 0.67880513 * 0.66347196 * 0.90507351 = 0.40761630
    # so dimension 5 becomes 0 + 0.40761630 and every other dimension keeps the
    # embedding (the residual).  Gate and up swapped would give 0.43742487, the
    # attention norm's gains 1.95460376.
    shape = dataclasses.replace(TINY, n_layers=1)
    w = synth.model_weights(shape, seed=7)
    w = {**w, "embed": np.array(w["embed"], dtype=np.float64), "layers": [dict(w["layers"][0])]}
    l = w["layers"][0]
    d, f = shape.d_model, shape.d_ffn
    tok = 9
    w["embed"][tok] = 0.0
    w["embed"][tok, 0], w["embed"][tok, 1] = 3.0, 4.0
    l["wo"] = np.zeros_like(l["wo"])
    l["attn_norm"] = np.ones(d)
    l["ffn_norm"] = np.full(d, 0.5)
    l["wg"] = np.zeros((f, d))
    l["wg"][0, 0] = 0.2
    l["wu"] = np.zeros((f, d))
    l["wu"][0, 1] = 0.2
    l["wd"] = np.zeros((d, f))
    l["wd"][5, 0] = 1.0
    x = oracle.forward(w, shape, np.array([tok]), None, mode="causal")[0]
    want = np.zeros(d)
    want[0], want[1], want[5] = 3.0, 4.0, 0.40761630
    np.testing.assert_allclose(x, want, rtol=0, atol=5e-9)


def test_o_proj_adapter_by_hand():
    # The draft adapter adds scale * (o A^T) B^T to the output projection, o
    # being the attention output (the projection's input), not the layer input.
    # Identity attention model (values = normalised inputs, wo = I, FFN off),
    # two tokens in causal mode, rank 1: A = e_2^T (reads o[2]), B = e_7 (writes
    # dimension 7), scale 4.  Embedding rows: token 0 = 2 e_2, token 1 = 6 e_3
    # (d = 128).  By hand, for token 1:
    #   n_0 = 2 e_2 / sqrt(4/128 + 1e-5)  = 11.3118987 e_2
    #   n_1 = 6 e_3 / sqrt(36/128 + 1e-5) = 11.3135074 e_3
    #   o_1 = (n_0 + n_1) / 2              = 5.6559494 e_2 + 5.6567537 e_3
    #   x_1 = 6 e_3 + o_1 + 4 * o_1[2] e_7 = 5.6559494 e_2 + 11.6567537 e_3 + 22.6237975 e_7
    # The adapter on the token's own normalised row instead of o gives 0 in
    # dimension 7, without its scale 5.6559494.
    shape, w = _identity_attention_model(seed=2)
    w = {**w, "embed": np.array(w["embed"], dtype=np.float64), "layers": [dict(w["layers"][0])]}
    d = shape.d_model
    w["layers"][0]["attn_norm"] = np.ones(d)
    w["embed"][11] = 0.0
    w["embed"][11, 2] = 2.0
    w["embed"][12] = 0.0
    w["embed"][12, 3] = 6.0
    a = np.zeros((1, shape.n_heads * shape.head_dim))
    a[0, 2] = 1.0
    b = np.zeros((d, 1))
    b[7, 0] = 1.0
    lora = {"a": [a], "b": [b], "scale": 4.0}
    x = oracle.forward(w, shape, np.array([11, 12]), None, mode="causal", lora=lora)[1]
    want = np.zeros(d)
    want[2], want[3], want[7] = 5.6559494, 11.6567537, 22.6237975
    np.testing.assert_allclose(x, want, rtol=0, atol=5e-7)


def test_rope_makes_attention_relative_in_the_forward():
    # Rotating both queries and keys by their positions makes every score depend
    # only on the position difference (the rotation property of RoPE), so the
    # forward is unchanged when every position moves by the same amount; a
    # rotation of only one side depends on absolute positions.  And RoPE must
    # act at all: without it, bidirectional attention would not see the order
    # of its keys, and reversing the tokens would only reverse the outputs.
    shape = dataclasses.replace(TINY, n_layers=1)
    w = synth.model_weights(shape, seed=11)
    tok = np.array([5, 77, 300, 12, 900, 41])
    t = len(tok)
    for mode in ("causal", "block"):
        x0 = oracle.forward(w, shape, tok, None, mode=mode, positions=np.arange(t))
        x1 = oracle.forward(w, shape, tok, None, mode=mode, positions=137 + np.arange(t))
        np.testing.assert_allclose(x1, x0, rtol=0, atol=1e-9)
    xb = oracle.forward(w, shape, tok, None, mode="block")
    xr = oracle.forward(w, shape, tok[::-1], None, mode="block")
    assert np.abs(xr[::-1] - xb).max() > 1e-3
