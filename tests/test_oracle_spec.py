"""Linear self-speculation in the oracle (MLX guide, sec. 3.3 and 8): a draft
block from one bidirectional pass with the o_proj LoRA on, a causal verification
with it off, longest accepted prefix plus one correction, cache trimmed back.

Pins: the output equals greedy causal decoding token for token (the method is
lossless by construction; generate_ar is itself pinned against recompute), the
trimmed cache equals a causal prefill of the emitted tokens, the adaptive window
follows the page's rule, and the LoRA term is pinned through a case where it
cancels the output projection exactly."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from synth import TINY


@pytest.fixture(scope="module")
def tiny():
    w = synth.model_weights(TINY, seed=0, lm_head_gain=30.0)
    lora = synth.lora_weights(TINY, rank=128, scale=4.0, seed=1)
    prompt = synth.prompt(TINY, 1, 12, seed=2)[0]
    return w, lora, prompt


@pytest.mark.parametrize("window,adaptive", [(4, False), (8, False), (32, False), (8, True)])
def test_spec_equals_greedy_ar(tiny, window, adaptive):
    w, lora, prompt = tiny
    n_new = 24
    got, accepted, windows, _ = oracle.generate_linear_spec(w, TINY, prompt, n_new, lora, window, adaptive)
    want = oracle.generate_ar(w, TINY, prompt, n_new)
    np.testing.assert_array_equal(got, want)
    assert len(accepted) == len(windows) and all(0 <= a < W for a, W in zip(accepted, windows))
    # every round emits its known token plus the accepted drafts
    assert sum(a + 1 for a in accepted) >= n_new


def test_spec_trimmed_cache_is_prefill_of_emitted(tiny):
    w, lora, prompt = tiny
    _, _, _, cache = oracle.generate_linear_spec(w, TINY, prompt, 20, lora, 8, False)
    n_emitted = cache.length - len(prompt)
    emitted = oracle.generate_ar(w, TINY, prompt, n_emitted)
    ref, _ = oracle.prefill(w, TINY, np.concatenate([prompt, emitted]))
    for li in range(TINY.n_layers):
        np.testing.assert_allclose(cache.k[li], ref.k[li], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(cache.v[li], ref.v[li], rtol=1e-12, atol=1e-12)


def test_draft_accepts_everything_when_draft_equals_verifier(tiny):
    # a "draft" that is the causal model itself: with the causal mask in the
    # draft pass every draft is the greedy continuation, so every round accepts
    # all W - 1 drafts and emits W tokens -- checks the acceptance bookkeeping
    w, _, prompt = tiny
    cache, x = oracle.prefill(w, TINY, prompt)
    ar = oracle.generate_ar(w, TINY, prompt, 9)
    nxt, W = int(ar[0]), 8
    block = [nxt]
    for j in range(W - 1):  # causal drafting == AR continuation of the block
        block.append(int(ar[j + 1]))
    xv = oracle.append_block(w, TINY, cache, np.array(block))
    _, ver = oracle.confidence(oracle.head_logits(w, TINY, xv))
    drafts = np.array(block[1:])
    a = 0
    while a < W - 1 and drafts[a] == ver[a]:
        a += 1
    assert a == W - 1 and ver[a] == ar[W]


@pytest.mark.parametrize("window,accepted,expect", [(8, 7, 16), (16, 15, 32), (32, 31, 32), (8, 3, 4), (8, 4, 8),
                                                    (4, 1, 2), (2, 0, 2), (32, 16, 32), (32, 15, 16)])
def test_next_draft_window(window, accepted, expect):
    assert oracle.next_draft_window(window, accepted) == expect


def test_lora_can_cancel_the_output_projection(tiny):
    # with A = I (rank = H*hd) and B = -Wo / scale the adapter removes the
    # attention output: the pass then equals one with every Wo set to zero
    w, _, prompt = tiny
    scale = 4.0
    lora = {"a": [np.eye(TINY.q_dim) for _ in range(TINY.n_layers)],
            "b": [-np.asarray(lw["wo"], np.float64) / scale for lw in w["layers"]], "scale": scale}
    w0 = dict(w)
    w0["layers"] = [dict(lw, wo=np.zeros_like(lw["wo"])) for lw in w["layers"]]
    x1 = oracle.forward(w, TINY, prompt, None, mode="block", lora=lora)
    x0 = oracle.forward(w0, TINY, prompt, None, mode="block")
    np.testing.assert_allclose(x1, x0, rtol=1e-10, atol=1e-12)
    # and a zero adapter changes nothing
    zero = {"a": lora["a"], "b": [np.zeros_like(b) for b in lora["b"]], "scale": scale}
    np.testing.assert_allclose(oracle.forward(w, TINY, prompt, None, mode="block", lora=zero),
                               oracle.forward(w, TINY, prompt, None, mode="block"), rtol=0, atol=0)


def _copy_model(next_of):
    """One layer whose attention and FFN add nothing (wo = wd = 0), one-hot
    embeddings (token t < d is e_t), and a head under which token t predicts
    next_of[t]: every prediction depends only on the token at its position, in
    the bidirectional draft and in the causal verification alike."""
    shape = dataclasses.replace(TINY, n_layers=1)
    w = synth.model_weights(shape, seed=3)
    layer = dict(w["layers"][0])
    layer["wo"] = np.zeros_like(layer["wo"])
    layer["wd"] = np.zeros_like(layer["wd"])
    embed = np.zeros((shape.vocab, shape.d_model))
    embed[np.arange(shape.d_model), np.arange(shape.d_model)] = 1.0
    head = np.zeros((shape.vocab, shape.d_model))
    for t, nxt in next_of.items():
        head[nxt, t] = 1.0
    w = {**w, "layers": [layer], "embed": embed, "lm_head": head, "final_norm": np.ones(shape.d_model)}
    return shape, w


def test_spec_acceptance_on_a_copy_model():
    # Every draft of a masked position is next_of[MASK] = 5.  Chain 7 -> 9 -> 11
    # -> ...: a draft 5 is never the causal prediction, so each round accepts
    # nothing and emits only its known token; a check of draft a against the
    # prediction after position a + 1 (instead of a) would accept the 5s, which
    # also predict 5.  Chain 7 -> 9 -> 5 -> 5: every draft is right, so each round
    # of window W accepts W - 1 drafts.  Both must equal greedy AR.
    mask = TINY.mask_id
    lora = {"a": [np.zeros((1, TINY.n_heads * TINY.head_dim))], "b": [np.zeros((TINY.d_model, 1))], "scale": 4.0}
    prompt = np.array([3, 7])
    chain = {mask: 5, 5: 5, 3: 7, **{t: t + 2 for t in range(7, 40, 2)}}
    shape, w = _copy_model(chain)
    ar = oracle.generate_ar(w, shape, prompt, 8)
    assert ar.tolist() == [9, 11, 13, 15, 17, 19, 21, 23]
    out, accepted, _, _ = oracle.generate_linear_spec(w, shape, prompt, 8, lora, window=4)
    assert out.tolist() == ar.tolist() and accepted == [0] * 8
    shape, w = _copy_model({mask: 5, 5: 5, 3: 7, 7: 9, 9: 5})
    ar = oracle.generate_ar(w, shape, prompt, 8)
    assert ar.tolist() == [9, 5, 5, 5, 5, 5, 5, 5]
    out, accepted, _, _ = oracle.generate_linear_spec(w, shape, prompt, 8, lora, window=4)
    assert out.tolist() == ar.tolist() and accepted == [3, 3]
