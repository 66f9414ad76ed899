"""Pins of the anchor-token layout (MLX guide, sec. 6: position 0 of a block is
the causal argmax after everything before it; the rest is denoised)."""
import numpy as np

import oracle
import synth
from synth import TINY


def _model():
    return synth.model_weights(TINY, seed=0, lm_head_gain=30.0)


def test_anchor_quota1_threshold1_takes_L_minus_1_steps():
    w = _model()
    prompt = synth.prompt(TINY, 1, 24, seed=3)[0]
    L = 8
    _, st, _ = oracle.generate_block_diffusion(w, TINY, prompt, 2 * L, L, 32, tau=1.0, quota=1, anchor=True)
    assert st.steps_per_block == [L - 1, L - 1]
    assert st.denoise_nfe == 2 * (L - 1) and st.post_block_nfe == 2
    _, st0, _ = oracle.generate_block_diffusion(w, TINY, prompt, 2 * L, L, 32, tau=1.0, quota=1)
    assert st0.steps_per_block == [L, L]                  # without the anchor: L steps


def test_anchor_is_the_greedy_causal_next_token():
    w = _model()
    prompt = synth.prompt(TINY, 1, 20, seed=4)[0]
    L = 8
    toks, _, cache = oracle.generate_block_diffusion(w, TINY, prompt, 3 * L, L, 16, anchor=True)
    for k in range(3):
        before = np.concatenate([prompt, toks[:k * L]])
        nxt = oracle.generate_ar_recompute(w, TINY, before, 1)[0]
        assert toks[k * L] == nxt, k
    # the cache still equals a causal prefill of everything
    ref, _ = oracle.prefill(w, TINY, np.concatenate([prompt, toks]))
    for l in range(TINY.n_layers):
        np.testing.assert_allclose(cache.k[l][:, :ref.length], ref.k[l][:, :ref.length], rtol=1e-9, atol=1e-9)


def test_anchor_positions_are_never_rewritten():
    w = _model()
    prompt = synth.prompt(TINY, 1, 16, seed=5)[0]
    L = 8
    toks, st, _ = oracle.generate_block_diffusion(w, TINY, prompt, 2 * L, L, 16, anchor=True, keep_trace=True)
    opened = [set(o) for o, _ in st.trace]
    assert all(0 not in o for o in opened)               # position 0 is never opened: it was never masked
    assert sum(len(o) for o in opened) == 2 * (L - 1)
