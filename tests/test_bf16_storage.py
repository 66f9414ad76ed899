"""The bf16-storage variant of the oracle forward that sets the tolerances of the
large-gain parity tests: its rounding is IEEE round-to-nearest-even to 8
significant bits, it equals the oracle when nothing needs rounding, and it
shows the fact the tolerances rest on -- at a head gain of 30, bf16 storage
alone moves confidences by more than 1e-2, and the head's own input rounding is
the smaller part of that."""
import numpy as np

import bf16_storage as B
import oracle
import synth

TINY = synth.TINY


def test_round_to_nearest_even_hand_values():
    # bf16 keeps 8 significant bits: around 1 the spacing is 2^-7, and halfway
    # cases go to the even neighbour.  float32 3e38 is 0x7F61B1E6: the dropped
    # half 0xB1E6 is above 0x8000, so it rounds up to 0x7F62 (3.0040553e38);
    # the subnormal 1e-40 is 0x000116C2 and rounds down to 0x0001 (2^-133).
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -7 + 2 ** -9, -2.5, 3.0e38, 1e-40])
    want = np.array([1.0, 1.0, 1 + 2 ** -6, 1 + 2 ** -7, -2.5, 3.0040553e38, 2.0 ** -133])
    got = B.bf16(x)
    np.testing.assert_array_equal(got[:5], want[:5])
    np.testing.assert_allclose(got[5:], want[5:], rtol=1e-4)


def _canvas_case(gain):
    w = synth.model_weights(TINY, seed=0, lm_head_gain=gain)
    prompt = synth.prompt(TINY, 1, 12, seed=2)[0]
    canvas = np.full(16, TINY.mask_id, np.int64)
    canvas[:3] = prompt[:3]
    return w, prompt, canvas, canvas == TINY.mask_id


def test_bf16_values_pass_through_unchanged():
    # weights and embeddings are bf16 values already; a zero stack leaves them
    w, prompt, canvas, mk = _canvas_case(1.0)
    w0 = {**w, "layers": [dict(l, wo=np.zeros_like(l["wo"]), wd=np.zeros_like(l["wd"])) for l in w["layers"]]}
    x16 = B.forward(w0, TINY, canvas, oracle.KVCache(TINY), "block")
    np.testing.assert_array_equal(x16, np.asarray(w["embed"], np.float64)[canvas])


def test_bf16_storage_alone_exceeds_the_conf_bar_at_gain_30():
    out = {}
    for gain in (20.0, 30.0):
        w, prompt, canvas, mk = _canvas_case(gain)
        cache = oracle.prefill(w, TINY, prompt)[0]
        lo = oracle.denoise_logits(w, TINY, cache, canvas)
        c_o, _ = oracle.confidence(lo)
        c_16, _ = oracle.confidence(B.denoise_logits(w, TINY, B.prefill(w, TINY, prompt), canvas))
        # the head's input alone in bf16, everything before it exact
        n16 = B.bf16(oracle.model.rms_norm(oracle.forward(w, TINY, canvas, cache, mode="block"), w["final_norm"],
                                           TINY.rms_eps))
        lh = n16 @ np.asarray(w["lm_head"], np.float64).T
        lh[:, TINY.mask_id] = -np.inf
        c_h, _ = oracle.confidence(lh)
        out[gain] = (np.abs(c_16 - c_o)[mk].max(), np.abs(c_h - c_o)[mk].max())
    assert out[20.0][0] < 1e-2
    assert B.conf_bar(np.zeros(1), np.full(1, 4e-3), [0]) == 1e-2
    assert B.conf_bar(np.zeros(1), np.full(1, 0.014), [0]) == 0.028
    assert out[30.0][0] > 1e-2
    assert out[30.0][1] < 0.5 * out[30.0][0]


def test_norm_output_rounded_residual_exact():
    # One token through an identity-attention layer (zero queries and keys, the
    # value projection 0.3 I, the output projection I, MHA, FFN off): the
    # attention output is the token's own stored value, so the stream must be
    # e + bf16(0.3 bf16(RMSNorm(e))) -- the norm output and the value rounded
    # where the device stores them, the fp32 residual sum not rounded.
    import dataclasses
    shape = dataclasses.replace(TINY, n_layers=1, n_kv_heads=TINY.n_heads)
    w = synth.model_weights(shape, seed=4)
    d = shape.d_model
    l = dict(w["layers"][0])
    l.update(wq=np.zeros_like(l["wq"]), wk=np.zeros_like(l["wk"]), wv=0.3 * np.eye(d), wo=np.eye(d),
             wd=np.zeros_like(l["wd"]))
    w = {**w, "layers": [l]}
    tok = np.array([321])
    e = np.asarray(w["embed"], np.float64)[tok]
    n = oracle.model.rms_norm(e, l["attn_norm"], shape.rms_eps)
    x16 = B.forward(w, shape, tok, oracle.KVCache(shape), "causal")
    want = e + B.bf16(0.3 * B.bf16(n))
    np.testing.assert_array_equal(x16, want)
    assert not np.array_equal(want, e + B.bf16(0.3 * n))   # the norm's rounding shows
    assert not np.array_equal(B.bf16(want), want)          # the sum itself is not a bf16 value
    # Two tokens, causal: the second averages both stored values (equal scores),
    # so the value rounding shows before the attention output is rounded.
    toks = np.array([321, 77])
    e2 = np.asarray(w["embed"], np.float64)[toks]
    v = B.bf16(0.3 * B.bf16(oracle.model.rms_norm(e2, l["attn_norm"], shape.rms_eps)))
    x2 = B.forward(w, shape, toks, oracle.KVCache(shape), "causal")
    want2 = e2[1] + B.bf16((v[0] + v[1]) / 2)
    np.testing.assert_array_equal(x2[1], want2)
    vr = 0.3 * B.bf16(oracle.model.rms_norm(e2, l["attn_norm"], shape.rms_eps))
    assert not np.array_equal(want2, e2[1] + B.bf16((vr[0] + vr[1]) / 2))   # the value rounding shows
