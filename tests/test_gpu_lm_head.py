"""Fused LM head -> confidence vs the oracle's softmax over float64 logits of the
same bf16 hidden rows and head weights.  Bars: confidence within 1e-2 absolute;
argmax equal wherever the oracle's top-1 logit margin exceeds 5e-2; optional
logits within 2e-2 relative RMS; the mask id never chosen."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import announce, bf16, f32, host, i32, p, rel_rms, stream, sync, workspace
from masked_block_diffusion_denoise_amd import _lib as L

pytestmark = pytest.mark.gpu


def oracle_logits(h, w, mask_id):
    lg = h.astype(np.float64) @ w.astype(np.float64).T
    lg[:, mask_id] = -np.inf
    return lg


def check(R, V, d, mask_id, seed, planted=True, with_logits=True):
    w = synth.normal(seed, 60, (V, d), 0.02)
    if planted:
        h, _ = synth.planted_hidden(w, R, seed=seed)
    else:
        h = synth.hidden_rows(R, d, seed=seed)
    th, tw = bf16(h), bf16(w)
    conf = torch.zeros(R, dtype=torch.float32, device="cuda")
    arg = torch.zeros(R, dtype=torch.int32, device="cuda")
    ent = torch.zeros(R, dtype=torch.float32, device="cuda")
    logits = torch.zeros(R, V, dtype=torch.float32, device="cuda") if with_logits else None
    flags = i32(np.zeros(2))
    ws, n = workspace(L.load().dlm_op_lm_head_workspace_bytes(R, V))
    L.call("dlm_op_lm_head", p(th), R, d, p(tw), V, mask_id, p(conf), p(arg), p(ent), p(logits), p(flags), ws, n,
           stream())
    sync()
    lg = oracle_logits(h, w, mask_id)
    c_want, a_want = oracle.confidence(lg)
    c_got, a_got = host(conf), host(arg)
    assert np.abs(c_got - c_want).max() < 1e-2
    # entropy: fp32 logits of the same bf16 products (summation order only) and
    # fp32 accumulation of the two sums over V; 1e-3 nats covers both at V <= 131072
    assert np.abs(host(ent) - oracle.entropy(lg)).max() < 1e-3
    top2 = np.sort(lg, axis=1)[:, -2:]
    margin = top2[:, 1] - top2[:, 0]
    sure = margin > 5e-2
    np.testing.assert_array_equal(a_got[sure], a_want[sure])
    assert (a_got != mask_id).all()
    assert host(flags)[0] == 0
    if with_logits:
        lgot = host(logits)
        assert np.isneginf(lgot[:, mask_id]).all()
        fin = np.isfinite(lg)
        for r in range(R):
            assert rel_rms(lgot[r][fin[r]], lg[r][fin[r]]) < 2e-2
    return c_want


@pytest.mark.parametrize("R,V,d,mask_id", [(16, 4096, 256, 0), (7, 1024, 128, 5), (64, 2048, 512, 2047),
                                           (300, 4096, 256, 100), (40, 1024, 128, 0),
                                           # full 256-row tiles only / 64-row remainder tiles only / both
                                           (256, 2048, 256, 9), (100, 2048, 256, 3), (577, 1024, 128, 1),
                                           # rows split evenly over 3 tiles of up to 320 / four 256-row tiles
                                           (900, 1024, 128, 7), (1000, 1024, 128, 3),
                                           # 256-row tiles: ragged second tile over eight stages, one
                                           # partly live tile over three
                                           (496, 2048, 512, 11), (200, 2048, 192, 4)])
def test_lm_head_small(R, V, d, mask_id):
    announce(f"lm head R={R} V={V} d={d}")
    c = check(R, V, d, mask_id, seed=R)
    assert c.max() > 0.5 and c.min() < 0.2          # planted rows spread the confidences


def test_lm_head_8b_vocab_batch1():
    announce("lm head 8b b1")
    check(16, 131072, 4096, 100, seed=11)


def test_lm_head_8b_vocab_many_rows():
    announce("lm head 8b 520 rows")
    check(520, 131072, 4096, 100, seed=12, with_logits=False)


def test_lm_head_random_rows_near_uniform():
    announce("lm head random rows")
    c = check(32, 8192, 256, 100, seed=13, planted=False)
    assert c.max() < 0.05


def test_lm_head_flags_non_finite():
    announce("lm head nan")
    R, V, d = 4, 1024, 128
    w = synth.normal(1, 60, (V, d), 0.02)
    h = synth.hidden_rows(R, d, seed=1)
    h[2, 7] = np.nan
    th, tw = bf16(h), bf16(w)
    conf = torch.zeros(R, dtype=torch.float32, device="cuda")
    arg = torch.zeros(R, dtype=torch.int32, device="cuda")
    flags = i32(np.zeros(2))
    ws, n = workspace(L.load().dlm_op_lm_head_workspace_bytes(R, V))
    L.call("dlm_op_lm_head", p(th), R, d, p(tw), V, 0, p(conf), p(arg), None, None, p(flags), ws, n, stream())
    sync()
    assert host(flags)[0] > 0
