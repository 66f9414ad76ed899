"""The oracle's forward with bf16 storage of the activations -- test infrastructure.

The path under test stores its activations in bf16 and accumulates in fp32.
This module answers one question for the tolerances of the parity tests: how
far does bf16 storage *alone* move the oracle's numbers?  Every product, sum,
norm, softmax and rotation here is the oracle's own float64 arithmetic (its
functions are called); only the values the device keeps in bf16 are rounded
to bf16 (nearest even) at the points where it stores them:

  * each RMSNorm output (the input of the next product, the head's too);
  * q, k, v as the QKV product writes them, and q, k after RoPE (k, v are the
    bf16 KV cache);
  * the attention probabilities as an operand of the P.V product (the
    normaliser is summed from the unrounded values);
  * the attention output, the adapter's intermediate (o A^T), the SwiGLU output.

The residual stream stays float64 (the device keeps it in fp32).  A head gain
scales every logit and so every logit error: where bf16 storage alone already
moves a confidence by more than the 1e-2 parity bar, no bf16-storage
implementation meets that bar, and the tests bound the device's error by twice
this one instead (``conf_bar``); where it is at most half the bar, the bar
stays 1e-2.
"""
from __future__ import annotations

import numpy as np

import oracle
from oracle.model import F64, rms_norm, rope, silu


def bf16(a) -> np.ndarray:
    """Round to the nearest bf16 (ties to even), returned as float64."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def _attend16(q, k, v, allowed):
    """oracle.attend with the probabilities rounded to bf16 as the P.V operand."""
    n_heads, n_kv = q.shape[0], k.shape[0]
    group = n_heads // n_kv
    out = np.empty_like(q)
    for h in range(n_heads):
        g = h // group
        s = (q[h] @ k[g].T) / np.sqrt(F64(q.shape[-1]))
        s = np.where(allowed, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        out[h] = (bf16(p) @ v[g]) / p.sum(axis=1, keepdims=True)
    return out


def forward(w, shape, tokens, cache, mode, write_cache=False, lora=None):
    """oracle.forward with bf16 storage; ``cache`` is an oracle.KVCache whose
    entries this module wrote (bf16 values)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    t = len(tokens)
    n_prefix = cache.length
    positions = n_prefix + np.arange(t)
    key_pos = np.concatenate([np.arange(n_prefix), positions])
    allowed = (key_pos[None, :] <= positions[:, None]) if mode == "causal" else np.ones((t, n_prefix + t), bool)
    h_, g_, hd = shape.n_heads, shape.n_kv_heads, shape.head_dim
    x = np.asarray(w["embed"], F64)[tokens]
    new_k, new_v = [], []
    for li, lw in enumerate(w["layers"]):
        n = bf16(rms_norm(x, lw["attn_norm"], shape.rms_eps))
        q = bf16(n @ np.asarray(lw["wq"], F64).T).reshape(t, h_, hd).transpose(1, 0, 2)
        k = bf16(n @ np.asarray(lw["wk"], F64).T).reshape(t, g_, hd).transpose(1, 0, 2)
        v = bf16(n @ np.asarray(lw["wv"], F64).T).reshape(t, g_, hd).transpose(1, 0, 2)
        q = bf16(rope(q, positions, shape.rope_base))
        k = bf16(rope(k, positions, shape.rope_base))
        kk = np.concatenate([cache.k[li], k], axis=1)
        vv = np.concatenate([cache.v[li], v], axis=1)
        o = bf16(_attend16(q, kk, vv, allowed).transpose(1, 0, 2).reshape(t, h_ * hd))
        x = x + o @ np.asarray(lw["wo"], F64).T
        if lora is not None:
            mid = bf16(o @ np.asarray(lora["a"][li], F64).T)
            x = x + lora["scale"] * (mid @ np.asarray(lora["b"][li], F64).T)
        n2 = bf16(rms_norm(x, lw["ffn_norm"], shape.rms_eps))
        u = bf16(silu(n2 @ np.asarray(lw["wg"], F64).T) * (n2 @ np.asarray(lw["wu"], F64).T))
        x = x + u @ np.asarray(lw["wd"], F64).T
        new_k.append(k)
        new_v.append(v)
    if write_cache:
        for li in range(shape.n_layers):
            cache.k[li] = np.concatenate([cache.k[li], new_k[li]], axis=1)
            cache.v[li] = np.concatenate([cache.v[li], new_v[li]], axis=1)
    return x


def head_logits(w, shape, x):
    n = bf16(rms_norm(x, w["final_norm"], shape.rms_eps))
    lo = n @ np.asarray(w["lm_head"], F64).T
    lo[..., shape.mask_id] = -np.inf
    return lo


def prefill(w, shape, prompt):
    cache = oracle.KVCache(shape)
    forward(w, shape, prompt, cache, "causal", write_cache=True)
    return cache


def denoise_logits(w, shape, cache, canvas, lora=None):
    return head_logits(w, shape, forward(w, shape, canvas, cache, "block", lora=lora))


def append_block(w, shape, cache, block):
    return forward(w, shape, block, cache, "causal", write_cache=True)


def conf_bar(conf_o, conf_16, rows, base=1e-2):
    """The confidence (or entropy) bar: ``base`` (the parity bar) or twice what
    bf16 storage alone moves the values of ``rows``, whichever is larger -- so
    exactly ``base`` wherever bf16 storage alone moves them by at most half of it."""
    e16 = float(np.abs(np.asarray(conf_16)[rows] - np.asarray(conf_o)[rows]).max())
    return max(base, 2.0 * e16)
