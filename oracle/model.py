"""Oracle transformer forward (float64, one sequence at a time) -- test infrastructure.

The network is the dense decoder of the MLX guide, sec. 7 (architecture):
a stack of pre-norm layers, each RMSNorm -> grouped-query attention with RoPE
-> residual -> RMSNorm -> SwiGLU (SiLU gate) -> residual, then a final RMSNorm
and an untied head over the vocabulary.  The same weights serve causal
(prefill, append, AR) and bidirectional-block (denoise) attention; only the
attention mask changes (NLD tutorial, sec. 3.1).

Readings where the pages are silent (each also listed in the design notes):
  * RMSNorm is x / sqrt(mean(x^2) + eps) * g with eps = 1e-5.
  * RoPE rotates the pairs (i, i + hd/2) by angle pos * base^(-2i/hd)
    ("rotate half"), at absolute positions; no long-context scaling.
  * Query head h reads KV head floor(h / (H/G)).
  * Attention scale 1/sqrt(hd); no biases; no embedding scaling.
  * The head's logit for the mask id is -inf: the mask token is never a
    prediction (Module 12, sec. 7 and sec. 12: the output parametrisation
    forbids choosing the mask as a final token).
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def rms_norm(x, g, eps):
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    x = np.asarray(x, dtype=F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, dtype=F64)


def silu(z):
    z = np.asarray(z, dtype=F64)
    return z / (1.0 + np.exp(-z))


def rope(x, positions, base):
    """Rotate the last axis of x [..., T, hd] for token positions [T] (rotate-half pairing)."""
    x = np.asarray(x, dtype=F64)
    hd = x.shape[-1]
    half = hd // 2
    freq = np.power(F64(base), -2.0 * np.arange(half, dtype=F64) / hd)
    ang = np.asarray(positions, dtype=F64)[:, None] * freq[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attend(q, k, v, allowed):
    """Grouped-query attention with an explicit boolean mask.

    q [H, Tq, hd]; k, v [G, Tk, hd]; allowed [Tq, Tk] (True = may attend).
    Returns [H, Tq, hd].  Each query row must be allowed at least one key.
    """
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    n_heads, n_kv, hd = q.shape[0], k.shape[0], q.shape[-1]
    group = n_heads // n_kv
    allowed = np.asarray(allowed, dtype=bool)
    if not allowed.any(axis=1).all():
        raise ValueError("every query needs at least one visible key")
    out = np.empty_like(q)
    for h in range(n_heads):
        g = h // group
        s = (q[h] @ k[g].T) / np.sqrt(F64(hd))
        s = np.where(allowed, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[h] = p @ v[g]
    return out


class KVCache:
    """Per-layer post-RoPE keys and values of the finished prefix: [G, P, hd] each."""

    def __init__(self, shape):
        self.shape = shape
        g, hd = shape.n_kv_heads, shape.head_dim
        self.k = [np.zeros((g, 0, hd)) for _ in range(shape.n_layers)]
        self.v = [np.zeros((g, 0, hd)) for _ in range(shape.n_layers)]

    @property
    def length(self) -> int:
        return self.k[0].shape[1]

    def copy(self) -> "KVCache":
        c = KVCache(self.shape)
        c.k = [a.copy() for a in self.k]
        c.v = [a.copy() for a in self.v]
        return c

    def truncate(self, n: int) -> None:
        self.k = [a[:, :n] for a in self.k]
        self.v = [a[:, :n] for a in self.v]


def _mask_for(mode, positions, n_prefix):
    """Boolean [T, n_prefix + T] attention mask for tokens at ``positions`` after a cached prefix.

    causal: a query sees every key whose position is not after its own.
    block:  a canvas query sees every cached prefix key and every canvas key,
            masked or not (Module 12, sec. 14: the active block reads the
            finished prefix and all of its own positions).
    """
    t = len(positions)
    key_pos = np.concatenate([np.arange(n_prefix), np.asarray(positions)])
    if isinstance(mode, np.ndarray):
        return mode
    if mode == "causal":
        return key_pos[None, :] <= np.asarray(positions)[:, None]
    if mode == "block":
        return np.ones((t, n_prefix + t), dtype=bool)
    raise ValueError(f"unknown attention mode {mode!r}")


def forward(w, shape, tokens, cache=None, mode="causal", write_cache=False,
            positions=None, lora=None):
    """Run the decoder stack over ``tokens`` placed after the cached prefix.

    Returns the final residual stream [T, d] (before the final norm).  With
    ``write_cache`` the new keys/values are appended to ``cache``; the denoise
    pass never writes (its keys/values were computed from a masked canvas and
    may not enter the history; Module 12, sec. 14).  ``mode`` is "causal",
    "block" or an explicit boolean mask [T, P + T].

    ``lora`` (optional): {"a": per-layer [r, H*hd], "b": per-layer [d, r],
    "scale": s} adds s * (o A^T) B^T to every layer's output projection -- the
    draft-only adapter of linear self-speculation (MLX guide, sec. 3.3 and 8:
    rank 128, scale 4.0, on self_attn.o_proj only).
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    t = tokens.shape[0]
    n_prefix = cache.length if cache is not None else 0
    if positions is None:
        positions = n_prefix + np.arange(t)
    allowed = _mask_for(mode, positions, n_prefix)
    h_, g_, hd = shape.n_heads, shape.n_kv_heads, shape.head_dim
    x = np.asarray(w["embed"], dtype=F64)[tokens]
    new_k, new_v = [], []
    for li, lw in enumerate(w["layers"]):
        n = rms_norm(x, lw["attn_norm"], shape.rms_eps)
        q = (n @ np.asarray(lw["wq"], F64).T).reshape(t, h_, hd).transpose(1, 0, 2)
        k = (n @ np.asarray(lw["wk"], F64).T).reshape(t, g_, hd).transpose(1, 0, 2)
        v = (n @ np.asarray(lw["wv"], F64).T).reshape(t, g_, hd).transpose(1, 0, 2)
        q = rope(q, positions, shape.rope_base)
        k = rope(k, positions, shape.rope_base)
        if cache is not None:
            kk = np.concatenate([cache.k[li], k], axis=1)
            vv = np.concatenate([cache.v[li], v], axis=1)
        else:
            kk, vv = k, v
        o = attend(q, kk, vv, allowed).transpose(1, 0, 2).reshape(t, h_ * hd)
        x = x + o @ np.asarray(lw["wo"], F64).T
        if lora is not None:
            a_, b_ = np.asarray(lora["a"][li], F64), np.asarray(lora["b"][li], F64)
            x = x + lora["scale"] * ((o @ a_.T) @ b_.T)
        n2 = rms_norm(x, lw["ffn_norm"], shape.rms_eps)
        gate = n2 @ np.asarray(lw["wg"], F64).T
        up = n2 @ np.asarray(lw["wu"], F64).T
        x = x + (silu(gate) * up) @ np.asarray(lw["wd"], F64).T
        new_k.append(k)
        new_v.append(v)
    if write_cache:
        if cache is None:
            raise ValueError("write_cache needs a cache")
        for li in range(shape.n_layers):
            cache.k[li] = np.concatenate([cache.k[li], new_k[li]], axis=1)
            cache.v[li] = np.concatenate([cache.v[li], new_v[li]], axis=1)
    return x


def head_logits(w, shape, x):
    """Final RMSNorm and the untied head; the mask id gets -inf (never predicted)."""
    n = rms_norm(x, w["final_norm"], shape.rms_eps)
    logits = n @ np.asarray(w["lm_head"], F64).T
    logits[..., shape.mask_id] = -np.inf
    return logits


def confidence(logits):
    """Per row: (max softmax probability, argmax id with ties to the lowest id).

    The confidence of a position is the probability of its greedy candidate
    (Module 12, sec. 9 and 12: candidates are the per-position argmax, ranked
    by their probability).  conf = 1 / sum_v exp(l_v - max_v l_v).
    Raises ValueError on non-finite logits other than the masked-out -inf.
    """
    logits = np.atleast_2d(np.asarray(logits, dtype=F64))
    if np.isnan(logits).any() or np.isposinf(logits).any():
        raise ValueError("logits must be finite")
    if not np.isfinite(logits).any(axis=1).all():
        raise ValueError("every row needs a finite logit")
    m = logits.max(axis=1)
    arg = np.argmax(logits, axis=1)          # first (lowest) index among equal maxima
    s = np.exp(logits - m[:, None]).sum(axis=1)
    return 1.0 / s, arg.astype(np.int64)


def entropy(logits):
    """Per row: entropy in nats of the softmax of the raw logits, -sum_v p_v ln p_v.

    The EntropyBoundScheduler and adaptive stopping of the DiffusionGemma docs
    (Schedulers; adaptive stopping) rank and stop on per-token entropy.  The
    masked-out -inf logit has probability 0 and contributes nothing.  Raises
    ValueError on other non-finite logits, like ``confidence``.
    """
    logits = np.atleast_2d(np.asarray(logits, dtype=F64))
    if np.isnan(logits).any() or np.isposinf(logits).any():
        raise ValueError("logits must be finite")
    if not np.isfinite(logits).any(axis=1).all():
        raise ValueError("every row needs a finite logit")
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)                   # exp(-inf) = 0 for the mask id
    p = e / e.sum(axis=1, keepdims=True)
    terms = np.zeros_like(p)
    pos = p > 0
    terms[pos] = p[pos] * np.log(p[pos])
    return -terms.sum(axis=1)
