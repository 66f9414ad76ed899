"""Seeded synthetic inputs for the block-diffusion denoising path.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It holds random draws, shapes and the rounding of drawn values to
bf16-representable numbers -- nothing of the method's arithmetic (no norm, no
attention, no softmax, no commit rule).

Every tensor is drawn from ``numpy.random.default_rng([seed, k])`` with one
stream index ``k`` per tensor, so the same seed gives the same inputs on every
machine.  Values are drawn in float32 and rounded once to bf16 (round to
nearest, ties to even); both the oracle (upcast to float64) and the GPU path
(stored as bf16) consume exactly those values.

Shapes follow the dense decoder described on the MLX-VLM Nemotron Labs
Diffusion guide (section 7, architecture: hidden 4096, 32 query / 8 KV heads of
width 128, SwiGLU 14336, untied head over a 131072 vocabulary, mask token 100,
rope_theta 1e6) with 32 layers, and a tiny model of the same structure.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

# Stream offsets: one per kind of input.
K_WEIGHTS = 0
K_PROMPT = 1
K_CANVAS = 2
K_KV = 3
K_HIDDEN = 4
K_CONF = 5


@dataclass(frozen=True)
class ModelShape:
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    mask_id: int
    rope_base: float
    rms_eps: float = 1e-5

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def with_layers(self, n: int) -> "ModelShape":
        return dataclasses.replace(self, n_layers=n)


# Tiny model: 2 layers, d=128, 4 query / 2 KV heads of width 32, SwiGLU 512,
# vocab 1024 with id 0 = MASK, RoPE base 10000.
TINY = ModelShape(n_layers=2, d_model=128, n_heads=4, n_kv_heads=2, head_dim=32,
                  d_ffn=512, vocab=1024, mask_id=0, rope_base=10000.0)

# 8B-class dense model (32 layers).
DENSE_8B = ModelShape(n_layers=32, d_model=4096, n_heads=32, n_kv_heads=8,
                      head_dim=128, d_ffn=14336, vocab=131072, mask_id=100,
                      rope_base=1.0e6)

# One decoder layer at 8B-class shapes, with the full head.
LAYER_8B = DENSE_8B.with_layers(1)


def rng(seed: int, k: int, *sub: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(k), *[int(s) for s in sub]])


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    out = u.astype(np.uint32).view(np.float32)
    # Keep NaN as NaN (the add above can carry into the exponent of a NaN payload).
    return np.where(np.isnan(a), a, out).reshape(a.shape)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of bf16-representable float32 values, as uint16 (for upload)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def normal(seed: int, k: int, shape, std: float = 1.0, *sub: int) -> np.ndarray:
    g = rng(seed, k, *sub)
    return bf16_round(g.standard_normal(size=shape, dtype=np.float32) * np.float32(std))


def model_weights(shape: ModelShape, seed: int = 0, std: float = 0.02,
                  lm_head_gain: float = 1.0) -> dict:
    """Random-init weights, N(0, std) for matrices and the embedding, ones for norm gains.

    Matrices are [out_features, in_features]; a projection is ``y = x @ W.T``.
    ``lm_head_gain`` scales the head (a test-only knob that makes confidences
    large enough for the threshold branch of the commit rule to fire).
    """
    d, f, v = shape.d_model, shape.d_ffn, shape.vocab
    ones = np.ones(d, dtype=np.float32)
    w = {
        "embed": normal(seed, K_WEIGHTS, (v, d), std, 0),
        "lm_head": normal(seed, K_WEIGHTS, (v, d), std * lm_head_gain, 1),
        "final_norm": ones.copy(),
        "layers": [],
    }
    for i in range(shape.n_layers):
        s = 16 + 16 * i
        w["layers"].append({
            "attn_norm": ones.copy(),
            "wq": normal(seed, K_WEIGHTS, (shape.q_dim, d), std, s + 0),
            "wk": normal(seed, K_WEIGHTS, (shape.kv_dim, d), std, s + 1),
            "wv": normal(seed, K_WEIGHTS, (shape.kv_dim, d), std, s + 2),
            "wo": normal(seed, K_WEIGHTS, (d, shape.q_dim), std, s + 3),
            "ffn_norm": ones.copy(),
            "wg": normal(seed, K_WEIGHTS, (f, d), std, s + 4),
            "wu": normal(seed, K_WEIGHTS, (f, d), std, s + 5),
            "wd": normal(seed, K_WEIGHTS, (d, f), std, s + 6),
        })
    return w


def lora_weights(shape: ModelShape, rank: int = 128, scale: float = 4.0, seed: int = 0,
                 std: float = 0.02) -> dict:
    """Random-init low-rank adapter for every layer's output projection:
    a [rank, H*hd] and b [d, rank], N(0, std) from their own seeded streams."""
    a, b = [], []
    for i in range(shape.n_layers):
        s = 16 + 16 * i
        a.append(normal(seed, K_WEIGHTS, (rank, shape.q_dim), std, s + 7))
        b.append(normal(seed, K_WEIGHTS, (shape.d_model, rank), std, s + 8))
    return {"a": a, "b": b, "scale": float(scale)}


def prompt(shape: ModelShape, batch: int, length: int, seed: int = 0) -> np.ndarray:
    """Uniform random token ids over [0, V) without the mask id, int32 [B, T]."""
    g = rng(seed, K_PROMPT)
    t = g.integers(0, shape.vocab - 1, size=(batch, length), dtype=np.int64)
    t = t + (t >= shape.mask_id)            # skip the mask id
    return t.astype(np.int32)


def ragged_canvas(shape: ModelShape, batch: int, length: int, seed: int = 0,
                  p_masked: float = 0.5):
    """Canvas with each position masked with probability ``p_masked`` (at least one per row).

    Returns (canvas int32 [B, L], masked uint8 [B, L]); masked positions hold the
    mask id, the others hold uniform random non-mask tokens.
    """
    g = rng(seed, K_CANVAS)
    masked = g.random(size=(batch, length)) < p_masked
    for b in range(batch):
        if not masked[b].any():
            masked[b, g.integers(0, length)] = True
    tok = g.integers(0, shape.vocab - 1, size=(batch, length), dtype=np.int64)
    tok = tok + (tok >= shape.mask_id)
    canvas = np.where(masked, shape.mask_id, tok).astype(np.int32)
    return canvas, masked.astype(np.uint8)


def kv_prefix(shape: ModelShape, batch: int, length: int, seed: int = 0, layer: int = 0):
    """N(0,1) key and value prefixes, bf16-rounded, float32 [B, G, P, hd] each.

    Keys are taken as already rotated (they stand for a cached, post-RoPE prefix).
    """
    dims = (batch, shape.n_kv_heads, length, shape.head_dim)
    return (normal(seed, K_KV, dims, 1.0, layer, 0),
            normal(seed, K_KV, dims, 1.0, layer, 1))


def hidden_rows(rows: int, d: int, seed: int = 0, std: float = 1.0) -> np.ndarray:
    return normal(seed, K_HIDDEN, (rows, d), std)


def planted_hidden(lm_head: np.ndarray, rows: int, seed: int = 0):
    """Hidden rows aimed at one head row each, so max-probabilities spread over (0, 1).

    Row r is ``delta_r * W[t_r] / |W[t_r]|^2 + n_r``: its logit for token t_r
    exceeds the others by about delta_r (uniform in [0, ln V + 6]), and the noise
    n_r gives the other logits a spread of about one unit.  Returns
    (hidden float32 [R, d] bf16-rounded, targets int32 [R]).
    """
    g = rng(seed, K_HIDDEN, 7)
    v, d = lm_head.shape
    t = g.integers(0, v, size=rows)
    delta = g.uniform(0.0, np.log(v) + 6.0, size=rows)
    w = lm_head[t].astype(np.float64)
    w2 = (w * w).sum(axis=1, keepdims=True)
    col_rms = np.sqrt(np.mean(lm_head[: min(v, 4096)].astype(np.float64) ** 2))
    noise = g.standard_normal((rows, d)) / (col_rms * np.sqrt(d))
    h = delta[:, None] * w / w2 + noise
    return bf16_round(h.astype(np.float32)), t.astype(np.int32)


def confidences(batch: int, length: int, vocab: int, seed: int = 0, ties: bool = False):
    """Random (conf float32 [B, L], argmax int32 [B, L]) pairs for commit-rule tests.

    With ``ties`` the confidences are drawn from a handful of values so that
    equal confidences (and values right at 0.9) are common.
    """
    g = rng(seed, K_CONF)
    if ties:
        vals = np.array([0.05, 0.3, 0.5, 0.9, 0.9000001, 0.95, 1.0], dtype=np.float32)
        conf = vals[g.integers(0, len(vals), size=(batch, length))]
    else:
        conf = g.random(size=(batch, length), dtype=np.float32)
    arg = g.integers(1, vocab, size=(batch, length)).astype(np.int32)
    return conf.astype(np.float32), arg
