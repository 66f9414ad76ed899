"""Oracle decoding loops and the commit rule (float64) -- test infrastructure.

Block diffusion (MLX guide, sec. 6; Module 12, sec. 14): the prompt is
prefilled causally into the KV cache; each block of L positions starts fully
masked and is denoised by repeated bidirectional passes against the cached
prefix; after each pass the commit rule unmasks some positions and leaves the
rest masked; when no mask is left the finished block goes through one causal
pass whose keys/values are appended to the cache.

Commit rule (MLX guide, sec. 5.2 native sampler and sec. 6; NLD tutorial,
sec. 3.1; DiffusionGemma, BlockRefinementScheduler), with these readings:
  * candidates are each masked position's argmax, ranked by confidence, ties
    to the smaller position (Module 12, sec. 12 contract);
  * A = {masked j : conf_j > tau} (strictly above the threshold);
  * at least q = min(quota, #masked) positions open per step; on the last
    allowed step every remaining mask is committed (forced completion);
  * n = max(|A|, q) top-ranked positions are committed; the others stay masked;
  * committed positions never change (no editing).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .model import KVCache, forward, head_logits, confidence, entropy


def commit(conf, argmax, canvas, masked, tau, quota, step, max_steps):
    """Apply the commit rule to one row.

    conf, argmax: per-position confidence and candidate ([L]); only masked
    positions are read.  canvas [L] ints, masked [L] bools.  ``step`` is the
    number of denoise steps this row has already taken in the block.
    Returns (canvas, masked, step, n_committed) as new arrays.  A row with no
    mask left is frozen: nothing changes and the step count stays.
    """
    canvas = np.array(canvas, copy=True)
    masked = np.array(masked, dtype=bool, copy=True)
    idx = np.flatnonzero(masked)
    if idx.size == 0:
        return canvas, masked, step, 0
    conf = np.asarray(conf)
    above = [j for j in idx if conf[j] > tau]
    if step >= max_steps - 1:
        q = idx.size                      # forced completion on the last allowed step
    else:
        q = min(int(quota), idx.size)
    n = max(len(above), q)
    ranked = sorted(idx.tolist(), key=lambda j: (-float(conf[j]), j))
    for j in ranked[:n]:
        canvas[j] = argmax[j]
        masked[j] = False
    return canvas, masked, step + 1, n


def commit_batch(conf, argmax, canvas, masked, tau, quota, steps, max_steps):
    """Row-wise ``commit`` over a batch; tau and quota may be scalars or per row.

    Returns (canvas, masked, steps, n_committed, n_left) as new arrays.
    """
    b = np.asarray(canvas).shape[0]
    tau = np.broadcast_to(np.asarray(tau), (b,))
    quota = np.broadcast_to(np.asarray(quota), (b,))
    out_c, out_m, out_s, out_n = [], [], [], []
    for r in range(b):
        c, m, s, n = commit(conf[r], argmax[r], canvas[r], masked[r], tau[r], quota[r],
                            int(steps[r]), max_steps)
        out_c.append(c)
        out_m.append(m)
        out_s.append(s)
        out_n.append(n)
    masked_new = np.array(out_m)
    return (np.array(out_c), masked_new, np.array(out_s), np.array(out_n),
            masked_new.sum(axis=1))


# ------------------------------------------------------ sampler variants ----
# The other samplers of the pages, as commit rules of one row.  Where the GPU
# decides an integer from float32 values (a threshold test, a cumulative sum, a
# mean), the same float32 operations are done here in the same order, on the
# float32 inputs both sides are given.
RULES = ("threshold", "bound", "entropy")
F32 = np.float32


def _bound_threshold(j, scaling):
    """Position-dependent threshold 1 - scaling / (j + 2) of the bounded sampler, in float32."""
    return F32(1.0) - F32(scaling) / F32(j + 2)


def commit_rule(conf, argmax, canvas, masked, tau, quota, step, max_steps, rule="threshold",
                min_threshold=0.45, scaling=2.0, entropy=None, entropy_bound=0.1, max_transfer=0):
    """Commit rules of the samplers on the pages, one row; returns
    (canvas, masked, step, n_committed) like ``commit``.

    rule "threshold" (native; MLX guide sec. 5.2): A = {masked j : conf_j > tau}.
    rule "bound" (confidence_threshold_bound; MLX guide sec. 5.2): a position
      qualifies when its confidence reaches the global threshold, conf_j >= tau,
      or is at least min_threshold (0.45) and at least the position-dependent
      threshold 1 - scaling / (j + 2) (scaling 2.0); j is the position in the
      block (a reading: the page names the position without its origin).
    rule "entropy" (EntropyBoundScheduler; DiffusionGemma docs, Schedulers):
      masked positions in order of (entropy, position); A is the longest prefix
      whose cumulative entropy (float32, in that order) stays <= entropy_bound.
    Then, as for the native rule: on the last allowed step every remaining mask
    is committed; otherwise at least q = min(quota, #masked) positions open --
    A when |A| >= q, else A plus the best-ranked others -- and with
    max_transfer > 0 (MLX guide sec. 5.5, --max-transfer-per-step) at most that
    many, the best-ranked of the chosen.  Ranking: (-conf, position) for the
    confidence rules, (entropy, position) for the entropy rule.
    """
    if rule not in RULES:
        raise ValueError(f"unknown rule {rule!r}")
    canvas = np.array(canvas, copy=True)
    masked = np.array(masked, dtype=bool, copy=True)
    idx = np.flatnonzero(masked).tolist()
    if not idx:
        return canvas, masked, step, 0
    conf = np.asarray(conf, dtype=F32)
    if rule == "entropy":
        if entropy is None:
            raise ValueError("the entropy rule needs per-position entropies")
        ent = np.asarray(entropy, dtype=F32)
        key = lambda j: (float(ent[j]), j)
    else:
        key = lambda j: (-float(conf[j]), j)
    ranked = sorted(idx, key=key)
    if step >= max_steps - 1:
        chosen = ranked                      # forced completion
    else:
        if rule == "threshold":
            A = [j for j in ranked if conf[j] > F32(tau)]
        elif rule == "bound":
            A = [j for j in ranked if conf[j] >= F32(tau) or
                 (conf[j] >= F32(min_threshold) and conf[j] >= _bound_threshold(j, scaling))]
        else:
            A, total = [], F32(0.0)
            for j in ranked:
                total = F32(total + ent[j])
                if total > F32(entropy_bound):
                    break
                A.append(j)
        q = min(int(quota), len(idx))
        chosen = A + [j for j in ranked if j not in A][:max(0, q - len(A))]
        if max_transfer > 0 and len(chosen) > max_transfer:
            chosen = sorted(chosen, key=key)[:max_transfer]
    for j in chosen:
        canvas[j] = argmax[j]
        masked[j] = False
    return canvas, masked, step + 1, len(chosen)


def adaptive_stop(argmax, prev_argmax, masked, entropy, stable, stability_steps, stop_entropy):
    """Adaptive stopping of one row (DiffusionGemma docs, adaptive stopping).

    ``stable`` counts the consecutive steps whose argmax at every masked
    position equals the previous step's (prev_argmax; -1 before the first step
    of a block).  The row stops when that count reaches stability_steps and the
    mean entropy of its masked positions (float32 sum in position order, then
    the division) is below stop_entropy (0.005 for the published checkpoint);
    a stopped row commits every remaining mask with its argmax (a reading: the
    page freezes the sample's current predictions).  Returns (stop, stable).
    """
    idx = np.flatnonzero(np.asarray(masked, dtype=bool))
    if idx.size == 0:
        return False, stable
    same = all(int(argmax[j]) == int(prev_argmax[j]) for j in idx)
    stable = stable + 1 if same else 0
    total = F32(0.0)
    for j in idx:
        total = F32(total + F32(entropy[j]))
    mean = F32(total / F32(idx.size))
    return bool(stable >= stability_steps and mean < F32(stop_entropy)), stable


def commit_ex(conf, argmax, canvas, masked, tau, quota, step, max_steps, entropy=None,
              prev_argmax=None, stable=0, stability_steps=0, stop_entropy=0.005, **rule_kw):
    """``commit_rule`` preceded by adaptive stopping when stability_steps > 0.

    Returns (canvas, masked, step, n_committed, prev_argmax, stable): prev_argmax
    takes this step's argmax at the positions that were masked.
    """
    masked = np.asarray(masked, dtype=bool)
    if stability_steps > 0:
        stop, stable = adaptive_stop(argmax, prev_argmax, masked, entropy, stable, stability_steps,
                                     stop_entropy)
        prev_argmax = np.array(prev_argmax, copy=True)
        prev_argmax[masked] = np.asarray(argmax)[masked]
        if stop:
            idx = np.flatnonzero(masked)
            canvas = np.array(canvas, copy=True)
            canvas[idx] = np.asarray(argmax)[idx]
            return canvas, np.zeros_like(masked), step + 1, int(idx.size), prev_argmax, stable
    c, m, s, n = commit_rule(conf, argmax, canvas, masked, tau, quota, step, max_steps, entropy=entropy,
                             **rule_kw)
    return c, m, s, n, prev_argmax, stable


def linear_mask_schedule(length: int, steps: int):
    """Target mask counts m_s = ceil(N (S - s) / S), s = 0..S (Module 12, sec. 6)."""
    if length <= 0 or steps <= 0:
        raise ValueError("length and steps must be positive")
    return tuple(-(-(length * (steps - s)) // steps) for s in range(steps + 1))


def sample_fixed_schedule(predict, length, steps, mask_id):
    """Greedy confidence reveal opening exactly the scheduled number of positions per call.

    ``predict(tokens, step)`` returns logits [L, V]; one call per iteration.
    Uses the commit rule with an unreachable threshold and the per-step quota
    m_{s-1} - m_s, so it is the Module 12 sec. 9/12 sampler expressed through
    ``commit``.  Returns (tokens, trace) with trace = [(opened positions, tokens)].
    """
    sched = linear_mask_schedule(length, steps)
    tokens = np.full(length, mask_id, dtype=np.int64)
    masked = np.ones(length, dtype=bool)
    trace = []
    for s in range(1, steps + 1):
        logits = np.asarray(predict(tokens.copy(), s), dtype=np.float64)
        conf, arg = confidence(logits)
        before = masked.copy()
        quota = sched[s - 1] - sched[s]
        tokens, masked, _, _ = commit(conf, arg, tokens, masked, np.inf, quota, s - 1,
                                      steps + 1)
        opened = tuple(np.flatnonzero(before & ~masked).tolist())
        trace.append((opened, tokens.copy()))
    return tokens, trace


def prefill(w, shape, prompt):
    """Causal pass over the prompt; returns (cache, final residual stream [T, d])."""
    cache = KVCache(shape)
    x = forward(w, shape, prompt, cache, mode="causal", write_cache=True)
    return cache, x


def denoise_logits(w, shape, cache, canvas, lora=None):
    """One bidirectional-block pass of the canvas against the cached prefix; no cache write."""
    x = forward(w, shape, canvas, cache, mode="block", write_cache=False, lora=lora)
    return head_logits(w, shape, x)


def append_block(w, shape, cache, block):
    """Causal pass of the finished block; its keys/values are appended to the cache."""
    return forward(w, shape, block, cache, mode="causal", write_cache=True)


@dataclass
class BlockStats:
    """Counters of the MLX guide, sec. 9 (denoise and post-block forwards, tokens per forward)."""
    denoise_nfe: int = 0
    post_block_nfe: int = 0
    blocks: int = 0
    accepted_tokens: int = 0
    masked_rows_scored: int = 0
    steps_per_block: list = field(default_factory=list)
    trace: list = field(default_factory=list)

    @property
    def tokens_per_denoise_forward(self) -> float:
        return self.accepted_tokens / max(self.denoise_nfe, 1)


def generate_block_diffusion(w, shape, prompt, gen_length, block_length, max_steps,
                             tau=0.9, quota=1, keep_trace=False, sampler=None, anchor=False):
    """Block-diffusion decoding of one sequence; returns (generated tokens, stats, cache).

    All block positions start as the mask id; with ``anchor`` (the MLX guide's
    native layout, sec. 6) position 0 of each block instead holds the causal
    argmax after everything before the block -- from the prompt's prefill for
    the first block, from the previous block's post-block pass after that --
    and only positions 1..L-1 are denoised.  A generation length that is not a
    multiple of the block length is rounded up.  With
    ``sampler`` (keyword arguments of ``commit_ex``: rule, min_threshold,
    scaling, entropy_bound, max_transfer, stability_steps, stop_entropy) the
    step uses that commit rule; confidences and entropies are rounded to float32
    first, as the device computes them.
    """
    cache, x = prefill(w, shape, prompt)
    n_blocks = -(-gen_length // block_length)
    out = []
    st = BlockStats()
    for _ in range(n_blocks):
        canvas = np.full(block_length, shape.mask_id, dtype=np.int64)
        masked = np.ones(block_length, dtype=bool)
        if anchor:
            canvas[0] = int(np.argmax(head_logits(w, shape, x[-1:])[0]))
            masked[0] = False
        step = 0
        prev, stable = np.full(block_length, -1), 0
        while masked.any():
            logits = denoise_logits(w, shape, cache, canvas)
            st.masked_rows_scored += int(masked.sum())
            conf, arg = confidence(logits)
            if sampler is None:
                canvas, masked_new, step, n = commit(conf, arg, canvas, masked, tau, quota,
                                                     step, max_steps)
            else:
                ent = entropy(logits).astype(np.float32)
                canvas, masked_new, step, n, prev, stable = commit_ex(
                    conf.astype(np.float32), arg, canvas, masked, tau, quota, step, max_steps, entropy=ent,
                    prev_argmax=prev, stable=stable, **sampler)
            if keep_trace:
                st.trace.append((tuple(np.flatnonzero(masked & ~masked_new).tolist()),
                                 canvas.copy()))
            masked = masked_new
            st.denoise_nfe += 1
            st.accepted_tokens += n
        x = append_block(w, shape, cache, canvas)
        st.post_block_nfe += 1
        st.blocks += 1
        st.steps_per_block.append(step)
        out.extend(canvas.tolist())
    return np.array(out, dtype=np.int64), st, cache


def generate_ar(w, shape, prompt, n_new):
    """Greedy causal decoding with the KV cache (MLX guide, sec. 3.1 autoregressive path)."""
    cache = KVCache(shape)
    x = forward(w, shape, prompt, cache, mode="causal", write_cache=True)
    out = []
    for i in range(n_new):
        _, arg = confidence(head_logits(w, shape, x[-1:]))
        tok = int(arg[0])
        out.append(tok)
        if i + 1 < n_new:
            x = forward(w, shape, np.array([tok]), cache, mode="causal", write_cache=True)
    return np.array(out, dtype=np.int64)


def generate_ar_recompute(w, shape, prompt, n_new):
    """Greedy decoding that re-runs the whole sequence causally each step, without a cache."""
    seq = list(np.asarray(prompt).tolist())
    out = []
    for _ in range(n_new):
        x = forward(w, shape, np.array(seq), None, mode="causal")
        _, arg = confidence(head_logits(w, shape, x[-1:]))
        out.append(int(arg[0]))
        seq.append(int(arg[0]))
    return np.array(out, dtype=np.int64)


# ------------------------------------------------------------ linear self-speculation
def next_draft_window(window, accepted, max_window=32, min_window=2):
    """Adaptive draft window of linear self-speculation (MLX guide, sec. 8): it
    starts at 8, doubles (up to 32) when a round accepts every draft token, and
    halves when at most half of them are accepted.  ``window`` counts the known
    token plus window - 1 drafted positions; the floor of 2 keeps one drafted
    position (a reading: the page gives no lower bound)."""
    drafts = window - 1
    if accepted == drafts:
        return min(window * 2, max_window)
    if accepted * 2 <= drafts:
        return max(window // 2, min_window)
    return window


def generate_linear_spec(w, shape, prompt, n_new, lora, window=32, adaptive=False):
    """Linear self-speculation, greedy (MLX guide, sec. 8; NLD tutorial, sec. 3.1).

    Each round drafts a block with one bidirectional pass of the canvas
    [t, MASK x (W - 1)] -- t is the next token, already known -- with the LoRA
    adapter on, taking the argmax of every masked position.  A causal pass over
    [t, drafts] with the adapter off then verifies them: the longest prefix of
    drafts equal to the causal argmax is accepted, and the causal argmax after it
    is the next known token (the correction).  The cache is trimmed back to the
    known token and the accepted drafts.  Every emitted token is the greedy
    causal prediction of its prefix, so the output equals ``generate_ar``.

    Returns (tokens [n_new], accepted drafts per round, windows per round, cache).
    """
    cache, x = prefill(w, shape, prompt)
    _, arg = confidence(head_logits(w, shape, x[-1:]))
    nxt = int(arg[0])
    out, accepted, windows = [], [], []
    W = 8 if adaptive else window
    while len(out) < n_new:
        p0 = cache.length
        canvas = np.array([nxt] + [shape.mask_id] * (W - 1), dtype=np.int64)
        _, drafts = confidence(denoise_logits(w, shape, cache, canvas, lora=lora))
        drafts = drafts[1:]
        block = np.concatenate([[nxt], drafts])
        xv = append_block(w, shape, cache, block)
        _, ver = confidence(head_logits(w, shape, xv))   # ver[j]: causal argmax after block[j]
        a = 0
        while a < W - 1 and drafts[a] == ver[a]:
            a += 1
        out.extend(block[:a + 1].tolist())
        nxt = int(ver[a])
        cache.truncate(p0 + a + 1)
        accepted.append(a)
        windows.append(W)
        if adaptive:
            W = next_draft_window(W, a)
    return np.array(out[:n_new], dtype=np.int64), accepted, windows, cache
