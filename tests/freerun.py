"""End-to-end comparison of free-running block diffusion with the oracle.

The exactness rule: committed tokens must equal the oracle's at every position
whose oracle top-1 margin (logit gap l1 - l2) and threshold distance
|conf - tau| both exceed 5e-2.  Two checks make it concrete.

* ``oracle_run`` + ``compare_until_ambiguity``: the oracle decodes on its own
  and marks the first step whose decision it takes with less than 5e-2 to
  spare (a masked position within 5e-2 of the threshold, a log-confidence gap
  below 5e-2 between the last committed and the first left position of the
  (-conf, position) ranking, or a committed position with a top-1 margin below
  5e-2), each margin widened to twice what bf16 storage alone moves the
  quantity where that is larger (a large test head gain).  Every canvas before
  that step must be identical on the device.

* ``check_trajectory_step``: the device decodes on its own; at each step the
  oracle scores the device's canvas (with a cache built from the device's own
  committed blocks) and the device's commit must be one the rule allows:
  tokens equal to the oracle's argmax where its margin exceeds 5e-2 (within
  5e-2 of the top logit otherwise), every position clearly above the threshold
  committed, nothing clearly less confident committed ahead of a position left
  masked, at least the quota, and beyond the quota only positions that may be
  above the threshold.  Where the decision is unambiguous this leaves exactly
  the oracle's commit.

Rule sources: MLX guide sec. 5.2 and 6 (native sampler: threshold, at least one
per step, completion on the last step), Module 12 sec. 12 (one call per step,
ranking ties to the smaller position).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

import oracle

MARGIN = 5e-2


@dataclass
class Step:
    block: int
    step: int              # step within the block
    canvas_after: np.ndarray
    masked_after: np.ndarray
    ambiguous: list        # reasons this step's decision is within MARGIN ([] if clear)
    canvas_before: np.ndarray = None
    masked_before: np.ndarray = None
    logits: np.ndarray = None
    last: bool = False     # the block's last allowed step


def step_ambiguity(logits, conf, masked, committed, n, tau, last, margin=MARGIN, logits_16=None):
    """Reasons the oracle's commit at this step is within ``margin`` of another decision.

    With ``logits_16`` (the same step under bf16 storage alone, bf16_storage),
    each margin is at least twice what bf16 storage alone moves the quantity it
    guards -- confidences for the threshold, log-confidences for the selection,
    logits for the tokens -- since no bf16-storage implementation is held to a
    finer decision than that."""
    mk = np.flatnonzero(masked)
    m_c = m_s = m_t = margin
    if logits_16 is not None:
        conf_16, _ = oracle.confidence(logits_16)
        m_c = max(margin, 2.0 * np.abs(conf_16 - conf)[mk].max())
        m_s = max(margin, 2.0 * np.abs(np.log(conf_16) - np.log(conf))[mk].max())
        fin = np.isfinite(logits[0])
        m_t = max([margin] + [2.0 * np.abs(logits_16[j][fin] - logits[j][fin]).max() for j in committed])
    why = []
    if not last and np.abs(conf[mk] - tau).min() < m_c:
        why.append("threshold")
    ranked = sorted(mk.tolist(), key=lambda j: (-conf[j], j))
    if n < len(ranked) and np.log(conf[ranked[n - 1]]) - np.log(conf[ranked[n]]) < m_s:
        why.append("selection")
    for j in committed:
        top2 = np.sort(logits[j][np.isfinite(logits[j])])[-2:]
        if top2[1] - top2[0] < m_t:
            why.append("token")
            break
    return why


def oracle_run(w, shape, prompt, n_blocks, Lb, max_steps, tau, quota=1, margin=MARGIN, bf16_margins=True):
    """The oracle's own free-running decode, step by step, with each step's
    ambiguity (margins widened by bf16 storage's own effect when
    ``bf16_margins``: the same canvases scored with bf16_storage)."""
    import bf16_storage
    cache, _ = oracle.prefill(w, shape, prompt)
    cache16 = bf16_storage.prefill(w, shape, prompt) if bf16_margins else None
    steps = []
    for blk in range(n_blocks):
        canvas = np.full(Lb, shape.mask_id, np.int64)
        masked = np.ones(Lb, bool)
        s = 0
        while masked.any():
            lo = oracle.denoise_logits(w, shape, cache, canvas)
            conf, arg = oracle.confidence(lo)
            c2, m2, s2, n = oracle.commit(conf, arg, canvas, masked, tau, quota, s, max_steps)
            committed = np.flatnonzero(masked & ~m2)
            lo16 = bf16_storage.denoise_logits(w, shape, cache16, canvas) if bf16_margins else None
            why = step_ambiguity(lo, conf, masked, committed, n, tau, s >= max_steps - 1, margin, lo16)
            steps.append(Step(blk, s, c2.copy(), m2.copy(), why, canvas.copy(), masked.copy(), lo,
                              s >= max_steps - 1))
            canvas, masked, s = c2, m2, s2
        oracle.append_block(w, shape, cache, canvas)
        if bf16_margins:
            bf16_storage.append_block(w, shape, cache16, canvas)
    return steps


def first_ambiguous(steps):
    for i, st in enumerate(steps):
        if st.ambiguous:
            return i
    return len(steps)


def compare_until_ambiguity(steps, device_canvases):
    """Assert the device's canvas after each step equals the oracle's up to the
    oracle's first ambiguous step.  Returns (first ambiguous step index, number
    of whole blocks compared)."""
    stop = first_ambiguous(steps)
    assert len(device_canvases) >= stop, f"device ran {len(device_canvases)} steps, oracle {stop} clear ones"
    for i in range(stop):
        got, want = np.asarray(device_canvases[i]), steps[i].canvas_after
        assert np.array_equal(got, want), (
            f"step {i} (block {steps[i].block}, step {steps[i].step}): device {got.tolist()} "
            f"!= oracle {want.tolist()}")
    blocks = sum(1 for i in range(stop) if not steps[i].masked_after.any())
    return stop, blocks


def check_trajectory_step(logits, canvas, masked, canvas_after, masked_after, tau, quota, last,
                          mask_id, margin=MARGIN):
    """Check one device commit against the oracle's scores of the same canvas.

    logits: the oracle's [L, V] logits for ``canvas``; canvas/masked before the
    step, canvas_after/masked_after the device's result.  Returns the number of
    committed positions whose token was checked exactly (margin above ``margin``).
    """
    conf, arg = oracle.confidence(logits)
    canvas, masked = np.asarray(canvas), np.asarray(masked, bool)
    canvas_after, masked_after = np.asarray(canvas_after), np.asarray(masked_after, bool)
    mk = np.flatnonzero(masked)
    assert not (masked_after & ~masked).any(), "a committed position was remasked"
    kept = ~masked
    assert np.array_equal(canvas_after[kept], canvas[kept]), "a committed token changed"
    com = np.flatnonzero(masked & ~masked_after)
    left = np.flatnonzero(masked_after)
    assert (canvas_after[left] == mask_id).all(), "a masked position holds a token"
    exact = 0
    for j in com:
        fin = logits[j][np.isfinite(logits[j])]
        top2 = np.sort(fin)[-2:]
        if top2[1] - top2[0] > margin:
            assert canvas_after[j] == arg[j], f"position {j}: token {canvas_after[j]} != oracle {arg[j]}"
            exact += 1
        else:
            assert canvas_after[j] != mask_id and logits[j][canvas_after[j]] >= top2[1] - margin, (
                f"position {j}: token {canvas_after[j]} is not a near-top candidate")
    if last:
        assert len(left) == 0, "the last allowed step must commit every remaining mask"
        return exact
    q = min(int(quota), len(mk))
    assert len(com) >= q, f"{len(com)} committed, quota {q}"
    for j in mk:
        if conf[j] > tau + margin:
            assert j in com, f"position {j} (conf {conf[j]:.4f}) is clearly above the threshold"
    if len(com) > q:  # more than the quota: the committed set is the threshold set
        for j in com:
            assert conf[j] > tau - margin, (
                f"position {j} (conf {conf[j]:.4f}) committed beyond the quota but clearly below the threshold")
    for j in com:
        for k in left:
            assert np.log(conf[k]) - np.log(conf[j]) < margin, (
                f"position {j} (conf {conf[j]:.4g}) committed ahead of position {k} (conf {conf[k]:.4g})")
    return exact
