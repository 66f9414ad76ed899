"""CPU oracle for masked block-diffusion denoising -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 NumPy code that states what the GPU path must compute.
Only the test-suite, the package smoke check and the benchmark's CPU-baseline
leg may import or run anything in this package; the product path never does,
and this package imports nothing from the product package or its compiled
library (the two share only the seeded input generators in ``synth``).

Sources (web pages this follows; cited by title and section):
  [MLX guide]   "MLX-VLM: running NVIDIA Nemotron Labs Diffusion -- AR, block
                diffusion and linear self-speculation decoding" (xxqk.cn):
                sec. 3.3 LoRA adapter, 5.2 samplers, 5.3 head scoring, 6 masked
                block denoising, 7 architecture, 8 linear self-speculation,
                9 statistics.
  [NLD tutorial] "NVlabs/Nemotron-Labs-Diffusion -- Tri-Mode diffusion LM
                tutorial": sec. 3.1 (one set of weights, three decoding loops).
  [DiffusionGemma] diffusers "DiffusionGemma" pipeline docs: Schedulers
                (BlockRefinementScheduler), adaptive stopping.
  [Module 12]   "Modern LLMs, Module 12: Diffusion LLMs": sec. 5 absorbing
                masking, 6 worked example A (reveal schedule), 9 sampling,
                10-11 teaching roofline, 12 level-1 code contracts, 14 block
                diffusion and the KV cache.

Pins (what each function is checked against, in tests/test_oracle_*.py):
  rms_norm, rope, attend     closed forms and hand-computed values
  forward (causal / block)   structural special cases with closed forms,
                             cache == from-scratch recompute with an explicit mask,
                             the SwiGLU FFN (its norm, gate/up roles, residual) and the
                             draft adapter on o_proj (its input, scale, A/B roles) by hand,
                             RoPE on both queries and keys (shift invariance, order)
  head_logits, confidence    hand-computed softmax values, tie and mask rules
  commit and the block loop  step counts fixed by the rule (threshold 1.0 with
                             quota 1 takes L steps; all-confident takes 1),
                             never-remask, forced completion, worked example A
  generate_ar                equals recompute-from-scratch causal argmax decoding
  entropy                    uniform over the V-1 non-mask ids is ln(V-1), a
                             two-way split is the binary entropy, one dominant
                             logit tends to 0
  commit_rule, adaptive_stop hand-worked cases from the page statements
                             (tests/golden/sampler_rules.json and direct cases:
                             the bounded rule's tie at the threshold, the
                             per-step cap), the native rule equal to ``commit``,
                             brute force over tiny cases
  generate_linear_spec       equals generate_ar token for token (lossless), with
                             and without the adaptive window, also on a
                             hand-built model whose drafts are all rejected or
                             all accepted; its trimmed cache equals a causal
                             prefill of prompt + output
Whole-model numeric values of a random-init network are not printed on any
page: beyond the pins above, those are "parity unpinned" (self-consistency only).
"""
from .model import (KVCache, rms_norm, rope, attend, forward, head_logits,
                    confidence, entropy, silu)
from .decode import (commit, commit_batch, linear_mask_schedule, sample_fixed_schedule,
                     generate_block_diffusion, generate_ar, generate_ar_recompute,
                     denoise_logits, append_block, prefill, BlockStats,
                     generate_linear_spec, next_draft_window, commit_rule, adaptive_stop,
                     commit_ex, RULES)

__all__ = [
    "KVCache", "rms_norm", "rope", "attend", "forward", "head_logits", "confidence",
    "silu", "commit", "commit_batch", "linear_mask_schedule", "sample_fixed_schedule",
    "generate_block_diffusion", "generate_ar", "generate_ar_recompute",
    "denoise_logits", "append_block", "prefill", "BlockStats",
    "generate_linear_spec", "next_draft_window", "entropy", "commit_rule", "adaptive_stop",
    "commit_ex", "RULES",
]
