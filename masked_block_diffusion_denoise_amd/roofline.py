"""Roofline arithmetic for the denoising path (host-side, no GPU needed).

Two uses:
  * the teaching model of the "Modern LLMs, Module 12: Diffusion LLMs" page
    (sec. 1, sec. 10 and sec. 11): one forward pass costs at least the larger of
    reading every weight once and doing 2 flops per parameter per position, and
    a decoder that needs S passes for N positions is bounded by N / (S t_pass);
  * the per-kernel bound of the measured step: the algorithmic bytes a kernel
    must move and the flops it must do (not what a particular kernel happens to
    move), against the MI355X peaks.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Peaks:
    hbm_bytes_per_s: float
    flops_per_s: float

    @property
    def ridge(self) -> float:
        """Arithmetic intensity (flop/byte) where the two bounds meet."""
        return self.flops_per_s / self.hbm_bytes_per_s


# AMD's published MI355X figures: 8 TB/s HBM3E, 2.5 PFLOP/s dense bf16 MFMA.
MI355X_BF16 = Peaks(hbm_bytes_per_s=8.0e12, flops_per_s=2.5e15)


# ---------------------------------------------------------------- teaching model
def weight_read_s(params: float, bytes_per_param: float, hw: Peaks) -> float:
    """Time to stream every weight once (the batch-1 lower bound of one pass)."""
    return params * bytes_per_param / hw.hbm_bytes_per_s


def pass_compute_s(params: float, positions: int, hw: Peaks) -> float:
    """Ideal dense arithmetic of one pass: 2 flops per parameter per position."""
    return 2.0 * params * positions / hw.flops_per_s


def pass_s(params: float, bytes_per_param: float, positions: int, hw: Peaks) -> float:
    """Lower bound of one pass over `positions` positions: the larger of the two."""
    return max(weight_read_s(params, bytes_per_param, hw), pass_compute_s(params, positions, hw))


def tokens_per_s_bound(positions: int, passes: int, t_pass: float) -> float:
    """Upper bound on decoded tokens/s when `passes` passes finish `positions` tokens."""
    return positions / (passes * t_pass)


def parity_passes(positions: int, t_pass: float, ar_tokens_per_s: float) -> float:
    """Number of passes at which the diffusion bound falls to the AR bound."""
    return positions / (t_pass * ar_tokens_per_s)


# ---------------------------------------------------------------- measured kernels
def kernel_work(name: str, B: int, L: int, P: int, masked_rows: int, d: int, H: int, G: int, hd: int, F: int,
                V: int) -> tuple[float, float]:
    """(bytes, flops) one launch of `name` must move / compute in one denoise step.

    B rows of L canvas positions each over a P-position cached prefix; the LM head
    scores `masked_rows` rows.  Bytes count each operand read once and each output
    written once: weights bf16, activations bf16, the fp32 residual read and written.
    """
    M = B * L
    if name == "lm_head":          # weights + the scored hidden rows; the logits are never written
        return V * d * 2 + masked_rows * d * 2, 2.0 * masked_rows * d * V
    if name == "attention":        # keys and values of prefix + canvas, q in, o out
        kv = P + L
        return B * kv * G * hd * 2 * 2 + M * H * hd * 2 * 2, 4.0 * B * L * H * hd * kv
    if name == "qkv":
        n = (H + 2 * G) * hd
        return n * d * 2 + M * d * 2 + M * n * 2, 2.0 * M * d * n
    if name == "o_proj":           # residual epilogue: fp32 stream read and written
        return d * H * hd * 2 + M * H * hd * 2 + M * d * 4 * 2, 2.0 * M * H * hd * d
    if name == "gate_up":          # SwiGLU epilogue writes F outputs from 2F columns
        return 2 * F * d * 2 + M * d * 2 + M * F * 2, 2.0 * M * d * 2 * F
    if name == "down":
        return d * F * 2 + M * F * 2 + M * d * 4 * 2, 2.0 * M * F * d
    raise KeyError(name)


def roofline(bytes_: float, flops: float, ms: float, traffic=None, hw: Peaks = MI355X_BF16) -> dict:
    """Achieved rate of a launch of `ms` milliseconds against the bound its intensity selects."""
    s = ms * 1e-3
    if flops / bytes_ >= hw.ridge:
        a = flops / s / 1e12
        peak = hw.flops_per_s / 1e12
        return {"bound": "mfma", "achieved": round(a, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(a / peak, 4), "traffic": traffic}
    a = bytes_ / s / 1e9
    peak = hw.hbm_bytes_per_s / 1e9
    return {"bound": "hbm", "achieved": round(a, 1), "peak": peak, "unit": "GB/s",
            "frac": round(a / peak, 4), "traffic": traffic}
