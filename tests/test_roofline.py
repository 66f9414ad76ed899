"""Roofline arithmetic pinned to the teaching model printed on the "Modern LLMs,
Module 12: Diffusion LLMs" page (sec. 1, sec. 10, sec. 11): a dense 8B bf16 model on
a hypothetical 3.35 TB/s, 990 TFLOP/s accelerator.  Each value is compared to the
digits the page prints (tests/golden/teaching_roofline.json)."""
import json
import os

import pytest

from masked_block_diffusion_denoise_amd import roofline as R

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "teaching_roofline.json")))
HW = R.Peaks(hbm_bytes_per_s=G["hbm_bytes_per_s"], flops_per_s=G["flops_per_s"])
P, BPP = G["params"], G["bytes_per_param"]


def digits(x, printed):
    """x rounded to as many decimals as the page printed equals the printed value."""
    s = repr(printed)
    nd = len(s.split(".")[1]) if "." in s else 0
    return round(x, nd) == printed


def test_ar_step_bounds():
    t_mem = R.weight_read_s(P, BPP, HW)
    t_cmp = R.pass_compute_s(P, 1, HW)
    assert digits(t_mem * 1e3, G["ar_step_weight_read_ms"])
    assert digits(t_cmp * 1e6, G["ar_ideal_compute_us"])
    assert digits(100 * t_cmp / t_mem, G["ar_compute_fraction_percent"])
    assert R.pass_s(P, BPP, 1, HW) == t_mem                      # batch 1 AR is weight-bound
    assert digits(R.tokens_per_s_bound(1, 1, t_mem), G["ar_tokens_per_s_bound"])


def test_full_canvas_pass_and_diffusion_bound():
    N, S = G["full_canvas_tokens"], G["dllm_steps"]
    assert digits(2 * P * N / 1e12, G["full_canvas_tflop"])
    t = R.pass_s(P, BPP, N, HW)
    assert t == R.pass_compute_s(P, N, HW)                      # the 1024 canvas is compute-bound
    assert digits(t * 1e3, G["full_canvas_ms"])
    q = R.tokens_per_s_bound(N, S, t)
    assert digits(q, G["dllm_tokens_per_s_bound"])
    ar = R.tokens_per_s_bound(1, 1, R.pass_s(P, BPP, 1, HW))
    s_star = R.parity_passes(N, t, ar)
    assert digits(s_star, G["parity_steps"])
    # the page: 295 whole steps are still (slightly) faster than AR, 296 are not
    assert R.tokens_per_s_bound(N, 295, t) > ar > R.tokens_per_s_bound(N, 296, t)
    assert digits(q / ar, G["batch_crossover"])


def test_block256_bf16_and_int4():
    t_cmp = R.pass_compute_s(P, 256, HW)
    assert digits(t_cmp * 1e3, G["block256_compute_ms"])
    assert R.pass_s(P, BPP, 256, HW) == R.weight_read_s(P, BPP, HW)   # bf16: memory-bound
    t4 = R.weight_read_s(P, 0.5, HW)
    assert digits(t4 * 1e3, G["int4_weight_read_ms"])
    t = R.pass_s(P, 0.5, 256, HW)
    assert t == t_cmp                                                  # 4-bit: compute-bound
    assert digits(R.tokens_per_s_bound(256, G["int4_block256_steps"], t), G["int4_block256_tokens_per_s"])


def test_planted_mistakes_fail():
    # a pass bound that forgot the factor 2 or used the sum instead of the max misses the page's digits
    t_bad = P * 1024 / HW.flops_per_s
    assert not digits(t_bad * 1e3, G["full_canvas_ms"])
    t_sum = R.weight_read_s(P, BPP, HW) + R.pass_compute_s(P, 1024, HW)
    assert not digits(R.tokens_per_s_bound(1024, 64, t_sum), G["dllm_tokens_per_s_bound"])


SHAPE = dict(d=4096, H=32, G=8, hd=128, F=14336, V=131072)


def test_kernel_work_weights_are_one_layer():
    # with no rows, the four projections move exactly one layer's weights once
    n = sum(R.kernel_work(k, 0, 0, 0, 0, **SHAPE)[0] for k in ("qkv", "o_proj", "gate_up", "down"))
    d, H, Gk, hd, F = 4096, 32, 8, 128, 14336
    params = d * (H + 2 * Gk) * hd + H * hd * d + 3 * d * F
    assert n == 2 * params == 436207616


def test_kernel_work_intensity_regimes():
    # batch 1: GEMMs and attention sit below the MI355X ridge (HBM-bound);
    # batch 32 with 512 scored rows: the GEMMs and the head sit above it (MFMA-bound)
    ridge = R.MI355X_BF16.ridge
    for k in ("qkv", "o_proj", "gate_up", "down", "attention", "lm_head"):
        b, f = R.kernel_work(k, 1, 32, 4096, 16, **SHAPE)
        assert f / b < ridge, k
    for k in ("qkv", "gate_up", "down", "lm_head"):
        b, f = R.kernel_work(k, 32, 32, 4096, 512, **SHAPE)
        assert f / b > ridge, k
    b, f = R.kernel_work("attention", 32, 32, 4096, 512, **SHAPE)
    assert f / b < ridge


@pytest.mark.parametrize("ms,bound", [(1.0, "mfma"), (0.1, "mfma")])
def test_roofline_record(ms, bound):
    b, f = R.kernel_work("lm_head", 32, 32, 4096, 512, **SHAPE)
    r = R.roofline(b, f, ms)
    assert r["bound"] == bound and r["unit"] == "TFLOP/s"
    assert r["frac"] == pytest.approx(f / (ms * 1e-3) / 2.5e15, rel=1e-3)


# One 8B-class layer and head (d 4096, 32/8 heads of 128, SwiGLU 14336, vocab
# 131072) over a 4096-position prefix with 32-position canvases; every operand
# counted once, bf16 except the fp32 residual stream (read and written).
#   lm_head:   weights V*d*2 + scored rows r*d*2;        flops 2*r*d*V
#   attention: K and V of prefix + canvas B*4128*8*128*2*2 + q in and o out M*4096*2*2;
#              flops 2*M*32*128*4128 for Q K^T and as much for P V
#   qkv:       weights 6144*4096*2 + rows in M*4096*2 + q/k/v out M*6144*2
#   o_proj:    weights 4096*4096*2 + rows in M*4096*2 + residual M*4096*4*2
#   gate_up:   weights 28672*4096*2 + rows in M*4096*2 + SwiGLU out M*14336*2
#   down:      weights 4096*14336*2 + rows in M*14336*2 + residual M*4096*4*2
# (M = 32 * B canvas rows; r = 496 scored rows at batch 32, 19 at batch 1.)
KERNEL_WORK_BY_HAND = {
    (32, 496): {"lm_head": (1077805056, 532575944704), "attention": (557842432, 69256347648),
                "qkv": (71303168, 51539607552), "o_proj": (75497472, 34359738368),
                "gate_up": (272629760, 240518168576), "down": (180355072, 120259084288)},
    (1, 19): {"lm_head": (1073897472, 20401094656), "attention": (17432576, 2164260864),
              "qkv": (50987008, 1610612736), "o_proj": (34865152, 1073741824),
              "gate_up": (236060672, 7516192768), "down": (119406592, 3758096384)},
}


@pytest.mark.parametrize("B,rows", list(KERNEL_WORK_BY_HAND))
def test_kernel_work_by_hand(B, rows):
    for name, (by, fl) in KERNEL_WORK_BY_HAND[(B, rows)].items():
        assert R.kernel_work(name, B, 32, 4096, rows, **SHAPE) == (by, fl), name
