"""bf16 MFMA GEMM epilogues vs float64 products of the same bf16 values.

Shapes cover the skinny paths (M <= 64, with and without split-K, 128- and
256-wide weight tiles), each tile shape of the tiled path (M > 64, ragged last
row tile) and the 8B-class projection sizes.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import announce, bf16, f32, host, p, rel_rms, stream, sync, workspace
from masked_block_diffusion_denoise_amd import _lib as L

pytestmark = pytest.mark.gpu

SHAPES = [(16, 256, 128), (13, 1024, 512), (32, 6144, 4096), (64, 384, 256), (32, 4096, 14336),
          (128, 256, 128), (200, 384, 512), (1024, 512, 4096), (96, 1024, 1024),
          # the tiny model's projections (K parts of one or no 32-deep step per wavefront)
          (32, 256, 128), (32, 128, 128), (32, 128, 512), (64, 256, 128), (48, 128, 512), (2, 1024, 128),
          (80, 256, 128),
          # short and wide: 256 x 64 tiles, K split (ragged rows)
          (20, 32768, 2048),
          # more than one 128 x 128 tile per CU, at most one 192 x 128 tile per CU (ragged rows),
          # and the QKV projection of the 8B-class model at batch 32
          (1000, 4608, 256), (1024, 6144, 4096),
          # 192 x 128 tiles whose last row tile leaves one wavefront a single live fragment (plain ring)
          (968, 6144, 512),
          # long K with few 256 x 256 tiles: K split, weight tiles fastest in the tile order
          # (the down projection at batch 32; ragged rows over an 8-way split)
          (1024, 4096, 14336), (520, 1024, 8192),
          # the O projection at batch 32 (128 x 128 tiles, one per CU)
          (1024, 4096, 4096),
          # more than one 128 x 128 or 192 x 128 tile per CU, too few 256 x 256 tiles:
          # 256 x 128 (ragged rows)
          (1000, 5120, 256),
          # at most one 128 x 128 tile per CU, several row tiles (ragged rows)
          (1000, 2048, 256),
          # at least one 256 x 256 tile per CU: one 64-deep stage, two, three (ragged rows; the last
          # row tile's second wavefront row is idle), the split ring's activation buffers reused
          (520, 32768, 64), (520, 32768, 128), (520, 32768, 192), (264, 65536, 512),
          # long K over few 256 x 256 tiles: K split into 8 parts of 16 stages
          (300, 1024, 8192)]


def operands(M, N, K, seed):
    a = synth.normal(seed, 90, (M, K), 1.0)
    w = synth.normal(seed, 91, (N, K), 0.02)
    return a, w


def run(a, w, epi, out, M, N, K, ldc):
    ta, tw = bf16(a), bf16(w)
    ws, n = workspace(L.load().dlm_op_gemm_workspace_bytes(M, N, K))
    L.call("dlm_op_gemm", p(ta), p(tw), p(out), M, N, K, K, ldc, epi, ws, n, stream())
    sync()


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_store_bf16(M, N, K):
    announce(f"gemm store {M}x{N}x{K}")
    a, w = operands(M, N, K, 1)
    out = torch.zeros(M, N, dtype=torch.bfloat16, device="cuda")
    run(a, w, L.EPI_STORE_BF16, out, M, N, K, N)
    want = a.astype(np.float64) @ w.astype(np.float64).T
    got = host(out)
    assert rel_rms(got, want) < 4e-3
    assert np.abs(got - want).max() <= 2 ** -7 * np.abs(want).max() + 1e-6


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_residual_f32(M, N, K):
    announce(f"gemm residual {M}x{N}x{K}")
    a, w = operands(M, N, K, 2)
    x0 = synth.normal(2, 92, (M, N), 1.0)
    out = f32(x0)
    run(a, w, L.EPI_RESIDUAL_F32, out, M, N, K, N)
    prod = a.astype(np.float64) @ w.astype(np.float64).T
    got = host(out) - x0
    # fp32 accumulation of bf16 products: relative error of the product ~ K * 2^-24
    assert rel_rms(got, prod) < 1e-5 * max(1.0, np.sqrt(K / 128))


@pytest.mark.parametrize("M,N,K", [(16, 1024, 128), (32, 28672, 4096), (40, 512, 256), (160, 1024, 512),
                                   (1024, 2048, 4096), (32, 1024, 128), (64, 1024, 128), (80, 1024, 128),
                                   (1000, 4608, 256), (520, 32768, 128)])
def test_gemm_swiglu(M, N, K):
    announce(f"gemm swiglu {M}x{N}x{K}")
    a, w = operands(M, N, K, 3)
    out = torch.zeros(M, N // 2, dtype=torch.bfloat16, device="cuda")
    run(a, w, L.EPI_SWIGLU, out, M, N, K, N // 2)
    wr = w.reshape(N // 32, 2, 16, K)
    wg = wr[:, 0].reshape(N // 2, K).astype(np.float64)
    wu = wr[:, 1].reshape(N // 2, K).astype(np.float64)
    a64 = a.astype(np.float64)
    want = oracle.silu(a64 @ wg.T) * (a64 @ wu.T)
    assert rel_rms(host(out), want) < 5e-3


def test_gemm_split_k_is_deterministic():
    announce("gemm determinism")
    M, N, K = 32, 4096, 14336
    a, w = operands(M, N, K, 4)
    outs = []
    for _ in range(3):
        out = torch.zeros(M, N, dtype=torch.float32, device="cuda")
        run(a, w, L.EPI_RESIDUAL_F32, out, M, N, K, N)
        outs.append(host(out))
    assert (outs[0] == outs[1]).all() and (outs[0] == outs[2]).all()
