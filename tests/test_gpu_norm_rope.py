"""RMSNorm and RoPE + KV-cache write vs the oracle; cache placement exact."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import announce, bf16, f32, host, i32, p, stream, sync, workspace
from masked_block_diffusion_denoise_amd import _lib as L

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,d", [(1, 128), (37, 4096), (1024, 4096), (5, 64)])
def test_rmsnorm(M, d):
    announce(f"rmsnorm {M}x{d}")
    x = synth.normal(0, 80, (M, d), 3.0)
    g = synth.normal(0, 81, (d,), 1.0)
    out = torch.zeros(M, d, dtype=torch.bfloat16, device="cuda")
    tx, tg = f32(x), bf16(g)
    L.call("dlm_op_rmsnorm", p(tx), M, d, p(tg), 1e-5, p(out), stream())
    sync()
    want = oracle.rms_norm(x, g, 1e-5)
    got = host(out)
    # one bf16 rounding of the result: |err| <= 2^-8 |value|
    assert np.all(np.abs(got - want) <= 2 ** -8 * np.abs(want) + 1e-30)


@pytest.mark.parametrize("H,G,hd,base", [(4, 2, 32, 1e4), (32, 8, 128, 1e6)])
@pytest.mark.parametrize("Lq", [32, 13])  # 13: groups of 16 rows span two batch rows
def test_rope_kv_write(H, G, hd, base, Lq):
    announce(f"rope H={H} G={G} hd={hd} Lq={Lq}")
    B, cap = 3, 70144
    prefix = np.array([0, 100, 70000], dtype=np.int32)
    off = 5
    nh = H + 2 * G
    qkv = synth.normal(1, 82, (B * Lq, nh * hd), 1.0)
    tq = bf16(qkv)
    sentinel = torch.tensor(7.0, dtype=torch.bfloat16)
    kc = torch.full((B * G * cap * hd,), 7.0, dtype=torch.bfloat16, device="cuda")
    vc = torch.full((B * G * cap * hd,), 7.0, dtype=torch.bfloat16, device="cuda")
    tp = i32(prefix)
    ws, n = workspace(L.load().dlm_op_rope_workspace_bytes(B, Lq, hd))
    # rows of batch row 2 reach positions 70005..70036 < cap; nothing beyond cap is written
    L.call("dlm_op_rope_kv", p(tq), B, Lq, H, G, hd, base, p(kc), p(vc), p(tp), off, cap, ws, n, stream())
    sync()
    got_q = host(tq).reshape(B, Lq, nh, hd)
    kl = host(kc).reshape(B, G, cap, hd)
    vl = host(vc).reshape(B, G, cap // 16, hd, 16).transpose(0, 1, 2, 4, 3).reshape(B, G, cap, hd)
    x = qkv.reshape(B, Lq, nh, hd).astype(np.float64)
    written = np.zeros((B, cap), bool)
    for b in range(B):
        pos = prefix[b] + off + np.arange(Lq)
        written[b, pos] = True
        q_want = oracle.rope(x[b, :, :H].transpose(1, 0, 2), pos, base).transpose(1, 0, 2)
        k_want = oracle.rope(x[b, :, H:H + G].transpose(1, 0, 2), pos, base)
        assert np.all(np.abs(got_q[b, :, :H] - q_want) <= 2 ** -8 * np.abs(q_want) + 2e-5)
        assert np.all(np.abs(kl[b][:, pos] - k_want) <= 2 ** -8 * np.abs(k_want) + 2e-5)
        np.testing.assert_array_equal(vl[b][:, pos], x[b, :, H + G:].transpose(1, 0, 2))
    # key/value heads of the qkv rows are left as they were
    np.testing.assert_array_equal(got_q[:, :, H:], qkv.reshape(B, Lq, nh, hd)[:, :, H:])
    # every other cache slot still holds the sentinel
    assert (kl.transpose(0, 2, 1, 3)[~written] == 7.0).all()
    assert (vl.transpose(0, 2, 1, 3)[~written] == 7.0).all()
