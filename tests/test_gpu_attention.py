"""Block attention (bidirectional canvas, causal passes, split-KV) vs the oracle's
brute-force attention with an explicit mask."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import announce, bf16, host, i32, p, rel_rms, stream, sync, workspace
from masked_block_diffusion_denoise_amd import _lib as L

pytestmark = pytest.mark.gpu


def run_case(B, Lq, H, G, hd, prefix, pos_offset, causal, seed, check_rows=None, poison=False):
    p0 = (np.zeros(B, np.int64) if prefix is None else np.asarray(prefix)) + pos_offset
    kv_len = p0 + Lq
    max_kv = int(kv_len.max())
    cap = (max_kv + 63) // 64 * 64 + 64
    q = synth.normal(seed, 70, (B * Lq, H * hd), 1.0)
    k = synth.normal(seed, 71, (B, G, cap, hd), 1.0)
    v = synth.normal(seed, 72, (B, G, cap, hd), 1.0)
    if poison:  # cache slots past a row's end may hold anything, NaN and Inf included
        for b in range(B):
            k[b, :, kv_len[b]:] = np.nan
            v[b, :, kv_len[b]:] = np.inf
    vb = v.reshape(B, G, cap // 16, 16, hd).transpose(0, 1, 2, 4, 3)  # blocked layout
    tq, tk, tv = bf16(q), bf16(k), bf16(np.ascontiguousarray(vb))
    to = torch.zeros(B * Lq, H * hd, dtype=torch.bfloat16, device="cuda")
    tp = None if prefix is None else i32(prefix)
    ws, n = workspace(L.load().dlm_op_attention_workspace_bytes(B, Lq, H, G, hd, max_kv))
    L.call("dlm_op_attention", p(tq), H * hd, p(tk), p(tv), p(to), p(tp), pos_offset, B, Lq, H, G, hd, cap,
           int(causal), max_kv, ws, n, stream())
    sync()
    got = host(to).reshape(B, Lq, H, hd)
    rows = range(B) if check_rows is None else check_rows
    for b in rows:
        n_keys = int(kv_len[b])
        qpos = p0[b] + np.arange(Lq)
        keys = np.arange(n_keys)
        allowed = (keys[None, :] <= qpos[:, None]) if causal else np.ones((Lq, n_keys), bool)
        want = oracle.attend(q.reshape(B, Lq, H, hd)[b].transpose(1, 0, 2), k[b, :, :n_keys],
                             v[b, :, :n_keys], allowed).transpose(1, 0, 2)
        assert rel_rms(got[b], want) < 1e-2, (b, rel_rms(got[b], want))
        assert np.abs(got[b] - want).max() < 3e-2


@pytest.mark.parametrize("causal", [0, 1])
def test_attention_tiny_ragged(causal):
    announce(f"attention tiny causal={causal}")
    run_case(3, 16, 4, 2, 32, [0, 37, 300], 0, causal, seed=1)


@pytest.mark.parametrize("causal", [0, 1])
def test_attention_8b_split_kv(causal):
    announce(f"attention 8b split causal={causal}")
    run_case(2, 32, 32, 8, 128, [4096, 1000], 0, causal, seed=2)


def test_attention_prefill_chunk_causal():
    announce("attention prefill chunk")
    run_case(1, 96, 32, 8, 128, None, 40, 1, seed=3)
    run_case(2, 70, 4, 2, 32, None, 0, 1, seed=4)


def test_attention_single_key_is_the_value():
    announce("attention single key")
    run_case(1, 1, 4, 4, 32, [0], 0, 0, seed=5)
    run_case(1, 1, 32, 8, 128, [0], 0, 1, seed=6)


def test_attention_batch32_prefix4096():
    announce("attention b32 p4096")
    run_case(32, 32, 32, 8, 128, [4096] * 32, 0, 0, seed=7, check_rows=[0, 17, 31])


def test_attention_batch4_prefix65536():
    announce("attention b4 p65536")
    # the long-context decode shape: 64-way split KV, every row ragged by 3
    run_case(4, 32, 32, 8, 128, [65536, 65533, 65530, 65527], 0, 0, seed=10, check_rows=[0, 3])


@pytest.mark.parametrize("causal", [0, 1])
def test_attention_three_stage_ring_ragged_poisoned(causal):
    announce(f"attention three-stage ring, ragged poisoned tails, causal={causal}")
    # 8 rows x 8 KV heads x 4 key splits = 256 workgroups of >= 2048 keys: the
    # three-stage ring with spread loads.  Ragged ends inside a tile, ranges of
    # an odd number of tiles (a one-tile last stage), an empty last split for
    # the shortest row, and NaN/Inf past every row's end.
    prefix = [9000, 8999, 8961, 8007, 7001, 6543, 8590, 8191]
    run_case(8, 32, 32, 8, 128, prefix, 0, causal, seed=12, check_rows=[0, 2, 5, 7], poison=True)


@pytest.mark.parametrize("causal", [0, 1])
def test_attention_two_workgroups_per_cu_poisoned(causal):
    announce(f"attention two-stage spread ring, poisoned tail, causal={causal}")
    # a prefill-shaped pass: 1024 queries (32 query blocks) x 8 KV heads x 2 key
    # splits = 512 workgroups, two per CU, each with the two-stage ring and
    # spread loads; causal key ranges end mid-tile, NaN/Inf past the row's end
    run_case(1, 1024, 32, 8, 128, [5200], 0, causal, seed=13, poison=True)


@pytest.mark.parametrize("hd,H,G", [(32, 4, 2), (128, 32, 8)])
@pytest.mark.parametrize("causal", [0, 1])
def test_attention_ignores_slots_past_the_end(hd, H, G, causal):
    announce(f"attention poisoned tail hd={hd} causal={causal}")
    # ragged ends inside a 32-key tile, a split case (one row, long prefix) and a batch case
    run_case(3, 16, H, G, hd, [5, 37, 301], 0, causal, seed=8, poison=True)
    run_case(1, 32, H, G, hd, [2077], 0, causal, seed=9, poison=True)
