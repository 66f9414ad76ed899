"""Whole denoising path through the C ABI vs the oracle.

* Tiny model (2 layers, d=128, vocab 1024): prefill cache, teacher-forced
  denoise steps (conf within 1e-2, logits within 2e-2 relative RMS, argmax equal
  where the top-1 margin exceeds 5e-2), commit bit-exact on the oracle's
  (conf, argmax), append cache equal to the oracle's.
* Free-running block diffusion: the device's decode equals the oracle's canvas
  after canvas where every oracle decision is clear of the 5e-2 margins, and at
  every step of the device's own decode (unit gain = config 1, and larger head
  gains) each commit is one the rule allows given the oracle's scores of the
  device's canvas, with exact tokens wherever the oracle's margin is clear.
* One decoder layer at 8B-class shapes with the 131072-vocab head over a 4096-key
  N(0,1) prefix, batch 1 and 32 (sampled rows at 32).
"""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle
import synth
import bf16_storage
import test_freerun_compare as freerun_cases
from freerun import check_trajectory_step, compare_until_ambiguity
from gpu_helpers import announce, f32, host, i32, p, rel_rms, stream, sync, u8
from masked_block_diffusion_denoise_amd import _lib as L
from masked_block_diffusion_denoise_amd import runtime as R

pytestmark = pytest.mark.gpu

TINY = synth.TINY


def make(shape, w):
    return R.DlmModel.from_arrays(R.ModelConfig.of(shape), w)


def cache_close(sess, cache, b, upto, tol=1e-2):
    kl = host(sess.kv.k_logical().float())
    vl = host(sess.kv.v_logical().float())
    for l in range(cache.shape.n_layers):
        assert rel_rms(kl[l, b, :, :upto], cache.k[l][:, :upto]) < tol, ("k", l)
        assert rel_rms(vl[l, b, :, :upto], cache.v[l][:, :upto]) < tol, ("v", l)


def check_step(conf_g, arg_g, logits_g, logits_o, masked):
    conf_o, arg_o = oracle.confidence(logits_o)
    mk = np.flatnonzero(masked)
    assert np.abs(conf_g[mk] - conf_o[mk]).max() < 1e-2
    fin = np.isfinite(logits_o[0])
    for j in mk:
        assert rel_rms(logits_g[j][fin], logits_o[j][fin]) < 2e-2
        top2 = np.sort(logits_o[j][fin])[-2:]
        if top2[1] - top2[0] > 5e-2:
            assert arg_g[j] == arg_o[j]
    return conf_o, arg_o


def test_tiny_prefill_cache_and_last_token():
    announce("tiny prefill")
    w = synth.model_weights(TINY, seed=0, lm_head_gain=20.0)
    m = make(TINY, w)
    B, T = 2, 40
    prompt = synth.prompt(TINY, B, T, seed=1)
    sess = R.Session(m, B, 128, 16)
    tp = i32(prompt)
    last_a = i32(np.zeros(B))
    last_c = f32(np.zeros(B))
    # a workspace for 32-row passes forces two prefill passes (32 + 8 positions)
    ws, n = sess.ws.get(m.workspace_bytes(B * 32, T))
    L.call("dlm_prefill", m.handle, C.byref(sess.kv.c), p(tp), B, T, p(sess.prefix), p(last_a), p(last_c),
           p(sess.flags), ws, n, stream())
    sync()
    assert (host(sess.prefix) == T).all()
    for b in range(B):
        cache, x = oracle.prefill(w, TINY, prompt[b])
        cache_close(sess, cache, b, T)
        lg = oracle.head_logits(w, TINY, x[-1:])
        c, a = oracle.confidence(lg)
        assert abs(host(last_c)[b] - c[0]) < 1e-2
        top2 = np.sort(lg[0][np.isfinite(lg[0])])[-2:]
        if top2[1] - top2[0] > 5e-2:
            assert host(last_a)[b] == a[0]
    assert (host(sess.flags) == 0).all()


@pytest.mark.parametrize("B,T,cap", [(2, 1, 64), (1, 128, 128), (3, 97, 128)])
def test_tiny_prefill_edges(B, T, cap):
    """Prefill at its edges: a one-token prompt, a prompt that fills the cache to
    its capacity, a ragged length in one pass.  The cache and the last position's
    greedy prediction equal the oracle's causal pass."""
    announce(f"tiny prefill edges B={B} T={T} capacity={cap}")
    w = synth.model_weights(TINY, seed=0, lm_head_gain=20.0)
    m = make(TINY, w)
    prompt = synth.prompt(TINY, B, T, seed=12)
    sess = R.Session(m, B, cap, 16)
    last_a = i32(np.zeros(B))
    last_c = f32(np.zeros(B))
    sess.prefill(i32(prompt), last_argmax=last_a, last_conf=last_c)
    sync()
    assert (host(sess.prefix) == T).all()
    for b in range(B):
        cache, x = oracle.prefill(w, TINY, prompt[b])
        cache_close(sess, cache, b, T)
        lg = oracle.head_logits(w, TINY, x[-1:])
        c, a = oracle.confidence(lg)
        c16 = oracle.KVCache(TINY)
        x16 = bf16_storage.forward(w, TINY, prompt[b], c16, "causal")
        c_16, _ = oracle.confidence(bf16_storage.head_logits(w, TINY, x16[-1:]))
        assert abs(host(last_c)[b] - c[0]) < bf16_storage.conf_bar(c, c_16, [0]), b
        top2 = np.sort(lg[0][np.isfinite(lg[0])])[-2:]
        if top2[1] - top2[0] > 5e-2:
            assert host(last_a)[b] == a[0], b
    assert (host(sess.flags) == 0).all()


def test_tiny_prefill_short_last_pass_stays_in_workspace():
    """A prompt of 1286 positions through a workspace sized for 428-row passes:
    428 + 428 + 428 + 2 positions, the last pass short (fewer rows, other split
    counts).  Every pass must stay inside ws_bytes -- a canary written past the
    workspace is unchanged -- and the cache equals the oracle's causal prefill."""
    announce("tiny prefill, short last pass, workspace canary")
    w = synth.model_weights(TINY, seed=0, lm_head_gain=20.0)
    m = make(TINY, w)
    B, T = 1, 1286
    prompt = synth.prompt(TINY, B, T, seed=11)
    sess = R.Session(m, B, T + 64, 16)
    n = m.workspace_bytes(428, T)
    canary = 1 << 20
    buf = torch.empty(n + canary + 256, dtype=torch.uint8, device="cuda")
    base = (buf.data_ptr() + 255) & ~255
    off = base - buf.data_ptr()
    buf[off + n:].fill_(0xA5)
    tp = i32(prompt)
    L.call("dlm_prefill", m.handle, C.byref(sess.kv.c), p(tp), B, T, p(sess.prefix), None, None,
           p(sess.flags), C.c_void_p(base), C.c_size_t(n), stream())
    sync()
    assert (host(buf[off + n:]) == 0xA5).all(), "prefill wrote past its workspace"
    assert int(host(sess.prefix)[0]) == T
    cache, _ = oracle.prefill(w, TINY, prompt[0])
    cache_close(sess, cache, 0, T)


@pytest.mark.parametrize("gain,tau", [(1.0, 0.9), (60.0, 0.9)])
def test_tiny_teacher_forced_blocks(gain, tau):
    announce(f"tiny teacher-forced gain={gain}")
    w = synth.model_weights(TINY, seed=0, lm_head_gain=gain)
    m = make(TINY, w)
    prompt = synth.prompt(TINY, 1, 32, seed=0)
    Lb, max_steps = 16, 16
    sess = R.Session(m, 1, 128, Lb)
    sess.prefill(i32(prompt))
    cache, _ = oracle.prefill(w, TINY, prompt[0])
    logits = torch.zeros(Lb, TINY.vocab, dtype=torch.float32, device="cuda")
    tau_t, q_t = f32([tau]), i32([1])
    for blk in range(2):
        canvas = np.full(Lb, TINY.mask_id, np.int64)
        masked = np.ones(Lb, bool)
        step = 0
        while masked.any():
            lo = oracle.denoise_logits(w, TINY, cache, canvas)
            sess.canvas.copy_(i32(canvas[None]))
            sess.masked.copy_(u8(masked[None]))
            sess.denoise_step(logits)
            sync()
            conf_o, arg_o = check_step(host(sess.conf)[0], host(sess.argmax)[0], host(logits), lo, masked)
            # commit on the device fed with the oracle's confidences: bit-exact
            sess.conf.copy_(f32(conf_o[None]))
            sess.argmax.copy_(i32(arg_o[None]))
            sess.steps.fill_(step)
            sess.commit(tau_t, q_t, max_steps)
            canvas, masked, step, n = oracle.commit(conf_o.astype(np.float32), arg_o, canvas, masked, tau, 1,
                                                    step, max_steps)
            sync()
            np.testing.assert_array_equal(host(sess.canvas)[0], canvas)
            np.testing.assert_array_equal(host(sess.masked)[0].astype(bool), masked)
            assert host(sess.steps)[0] == step and host(sess.n_committed)[0] == n
        if gain == 1.0:
            assert step == Lb                    # no confidence reaches 0.9: one commit per step
        sess.append_block()
        oracle.append_block(w, TINY, cache, canvas)
        sync()
        assert host(sess.prefix)[0] == cache.length
        cache_close(sess, cache, 0, cache.length)
    assert (host(sess.flags) == 0).all()


def gpu_free_run(sess, prompt, n_blocks, max_steps, tau, on_step=None):
    """The device decodes on its own (threshold tau, quota 1), one step at a
    time; returns its canvas after every step.  on_step(block, canvas, masked,
    canvas_after, masked_after, last) sees each step; a block ends when no mask
    is left, then the device appends it."""
    sess.prefill(i32(prompt[None]))
    tau_t, q_t = f32([tau]), i32([1])
    out = []
    for blk in range(n_blocks):
        sess.begin_block()
        while True:
            sync()
            c0, m0 = host(sess.canvas)[0], host(sess.masked)[0].astype(bool)
            last = int(host(sess.steps)[0]) >= max_steps - 1
            sess.denoise_step()
            sess.commit(tau_t, q_t, max_steps)
            sync()
            c1, m1 = host(sess.canvas)[0], host(sess.masked)[0].astype(bool)
            out.append(c1)
            if on_step:
                on_step(blk, c0, m0, c1, m1, last)
            if not m1.any():
                break
        sess.append_block()
    sync()
    return out


@pytest.mark.parametrize("Lb", [16, 1, 64])
def test_tiny_ragged_prefixes_and_degenerate_masks(Lb):
    """Denoise steps at the edges of the method: rows at different prefix lengths
    (0 included: a row with no cached key), with every, some, one or no position
    masked; blocks of one position and of the 64 the entry point allows; a step with nothing masked (nothing is
    scored, nothing written); and a step with no cached prefix in any row (the
    first block of an unprompted decode).  Scored positions match the oracle;
    conf and argmax keep their earlier values everywhere else."""
    announce(f"tiny ragged prefixes and degenerate masks L={Lb}")
    w = synth.model_weights(TINY, seed=0, lm_head_gain=1.0)
    m = make(TINY, w)
    B, T = 4, 64
    prompt = synth.prompt(TINY, B, T, seed=5)
    sess = R.Session(m, B, 192, Lb)
    sess.prefill(i32(prompt))
    pre = np.array([0, 5, 40, 64])
    sess.prefix.copy_(i32(pre))                 # the host bound max_prefix stays T
    tok = synth.prompt(TINY, B, Lb, seed=6)
    masked = np.zeros((B, Lb), bool)
    masked[0] = True                            # every position
    masked[2, ::3] = True                       # some
    masked[3, Lb // 2] = True                   # one; row 1: none
    canvas = np.where(masked, TINY.mask_id, tok)
    logits = torch.zeros(B * Lb, TINY.vocab, dtype=torch.float32, device="cuda")

    def step(canvas, masked, with_logits=True):
        sess.canvas.copy_(i32(canvas))
        sess.masked.copy_(u8(masked))
        sess.conf.fill_(-7.0)
        sess.argmax.fill_(-7)
        logits.zero_()
        sess.denoise_step(logits if with_logits else None)
        sync()
        return host(sess.conf), host(sess.argmax), host(logits).reshape(B, Lb, -1)

    conf_g, arg_g, lg = step(canvas, masked)
    for b in range(B):
        mk = masked[b]
        if mk.any():
            cache = oracle.prefill(w, TINY, prompt[b, :pre[b]])[0] if pre[b] else oracle.KVCache(TINY)
            check_step(conf_g[b], arg_g[b], lg[b], oracle.denoise_logits(w, TINY, cache, canvas[b]), mk)
        assert (conf_g[b, ~mk] == -7.0).all() and (arg_g[b, ~mk] == -7).all(), b
        assert (lg[b, ~mk] == 0).all(), b
    # nothing masked anywhere: no position is scored or written
    conf_g, arg_g, lg = step(tok, np.zeros((B, Lb), bool))
    assert (conf_g == -7.0).all() and (arg_g == -7).all() and (lg == 0).all()
    # no cached prefix in any row, every position masked: every row scores the same canvas
    sess.prefix.zero_()
    sess.max_prefix = 0
    full = np.full((B, Lb), TINY.mask_id)
    conf_g, arg_g, lg = step(full, np.ones((B, Lb), bool))
    lo = oracle.denoise_logits(w, TINY, oracle.KVCache(TINY), full[0])
    for b in range(B):
        check_step(conf_g[b], arg_g[b], lg[b], lo, np.ones(Lb, bool))
    assert (host(sess.flags) == 0).all()


@pytest.mark.parametrize("Lb", [16, 1])
def test_tiny_append_block_ragged_prefixes(Lb):
    """dlm_append_block with every row at its own prefix length (0 included):
    each row's block lands in cache slots [P_b, P_b + L), P_b advances by L, and
    the keys/values and the causal next-token predictions equal the oracle's
    causal pass over the row's prompt prefix followed by the block."""
    announce(f"tiny append, ragged prefixes L={Lb}")
    w = synth.model_weights(TINY, seed=0, lm_head_gain=20.0)
    m = make(TINY, w)
    B, T = 3, 64
    prompt = synth.prompt(TINY, B, T, seed=7)
    sess = R.Session(m, B, 192, Lb)
    sess.prefill(i32(prompt))
    pre = np.array([0, 7, 64])
    sess.prefix.copy_(i32(pre))                 # the host bound max_prefix stays T
    block = synth.prompt(TINY, B, Lb, seed=8)
    sess.canvas.copy_(i32(block))
    arg = torch.zeros(B, Lb, dtype=torch.int32, device="cuda")
    conf = torch.zeros(B, Lb, dtype=torch.float32, device="cuda")
    sess.append_block(arg, conf)
    sync()
    assert (host(sess.prefix) == pre + Lb).all() and sess.max_prefix == T + Lb
    for b in range(B):
        cache = oracle.prefill(w, TINY, prompt[b, :pre[b]])[0] if pre[b] else oracle.KVCache(TINY)
        x = oracle.append_block(w, TINY, cache, block[b])
        cache_close(sess, cache, b, pre[b] + Lb)
        lo = oracle.head_logits(w, TINY, x)
        conf_o, arg_o = oracle.confidence(lo)
        # at this head gain bf16 storage alone moves some confidences by more
        # than half the 1e-2 bar: the bar is then twice that
        c16 = bf16_storage.prefill(w, TINY, prompt[b, :pre[b]]) if pre[b] else oracle.KVCache(TINY)
        conf_16, _ = oracle.confidence(bf16_storage.head_logits(w, TINY, bf16_storage.append_block(w, TINY, c16,
                                                                                                   block[b])))
        bar = bf16_storage.conf_bar(conf_o, conf_16, np.arange(Lb))
        assert np.abs(host(conf)[b] - conf_o).max() < bar, b
        for j in range(Lb):
            top2 = np.sort(lo[j][np.isfinite(lo[j])])[-2:]
            if top2[1] - top2[0] > 5e-2:
                assert host(arg)[b, j] == arg_o[j], (b, j)
    assert (host(sess.flags) == 0).all()


def test_tiny_block_ending_at_the_cache_capacity():
    """A block whose last position is the cache's last slot: the denoise step and
    the append at prefix + L == capacity match the oracle, and the next block's
    step is refused (DLM_ERR_CAPACITY) before any device work."""
    announce("tiny block at the cache capacity")
    w = synth.model_weights(TINY, seed=0, lm_head_gain=1.0)
    m = make(TINY, w)
    B, T, Lb, cap = 2, 112, 16, 128
    prompt = synth.prompt(TINY, B, T, seed=13)
    sess = R.Session(m, B, cap, Lb)
    sess.prefill(i32(prompt))
    full = np.full((B, Lb), TINY.mask_id)
    sess.canvas.copy_(i32(full))
    sess.masked.copy_(u8(np.ones((B, Lb), bool)))
    logits = torch.zeros(B * Lb, TINY.vocab, dtype=torch.float32, device="cuda")
    sess.denoise_step(logits)
    sync()
    conf_g, arg_g, lg = host(sess.conf), host(sess.argmax), host(logits).reshape(B, Lb, -1)
    block = synth.prompt(TINY, B, Lb, seed=14)
    caches = []
    for b in range(B):
        cache, _ = oracle.prefill(w, TINY, prompt[b])
        check_step(conf_g[b], arg_g[b], lg[b], oracle.denoise_logits(w, TINY, cache, full[b]), np.ones(Lb, bool))
        oracle.append_block(w, TINY, cache, block[b])
        caches.append(cache)
    sess.canvas.copy_(i32(block))
    sess.append_block()
    sync()
    assert (host(sess.prefix) == cap).all() and sess.max_prefix == cap
    for b in range(B):
        cache_close(sess, caches[b], b, cap)
    with pytest.raises(L.DlmError) as e:
        sess.denoise_step()
    assert e.value.status == -3                 # DLM_ERR_CAPACITY
    assert (host(sess.flags) == 0).all()


@pytest.mark.parametrize("case", freerun_cases.CLEAR)
def test_tiny_free_running_identical_to_oracle(case):
    """Clear cases (every oracle decision more than 5e-2 from another one): the
    device's own decode equals the oracle's canvas after canvas, through both
    blocks and the append between them."""
    gain, wseed, pseed = case
    announce(f"tiny free-running, clear case {case}")
    w, prompt, steps = freerun_cases.decode(gain, wseed, pseed)
    m = make(TINY, w)
    sess = R.Session(m, 1, 128, 16)
    canv = gpu_free_run(sess, prompt, 2, 16, 0.9)
    stop, blocks = compare_until_ambiguity(steps, canv)
    assert stop == len(steps) == len(canv) and blocks == 2
    assert (host(sess.flags) == 0).all()


@pytest.mark.parametrize("gain,min_exact", [(1.0, 4), (20.0, 24), (60.0, 12)])
def test_tiny_free_running_every_step_valid(gain, min_exact):
    """The device decodes on its own for two blocks of 16 (unit gain: config 1
    itself).  At every step the oracle scores the device's canvas, with a cache
    built from the prompt and the device's own earlier blocks: committed tokens
    equal the oracle's argmax wherever its top-1 margin exceeds 5e-2, and the
    positions committed are a choice the rule allows given the oracle's
    confidences to 5e-2 (exactly the oracle's choice wherever that is clear).
    After each append the device's cache equals the oracle's."""
    announce(f"tiny free-running trajectory, gain {gain}")
    w = synth.model_weights(TINY, seed=0, lm_head_gain=gain)
    m = make(TINY, w)
    prompt = synth.prompt(TINY, 1, 32, seed=0)[0]
    sess = R.Session(m, 1, 128, 16)
    cache, _ = oracle.prefill(w, TINY, prompt)
    state = {"exact": 0, "steps": 0}

    def on_step(blk, c0, m0, c1, m1, last):
        lo = oracle.denoise_logits(w, TINY, cache, c0)
        state["exact"] += check_trajectory_step(lo, c0, m0, c1, m1, 0.9, 1, last, TINY.mask_id)
        state["steps"] += 1
        if not m1.any():                        # the device appends this block next
            oracle.append_block(w, TINY, cache, c1)

    gpu_free_run(sess, prompt, 2, 16, 0.9, on_step)
    assert state["exact"] >= min_exact, state
    cache_close(sess, cache, 0, cache.length)
    assert cache.length == 64 and (host(sess.flags) == 0).all()


@pytest.fixture(scope="module")
def layer8b():
    announce("generating one 8B-class layer")
    shape = synth.LAYER_8B
    w = synth.model_weights(shape, seed=0)
    return shape, w, make(shape, w)


@pytest.mark.parametrize("B,rows", [(1, [0]), (32, [0, 13, 31])])
def test_layer8b_denoise_step(layer8b, B, rows):
    announce(f"8B layer denoise B={B}")
    shape, w, m = layer8b
    P, Lb = 4096, 32
    k, v = synth.kv_prefix(shape, B, P, seed=3)
    canvas, masked = synth.ragged_canvas(shape, B, Lb, seed=3)
    sess = R.Session(m, B, P + Lb + 64, Lb)
    sess.kv.write(0, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    sess.prefix.fill_(P)
    sess.max_prefix = P
    sess.canvas.copy_(i32(canvas))
    sess.masked.copy_(u8(masked))
    logits = torch.zeros(B * Lb, shape.vocab, dtype=torch.float32, device="cuda") if B == 1 else None
    sess.denoise_step(logits)
    sync()
    conf_g, arg_g = host(sess.conf), host(sess.argmax)
    lg_all = host(logits).reshape(B, Lb, -1) if logits is not None else None
    for b in rows:
        cache = oracle.KVCache(shape)
        cache.k[0] = k[b].astype(np.float64)
        cache.v[0] = v[b].astype(np.float64)
        lo = oracle.denoise_logits(w, shape, cache, canvas[b])
        conf_o, arg_o = oracle.confidence(lo)
        mk = np.flatnonzero(masked[b])
        assert np.abs(conf_g[b, mk] - conf_o[mk]).max() < 1e-2
        for j in mk:
            top2 = np.sort(lo[j][np.isfinite(lo[j])])[-2:]
            if top2[1] - top2[0] > 5e-2:
                assert arg_g[b, j] == arg_o[j], (b, j)
            if lg_all is not None:
                fin = np.isfinite(lo[j])
                assert rel_rms(lg_all[b, j][fin], lo[j][fin]) < 2e-2
    assert (host(sess.flags) == 0).all()


def test_layer8b_append_block_batch1(layer8b):
    # batch 1 runs the K-split projections whose partial sums fold into RoPE + KV
    # write and into the residual add + norm: the appended keys/values and the
    # causal next-token predictions must match the oracle's causal pass
    announce("8B layer append B=1")
    shape, w, m = layer8b
    B, P, Lb = 1, 4096, 32
    k, v = synth.kv_prefix(shape, B, P, seed=5)
    block = synth.prompt(shape, B, Lb, seed=5)
    sess = R.Session(m, B, P + Lb + 64, Lb)
    sess.kv.write(0, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    sess.prefix.fill_(P)
    sess.max_prefix = P
    sess.canvas.copy_(i32(block))
    arg = torch.zeros(B, Lb, dtype=torch.int32, device="cuda")
    conf = torch.zeros(B, Lb, dtype=torch.float32, device="cuda")
    sess.append_block(arg, conf)
    sync()
    cache = oracle.KVCache(shape)
    cache.k[0] = k[0].astype(np.float64)
    cache.v[0] = v[0].astype(np.float64)
    x = oracle.append_block(w, shape, cache, block[0])
    kg = host(sess.kv.k_logical()[0, 0, :, P:P + Lb].float())
    vg = host(sess.kv.v_logical()[0, 0, :, P:P + Lb].float())
    assert rel_rms(kg, cache.k[0][:, P:P + Lb]) < 1e-2
    assert rel_rms(vg, cache.v[0][:, P:P + Lb]) < 1e-2
    assert int(host(sess.prefix)[0]) == P + Lb
    lo = oracle.head_logits(w, shape, x)
    conf_o, arg_o = oracle.confidence(lo)
    assert np.abs(host(conf)[0] - conf_o).max() < 1e-2
    for j in range(Lb):
        top2 = np.sort(lo[j][np.isfinite(lo[j])])[-2:]
        if top2[1] - top2[0] > 5e-2:
            assert host(arg)[0, j] == arg_o[j], j


# Two layers wide enough (d 1024) that the batch-1 projections split over K:
# the partial sums fold into RoPE + KV write and into the residual add + the
# next RMSNorm (after the output projection and after the down projection,
# which normalises for the next layer).
WIDE2 = synth.ModelShape(n_layers=2, d_model=1024, n_heads=8, n_kv_heads=2, head_dim=128, d_ffn=2048,
                         vocab=2048, mask_id=0, rope_base=1.0e6)


def test_two_wide_layers_split_reductions_prefill_denoise_append():
    announce("two wide layers: K-split reductions fused")
    shape = WIDE2
    # head gain 2: logit spread ~1.3 as for the 8B-class head at unit gain (a
    # larger gain pushes confidences near 1, where the bf16 logit error alone
    # moves them by ~1e-2)
    w = synth.model_weights(shape, seed=4, lm_head_gain=2.0)
    m = make(shape, w)
    T, Lb = 40, 32
    prompt = synth.prompt(shape, 1, T, seed=6)
    sess = R.Session(m, 1, 128, Lb)
    sess.prefill(i32(prompt))
    cache, _ = oracle.prefill(w, shape, prompt[0])
    sync()
    for layer in range(shape.n_layers):
        kg = host(sess.kv.k_logical()[layer, 0, :, :T].float())
        vg = host(sess.kv.v_logical()[layer, 0, :, :T].float())
        assert rel_rms(kg, cache.k[layer][:, :T]) < 1e-2, layer
        assert rel_rms(vg, cache.v[layer][:, :T]) < 1e-2, layer

    canvas, masked = synth.ragged_canvas(shape, 1, Lb, seed=6)
    sess.canvas.copy_(i32(canvas))
    sess.masked.copy_(u8(masked))
    logits = torch.zeros(Lb, shape.vocab, dtype=torch.float32, device="cuda")
    sess.denoise_step(logits)
    sync()
    lo = oracle.denoise_logits(w, shape, cache, canvas[0])
    conf_o, arg_o = oracle.confidence(lo)
    lg = host(logits)
    mk = np.flatnonzero(masked[0])
    assert np.abs(host(sess.conf)[0, mk] - conf_o[mk]).max() < 1e-2
    for j in mk:
        fin = np.isfinite(lo[j])
        assert rel_rms(lg[j][fin], lo[j][fin]) < 2e-2, j
        top2 = np.sort(lo[j][fin])[-2:]
        if top2[1] - top2[0] > 5e-2:
            assert host(sess.argmax)[0, j] == arg_o[j], j

    block = synth.prompt(shape, 1, Lb, seed=7)
    arg = torch.zeros(1, Lb, dtype=torch.int32, device="cuda")
    conf = torch.zeros(1, Lb, dtype=torch.float32, device="cuda")
    sess.append(i32(block), arg, conf)
    x = oracle.append_block(w, shape, cache, block[0])
    sync()
    for layer in range(shape.n_layers):
        kg = host(sess.kv.k_logical()[layer, 0, :, T:T + Lb].float())
        vg = host(sess.kv.v_logical()[layer, 0, :, T:T + Lb].float())
        assert rel_rms(kg, cache.k[layer][:, T:T + Lb]) < 1e-2, layer
        assert rel_rms(vg, cache.v[layer][:, T:T + Lb]) < 1e-2, layer
    lo = oracle.head_logits(w, shape, x)
    conf_o, arg_o = oracle.confidence(lo)
    assert np.abs(host(conf)[0] - conf_o).max() < 1e-2
    for j in range(Lb):
        top2 = np.sort(lo[j][np.isfinite(lo[j])])[-2:]
        if top2[1] - top2[0] > 5e-2:
            assert host(arg)[0, j] == arg_o[j], j
    assert (host(sess.flags) == 0).all()


def check_step_bf16(conf_g, arg_g, ent_g, logits_g, logits_o, logits_16, masked):
    """check_step for a large test head gain, which scales the logits and so
    every logit error.  The logits stay within 2e-2 relative RMS; confidence and
    entropy within 1e-2 (nats), or, where bf16 storage alone moves them further
    (the oracle's arithmetic with the device's bf16 storage points, float64
    otherwise), within twice that; the argmax equals the oracle's wherever the
    top-1 margin exceeds 5e-2 and twice the row's largest logit change under
    bf16 storage alone."""
    conf_o, arg_o = oracle.confidence(logits_o)
    conf_16, _ = oracle.confidence(logits_16)
    ent_o, ent_16 = oracle.entropy(logits_o), oracle.entropy(logits_16)
    mk = np.flatnonzero(masked)
    fin = np.isfinite(logits_o[0])
    assert np.abs(conf_g[mk] - conf_o[mk]).max() <= bf16_storage.conf_bar(conf_o, conf_16, mk)
    if ent_g is not None:
        assert np.abs(ent_g[mk] - ent_o[mk]).max() <= bf16_storage.conf_bar(ent_o, ent_16, mk)
    for j in mk:
        l, g = logits_o[j][fin], logits_g[j][fin]
        assert rel_rms(g, l) < 2e-2
        top2 = np.sort(l)[-2:]
        if top2[1] - top2[0] > max(5e-2, 2.0 * np.abs(logits_16[j][fin] - l).max()):
            assert arg_g[j] == arg_o[j]
    return conf_o, arg_o, ent_o


@pytest.mark.parametrize("sampler", [dict(rule="entropy", entropy_bound=0.5), dict(rule="bound"),
                                     dict(rule="threshold", max_transfer=2),
                                     dict(rule="threshold", stability_steps=2, stop_entropy=0.5)],
                         ids=["entropy", "bound", "cap2", "adaptive-stop"])
def test_tiny_teacher_forced_samplers(sampler):
    """Sampler variants through whole blocks: the device's entropies against the
    oracle's, and dlm_commit_ex fed the oracle's confidences and entropies
    bit-exact with the oracle's commit_ex (adaptive-stopping state included)."""
    announce(f"tiny teacher-forced sampler {sampler}")
    w = synth.model_weights(TINY, seed=0, lm_head_gain=60.0)
    m = make(TINY, w)
    prompt = synth.prompt(TINY, 1, 32, seed=0)
    Lb, max_steps, tau = 16, 16, 0.9
    sess = R.Session(m, 1, 128, Lb)
    sess.prefill(i32(prompt))
    cache, _ = oracle.prefill(w, TINY, prompt[0])
    logits = torch.zeros(Lb, TINY.vocab, dtype=torch.float32, device="cuda")
    ent_g = torch.zeros(1, Lb, dtype=torch.float32, device="cuda")
    smp = R.Sampler(**sampler)
    tau_t, q_t = f32([tau]), i32([1])
    steps_seen = []
    cache16 = bf16_storage.prefill(w, TINY, prompt[0])
    for blk in range(2):
        sess.begin_block()
        canvas = np.full(Lb, TINY.mask_id, np.int64)
        masked = np.ones(Lb, bool)
        step, prev, stable = 0, np.full(Lb, -1), 0
        while masked.any():
            lo = oracle.denoise_logits(w, TINY, cache, canvas)
            lo16 = bf16_storage.denoise_logits(w, TINY, cache16, canvas)
            sess.canvas.copy_(i32(canvas[None]))
            sess.masked.copy_(u8(masked[None]))
            sess.denoise_step(logits, ent_g)
            sync()
            conf_o, arg_o, ent_o = check_step_bf16(host(sess.conf)[0], host(sess.argmax)[0], host(ent_g)[0],
                                                   host(logits), lo, lo16, masked)
            # commit on the device fed with the oracle's values: bit-exact
            c32, e32 = conf_o.astype(np.float32), ent_o.astype(np.float32)
            sess.conf.copy_(f32(c32[None]))
            sess.argmax.copy_(i32(arg_o[None]))
            ent_g.copy_(f32(e32[None]))
            sess.steps.fill_(step)
            sess.commit_ex(tau_t, q_t, max_steps, smp, ent_g)
            canvas, masked, step, n, prev, stable = oracle.commit_ex(
                c32, arg_o, canvas, masked, tau, 1, step, max_steps, entropy=e32, prev_argmax=prev,
                stable=stable, **sampler)
            sync()
            np.testing.assert_array_equal(host(sess.canvas)[0], canvas)
            np.testing.assert_array_equal(host(sess.masked)[0].astype(bool), masked)
            assert host(sess.steps)[0] == step and host(sess.n_committed)[0] == n
            if smp.stability_steps:
                np.testing.assert_array_equal(host(sess.prev_argmax)[0], prev)
                assert host(sess.stable)[0] == stable
        steps_seen.append(step)
        sess.append_block()
        oracle.append_block(w, TINY, cache, canvas)
        bf16_storage.append_block(w, TINY, cache16, canvas)
        sync()
        cache_close(sess, cache, 0, cache.length)
    if sampler.get("max_transfer"):
        assert max(steps_seen) >= Lb // 2                   # at most 2 per step: at least 8 steps a block


def test_tiny_anchor_blocks():
    """Anchor layout on the device: each block's first token is the causal
    argmax after everything before it (the oracle's, wherever its top-1 margin
    is clear), it is never reopened, and a block takes at most L - 1 steps."""
    announce("tiny anchor blocks")
    w = synth.model_weights(TINY, seed=0, lm_head_gain=20.0)
    m = make(TINY, w)
    prompt = synth.prompt(TINY, 1, 32, seed=2)
    Lb, max_steps, n_blocks = 16, 16, 3
    sess = R.Session(m, 1, 128, Lb)
    out, st = sess.generate(i32(prompt), n_blocks * Lb, max_steps, 0.9, 1, anchor=True)
    toks = host(out)[0]
    assert all(s <= Lb - 1 for s in st.steps_per_block), st.steps_per_block
    assert st.accepted_tokens == n_blocks * (Lb - 1)      # the anchors are not denoised
    checked = 0
    for k in range(n_blocks):
        before = np.concatenate([prompt[0], toks[:k * Lb]])
        _, x = oracle.prefill(w, TINY, before)
        lo = oracle.head_logits(w, TINY, x[-1:])[0]
        top2 = np.sort(lo[np.isfinite(lo)])[-2:]
        if top2[1] - top2[0] > 5e-2:
            assert toks[k * Lb] == int(np.argmax(lo)), k
            checked += 1
    assert checked >= 2
    assert (toks != TINY.mask_id).all()


@pytest.mark.parametrize("K,anchor,rule", [(4, False, None), (3, True, None), (5, False, "entropy")])
def test_tiny_graph_replay_equals_eager(K, anchor, rule):
    """The block loop replaying a captured graph of K steps (eager fills and host
    reads between the replays) produces exactly the eager loop's tokens and step
    counts, block after block."""
    announce(f"tiny graph replay K={K} anchor={anchor} rule={rule}")
    w = synth.model_weights(TINY, seed=0, lm_head_gain=60.0)
    m = make(TINY, w)
    prompt = synth.prompt(TINY, 2, 32, seed=7)
    Lb, max_steps = 16, 16
    smp = R.Sampler(rule=rule, entropy_bound=0.5) if rule else None
    runs = []
    for gs in (0, K):
        sess = R.Session(m, 2, 128, Lb)
        out, st = sess.generate(i32(prompt), 3 * Lb, max_steps, 0.9, 1, sampler=smp, anchor=anchor, graph_steps=gs)
        sync()
        runs.append((host(out), st.steps_per_block, st.accepted_tokens, host(sess.prefix)))
    (o0, s0, a0, p0), (o1, s1, a1, p1) = runs
    np.testing.assert_array_equal(o1, o0)
    assert s1 == s0 and a1 == a0
    np.testing.assert_array_equal(p1, p0)
    assert (o0 != TINY.mask_id).all()
