"""dlm_denoise_step_noalloc (the allocation-free denoise step, scratch in a fixed
device array of the library) against dlm_denoise_step_ex with a caller
workspace: the same kernels on the same inputs, so every output is identical,
bit for bit.  Two calls in a row, the second smaller (the fixed scratch keeps
the first call's contents); the caller's workspace is filled with NaN bytes
first, so neither side can lean on zeroed memory."""
import ctypes as C

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import announce, host, i32, p, stream, sync, u8
from masked_block_diffusion_denoise_amd import _lib as L
from masked_block_diffusion_denoise_amd import runtime as R

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def layer8b_model():
    announce("no-alloc: generating one 8B-class layer")
    shape = synth.LAYER_8B
    w = synth.model_weights(shape, seed=0)
    return shape, R.DlmModel.from_arrays(R.ModelConfig.of(shape), w)


def run_both(m, sess, B, Lb, P, seed):
    shape = m.cfg
    c = L.load()
    canvas, masked = synth.ragged_canvas(synth.LAYER_8B, B, Lb, seed=seed)
    tc, tm = i32(canvas), u8(masked)
    sess.prefix[:B].fill_(P)
    outs = []
    for which in ("ex", "noalloc"):
        conf = torch.full((B, Lb), -1.0, dtype=torch.float32, device="cuda")
        arg = torch.full((B, Lb), -1, dtype=torch.int32, device="cuda")
        ent = torch.full((B, Lb), -1.0, dtype=torch.float32, device="cuda")
        logits = torch.zeros(B * Lb, shape.vocab, dtype=torch.float32, device="cuda")
        if which == "ex":
            n = m.workspace_bytes(B * Lb, P + Lb)
            ws = torch.full((n + 256,), 0xFF, dtype=torch.uint8, device="cuda")
            base = (ws.data_ptr() + 255) & ~255
            st = c.dlm_denoise_step_ex(m.handle, C.byref(sess.kv.c), p(sess.prefix), P, p(tc), p(tm), B, Lb, p(conf),
                                       p(arg), p(ent), p(logits), p(sess.flags), C.c_void_p(base), C.c_size_t(n),
                                       stream())
        else:
            st = c.dlm_denoise_step_noalloc(m.handle, C.byref(sess.kv.c), p(sess.prefix), P, p(tc), p(tm), B, Lb,
                                            p(conf), p(arg), p(ent), p(logits), p(sess.flags), stream())
        L.check("dlm_denoise_step_" + which, st)
        sync()
        outs.append((host(conf), host(arg), host(ent), host(logits)))
    (c0, a0, e0, l0), (c1, a1, e1, l1) = outs
    mk = masked.astype(bool)
    assert mk.any()
    np.testing.assert_array_equal(c1[mk], c0[mk])
    np.testing.assert_array_equal(a1[mk], a0[mk])
    np.testing.assert_array_equal(e1[mk], e0[mk])
    rows = np.flatnonzero(mk.reshape(-1))
    np.testing.assert_array_equal(l1[rows], l0[rows])
    assert (c0[mk] > 0).all() and (c0[mk] <= 1).all()
    assert (host(sess.flags) == 0).all()


def test_noalloc_step_equals_workspace_step_twice_second_smaller(layer8b_model):
    shape, m = layer8b_model
    P1, L1 = 4096, 32
    sess = R.Session(m, 1, P1 + L1 + 64, L1)
    k, v = synth.kv_prefix(shape, 1, P1, seed=3)
    sess.kv.write(0, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    announce("no-alloc: batch 1, 32 positions over a 4096-position prefix")
    run_both(m, sess, 1, L1, P1, seed=3)
    announce("no-alloc: batch 1, 16 positions over a 1024-position prefix")
    run_both(m, sess, 1, 16, 1024, seed=4)
