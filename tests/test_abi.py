"""The C ABI on the CPU: the library loads, exports every declared entry point, and
rejects bad arguments on the host before anything is enqueued (no GPU needed:
every call here fails validation, so no kernel is launched)."""
import ctypes as C
import os
import re

import pytest

from masked_block_diffusion_denoise_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = C.c_void_p(4096)   # aligned, never dereferenced: validation fails first


def declared_functions():
    names = set()
    for h in ("libdlm.h", "libdlm_ops.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(dlm_[a-z_0-9]+)\s*\(", text))
    return names


def exported_symbols():
    lib = L.load()
    return {n for n in declared_functions() if hasattr(lib, n)}


def test_library_exports_every_declared_function():
    decl = declared_functions()
    assert len(decl) >= 17
    assert exported_symbols() == decl
    assert set(L.EXPORTS) == decl


def tiny_cfg(**kw):
    base = dict(n_layers=2, d_model=128, n_heads=4, n_kv_heads=2, head_dim=32, d_ffn=512, vocab=1024,
                mask_id=0, rope_base=10000.0, rms_eps=1e-5)
    base.update(kw)
    return L.Config(*base.values())


def fake_weights(n_layers=2):
    arr = (C.c_void_p * n_layers)(*([4096] * n_layers))
    p = C.cast(arr, C.POINTER(C.c_void_p))
    return L.Weights(4096, 4096, 4096, p, p, p, p, p, p), arr


def create(cfg):
    lib = L.load()
    w, keep = fake_weights(cfg.n_layers)
    h = C.c_void_p()
    st = lib.dlm_model_create(C.byref(cfg), C.byref(w), C.byref(h))
    return st, h


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), -4), (dict(n_heads=3), -2), (dict(n_heads=16, n_kv_heads=2), -4),
    (dict(mask_id=1024), -1), (dict(mask_id=-1), -1), (dict(vocab=1000), -4), (dict(vocab=1152), -4),
    (dict(d_ffn=500), -4), (dict(rope_base=float("nan")), -1), (dict(rms_eps=0.0), -1),
    (dict(n_layers=0), -2), (dict(d_model=8448), -4),
])
def test_model_create_rejects_bad_config(kw, status):
    st, _ = create(tiny_cfg(**kw))
    assert st == status, L.load().dlm_last_error()


def test_model_create_rejects_null_and_misaligned_weights():
    lib = L.load()
    cfg = tiny_cfg()
    arr = (C.c_void_p * 2)(4096, 4098)
    p = C.cast(arr, C.POINTER(C.c_void_p))
    w = L.Weights(4096, 4096, 4096, p, p, p, p, p, p)
    h = C.c_void_p()
    assert lib.dlm_model_create(C.byref(cfg), C.byref(w), C.byref(h)) == -1
    w = L.Weights(None, 4096, 4096, p, p, p, p, p, p)
    assert lib.dlm_model_create(C.byref(cfg), C.byref(w), C.byref(h)) == -1


@pytest.fixture
def model():
    st, h = create(tiny_cfg())
    assert st == 0
    yield h
    L.load().dlm_model_destroy(h)


def test_workspace_bytes_grows_with_rows_and_keys(model):
    lib = L.load()
    a = lib.dlm_workspace_bytes(model, 16, 64)
    b = lib.dlm_workspace_bytes(model, 32, 64)
    c = lib.dlm_workspace_bytes(model, 32, 4096)
    assert 0 < a < b <= c
    assert lib.dlm_workspace_bytes(model, 0, 64) == 0
    assert a % 256 == 0


def test_workspace_bound_never_shrinks_with_rows():
    """dlm_prefill sizes every pass (the shorter last one included) with the bound
    over B*C rows.  A product's K-split count falls as its rows fill more tiles,
    so the split workspace S(r) * r is not monotone in r (8B-class down
    projection: 8 splits at 483 rows, 6 at 544); the bound must still never
    shrink as rows grow, or a short last pass writes past the workspace."""
    lib = L.load()
    cfgs = [tiny_cfg(),
            tiny_cfg(n_layers=32, d_model=4096, n_heads=32, n_kv_heads=8, head_dim=128, d_ffn=14336,
                     vocab=131072, mask_id=100, rope_base=1e6)]
    for cfg in cfgs:
        st, h = create(cfg)
        assert st == 0
        try:
            for kv in (64, 1027, 4128):
                prev = 0
                for r in range(1, 1100):
                    b = lib.dlm_workspace_bytes(h, r, kv)
                    assert b >= prev, (cfg.d_model, kv, r, b, prev)
                    prev = b
            if cfg.d_model == 4096:
                # the 483-row down projection's eight fp32 partial planes fit the
                # bound of a 544-row pass (whose own split count is only 6)
                assert lib.dlm_workspace_bytes(h, 544, 1027) >= 8 * 483 * 4096 * 4
        finally:
            lib.dlm_model_destroy(h)


def test_denoise_step_validation(model):
    lib = L.load()
    kv = L.KV(4096, 4096, 2, 128)
    args = lambda **o: dict(dict(prefix=FAKE, max_prefix=64, canvas=FAKE, masked=FAKE, B=2, Lb=16,
                                 conf=FAKE, argmax=FAKE, logits=None, ws=FAKE, nws=0), **o)

    def run(kvv=kv, **o):
        a = args(**o)
        return lib.dlm_denoise_step(model, C.byref(kvv), a["prefix"], a["max_prefix"], a["canvas"], a["masked"],
                                    a["B"], a["Lb"], a["conf"], a["argmax"], a["logits"], None, a["ws"],
                                    a["nws"], None)
    assert run(B=0) == -2
    assert run(B=3) == -2                      # more rows than the cache holds
    assert run(Lb=65) == -2
    assert run(Lb=0) == -2
    assert run(max_prefix=120) == -3           # 120 + 16 > 128
    assert run(max_prefix=113) == -3           # one slot past the capacity
    assert run(max_prefix=112) == -6           # an exact fit passes, then the (empty) workspace fails
    assert run(max_prefix=-1) == -1
    assert run(canvas=None) == -1
    assert run(conf=C.c_void_p(4098)) == -1    # misaligned
    assert run(logits=C.c_void_p(4100)) == -1
    assert run(kvv=L.KV(4096, 4096, 2, 100)) == -2   # capacity not a multiple of 64
    assert run(nws=16) == -6                   # workspace too small
    assert run(ws=C.c_void_p(4096 + 64), nws=1 << 40) == -1   # workspace not 256-aligned
    assert b"workspace" in lib.dlm_last_error()


def test_noalloc_step_validation_and_scratch_limit():
    """The allocation-free step validates like dlm_denoise_step_ex and refuses a
    pass larger than its fixed scratch before any device call."""
    lib = L.load()
    st, h = create(tiny_cfg(n_layers=1, d_model=4096, n_heads=32, n_kv_heads=8, head_dim=128, d_ffn=14336,
                            vocab=131072, mask_id=100, rope_base=1e6))
    assert st == 0
    try:
        run = lambda B, Lb, P, cap=8192, canvas=FAKE: lib.dlm_denoise_step_noalloc(
            h, C.byref(L.KV(4096, 4096, 32, cap)), FAKE, P, canvas, FAKE, B, Lb, FAKE, FAKE, None, None, None, None)
        assert run(0, 32, 4096) == -2
        assert run(1, 65, 4096) == -2
        assert run(1, 32, 8192) == -3
        assert run(1, 32, 4096, canvas=None) == -1
        assert L.NOALLOC_SCRATCH_BYTES == 64 << 20
        assert lib.dlm_workspace_bytes(h, 32 * 32, 4096 + 32) > L.NOALLOC_SCRATCH_BYTES
        assert run(32, 32, 4096) == -6                 # batch 32 needs more than 64 MiB
        assert run(8, 32, 4096) == -6                  # batch 8 needs 71.8 MB, just over
        assert b"scratch" in lib.dlm_last_error()
    finally:
        lib.dlm_model_destroy(h)


def test_commit_validation():
    lib = L.load()
    f = FAKE

    def run(B=2, Lb=8, max_steps=4, conf=f, masked=f):
        return lib.dlm_commit(conf, f, f, masked, B, Lb, f, f, f, max_steps, f, f, None)
    assert run(B=0) == -2
    assert run(Lb=65) == -2
    assert run(max_steps=0) == -1
    assert run(conf=None) == -1
    assert run(masked=None) == -1


def test_commit_ex_validation():
    lib = L.load()
    f = FAKE

    def run(rule=L.RULE_THRESHOLD, entropy=None, B=2, Lb=8, max_steps=4, opts=True, **kw):
        o = L.CommitOpts(rule=rule, min_threshold=0.45, scaling=2.0, entropy_bound=0.1, max_transfer=0,
                         stability_steps=0, stop_entropy=0.005, prev_argmax=None, stable=None)
        for k, v in kw.items():
            setattr(o, k, v)
        return lib.dlm_commit_ex(f, f, entropy, f, f, B, Lb, f, f, f, max_steps, C.byref(o) if opts else None,
                                 f, f, None)
    assert run(B=0) == -2
    assert run(Lb=65) == -2
    assert run(max_steps=0) == -1
    assert run(opts=False) == -1
    assert run(rule=3) == -1
    assert run(rule=-1) == -1
    assert run(rule=L.RULE_ENTROPY) == -1                 # the entropy rule needs entropies
    assert run(min_threshold=float("nan")) == -1
    assert run(scaling=float("inf")) == -1
    assert run(max_transfer=-1) == -1
    assert run(stability_steps=-2) == -1
    assert run(stability_steps=2, entropy=f) == -1        # stopping needs its state buffers
    assert run(stability_steps=2) == -1                   # ... and entropies
    assert b"adaptive" in lib.dlm_last_error() or b"entrop" in lib.dlm_last_error()


def test_denoise_step_ex_validation(model):
    lib = L.load()
    kv = L.KV(4096, 4096, 1, 64)
    # a misaligned entropy buffer is refused before anything runs
    assert lib.dlm_denoise_step_ex(model, C.byref(kv), FAKE, 0, FAKE, FAKE, 1, 16, FAKE, FAKE, C.c_void_p(4098),
                                   None, None, FAKE, 1 << 30, None) == -1


def test_prefill_and_append_validation(model):
    lib = L.load()
    kv = L.KV(4096, 4096, 1, 64)
    assert lib.dlm_prefill(model, C.byref(kv), FAKE, 1, 65, FAKE, None, None, None, FAKE, 1 << 30, None) == -3
    assert lib.dlm_prefill(model, C.byref(kv), FAKE, 1, 0, FAKE, None, None, None, FAKE, 1 << 30, None) == -2
    assert lib.dlm_prefill(model, C.byref(kv), FAKE, 1, 32, FAKE, FAKE, None, None, FAKE, 1 << 30, None) == -1
    assert lib.dlm_prefill(model, C.byref(kv), FAKE, 1, 64, FAKE, None, None, None, FAKE, 16, None) == -6
    assert lib.dlm_append_block(model, C.byref(kv), FAKE, 40, FAKE, 1, 32, None, None, None, FAKE,
                                1 << 30, None) == -3
    assert lib.dlm_append_block(model, C.byref(kv), FAKE, 0, FAKE, 1, 16, FAKE, None, None, FAKE,
                                1 << 30, None) == -1


def test_op_validation():
    lib = L.load()
    assert lib.dlm_op_gemm(FAKE, FAKE, FAKE, 32, 100, 128, 128, 100, 0, FAKE, 1 << 30, None) == -2
    assert lib.dlm_op_gemm(FAKE, FAKE, FAKE, 32, 128, 300, 300, 128, 0, FAKE, 1 << 30, None) == -2
    assert lib.dlm_op_gemm(FAKE, FAKE, FAKE, 32, 128, 128, 128, 128, 3, FAKE, 1 << 30, None) == -1
    assert lib.dlm_op_gemm(FAKE, FAKE, FAKE, 32, 128, 128, 64, 128, 0, FAKE, 1 << 30, None) == -2
    assert lib.dlm_op_lm_head(FAKE, 4, 128, FAKE, 1024, 1024, FAKE, FAKE, None, None, None, FAKE, 1 << 30,
                              None) == -1
    # the head's vocabulary tiles are 256 wide
    assert lib.dlm_op_lm_head(FAKE, 4, 128, FAKE, 1152, 0, FAKE, FAKE, None, None, None, FAKE, 1 << 30,
                              None) == -2
    assert lib.dlm_op_lm_head(FAKE, 4, 128, FAKE, 1024, 0, FAKE, FAKE, C.c_void_p(4098), None, None, FAKE,
                              1 << 30, None) == -1  # misaligned entropy
    assert lib.dlm_op_attention(FAKE, 128, FAKE, FAKE, FAKE, None, 0, 1, 16, 4, 2, 64, 64, 0, 16, FAKE,
                                1 << 30, None) == -4
    assert lib.dlm_op_attention(FAKE, 128, FAKE, FAKE, FAKE, None, 0, 1, 16, 4, 2, 32, 64, 0, 65, FAKE,
                                1 << 30, None) == -3
    assert lib.dlm_op_rmsnorm(FAKE, 4, 12, FAKE, 1e-5, FAKE, None) == -2
    assert lib.dlm_op_rope_kv(FAKE, 1, 4, 4, 2, 48, 1e4, FAKE, FAKE, None, 0, 64, FAKE, 1 << 20, None) == -2


def test_status_strings():
    lib = L.load()
    for s in range(-6, 1):
        assert lib.dlm_status_string(s)
    assert lib.dlm_status_string(-6) == b"workspace too small"


def test_lora_adapter_validation():
    lib = L.load()
    st, h = create(tiny_cfg())
    assert st == 0
    try:
        arr = (C.c_void_p * 2)(4096, 4096)
        pa = C.cast(arr, C.POINTER(C.c_void_p))
        bad = (C.c_void_p * 2)(4096, 4100)  # misaligned second layer
        pb = C.cast(bad, C.POINTER(C.c_void_p))
        assert lib.dlm_model_enable_lora(h, 1) == -1            # nothing set yet
        assert lib.dlm_model_set_lora(h, pa, None, 128, 4.0) == -1
        assert lib.dlm_model_set_lora(h, pa, pa, 64, 4.0) == -4  # rank not a multiple of 128
        assert lib.dlm_model_set_lora(h, pa, pa, 384, 4.0) == -4  # above DLM_MAX_LORA_RANK
        assert lib.dlm_model_set_lora(h, pa, pa, 128, float("inf")) == -1
        assert lib.dlm_model_set_lora(h, pa, pb, 128, 4.0) == -1
        assert lib.dlm_model_set_lora(h, pa, pa, 128, 4.0) == 0
        assert lib.dlm_model_enable_lora(h, 1) == 0
        assert lib.dlm_model_enable_lora(h, 0) == 0
        assert lib.dlm_model_set_lora(h, None, None, 0, 0.0) == 0  # removal
        assert lib.dlm_model_enable_lora(h, 1) == -1
    finally:
        lib.dlm_model_destroy(h)


def test_missing_library_raises_instead_of_falling_back(monkeypatch, tmp_path):
    # the binding has no CPU or eager path: without the built library it refuses
    monkeypatch.setattr(L, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        L.load(str(tmp_path / "libdlm.so"))
