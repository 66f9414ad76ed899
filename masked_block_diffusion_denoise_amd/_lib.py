"""ctypes binding of libdlm.so: the C ABI of include/libdlm.h and include/libdlm_ops.h.

Argument marshalling only.  Every step of the path runs in the library's HIP
kernels; if the library is missing this module raises instead of falling back.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdlm.so")

DLM_OK = 0
NOALLOC_SCRATCH_BYTES = 64 << 20   # DLM_NOALLOC_SCRATCH_BYTES
STATUS = {0: "DLM_OK", -1: "DLM_ERR_INVALID_ARG", -2: "DLM_ERR_SHAPE", -3: "DLM_ERR_CAPACITY",
          -4: "DLM_ERR_UNSUPPORTED", -5: "DLM_ERR_HIP", -6: "DLM_ERR_WORKSPACE"}

EPI_STORE_BF16, EPI_RESIDUAL_F32, EPI_SWIGLU = 0, 1, 2
TIMER_LM_HEAD, TIMER_ATTENTION, TIMER_GATE_UP, TIMER_DOWN, TIMER_QKV = 0, 1, 2, 3, 4

# Every function declared in include/libdlm.h and include/libdlm_ops.h.
EXPORTS = [
    "dlm_model_create", "dlm_model_destroy", "dlm_model_set_lora", "dlm_model_enable_lora",
    "dlm_workspace_bytes", "dlm_prefill", "dlm_denoise_step", "dlm_denoise_step_ex",
    "dlm_commit", "dlm_commit_ex", "dlm_append_block", "dlm_denoise_step_noalloc", "dlm_status_string", "dlm_last_error", "dlm_set_kernel_timer",
    "dlm_op_gemm_workspace_bytes", "dlm_op_gemm", "dlm_op_rmsnorm", "dlm_op_rope_workspace_bytes",
    "dlm_op_rope_kv", "dlm_op_attention_workspace_bytes", "dlm_op_attention",
    "dlm_op_lm_head_workspace_bytes", "dlm_op_lm_head",
]


class DlmError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} -> {STATUS.get(status, status)}: {detail}")
        self.status = status


class Config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("d_ffn", C.c_int32),
                ("vocab", C.c_int32), ("mask_id", C.c_int32), ("rope_base", C.c_float),
                ("rms_eps", C.c_float)]


class Weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("final_norm", C.c_void_p), ("lm_head", C.c_void_p),
                ("attn_norm", C.POINTER(C.c_void_p)), ("wqkv", C.POINTER(C.c_void_p)),
                ("wo", C.POINTER(C.c_void_p)), ("ffn_norm", C.POINTER(C.c_void_p)),
                ("wgu", C.POINTER(C.c_void_p)), ("wdown", C.POINTER(C.c_void_p))]


class KV(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("batch", C.c_int32), ("capacity", C.c_int32)]


RULE_THRESHOLD, RULE_BOUND, RULE_ENTROPY = 0, 1, 2


class CommitOpts(C.Structure):
    """dlm_commit_opts: the sampler rule and its parameters (libdlm.h)."""
    _fields_ = [("rule", C.c_int32), ("min_threshold", C.c_float), ("scaling", C.c_float),
                ("entropy_bound", C.c_float), ("max_transfer", C.c_int32), ("stability_steps", C.c_int32),
                ("stop_entropy", C.c_float), ("prev_argmax", C.c_void_p), ("stable", C.c_void_p)]


_lib = None

vp, i32, f32, sz = C.c_void_p, C.c_int32, C.c_float, C.c_size_t

_SIGS = {
    "dlm_model_create": (i32, [C.POINTER(Config), C.POINTER(Weights), C.POINTER(vp)]),
    "dlm_model_destroy": (None, [vp]),
    "dlm_model_set_lora": (i32, [vp, C.POINTER(vp), C.POINTER(vp), i32, f32]),
    "dlm_model_enable_lora": (i32, [vp, i32]),
    "dlm_workspace_bytes": (sz, [vp, i32, i32]),
    "dlm_prefill": (i32, [vp, C.POINTER(KV), vp, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
    "dlm_denoise_step": (i32, [vp, C.POINTER(KV), vp, i32, vp, vp, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
    "dlm_commit": (i32, [vp, vp, vp, vp, i32, i32, vp, vp, vp, i32, vp, vp, vp]),
    "dlm_denoise_step_ex": (i32, [vp, C.POINTER(KV), vp, i32, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]),
    "dlm_denoise_step_noalloc": (i32, [vp, C.POINTER(KV), vp, i32, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp]),
    "dlm_commit_ex": (i32, [vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, i32, C.POINTER(CommitOpts), vp, vp, vp]),
    "dlm_append_block": (i32, [vp, C.POINTER(KV), vp, i32, vp, i32, i32, vp, vp, vp, vp, sz, vp]),
    "dlm_status_string": (C.c_char_p, [i32]),
    "dlm_set_kernel_timer": (i32, [i32, vp, vp]),
    "dlm_last_error": (C.c_char_p, []),
    "dlm_op_gemm_workspace_bytes": (sz, [i32, i32, i32]),
    "dlm_op_gemm": (i32, [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, sz, vp]),
    "dlm_op_rmsnorm": (i32, [vp, i32, i32, vp, f32, vp, vp]),
    "dlm_op_rope_workspace_bytes": (sz, [i32, i32, i32]),
    "dlm_op_rope_kv": (i32, [vp, i32, i32, i32, i32, i32, f32, vp, vp, vp, i32, i32, vp, sz, vp]),
    "dlm_op_attention_workspace_bytes": (sz, [i32, i32, i32, i32, i32, i32]),
    "dlm_op_attention": (i32, [vp, i32, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, vp,
                               sz, vp]),
    "dlm_op_lm_head_workspace_bytes": (sz, [i32, i32]),
    "dlm_op_lm_head": (i32, [vp, i32, i32, vp, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]),
}


def load(path: str | None = None):
    """Load libdlm.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    # torch ships its own HIP runtime; load it first so that libdlm binds to the
    # same runtime (one set of device pointers and streams in the process).
    import torch  # noqa: F401
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m masked_block_diffusion_denoise_amd.csrc.build` "
                           "(there is no fallback path)")
    lib = C.CDLL(p)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != DLM_OK:
        detail = _lib.dlm_last_error().decode(errors="replace") if _lib is not None else ""
        raise DlmError(fn, status, detail)


def call(fn: str, *args):
    lib = load()
    st = getattr(lib, fn)(*args)
    check(fn, st)
    return st
