"""Helpers for the GPU parity tests: device copies, workspaces and error measures."""
import ctypes as C

import numpy as np
import torch

from masked_block_diffusion_denoise_amd import _lib as L
from masked_block_diffusion_denoise_amd import runtime as R

DEV = "cuda"


def bf16(a):
    return R.to_bf16_device(a, DEV)


def f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def host(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


_ws = {}


def workspace(nbytes):
    w = _ws.setdefault("w", R.Workspace(DEV))
    return w.get(max(int(nbytes), 256))


def stream():
    return R.stream_handle()


def sync():
    torch.cuda.synchronize()


def rel_rms(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.sqrt(np.mean((a - b) ** 2)) / max(np.sqrt(np.mean(b ** 2)), 1e-30))


def announce(msg):
    print(f"[gpu-test] {msg}", flush=True)
