"""Benchmark of the masked block-diffusion denoising step on one MI355X.

Workload (default): one 8B-class decoder layer (hidden 4096, 32 query / 8 KV
heads of width 128, SwiGLU 14336) with the final norm, the fused 131072-vocab
LM head to confidence, and the threshold-0.9 commit; a 4096-position N(0,1)
KV prefix per row and a 32-position canvas with about half of it masked
(ragged per row); batch 32 (the headline) and batch 1.  Weights are random
N(0, 0.02) bf16 from a fixed seed.  One step = restore the canvas, one
dlm_denoise_step, one dlm_commit; inputs are resident in HBM before timing.

Prints one JSON line.  Per-kernel times come from HIP events that the library
records around the kernel inside the real step (dlm_set_kernel_timer).
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from masked_block_diffusion_denoise_amd import roofline as RL  # noqa: E402

METRIC = "committed tokens/s & denoise steps/s, 8B-class bf16 b=1/32; % HBM/MFMA roofline"


class HipEvents:
    """hipEvent_t pairs from the HIP runtime that torch (and so libdlm) uses."""

    def __init__(self):
        import torch
        self.h = C.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        self.h.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.h.hipEventDestroy.argtypes = [C.c_void_p]
        self.events = []

    def new(self):
        e = C.c_void_p()
        if self.h.hipEventCreate(C.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self.events.append(e)
        return e

    def ms(self, a, b) -> float:
        t = C.c_float()
        if self.h.hipEventElapsedTime(C.byref(t), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed (event not recorded?)")
        return float(t.value)

    def close(self):
        for e in self.events:
            self.h.hipEventDestroy(e)
        self.events = []


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("k_gemm.hip", "dlm_device.h", "dlm_internal.h"):
        h.update(open(os.path.join(ROOT, "masked_block_diffusion_denoise_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, batch: int):
    """HBM bytes per launch from committed rocprofv3 counter runs, if taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", "lm_head_traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p))
        if rec.get("source_hash") != kernel_source_hash():
            return None
        return rec.get("per_launch_bytes", {}).get(f"{kernel}_b{batch}")
    except Exception:
        return None


TIMERS = {"lm_head": 0, "attention": 1, "gate_up": 2, "down": 3, "qkv": 4}

# LM-head launches in a counter run, told apart from the other GEMMs by the
# head epilogue's template argument and the tile (k_gemm_tiled<EPI, BN, BM, ...>,
# EPI_HEAD = 3): 256 x 256 tiles at batch 32, 256 x 64 tiles at batch 1.
HEAD_KERNELS = {"lm_head_b32": re.compile(r"k_gemm_tiled<3, 256, 256,"), "lm_head_b1": re.compile(r"k_gemm_tiled<3, 256, 64,")}
COPY_KERNEL = re.compile(r"copyBuffer")


def copy_probe(mib: int) -> None:
    """A plain device-to-device copy of `mib` MiB, run three times before the steps
    so that a counter run sees a kernel whose HBM bytes are known."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def _counter_means(d: str, counter: str) -> dict:
    """Mean per-dispatch value of `counter` for each kernel name in a rocprofv3 csv directory."""
    import csv
    import glob
    vals: dict = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            if row["Counter_Name"] != counter:
                continue
            vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return vals


def traffic_from(fetch_dir: str, write_dir: str, copy_mib: int, command: str) -> dict:
    """Per-launch HBM bytes of the LM head from a FETCH_SIZE run and a WRITE_SIZE run,
    each scaled by what the counter read for the copy probe (known bytes / counter bytes)."""
    out = {"source_hash": kernel_source_hash(), "command": command, "copy_probe_bytes": copy_mib << 20,
           "per_launch_bytes": {}, "raw_kib": {}}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = _counter_means(d, counter)
        copies = [max(v) for k, v in vals.items() if COPY_KERNEL.search(k)]
        if not copies:
            raise SystemExit(f"no copy dispatch with {counter} in {d}")
        scale = (copy_mib << 20) / (max(copies) * 1024.0)
        out[f"{counter.lower()}_scale"] = round(scale, 4)
        for key, pat in HEAD_KERNELS.items():
            launches = [x for k, v in vals.items() if pat.search(k) for x in v]
            if not launches:
                continue
            kib = sum(launches) / len(launches)
            out["raw_kib"][f"{key}_{counter}"] = round(kib, 1)
            out["per_launch_bytes"][key] = out["per_launch_bytes"].get(key, 0) + round(kib * 1024.0 * scale)
    return out


def run_batch(model, shape, B, steps, warmup, P=4096, Lb=32, seed=3):
    import numpy as np
    import torch

    import synth
    from masked_block_diffusion_denoise_amd import _lib as L
    from masked_block_diffusion_denoise_amd import runtime as R

    sess = R.Session(model, B, P + Lb + 64, Lb)
    k, v = synth.kv_prefix(shape, B, P, seed=seed)
    sess.kv.write(0, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    del k, v
    sess.prefix.fill_(P)
    sess.max_prefix = P
    canvas, masked = synth.ragged_canvas(shape, B, Lb, seed=seed)
    tc = torch.from_numpy(canvas).cuda()
    tm = torch.from_numpy(masked).cuda()
    tau = torch.full((B,), 0.9, dtype=torch.float32, device="cuda")
    quota = torch.ones(B, dtype=torch.int32, device="cuda")
    max_steps = 32
    ev = HipEvents()
    lib = L.load()

    def step():
        sess.canvas.copy_(tc)
        sess.masked.copy_(tm)
        sess.steps.zero_()
        sess.denoise_step()
        sess.commit(tau, quota, max_steps)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    pairs = {n: [(ev.new(), ev.new()) for _ in range(steps)] for n in TIMERS}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        for n, kid in TIMERS.items():
            lib.dlm_set_kernel_timer(kid, pairs[n][i][0], pairs[n][i][1])
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for kid in TIMERS.values():
        lib.dlm_set_kernel_timer(kid, None, None)
    ms_step = (t1 - t0) * 1e3 / steps
    kms = {n: sum(ev.ms(a, b) for a, b in pairs[n]) / steps for n in TIMERS}
    ev.close()
    committed = int(sess.n_committed.sum().item())
    flags = sess.flags.cpu().tolist()
    mrows = int(masked.sum())
    kernels = {}
    for n, t in kms.items():
        by, fl = RL.kernel_work(n, B, Lb, P, mrows, shape.d_model, shape.n_heads, shape.n_kv_heads,
                                shape.head_dim, shape.d_ffn, shape.vocab)
        kernels[n] = {"ms": round(t, 4), "bytes": by, "flops": fl,
                      "roofline": RL.roofline(by, fl, t, traffic_for(n, B))}
    return {"batch": B, "ms_per_step": ms_step, "steps_per_s": 1e3 / ms_step,
            "committed_per_step": committed, "committed_tokens_per_s": committed * 1e3 / ms_step,
            "masked_rows": mrows, "kernels": kernels, "flags": flags,
            "inputs": (canvas, masked)}


def cpu_baseline(w, shape, B, canvas, masked, P=4096, seed=3, rows=16):
    """The oracle (float64 NumPy) on a bounded sample: `rows` batch rows of the step."""
    import numpy as np

    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        threads = len(os.sched_getaffinity(0))
    k, v = synth.kv_prefix(shape, min(rows, B), P, seed=seed) if B >= rows else synth.kv_prefix(shape, B, P, seed)
    n = min(rows, B)
    t0 = time.perf_counter()
    for b in range(n):
        cache = oracle.KVCache(shape)
        cache.k[0] = k[b].astype(np.float64)
        cache.v[0] = v[b].astype(np.float64)
        lo = oracle.denoise_logits(w, shape, cache, canvas[b])
        conf, arg = oracle.confidence(lo)
        oracle.commit(conf, arg, canvas[b], masked[b].astype(bool), 0.9, 1, 0, 32)
    t = (time.perf_counter() - t0) / n
    return {"value": round(1.0 / (t * B), 6), "unit": "denoise steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of the {B} batch rows of one step (layer + head over all 32 canvas rows + commit, "
                      f"float64 NumPy), {t:.2f} s per row, scaled to the whole batch"}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--batches", default="32,1", help="batch sizes; the first is the headline")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run a plain copy of this many MiB first (scale for counter runs)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: digest two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "`bench.py --copy-probe-mib N` into profiles/lm_head_traffic.json")
    ap.add_argument("--traffic-command", default="", help="the counter command, recorded with --traffic-from")
    a = ap.parse_args(argv)
    if a.traffic_from:
        rec = traffic_from(a.traffic_from[0], a.traffic_from[1], a.copy_probe_mib or 1024, a.traffic_command)
        with open(os.path.join(ROOT, "profiles", "lm_head_traffic.json"), "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))
        return 0
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: libdlm has no multi-GPU path (batch rows would shard across "
              "GPUs by data parallelism with no exchange). Run with --gpus 1.", file=sys.stderr)
        return 2
    import numpy as np
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        return 1
    import synth
    from masked_block_diffusion_denoise_amd import runtime as R

    if a.copy_probe_mib:
        copy_probe(a.copy_probe_mib)
    shape = synth.LAYER_8B
    print(f"[bench] generating weights", file=sys.stderr, flush=True)
    w = synth.model_weights(shape, seed=0)
    model = R.DlmModel.from_arrays(R.ModelConfig.of(shape), w)
    batches = [int(x) for x in a.batches.split(",")]
    res = {}
    for B in batches:
        print(f"[bench] batch {B}", file=sys.stderr, flush=True)
        res[B] = run_batch(model, shape, B, a.steps, a.warmup)
    head = res[batches[0]]
    B0 = batches[0]
    dom = max(head["kernels"], key=lambda n: head["kernels"][n]["ms"])
    out = {
        "metric": METRIC,
        "value": round(head["steps_per_s"], 3),
        "unit": "denoise steps/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded random-init N(0,0.02) bf16 weights, N(0,1) 4096-position KV prefix, "
                "ragged ~50%-masked 32-position canvas",
        "config": {"workload": f"one 8B-class decoder layer (d 4096, 32/8 heads x 128, SwiGLU 14336) + final "
                               f"norm + fused 131072-vocab LM head to confidence + threshold-0.9 commit; "
                               f"prefix 4096, canvas 32; batch {B0}",
                   "global_batch": B0, "seq_len": 4096 + 32, "parallelism": "single GPU"},
        "committed_tokens_per_s": round(head["committed_tokens_per_s"], 2),
        "committed_per_step": head["committed_per_step"],
        "dominant_kernel": dom,
        "roofline": head["kernels"][dom]["roofline"],
        "kernels": {n: {"ms": k["ms"], **k["roofline"]} for n, k in head["kernels"].items()},
    }
    for B in batches[1:]:
        r = res[B]
        out[f"b{B}"] = {"steps_per_s": round(r["steps_per_s"], 3), "ms_per_step": round(r["ms_per_step"], 4),
                        "committed_tokens_per_s": round(r["committed_tokens_per_s"], 2),
                        "kernels": {n: {"ms": k["ms"], **k["roofline"]} for n, k in r["kernels"].items()}}
    if not a.no_cpu:
        print(f"[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        canvas, masked = head["inputs"]
        out["cpu_baseline"] = cpu_baseline(w, shape, B0, canvas, masked)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
