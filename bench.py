"""Benchmark of the masked block-diffusion denoising step on one MI355X.

Workload (default): one 8B-class decoder layer (hidden 4096, 32 query / 8 KV
heads of width 128, SwiGLU 14336) with the final norm, the fused 131072-vocab
LM head to confidence, and the threshold-0.9 commit; a 4096-position N(0,1)
KV prefix per row and a 32-position canvas with about half of it masked
(ragged per row); batch 32 (the headline) and batch 1.  Weights are random
N(0, 0.02) bf16 from a fixed seed.  One step = one dlm_denoise_step and one
dlm_commit on a canvas of its own; every step's inputs are staged in HBM
before timing.

Prints one JSON line.  Per-kernel times come from HIP events that the library
records around the kernel inside the real step (dlm_set_kernel_timer).  The
single-layer steps rotate over three copies of the layer weights and of the KV
prefix (the last-level cache holds 256 MB; one copy would let a step reuse the
previous step's weights, which a 32-layer model never can); the median and
p10/p90 of per-step event times are reported beside the wall-clock mean, with
the GPU clock sampled during the timed steps and the ROCm version.

The same line carries, under "e2e", the full 32-layer 8B-class model (random
N(0, 0.02) bf16 weights drawn on the device): block-diffusion decoding at batch
1 (1024-token prompt) and batch 32 (2048-token prompts), a batch-4 run over a
65536-position synthetic N(0,1) K/V prefix, greedy causal (AR) decoding and
greedy linear self-speculation with a rank-128 o_proj adapter, and the
runtime's whole block loop at batch 1 eager and with the anchor-token layout
replaying a captured graph, 256 generated tokens per sequence each (--no-e2e
skips them).
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

    def record(self, e) -> None:
        """Record e on the stream libdlm launches on (torch's current stream)."""
        import torch
        self.h.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        if self.h.hipEventRecord(e, C.c_void_p(torch.cuda.current_stream().cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def close(self):
        for e in self.events:
            self.h.hipEventDestroy(e)
        self.events = []


def kernel_source_hash() -> str:
    """Hash of the kernel sources without comments and whitespace: a counter
    record stays valid across comment-only edits, not across code changes."""
    h = hashlib.sha256()
    for f in ("k_gemm.hip", "k_attention.hip", "k_small.hip", "dlm_device.h", "dlm_internal.h"):
        text = open(os.path.join(ROOT, "masked_block_diffusion_denoise_amd", "csrc", f)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("".join(text.split()).encode())
    return h.hexdigest()[:16]


COUNTERS_FILE = os.path.join(ROOT, "profiles", "kernel_counters.json")


def traffic_for(kernel: str, batch: int):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by a copy of known
    size) from the committed counter record, if taken on the current kernel source."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    try:
        rec = json.load(open(COUNTERS_FILE))
        if rec.get("source_hash") != kernel_source_hash():
            return None
        return rec.get("kernels", {}).get(f"{kernel}_b{batch}", {}).get("hbm_bytes")
    except Exception:
        return None


TIMERS = {"lm_head": 0, "attention": 1, "gate_up": 2, "down": 3, "qkv": 4, "o_proj": 5, "final_norm": 6}
ROTATE = 3   # weight/KV copies the single-layer steps rotate over

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


# The libdlm launches of one denoise step in order, labelled by position: the
# k-th tiled GEMM of a step is QKV, O, gate/up, down (the head is told apart by
# its epilogue argument, EPI_HEAD = 3, or its own kernel).
_GEMM_ORDER = ("qkv", "o_proj", "gate_up", "down")
_NAMED = [("k_embed_norm", "embed_norm"), ("k_rope_kv", "rope_kv"), ("k_attn_merge", "attention_merge"),
          ("k_attn<", "attention"), ("k_resid_norm", "resid_norm"), ("k_rmsnorm", "rmsnorm"),
          ("k_splitk_reduce", "splitk_reduce"), ("k_masked_norm", "final_norm"), ("k_head_merge", "head_merge"),
          ("k_commit", "commit"), ("k_gemm_head_rows", "lm_head"), ("k_gemm_tiled<3,", "lm_head")]


def label_steps(dispatches):
    """[(kernel name, grid size, {counter: value})] in dispatch order -> per-step
    lists of (label, values); a step starts at the embedding kernel.  The
    residual norm after O is 'o_norm', after down 'down_norm'; the reduction
    after gate/up is 'gate_up_reduce'.  The batch of a step is the final norm's
    grid (one 256-thread workgroup per canvas row, 32 rows per sequence)."""
    steps, cur, ngemm = [], None, 0
    for name, grid, vals in dispatches:
        if "dlm::" not in name:
            continue
        if "k_embed_norm" in name:
            cur = {"items": [], "batch": None}
            steps.append(cur)
            ngemm = 0
        if cur is None:
            continue
        lab = None
        for pat, l in _NAMED:
            if pat in name:
                lab = l
                break
        if lab is None and "k_gemm_tiled<" in name:
            lab = _GEMM_ORDER[ngemm] if ngemm < len(_GEMM_ORDER) else "gemm"
            ngemm += 1
        if lab in ("resid_norm", "rmsnorm"):
            lab = "o_norm" if ngemm <= 2 else "down_norm"
        if lab == "splitk_reduce":
            lab = "gate_up_reduce"
        if lab == "final_norm" and grid:
            cur["batch"] = max(1, grid // 256 // 32)
        cur["items"].append((lab or name, vals))
    return steps


def _read_counters(dirs):
    """Dispatches of rocprofv3 counter-collection csv files: {dispatch id: [name, grid, {counter: value}]}."""
    import csv
    import glob
    d = {}
    for base in dirs:
        for f in glob.glob(os.path.join(base, "**", "*counter_collection.csv"), recursive=True):
            for row in csv.DictReader(open(f)):
                key = (base, int(row["Dispatch_Id"]))
                rec = d.setdefault(key, [row["Kernel_Name"], int(float(row.get("Grid_Size", 0) or 0)), {}])
                rec[2][row["Counter_Name"]] = rec[2].get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    return d


def counters_from(dirs, copy_mib: int, command: str) -> dict:
    """Per-kernel counter means from rocprofv3 --pmc runs of `bench.py --no-e2e
    --copy-probe-mib N` (one run per counter group), labelled by position in
    the step and batch.  FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled
    by what each read for the copy probe of known size; hbm_bytes is their sum."""
    out = {"source_hash": kernel_source_hash(), "command": command, "copy_probe_bytes": copy_mib << 20,
           "scale": {}, "kernels": {}}
    agg = {}
    for base in dirs:
        disp = _read_counters([base])
        order = sorted(disp.items(), key=lambda kv: kv[0][1])
        for name, grid, vals in (v for _, v in order):
            if COPY_KERNEL.search(name):
                for c, x in vals.items():
                    if c in ("FETCH_SIZE", "WRITE_SIZE"):
                        out["scale"][c] = max(out["scale"].get(c, 0.0), x)
        for st in label_steps([v for _, v in order]):
            if not st["batch"]:
                continue
            for lab, vals in st["items"]:
                rec = agg.setdefault(f"{lab}_b{st['batch']}", {})
                for c, x in vals.items():
                    rec.setdefault(c, []).append(x)
    for c in list(out["scale"]):
        out["scale"][c] = round((copy_mib << 20) / (out["scale"][c] * 1024.0), 4)
    for key, rec in sorted(agg.items()):
        k = {c: round(sum(v) / len(v), 1) for c, v in rec.items()}
        k["dispatches"] = max(len(v) for v in rec.values())
        by = 0.0
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            if c in k and c in out["scale"]:
                by += k[c] * 1024.0 * out["scale"][c]
        if by:
            k["hbm_bytes"] = round(by)
        out["kernels"][key] = k
    return out


def _pct(xs, q):
    import numpy as np
    return round(float(np.percentile(np.asarray(xs), q)), 4)


class ClockSampler:
    """Samples the GPU's current shader clock (sysfs pp_dpm_sclk, the '*' level)
    in a thread while the timed steps run; no-op where sysfs is not readable."""

    def __init__(self, period_s=0.002):
        import glob
        import threading
        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.samples, self.period = [], period_s
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        for pth in self.paths:
            try:
                for line in open(pth):
                    if line.rstrip().endswith("*"):
                        m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                        if m:
                            return int(m.group(1))
            except OSError:
                continue
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.paths:
            self._t.start()
        return self

    def __exit__(self, *a):
        self._stop.set()
        if self.paths:
            self._t.join(timeout=2)

    def summary(self):
        if not self.samples:
            return None
        xs = sorted(self.samples)
        return {"samples": len(xs), "min_mhz": xs[0], "median_mhz": xs[len(xs) // 2], "max_mhz": xs[-1]}


def gpu_info() -> dict:
    import torch
    props = torch.cuda.get_device_properties(0)
    out = {"device": torch.cuda.get_device_name(0) or getattr(props, "gcnArchName", ""),
           "compute_units": props.multi_processor_count, "hip_runtime": torch.version.hip}
    try:
        out["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        out["rocm"] = None
    return out


def layer_copies(model, n):
    """``model`` and n - 1 copies of its layer weights on the device (embedding,
    final norm and the 1 GB head shared)."""
    from masked_block_diffusion_denoise_amd import runtime as R
    out = [model]
    for _ in range(n - 1):
        t = dict(model.t)
        for k in ("attn_norm", "wqkv", "wo", "ffn_norm", "wgu", "wdown"):
            t[k] = [x.clone() for x in model.t[k]]
        out.append(R.DlmModel(model.cfg, t, model.device))
    return out


def run_batch(models, shape, B, steps, warmup, P=4096, Lb=32, seed=3):
    import numpy as np
    import torch

    import synth
    from masked_block_diffusion_denoise_amd import _lib as L
    from masked_block_diffusion_denoise_amd import runtime as R

    k, v = synth.kv_prefix(shape, B, P, seed=seed)
    kt, vt = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    del k, v
    sessions = []
    for m in models:        # one KV prefix per weight copy: a step reads neither the previous one's
        sess = R.Session(m, B, P + Lb + 64, Lb)
        sess.kv.write(0, kt, vt)
        sess.prefix.fill_(P)
        sess.max_prefix = P
        sessions.append(sess)
    del kt, vt
    canvas, masked = synth.ragged_canvas(shape, B, Lb, seed=seed)
    tc = torch.from_numpy(canvas).cuda()
    tm = torch.from_numpy(masked).cuda()
    tau = torch.full((B,), 0.9, dtype=torch.float32, device="cuda")
    quota = torch.ones(B, dtype=torch.int32, device="cuda")
    max_steps = 32
    ev = HipEvents()
    lib = L.load()

    # The commit rewrites the canvas, the mask and the step counter in place, so
    # every step gets its own copies of the synthetic inputs, staged in HBM
    # before any timing: the timed region holds the denoise step and the commit
    # only, not the restores.
    def stage(count):
        return [(tc.clone(), tm.clone(), torch.zeros(B, dtype=torch.int32, device="cuda")) for _ in range(count)]

    def step(sess, bufs):
        sess.canvas, sess.masked, sess.steps = bufs
        sess.denoise_step()
        sess.commit(tau, quota, max_steps)

    n = len(sessions)
    warm_in, timed_in, one_in = stage(warmup), stage(steps), stage(steps)
    for i in range(warmup):
        step(sessions[i % n], warm_in[i])
    torch.cuda.synchronize()
    pairs = {nm: [(ev.new(), ev.new()) for _ in range(steps)] for nm in TIMERS}
    step_ev = [(ev.new(), ev.new()) for _ in range(steps)]
    torch.cuda.synchronize()
    with ClockSampler() as clk:
        t0 = time.perf_counter()
        for i in range(steps):
            for nm, kid in TIMERS.items():
                lib.dlm_set_kernel_timer(kid, pairs[nm][i][0], pairs[nm][i][1])
            ev.record(step_ev[i][0])
            step(sessions[i % n], timed_in[i])
            ev.record(step_ev[i][1])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    for kid in TIMERS.values():
        lib.dlm_set_kernel_timer(kid, None, None)
    ms_step = (t1 - t0) * 1e3 / steps
    per_step = [ev.ms(a, b) for a, b in step_ev]
    kms = {nm: [ev.ms(a, b) for a, b in pairs[nm]] for nm in TIMERS}
    # the same steps on one weight/KV copy: what the last-level cache gives back
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(steps):
        step(sessions[0], one_in[i])
    torch.cuda.synchronize()
    one_copy_ms = (time.perf_counter() - t2) * 1e3 / steps
    ev.close()
    last = sessions[(steps - 1) % n]
    committed = int(last.n_committed.sum().item())
    flags = [int(x) for s_ in sessions for x in s_.flags.cpu().tolist()]
    mrows = int(masked.sum())
    kernels = {}
    for nm, ts in kms.items():
        t = sum(ts) / len(ts)
        rec = {"ms": round(t, 4), "ms_median": _pct(ts, 50)}
        if nm != "final_norm":
            by, fl = RL.kernel_work(nm, B, Lb, P, mrows, shape.d_model, shape.n_heads, shape.n_kv_heads,
                                    shape.head_dim, shape.d_ffn, shape.vocab)
            rec.update(bytes=by, flops=fl, roofline=RL.roofline(by, fl, t, traffic_for(nm, B)))
        kernels[nm] = rec
    # The last layer's down projection, when split over K, leaves its partial
    # products to the final norm of the masked rows (final_norm), so "down"
    # alone times only the partials: down + final_norm bounds it with its reduction.
    dn = kernels["down"]
    t = dn["ms"] + kernels["final_norm"]["ms"]
    kernels["down_with_final_norm"] = {"ms": round(t, 4), "bytes": dn["bytes"], "flops": dn["flops"],
                                       "roofline": RL.roofline(dn["bytes"], dn["flops"], t, None)}
    return {"batch": B, "ms_per_step": ms_step, "steps_per_s": 1e3 / ms_step,
            "step_ms": {"wall_mean": round(ms_step, 4), "median": _pct(per_step, 50), "p10": _pct(per_step, 10),
                        "p90": _pct(per_step, 90), "one_copy_wall_mean": round(one_copy_ms, 4)},
            "gpu_clock": clk.summary(),
            "committed_per_step": committed, "committed_tokens_per_s": committed * 1e3 / ms_step,
            "masked_rows": mrows, "kernels": kernels, "flags": flags,
            "inputs": (canvas, masked)}


def blas_setup():
    """The BLAS thread count for the oracle: the host's CPU share (the affinity
    set, capped by OMP_NUM_THREADS where the machine sets it), set explicitly."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    info = {"threads": n, "affinity_cpus": len(os.sched_getaffinity(0)), "blas": None, "cpu_model": None}
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            info["blas"] = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return info


def cpu_baseline(w, shape, inputs, P=4096, sample_rows=16):
    """The oracle (float64 NumPy) on bounded samples of the configured workloads:
    the one-layer step at batch 32 (``sample_rows`` rows, scaled to the batch; the
    headline leg), the same step at batch 1, and config 1 (the tiny model) end to end."""
    import numpy as np

    import oracle
    import synth
    import contextlib
    info = blas_setup()
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=info["threads"], user_api="blas")
    except Exception:
        limit = contextlib.nullcontext()

    def layer_rows(B, n):
        canvas, masked = inputs[B]
        k, v = synth.kv_prefix(shape, n, P, seed=3)
        t0 = time.perf_counter()
        for b in range(n):
            cache = oracle.KVCache(shape)
            cache.k[0] = k[b].astype(np.float64)
            cache.v[0] = v[b].astype(np.float64)
            lo = oracle.denoise_logits(w, shape, cache, canvas[b])
            conf, arg = oracle.confidence(lo)
            oracle.commit(conf, arg, canvas[b], masked[b].astype(bool), 0.9, 1, 0, 32)
        return (time.perf_counter() - t0) / n

    legs = {}
    rows = min(sample_rows, 32)
    with limit:
        t32 = layer_rows(32, rows) if 32 in inputs else None
        t1 = layer_rows(1, 1) if 1 in inputs else None
        tiny = synth.TINY
        wt = synth.model_weights(tiny, seed=0)
        pr = synth.prompt(tiny, 1, 32, seed=0)[0]
        t0 = time.perf_counter()
        out, st, _ = oracle.generate_block_diffusion(wt, tiny, pr, 32, 16, 16, 0.9, 1)
        tt = time.perf_counter() - t0
    if t1 is not None:
        legs["layer_step_b1"] = {"value": round(1.0 / t1, 6), "unit": "denoise steps/s",
                                 "sample": "the whole batch-1 step (one row: layer + head + commit)"}
    legs["tiny_e2e_b1"] = {"value": round(len(out) / tt, 3), "unit": "committed tokens/s",
                           "denoise_steps_per_s": round(st.denoise_nfe / tt, 3),
                           "sample": "the tiny model (2 layers, d 128, vocab 1024), 32-token prompt, 32 tokens in "
                                     "2 blocks of 16, prefill and appends included"}
    head = {"value": round(1.0 / (t32 * 32), 6), "unit": "denoise steps/s", "cores": info["threads"],
            "kind": "oracle",
            "sample": f"{rows} of the 32 batch rows of one batch-32 step (layer + head over all 32 canvas rows + "
                      f"commit, float64 NumPy), {t32:.2f} s per row, scaled to the whole batch"} if t32 else {}
    head.update({"cpu_model": info["cpu_model"], "blas": info["blas"], "affinity_cpus": info["affinity_cpus"],
                 "legs": legs})
    return head


# ------------------------------------------------------------------ full model
def _step_bound_ms(shape, B, L, P, masked_rows) -> float:
    """Roofline of one denoise step of the whole model: per kernel the larger of
    its HBM and MFMA time, summed over the layers, plus the head."""
    hw = RL.MI355X_BF16
    t = 0.0
    for n in ("qkv", "attention", "o_proj", "gate_up", "down"):
        by, fl = RL.kernel_work(n, B, L, P, masked_rows, shape.d_model, shape.n_heads, shape.n_kv_heads,
                                shape.head_dim, shape.d_ffn, shape.vocab)
        t += shape.n_layers * max(by / hw.hbm_bytes_per_s, fl / hw.flops_per_s)
    by, fl = RL.kernel_work("lm_head", B, L, P, masked_rows, shape.d_model, shape.n_heads, shape.n_kv_heads,
                            shape.head_dim, shape.d_ffn, shape.vocab)
    return 1e3 * (t + max(by / hw.hbm_bytes_per_s, fl / hw.flops_per_s))


def e2e_block_diffusion(model, shape, B, T, gen, Lb, max_steps, synthetic_prefix=False, seed=1):
    """Prefill (or a synthetic N(0,1) K/V prefix), then blocks of denoise + commit
    until no mask is left (one host read of the rows' remaining masks per step),
    then the post-block append; threshold 0.9, quota 1."""
    import torch

    import synth
    from masked_block_diffusion_denoise_amd import runtime as R

    sess = R.Session(model, B, T + gen + Lb, Lb)
    dev = model.device
    prefill_ms = None
    if synthetic_prefix:
        c, kv = model.cfg, sess.kv
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        kv.k.view(c.n_layers, B, c.n_kv_heads, kv.capacity, c.head_dim)[:, :, :, :T].normal_(generator=g)
        kv.v.view(c.n_layers, B, c.n_kv_heads, kv.capacity // 16, c.head_dim, 16)[:, :, :, :T // 16].normal_(
            generator=g)
        sess.prefix.fill_(T)
        sess.max_prefix = T
    else:
        prompt = torch.from_numpy(synth.prompt(shape, B, T, seed=seed)).to(dev)
        sess.prefill(prompt[:, :min(T, 64)], ws_rows=min(B * T, 8192))  # warm-up of the prefill path
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        sess.prefill(prompt, ws_rows=min(B * T, 8192))
        torch.cuda.synchronize()
        prefill_ms = (time.perf_counter() - t0) * 1e3
    tau = torch.full((B,), 0.9, dtype=torch.float32, device=dev)
    quota = torch.ones(B, dtype=torch.int32, device=dev)
    ev = HipEvents()
    steps, appends, per_block = [], [], []
    n_blocks = -(-gen // Lb)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_blocks):
        sess.begin_block()
        n = 0
        while True:
            a, b = ev.new(), ev.new()
            ev.record(a)
            sess.denoise_step()
            sess.commit(tau, quota, max_steps)
            ev.record(b)
            steps.append((a, b))
            n += 1
            if int(sess.n_left.max().item()) == 0:
                break
        a, b = ev.new(), ev.new()
        ev.record(a)
        sess.append_block()
        ev.record(b)
        appends.append((a, b))
        per_block.append(n)
    torch.cuda.synchronize()
    decode_s = time.perf_counter() - t0
    step_ms = sum(ev.ms(a, b) for a, b in steps) / len(steps)
    append_ms = sum(ev.ms(a, b) for a, b in appends) / len(appends)
    ev.close()
    tokens = B * n_blocks * Lb
    nfe = len(steps)
    # masked rows scored, averaged over the steps: each step of a block commits
    # one position per row until the last allowed step commits the rest
    masked = sum(B * (Lb - s) for blk in per_block for s in range(blk)) / nfe
    bound = _step_bound_ms(shape, B, Lb, T + gen // 2, masked)
    del sess
    torch.cuda.empty_cache()
    out = {"batch": B, "prompt": T, "synthetic_prefix": synthetic_prefix, "generated_per_row": n_blocks * Lb,
           "block": Lb, "max_steps": max_steps,
           "decode_s": round(decode_s, 4), "committed_tokens_per_s": round(tokens / decode_s, 2),
           "denoise_nfe": nfe, "post_block_nfe": n_blocks, "tokens_per_forward": round(n_blocks * Lb / nfe, 3),
           "ms_per_denoise_step": round(step_ms, 4), "denoise_steps_per_s": round(1e3 / step_ms, 3),
           "ms_per_append": round(append_ms, 4), "steps_per_block": per_block,
           "step_roofline_ms": round(bound, 4), "step_roofline_frac": round(bound / step_ms, 4)}
    if prefill_ms is not None:
        out["prefill_ms"] = round(prefill_ms, 3)
        out["e2e_tokens_per_s"] = round(tokens / (decode_s + prefill_ms / 1e3), 2)
    return out


def e2e_generate(model, shape, B, T, gen, Lb, max_steps, anchor=False, graph_steps=0, seed=1):
    """The runtime's whole block loop (prefill included): eager, or with the
    anchor layout and the loop replaying a captured graph of graph_steps steps."""
    import torch

    import synth
    from masked_block_diffusion_denoise_amd import runtime as R

    prompt = torch.from_numpy(synth.prompt(shape, B, T, seed=seed)).to(model.device)
    R.Session(model, B, T + Lb + 64, Lb).generate(prompt, Lb, max_steps, anchor=anchor,
                                                  graph_steps=graph_steps)  # warm-up
    sess = R.Session(model, B, T + gen + Lb, Lb)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _, st = sess.generate(prompt, gen, max_steps, anchor=anchor, graph_steps=graph_steps)
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    del sess
    torch.cuda.empty_cache()
    return {"batch": B, "prompt": T, "generated_per_row": gen, "anchor": anchor, "graph_steps": graph_steps,
            "e2e_s": round(total, 4), "e2e_tokens_per_s": round(B * gen / total, 2),
            "denoise_nfe": st.denoise_nfe, "steps_per_block": st.steps_per_block,
            "tokens_per_forward": round(st.tokens_per_denoise_forward, 3)}


def e2e_ar(model, shape, T, n_new, seed=1):
    """Greedy causal decoding at batch 1: prefill, then one-token appends."""
    import torch

    import synth
    from masked_block_diffusion_denoise_amd import runtime as R

    sess = R.Session(model, 1, T + n_new + 64, 1)
    prompt = torch.from_numpy(synth.prompt(shape, 1, T, seed=seed)).to(model.device)
    sess.generate_ar(prompt[:, :64], 4)  # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    toks = sess.generate_ar(prompt, n_new)
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    del sess
    torch.cuda.empty_cache()
    return {"batch": 1, "prompt": T, "generated": n_new, "e2e_s": round(total, 4),
            "e2e_tokens_per_s": round(n_new / total, 2)}, toks.cpu().numpy()[0]


def e2e_linear_spec(model, shape, T, n_new, window=32, rank=128, scale=4.0, seed=1, ar_tokens=None):
    """Greedy linear self-speculation at batch 1 with a random-init rank-128
    adapter (N(0, 0.02)) on every layer's output projection, used by the draft."""
    import numpy as np
    import torch

    import synth
    from masked_block_diffusion_denoise_amd import runtime as R

    c, dev = model.cfg, model.device
    g = torch.Generator(device=dev)
    g.manual_seed(seed + 100)
    rn = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device=dev).normal_(0.0, 0.02, generator=g)
    model.set_lora({"a": [rn(rank, c.n_heads * c.head_dim) for _ in range(c.n_layers)],
                    "b": [rn(c.d_model, rank) for _ in range(c.n_layers)], "scale": scale})
    sess = R.Session(model, 1, T + n_new + 2 * window, window)
    prompt = torch.from_numpy(synth.prompt(shape, 1, T, seed=seed)).to(dev)
    sess.generate_linear_spec(prompt[:, :64], 4, window)  # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    toks, accepted, _ = sess.generate_linear_spec(prompt, n_new, window)
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    model.set_lora(None)
    del sess
    torch.cuda.empty_cache()
    out = {"batch": 1, "prompt": T, "generated": n_new, "window": window, "lora_rank": rank, "lora_scale": scale,
           "rounds": len(accepted), "mean_accepted_drafts": round(float(np.mean(accepted)), 3),
           "tokens_per_round": round(n_new / len(accepted), 3), "accepted_per_round": accepted,
           "e2e_s": round(total, 4), "e2e_tokens_per_s": round(n_new / total, 2)}
    if ar_tokens is not None:
        same = np.asarray(toks[:n_new]) == np.asarray(ar_tokens[:n_new])
        out["agrees_with_ar_for_first"] = int(n_new if same.all() else np.argmin(same))
    return out


def run_e2e(gen=256) -> dict:
    import torch

    import synth
    from masked_block_diffusion_denoise_amd import runtime as R

    shape = synth.DENSE_8B
    print("[bench] e2e: drawing 8B-class weights on the device", file=sys.stderr, flush=True)
    model = R.DlmModel.random(R.ModelConfig.of(shape), seed=0)
    res = {"model": "dense 8B-class, 32 layers, d 4096, 32/8 heads x 128, SwiGLU 14336, vocab 131072, "
                    "random N(0,0.02) bf16 weights"}
    legs = [("block_diffusion_b1", dict(B=1, T=1024, gen=gen, Lb=32, max_steps=32)),
            ("block_diffusion_b32", dict(B=32, T=2048, gen=gen, Lb=32, max_steps=16)),
            ("long_prefix_b4", dict(B=4, T=65536, gen=gen, Lb=32, max_steps=16, synthetic_prefix=True))]
    for name, kw in legs:
        print(f"[bench] e2e {name}", file=sys.stderr, flush=True)
        res[name] = e2e_block_diffusion(model, shape, **kw)
    for name, kw in (("generate_b1_eager", dict()), ("generate_b1_anchor_graph", dict(anchor=True, graph_steps=31))):
        print(f"[bench] e2e {name}", file=sys.stderr, flush=True)
        res[name] = e2e_generate(model, shape, 1, 1024, gen, 32, 32, **kw)
    print("[bench] e2e ar_b1", file=sys.stderr, flush=True)
    res["ar_b1"], ar_tokens = e2e_ar(model, shape, 1024, gen)
    print("[bench] e2e linear_spec_b1", file=sys.stderr, flush=True)
    res["linear_spec_b1"] = e2e_linear_spec(model, shape, 1024, gen, ar_tokens=ar_tokens)
    del model
    torch.cuda.empty_cache()
    return res


def assemble(res: dict, batches: list, steps: int, warmup: int, gpu: dict) -> dict:
    """The bench line (one JSON object) from the per-batch results of run_batch."""
    head = res[batches[0]]
    B0 = batches[0]
    timed = ("lm_head", "attention", "gate_up", "down", "qkv", "o_proj")
    dom = max(timed, key=lambda n: head["kernels"][n]["ms"])
    kern = lambda r: {n: {"ms": k["ms"], "ms_median": k.get("ms_median"), **k.get("roofline", {})}
                      for n, k in r["kernels"].items()}
    out = {
        "metric": METRIC,
        "value": round(head["steps_per_s"], 3),
        "unit": "denoise steps/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded random-init N(0,0.02) bf16 weights, N(0,1) 4096-position KV prefix, "
                "ragged ~50%-masked 32-position canvas",
        "config": {"workload": f"one 8B-class decoder layer (d 4096, 32/8 heads x 128, SwiGLU 14336) + final "
                               f"norm + fused 131072-vocab LM head to confidence + threshold-0.9 commit; "
                               f"prefix 4096, canvas 32; batch {B0}; value = steps/s of this one-layer step "
                               f"(full 32-layer model figures: e2e)",
                   "global_batch": B0, "seq_len": 4096 + 32, "parallelism": "single GPU"},
        "step_ms": head["step_ms"],
        "timing": {"protocol": f"{warmup} untimed steps, then {steps} timed between two device syncs "
                               f"(value, ms_per_step), each step on its own canvas, mask and step counter staged "
                               f"before timing; per-step HIP events give median/p10/p90; the steps rotate "
                               f"over {ROTATE} copies of the layer weights and KV prefix (one_copy_wall_mean: "
                               f"the same steps on one copy)",
                   "gpu_clock_during_steps": head["gpu_clock"], **gpu},
        "single_layer_step_committed_tokens_per_s": round(head["committed_tokens_per_s"], 2),
        "committed_per_step": head["committed_per_step"],
        "dominant_kernel": dom,
        "roofline": head["kernels"][dom]["roofline"],
        "kernels": kern(head),
    }
    for B in batches[1:]:
        r = res[B]
        out[f"b{B}"] = {"steps_per_s": round(r["steps_per_s"], 3), "ms_per_step": round(r["ms_per_step"], 4),
                        "step_ms": r["step_ms"], "gpu_clock_during_steps": r["gpu_clock"],
                        "single_layer_step_committed_tokens_per_s": round(r["committed_tokens_per_s"], 2),
                        "kernels": kern(r)}
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-e2e", action="store_true", help="skip the full 32-layer model runs")
    ap.add_argument("--batches", default="32,1", help="batch sizes; the first is the headline")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run a plain copy of this many MiB first (scale for counter runs)")
    ap.add_argument("--counters-from", nargs="+", metavar="DIR",
                    help="no GPU: digest rocprofv3 --pmc runs of `bench.py --no-e2e --copy-probe-mib N` (one "
                         "directory per counter group) into profiles/kernel_counters.json")
    ap.add_argument("--counters-command", default="", help="the counter commands, recorded with --counters-from")
    a = ap.parse_args(argv)
    if a.counters_from:
        rec = counters_from(a.counters_from, a.copy_probe_mib or 1024, a.counters_command)
        with open(COUNTERS_FILE, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec)[:2000])
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
    models = layer_copies(model, ROTATE)
    batches = [int(x) for x in a.batches.split(",")]
    res = {}
    for B in batches:
        print(f"[bench] batch {B}", file=sys.stderr, flush=True)
        res[B] = run_batch(models, shape, B, a.steps, a.warmup)
    out = assemble(res, batches, a.steps, a.warmup, gpu_info())
    inputs = {B: res[B]["inputs"] for B in batches}
    del model, models, res
    torch.cuda.empty_cache()
    if not a.no_e2e:
        out["e2e"] = run_e2e()
        out["model_committed_tokens_per_s"] = {
            "b1": out["e2e"]["block_diffusion_b1"]["committed_tokens_per_s"],
            "b32": out["e2e"]["block_diffusion_b32"]["committed_tokens_per_s"],
            "note": "full 32-layer 8B-class model, decode after prefill (e2e.block_diffusion_*)"}
    if not a.no_cpu:
        print(f"[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, shape, inputs)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
