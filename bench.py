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
    """Hash of the GEMM sources without comments and whitespace: the traffic
    record stays valid across comment-only edits, not across code changes."""
    h = hashlib.sha256()
    for f in ("k_gemm.hip", "dlm_device.h", "dlm_internal.h"):
        text = open(os.path.join(ROOT, "masked_block_diffusion_denoise_amd", "csrc", f)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("".join(text.split()).encode())
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
# EPI_HEAD = 3).  At batch 32 one head is two launches, 256-row and up-to-320-row
# tiles, of which only one does the work (the other reads the row count and
# exits); a head's bytes are the sum of the two.  Batch 1: 256 x 32 (up to 32 rows) or
# 256 x 64 tiles.
HEAD_KERNELS = {"lm_head_b32": [re.compile(r"k_gemm_tiled<3, 256, 256,"), re.compile(r"k_gemm_tiled<3, 256, 320,")],
                "lm_head_b1": [re.compile(r"k_gemm_tiled<3, 256, (32|64),")]}
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
        for key, pats in HEAD_KERNELS.items():
            kib = 0.0
            for pat in pats:
                launches = [x for k, v in vals.items() if pat.search(k) for x in v]
                if launches:
                    kib += sum(launches) / len(launches)
            if kib == 0.0:
                continue
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
    del model, res
    torch.cuda.empty_cache()
    if not a.no_e2e:
        out["e2e"] = run_e2e()
    if not a.no_cpu:
        print(f"[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        canvas, masked = head["inputs"]
        out["cpu_baseline"] = cpu_baseline(w, shape, B0, canvas, masked)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
