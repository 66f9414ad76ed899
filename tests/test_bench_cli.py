"""bench.py's command line on the host: a run on more than one GPU is refused
before anything touches a GPU (libdlm has no multi-GPU path)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
    assert not r.stdout.strip().startswith("{")     # no bench line


def _fake_batch(B):
    """The structure run_batch returns, with made-up times (no GPU)."""
    import bench
    from masked_block_diffusion_denoise_amd import roofline as RL
    kernels = {}
    for n, ms in (("lm_head", 0.54), ("attention", 0.1), ("gate_up", 0.26), ("down", 0.13), ("qkv", 0.08),
                  ("o_proj", 0.05), ("final_norm", 0.01)):
        rec = {"ms": ms, "ms_median": ms}
        if n != "final_norm":
            by, fl = RL.kernel_work(n, B, 32, 4096, 16 * B, 4096, 32, 8, 128, 14336, 131072)
            rec.update(bytes=by, flops=fl, roofline=RL.roofline(by, fl, ms, None))
        kernels[n] = rec
    kernels["down_with_final_norm"] = {"ms": 0.14, "bytes": 1, "flops": 1, "roofline": RL.roofline(1, 1, 0.14)}
    return {"batch": B, "ms_per_step": 1.25, "steps_per_s": 800.0,
            "step_ms": {"wall_mean": 1.25, "median": 1.24, "p10": 1.2, "p90": 1.3, "one_copy_wall_mean": 1.2},
            "gpu_clock": {"samples": 3, "min_mhz": 2000, "median_mhz": 2100, "max_mhz": 2400},
            "committed_per_step": B, "committed_tokens_per_s": B * 800.0, "masked_rows": 16 * B,
            "kernels": kernels, "flags": [0, 0]}


def test_bench_line_has_the_contract_fields():
    import json
    import bench
    out = bench.assemble({32: _fake_batch(32), 1: _fake_batch(1)}, [32, 1], 20, 5, {"rocm": "x"})
    line = json.loads(json.dumps(out))
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert k in line, k
    assert line["n_gpus"] == 1 and line["steps"] == 20 and line["warmup"] == 5
    assert line["config"]["workload"] and line["config"]["global_batch"] == 32
    r = line["roofline"]
    assert r["bound"] in ("hbm", "mfma") and 0 < r["frac"] < 1 and r["peak"] in (8000.0, 2500.0)
    assert line["dominant_kernel"] == "lm_head"
    assert "committed_tokens_per_s" not in line          # single-layer tokens/s is labelled as such
    assert line["single_layer_step_committed_tokens_per_s"] == 32 * 800.0
    assert set(line["step_ms"]) >= {"median", "p10", "p90", "one_copy_wall_mean"}
    assert "b1" in line and "down_with_final_norm" in line["b1"]["kernels"]
