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


def test_counter_digest_labels_each_kernel_of_a_step(tmp_path):
    """The counter digest on a made-up rocprofv3 counter csv: dispatches are
    labelled by their place in the step, the batch comes from the final norm's
    grid, and FETCH_SIZE is scaled by what it read for the 1 GiB copy."""
    import csv
    import bench
    b32 = ["void dlm::k_embed_norm<512>(int const*)", "void dlm::k_gemm_tiled<0, 192, 128, 2, 2, 2, 64, false>(x)",
           "void dlm::k_rope_kv<false>(x)", "void dlm::k_attn<128, 4, true>(x)",
           "void dlm::k_gemm_tiled<1, 128, 128, 2, 2, 2, 64, false>(x)", "dlm::k_rmsnorm(float const*)",
           "void dlm::k_gemm_tiled<2, 256, 256, 4, 2, 2, 64, false>(x)",
           "void dlm::k_gemm_tiled<4, 256, 256, 4, 2, 2, 64, false>(x)", "dlm::k_masked_norm(x)",
           "dlm::k_gemm_head_rows(dlm::GemmArgs)", "dlm::k_head_merge(x)", "dlm::k_commit(x)"]
    b1 = ["void dlm::k_embed_norm<512>(int const*)", "void dlm::k_gemm_tiled<4, 128, 64, 4, 1, 3, 64, false>(x)",
          "void dlm::k_rope_kv<true>(x)", "void dlm::k_attn<128, 4, false>(x)", "void dlm::k_attn_merge<128>(x)",
          "void dlm::k_gemm_tiled<4, 128, 64, 4, 1, 3, 64, false>(x)", "void dlm::k_resid_norm<512>(x)",
          "void dlm::k_gemm_tiled<4, 256, 64, 4, 1, 2, 64, false>(x)", "void dlm::k_splitk_reduce<2>(x)",
          "void dlm::k_gemm_tiled<4, 128, 64, 4, 1, 3, 64, false>(x)", "dlm::k_masked_norm(x)",
          "void dlm::k_gemm_tiled<3, 256, 32, 4, 1, 2, 64, false>(x)", "dlm::k_head_merge(x)", "dlm::k_commit(x)"]
    rows, did = [], 0

    def add(name, grid, kib):
        nonlocal did
        did += 1
        rows.append({"Dispatch_Id": did, "Kernel_Name": name, "Grid_Size": grid, "Counter_Name": "FETCH_SIZE",
                     "Counter_Value": kib})
    add("__amd_rocclr_copyBuffer", 4096, 524288.0)
    for _ in range(2):
        for i, n in enumerate(b32):
            add(n, 1024 * 256 if "masked_norm" in n else 256, 100.0 + i)
    for i, n in enumerate(b1):
        add(n, 32 * 256 if "masked_norm" in n else 256, 10.0 + i)
    d = tmp_path / "pmc_fetch" / "x"
    d.mkdir(parents=True)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)
    rec = bench.counters_from([str(tmp_path / "pmc_fetch")], 1024, "cmd")
    k = rec["kernels"]
    assert rec["scale"]["FETCH_SIZE"] == 2.0
    assert k["qkv_b32"]["FETCH_SIZE"] == 101.0 and k["qkv_b32"]["dispatches"] == 2
    assert k["lm_head_b32"]["FETCH_SIZE"] == 109.0 and k["down_b32"]["FETCH_SIZE"] == 107.0
    assert k["o_norm_b32"]["FETCH_SIZE"] == 105.0 and k["gate_up_b32"]["FETCH_SIZE"] == 106.0
    assert k["attention_merge_b1"]["FETCH_SIZE"] == 14.0 and k["o_norm_b1"]["FETCH_SIZE"] == 16.0
    assert k["gate_up_reduce_b1"]["FETCH_SIZE"] == 18.0 and k["down_b1"]["FETCH_SIZE"] == 19.0
    assert k["lm_head_b1"]["hbm_bytes"] == round(21.0 * 1024 * 2.0)
