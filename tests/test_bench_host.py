"""The benchmark's bookkeeping on the CPU: the algorithmic work behind the
roofline figures, tied to counts the pages print, and the one-GPU contract."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402

GOLD = json.load(open(os.path.join(ROOT, "tests", "golden", "page_figures.json")))

GEMM_STAGES = ("qkv_rope_append", "o_proj_residual", "gate_up_swiglu", "down_residual")


def test_gemm_flops_are_two_per_weight_per_token():
    """"Llama 4 From Scratch" / "From GPT-2 to Llama": 218 M weights per 8B
    block; the four products do 2 flops per weight per token."""
    w = workloads.get("llama3_8b_prefill")
    work = bench.stage_work(w)
    flops = sum(work[s]["flops"] for s in GEMM_STAGES)
    assert flops == 2 * w.M * workloads.param_count(w)["total_linear"]
    assert round(workloads.param_count(w)["total_linear"] / 1e6) == GOLD["llama3_8b_block_params_millions"]["value"]


def test_decode_attention_bytes_are_the_cache():
    """The 8B decode attention reads every cached K and V value once: 32
    sequences x 8192 positions x 2048 values per token per layer ("Llama 4
    From Scratch", Worked example) x 2 bytes, plus q in and o out."""
    w = workloads.get("llama3_8b_decode")
    per_token = GOLD["kv_values_per_token_per_layer_llama3_8b"]["value"]
    cache = w.B * (w.start_pos + w.S) * per_token * 2
    att = bench.stage_work(w)["attention"]["bytes"]
    assert att == cache + 2 * w.M * w.H * w.d_head * 2
    assert abs(cache / 1e9 - 1.074) < 1e-3


def test_causal_attention_flops_count_visible_pairs():
    """Prefill from 0: query s sees s + 1 keys, so a sequence of S has
    S(S+1)/2 pairs per head, 4 dh flops each (QK^T and PV)."""
    w = workloads.get("llama3_8b_prefill")
    pairs = w.B * w.S * (w.S + 1) // 2
    assert bench.stage_work(w)["attention"]["flops"] == 4 * w.d_head * pairs * w.H


def test_moe_work_reduces_to_a_wider_dense_ffn():
    """One expert chosen by every token (E = k = 1) does the work of a dense
    FFN of width d_ff + d_ff_expert, plus the router."""
    base = dict(name="m", dtype="bf16", B=2, S=64, start_pos=0, d=512, H=8, n_kv=2, d_head=64, d_ff=1024,
                theta=5e5, eps=1e-5, w_std=0.02)
    moe = workloads.BlockWorkload(**base, n_experts=1, top_k=1, d_ff_expert=768)
    dense = workloads.BlockWorkload(**dict(base, d_ff=1024 + 768))
    wm, wd = bench.stage_work(moe), bench.stage_work(dense)
    assert wm["gate_up_swiglu"]["flops"] == wd["gate_up_swiglu"]["flops"] + 2 * moe.M * 1 * moe.d
    assert wm["down_residual"]["flops"] == wd["down_residual"]["flops"]
    for s in ("rmsnorm_1", "qkv_rope_append", "attention", "o_proj_residual", "rmsnorm_2"):
        assert wm[s] == wd[s]


def test_moe_weight_bytes_count_only_the_experts_used():
    w = workloads.get("llama4_moe_decode")
    all_e = bench.stage_work(w)
    some = bench.stage_work(w, active_experts=12)
    per_expert = 3 * w.d * w.d_ff_expert * 2
    got = (all_e["gate_up_swiglu"]["bytes"] + all_e["down_residual"]["bytes"]) - \
          (some["gate_up_swiglu"]["bytes"] + some["down_residual"]["bytes"])
    assert got == (w.n_experts - 12) * per_expert


def test_roofline_fraction_is_achieved_over_peak():
    w = workloads.get("llama3_8b_decode")
    work = bench.stage_work(w)
    ms = 0.2
    roof, stages = bench.roofline(w, {"attention": ms}, "attention", ms, "hbm")
    assert roof["unit"] == "GB/s" and roof["peak"] == bench.HBM_PEAK_GBS
    assert abs(roof["achieved"] - work["attention"]["bytes"] / (ms * 1e-3) / 1e9) < 0.1
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-4


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_cpu_baseline_times_the_oracle_on_the_workload():
    """The CPU baseline runs the oracle on the workload's own tensors: every row,
    or a stated row sample whose tokens/s counts only those rows."""
    import workloads
    w = workloads.with_overrides(workloads.get("tiny_f32"), B=2, S=8, start_pos=4, max_seq=12)
    t = workloads.generate(w)
    full = bench.cpu_baseline(w, t, repeats=3)
    assert full["kind"] == "oracle" and full["runs"] == 3 and full["cores"] >= 1
    assert full["value"] > 0 and "all 16 token rows" in full["sample"] and full["cpu_model"]
    part = bench.cpu_baseline(w, t, rows=[0, 1, 2])
    assert "first 3 token rows" in part["sample"]
