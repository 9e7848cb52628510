"""The decode step that allocates nothing (llama_block_forward_decode_static):
its scratch lives in the library's static per-GPU array instead of the
handle's workspace.  Checked through the C ABI against llama_block_forward on
the same inputs (bitwise: the same kernels run in the same order), on two
calls in a row, the second with a smaller batch at the next position, and
against the oracle at the bf16 block bar.  Also: the shapes it refuses."""
import numpy as np
import pytest
import torch

import decoder_only_transformer_amd as lbmod
import workloads
from block_harness import BlockOnGpu, config_for, gpu_cache, log, oracle_rows, rel_err

pytestmark = pytest.mark.gpu


def _twin_cache(w, t):
    k, v = gpu_cache(w, t)
    return (k, v), (k.clone(), v.clone())


def test_static_decode_equals_forward_twice():
    w = workloads.with_overrides(workloads.get("llama3_8b_decode"), B=32, start_pos=100, max_seq=128,
                                 seed=81)
    log(f"[case] static-scratch decode {w.name} B={w.B} then B=5, start_pos {w.start_pos}")
    t = workloads.generate(w)
    run = BlockOnGpu(w, t)
    kv_a, kv_b = _twin_cache(w, t)
    # call 1: the workload's 32 sequences
    y_a = torch.empty_like(run.x)
    y_b = torch.full_like(run.x, float("nan"))
    run.block.forward(run.x, w.start_pos, kv_a, y_a)
    lbmod.llama_block_forward_decode_static(run.block.handle, run.x, w.start_pos, kv_b, y_b)
    torch.cuda.synchronize()
    assert torch.equal(y_a, y_b)
    assert torch.equal(kv_a[0], kv_b[0]) and torch.equal(kv_a[1], kv_b[1])
    y_orc, *_ = oracle_rows(w, t)
    e = rel_err(y_b.double().cpu().numpy().reshape(w.M, w.d), y_orc.reshape(w.M, w.d))
    log(f"    call 1: bitwise equal to llama_block_forward; max|err|/rms vs oracle {e:.3e}")
    assert e <= 2e-2
    # call 2: five sequences, one position later, new inputs
    g = torch.Generator(device="cpu").manual_seed(82)
    x2 = torch.randn(5, 1, w.d, generator=g).to(torch.bfloat16).to("cuda")
    sub_a = (kv_a[0][:5], kv_a[1][:5])
    sub_b = (kv_b[0][:5], kv_b[1][:5])
    y2_a = torch.empty_like(x2)
    y2_b = torch.full_like(x2, float("nan"))
    run.block.forward(x2, w.start_pos + 1, sub_a, y2_a)
    lbmod.llama_block_forward_decode_static(run.block.handle, x2, w.start_pos + 1, sub_b, y2_b)
    torch.cuda.synchronize()
    assert torch.equal(y2_a, y2_b)
    assert torch.equal(kv_a[0], kv_b[0]) and torch.equal(kv_a[1], kv_b[1])
    assert not torch.isnan(y2_b.float()).any()
    log("    call 2 (5 sequences at the next position): bitwise equal")
    run.close()


def test_static_decode_refuses_what_it_cannot_hold():
    # an fp32 block
    w = workloads.with_overrides(workloads.get("tiny_f32"), B=2, S=1, start_pos=3, max_seq=16)
    t = workloads.generate(w)
    run = BlockOnGpu(w, t)
    y = torch.empty_like(run.x)
    with pytest.raises(lbmod.LlamaBlockError) as ei:
        lbmod.llama_block_forward_decode_static(run.block.handle, run.x, w.start_pos, run.kv, y)
    assert ei.value.status == lbmod.LB_ERR_UNSUPPORTED
    run.close()
    # a width whose decode buffers exceed the static array at 64 sequences
    # (d 16384 with 128 heads: 2 MB per activation row set, 21 MB of attention
    # partials) but fit at 32; weights drawn on the device
    d, H, G, dh, dff = 16384, 128, 8, 128, 1024
    big = workloads.BlockWorkload("static_limit", "bf16", B=64, S=1, start_pos=8, d=d, H=H, n_kv=G,
                                  d_head=dh, d_ff=dff, theta=5e5, eps=1e-5, w_std=0.01, max_seq=16)
    gen = torch.Generator(device="cuda").manual_seed(83)
    shapes = {"attn_norm": (d,), "wq": (H * dh, d), "wk": (G * dh, d), "wv": (G * dh, d),
              "wo": (d, H * dh), "ffn_norm": (d,), "w_gate": (dff, d), "w_up": (dff, d),
              "w_down": (d, dff)}
    wts = {n: (torch.randn(s, device="cuda", generator=gen) * (1.0 if "norm" in n else 0.01)
               ).to(torch.bfloat16) for n, s in shapes.items()}
    blk = lbmod.LlamaBlock(config_for(big, max_tokens=64), wts)
    del wts
    k, v = lbmod.new_kv_cache(64, G, 16, dh, torch.bfloat16)
    x = torch.randn(64, 1, d, device="cuda", generator=gen).to(torch.bfloat16)
    y = torch.empty_like(x)
    with pytest.raises(lbmod.LlamaBlockError) as ei:
        lbmod.llama_block_forward_decode_static(blk.handle, x, 8, (k, v), y)
    assert ei.value.status == lbmod.LB_ERR_UNSUPPORTED
    log(f"    refused at 64 sequences: {ei.value}")
    # 32 sequences fit, and equal the workspace forward
    y32 = torch.empty_like(x[:32])
    y32_ref = torch.empty_like(x[:32])
    k2, v2 = k.clone(), v.clone()
    lbmod.llama_block_forward_decode_static(blk.handle, x[:32], 8, (k[:32], v[:32]), y32)
    blk.forward(x[:32], 8, (k2[:32], v2[:32]), y32_ref)
    torch.cuda.synchronize()
    assert torch.equal(y32, y32_ref)
    blk.close()
