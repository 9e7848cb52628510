"""GPU checks of the fp16 operand path's range guard and of init's errors.

A bf16 block computes its matrix products on fp16 operands by default: the
weights widen to fp16 at init and the activations that feed products are
rounded to fp16 ("Mini Llama 2 Implementation", RMS normalization: normalise
in fp32, cast back for the next product).  fp16's largest finite value is
65504, far below bf16's, so init bounds every such activation from the
weights and gains (bounds that hold for any input; stated in the header) and
takes bf16 operands (AUTO) or refuses (F16) when a bound does not fit.
"""
import pytest
import torch

import decoder_only_transformer_amd as lbmod
import workloads
from block_harness import (BF16_OPERANDS_BAR, check_block, config_for, device_weights,
                           log)

pytestmark = pytest.mark.gpu


def _smol(**kw):
    return workloads.with_overrides(workloads.get("smollm2_135m_prefill"), B=2, S=96, **kw)


def test_large_gains_inside_the_bounds_keep_fp16():
    """Gains ~8: RMSNorm outputs reach a few hundred and SiLU(gate)*up a few
    thousand, inside fp16: operands stay fp16 and the block meets the bar."""
    w = _smol(g_mean=8.0, g_std=0.5, seed=71)
    run, *_ = check_block(w)
    assert run.block.operand_type == "f16"
    run.close()


def test_gains_beyond_the_fp16_bounds_take_bf16_operands():
    """An RMSNorm_2 gain of ~300 (the attention's gain left at ~1, so that its
    softmax stays well conditioned): SiLU(gate)*up then reaches ~1e5 on these
    inputs, past fp16's 65504 (fp16 operands would turn it into inf).  AUTO
    takes bf16 operands, and the result meets the bf16-operand bound; asking
    for fp16 operands is refused with LB_ERR_UNSUPPORTED, naming the bound."""
    w = _smol(g_mean=1.0, g_std=0.05, seed=72)
    t = workloads.generate(w)
    t["ffn_norm"] = (t["ffn_norm"].float() * 300.0).to(torch.bfloat16)
    run, *_ = check_block(w, tol=BF16_OPERANDS_BAR, tensors=t)
    assert run.block.operand_type == "bf16"
    run.close()
    with pytest.raises(lbmod.LlamaBlockError) as ei:
        lbmod.LlamaBlock(config_for(w, "f16"), device_weights(t))
    assert ei.value.status == lbmod.LB_ERR_UNSUPPORTED
    log(f"    refused: {ei.value}")
    assert "SwiGLU" in str(ei.value)


@pytest.mark.parametrize("what", ["huge", "tiny"])
def test_weights_fp16_cannot_hold(what):
    """A weight above 65504 (inf in fp16), or a matrix whose values mostly sit
    below fp16's normal range (2^-14) so that widening loses their bits: AUTO
    takes bf16 operands, F16 is refused."""
    w = _smol(seed=73)
    t = workloads.generate(w)
    if what == "huge":
        t["wo"][3, 5] = 1.0e5
    else:
        t["w_down"] = (t["w_down"].float() * 1e-5).to(torch.bfloat16)
    blk = lbmod.LlamaBlock(config_for(w, "auto"), device_weights(t))
    assert blk.operand_type == "bf16"
    blk.close()
    with pytest.raises(lbmod.LlamaBlockError) as ei:
        lbmod.LlamaBlock(config_for(w, "f16"), device_weights(t))
    assert ei.value.status == lbmod.LB_ERR_UNSUPPORTED
    log(f"    {what}: refused: {ei.value}")


def test_benchmark_weights_take_fp16():
    """The 8B-width benchmark block (weights N(0, 0.02), gains N(1, 0.05))
    passes the check with a wide margin."""
    w = workloads.with_overrides(workloads.get("llama3_8b_prefill"), B=1, S=16)
    t = workloads.generate(w)
    blk = lbmod.LlamaBlock(config_for(w, "auto"), device_weights(t))
    assert blk.operand_type == "f16"
    blk.close()


def test_out_of_memory_is_reported_and_recoverable():
    """An absurd workspace (2^28 token rows at d 4096: terabytes) fails with
    LB_ERR_OOM, and the device stays usable: a normal block runs after it."""
    w = _smol(seed=74)
    t = workloads.generate(w)
    cfg = config_for(w, "auto", max_tokens=1 << 28)
    with pytest.raises(lbmod.LlamaBlockError) as ei:
        lbmod.LlamaBlock(cfg, device_weights(t))
    assert ei.value.status == lbmod.LB_ERR_OOM
    log(f"    refused: {ei.value}")
    run, *_ = check_block(w)
    run.close()
