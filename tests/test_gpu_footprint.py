"""GPU checks of the device memory a handle holds.

llama_block_footprint sizes a block or a stack from its config alone, on the
host; these tests check that a live handle holds exactly that many bytes and
that the device's free memory drops by that much (up to the allocator's
rounding), so that the one packed copy of the weights per block is what the
device really holds ("The Evolving Transformer 04 LLaMA", 07 ASSEMBLE LLAMA:
a model is N such blocks, so per-block weight memory multiplies by N).
"""
import pytest
import torch

import decoder_only_transformer_amd as lbmod
import workloads
from block_harness import config_for, log

pytestmark = pytest.mark.gpu

# the allocator rounds each allocation up (to at most 2 MiB here) and init
# creates one stream; a second copy of any weight matrix is far above this
SLACK = 64 << 20


def _warm():
    """Load the library's code objects (and its static scratch) before any
    free-memory reading, with a tiny block."""
    w = workloads.with_overrides(workloads.get("tiny_f32"), B=1, S=4)
    t = workloads.generate(w)
    blk = lbmod.LlamaBlock(config_for(w), {n: t[n].to("cuda") for n in lbmod.WEIGHT_NAMES})
    blk.close()
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["llama3_8b_prefill", "smollm2_135m_prefill", "tiny_f32"])
def test_block_holds_its_footprint(name):
    _warm()
    w = workloads.with_overrides(workloads.get(name), B=1, S=64)
    t = workloads.generate_stack_on_device(w, 1)["layers"][0]
    cfg = config_for(w, max_tokens=256)
    fp = lbmod.llama_block_footprint(cfg)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    blk = lbmod.LlamaBlock(cfg, {n: t[n] for n in lbmod.WEIGHT_NAMES})
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    held = free0 - free1
    log(f"    {name}: footprint weights {fp['weights']} workspace {fp['workspace']}, "
        f"handle {blk.device_bytes}, free memory dropped by {held}")
    assert blk.device_bytes == fp["weights"] + fp["workspace"]
    assert abs(held - blk.device_bytes) <= SLACK
    blk.close()
    torch.cuda.synchronize()
    free2, _ = torch.cuda.mem_get_info()
    assert abs(free2 - free0) <= SLACK


def test_stack_holds_its_footprint():
    """A 30-block SmolLM2-width stack (the model's depth): n_layers blocks'
    weights plus one shared workspace."""
    _warm()
    w = workloads.with_overrides(workloads.get("smollm2_135m_decode"), B=2, S=1)
    g = workloads.generate_stack_on_device(w, 30)
    cfg = config_for(w, max_tokens=64)
    fp = lbmod.llama_block_footprint(cfg, 30)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    st = lbmod.LlamaStack(cfg, [{n: l[n] for n in lbmod.WEIGHT_NAMES} for l in g["layers"]],
                          g["final_norm"])
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    held = free0 - free1
    log(f"    stack: footprint {fp}, handle {st.device_bytes}, free memory dropped by {held}")
    assert st.device_bytes == fp["weights"] + fp["workspace"]
    assert abs(held - st.device_bytes) <= SLACK
    st.close()
