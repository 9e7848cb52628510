"""GPU parity over the head layouts the attention kernels specialise on.

Query head h reads key/value head floor(h / n_rep), n_rep = n_heads / n_kv_heads
("The Evolving Transformer 04 LLaMA", 05 GQA).  The prefill kernels pick their
block shape from n_rep and d_head, and a prefill at start_pos > 0 (a chunk after
a cached prefix) reads the bf16 cache instead of the operand-type copies a
prefill from position 0 uses, so each combination below runs a different
kernel instantiation:

  * n_kv = H (plain multi-head attention, n_rep = 1): "From GPT-2 to Llama",
    Keys and values get shared (full heads are the n_rep = 1 case), and the
    Llama 2 7B row of "The Evolving Transformer 04 LLaMA", 08 COMPARISON;
  * eight query heads per KV head at d_head 128 (the 70B head shape of "Full
    Llama 3 transformer block", How it works) in a chunked prefill, with fp16
    and with bf16 matrix operands;
  * six heads per group (an even group that is not a power of two), three
    heads per group at d_head 128 (an odd group).

Every case is held to the block bar on every output row and every written
cache row.  FFN widths are narrow so that the oracle finishes in seconds.
"""
import pytest

import workloads
from block_harness import check_block

pytestmark = pytest.mark.gpu


def _w(name, H, n_kv, dh, B, S, start_pos, seed, d_ff=1024):
    cap = (start_pos + S + 7) // 8 * 8
    return workloads.BlockWorkload(name, "bf16", B=B, S=S, start_pos=start_pos, d=H * dh, H=H,
                                   n_kv=n_kv, d_head=dh, d_ff=d_ff, theta=5e5, eps=1e-5,
                                   w_std=0.02, g_mean=1.0, g_std=0.05, max_seq=cap, seed=seed)


# (B, S, start_pos): a prefill from position 0 with a ragged last query block,
# a chunk after a cached prefix, and a decode step
_CALLS = [(2, 70, 0), (2, 40, 51), (5, 1, 200)]


@pytest.mark.parametrize("dh", [64, 128])
@pytest.mark.parametrize("B,S,start_pos", _CALLS)
def test_mha_one_head_per_kv_head(dh, B, S, start_pos):
    w = _w("mha", 512 // dh, 512 // dh, dh, B, S, start_pos, seed=40 + S + dh)
    run, *_ = check_block(w)
    run.close()


@pytest.mark.parametrize("operands", ["auto", "bf16"])
def test_eight_heads_per_group_dh128_chunked(operands):
    w = _w("group8", 16, 2, 128, 2, 70, 45, seed=48)
    run, *_ = check_block(w, operands=operands)
    run.close()


def test_eight_heads_per_group_dh128_from_zero():
    w = _w("group8", 16, 2, 128, 1, 130, 0, seed=49)
    run, *_ = check_block(w)
    run.close()


@pytest.mark.parametrize("B,S,start_pos", _CALLS)
def test_six_heads_per_group(B, S, start_pos):
    w = _w("group6", 12, 2, 128, B, S, start_pos, seed=60 + S)
    run, *_ = check_block(w)
    run.close()


@pytest.mark.parametrize("B,S,start_pos", _CALLS[:2])
def test_three_heads_per_group_dh128(B, S, start_pos):
    w = _w("group3", 6, 2, 128, B, S, start_pos, seed=30 + S)
    run, *_ = check_block(w)
    run.close()
