"""Seeded random block shapes against the oracle.

The other GPU cases pin chosen shapes (the benchmark's, tile edges, head
layouts); this sweep draws the rest of the space the library accepts from a
fixed seed, so that combinations nobody picked by hand run too: heads per KV
group from 1 to 16, d_head 64 and 128, widths and FFN widths that are not
multiples of any tile, batch sizes that give 1, 2 or 4 token tiles at decode,
prefills from position 0 and chunked prefills that read a cached prefix,
both RoPE pair layouts and the Llama 3.1 frequency scaling, and fp32 blocks.
Every output row and every cache row a call writes is held to the same bar
as the other parity tests ("Full Llama 3 transformer block", How it works:
the block is x -> x + Attn(RMSNorm(x)) -> h + FFN(RMSNorm(h)); "The Evolving
Transformer 04 LLaMA", 05 GQA for the grouping).
"""
import random

import pytest

import workloads
from block_harness import check_block, log

pytestmark = pytest.mark.gpu

N_CASES = 24


def _draw(i: int) -> workloads.BlockWorkload:
    rng = random.Random(20261203 + 7919 * i)
    if rng.random() < 0.15:
        # fp32 blocks: d_head a multiple of 8, d % 8, d_ff % 4
        dh = rng.choice([8, 16, 24, 32, 40, 64])
        n_kv = rng.choice([1, 2, 3])
        n_rep = rng.choice([1, 2, 3, 4])
        H = n_kv * n_rep
        d = H * dh
        d_ff = 4 * rng.randint(8, 160)
        dtype = "f32"
    else:
        dh = rng.choice([64, 128])
        n_rep = rng.choice([1, 2, 3, 4, 5, 6, 8, 16])
        n_kv = rng.choice([1, 2, 3, 4]) if n_rep <= 4 else rng.choice([1, 2])
        H = n_kv * n_rep
        while H * dh > 2048:
            n_kv = max(1, n_kv // 2) if n_kv > 1 else n_kv
            if n_kv * n_rep * dh > 2048:
                n_rep = max(1, n_rep // 2)
            H = n_kv * n_rep
        d = H * dh
        d_ff = 64 * rng.randint(1, 48)
        dtype = "bf16"
    kind = rng.choice(["decode", "decode", "prefill0", "chunked"])
    if kind == "decode":
        B = rng.choice([1, 3, 16, 17, 32, 40, 64])
        S = 1
        start = rng.randint(0, 300)
    elif kind == "prefill0":
        B = rng.randint(1, 4)
        S = rng.randint(2, 300)
        start = 0
    else:
        B = rng.randint(1, 3)
        S = rng.randint(2, 160)
        start = rng.randint(1, 200)
    rope_half = rng.random() < 0.3
    scaling = (8.0, 1.0, 4.0, float(rng.choice([64, 256]))) if rng.random() < 0.2 else None
    return workloads.BlockWorkload(
        f"shape{i}", dtype, B=B, S=S, start_pos=start, d=d, H=H, n_kv=n_kv, d_head=dh, d_ff=d_ff,
        theta=rng.choice([1e4, 5e5]), eps=1e-5, w_std=0.02, g_mean=1.0, g_std=0.05,
        max_seq=start + S + rng.randint(0, 16), seed=100 + i, rope_half=rope_half, rope_scaling=scaling)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    w = _draw(i)
    log(f"    shape {i}: rope_half={w.rope_half} scaling={w.rope_scaling} capacity={w.capacity}")
    run, *_ = check_block(w)
    run.close()
