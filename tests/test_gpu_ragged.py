"""GPU parity for ragged batches (llama_block_forward_ragged): every sequence
at its own start position.  "Full Llama 3 transformer block", How it works:
the cache offset and the causal rule belong to each sequence, so the oracle
runs each sequence as its own one-sequence forward at its own position, with
its own cache history, and the GPU batch must agree with every one of them.

The GPU cache is pre-filled with the workload's drawn history up to the largest
position; sequence b reads positions [0, p_b) of it, writes [p_b, p_b + S),
and must leave every other row exactly as it was.
"""
import numpy as np
import pytest
import torch

import workloads
from block_harness import BlockOnGpu, gpu_cache_rows, log, oracle_rows, rel_err, tol_of

pytestmark = pytest.mark.gpu


def _sequence_oracle(w, t, b, p):
    """One-sequence oracle forward of sequence b at start position p."""
    wb = workloads.with_overrides(w, B=1, start_pos=p, max_seq=0)
    tb = dict(t)
    tb["x"] = t["x"][b:b + 1]
    if p > 0:
        tb["k_prefix"] = t["k_prefix"][b:b + 1, :, :p]
        tb["v_prefix"] = t["v_prefix"][b:b + 1, :, :p]
    y, kc, vc, _ = oracle_rows(wb, tb)
    return y.reshape(w.S, w.d), kc[0], vc[0]


def _check_ragged(w, positions, operands="auto"):
    """w.start_pos must be max(positions): the drawn history covers every sequence."""
    assert w.start_pos == max(positions) and len(positions) == w.B
    log(f"[case] ragged {w.name} B={w.B} S={w.S} positions={list(positions)} d={w.d} H={w.H} "
        f"n_kv={w.n_kv} dh={w.d_head} dtype={w.dtype} operands={operands}")
    t = workloads.generate(w)
    run = BlockOnGpu(w, t, operands=operands)
    k0 = run.kv[0].clone()
    v0 = run.kv[1].clone()
    y = run.forward(start_pos=list(positions)).double().cpu().numpy().reshape(w.B, w.S, w.d)
    tol = tol_of(w)
    for b, p in enumerate(positions):
        y_orc, kc, vc = _sequence_oracle(w, t, b, p)
        err = rel_err(y[b], y_orc)
        kk, vv = gpu_cache_rows(w, run.kv, b, p, p + w.S)
        ek = rel_err(kk, kc[:, p:p + w.S, :])
        ev = rel_err(vv, vc[:, p:p + w.S, :])
        log(f"    seq {b} @ {p}: y {err:.3e}  k {ek:.3e}  v {ev:.3e} (tol {tol:g})")
        assert err <= tol and ek <= tol and ev <= tol, (b, p, err, ek, ev)
        # rows outside [p, p + S) of this sequence are untouched
        for cache, before in ((run.kv[0], k0), (run.kv[1], v0)):
            assert torch.equal(cache[b, :, :p], before[b, :, :p]), ("rows below", b, p)
            assert torch.equal(cache[b, :, p + w.S:], before[b, :, p + w.S:]), ("rows above", b, p)
    # sequences past the batch are untouched
    if run.kv[0].shape[0] > w.B:
        assert torch.equal(run.kv[0][w.B:], k0[w.B:]) and torch.equal(run.kv[1][w.B:], v0[w.B:])
    run.close()


def test_ragged_decode_llama3_width():
    """Decode at the 8B width, 32 sequences at positions from 0 (the new token
    is the only key) to 300: 256 (sequence, KV group) pairs, so one attention
    block per pair covers the longest sequence and shorter ones leave some of
    its wavefronts without keys."""
    pos = [0, 1, 300] + [(97 * b) % 300 for b in range(3, 32)]
    w = workloads.with_overrides(workloads.get("llama3_8b_decode"), B=len(pos), start_pos=max(pos),
                                 max_seq=304, seed=11)
    _check_ragged(w, pos)


def test_ragged_decode_split_attention():
    """Decode with 40 sequences of a narrow block (four 16-row token tiles in
    the decode GEMMs; the keys of a group split over several attention blocks,
    some of which hold no key of the shorter sequences)."""
    pos = [(37 * b) % 700 for b in range(40)]
    pos[5] = 700
    w = workloads.BlockWorkload("ragged_decode", "bf16", B=40, S=1, start_pos=700, d=512, H=8,
                                n_kv=2, d_head=64, d_ff=1024, theta=5e5, eps=1e-5, w_std=0.02,
                                g_mean=1.0, g_std=0.05, max_seq=704, seed=40)
    _check_ragged(w, pos)


def test_ragged_decode_maximum_batch():
    """64 sequences, the most a ragged call takes, each at its own position
    from 0 to 250 (four 16-row token tiles in the decode GEMMs)."""
    pos = [(53 * b) % 251 for b in range(64)]
    w = workloads.BlockWorkload("ragged_max", "bf16", B=64, S=1, start_pos=max(pos), d=512, H=8,
                                n_kv=2, d_head=64, d_ff=1024, theta=5e5, eps=1e-5, w_std=0.02,
                                g_mean=1.0, g_std=0.05, max_seq=256, seed=64)
    _check_ragged(w, pos)


def test_ragged_prefill_chunks_dh64():
    """Prefill chunks of 24 tokens at three offsets, SmolLM2 width (d_head 64,
    three heads per KV group)."""
    pos = [0, 7, 50]
    w = workloads.with_overrides(workloads.get("smollm2_135m_prefill"), B=3, S=24,
                                 start_pos=max(pos), max_seq=80, seed=5)
    _check_ragged(w, pos)


def test_ragged_prefill_chunks_dh128():
    """Prefill chunks of 40 tokens at three offsets, d_head 128 with four heads
    per KV group: attention reads the bf16 cache (earlier positions plus the
    rows this call wrote) with fp16 queries."""
    pos = [0, 9, 70]
    w = workloads.BlockWorkload("ragged_dh128", "bf16", B=3, S=40, start_pos=max(pos), d=512, H=4,
                                n_kv=1, d_head=128, d_ff=1408, theta=5e5, eps=1e-5, w_std=0.02,
                                g_mean=1.0, g_std=0.05, max_seq=112, seed=9)
    _check_ragged(w, pos)


def test_ragged_fp32_block():
    """fp32 block (1e-4 bar), prefill chunks of 4 tokens at three offsets."""
    pos = [0, 3, 9]
    w = workloads.with_overrides(workloads.get("tiny_f32"), B=3, S=4, start_pos=max(pos),
                                 max_seq=16, seed=3)
    _check_ragged(w, pos)


@pytest.mark.parametrize("i", range(8))
def test_ragged_random_shapes(i):
    """Seeded random ragged calls: heads per group 1 to 8, d_head 64 and 128,
    1 to 40 sequences, one token (decode) or chunks of up to 48, each
    sequence at its own position (0 included) and both RoPE layouts."""
    import random
    rng = random.Random(8675309 + 104729 * i)
    dh = rng.choice([64, 128])
    n_kv = rng.choice([1, 2])
    n_rep = rng.choice([1, 2, 3, 4, 8])
    H = n_kv * n_rep
    S = 1 if rng.random() < 0.5 else rng.randint(2, 48)
    B = rng.randint(2, 40) if S == 1 else rng.randint(2, 5)
    pos = [rng.randint(0, 260) for _ in range(B)]
    pos[rng.randrange(B)] = 0
    w = workloads.BlockWorkload(f"ragged_rand{i}", "bf16", B=B, S=S, start_pos=max(pos), d=H * dh, H=H,
                                n_kv=n_kv, d_head=dh, d_ff=64 * rng.randint(2, 32), theta=5e5, eps=1e-5,
                                w_std=0.02, g_mean=1.0, g_std=0.05, max_seq=max(pos) + S + rng.randint(0, 9),
                                seed=500 + i, rope_half=rng.random() < 0.4)
    _check_ragged(w, pos)


@pytest.mark.parametrize("S", [1, 24])
def test_ragged_with_equal_positions_is_the_uniform_forward(S):
    """Every sequence at one position: the ragged call computes bitwise what
    the uniform call computes (output and cache)."""
    w = workloads.BlockWorkload("ragged_equal", "bf16", B=4, S=S, start_pos=33, d=512, H=8,
                                n_kv=2, d_head=64, d_ff=1024, theta=5e5, eps=1e-5, w_std=0.02,
                                g_mean=1.0, g_std=0.05, max_seq=64, seed=21)
    t = workloads.generate(w)
    a = BlockOnGpu(w, t)
    b = BlockOnGpu(w, t)
    ya = a.forward(start_pos=w.start_pos).clone()
    yb = b.forward(start_pos=[w.start_pos] * w.B).clone()
    assert torch.equal(ya, yb)
    assert torch.equal(a.kv[0], b.kv[0]) and torch.equal(a.kv[1], b.kv[1])
    a.close()
    b.close()


def test_ragged_rejects_bad_positions_without_writing():
    import decoder_only_transformer_amd as lbmod
    w = workloads.BlockWorkload("ragged_bad", "bf16", B=3, S=2, start_pos=8, d=512, H=8, n_kv=2,
                                d_head=64, d_ff=1024, theta=5e5, eps=1e-5, w_std=0.02, g_mean=1.0,
                                g_std=0.05, max_seq=16, seed=1)
    t = workloads.generate(w)
    run = BlockOnGpu(w, t)
    sentinel = torch.full_like(run.x, 7.0)
    run.out.copy_(sentinel)
    k0, v0 = run.kv[0].clone(), run.kv[1].clone()
    bad = {"negative": [0, -1, 3], "past the cache": [0, 15, 3], "wrong count": [0, 1]}
    # 65 sequences, one over the ragged maximum, on a block and cache that
    # would take them
    w65 = workloads.with_overrides(w, B=65, S=1, start_pos=0, max_seq=16)
    run65 = BlockOnGpu(w65, workloads.generate(w65))
    o65 = torch.full_like(run65.x, 7.0)
    with pytest.raises(lbmod.LlamaBlockError) as e:
        run65.block.forward(run65.x, [0] * 65, run65.kv, o65)
    log(f"    65 sequences: {e.value}")
    assert "at most 64" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(o65 == 7.0)
    run65.close()
    for name, pos in bad.items():
        with pytest.raises((lbmod.LlamaBlockError, ValueError)) as e:
            run.block.forward(run.x, pos, run.kv, run.out)
        log(f"    {name}: {e.value}")
    torch.cuda.synchronize()
    assert torch.equal(run.out, sentinel)
    assert torch.equal(run.kv[0], k0) and torch.equal(run.kv[1], v0)
    run.close()
