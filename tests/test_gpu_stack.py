"""GPU parity for stacks of blocks (llama_stack_*): N blocks, each with its own
weights and cache, then the final RMSNorm ("The Evolving Transformer 04
LLaMA", 07 ASSEMBLE LLAMA).

Each call is checked block by block against the fp64 oracle with the GPU's
own block inputs (the hidden states the stack hands from block to block, in
the block dtype) and the GPU's own cache history, so every block meets the
single-block bar (2e-2 rms for bf16, 1e-4 for fp32) exactly as in the block
tests; the final norm is checked elementwise against RMSNorm of the GPU's last
hidden state.  The whole stack is also compared with the oracle's
free-running fp64 composition: there each block's error reaches the output
through the later blocks, so the bar is the sum of the per-block bars, L times
the block bar (the residual stream carries an earlier error forward at its
size relative to the stream, and the final norm rescales by the stream's rms).
"""
import numpy as np
import pytest
import torch

import decoder_only_transformer_amd as lbmod
import oracle
import workloads
from block_harness import config_for, log, rel_err, tol_of

pytestmark = pytest.mark.gpu


class StackRun:
    def __init__(self, w, n_layers, operands="auto", cap=None, max_tokens=None):
        self.w, self.L = w, n_layers
        self.t = workloads.generate_stack(w, n_layers)
        self.cap = cap or w.capacity
        if w.dtype == "bf16":
            self.cap = (self.cap + 7) // 8 * 8
        cfg = config_for(w, operands, max_tokens=max_tokens or w.M, max_seq_len=self.cap)
        layers = [{n: lt[n].to("cuda") for n in lbmod.WEIGHT_NAMES} for lt in self.t["layers"]]
        self.stack = lbmod.LlamaStack(cfg, layers, self.t["final_norm"].to("cuda"))
        del layers
        self.kv = []
        for lt in self.t["layers"]:
            k, v = lbmod.new_kv_cache(w.B, w.n_kv, self.cap, w.d_head, w.torch_dtype)
            if w.start_pos > 0:
                k[:, :, :w.start_pos] = lt["k_prefix"].to("cuda")
                v[:, :, :w.start_pos] = lt["v_prefix"].to("cuda")
            self.kv.append((k, v))
        self.cfg = oracle.cfg_of(w)
        self.gf = self.t["final_norm"].double().numpy()

    def caches_cpu(self):
        return [(k.double().cpu().numpy(), v.double().cpu().numpy()) for k, v in self.kv]

    def close(self):
        self.stack.close()


def check_call(run, x, positions, out, hidden, before, tol=None):
    """Block-by-block check of one stack call that ran at `positions` (one
    per sequence) with inputs x; `before`: the GPU caches before the call."""
    w, L = run.w, run.L
    S = x.shape[1]
    tol = tol or tol_of(w)
    xs = x.double().cpu().numpy()
    hid = hidden.double().cpu().numpy()
    after = run.caches_cpu()
    worst = 0.0
    for b, p in enumerate(positions):
        inp = xs[b:b + 1]
        for l in range(L):
            kc = np.zeros((1, w.n_kv, run.cap, w.d_head))
            vc = np.zeros_like(kc)
            kc[:, :, :p] = before[l][0][b:b + 1, :, :p]
            vc[:, :, :p] = before[l][1][b:b + 1, :, :p]
            y, _ = oracle.block_forward(run.cfg, inp, run.t["layers"][l], p, kc, vc)
            e = rel_err(hid[l, b:b + 1], y)
            ek = rel_err(after[l][0][b, :, p:p + S], kc[0, :, p:p + S])
            ev = rel_err(after[l][1][b, :, p:p + S], vc[0, :, p:p + S])
            worst = max(worst, e, ek, ev)
            assert e <= tol and ek <= tol and ev <= tol, ("block", l, "seq", b, "pos", p, e, ek, ev)
            # rows of the cache outside [p, p + S) are untouched
            for c in (0, 1):
                assert np.array_equal(after[l][c][b, :, :p], before[l][c][b, :, :p]), ("below", l, b)
                assert np.array_equal(after[l][c][b, :, p + S:], before[l][c][b, :, p + S:]), ("above", l, b)
            inp = hid[l, b:b + 1]
    # final norm of the GPU's last hidden state: bf16 rounding of the result
    # (2^-9 relative) and fp32 arithmetic, elementwise
    last = hid[L - 1]
    want = last / np.sqrt(np.mean(last * last, axis=-1, keepdims=True) + w.eps) * run.gf
    got = out.double().cpu().numpy()
    rel = 2.0 ** -8 if w.dtype == "bf16" else 1e-5
    bad = np.abs(got - want) > rel * np.abs(want) + 1e-6 * np.sqrt(np.mean(want * want))
    assert not bad.any(), ("final norm", int(bad.sum()))
    return worst


def free_running(run, steps):
    """The oracle's own fp64 composition over a sequence of uniform calls
    [(x, start_pos)], each block with its own fp64 cache (pre-filled rows
    from the workload).  Returns the output of every call."""
    w = run.w
    caches = []
    for lt in run.t["layers"]:
        kc, vc = oracle.empty_cache(w, run.cap)
        if w.start_pos > 0:
            kc[:, :, :w.start_pos] = lt["k_prefix"].double().numpy()
            vc[:, :, :w.start_pos] = lt["v_prefix"].double().numpy()
        caches.append((kc, vc))
    outs = []
    for x, p in steps:
        y, _ = oracle.stack_forward(run.cfg, x, run.t["layers"], run.t["final_norm"], p, caches)
        outs.append(y)
    return outs


def _prefill_then_decode(w, L, n_decode, operands="auto"):
    log(f"[case] stack {w.name} L={L} B={w.B} S={w.S} start={w.start_pos} d={w.d} H={w.H} n_kv={w.n_kv} "
        f"dh={w.d_head} dtype={w.dtype} then {n_decode} decode steps")
    cap = w.start_pos + w.S + n_decode
    run = StackRun(w, L, operands, cap=cap)
    gen = torch.Generator().manual_seed(w.seed + 99)
    calls = [(run.t["x"], w.start_pos)]
    for i in range(n_decode):
        xd = (torch.randn((w.B, 1, w.d), generator=gen) * w.x_std).to(w.torch_dtype)
        calls.append((xd, w.start_pos + w.S + i))
    outs = []
    for x_cpu, p in calls:
        x = x_cpu.to("cuda")
        out = torch.empty_like(x)
        hidden = torch.empty((L,) + tuple(x.shape), dtype=x.dtype, device="cuda")
        before = run.caches_cpu()
        run.stack.forward(x, p, run.kv, out, hidden)
        torch.cuda.synchronize()
        worst = check_call(run, x, [p] * w.B, out, hidden, before)
        log(f"    call S={x.shape[1]} at {p}: worst block error {worst:.3e} (tol {tol_of(w):g})")
        outs.append(out.double().cpu().numpy())
    ref = free_running(run, [(x.double().numpy(), p) for x, p in calls])
    bar = L * tol_of(w)
    for (x_cpu, p), got, want in zip(calls, outs, ref):
        e = rel_err(got, want)
        log(f"    free-running fp64 stack, call at {p}: {e:.3e} (bar L * block bar = {bar:g})")
        assert e <= bar, (p, e)
    run.close()


def test_stack_smollm2_width_prefill_then_decode():
    """Four blocks of the SmolLM2 width (d_head 64, three heads per KV group):
    a 40-token prefill from 0, then three decode steps."""
    w = workloads.with_overrides(workloads.get("smollm2_135m_prefill"), B=2, S=40, g_std=0.05, seed=31)
    _prefill_then_decode(w, 4, 3)


def test_stack_dh128_prefill_at_offset_then_decode():
    """Three blocks with d_head 128 and four heads per KV group, a 24-token
    chunk at position 17 over pre-filled history, then two decode steps."""
    w = workloads.BlockWorkload("stack_dh128", "bf16", B=3, S=24, start_pos=17, d=512, H=4, n_kv=1,
                                d_head=128, d_ff=1408, theta=5e5, eps=1e-5, w_std=0.02, g_mean=1.0,
                                g_std=0.05, seed=17)
    _prefill_then_decode(w, 3, 2)


def test_stack_fp32():
    """fp32 stack (1e-4 block bar): three tiny blocks, prefill then decode."""
    w = workloads.with_overrides(workloads.get("tiny_f32"), B=2, S=8, seed=4)
    _prefill_then_decode(w, 3, 2)


def test_stack_llama3_width_decode():
    """Two blocks at the 8B width, 4 sequences decoding at position 200 over
    drawn history (the decode GEMMs and split-KV attention of that width)."""
    w = workloads.with_overrides(workloads.get("llama3_8b_decode"), B=4, start_pos=200, max_seq=208, seed=8)
    _prefill_then_decode(w, 2, 1)


def test_stack_ragged_decode():
    """Ragged decode through a stack: 6 sequences at their own positions."""
    w = workloads.BlockWorkload("stack_ragged", "bf16", B=6, S=1, start_pos=90, d=512, H=8, n_kv=2,
                                d_head=64, d_ff=1024, theta=5e5, eps=1e-5, w_std=0.02, g_mean=1.0,
                                g_std=0.05, max_seq=96, seed=23)
    pos = [0, 90, 45, 7, 63, 1]
    log(f"[case] stack ragged decode L=3 positions={pos}")
    run = StackRun(w, 3)
    x = run.t["x"].to("cuda")
    out = torch.empty_like(x)
    hidden = torch.empty((3,) + tuple(x.shape), dtype=x.dtype, device="cuda")
    before = run.caches_cpu()
    run.stack.forward(x, pos, run.kv, out, hidden)
    torch.cuda.synchronize()
    log(f"    worst block error {check_call(run, x, pos, out, hidden, before):.3e}")
    run.close()


def _device_pos_case(w, L, pos, advance=True):
    run = StackRun(w, L)
    x = run.t["x"].to("cuda")
    out = torch.empty_like(x)
    hidden = torch.empty((L,) + tuple(x.shape), dtype=x.dtype, device="cuda")
    positions = torch.tensor(pos, dtype=torch.int32, device="cuda")
    before = run.caches_cpu()
    run.stack.forward_device_pos(x, positions, run.kv, out, advance=advance, hidden=hidden)
    torch.cuda.synchronize()
    return run, x, out, hidden, positions, before


def test_stack_device_positions_prefill_and_decode():
    """Start positions read from device memory (the capturable call): the
    blocks meet the bar at those positions and the positions move on by S."""
    for S, pos in ((12, [0, 20, 7]), (1, [50, 3, 31])):
        w = workloads.BlockWorkload("stack_devpos", "bf16", B=3, S=S, start_pos=50, d=576, H=9, n_kv=3,
                                    d_head=64, d_ff=1536, theta=1e5, eps=1e-5, w_std=0.02, g_mean=1.0,
                                    g_std=0.05, max_seq=64, seed=5 + S)
        log(f"[case] stack device positions S={S} positions={pos}")
        run, x, out, hidden, positions, before = _device_pos_case(w, 2, pos)
        log(f"    worst block error {check_call(run, x, pos, out, hidden, before):.3e}")
        assert positions.cpu().tolist() == [p + S for p in pos]
        run.close()


def test_stack_device_positions_are_clamped_into_the_cache():
    """Device positions outside [0, capacity - S] are read as the nearest end:
    the call computes what it computes at the clamped positions, and writes
    only inside the cache."""
    w = workloads.BlockWorkload("stack_clamp", "bf16", B=3, S=1, start_pos=63, d=512, H=8, n_kv=2,
                                d_head=64, d_ff=1024, theta=5e5, eps=1e-5, w_std=0.02, g_mean=1.0,
                                g_std=0.05, max_seq=64, seed=2)
    raw = [-7, 10 ** 6, 20]
    log(f"[case] stack clamped device positions {raw} (capacity 64)")
    run, x, out, hidden, positions, before = _device_pos_case(w, 2, raw, advance=False)
    log(f"    worst block error {check_call(run, x, [0, 63, 20], out, hidden, before):.3e}")
    assert positions.cpu().tolist() == raw
    run.close()


def test_stack_graph_replays_match_eager_device_pos():
    """A captured decode step replayed five times, with eager work and
    synchronisations between the replays: every replay's output, caches and
    positions equal bitwise those of the same eager call on a twin set of
    caches (the eager call is checked against the oracle above)."""
    w = workloads.BlockWorkload("stack_graph", "bf16", B=4, S=1, start_pos=30, d=576, H=9, n_kv=3,
                                d_head=64, d_ff=1536, theta=1e5, eps=1e-5, w_std=0.02, g_mean=1.0,
                                g_std=0.05, max_seq=40, seed=12)
    L = 3
    log(f"[case] stack graph L={L} B={w.B} decode from {w.start_pos}")
    run = StackRun(w, L)
    twin = [(k.clone(), v.clone()) for k, v in run.kv]
    start = [30, 12, 0, 25]
    pos_g = torch.tensor(start, dtype=torch.int32, device="cuda")
    pos_e = pos_g.clone()
    xg = torch.empty((w.B, 1, w.d), dtype=w.torch_dtype, device="cuda")
    og = torch.empty_like(xg)
    graph = run.stack.capture(xg, pos_g, run.kv, og)
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(77)
    for step in range(5):
        x = (torch.randn((w.B, 1, w.d), generator=gen)).to(w.torch_dtype).to("cuda")
        oe = torch.empty_like(x)
        run.stack.forward_device_pos(x, pos_e, twin, oe, advance=True)
        _ = (x.float() * 2).sum().item()  # eager work and a synchronisation between replays
        xg.copy_(x)
        graph.launch()
        torch.cuda.synchronize()
        assert torch.equal(og, oe), step
        assert torch.equal(pos_g, pos_e), step
        for (ka, va), (kb, vb) in zip(run.kv, twin):
            assert torch.equal(ka, kb) and torch.equal(va, vb), step
        log(f"    replay {step}: bitwise equal to eager, positions {pos_g.cpu().tolist()}")
    assert pos_g.cpu().tolist() == [p + 5 for p in start]
    run.close()


def test_stack_rejects_bad_calls_without_writing():
    w = workloads.BlockWorkload("stack_bad", "bf16", B=2, S=2, start_pos=0, d=512, H=8, n_kv=2,
                                d_head=64, d_ff=1024, theta=5e5, eps=1e-5, w_std=0.02, g_mean=1.0,
                                g_std=0.05, max_seq=16, seed=1)
    run = StackRun(w, 2)
    x = run.t["x"].to("cuda")
    out = torch.full_like(x, 7.0)
    before = [(k.clone(), v.clone()) for k, v in run.kv]
    cases = {
        "past the cache": lambda: run.stack.forward(x, 15, run.kv, out),
        "second cache holds one sequence": lambda: run.stack.forward(
            x, 0, run.kv[:1] + [(run.kv[1][0][:1], run.kv[1][1][:1])], out),
        "hidden overlaps out": lambda: run.stack.forward(x, 0, run.kv, out,
                                                         hidden=out.expand((2,) + tuple(x.shape))),
    }
    for name, fn in cases.items():
        with pytest.raises((lbmod.LlamaBlockError, ValueError)) as e:
            fn()
        log(f"    {name}: {e.value}")
    torch.cuda.synchronize()
    assert torch.equal(out, torch.full_like(x, 7.0))
    for (ka, va), (kb, vb) in zip(run.kv, before):
        assert torch.equal(ka, kb) and torch.equal(va, vb)
    run.close()
