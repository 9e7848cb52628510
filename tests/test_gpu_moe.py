"""GPU parity for mixture-of-experts blocks (llama_moe_block_init): the FFN is
a shared expert plus the router's top-k experts ("Llama 4 From Scratch", The
idea).

The choice of experts is an integer decision taken from floating-point
logits: the library scores in fp32 from the operand-type (fp16) normalised row,
the oracle in fp64.  So the tests check, per token:
  * the library's logits against the oracle's within d_t = 2^-10 * max_e
    sum_i |n_i r_ei|, twice the effect of rounding n to fp16 (unit roundoff
    2^-11, the router weights being exact in fp16), the fp32 sums adding far
    less;
  * that the library's choice is a valid top k of the oracle's logits within
    2 d_t (every chosen logit at least every unchosen one minus 2 d_t, and in
    order), so only near-ties may be resolved differently;
  * y, and the written cache rows, against the oracle run with the library's
    choice, at the block bar (2e-2 rms), and the weights against the
    oracle's softmax of the chosen logits within 4 d_t;
  * every routed expert's output row (before its weight) against that
    expert's FFN of the library's n2 row, at 2e-2 of those rows' own rms.
"""
import numpy as np
import pytest
import torch

import decoder_only_transformer_amd as lbmod
import oracle
import workloads
from block_harness import config_for, gpu_cache, gpu_cache_rows, log, rel_err, tol_of

pytestmark = pytest.mark.gpu


def _moe_weights(t):
    return {n: t[n].to("cuda") for n in list(lbmod.WEIGHT_NAMES) + list(lbmod.MOE_WEIGHT_NAMES.values())}


class MoeRun:
    def __init__(self, w, t, max_tokens=None, cap=None):
        self.w, self.t = w, t
        self.cap = cap or w.capacity
        cfg = config_for(w, max_tokens=max_tokens or w.M, max_seq_len=(self.cap + 7) // 8 * 8)
        self.block = lbmod.LlamaMoeBlock(cfg, _moe_weights(t), w.moe)
        self.kv = gpu_cache(w, t, cap=self.cap)
        self.x = t["x"].to("cuda")
        self.out = torch.empty_like(self.x)

    def forward(self, start_pos=None):
        self.block.forward(self.x, self.w.start_pos if start_pos is None else start_pos, self.kv, self.out)
        torch.cuda.synchronize()
        return self.out

    def close(self):
        self.block.close()


def _logit_bound(n2, router):
    """Per row: 2^-10 * max_e sum_i |n_i r_ei| (see the module docstring)."""
    return 2.0 ** -10 * np.max(np.abs(n2) @ np.abs(router).T, axis=1)


def _worst(got, want, rows, sel, k=1):
    """Where the largest error of got against want sits: flat row (and, for
    routed rows, its token and choice), column, both values, expert(s)."""
    i, c = np.unravel_index(np.argmax(np.abs(got - want)), got.shape)
    r = rows[i]
    where = f"token {r // k} choice {r % k}" if k > 1 else f"row {r}"
    return f"worst at {where} col {c}: {got[i, c]:.6g} vs {want[i, c]:.6g}, expert(s) {list(sel[r])}"


def check_moe(w, rows=None, start_pos=None):
    """Run w on the GPU and check it as the module docstring says; rows:
    optional flat rows to check (all when None)."""
    log(f"[case] moe {w.name} B={w.B} S={w.S} start={w.start_pos} d={w.d} E={w.n_experts} k={w.top_k} "
        f"fe={w.d_ff_expert} d_ff={w.d_ff}")
    t = workloads.generate(w)
    run = MoeRun(w, t)
    y = run.forward().double().cpu().numpy().reshape(w.M, w.d)
    sel, wts, lg = (a.cpu().numpy() for a in run.block.routing(w.M))
    n2 = run.block.stage("n2", w.M).double().cpu().numpy()
    cfg, moe = oracle.cfg_of(w), w.moe
    kc, vc = oracle.empty_cache(w, run.cap)
    if w.start_pos > 0:
        kc[:, :, :w.start_pos] = t["k_prefix"].double().numpy()
        vc[:, :, :w.start_pos] = t["v_prefix"].double().numpy()
    rows = list(range(w.M)) if rows is None else list(rows)
    # the oracle with the library's choice (its logits do not depend on it)
    k1, v1 = kc.copy(), vc.copy()
    y_o, _, wts_o, lg_o = oracle.moe_block_forward(cfg, moe, t["x"], t, w.start_pos, k1, v1, rows=rows,
                                                   force_sel=sel)
    y_o = y_o.reshape(w.M, w.d)
    sel_o = np.argsort(-lg_o, axis=1, kind="stable")[:, :w.top_k]   # the exact top k
    bound = _logit_bound(n2, t["router"].double().numpy())
    K, E = w.top_k, w.n_experts
    differ = 0
    for r in rows:
        d = bound[r]
        assert np.max(np.abs(lg[r] - lg_o[r])) <= d, ("logits", r, np.max(np.abs(lg[r] - lg_o[r])), d)
        chosen = list(sel[r])
        assert len(set(chosen)) == K and all(0 <= e < E for e in chosen), ("choice", r, chosen)
        rest = [e for e in range(E) if e not in chosen]
        if rest:
            assert min(lg_o[r][chosen]) >= max(lg_o[r][rest]) - 2 * d, ("not a top k", r)
        for j in range(K - 1):
            assert lg_o[r][chosen[j]] >= lg_o[r][chosen[j + 1]] - 2 * d, ("order", r)
        differ += int(chosen != list(sel_o[r]))
    err = rel_err(y[rows], y_o[rows])
    werr = np.max(np.abs(wts[rows] - wts_o[rows]) / (4 * bound[rows, None] + 1e-7))
    tol = tol_of(w)
    log(f"    y {err:.3e} (tol {tol:g}); choices differing from the exact top k: {differ} of {len(rows)}; "
        f"weights within {werr:.2f} of their bound; {_worst(y[rows], y_o[rows], rows, sel)}")
    assert err <= tol, err
    assert werr <= 1.0, werr
    # every routed expert's output at its own scale (a few % of y's rms at
    # these weights, so y alone would hide errors in it): the oracle's FFN of
    # that expert alone (top 1 forced to it, shared expert zeroed) on the
    # library's n2 row
    r_gpu = run.block.stage("routed", w.M * K).double().cpu().numpy().reshape(w.M, K, w.d)
    one = dict(moe, n_experts=1, top_k=1)
    solo = {n: np.zeros(tuple(t[n].shape)) for n in ("w_gate", "w_up", "w_down")}
    r_o = np.zeros((len(rows), K, w.d))
    for e in sorted({int(sel[r][j]) for r in rows for j in range(K)}):
        solo.update({n: t[n][e:e + 1].double().numpy() for n in oracle.MOE_WEIGHT_NAMES})
        for i, r in enumerate(rows):
            for j in range(K):
                if int(sel[r][j]) == e:
                    r_o[i, j] = oracle.moe_ffn(cfg, one, n2[r], solo, force_sel=[0])[0]
    rerr = rel_err(r_gpu[rows], r_o)
    log(f"    routed expert rows {rerr:.3e} (tol {tol:g}); "
        f"{_worst(r_gpu[rows].reshape(len(rows) * K, w.d), r_o.reshape(len(rows) * K, w.d), [r * K + j for r in rows for j in range(K)], sel.reshape(-1, 1), K)}")
    assert rerr <= tol, rerr
    seqs = sorted({r // w.S for r in rows})
    for b in seqs:
        hi = max(r % w.S for r in rows if r // w.S == b) + 1
        kk, vv = gpu_cache_rows(w, run.kv, b, w.start_pos, w.start_pos + hi)
        ek = rel_err(kk, k1[b, :, w.start_pos:w.start_pos + hi])
        ev = rel_err(vv, v1[b, :, w.start_pos:w.start_pos + hi])
        assert ek <= tol and ev <= tol, (b, ek, ev)
    run.close()
    return differ


def _small(**kw):
    base = dict(name="moe_small", dtype="bf16", B=2, S=100, start_pos=0, d=512, H=8, n_kv=2, d_head=64,
                d_ff=1024, theta=5e5, eps=1e-5, w_std=0.02, g_mean=1.0, g_std=0.05, seed=3,
                n_experts=8, top_k=2, d_ff_expert=512)
    base.update(kw)
    return workloads.BlockWorkload(**base)


def test_moe_prefill_top2_of_8():
    """200 tokens, 8 experts, top 2: about 50 rows per expert, every expert's
    rows one partial 128-row tile."""
    check_moe(_small())


def test_moe_prefill_smollm2_width_top1_of_16():
    """SmolLM2 width (d_head 64, three heads per KV group), 16 experts, top 1,
    expert width 768, 4 x 96 tokens."""
    check_moe(_small(name="moe_smol", B=4, S=96, d=576, H=9, n_kv=3, d_ff=1536, theta=1e5, n_experts=16,
                     top_k=1, d_ff_expert=768, seed=5))


def test_moe_decode_most_experts_empty():
    """Decode of 5 sequences at position 300: 10 (token, choice) pairs over 16
    experts, so most experts get no rows and their tiles are skipped."""
    check_moe(_small(name="moe_decode", B=5, S=1, start_pos=300, max_seq=304, n_experts=16, top_k=2,
                     seed=7))


def test_moe_every_expert_taken():
    """top_k = n_experts = 4: every token uses every expert."""
    check_moe(_small(name="moe_all", B=1, S=70, n_experts=4, top_k=4, d_ff_expert=256, seed=9))


def test_moe_single_expert():
    """One routed expert (weight exactly 1) beside the shared one."""
    check_moe(_small(name="moe_one", B=2, S=33, n_experts=1, top_k=1, seed=10))


def test_moe_large_groups():
    """600 tokens over 4 experts, top 1: groups of several full 128-row tiles
    plus a partial one."""
    check_moe(_small(name="moe_large", B=2, S=300, n_experts=4, top_k=1, d_ff_expert=1024, seed=12))


@pytest.mark.parametrize("E,k", [(2, 1), (4, 2)])
def test_moe_256_row_tiles(E, k):
    """600 tokens with at least 256 (token, choice) pairs per expert on
    average: the experts run on the 256 x 256 grouped kernel, each group one
    full tile plus a partial one."""
    check_moe(_small(name=f"moe_big_tiles_{E}_{k}", B=2, S=300, n_experts=E, top_k=k, d_ff_expert=512,
                     seed=20 + E))


@pytest.mark.parametrize("E,k,seed", [(20, 2, 31), (40, 2, 32), (100, 3, 33), (256, 8, 34)])
def test_moe_router_expert_tiles(E, k, seed):
    """Routers over 2, 4, 8 and 16 tiles of 16 experts (the last tile partial
    where E is not a multiple of 16), up to the largest expert count and top k
    the library takes; 200 tokens, so the last block of 16 tokens is partial."""
    check_moe(_small(name=f"moe_router_{E}_{k}", B=2, S=100, n_experts=E, top_k=k, d_ff_expert=128, seed=seed))


def test_moe_llama3_width_sampled():
    """The 8B-width attention with a MoE FFN (8 experts of width 4096, top 2,
    shared expert 4096) over 2 x 256 tokens; rows sampled at the ends of each
    sequence and across the tile edges."""
    w = workloads.BlockWorkload("moe_8b", "bf16", B=2, S=256, start_pos=0, d=4096, H=32, n_kv=8, d_head=128,
                                d_ff=4096, theta=5e5, eps=1e-5, w_std=0.02, g_mean=1.0, g_std=0.05, seed=14,
                                n_experts=8, top_k=2, d_ff_expert=4096)
    rows = sorted({b * w.S + s for b in range(w.B) for s in (0, 1, 63, 64, 127, 128, 200, 254, 255)})
    check_moe(w, rows=rows)


def test_moe_benchmark_shape_sampled():
    """The benchmark's MoE prefill shape and launch path (16 experts of 8192,
    top 1, shared expert 8192, d 4096, 2 x 2048 tokens: 256-row grouped
    tiles), rows sampled at both ends of each sequence and across tiles."""
    w = workloads.get("llama4_moe_prefill")
    rows = sorted({b * w.S + s for b in range(w.B) for s in (0, 1, 255, 256, 1023, 2047)})
    check_moe(w, rows=rows)


def test_moe_decode_benchmark_shape():
    """The benchmark's MoE decode shape and launch path (32 sequences at
    position 8191 over a drawn cache, 16 experts of 8192, top 1, shared expert
    8192, d 4096: 32-row expert tiles streamed non-temporally), every row."""
    check_moe(workloads.get("llama4_moe_decode"))


def test_moe_zero_router_takes_the_first_experts():
    """A zero router scores every expert 0: the library takes experts 0 and 1,
    each weighted 1/2, exactly as the tie rule says."""
    w = _small(name="moe_zero", B=1, S=40, seed=15)
    t = workloads.generate(w)
    t["router"] = torch.zeros_like(t["router"])
    run = MoeRun(w, t)
    run.forward()
    sel, wts, lg = run.block.routing(w.M)
    assert torch.equal(lg, torch.zeros_like(lg))
    assert (sel.cpu() == torch.tensor([0, 1], dtype=torch.int32)).all()
    assert (wts.cpu() == 0.5).all()
    y = run.out.double().cpu().numpy().reshape(w.M, w.d)
    kc, vc = oracle.empty_cache(w)
    y_o, sel_o, _, _ = oracle.moe_block_forward(oracle.cfg_of(w), w.moe, t["x"], t, 0, kc, vc)
    assert (sel_o == np.array([0, 1])).all()
    err = rel_err(y, y_o.reshape(w.M, w.d))
    log(f"    y {err:.3e}")
    assert err <= tol_of(w)
    run.close()


def test_moe_deterministic_bitwise():
    """Two forwards of the same input give the same bits (rows may land in
    other places inside an expert's group; each row's value does not depend
    on its place)."""
    w = _small(name="moe_det", B=2, S=150, seed=16)
    t = workloads.generate(w)
    run = MoeRun(w, t)
    a = run.forward().clone()
    b = run.forward().clone()
    assert torch.equal(a, b)
    run.close()


def test_moe_ragged_decode():
    """Ragged decode through a MoE block: each sequence at its own position
    against a one-sequence oracle run with the library's choice."""
    w = _small(name="moe_ragged", B=4, S=1, start_pos=60, max_seq=64, n_experts=8, top_k=2, seed=17)
    pos = [0, 60, 13, 42]
    t = workloads.generate(w)
    run = MoeRun(w, t)
    y = run.forward(start_pos=pos).double().cpu().numpy().reshape(w.B, w.d)
    sel = run.block.routing(w.M)[0].cpu().numpy()
    for b, p in enumerate(pos):
        wb = workloads.with_overrides(w, B=1, start_pos=p, max_seq=0)
        tb = dict(t)
        tb["x"] = t["x"][b:b + 1]
        kc, vc = oracle.empty_cache(wb, 64)
        kc[:, :, :p] = t["k_prefix"][b:b + 1, :, :p].double().numpy()
        vc[:, :, :p] = t["v_prefix"][b:b + 1, :, :p].double().numpy()
        y_o, _, _, _ = oracle.moe_block_forward(oracle.cfg_of(wb), w.moe, tb["x"], tb, p, kc, vc,
                                                force_sel=sel[b:b + 1])
        err = rel_err(y[b], y_o.reshape(-1))
        log(f"    seq {b} @ {p}: y {err:.3e}")
        assert err <= tol_of(w)
    run.close()
