"""Seeded synthetic workloads for one Llama pre-norm decoder block.

This module only names shapes and draws random tensors.  It holds none of the
block's arithmetic, so both the fp64 oracle (test infrastructure) and the HIP
library's callers (tests, bench) can take their inputs from it without sharing
any part of the computation.

Shapes follow the pages:
  * the Llama-3-8B width (d 4096, 32 query heads, 8 KV heads of 128, FFN 14336,
    rotation base 500 000) -- "The Evolving Transformer 04 LLaMA", section
    "00 CONFIG"; "Full Llama 3 transformer block", section "How it works";
  * the Llama-3-70B width (d 8192, FFN 28672, head 128, 8 KV heads) -- "Full
    Llama 3 transformer block", section "How it works";
  * the SmolLM2-135M width (d 576, 9 query / 3 KV heads, FFN 1536, base
    100 000) -- "From GPT-2 to Llama", sections "Positions become a rotation",
    "The feed-forward grows a gate" and "Keys and values get shared".

Draw protocol (one torch CPU generator per workload, seeded):
  x, g1, Wq, Wk, Wv, Wo, g2, W_gate, W_up, W_down, then the pre-filled K and V
  cache rows (decode workloads only), then for mixture-of-experts blocks the
  router [E][d] and the experts' gate [E][f][d], up [E][f][d], down [E][d][f].  Each draw is randn(shape, fp32) * std +
  mean, then rounded to the workload dtype (round-to-nearest-even for bf16).
  Gains given as "ones" consume no draws.  The second parameter of N(mu, s) is
  the standard deviation.

Layouts: activations [B][S][d]; weights [out][in] (nn.Linear); pre-filled cache
rows are drawn as K[B][n_kv][start_pos][d_head] and V[B][n_kv][start_pos][d_head]
(natural per-position rows; callers re-layout them for their own cache format).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Dict, Optional

import torch

__all__ = ["BlockWorkload", "WORKLOADS", "get", "generate", "generate_stack",
           "generate_stack_on_device", "param_count", "stack_layer_seed", "with_overrides"]


@dataclass(frozen=True)
class BlockWorkload:
    name: str
    dtype: str            # "f32" or "bf16": dtype of x, weights, gains, cache, out
    B: int                # sequences
    S: int                # new tokens per sequence in this call
    start_pos: int        # absolute position of the first new token
    d: int                # model width
    H: int                # query heads
    n_kv: int             # key/value heads
    d_head: int
    d_ff: int
    theta: float          # rotation base
    eps: float            # RMSNorm epsilon
    w_std: float          # projection weights ~ N(0, w_std)
    g_mean: float = 1.0   # RMSNorm gains ~ N(g_mean, g_std); g_std None -> exactly ones
    g_std: Optional[float] = None
    x_std: float = 1.0    # x ~ N(0, x_std)
    cache_std: float = 1.0  # pre-filled cache rows ~ N(0, cache_std)
    max_seq: int = 0      # cache capacity per sequence (0 -> start_pos + S)
    seed: int = 0
    rope_half: bool = False   # RoPE pairs (i, i + d_head/2) instead of (2i, 2i+1)
    rope_scaling: Optional[tuple] = None  # (scale, low, high, original length) or None
    # mixture-of-experts FFN: n_experts > 0 adds a router and n_experts routed
    # SwiGLU experts of width d_ff_expert, top_k per token; the block's own
    # FFN (width d_ff) is then the always-on shared expert
    n_experts: int = 0
    top_k: int = 0
    d_ff_expert: int = 0

    @property
    def capacity(self) -> int:
        return self.max_seq if self.max_seq > 0 else self.start_pos + self.S

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"f32": torch.float32, "bf16": torch.bfloat16}[self.dtype]

    @property
    def M(self) -> int:
        return self.B * self.S

    @property
    def n_rep(self) -> int:
        return self.H // self.n_kv

    @property
    def moe(self) -> Optional[Dict]:
        if self.n_experts <= 0:
            return None
        return {"n_experts": self.n_experts, "top_k": self.top_k, "d_ff_expert": self.d_ff_expert}


WORKLOADS: Dict[str, BlockWorkload] = {
    # tiny fp32 block: d_ff 176 = 8/3 * 64 rounded up to a multiple of 16
    "tiny_f32": BlockWorkload("tiny_f32", "f32", B=1, S=16, start_pos=0, d=64, H=4, n_kv=2,
                              d_head=16, d_ff=176, theta=1e4, eps=1e-5, w_std=0.02,
                              g_mean=1.0, g_std=0.1),
    "smollm2_135m_prefill": BlockWorkload("smollm2_135m_prefill", "bf16", B=4, S=512, start_pos=0,
                                          d=576, H=9, n_kv=3, d_head=64, d_ff=1536, theta=1e5,
                                          eps=1e-5, w_std=0.02),
    "llama3_8b_prefill": BlockWorkload("llama3_8b_prefill", "bf16", B=2, S=2048, start_pos=0,
                                       d=4096, H=32, n_kv=8, d_head=128, d_ff=14336, theta=5e5,
                                       eps=1e-5, w_std=0.02, g_mean=1.0, g_std=0.05),
    "llama3_8b_decode": BlockWorkload("llama3_8b_decode", "bf16", B=32, S=1, start_pos=8191,
                                      d=4096, H=32, n_kv=8, d_head=128, d_ff=14336, theta=5e5,
                                      eps=1e-5, w_std=0.02, g_mean=1.0, g_std=0.05,
                                      cache_std=1.0, max_seq=8192),
    # SmolLM2-135M decode at the end of a 1,024-token text (the length the
    # page measures the model on), 32 sequences and a single one
    "smollm2_135m_decode": BlockWorkload("smollm2_135m_decode", "bf16", B=32, S=1, start_pos=1023,
                                         d=576, H=9, n_kv=3, d_head=64, d_ff=1536, theta=1e5,
                                         eps=1e-5, w_std=0.02, max_seq=1024),
    "smollm2_135m_decode_b1": BlockWorkload("smollm2_135m_decode_b1", "bf16", B=1, S=1, start_pos=1023,
                                            d=576, H=9, n_kv=3, d_head=64, d_ff=1536, theta=1e5,
                                            eps=1e-5, w_std=0.02, max_seq=1024),
    # a mixture-of-experts block at the width of the Llama 4 page's
    # representative block (d 4096, 32 heads of 128, 8 KV heads): 16 routed
    # experts, top 1, expert and shared-expert width 8192 (the page gives no
    # expert counts or widths; these are this library's choice)
    "llama4_moe_prefill": BlockWorkload("llama4_moe_prefill", "bf16", B=2, S=2048, start_pos=0, d=4096, H=32,
                                        n_kv=8, d_head=128, d_ff=8192, theta=5e5, eps=1e-5, w_std=0.02,
                                        g_mean=1.0, g_std=0.05, n_experts=16, top_k=1, d_ff_expert=8192),
    "llama4_moe_decode": BlockWorkload("llama4_moe_decode", "bf16", B=32, S=1, start_pos=8191, d=4096, H=32,
                                       n_kv=8, d_head=128, d_ff=8192, theta=5e5, eps=1e-5, w_std=0.02,
                                       g_mean=1.0, g_std=0.05, cache_std=1.0, max_seq=8192, n_experts=16,
                                       top_k=1, d_ff_expert=8192),
    # one sequence decoding at the end of the 8B context: the per-token
    # latency case, bound by streaming the block's 436 MB of weights
    "llama3_8b_decode_b1": BlockWorkload("llama3_8b_decode_b1", "bf16", B=1, S=1, start_pos=8191, d=4096,
                                         H=32, n_kv=8, d_head=128, d_ff=14336, theta=5e5, eps=1e-5,
                                         w_std=0.02, g_mean=1.0, g_std=0.05, cache_std=1.0, max_seq=8192),
    "llama3_70b_prefill": BlockWorkload("llama3_70b_prefill", "bf16", B=1, S=4096, start_pos=0,
                                        d=8192, H=64, n_kv=8, d_head=128, d_ff=28672, theta=5e5,
                                        eps=1e-5, w_std=0.01),
}


def get(name: str) -> BlockWorkload:
    return WORKLOADS[name]


def with_overrides(w: BlockWorkload, **kw) -> BlockWorkload:
    """A copy of a workload with some fields changed (smaller B/S, other seed ...)."""
    return dataclasses.replace(w, **kw)


def param_count(w: BlockWorkload) -> Dict[str, int]:
    """Weight counts of one block (shape bookkeeping only)."""
    attn = w.d * w.H * w.d_head + 2 * w.d * w.n_kv * w.d_head + w.H * w.d_head * w.d
    ffn = 3 * w.d * w.d_ff
    norms = 2 * w.d
    return {"attn": attn, "ffn": ffn, "norms": norms, "total_linear": attn + ffn}


def _draw(gen: torch.Generator, shape, mean: float, std: float, dtype: torch.dtype) -> torch.Tensor:
    t = torch.randn(shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(dtype)


def generate(w: BlockWorkload, with_cache: bool = True) -> Dict[str, torch.Tensor]:
    """Draw every tensor of a workload on the CPU, in the workload dtype.

    Returns x [B][S][d], attn_norm / ffn_norm [d], wq [H*dh][d], wk / wv
    [n_kv*dh][d], wo [d][H*dh], w_gate / w_up [d_ff][d], w_down [d][d_ff], and,
    when start_pos > 0 and with_cache, k_prefix / v_prefix
    [B][n_kv][start_pos][d_head] holding the already-cached rows.
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed)
    dt = w.torch_dtype
    out: Dict[str, torch.Tensor] = {}
    out["x"] = _draw(gen, (w.B, w.S, w.d), 0.0, w.x_std, dt)

    def gain():
        if w.g_std is None:
            return torch.full((w.d,), w.g_mean, dtype=torch.float32).to(dt)
        return _draw(gen, (w.d,), w.g_mean, w.g_std, dt)

    out["attn_norm"] = gain()
    out["wq"] = _draw(gen, (w.H * w.d_head, w.d), 0.0, w.w_std, dt)
    out["wk"] = _draw(gen, (w.n_kv * w.d_head, w.d), 0.0, w.w_std, dt)
    out["wv"] = _draw(gen, (w.n_kv * w.d_head, w.d), 0.0, w.w_std, dt)
    out["wo"] = _draw(gen, (w.d, w.H * w.d_head), 0.0, w.w_std, dt)
    out["ffn_norm"] = gain()
    out["w_gate"] = _draw(gen, (w.d_ff, w.d), 0.0, w.w_std, dt)
    out["w_up"] = _draw(gen, (w.d_ff, w.d), 0.0, w.w_std, dt)
    out["w_down"] = _draw(gen, (w.d, w.d_ff), 0.0, w.w_std, dt)
    if with_cache and w.start_pos > 0:
        shape = (w.B, w.n_kv, w.start_pos, w.d_head)
        out["k_prefix"] = _draw(gen, shape, 0.0, w.cache_std, dt)
        out["v_prefix"] = _draw(gen, shape, 0.0, w.cache_std, dt)
    if w.n_experts > 0:
        # after everything above, so a block's dense draws do not depend on
        # whether it has experts
        E, fe = w.n_experts, w.d_ff_expert
        out["router"] = _draw(gen, (E, w.d), 0.0, w.w_std, dt)
        out["e_gate"] = _draw(gen, (E, fe, w.d), 0.0, w.w_std, dt)
        out["e_up"] = _draw(gen, (E, fe, w.d), 0.0, w.w_std, dt)
        out["e_down"] = _draw(gen, (E, w.d, fe), 0.0, w.w_std, dt)
    return out


def stack_layer_seed(seed: int, layer: int) -> int:
    """Seed of block `layer` of a stack drawn from a workload with `seed`."""
    return seed * 1_000_003 + 7919 * (layer + 1)


def generate_stack(w: BlockWorkload, n_layers: int, with_cache: bool = True) -> Dict:
    """Draw a stack of n_layers blocks of the workload's shape.

    x [B][S][d] and the final RMSNorm gain final_norm [d] come from the
    workload's own generator (x first, then the gain, drawn like the block's
    gains).  Block l's tensors are those of generate() for the same workload
    with seed stack_layer_seed(w.seed, l), without its x: its own weights and,
    for start_pos > 0, its own pre-filled cache rows.  Returns {"x", "final_norm",
    "layers": [dict per block]}.
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed)
    dt = w.torch_dtype
    x = _draw(gen, (w.B, w.S, w.d), 0.0, w.x_std, dt)
    if w.g_std is None:
        final = torch.full((w.d,), w.g_mean, dtype=torch.float32).to(dt)
    else:
        final = _draw(gen, (w.d,), w.g_mean, w.g_std, dt)
    layers = []
    for l in range(n_layers):
        t = generate(with_overrides(w, seed=stack_layer_seed(w.seed, l)), with_cache=with_cache)
        del t["x"]
        layers.append(t)
    return {"x": x, "final_norm": final, "layers": layers}


def generate_stack_on_device(w: BlockWorkload, n_layers: int, device="cuda") -> Dict:
    """A stack of the workload's shape drawn on the device with torch's device
    generator (for model-sized stacks, whose weights would take minutes to draw
    on the host).  Same distributions as generate_stack, other random streams:
    one generator seeded stack_layer_seed(w.seed, l) per block, drawing that
    block's tensors in the order of generate(); x and final_norm from a
    generator seeded w.seed.  Pre-filled cache rows (start_pos > 0) are drawn
    into the returned per-block "k_prefix" / "v_prefix" as in generate()."""
    def draw(gen, shape, mean, std):
        t = torch.randn(shape, generator=gen, dtype=torch.float32, device=device)
        if std != 1.0:
            t.mul_(std)
        if mean != 0.0:
            t.add_(mean)
        return t.to(w.torch_dtype)

    def gain(gen):
        if w.g_std is None:
            return torch.full((w.d,), w.g_mean, dtype=torch.float32, device=device).to(w.torch_dtype)
        return draw(gen, (w.d,), w.g_mean, w.g_std)

    g0 = torch.Generator(device=device)
    g0.manual_seed(w.seed)
    x = draw(g0, (w.B, w.S, w.d), 0.0, w.x_std)
    final = gain(g0)
    layers = []
    for l in range(n_layers):
        gen = torch.Generator(device=device)
        gen.manual_seed(stack_layer_seed(w.seed, l))
        t = {"attn_norm": gain(gen),
             "wq": draw(gen, (w.H * w.d_head, w.d), 0.0, w.w_std),
             "wk": draw(gen, (w.n_kv * w.d_head, w.d), 0.0, w.w_std),
             "wv": draw(gen, (w.n_kv * w.d_head, w.d), 0.0, w.w_std),
             "wo": draw(gen, (w.d, w.H * w.d_head), 0.0, w.w_std),
             "ffn_norm": gain(gen),
             "w_gate": draw(gen, (w.d_ff, w.d), 0.0, w.w_std),
             "w_up": draw(gen, (w.d_ff, w.d), 0.0, w.w_std),
             "w_down": draw(gen, (w.d, w.d_ff), 0.0, w.w_std)}
        if w.start_pos > 0:
            shape = (w.B, w.n_kv, w.start_pos, w.d_head)
            t["k_prefix"] = draw(gen, shape, 0.0, w.cache_std)
            t["v_prefix"] = draw(gen, shape, 0.0, w.cache_std)
        if w.n_experts > 0:
            E, fe = w.n_experts, w.d_ff_expert
            t["router"] = draw(gen, (E, w.d), 0.0, w.w_std)
            t["e_gate"] = draw(gen, (E, fe, w.d), 0.0, w.w_std)
            t["e_up"] = draw(gen, (E, fe, w.d), 0.0, w.w_std)
            t["e_down"] = draw(gen, (E, w.d, fe), 0.0, w.w_std)
        layers.append(t)
    return {"x": x, "final_norm": final, "layers": layers}
