"""Helpers for the GPU parity tests: run a workload through the HIP library
and through the fp64 oracle on the same seeded inputs, and compare.

Not a test module.  The GPU side goes through the C ABI only (the thin
binding in decoder_only_transformer_amd); the oracle side through oracle/.
"""
from __future__ import annotations

import sys
from typing import Dict, Optional, Sequence

import numpy as np
import torch

import decoder_only_transformer_amd as lbmod
import oracle
import workloads


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def config_for(w: workloads.BlockWorkload, operands: str = "auto", max_tokens: Optional[int] = None,
               max_seq_len: Optional[int] = None):
    return lbmod.make_config(w.d, w.H, w.n_kv, w.d_head, w.d_ff, max_tokens or w.M,
                             max_seq_len or w.capacity, w.theta, w.eps, w.dtype, operands,
                             rope_half=w.rope_half, rope_scaling=w.rope_scaling)


def device_weights(tensors: Dict[str, torch.Tensor]) -> Dict[str, torch.Tensor]:
    return {n: tensors[n].to("cuda") for n in lbmod.WEIGHT_NAMES}


def gpu_cache(w: workloads.BlockWorkload, tensors: Dict[str, torch.Tensor], fill: float = 0.0,
              cap: Optional[int] = None):
    """Cache in the library layout with the workload's pre-filled prefix copied in."""
    cap = cap or w.capacity
    if w.dtype == "bf16":
        cap = (cap + 7) // 8 * 8
    k, v = lbmod.new_kv_cache(w.B, w.n_kv, cap, w.d_head, w.torch_dtype, fill=fill)
    if w.start_pos > 0:
        k[:, :, : w.start_pos, :] = tensors["k_prefix"].to("cuda")
        v[:, :, : w.start_pos, :] = tensors["v_prefix"].to("cuda")
    return k, v


class BlockOnGpu:
    def __init__(self, w, tensors, operands="auto", max_tokens=None, fill=0.0, cap=None,
                 max_seq_len=None):
        self.w = w
        self.cap = cap
        cfg = config_for(w, operands, max_tokens, max_seq_len or (cap if cap else None))
        wd = device_weights(tensors)
        self.block = lbmod.LlamaBlock(cfg, wd)
        del wd
        self.kv = gpu_cache(w, tensors, fill=fill, cap=cap)
        self.x = tensors["x"].to("cuda")
        self.out = torch.empty_like(self.x)

    def forward(self, x=None, start_pos=None, out=None):
        x = self.x if x is None else x
        out = self.out if out is None else out
        sp = self.w.start_pos if start_pos is None else start_pos
        self.block.forward(x, sp, self.kv, out)
        torch.cuda.synchronize()
        return out

    def close(self):
        self.block.close()


def oracle_rows(w, tensors, rows: Optional[Sequence[int]] = None, stages=False):
    return oracle.run_workload(w, tensors, rows=rows, stages=stages)


def rel_err(got: np.ndarray, want: np.ndarray) -> float:
    """max |got - want| / rms(want)."""
    rms = float(np.sqrt(np.mean(want * want)))
    return float(np.max(np.abs(got - want))) / rms


def tol_of(w) -> float:
    return 1e-4 if w.dtype == "f32" else 2e-2


def gpu_cache_rows(w, kv, b, lo, hi):
    """GPU cache rows [lo, hi) of sequence b as fp64 arrays [n_kv][n][d_head] (K and V)."""
    k, v = kv
    kk = k[b, :, lo:hi, :].double().cpu().numpy()
    vv = v[b, :, lo:hi, :].double().cpu().numpy()
    return kk, vv


def sample_rows(w, per_seq: Sequence[int]):
    rows = []
    for b in range(w.B):
        for s in per_seq:
            if 0 <= s < w.S:
                rows.append(b * w.S + s)
    return sorted(set(rows))
