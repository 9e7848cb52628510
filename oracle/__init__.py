"""Python access to the fp64 C oracle (TEST INFRASTRUCTURE ONLY).

Only tests/, the smoke check and the benchmark's CPU-baseline leg import this
package.  The HIP library and its binding never do.

All arrays are numpy float64, C-contiguous, in the oracle's own layouts
(documented in oracle.h): the cache is [B][n_kv][cap][d_head] with one row per
absolute position, for both K and V.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


class _Cfg(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int), ("n_heads", ctypes.c_int), ("n_kv_heads", ctypes.c_int),
                ("d_head", ctypes.c_int), ("d_ff", ctypes.c_int),
                ("rope_theta", ctypes.c_double), ("norm_eps", ctypes.c_double),
                ("rope_half", ctypes.c_int), ("rope_scale", ctypes.c_double),
                ("rope_low", ctypes.c_double), ("rope_high", ctypes.c_double),
                ("rope_orig", ctypes.c_double)]


def _cfg_struct(cfg: Dict) -> "_Cfg":
    """cfg keys: d, H, n_kv, d_head, d_ff, theta, eps; optional rope_half (bool),
    rope_scaling (None or (scale, low, high, orig))."""
    sc = cfg.get("rope_scaling") or (0.0, 0.0, 0.0, 0.0)
    return _Cfg(cfg["d"], cfg["H"], cfg["n_kv"], cfg["d_head"], cfg["d_ff"], float(cfg["theta"]),
                float(cfg["eps"]), 1 if cfg.get("rope_half") else 0, float(sc[0]), float(sc[1]),
                float(sc[2]), float(sc[3]))


class _Weights(ctypes.Structure):
    _fields_ = [(n, _dp) for n in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm",
                                   "w_gate", "w_up", "w_down")]


STAGES = ("n1", "q", "k", "v", "o", "h", "n2", "z")


class _MoeCfg(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int), ("top_k", ctypes.c_int), ("d_ff_expert", ctypes.c_int)]


class _MoeWeights(ctypes.Structure):
    _fields_ = [("router", _dp), ("w_gate", _dp), ("w_up", _dp), ("w_down", _dp)]


MOE_WEIGHT_NAMES = ("router", "e_gate", "e_up", "e_down")


class _Stages(ctypes.Structure):
    _fields_ = [(n, _dp) for n in STAGES]


def lib():
    """Load liboracle.so, compiling it first if it is not there."""
    global _lib
    if _lib is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        L.orc_rms_norm.argtypes = [_dp, _dp, ctypes.c_int, ctypes.c_double, _dp]
        L.orc_linear.argtypes = [_dp, _dp, ctypes.c_int, ctypes.c_int, _dp]
        L.orc_rope.argtypes = [_dp, ctypes.c_int, ctypes.c_long, ctypes.c_double]
        L.orc_rope_freq.argtypes = [ctypes.POINTER(_Cfg), ctypes.c_int]
        L.orc_rope_freq.restype = ctypes.c_double
        L.orc_rope_cfg.argtypes = [_dp, ctypes.c_long, ctypes.POINTER(_Cfg)]
        L.orc_silu.argtypes = [ctypes.c_double]
        L.orc_silu.restype = ctypes.c_double
        L.orc_attend.argtypes = [_dp, _dp, _dp, ctypes.c_long, ctypes.c_int, _dp, _dp]
        L.orc_block_forward.argtypes = [ctypes.POINTER(_Cfg), ctypes.c_int, ctypes.c_int,
                                        ctypes.c_long, ctypes.c_long, _dp,
                                        ctypes.POINTER(_Weights), _dp, _dp, _dp,
                                        ctypes.POINTER(ctypes.c_int), ctypes.c_int,
                                        ctypes.POINTER(_Stages)]
        L.orc_block_forward.restype = ctypes.c_int
        _pp = ctypes.POINTER(_dp)
        L.orc_stack_forward.argtypes = [ctypes.POINTER(_Cfg), ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_long, ctypes.c_long, _dp,
                                        ctypes.POINTER(_Weights), _dp, _pp, _pp, _dp, _dp]
        L.orc_stack_forward.restype = ctypes.c_int
        _ip = ctypes.POINTER(ctypes.c_int)
        L.orc_moe_route.argtypes = [ctypes.POINTER(_MoeCfg), ctypes.c_int, _dp, _dp, _ip, ctypes.c_int,
                                    _dp, _dp]
        L.orc_moe_route.restype = ctypes.c_int
        L.orc_moe_ffn.argtypes = [ctypes.POINTER(_Cfg), ctypes.POINTER(_MoeCfg), _dp,
                                  ctypes.POINTER(_Weights), ctypes.POINTER(_MoeWeights), _ip,
                                  ctypes.c_int, _dp, _dp, _dp]
        L.orc_moe_ffn.restype = ctypes.c_int
        L.orc_moe_block_forward.argtypes = [ctypes.POINTER(_Cfg), ctypes.POINTER(_MoeCfg), ctypes.c_int,
                                            ctypes.c_int, ctypes.c_long, ctypes.c_long, _dp,
                                            ctypes.POINTER(_Weights), ctypes.POINTER(_MoeWeights), _dp,
                                            _dp, _dp, _ip, ctypes.c_int, _ip, ctypes.c_int, _dp, _dp]
        L.orc_moe_block_forward.restype = ctypes.c_int
        L.orc_num_threads.argtypes = []
        L.orc_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"], (a.dtype, a.flags)
    return a.ctypes.data_as(_dp)


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):  # torch tensor
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def num_threads() -> int:
    return lib().orc_num_threads()


# ---- single steps -------------------------------------------------------------------

def rms_norm(v, g, eps: float) -> np.ndarray:
    v, g = _f64(v), _f64(g)
    out = np.empty_like(v)
    lib().orc_rms_norm(_p(v), _p(g), v.shape[-1], eps, _p(out))
    return out


def linear(inp, w) -> np.ndarray:
    inp, w = _f64(inp), _f64(w)
    out = np.empty(w.shape[0], dtype=np.float64)
    lib().orc_linear(_p(inp), _p(w), w.shape[0], w.shape[1], _p(out))
    return out


def rope(v, pos: int, theta: float) -> np.ndarray:
    out = _f64(v).copy()
    lib().orc_rope(_p(out), out.shape[-1], int(pos), float(theta))
    return out


def rope_freq(cfg: Dict, i: int) -> float:
    """Rotation speed of pair i under cfg's RoPE settings (see _cfg_struct)."""
    c = _cfg_struct(cfg)
    return lib().orc_rope_freq(ctypes.byref(c), int(i))


def rope_cfg(v, pos: int, cfg: Dict) -> np.ndarray:
    """RoPE on one head vector with cfg's layout and frequency settings."""
    out = _f64(v).copy()
    c = _cfg_struct(cfg)
    lib().orc_rope_cfg(_p(out), int(pos), ctypes.byref(c))
    return out


def silu(a: float) -> float:
    return lib().orc_silu(float(a))


def attend(q, k_rows, v_rows) -> np.ndarray:
    q, k_rows, v_rows = _f64(q), _f64(k_rows), _f64(v_rows)
    n, dh = k_rows.shape
    scr = np.empty(max(n, 1), dtype=np.float64)
    out = np.empty(dh, dtype=np.float64)
    lib().orc_attend(_p(q), _p(k_rows), _p(v_rows), n, dh, _p(scr), _p(out))
    return out


# ---- whole block ----------------------------------------------------------------------

WEIGHT_NAMES = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")


def block_forward(cfg: Dict, x, weights: Dict, start_pos: int, k_cache: np.ndarray,
                  v_cache: np.ndarray, rows: Optional[Sequence[int]] = None,
                  stages: bool = False):
    """Run the block.  cfg keys: d, H, n_kv, d_head, d_ff, theta, eps.

    x: [B][S][d].  k_cache / v_cache: float64 [B][n_kv][cap][d_head], updated in
    place (rows [start_pos, start_pos+S) written).  Returns (y, stages_dict);
    with `rows`, only those flat rows of y (and of the stages) are meaningful.
    """
    x = _f64(x)
    B, S, d = x.shape
    assert d == cfg["d"]
    cap = k_cache.shape[2]
    c = _cfg_struct(cfg)
    ws = {n: _f64(weights[n]) for n in WEIGHT_NAMES}
    wstruct = _Weights(*[_p(ws[n]) for n in WEIGHT_NAMES])
    y = np.zeros((B, S, d), dtype=np.float64)
    M = B * S
    widths = {"n1": d, "q": cfg["H"] * cfg["d_head"], "k": cfg["n_kv"] * cfg["d_head"],
              "v": cfg["n_kv"] * cfg["d_head"], "o": cfg["H"] * cfg["d_head"], "h": d,
              "n2": d, "z": cfg["d_ff"]}
    st_arrays = {}
    st_ptr = None
    if stages:
        st_arrays = {n: np.zeros((M, widths[n]), dtype=np.float64) for n in STAGES}
        st_ptr = ctypes.pointer(_Stages(*[_p(st_arrays[n]) for n in STAGES]))
    if rows is not None:
        rarr = (ctypes.c_int * len(rows))(*[int(r) for r in rows])
        nrows = len(rows)
    else:
        rarr, nrows = None, 0
    rc = lib().orc_block_forward(ctypes.byref(c), B, S, int(start_pos), int(cap), _p(x),
                                 ctypes.byref(wstruct), _p(k_cache), _p(v_cache), _p(y),
                                 rarr, nrows, st_ptr)
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return y, st_arrays


def stack_forward(cfg: Dict, x, layers: Sequence[Dict], final_norm, start_pos: int,
                  caches: Sequence, hidden: bool = False):
    """Run a stack of blocks and the final RMSNorm (orc_stack_forward).

    layers: one weight dict per block (WEIGHT_NAMES).  caches: one (k, v) pair
    of float64 [B][n_kv][cap][d_head] arrays per block, updated in place.
    Returns (y, hidden) with hidden [n_layers][B][S][d] (each block's output)
    when asked for, else None.
    """
    x = _f64(x)
    B, S, d = x.shape
    L = len(layers)
    assert L >= 1 and len(caches) == L and d == cfg["d"]
    cap = caches[0][0].shape[2]
    for kc, vc in caches:
        assert kc.shape == vc.shape and kc.shape[2] == cap
        _p(kc), _p(vc)
    c = _cfg_struct(cfg)
    ws = [{n: _f64(lw[n]) for n in WEIGHT_NAMES} for lw in layers]
    warr = (_Weights * L)(*[_Weights(*[_p(w[n]) for n in WEIGHT_NAMES]) for w in ws])
    karr = (_dp * L)(*[_p(kc) for kc, _ in caches])
    varr = (_dp * L)(*[_p(vc) for _, vc in caches])
    g = _f64(final_norm)
    y = np.zeros((B, S, d), dtype=np.float64)
    hid = np.zeros((L, B, S, d), dtype=np.float64) if hidden else None
    rc = lib().orc_stack_forward(ctypes.byref(c), L, B, S, int(start_pos), int(cap), _p(x), warr,
                                 _p(g), karr, varr, _p(hid) if hidden else None, _p(y))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return y, hid


def _moe_struct(moe: Dict) -> "_MoeCfg":
    return _MoeCfg(int(moe["n_experts"]), int(moe["top_k"]), int(moe["d_ff_expert"]))


def moe_route(moe: Dict, n, router, force_sel=None):
    """Routing of one normalised row: returns (sel, wts, logits)."""
    n, r = _f64(n), _f64(router)
    E, K = int(moe["n_experts"]), int(moe["top_k"])
    sel = np.zeros(K, dtype=np.int32) if force_sel is None else np.array(force_sel, dtype=np.int32)
    wts = np.zeros(K)
    logits = np.zeros(E)
    rc = lib().orc_moe_route(ctypes.byref(_moe_struct(moe)), n.shape[-1], _p(n), _p(r),
                             sel.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), 0 if force_sel is None else 1,
                             _p(wts), _p(logits))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return sel, wts, logits


def moe_ffn(cfg: Dict, moe: Dict, n, weights: Dict, force_sel=None):
    """MoE FFN of one normalised row n [d] (shared expert = weights' w_gate /
    w_up / w_down).  Returns (out, sel, wts, logits)."""
    n = _f64(n)
    ws = {k: _f64(weights[k]) for k in ("w_gate", "w_up", "w_down") + MOE_WEIGHT_NAMES}
    wstruct = _Weights(*[(_p(ws[k]) if k in ws else None) for k in WEIGHT_NAMES])
    mstruct = _MoeWeights(*[_p(ws[k]) for k in MOE_WEIGHT_NAMES])
    E, K = int(moe["n_experts"]), int(moe["top_k"])
    sel = np.zeros(K, dtype=np.int32) if force_sel is None else np.array(force_sel, dtype=np.int32)
    wts, logits, out = np.zeros(K), np.zeros(E), np.zeros(cfg["d"])
    rc = lib().orc_moe_ffn(ctypes.byref(_cfg_struct(cfg)), ctypes.byref(_moe_struct(moe)), _p(n),
                           ctypes.byref(wstruct), ctypes.byref(mstruct),
                           sel.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), 0 if force_sel is None else 1,
                           _p(wts), _p(logits), _p(out))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return out, sel, wts, logits


def moe_block_forward(cfg: Dict, moe: Dict, x, weights: Dict, start_pos: int, k_cache: np.ndarray,
                      v_cache: np.ndarray, rows: Optional[Sequence[int]] = None, force_sel=None):
    """The block with the MoE FFN.  weights: the block's (its FFN is the
    shared expert) plus router / e_gate / e_up / e_down.  force_sel: optional
    [B*S][k] experts to use per row.  Returns (y, sel, wts, logits), per flat
    row; with `rows`, only those rows are meaningful."""
    x = _f64(x)
    B, S, d = x.shape
    cap = k_cache.shape[2]
    ws = {n: _f64(weights[n]) for n in WEIGHT_NAMES + MOE_WEIGHT_NAMES}
    wstruct = _Weights(*[_p(ws[n]) for n in WEIGHT_NAMES])
    mstruct = _MoeWeights(*[_p(ws[n]) for n in MOE_WEIGHT_NAMES])
    E, K = int(moe["n_experts"]), int(moe["top_k"])
    M = B * S
    if force_sel is None:
        sel = np.zeros((M, K), dtype=np.int32)
    else:
        sel = np.ascontiguousarray(np.asarray(force_sel, dtype=np.int32).reshape(M, K))
    wts = np.zeros((M, K))
    logits = np.zeros((M, E))
    y = np.zeros((B, S, d))
    if rows is not None:
        rarr = (ctypes.c_int * len(rows))(*[int(r) for r in rows])
        nrows = len(rows)
    else:
        rarr, nrows = None, 0
    rc = lib().orc_moe_block_forward(ctypes.byref(_cfg_struct(cfg)), ctypes.byref(_moe_struct(moe)), B, S,
                                     int(start_pos), int(cap), _p(x), ctypes.byref(wstruct),
                                     ctypes.byref(mstruct), _p(k_cache), _p(v_cache), _p(y), rarr, nrows,
                                     sel.ctypes.data_as(ctypes.POINTER(ctypes.c_int)),
                                     0 if force_sel is None else 1, _p(wts), _p(logits))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return y, sel, wts, logits


def cfg_of(w) -> Dict:
    """Oracle config dict from a workloads.BlockWorkload."""
    return {"d": w.d, "H": w.H, "n_kv": w.n_kv, "d_head": w.d_head, "d_ff": w.d_ff,
            "theta": w.theta, "eps": w.eps, "rope_half": w.rope_half, "rope_scaling": w.rope_scaling}


def empty_cache(w, cap: Optional[int] = None):
    cap = cap or w.capacity
    shape = (w.B, w.n_kv, cap, w.d_head)
    return np.zeros(shape, dtype=np.float64), np.zeros(shape, dtype=np.float64)


def run_workload(w, tensors: Dict, rows: Optional[Sequence[int]] = None, stages: bool = False):
    """Oracle forward of a generated workload: fills the pre-filled prefix, runs
    the block and returns (y, k_cache, v_cache, stages)."""
    kc, vc = empty_cache(w)
    if w.start_pos > 0:
        kc[:, :, : w.start_pos, :] = _f64(tensors["k_prefix"])
        vc[:, :, : w.start_pos, :] = _f64(tensors["v_prefix"])
    y, st = block_forward(cfg_of(w), tensors["x"], tensors, w.start_pos, kc, vc, rows=rows,
                          stages=stages)
    return y, kc, vc, st
