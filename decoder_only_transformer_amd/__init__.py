"""Python binding of libllama_block.so (the gfx950 Llama-block library).

Argument marshalling only: every step of the block runs in the library's HIP
kernels.  The names match the C ABI in include/llama_block.h.  Tensors are
torch tensors on the GPU; their data pointers and the current HIP stream are
handed to the library.  There is no fallback: if the library is missing, the
import of the entry points raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libllama_block.so")

LB_F32, LB_BF16 = 0, 1
LB_OPERANDS_AUTO, LB_OPERANDS_F16, LB_OPERANDS_BF16 = 0, 1, 2
LB_OK, LB_ERR_INVALID_ARG, LB_ERR_UNSUPPORTED, LB_ERR_OOM, LB_ERR_HIP = 0, 1, 2, 3, 4
STAGES = {"n1": 0, "q": 1, "o": 2, "h": 3, "n2": 4, "z": 5, "routed": 6}
ELEM_NAMES = {0: "f32", 1: "bf16", 2: "f16"}

MAX_RAGGED_BATCH = 64
EXPORTS = ("llama_block_init", "llama_block_forward", "llama_block_forward_ragged", "llama_block_destroy",
           "llama_block_status_string", "llama_block_last_error", "llama_block_stage_info",
           "llama_block_copy_stage", "llama_block_profile", "llama_block_profile_read",
           "llama_stack_init", "llama_stack_forward", "llama_stack_forward_device_pos",
           "llama_stack_graph_create", "llama_stack_graph_launch", "llama_stack_graph_destroy",
           "llama_stack_destroy", "llama_stack_num_layers", "llama_stack_last_error",
           "llama_moe_block_init", "llama_block_copy_routing", "llama_block_operand_type",
           "llama_stack_operand_type", "llama_block_forward_decode_static", "llama_block_footprint",
           "llama_block_device_bytes", "llama_stack_device_bytes")
MAX_STACK_LAYERS = 1024
STAGE_NAMES = ("rmsnorm_1", "qkv_rope_append", "attention", "o_proj_residual", "rmsnorm_2",
               "gate_up_swiglu", "down_residual")


class LbConfig(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("d_head", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32), ("rope_theta", ctypes.c_double),
                ("norm_eps", ctypes.c_double), ("dtype", ctypes.c_int),
                ("operands", ctypes.c_int), ("rope_layout", ctypes.c_int),
                ("rope_scale_factor", ctypes.c_double), ("rope_low_freq_factor", ctypes.c_double),
                ("rope_high_freq_factor", ctypes.c_double),
                ("rope_original_max_pos", ctypes.c_double)]


class LbWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm",
                                               "w_gate", "w_up", "w_down")]


class LbKVCache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("batch", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32)]


WEIGHT_NAMES = [f[0] for f in LbWeights._fields_]


class LbFootprint(ctypes.Structure):
    _fields_ = [("weights", ctypes.c_uint64), ("workspace", ctypes.c_uint64),
                ("init_staging", ctypes.c_uint64)]


class LbMoeConfig(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("d_ff_expert", ctypes.c_int32)]


class LbMoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("router", "w_gate", "w_up", "w_down")]


# names of the routed experts' tensors in weight dicts (the block's own FFN
# tensors are the shared expert)
MOE_WEIGHT_NAMES = {"router": "router", "w_gate": "e_gate", "w_up": "e_up", "w_down": "e_down"}


class LlamaBlockError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        L.llama_block_init.argtypes = [ctypes.POINTER(LbConfig), ctypes.POINTER(LbWeights),
                                       ctypes.POINTER(vp)]
        L.llama_block_init.restype = ctypes.c_int
        L.llama_block_forward.argtypes = [vp, vp, i32, i32, i32, ctypes.POINTER(LbKVCache), vp, vp]
        L.llama_block_forward.restype = ctypes.c_int
        L.llama_block_forward_ragged.argtypes = [vp, vp, i32, i32, ctypes.POINTER(ctypes.c_int32),
                                                 ctypes.POINTER(LbKVCache), vp, vp]
        L.llama_block_forward_ragged.restype = ctypes.c_int
        L.llama_block_forward_decode_static.argtypes = [vp, vp, i32, i32, ctypes.POINTER(LbKVCache), vp, vp]
        L.llama_block_forward_decode_static.restype = ctypes.c_int
        L.llama_block_destroy.argtypes = [vp]
        L.llama_block_destroy.restype = None
        L.llama_block_status_string.argtypes = [ctypes.c_int]
        L.llama_block_status_string.restype = ctypes.c_char_p
        L.llama_block_last_error.argtypes = [vp]
        L.llama_block_last_error.restype = ctypes.c_char_p
        L.llama_block_stage_info.argtypes = [vp, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                             ctypes.POINTER(ctypes.c_int64)]
        L.llama_block_stage_info.restype = ctypes.c_int
        L.llama_block_copy_stage.argtypes = [vp, ctypes.c_int, vp, ctypes.c_size_t, vp]
        L.llama_block_copy_stage.restype = ctypes.c_int
        L.llama_block_profile.argtypes = [vp, ctypes.c_uint32]
        L.llama_block_profile.restype = ctypes.c_int
        L.llama_block_profile_read.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.c_int,
                                               ctypes.POINTER(ctypes.c_int64)]
        L.llama_block_profile_read.restype = ctypes.c_int
        L.llama_moe_block_init.argtypes = [ctypes.POINTER(LbConfig), ctypes.POINTER(LbWeights),
                                           ctypes.POINTER(LbMoeConfig), ctypes.POINTER(LbMoeWeights),
                                           ctypes.POINTER(vp)]
        L.llama_moe_block_init.restype = ctypes.c_int
        L.llama_block_copy_routing.argtypes = [vp, vp, vp, vp, vp]
        L.llama_block_copy_routing.restype = ctypes.c_int
        kvp = ctypes.POINTER(LbKVCache)
        L.llama_stack_init.argtypes = [ctypes.POINTER(LbConfig), i32, ctypes.POINTER(LbWeights), vp,
                                       ctypes.POINTER(vp)]
        L.llama_stack_init.restype = ctypes.c_int
        L.llama_stack_forward.argtypes = [vp, vp, i32, i32, i32, ctypes.POINTER(ctypes.c_int32), kvp,
                                          vp, vp, vp]
        L.llama_stack_forward.restype = ctypes.c_int
        L.llama_stack_forward_device_pos.argtypes = [vp, vp, i32, i32, vp, i32, kvp, vp, vp, vp]
        L.llama_stack_forward_device_pos.restype = ctypes.c_int
        L.llama_stack_graph_create.argtypes = [vp, vp, i32, i32, vp, kvp, vp, ctypes.POINTER(vp)]
        L.llama_stack_graph_create.restype = ctypes.c_int
        L.llama_stack_graph_launch.argtypes = [vp, vp]
        L.llama_stack_graph_launch.restype = ctypes.c_int
        L.llama_stack_graph_destroy.argtypes = [vp]
        L.llama_stack_graph_destroy.restype = None
        L.llama_stack_destroy.argtypes = [vp]
        L.llama_stack_destroy.restype = None
        L.llama_stack_num_layers.argtypes = [vp]
        L.llama_stack_num_layers.restype = i32
        L.llama_block_operand_type.argtypes = [vp]
        L.llama_block_operand_type.restype = ctypes.c_int
        L.llama_stack_operand_type.argtypes = [vp]
        L.llama_stack_operand_type.restype = ctypes.c_int
        L.llama_block_footprint.argtypes = [ctypes.POINTER(LbConfig), i32, ctypes.POINTER(LbFootprint)]
        L.llama_block_footprint.restype = ctypes.c_int
        L.llama_block_device_bytes.argtypes = [vp]
        L.llama_block_device_bytes.restype = ctypes.c_uint64
        L.llama_stack_device_bytes.argtypes = [vp]
        L.llama_stack_device_bytes.restype = ctypes.c_uint64
        L.llama_stack_last_error.argtypes = [vp]
        L.llama_stack_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _check(handle, status: int, what: str):
    if status != LB_OK:
        L = lib()
        msg = L.llama_block_last_error(handle).decode() or L.llama_block_status_string(status).decode()
        raise LlamaBlockError(status, f"{what}: {msg}")


# ---- the C entry points, same names -------------------------------------------------

def llama_block_status_string(status: int) -> str:
    return lib().llama_block_status_string(status).decode()


def llama_block_last_error(handle=None) -> str:
    return lib().llama_block_last_error(handle).decode()


def llama_block_init(cfg: LbConfig, weights: Dict[str, "object"]) -> int:
    """cfg: LbConfig; weights: dict of device tensors named as LbWeights fields.
    Returns the opaque handle (an int).  Synchronous."""
    w = LbWeights(*[_ptr(weights[n]) for n in WEIGHT_NAMES])
    h = ctypes.c_void_p()
    st = lib().llama_block_init(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h))
    _check(None, st, "llama_block_init")
    return h.value


def llama_moe_block_init(cfg: LbConfig, weights: Dict[str, "object"], moe: Dict[str, int]) -> int:
    """A MoE block: weights as for llama_block_init (its FFN is the shared
    expert) plus the experts under the names of MOE_WEIGHT_NAMES' values;
    moe: n_experts, top_k, d_ff_expert."""
    w = LbWeights(*[_ptr(weights[n]) for n in WEIGHT_NAMES])
    ew = LbMoeWeights(*[_ptr(weights[MOE_WEIGHT_NAMES[f]]) for f, _ in LbMoeWeights._fields_])
    mc = LbMoeConfig(int(moe["n_experts"]), int(moe["top_k"]), int(moe["d_ff_expert"]))
    h = ctypes.c_void_p()
    st = lib().llama_moe_block_init(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(mc), ctypes.byref(ew),
                                    ctypes.byref(h))
    _check(None, st, "llama_moe_block_init")
    return h.value


def llama_block_copy_routing(handle: int, sel=None, weights=None, logits=None, stream=None) -> None:
    """Copy the last forward's routing into the given tensors (any may be None):
    sel int32 [rows][top_k], weights fp32 [rows][top_k], logits fp32 [rows][E]."""
    st = lib().llama_block_copy_routing(handle, _ptr(sel), _ptr(weights), _ptr(logits), _stream(stream))
    _check(handle, st, "llama_block_copy_routing")


def llama_block_forward(handle: int, x, start_pos: int, kv: Tuple, out, stream=None) -> None:
    """x, out: device tensors [B][S][d]; kv: (k_cache, v_cache) device tensors
    in the library's layout (see new_kv_cache).  Enqueued on `stream` (default:
    torch's current stream)."""
    k, v = kv
    B, S = int(x.shape[0]), int(x.shape[1])
    c = LbKVCache(_ptr(k), _ptr(v), int(k.shape[0]), int(k.shape[2]))
    st = lib().llama_block_forward(handle, _ptr(x), B, S, int(start_pos), ctypes.byref(c),
                                   _ptr(out), _stream(stream))
    _check(handle, st, "llama_block_forward")


def llama_block_forward_ragged(handle: int, x, start_pos, kv: Tuple, out, stream=None) -> None:
    """As llama_block_forward with one start position per sequence
    (start_pos: a sequence of len(x) ints, at most MAX_RAGGED_BATCH)."""
    k, v = kv
    B, S = int(x.shape[0]), int(x.shape[1])
    pos = [int(p) for p in start_pos]
    if len(pos) != B:
        raise ValueError(f"need one start position per sequence ({B}), got {len(pos)}")
    arr = (ctypes.c_int32 * B)(*pos)
    c = LbKVCache(_ptr(k), _ptr(v), int(k.shape[0]), int(k.shape[2]))
    st = lib().llama_block_forward_ragged(handle, _ptr(x), B, S, arr, ctypes.byref(c), _ptr(out),
                                          _stream(stream))
    _check(handle, st, "llama_block_forward_ragged")


def llama_block_forward_decode_static(handle: int, x, start_pos: int, kv: Tuple, out, stream=None) -> None:
    """One decode step (x, out: [B][1][d]) on the library's static scratch array
    instead of the handle's workspace; allocates nothing."""
    k, v = kv
    B, S = int(x.shape[0]), int(x.shape[1])
    if S != 1:
        raise ValueError(f"a decode step takes one token per sequence, got seq_len {S}")
    c = LbKVCache(_ptr(k), _ptr(v), int(k.shape[0]), int(k.shape[2]))
    st = lib().llama_block_forward_decode_static(handle, _ptr(x), B, int(start_pos), ctypes.byref(c),
                                                 _ptr(out), _stream(stream))
    _check(handle, st, "llama_block_forward_decode_static")


def llama_block_destroy(handle: int) -> None:
    if handle:
        lib().llama_block_destroy(handle)


def llama_block_operand_type(handle: int) -> str:
    """Operand type of the handle's matrix products: "f32", "f16" or "bf16"."""
    return ELEM_NAMES[lib().llama_block_operand_type(handle)]


def llama_stack_operand_type(handle: int) -> str:
    return ELEM_NAMES[lib().llama_stack_operand_type(handle)]


def llama_block_footprint(cfg: LbConfig, n_layers: int = 0) -> dict:
    """Device bytes of a block (n_layers 0) or a stack of n_layers blocks,
    from the config alone: {"weights", "workspace", "init_staging"}."""
    fp = LbFootprint()
    st = lib().llama_block_footprint(ctypes.byref(cfg), int(n_layers), ctypes.byref(fp))
    _check(None, st, "llama_block_footprint")
    return {"weights": fp.weights, "workspace": fp.workspace, "init_staging": fp.init_staging}


def llama_block_device_bytes(handle: int) -> int:
    return int(lib().llama_block_device_bytes(handle))


def llama_stack_device_bytes(handle: int) -> int:
    return int(lib().llama_stack_device_bytes(handle))


def llama_block_stage_info(handle: int, stage: str) -> Tuple[str, int]:
    e, cols = ctypes.c_int(), ctypes.c_int64()
    st = lib().llama_block_stage_info(handle, STAGES[stage], ctypes.byref(e), ctypes.byref(cols))
    _check(handle, st, "llama_block_stage_info")
    return ELEM_NAMES[e.value], cols.value


def llama_block_copy_stage(handle: int, stage: str, dst, stream=None) -> None:
    nbytes = dst.numel() * dst.element_size()
    st = lib().llama_block_copy_stage(handle, STAGES[stage], _ptr(dst), nbytes, _stream(stream))
    _check(handle, st, "llama_block_copy_stage")


PROFILE_ALL = (1 << len(STAGE_NAMES)) - 1


def llama_block_profile(handle: int, stages=PROFILE_ALL) -> None:
    """Time the given stages on every following forward: a bit mask, or an
    iterable of stage names; 0 / False / empty stops."""
    if stages is True:
        stages = PROFILE_ALL
    if isinstance(stages, (list, tuple, set, frozenset)):
        stages = sum(1 << STAGE_NAMES.index(n) for n in stages)
    _check(handle, lib().llama_block_profile(handle, int(stages)), "llama_block_profile")


def llama_block_profile_read(handle: int) -> Tuple[Dict[str, float], int]:
    """Summed milliseconds per stage since profiling was enabled, and the number
    of profiled forwards."""
    arr = (ctypes.c_double * len(STAGE_NAMES))()
    calls = ctypes.c_int64()
    st = lib().llama_block_profile_read(handle, arr, len(STAGE_NAMES), ctypes.byref(calls))
    _check(handle, st, "llama_block_profile_read")
    return {n: arr[i] for i, n in enumerate(STAGE_NAMES)}, calls.value


def _check_stack(handle, status: int, what: str):
    if status != LB_OK:
        L = lib()
        msg = L.llama_stack_last_error(handle).decode() or L.llama_block_status_string(status).decode()
        raise LlamaBlockError(status, f"{what}: {msg}")


def _kv_array(kv_list):
    arr = (LbKVCache * len(kv_list))()
    for i, (k, v) in enumerate(kv_list):
        arr[i] = LbKVCache(_ptr(k), _ptr(v), int(k.shape[0]), int(k.shape[2]))
    return arr


def llama_stack_init(cfg: LbConfig, layers, final_norm) -> int:
    """layers: one dict of device tensors per block (LbWeights names);
    final_norm: device tensor [d_model].  Returns the handle.  Synchronous."""
    n = len(layers)
    arr = (LbWeights * max(n, 1))()
    for i, w in enumerate(layers):
        arr[i] = LbWeights(*[_ptr(w[nm]) for nm in WEIGHT_NAMES])
    h = ctypes.c_void_p()
    st = lib().llama_stack_init(ctypes.byref(cfg), n, arr, _ptr(final_norm), ctypes.byref(h))
    _check_stack(None, st, "llama_stack_init")
    return h.value


def llama_stack_forward(handle: int, x, start_pos, kv_list, out, hidden=None, stream=None) -> None:
    """start_pos: one int, or one per sequence; kv_list: one (k, v) per block;
    hidden: optional device tensor [n_layers][B][S][d]."""
    B, S = int(x.shape[0]), int(x.shape[1])
    if hasattr(start_pos, "__len__"):
        pos = [int(p) for p in start_pos]
        if len(pos) != B:
            raise ValueError(f"need one start position per sequence ({B}), got {len(pos)}")
        starts, base = (ctypes.c_int32 * B)(*pos), 0
    else:
        starts, base = None, int(start_pos)
    st = lib().llama_stack_forward(handle, _ptr(x), B, S, base, starts, _kv_array(kv_list), _ptr(out),
                                   _ptr(hidden), _stream(stream))
    _check_stack(handle, st, "llama_stack_forward")


def llama_stack_forward_device_pos(handle: int, x, positions, advance: bool, kv_list, out, hidden=None,
                                   stream=None) -> None:
    """positions: int32 device tensor [B], read (and with advance, moved on by
    S) by the kernels."""
    B, S = int(x.shape[0]), int(x.shape[1])
    st = lib().llama_stack_forward_device_pos(handle, _ptr(x), B, S, _ptr(positions), 1 if advance else 0,
                                              _kv_array(kv_list), _ptr(out), _ptr(hidden), _stream(stream))
    _check_stack(handle, st, "llama_stack_forward_device_pos")


def llama_stack_graph_create(handle: int, x, positions, kv_list, out) -> int:
    B, S = int(x.shape[0]), int(x.shape[1])
    g = ctypes.c_void_p()
    st = lib().llama_stack_graph_create(handle, _ptr(x), B, S, _ptr(positions), _kv_array(kv_list),
                                        _ptr(out), ctypes.byref(g))
    _check_stack(handle, st, "llama_stack_graph_create")
    return g.value


def llama_stack_graph_launch(graph: int, stream=None, handle=None) -> None:
    st = lib().llama_stack_graph_launch(graph, _stream(stream))
    _check_stack(handle, st, "llama_stack_graph_launch")


def llama_stack_graph_destroy(graph: int) -> None:
    if graph:
        lib().llama_stack_graph_destroy(graph)


def llama_stack_destroy(handle: int) -> None:
    if handle:
        lib().llama_stack_destroy(handle)


def llama_stack_num_layers(handle: int) -> int:
    return int(lib().llama_stack_num_layers(handle))


def llama_stack_last_error(handle=None) -> str:
    return lib().llama_stack_last_error(handle).decode()


# ---- small conveniences (allocation / argument packing only) ----------------------------

def make_config(d_model, n_heads, n_kv_heads, d_head, d_ff, max_tokens, max_seq_len, rope_theta,
                norm_eps, dtype: str, operands: str = "auto", rope_half: bool = False,
                rope_scaling=None) -> LbConfig:
    """rope_scaling: None or (factor, low_freq_factor, high_freq_factor, original_max_pos)."""
    sc = rope_scaling or (0.0, 0.0, 0.0, 0.0)
    return LbConfig(d_model, n_heads, n_kv_heads, d_head, d_ff, max_tokens, max_seq_len,
                    float(rope_theta), float(norm_eps), {"f32": LB_F32, "bf16": LB_BF16}[dtype],
                    {"auto": LB_OPERANDS_AUTO, "f16": LB_OPERANDS_F16,
                     "bf16": LB_OPERANDS_BF16}[operands], 1 if rope_half else 0,
                    float(sc[0]), float(sc[1]), float(sc[2]), float(sc[3]))


def new_kv_cache(batch: int, n_kv: int, max_seq_len: int, d_head: int, dtype, device="cuda",
                 fill: Optional[float] = 0.0):
    """Allocate (k, v) in the library's cache layout: [B][n_kv][max_seq][d_head] each."""
    import torch
    k = torch.empty((batch, n_kv, max_seq_len, d_head), dtype=dtype, device=device)
    v = torch.empty((batch, n_kv, max_seq_len, d_head), dtype=dtype, device=device)
    if fill is not None:
        k.fill_(fill)
        v.fill_(fill)
    return k, v


class LlamaBlock:
    """Owns one library handle."""

    def __init__(self, cfg: LbConfig, weights: Dict[str, "object"]):
        self.cfg = cfg
        self.handle = llama_block_init(cfg, weights)

    def forward(self, x, start_pos, kv, out, stream=None):
        """start_pos: one int for every sequence, or one per sequence (ragged)."""
        if not hasattr(start_pos, "__len__"):
            llama_block_forward(self.handle, x, int(start_pos), kv, out, stream)
        else:
            llama_block_forward_ragged(self.handle, x, start_pos, kv, out, stream)
        return out

    @property
    def operand_type(self) -> str:
        return llama_block_operand_type(self.handle)

    @property
    def device_bytes(self) -> int:
        return llama_block_device_bytes(self.handle)

    def stage(self, name: str, rows: int):
        import torch
        elem, cols = llama_block_stage_info(self.handle, name)
        dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[elem]
        dst = torch.empty((rows, cols), dtype=dt, device="cuda")
        llama_block_copy_stage(self.handle, name, dst)
        return dst

    def close(self):
        if self.handle:
            llama_block_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class LlamaStack:
    """Owns one stack handle (and the graphs made from it)."""

    def __init__(self, cfg: LbConfig, layers, final_norm):
        self.cfg = cfg
        self.handle = llama_stack_init(cfg, layers, final_norm)
        self.graphs = []

    @property
    def n_layers(self) -> int:
        return llama_stack_num_layers(self.handle)

    @property
    def device_bytes(self) -> int:
        return llama_stack_device_bytes(self.handle)

    def forward(self, x, start_pos, kv_list, out, hidden=None, stream=None):
        llama_stack_forward(self.handle, x, start_pos, kv_list, out, hidden, stream)
        return out

    def forward_device_pos(self, x, positions, kv_list, out, advance=True, hidden=None, stream=None):
        llama_stack_forward_device_pos(self.handle, x, positions, advance, kv_list, out, hidden, stream)
        return out

    def capture(self, x, positions, kv_list, out) -> "StackGraph":
        g = StackGraph(self, llama_stack_graph_create(self.handle, x, positions, kv_list, out))
        self.graphs.append(g)
        return g

    def close(self):
        for g in self.graphs:
            g.close()
        self.graphs = []
        if self.handle:
            llama_stack_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class StackGraph:
    """A captured step of a stack: launch() replays it on a stream."""

    def __init__(self, stack: LlamaStack, graph: int):
        self.stack = stack
        self.graph = graph

    def launch(self, stream=None):
        llama_stack_graph_launch(self.graph, stream, self.stack.handle)

    def close(self):
        if self.graph:
            llama_stack_graph_destroy(self.graph)
            self.graph = None


class LlamaMoeBlock(LlamaBlock):
    """A block whose FFN is a mixture of experts with a shared expert."""

    def __init__(self, cfg: LbConfig, weights: Dict[str, "object"], moe: Dict[str, int]):
        self.cfg = cfg
        self.moe = dict(moe)
        self.handle = llama_moe_block_init(cfg, weights, moe)

    def routing(self, rows: int):
        """(sel, weights, logits) of the last forward's `rows` token rows, on the device."""
        import torch
        K, E = self.moe["top_k"], self.moe["n_experts"]
        sel = torch.empty((rows, K), dtype=torch.int32, device="cuda")
        wts = torch.empty((rows, K), dtype=torch.float32, device="cuda")
        lg = torch.empty((rows, E), dtype=torch.float32, device="cuda")
        llama_block_copy_routing(self.handle, sel, wts, lg)
        return sel, wts, lg
