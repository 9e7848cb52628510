"""The C-ABI library on the CPU: it loads, exports every function that
include/llama_block.h declares, its structs match the binding's ctypes layout,
and argument validation rejects bad configs before any device call.  No
compute is launched here."""
import ctypes
import os
import re
import subprocess

import pytest

import decoder_only_transformer_amd as lbmod

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "llama_block.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(llama_(?:block|stack|moe)_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(lbmod.EXPORTS), names
    L = lbmod.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", lbmod.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (\w+)", out))
    for n in names:
        assert n in exported, n


def test_struct_layouts_match_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text("""
#include <stdio.h>
#include <stddef.h>
#include "llama_block.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu\\n", sizeof(lb_config), offsetof(lb_config, rope_theta),
         offsetof(lb_config, norm_eps), offsetof(lb_config, dtype), offsetof(lb_config, operands),
         sizeof(lb_weights));
  printf("%zu %zu %zu\\n", sizeof(lb_kv_cache), offsetof(lb_kv_cache, batch), offsetof(lb_kv_cache, max_seq_len));
  printf("%zu %zu\\n", sizeof(lb_footprint), offsetof(lb_footprint, init_staging));
  return 0;
}
""")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    a, b, c = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")[:3]
    C = lbmod.LbConfig
    want_a = [ctypes.sizeof(C), C.rope_theta.offset, C.norm_eps.offset, C.dtype.offset,
              C.operands.offset, ctypes.sizeof(lbmod.LbWeights)]
    assert [int(v) for v in a.split()] == want_a
    K = lbmod.LbKVCache
    assert [int(v) for v in b.split()] == [ctypes.sizeof(K), K.batch.offset, K.max_seq_len.offset]
    F = lbmod.LbFootprint
    assert [int(v) for v in c.split()] == [ctypes.sizeof(F), F.init_staging.offset]


def _fake_weights():
    # non-NULL pointers that are never dereferenced: validation fails first
    return lbmod.LbWeights(*[0x1000 + 0x100 * i for i in range(9)])


@pytest.mark.parametrize("kw,status", [
    (dict(d_model=65), lbmod.LB_ERR_INVALID_ARG),              # d != H * d_head
    (dict(n_kv_heads=3), lbmod.LB_ERR_INVALID_ARG),            # H % n_kv != 0
    (dict(d_head=15, d_model=60), lbmod.LB_ERR_INVALID_ARG),   # odd d_head
    (dict(d_ff=0), lbmod.LB_ERR_INVALID_ARG),
    (dict(max_tokens=0), lbmod.LB_ERR_INVALID_ARG),
    (dict(rope_theta=0.0), lbmod.LB_ERR_INVALID_ARG),
    (dict(norm_eps=-1.0), lbmod.LB_ERR_INVALID_ARG),
    (dict(dtype=7), lbmod.LB_ERR_INVALID_ARG),
    (dict(dtype=lbmod.LB_BF16), lbmod.LB_ERR_UNSUPPORTED),     # d_head 16 in bf16
    (dict(d_head=12, d_model=48), lbmod.LB_ERR_UNSUPPORTED),   # fp32 d_head % 8
])
def test_init_rejects_invalid_config(kw, status):
    base = dict(d_model=64, n_heads=4, n_kv_heads=2, d_head=16, d_ff=176, max_tokens=16,
                max_seq_len=16, rope_theta=1e4, norm_eps=1e-5, dtype=lbmod.LB_F32,
                operands=lbmod.LB_OPERANDS_AUTO)
    base.update(kw)
    cfg = lbmod.LbConfig(**base)
    h = ctypes.c_void_p()
    st = lbmod.lib().llama_block_init(ctypes.byref(cfg), ctypes.byref(_fake_weights()), ctypes.byref(h))
    assert st == status
    assert h.value is None
    assert lbmod.llama_block_last_error(None) != ""


def test_init_rejects_null_pointers():
    cfg = lbmod.make_config(64, 4, 2, 16, 176, 16, 16, 1e4, 1e-5, "f32")
    w = _fake_weights()
    w.wo = None
    h = ctypes.c_void_p()
    L = lbmod.lib()
    assert L.llama_block_init(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h)) == lbmod.LB_ERR_INVALID_ARG
    assert L.llama_block_init(None, ctypes.byref(w), ctypes.byref(h)) == lbmod.LB_ERR_INVALID_ARG
    assert L.llama_block_forward(None, None, 1, 1, 0, None, None, None) == lbmod.LB_ERR_INVALID_ARG


def test_status_strings():
    for s in range(5):
        assert lbmod.llama_block_status_string(s)


def test_stack_init_rejects_bad_arguments_before_any_device_call():
    L = lbmod.lib()
    cfg = lbmod.make_config(64, 4, 2, 16, 176, 16, 16, 1e4, 1e-5, "f32")
    arr = (lbmod.LbWeights * 3)(_fake_weights(), _fake_weights(), _fake_weights())
    h = ctypes.c_void_p()
    gain = ctypes.c_void_p(0x9000)
    for n in (0, -1, lbmod.MAX_STACK_LAYERS + 1):
        assert L.llama_stack_init(ctypes.byref(cfg), n, arr, gain, ctypes.byref(h)) == lbmod.LB_ERR_INVALID_ARG
        assert h.value is None
        assert "n_layers" in lbmod.llama_stack_last_error(None)
    assert L.llama_stack_init(ctypes.byref(cfg), 3, arr, None, ctypes.byref(h)) == lbmod.LB_ERR_INVALID_ARG
    arr[2].w_up = None
    assert L.llama_stack_init(ctypes.byref(cfg), 3, arr, gain, ctypes.byref(h)) == lbmod.LB_ERR_INVALID_ARG
    assert "block 2" in lbmod.llama_stack_last_error(None)
    bad = lbmod.make_config(65, 4, 2, 16, 176, 16, 16, 1e4, 1e-5, "f32")
    assert L.llama_stack_init(ctypes.byref(bad), 2, arr, gain, ctypes.byref(h)) == lbmod.LB_ERR_INVALID_ARG
    assert h.value is None


def test_stack_calls_reject_null_handles():
    L = lbmod.lib()
    assert L.llama_stack_forward(None, None, 1, 1, 0, None, None, None, None, None) == lbmod.LB_ERR_INVALID_ARG
    assert L.llama_stack_forward_device_pos(None, None, 1, 1, None, 1, None, None, None, None) == \
        lbmod.LB_ERR_INVALID_ARG
    g = ctypes.c_void_p()
    assert L.llama_stack_graph_create(None, None, 1, 1, None, None, None, ctypes.byref(g)) == \
        lbmod.LB_ERR_INVALID_ARG
    assert L.llama_stack_graph_launch(None, None) == lbmod.LB_ERR_INVALID_ARG
    assert L.llama_stack_num_layers(None) == 0
    L.llama_stack_destroy(None)
    L.llama_stack_graph_destroy(None)


def test_moe_init_rejects_bad_arguments_before_any_device_call():
    L = lbmod.lib()
    cfg = lbmod.make_config(512, 8, 2, 64, 1024, 16, 64, 1e4, 1e-5, "bf16")
    w = _fake_weights()
    ew = lbmod.LbMoeWeights(0x5000, 0x6000, 0x7000, 0x8000)
    h = ctypes.c_void_p()
    for (E, K, fe) in ((0, 1, 64), (257, 1, 64), (8, 0, 64), (8, 9, 64), (4, 5, 64), (8, 2, 0)):
        mc = lbmod.LbMoeConfig(E, K, fe)
        st = L.llama_moe_block_init(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(mc), ctypes.byref(ew),
                                    ctypes.byref(h))
        assert st == lbmod.LB_ERR_INVALID_ARG, (E, K, fe)
        assert h.value is None
    mc = lbmod.LbMoeConfig(8, 2, 96)   # d_ff_expert not a multiple of 64
    assert L.llama_moe_block_init(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(mc), ctypes.byref(ew),
                                  ctypes.byref(h)) == lbmod.LB_ERR_UNSUPPORTED
    f32 = lbmod.make_config(64, 4, 2, 16, 176, 16, 16, 1e4, 1e-5, "f32")
    mc = lbmod.LbMoeConfig(8, 2, 64)
    assert L.llama_moe_block_init(ctypes.byref(f32), ctypes.byref(w), ctypes.byref(mc), ctypes.byref(ew),
                                  ctypes.byref(h)) == lbmod.LB_ERR_UNSUPPORTED
    ew.w_up = None
    assert L.llama_moe_block_init(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(mc), ctypes.byref(ew),
                                  ctypes.byref(h)) == lbmod.LB_ERR_INVALID_ARG
    assert L.llama_block_copy_routing(None, None, None, None, None) == lbmod.LB_ERR_INVALID_ARG


def _bytes_of_weights(d, H, n_kv, dh, dff, elem):
    """Bytes of one block's weights as the pages size them: Wq [H dh x d],
    Wk and Wv [n_kv dh x d], Wo [d x H dh], gate and up [d_ff x d], down
    [d x d_ff] ("Full Llama 3 transformer block", How it works), one copy in
    the operand type, plus the two gains in fp32."""
    mats = H * dh * d + 2 * n_kv * dh * d + d * H * dh + 3 * dff * d
    return mats * elem + 2 * d * 4


def test_footprint_holds_one_weight_copy_per_block():
    """8B width (d 4096, 32/8 heads of 128, d_ff 14336): one packed copy of
    the weights, 436,207,616 bytes of matrices, not two; an fp32 block holds
    4 bytes an element."""
    cfg = lbmod.make_config(4096, 32, 8, 128, 14336, 4096, 4096, 5e5, 1e-5, "bf16")
    fp = lbmod.llama_block_footprint(cfg)
    assert fp["weights"] == _bytes_of_weights(4096, 32, 8, 128, 14336, 2)
    assert fp["weights"] - 2 * 4096 * 4 == 436_207_616
    # staging of init: the largest matrix, gate/up [2 d_ff x d]
    assert fp["init_staging"] == 2 * 14336 * 4096 * 2
    small = lbmod.make_config(64, 4, 2, 16, 176, 16, 16, 1e4, 1e-5, "f32")
    fp32 = lbmod.llama_block_footprint(small)
    assert fp32["weights"] == _bytes_of_weights(64, 4, 2, 16, 176, 4)
    assert fp32["init_staging"] == 0


def test_footprint_of_a_70b_width_stack_fits_one_gpu():
    """80 blocks of the 70B width (d 8192, 64/8 heads of 128, d_ff 28672),
    "Full Llama 3 transformer block", How it works, with a workspace for 8192
    token rows and the KV caches of 8 sequences of 8192 positions: the whole
    model's blocks fit in one MI355X's 288 GB, and a stack's weights are
    exactly n_layers blocks' worth."""
    cfg = lbmod.make_config(8192, 64, 8, 128, 28672, 8192, 8192, 5e5, 1e-5, "bf16")
    one = lbmod.llama_block_footprint(cfg, 1)
    fp = lbmod.llama_block_footprint(cfg, 80)
    per_block = _bytes_of_weights(8192, 64, 8, 128, 28672, 2)
    assert fp["weights"] == 80 * per_block == 80 * one["weights"]
    assert fp["workspace"] == one["workspace"]
    # a stack adds the final gain and two activation buffers to a block's workspace
    blk = lbmod.llama_block_footprint(cfg, 0)
    assert fp["workspace"] == blk["workspace"] + 8192 * 4 + 2 * 8192 * 8192 * 2
    kv = 80 * 2 * 8 * 8192 * 8 * 128 * 2
    total = fp["weights"] + fp["workspace"] + fp["init_staging"] + kv
    assert total < 288e9, total / 1e9
    # two copies of the weights would not have fit beside the same caches
    assert 2 * fp["weights"] + fp["workspace"] + kv > 288e9


def test_footprint_rejects_what_init_rejects():
    L = lbmod.lib()
    bad = lbmod.make_config(65, 4, 2, 16, 176, 16, 16, 1e4, 1e-5, "f32")
    out = lbmod.LbFootprint()
    assert L.llama_block_footprint(ctypes.byref(bad), 0, ctypes.byref(out)) == lbmod.LB_ERR_INVALID_ARG
    assert "d_model" in lbmod.llama_block_last_error(None)
    ok = lbmod.make_config(64, 4, 2, 16, 176, 16, 16, 1e4, 1e-5, "f32")
    for n in (-1, lbmod.MAX_STACK_LAYERS + 1):
        assert L.llama_block_footprint(ctypes.byref(ok), n, ctypes.byref(out)) == lbmod.LB_ERR_INVALID_ARG
    assert L.llama_block_footprint(None, 0, ctypes.byref(out)) == lbmod.LB_ERR_INVALID_ARG
    assert L.llama_block_footprint(ctypes.byref(ok), 0, None) == lbmod.LB_ERR_INVALID_ARG
    assert L.llama_block_device_bytes(None) == 0
    assert L.llama_stack_device_bytes(None) == 0


def test_stage_numbers_match_header():
    """The binding's stage names carry the header's lb_stage values."""
    text = open(HEADER).read()
    body = re.search(r"typedef enum \{([^}]*)\} lb_stage;", text).group(1)
    header = {m.group(1).lower(): int(m.group(2)) for m in re.finditer(r"LB_STAGE_(\w+)\s*=\s*(\d+)", body)}
    assert header == lbmod.STAGES
