"""Pins for the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: figures the
pages print (tests/golden/page_figures.json), closed forms, invariants, special
cases that reduce to a library routine, or brute force on tiny inputs.  The
planted-mistake check at the end shows that a plausible slip in the oracle's
arithmetic is caught.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
import workloads

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def g(key):
    return GOLD[key]["value"]


def rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- RMSNorm ----

def test_rmsnorm_unit_gain_closed_form():
    """Unit gain: rms(out) = sqrt(ms / (ms + eps)); with eps = 0 exactly 1."""
    r = rng(1)
    for d, scale in [(64, 1.0), (576, 3.0), (4096, 0.01)]:
        v = r.normal(0, scale, d)
        ms = np.mean(v * v)
        for eps in (1e-5, 1e-6, 0.0):
            out = oracle.rms_norm(v, np.ones(d), eps)
            got = math.sqrt(np.mean(out * out))
            want = math.sqrt(ms / (ms + eps))
            assert abs(got - want) <= 1e-14 * want, (d, eps, got, want)
            # no centring: the output is a positive multiple of the input
            assert np.all(np.sign(out) == np.sign(v))


def test_rmsnorm_matches_torch_rms_norm():
    """Library special case: torch's F.rms_norm (named on the page "From GPT-2 to
    Llama", The norm stops centring) in fp64, with a learned gain."""
    r = rng(2)
    for d in (64, 576, 1000):
        v = r.normal(0, 1.7, (5, d))
        gain = r.normal(1, 0.1, d)
        want = F.rms_norm(torch.from_numpy(v), (d,), torch.from_numpy(gain), eps=1e-5).numpy()
        for i in range(5):
            got = oracle.rms_norm(v[i], gain, 1e-5)
            np.testing.assert_allclose(got, want[i], rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------- projections ----

def test_linear_matches_numpy_matmul():
    r = rng(3)
    for n_out, n_in in [(128, 64), (7, 176), (960, 576)]:
        w = r.normal(0, 0.02, (n_out, n_in))
        v = r.normal(0, 1, n_in)
        np.testing.assert_allclose(oracle.linear(v, w), w @ v, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------- RoPE ----

def _score(q, k, m, n, theta):
    return float(oracle.rope(q, m, theta) @ oracle.rope(k, n, theta))


def test_rope_relative_position_invariance():
    """"From GPT-2 to Llama", Positions become a rotation: the rotated score
    depends only on m - n (-13.4724 at (10,3) vs -13.4723 at (1010,1003)), and
    moving one step closer changes it (-10.786 at (10,4))."""
    figs = g("rope_score_invariance")
    assert abs(figs["m10_n3"] - figs["m1010_n1003"]) < 2e-4
    assert abs(figs["m10_n3"] - figs["m10_n4"]) > 1.0
    r = rng(4)
    for theta, dh in [(1e5, 64), (5e5, 128), (1e4, 16)]:
        for trial in range(3):
            q, k = r.normal(0, 1, dh), r.normal(0, 1, dh)
            base = _score(q, k, 10, 3, theta)
            for delta in (1, 1000, 5000, 100000):
                assert abs(_score(q, k, 10 + delta, 3 + delta, theta) - base) <= 1e-11 * (1 + abs(base))
            # one step closer is a different score
            assert abs(_score(q, k, 10, 4, theta) - base) > 1e-6


def _omegas(dh, theta):
    """Read each pair's angular speed back from the oracle: the turn of a unit
    vector in pair i over one position."""
    om = []
    for i in range(dh // 2):
        e = np.zeros(dh)
        e[2 * i] = 1.0
        r = oracle.rope(e, 1, theta)
        om.append(math.atan2(r[2 * i + 1], r[2 * i]))
    return np.array(om)


def test_rope_pair_periods_match_page():
    """"From GPT-2 to Llama", Positions become a rotation: with base 100 000 and
    heads of 64, the fastest pair turns once every 6.3 positions and the slowest
    once every ~438 000."""
    om = _omegas(64, 1e5)
    periods = 2 * math.pi / om
    assert round(periods[0], 1) == g("smollm2_rope_fastest_period_positions")
    assert abs(periods[-1] - g("smollm2_rope_slowest_period_positions")) / 438000 < 0.005
    # speeds fall monotonically from the first pair to the last (geometric schedule)
    assert np.all(np.diff(periods) > 0)
    ratios = om[1:] / om[:-1]
    np.testing.assert_allclose(ratios, ratios[0], rtol=1e-12)


def test_rope_is_complex_rotation_of_adjacent_pairs():
    """"Mini Llama 2 Implementation", Rotary positional embeddings: adjacent
    dimensions (2i, 2i+1) are the real and imaginary parts of one complex number,
    turned by e^(i m w_i).  Also: position 0 is the identity and each pair keeps
    its length."""
    dh, theta = 128, 5e5
    om = _omegas(dh, theta)
    r = rng(5)
    v = r.normal(0, 1, dh)
    np.testing.assert_array_equal(oracle.rope(v, 0, theta), v)
    for m in (1, 7, 2047, 8191):
        got = oracle.rope(v, m, theta)
        z = (v[0::2] + 1j * v[1::2]) * np.exp(1j * m * om)
        np.testing.assert_allclose(got[0::2], z.real, rtol=0, atol=1e-9)
        np.testing.assert_allclose(got[1::2], z.imag, rtol=0, atol=1e-9)
        np.testing.assert_allclose(np.hypot(got[0::2], got[1::2]), np.hypot(v[0::2], v[1::2]),
                                   rtol=1e-13)


# ------------------------------------------------------------ RoPE variants ----

_L31 = (8.0, 1.0, 4.0, 8192.0)  # scale, low and high frequency factors, original length


def _cfg(dh, theta, half=False, scaling=None):
    return {"d": dh, "H": 1, "n_kv": 1, "d_head": dh, "d_ff": 4, "theta": theta, "eps": 1e-5,
            "rope_half": half, "rope_scaling": scaling}


def test_rope_default_settings_are_the_plain_rotation():
    """The block's RoPE with interleaved pairs and no frequency scaling is the
    pinned plain rotation above, bit for bit."""
    r = rng(21)
    for dh, theta in [(16, 1e4), (64, 1e5), (128, 5e5)]:
        v = r.normal(0, 1, dh)
        for m in (0, 1, 37, 8191):
            np.testing.assert_array_equal(oracle.rope_cfg(v, m, _cfg(dh, theta)), oracle.rope(v, m, theta))


def test_rope_half_layout_is_a_permutation_of_interleaved():
    """"From GPT-2 to Llama", Positions become a rotation: the rotate_half form
    pairs dimension i with i + d_head/2; laid out so that those two sit side by
    side it is the interleaved rotation, bit for bit (both turn pair i by the
    same angle)."""
    r = rng(22)
    for dh, theta, sc in [(64, 1e5, None), (128, 5e5, _L31)]:
        half = dh // 2
        perm = np.empty(dh, dtype=int)            # interleaved slot -> half-layout index
        perm[0::2] = np.arange(half)
        perm[1::2] = np.arange(half) + half
        v = r.normal(0, 1, dh)
        for m in (0, 3, 999, 8191):
            got = oracle.rope_cfg(v, m, _cfg(dh, theta, half=True, scaling=sc))
            want_inter = oracle.rope_cfg(v[perm], m, _cfg(dh, theta, half=False, scaling=sc))
            np.testing.assert_array_equal(got[perm], want_inter)


def test_rope_llama31_scaling_counts_match_page():
    """"From GPT-2 to Llama", Positions become a rotation: Llama 3.1 8B (heads
    of 128, so 64 pairs, original length 8192) slows its 29 slowest pairs by a
    factor of 8, leaves its 29 fastest alone and blends the six between."""
    dh, theta = 128, 5e5
    base = np.array([oracle.rope_freq(_cfg(dh, theta), i) for i in range(dh // 2)])
    scaled = np.array([oracle.rope_freq(_cfg(dh, theta, scaling=_L31), i) for i in range(dh // 2)])
    same = np.sum(scaled == base)
    slowed = np.sum(scaled == base / 8.0)
    between = np.sum((scaled < base) & (scaled > base / 8.0))
    assert (same, slowed, between) == (29, 29, 6), (same, slowed, between)
    # the fast pairs are the first ones, the slowed ones the last
    assert np.all(scaled[:29] == base[:29]) and np.all(scaled[-29:] == base[-29:] / 8.0)


def test_rope_llama31_blend_meets_both_classes():
    """The blended speeds join the unchanged and the slowed classes without a
    jump: sweeping the base continuously moves pairs across the class
    boundaries, and the scaled speed changes only as much as the base does."""
    dh = 128
    i = 32
    prev = None
    for theta in np.geomspace(1e4, 1e7, 4001):
        base = oracle.rope_freq(_cfg(dh, theta), i)
        sc = oracle.rope_freq(_cfg(dh, theta, scaling=_L31), i)
        assert base / 8.0 - 1e-15 <= sc <= base + 1e-15
        if prev is not None:
            # neighbouring bases differ by < 0.5 %, so must the scaled speeds
            assert abs(sc / prev - 1.0) < 0.02, (theta, sc, prev)
        prev = sc


def test_rope_llama31_speeds_keep_their_order():
    """Slowing the slow pairs and blending the six between keeps the pairs in
    order: every scaled speed is below the one before it (pair i + 1 turns
    slower than pair i, as without scaling), across both class boundaries."""
    for dh, theta in ((128, 5e5), (64, 1e5), (128, 1e4)):
        scaled = np.array([oracle.rope_freq(_cfg(dh, theta, scaling=_L31), i) for i in range(dh // 2)])
        assert np.all(np.diff(scaled) < 0), (dh, theta)


def test_rope_variants_keep_relative_invariance():
    """Every layout / scaling variant still depends only on the distance m - n."""
    r = rng(23)
    for half, sc in [(True, None), (False, _L31), (True, _L31)]:
        c = _cfg(128, 5e5, half=half, scaling=sc)
        q, k = r.normal(0, 1, 128), r.normal(0, 1, 128)
        base = float(oracle.rope_cfg(q, 10, c) @ oracle.rope_cfg(k, 3, c))
        for delta in (1, 1000, 50000):
            s2 = float(oracle.rope_cfg(q, 10 + delta, c) @ oracle.rope_cfg(k, 3 + delta, c))
            assert abs(s2 - base) <= 1e-10 * (1 + abs(base))


# --------------------------------------------------------------------- SiLU ----

def test_silu_special_values_and_library():
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(40.0) - 40.0) < 1e-12
    assert abs(oracle.silu(-40.0)) < 1e-15
    for a in np.linspace(-12, 12, 97):
        assert abs(oracle.silu(a) - a * scipy.special.expit(a)) <= 1e-15 * (1 + abs(a))
    assert abs(oracle.silu(1.0) - F.silu(torch.tensor(1.0, dtype=torch.float64)).item()) < 1e-16


# ---------------------------------------------------------------- attention ----

def test_attention_uniform_cases():
    """Equal keys (or a zero query) give equal weights: the output is the mean
    of the value rows."""
    r = rng(6)
    dh = 16
    v = r.normal(0, 1, (9, dh))
    k = np.tile(r.normal(0, 1, dh), (9, 1))
    q = r.normal(0, 1, dh)
    np.testing.assert_allclose(oracle.attend(q, k, v), v.mean(0), rtol=1e-13, atol=1e-15)
    k2 = r.normal(0, 1, (9, dh))
    np.testing.assert_allclose(oracle.attend(np.zeros(dh), k2, v), v.mean(0), rtol=1e-13,
                               atol=1e-15)


def test_attention_two_key_closed_form_pins_scale():
    """Two keys whose scores differ by s/sqrt(dh): the first weight is
    sigmoid(s / sqrt(dh)) -- pins the 1/sqrt(d_head) scale of the equation in
    "The Evolving Transformer 04 LLaMA", 05 GQA."""
    for dh in (16, 64, 128):
        s = 3.0
        q = np.zeros(dh)
        q[0] = s
        k = np.zeros((2, dh))
        k[0, 0] = 1.0
        v = np.zeros((2, dh))
        v[0, 1] = 1.0
        v[1, 2] = 1.0
        out = oracle.attend(q, k, v)
        p = scipy.special.expit(s / math.sqrt(dh))
        assert abs(out[1] - p) < 1e-15 and abs(out[2] - (1 - p)) < 1e-15


def test_attention_matches_torch_sdpa():
    """Library special case: torch's scaled_dot_product_attention in fp64."""
    r = rng(7)
    for n, dh in [(1, 16), (37, 64), (300, 128)]:
        q = r.normal(0, 1.5, dh)
        k = r.normal(0, 1.5, (n, dh))
        v = r.normal(0, 1, (n, dh))
        want = F.scaled_dot_product_attention(torch.from_numpy(q)[None, None, None],
                                              torch.from_numpy(k)[None, None],
                                              torch.from_numpy(v)[None, None])[0, 0, 0].numpy()
        np.testing.assert_allclose(oracle.attend(q, k, v), want, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------ the block ----

def _small(name="tiny_f32", **kw):
    return workloads.with_overrides(workloads.get(name), **kw)


def _library_block(w, t, start_pos=0, k_prefix=None, v_prefix=None):
    """The block composed from torch library routines in fp64: F.rms_norm,
    F.linear, complex multiplication for the rotation (speeds read back from
    the oracle's own single-position rotation, pinned separately above), and
    F.scaled_dot_product_attention with grouped heads (enable_gqa repeats each
    KV head over consecutive query heads)."""
    d, H, G, dh = w.d, w.H, w.n_kv, w.d_head
    T = {k: v.double() for k, v in t.items()}
    x = T["x"]
    B, S, _ = x.shape
    n1 = F.rms_norm(x, (d,), T["attn_norm"], eps=w.eps)
    q = F.linear(n1, T["wq"]).view(B, S, H, dh)
    k = F.linear(n1, T["wk"]).view(B, S, G, dh)
    v = F.linear(n1, T["wv"]).view(B, S, G, dh)
    if w.rope_scaling:
        # scaled speeds read back from the oracle (pinned by the page's counts)
        om = torch.tensor([oracle.rope_freq(oracle.cfg_of(w), i) for i in range(dh // 2)],
                          dtype=torch.float64)
    else:
        om = torch.from_numpy(_omegas(dh, w.theta))
    pos = torch.arange(start_pos, start_pos + S, dtype=torch.float64)
    rot = torch.polar(torch.ones(S, dh // 2, dtype=torch.float64), pos[:, None] * om[None, :])

    def turn(a):
        if w.rope_half:
            # the rotate_half form: a * cos + rotate_half(a) * sin, with
            # rotate_half(a) = (-a[half:], a[:half]) and the angles repeated
            a1 = pos[:, None] * om[None, :]
            ang = torch.cat([a1, a1], dim=-1)[None, :, None, :]
            rh = torch.cat([-a[..., dh // 2:], a[..., : dh // 2]], dim=-1)
            return a * torch.cos(ang) + rh * torch.sin(ang)
        c = torch.view_as_complex(a.reshape(*a.shape[:-1], dh // 2, 2).contiguous())
        return torch.view_as_real(c * rot[None, :, None, :]).reshape(a.shape)

    q, k = turn(q), turn(k)
    q, k, v = q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2)
    if start_pos > 0:
        k = torch.cat([k_prefix.double(), k], dim=2)
        v = torch.cat([v_prefix.double(), v], dim=2)
    Tn = start_pos + S
    mask = torch.arange(Tn)[None, :] <= (start_pos + torch.arange(S))[:, None]
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, enable_gqa=True)
    o = o.transpose(1, 2).reshape(B, S, H * dh)
    h = x + F.linear(o, T["wo"])
    n2 = F.rms_norm(h, (d,), T["ffn_norm"], eps=w.eps)
    y = h + F.linear(F.silu(F.linear(n2, T["w_gate"])) * F.linear(n2, T["w_up"]), T["w_down"])
    return y.numpy()


@pytest.mark.parametrize("name,kw", [
    ("tiny_f32", {}),
    ("tiny_f32", {"B": 3, "S": 9, "seed": 5}),
    ("smollm2_135m_prefill", {"B": 2, "S": 33, "dtype": "f32"}),
])
def test_block_matches_library_composition(name, kw):
    w = _small(name, **kw)
    t = workloads.generate(w)
    y, _, _, _ = oracle.run_workload(w, t)
    want = _library_block(w, t)
    err = np.abs(y - want).max() / np.sqrt((want ** 2).mean())
    assert err < 1e-12, err


@pytest.mark.parametrize("half,scaling", [(True, None), (False, _L31), (True, _L31)])
def test_block_rope_variants_match_library_composition(half, scaling):
    """The rotate_half layout written the way "From GPT-2 to Llama" (Positions
    become a rotation) prints it, and the Llama 3.1 speeds, through the whole
    block at a cache offset."""
    w = _small("tiny_f32", B=2, S=5, start_pos=11, seed=7, rope_half=half, rope_scaling=scaling,
               theta=5e5)
    t = workloads.generate(w)
    y, _, _, _ = oracle.run_workload(w, t)
    want = _library_block(w, t, 11, t["k_prefix"], t["v_prefix"])
    err = np.abs(y - want).max() / np.sqrt((want ** 2).mean())
    assert err < 1e-12, err


def test_block_with_cache_offset_matches_library_composition():
    """Chunked call at start_pos > 0 reads the cached prefix ("Full Llama 3
    transformer block", How it works: start_pos and the cache offset)."""
    w = _small("tiny_f32", B=2, S=5, start_pos=11, seed=3)
    t = workloads.generate(w)
    y, _, _, _ = oracle.run_workload(w, t)
    want = _library_block(w, t, 11, t["k_prefix"], t["v_prefix"])
    err = np.abs(y - want).max() / np.sqrt((want ** 2).mean())
    assert err < 1e-12, err


def test_gqa_with_duplicated_heads_equals_mha_bitwise():
    """"From GPT-2 to Llama", Keys and values get shared: a copy with full
    key/value heads, each a duplicate of its group's, gives identical outputs."""
    w = _small("tiny_f32", B=2, S=7, seed=9)
    t = workloads.generate(w)
    y_gqa, _, _, _ = oracle.run_workload(w, t)
    rep = w.H // w.n_kv
    t2 = dict(t)
    for n in ("wk", "wv"):
        heads = t[n].view(w.n_kv, w.d_head, w.d)
        t2[n] = heads.repeat_interleave(rep, dim=0).reshape(w.H * w.d_head, w.d)
    w2 = workloads.with_overrides(w, n_kv=w.H)
    y_mha, _, _, _ = oracle.run_workload(w2, t2)
    np.testing.assert_array_equal(y_gqa, y_mha)
    # tiling the shared heads instead (the page's silent port mistake) differs
    t3 = dict(t)
    for n in ("wk", "wv"):
        heads = t[n].view(w.n_kv, w.d_head, w.d)
        t3[n] = heads.repeat(rep, 1, 1).reshape(w.H * w.d_head, w.d)
    y_tiled, _, _, _ = oracle.run_workload(w2, t3)
    assert np.abs(y_tiled - y_gqa).max() > 1e-6


def test_decode_token_by_token_equals_prefill():
    """"Full Llama 3 transformer block", How it works: incremental decoding with
    the cache offset gives the rows of one full causal prefill."""
    w = _small("tiny_f32", B=2, S=12, seed=11)
    t = workloads.generate(w)
    y_full, kc_full, vc_full, _ = oracle.run_workload(w, t)
    cfg = oracle.cfg_of(w)
    kc, vc = oracle.empty_cache(w)
    x = t["x"].double().numpy()
    for s in range(w.S):
        y_s, _ = oracle.block_forward(cfg, x[:, s:s + 1, :].copy(), t, s, kc, vc)
        np.testing.assert_allclose(y_s[:, 0, :], y_full[:, s, :], rtol=0, atol=1e-14)
    np.testing.assert_allclose(kc, kc_full, rtol=0, atol=0)
    np.testing.assert_allclose(vc, vc_full, rtol=0, atol=0)


@pytest.mark.parametrize("start_pos", [0, 5])
def test_row_subset_equals_full_computation_bitwise(start_pos):
    """The largest parity cases may ask the oracle for some output rows only.
    Each requested row, and every cache row up to the last requested position
    of its sequence, must be bitwise the row of the full computation: the
    subset runs the same per-row loops in the same order, it only skips rows.
    Rows are taken at both ends of each sequence and inside it, including a
    sequence with no requested row (its cache rows stay unwritten)."""
    w = _small("smollm2_135m_prefill", B=3, S=37, start_pos=start_pos, max_seq=48, seed=12,
               dtype="f32")
    t = workloads.generate(w)
    y_full, kc_full, vc_full, st_full = oracle.run_workload(w, t, stages=True)
    rows = [0, 1, 17, 36, 2 * 37 + 20]          # sequence 1 asks for nothing
    y_sub, kc_sub, vc_sub, st_sub = oracle.run_workload(w, t, rows=rows, stages=True)
    yf, ys = y_full.reshape(w.M, w.d), y_sub.reshape(w.M, w.d)
    np.testing.assert_array_equal(ys[rows], yf[rows])
    for name in ("n1", "q", "o", "h", "n2", "z"):
        np.testing.assert_array_equal(st_sub[name][rows], st_full[name][rows])
    for b, last in ((0, 36), (2, 20)):
        hi = start_pos + last + 1
        np.testing.assert_array_equal(kc_sub[b, :, :hi], kc_full[b, :, :hi])
        np.testing.assert_array_equal(vc_sub[b, :, :hi], vc_full[b, :, :hi])
    assert not np.any(kc_sub[1, :, start_pos:start_pos + w.S])
    # rows not asked for are left at zero, so the subset did skip work
    others = sorted(set(range(w.M)) - set(rows))
    assert not np.any(ys[others])


def test_residual_wiring_zero_weights():
    """"Full Llama 3 transformer block", How it works: h = x + Attn(...),
    y = h + FFN(...).  With Wo = 0 and W_down = 0, y = x exactly; with
    W_down = 0 alone, y = h."""
    w = _small("tiny_f32", B=1, S=6, seed=2)
    t = workloads.generate(w)
    t0 = dict(t, wo=torch.zeros_like(t["wo"]), w_down=torch.zeros_like(t["w_down"]))
    y, _, _, _ = oracle.run_workload(w, t0)
    np.testing.assert_array_equal(y, t["x"].double().numpy())
    t1 = dict(t, w_down=torch.zeros_like(t["w_down"]))
    y1, _, _, st = oracle.run_workload(w, t1, stages=True)
    np.testing.assert_array_equal(y1.reshape(-1, w.d), st["h"])


def test_kv_cache_values_written_per_token():
    """"Llama 4 From Scratch", Worked example: 2 x 8 x 128 = 2048 values per
    token per layer for the 8B heads (8192 with full heads); the call writes
    exactly those cache entries and nothing else."""
    for H, G, want_key in [(32, 8, "kv_values_per_token_per_layer_llama3_8b"),
                           (32, 32, "kv_values_per_token_per_layer_llama3_8b_full_heads")]:
        w = workloads.BlockWorkload("kvcount", "f32", B=1, S=3, start_pos=5, d=64, H=H, n_kv=G,
                                    d_head=128, d_ff=32, theta=5e5, eps=1e-5, w_std=0.02,
                                    max_seq=12)
        t = workloads.generate(w)
        kc = np.full((1, G, 12, 128), np.nan)
        vc = np.full((1, G, 12, 128), np.nan)
        kc[:, :, :5] = t["k_prefix"].double().numpy()
        vc[:, :, :5] = t["v_prefix"].double().numpy()
        oracle.block_forward(oracle.cfg_of(w), t["x"], t, 5, kc, vc)
        written = int(np.sum(~np.isnan(kc[:, :, 5:])) + np.sum(~np.isnan(vc[:, :, 5:])))
        assert written == w.S * g(want_key)
        assert np.all(np.isnan(kc[:, :, 8:])) and np.all(np.isnan(vc[:, :, 8:]))
    # all-layer totals quoted on the pages
    assert 32 * g("kv_values_per_token_per_layer_llama3_8b") == g("kv_values_per_token_llama3_8b_32_layers")
    assert 2 * g("kv_values_per_token_llama3_8b_32_layers") == g("kv_bytes_per_token_llama3_8b_16bit")
    assert 30 * 2 * 3 * 64 == g("kv_values_per_token_smollm2_30_layers")
    assert 30 * 2 * 9 * 64 == g("kv_values_per_token_smollm2_full_heads")
    assert 12 * 2 * 12 * 64 == g("kv_values_per_token_gpt2_small")
    gb = g("kv_bytes_per_token_llama3_8b_16bit") * 131072 / 1e9
    assert round(gb, 1) == g("llama31_8b_kv_gb_at_131072")
    assert round(4 * gb, 1) == g("llama31_8b_kv_gb_full_heads_at_131072")


def test_workload_shapes_match_pages():
    w8 = workloads.get("llama3_8b_prefill")
    s8 = g("llama3_8b_shape")
    assert (w8.d, w8.H, w8.n_kv, w8.d_head, w8.d_ff, w8.eps) == (
        s8["d"], s8["H"], s8["n_kv"], s8["d_head"], s8["d_ff"], s8["eps"])
    assert w8.theta == g("llama3_rope_base")
    pc = workloads.param_count(w8)
    assert round(pc["total_linear"] / 1e6) == g("llama3_8b_block_params_millions")
    assert round(pc["ffn"] / 1e6) == g("llama3_8b_block_ffn_params_millions")
    assert round(100 * pc["ffn"] / pc["total_linear"]) == g("llama3_8b_ffn_share_percent")
    mha = workloads.param_count(workloads.with_overrides(w8, n_kv=32))
    assert round(100 * mha["ffn"] / mha["total_linear"]) == g("llama3_8b_ffn_share_full_heads_percent")
    w70 = workloads.get("llama3_70b_prefill")
    wd = g("llama3_widths")
    assert w70.d == wd["d"][1] and w70.d_ff == wd["ffn"][1]
    assert w70.d_head == wd["head_dim"] and w70.n_kv == wd["n_kv"]
    ws = workloads.get("smollm2_135m_prefill")
    ss = g("smollm2_shape")
    assert (ws.d, ws.H, ws.n_kv, ws.d_head, ws.theta) == (ss["d"], ss["H"], ss["n_kv"], ss["d_head"],
                                                           ss["rope_base"])
    assert ws.d_ff == g("smollm2_ffn_width")
    ps = workloads.param_count(ws)
    assert round(100 * ps["ffn"] / ps["total_linear"]) == g("smollm2_ffn_share_percent")
    # full-head copy of all 30 layers adds 30 * 2 * 576 * 384 weights
    lo, hi = g("smollm2_full_head_copy_params_millions")
    full = workloads.param_count(workloads.with_overrides(ws, n_kv=9))
    assert abs(30 * (full["attn"] - ps["attn"]) / 1e6 - (hi - lo)) < 0.05
    # tiny block: d_ff is 8/3 * 64 rounded up to a multiple of 16
    wt = workloads.get("tiny_f32")
    assert wt.d_ff == 16 * math.ceil(8 * wt.d / 3 / 16)


# ------------------------------------------------------------------ stack ----
# "The Evolving Transformer 04 LLaMA", 07 ASSEMBLE LLAMA: N blocks, then a
# final RMSNorm; "Full Llama 3 transformer block", Overview: the block is the
# unit stacked L times.

def _np_rms(v, g, eps):
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps) * g


def _stack_caches(w, L):
    return [oracle.empty_cache(w) for _ in range(L)]


def test_stack_of_identity_blocks_is_the_final_norm():
    """Blocks with Wo = 0 and W_down = 0 pass the stream through unchanged, so
    every block output is x and y is RMSNorm(x) * final gain (closed form)."""
    w = _small("tiny_f32", B=2, S=5, seed=3)
    st = workloads.generate_stack(w, 3)
    layers = [dict(t, wo=torch.zeros_like(t["wo"]), w_down=torch.zeros_like(t["w_down"]))
              for t in st["layers"]]
    y, hid = oracle.stack_forward(oracle.cfg_of(w), st["x"], layers, st["final_norm"], 0,
                                  _stack_caches(w, 3), hidden=True)
    x = st["x"].double().numpy()
    for l in range(3):
        np.testing.assert_array_equal(hid[l], x)
    want = _np_rms(x, st["final_norm"].double().numpy(), w.eps)
    np.testing.assert_allclose(y, want, rtol=1e-14, atol=1e-15)


def _diag_stack(d, consts, seed):
    """Blocks whose output has a closed form: Wo = 0 (the attention branch adds
    exactly zero), W_gate = b I, W_up = a I, W_down = c I with d_ff = d (so
    FFN(n) = c SiLU(b n) (a n) per element), and Wk = k I with n_kv * d_head =
    d (so the K row a token writes at position 0, where the rotation is the
    identity, is k RMSNorm_1(input))."""
    r = rng(seed)
    I = np.eye(d)
    layers = []
    for (a, b, c, k) in consts:
        layers.append({"attn_norm": r.uniform(0.5, 1.5, d), "wq": r.normal(0, 0.2, (d, d)),
                       "wk": k * I, "wv": r.normal(0, 0.2, (d, d)), "wo": np.zeros((d, d)),
                       "ffn_norm": r.uniform(0.5, 1.5, d), "w_gate": b * I, "w_up": a * I,
                       "w_down": c * I})
    return layers


def test_stack_chains_blocks_in_order_closed_form():
    """Three blocks with different closed-form maps, one token per sequence at
    position 0: y and every block's K and V cache row follow from chaining
    the closed forms in order (block l reads block l-1's output, each writes
    its own cache, the final norm comes last)."""
    d, eps = 16, 1e-5
    cfg = {"d": d, "H": 2, "n_kv": 2, "d_head": 8, "d_ff": d, "theta": 1e4, "eps": eps}
    consts = [(1.3, 0.7, 0.9, 1.1), (-0.6, 1.9, 1.4, 0.8), (2.1, -1.2, -0.5, 1.7)]
    layers = _diag_stack(d, consts, 7)
    r = rng(8)
    x = r.normal(0, 1, (2, 1, d))
    gf = r.uniform(0.5, 1.5, d)
    caches = [(np.zeros((2, 2, 3, 8)), np.zeros((2, 2, 3, 8))) for _ in layers]
    y, hid = oracle.stack_forward(cfg, x, layers, gf, 0, caches, hidden=True)
    silu = lambda u: u / (1.0 + np.exp(-u))
    v = x[:, 0, :]
    for l, ((a, b, c, k), lw) in enumerate(zip(consts, layers)):
        n1 = _np_rms(v, lw["attn_norm"], eps)
        np.testing.assert_allclose(caches[l][0][:, :, 0, :].reshape(2, d), k * n1, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(caches[l][1][:, :, 0, :].reshape(2, d), n1 @ lw["wv"].T, rtol=1e-12,
                                   atol=1e-13)
        n2 = _np_rms(v, lw["ffn_norm"], eps)
        v = v + c * silu(b * n2) * (a * n2)
        np.testing.assert_allclose(hid[l][:, 0, :], v, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(y[:, 0, :], _np_rms(v, gf, eps), rtol=1e-13, atol=1e-14)


def test_stack_prefill_equals_token_by_token_decode():
    """"Full Llama 3 transformer block", How it works: with each block keeping
    its own cache, S single-token steps of the stack give the rows of one
    causal prefill of the stack, and leave the same caches."""
    w = _small("tiny_f32", B=2, S=7, seed=12)
    st = workloads.generate_stack(w, 3)
    cfg = oracle.cfg_of(w)
    full = _stack_caches(w, 3)
    y_full, _ = oracle.stack_forward(cfg, st["x"], st["layers"], st["final_norm"], 0, full)
    steps = _stack_caches(w, 3)
    x = st["x"].double().numpy()
    for s in range(w.S):
        y_s, _ = oracle.stack_forward(cfg, x[:, s:s + 1, :].copy(), st["layers"], st["final_norm"], s, steps)
        np.testing.assert_allclose(y_s[:, 0, :], y_full[:, s, :], rtol=0, atol=1e-13)
    for (ka, va), (kb, vb) in zip(full, steps):
        np.testing.assert_allclose(ka, kb, rtol=0, atol=1e-13)
        np.testing.assert_allclose(va, vb, rtol=0, atol=1e-13)


# -------------------------------------------------------------------- MoE ----
# "Llama 4 From Scratch", The idea: N expert FFNs, a router sending each token
# to the top k, one always-on shared expert.

_MOE_W = workloads.BlockWorkload("moe_pin", "f32", B=2, S=5, start_pos=0, d=32, H=4, n_kv=2, d_head=8,
                                 d_ff=48, theta=1e4, eps=1e-5, w_std=0.1, g_mean=1.0, g_std=0.1,
                                 seed=9, n_experts=6, top_k=2, d_ff_expert=40)


def _np_swiglu(n, gate, up, down):
    a = n @ gate.T
    return ((a / (1.0 + np.exp(-a))) * (n @ up.T)) @ down.T


def test_moe_route_is_top_k_by_brute_force():
    """Router logits are n . router^T (numpy); the chosen experts are the k
    largest, in order, ties to the lower index (numpy stable argsort); the
    weights are the softmax of the chosen logits (scipy)."""
    r = rng(31)
    for E, K in ((6, 2), (16, 1), (8, 8), (5, 3)):
        moe = {"n_experts": E, "top_k": K, "d_ff_expert": 4}
        for _ in range(20):
            n = r.normal(0, 1, 24)
            router = r.normal(0, 1, (E, 24))
            if r.random() < 0.3:      # equal logits: duplicated router rows
                i, j = r.choice(E, 2, replace=False)
                router[j] = router[i]
            sel, wts, logits = oracle.moe_route(moe, n, router)
            want_logits = n @ router.T
            np.testing.assert_allclose(logits, want_logits, rtol=1e-13, atol=1e-13)
            order = np.argsort(-logits, kind="stable")[:K]
            assert list(sel) == list(order)
            np.testing.assert_allclose(wts, scipy.special.softmax(logits[order]), rtol=1e-13)


def _moe_cfg(w):
    return oracle.cfg_of(w), w.moe


def _concat_ffn(t, parts):
    """The block's weights with its FFN replaced by the concatenation of
    several SwiGLU FFNs [(gate, up, down, scale)]: a SwiGLU of the
    concatenated hidden width is the sum of the parts."""
    g = np.concatenate([p[0] for p in parts], axis=0)
    u = np.concatenate([p[1] for p in parts], axis=0)
    dn = np.concatenate([p[2] * p[3] for p in parts], axis=1)
    out = {k: t[k].double().numpy() for k in oracle.WEIGHT_NAMES}
    out.update(w_gate=g, w_up=u, w_down=dn)
    return out


def test_moe_identical_experts_is_one_dense_ffn():
    """With every routed expert equal, the weights of the k chosen ones sum to
    1, so the MoE FFN is shared + expert: the dense block whose FFN is their
    concatenation, whatever the router picks."""
    w = _MOE_W
    t = workloads.generate(w)
    cfg, moe = _moe_cfg(w)
    E = w.n_experts
    for n in ("e_gate", "e_up", "e_down"):
        t[n] = t[n][:1].expand_as(t[n]).contiguous()
    kc, vc = oracle.empty_cache(w)
    y, sel, wts, _ = oracle.moe_block_forward(cfg, moe, t["x"], t, 0, kc, vc)
    assert len(set(sel.ravel().tolist())) > 1  # the router does spread the rows
    np.testing.assert_allclose(wts.sum(axis=1), 1.0, rtol=1e-14)
    sh = (t["w_gate"].double().numpy(), t["w_up"].double().numpy(), t["w_down"].double().numpy(), 1.0)
    ex = (t["e_gate"][0].double().numpy(), t["e_up"][0].double().numpy(), t["e_down"][0].double().numpy(), 1.0)
    dense = _concat_ffn(t, [sh, ex])
    kd, vd = oracle.empty_cache(w)
    yd, _ = oracle.block_forward(dict(cfg, d_ff=w.d_ff + w.d_ff_expert), t["x"], dense, 0, kd, vd)
    np.testing.assert_allclose(y, yd, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(kc, kd)


def test_moe_zero_router_takes_the_first_k_equally():
    """A zero router gives every expert the same logit: the tie rule picks
    experts 0 .. k-1, each weighted 1/k, so the block equals the dense block
    whose FFN concatenates the shared expert and those experts scaled by 1/k."""
    w = _MOE_W
    t = workloads.generate(w)
    t["router"] = torch.zeros_like(t["router"])
    cfg, moe = _moe_cfg(w)
    kc, vc = oracle.empty_cache(w)
    y, sel, wts, _ = oracle.moe_block_forward(cfg, moe, t["x"], t, 0, kc, vc)
    assert (sel == np.arange(w.top_k)).all()
    np.testing.assert_array_equal(wts, 1.0 / w.top_k)
    parts = [(t["w_gate"].double().numpy(), t["w_up"].double().numpy(), t["w_down"].double().numpy(), 1.0)]
    for e in range(w.top_k):
        parts.append((t["e_gate"][e].double().numpy(), t["e_up"][e].double().numpy(),
                      t["e_down"][e].double().numpy(), 1.0 / w.top_k))
    dense = _concat_ffn(t, parts)
    kd, vd = oracle.empty_cache(w)
    yd, _ = oracle.block_forward(dict(cfg, d_ff=w.d_ff + w.top_k * w.d_ff_expert), t["x"], dense, 0, kd, vd)
    np.testing.assert_allclose(y, yd, rtol=1e-12, atol=1e-12)


def test_moe_ffn_row_closed_form():
    """One row through orc_moe_ffn: shared SwiGLU plus the chosen experts'
    SwiGLUs weighted by the softmax of their logits, each SwiGLU written out
    in numpy; with forced experts the same formula over those experts."""
    w = _MOE_W
    t = workloads.generate(w)
    cfg, moe = _moe_cfg(w)
    r = rng(4)
    T = {k: t[k].double().numpy() for k in ("w_gate", "w_up", "w_down") + oracle.MOE_WEIGHT_NAMES}
    for force in (None, [3, 1], [5, 0]):
        n = r.normal(0, 1, w.d)
        out, sel, wts, logits = oracle.moe_ffn(cfg, moe, n, t, force_sel=force)
        if force is not None:
            assert list(sel) == force
        want = _np_swiglu(n, T["w_gate"], T["w_up"], T["w_down"])
        lg = n @ T["router"].T
        p = scipy.special.softmax(lg[list(sel)])
        for j, e in enumerate(sel):
            want = want + p[j] * _np_swiglu(n, T["e_gate"][e], T["e_up"][e], T["e_down"][e])
        np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-13)


def test_moe_block_decode_token_by_token_equals_prefill():
    """"Full Llama 3 transformer block", How it works: single-token steps give
    the rows of one prefill, with the MoE FFN too (it acts row by row)."""
    w = _MOE_W
    t = workloads.generate(w)
    cfg, moe = _moe_cfg(w)
    kc, vc = oracle.empty_cache(w)
    y_full, sel_full, _, _ = oracle.moe_block_forward(cfg, moe, t["x"], t, 0, kc, vc)
    k2, v2 = oracle.empty_cache(w)
    x = t["x"].double().numpy()
    for s in range(w.S):
        y_s, sel_s, _, _ = oracle.moe_block_forward(cfg, moe, x[:, s:s + 1].copy(), t, s, k2, v2)
        np.testing.assert_allclose(y_s[:, 0], y_full[:, s], rtol=0, atol=1e-13)
        assert (sel_s == sel_full.reshape(w.B, w.S, -1)[:, s]).all()


# ------------------------------------------------- planted mistakes are caught ----

MUTANTS = [
    # (what is planted, text in oracle.c, replacement, pins that must fail)
    ("RoPE exponent -i/dh", "-2.0 * (double)i / (double)d_head", "-1.0 * (double)i / (double)d_head",
     ["test_rope_pair_periods_match_page"]),
    ("RoPE rotation sign", "v[2 * i + 1] = u * s + w * c;", "v[2 * i + 1] = -u * s + w * c;",
     ["test_rope_is_complex_rotation_of_adjacent_pairs", "test_rope_relative_position_invariance"]),
    ("attention scale 1/dh", "1.0 / sqrt((double)d_head)", "1.0 / (double)d_head",
     ["test_attention_two_key_closed_form_pins_scale", "test_attention_matches_torch_sdpa"]),
    ("causal bound t < m", "const long n_keys = pos + 1;", "const long n_keys = pos > 0 ? pos : 1;",
     ["test_block_matches_library_composition"]),
    ("GQA tiling h % n_kv", "const int g = hh / n_rep;", "const int g = hh % G;",
     ["test_block_matches_library_composition"]),
    ("RMSNorm sum not mean", "sqrt(ss / (double)d + eps)", "sqrt(ss + eps)",
     ["test_rmsnorm_unit_gain_closed_form", "test_rmsnorm_matches_torch_rms_norm"]),
    ("missing attention residual", "h[i] = xr[i] + h[i];", "h[i] = h[i];",
     ["test_residual_wiring_zero_weights", "test_block_matches_library_composition"]),
    ("sigmoid instead of SiLU", "return a / (1.0 + exp(-a));", "return 1.0 / (1.0 + exp(-a));",
     ["test_silu_special_values_and_library", "test_block_matches_library_composition"]),
    ("transposed projection", "const double* row = w + (size_t)j * (size_t)n_in;",
     "const double* row = w + (size_t)j;",
     ["test_linear_matches_numpy_matmul"]),
    ("rotate_half partner off by one", "iw = c->rope_half ? i + half : 2 * i + 1;",
     "iw = c->rope_half ? (i + half + 1) % dh : 2 * i + 1;",
     ["test_rope_half_layout_is_a_permutation_of_interleaved"]),
    ("block RoPE sign", "v[iw] = u * sn + w * cs;", "v[iw] = -u * sn + w * cs;",
     ["test_rope_default_settings_are_the_plain_rotation", "test_block_matches_library_composition"]),
    ("scaling classes swapped", "if (wavelen < c->rope_orig / c->rope_high) return speed;",
     "if (wavelen < c->rope_orig / c->rope_low) return speed;",
     ["test_rope_llama31_scaling_counts_match_page"]),
    ("blend weight reversed", "return (1.0 - t) * speed / c->rope_scale + t * speed;",
     "return t * speed / c->rope_scale + (1.0 - t) * speed;",
     ["test_rope_llama31_blend_meets_both_classes"]),
    ("stack: every block reads x",
     "rc = orc_block_forward(c, B, S, start_pos, cap, stream, &layers[l]",
     "rc = orc_block_forward(c, B, S, start_pos, cap, x, &layers[l]",
     ["test_stack_chains_blocks_in_order_closed_form"]),
    ("stack: final norm left out",
     "orc_rms_norm(stream + (size_t)r * d, final_norm, d, c->norm_eps, y + (size_t)r * d);",
     "memcpy(y + (size_t)r * d, stream + (size_t)r * d, sizeof(double) * (size_t)d);",
     ["test_stack_of_identity_blocks_is_the_final_norm", "test_stack_chains_blocks_in_order_closed_form"]),
    ("stack: one cache for every block", "k_caches[l], v_caches[l]", "k_caches[0], v_caches[0]",
     ["test_stack_chains_blocks_in_order_closed_form", "test_stack_prefill_equals_token_by_token_decode"]),
    ("stack: last block dropped", "for (int l = 0; l < n_layers && rc == 0; ++l)",
     "for (int l = 0; l < n_layers - 1 && rc == 0; ++l)",
     ["test_stack_chains_blocks_in_order_closed_form"]),
    ("MoE: top-k takes the smallest", "if (!taken && (best < 0 || logits[e] > logits[best])) best = e;",
     "if (!taken && (best < 0 || logits[e] < logits[best])) best = e;",
     ["test_moe_route_is_top_k_by_brute_force"]),
    ("MoE: ties to the higher index", "if (!taken && (best < 0 || logits[e] > logits[best])) best = e;",
     "if (!taken && (best < 0 || logits[e] >= logits[best])) best = e;",
     ["test_moe_route_is_top_k_by_brute_force", "test_moe_zero_router_takes_the_first_k_equally"]),
    ("MoE: weights not normalised", "    for (int j = 0; j < K; ++j) wts[j] /= sum;\n", "\n",
     ["test_moe_identical_experts_is_one_dense_ffn", "test_moe_zero_router_takes_the_first_k_equally",
      "test_moe_route_is_top_k_by_brute_force"]),
    ("MoE: shared expert left out", "swiglu(n, w->w_gate, w->w_up, w->w_down, d, c->d_ff, out); /* the shared expert */",
     "memset(out, 0, sizeof(double) * (size_t)d);", ["test_moe_ffn_row_closed_form"]),
    ("MoE: up and gate swapped in the experts",
     "swiglu(n, mw->w_gate + e * (size_t)f * d, mw->w_up + e * (size_t)f * d,",
     "swiglu(n, mw->w_up + e * (size_t)f * d, mw->w_gate + e * (size_t)f * d,",
     ["test_moe_ffn_row_closed_form", "test_moe_zero_router_takes_the_first_k_equally"]),
    ("row subset: each sequence's cache one row short", "if (s + 1 > need[b]) need[b] = s + 1;",
     "if (s > need[b]) need[b] = s;", ["test_row_subset_equals_full_computation_bitwise"]),
]


def _build_mutant(tmp_path, old, new):
    import ctypes
    import subprocess
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    assert src.count(old) == 1, old
    d = tmp_path / "mut"
    d.mkdir(exist_ok=True)
    (d / "oracle.c").write_text(src.replace(old, new))
    (d / "oracle.h").write_text(open(os.path.join(os.path.dirname(oracle.__file__), "oracle.h")).read())
    so = d / "libmut.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-o", str(so), str(d / "oracle.c"), "-lm"], check=True)
    return so


@pytest.mark.parametrize("label,old,new,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, label, old, new, pins):
    so = _build_mutant(tmp_path, old, new)
    saved = oracle._lib
    try:
        oracle._lib = None
        real = oracle.lib()  # argtypes set on the real library object
        import ctypes
        mut = ctypes.CDLL(str(so))
        for name in ("orc_rms_norm", "orc_linear", "orc_rope", "orc_rope_freq", "orc_rope_cfg",
                     "orc_silu", "orc_attend", "orc_block_forward", "orc_stack_forward", "orc_moe_route",
                     "orc_moe_ffn", "orc_moe_block_forward"):
            getattr(mut, name).argtypes = getattr(real, name).argtypes
            getattr(mut, name).restype = getattr(real, name).restype
        oracle._lib = mut
        for pin in pins:
            fn = globals()[pin]
            args = {"test_block_matches_library_composition": ("tiny_f32", {"B": 3, "S": 9, "seed": 5}),
                    "test_row_subset_equals_full_computation_bitwise": (5,)}
            with pytest.raises(AssertionError):
                if pin in args:
                    fn(*args[pin])
                else:
                    fn()
    finally:
        oracle._lib = saved
