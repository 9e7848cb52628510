// Block executor and C ABI (include/llama_block.h).
//
// init: validate the config, pack the weights into library-owned device
// memory (fused [Wq;Wk;Wv], gate/up interleaved in groups of four rows,
// bf16 -> fp16 widening for fp16 operands), build the RoPE table and size the
// workspace.  forward: validate, then enqueue
//   RMSNorm_1 -> QKV GEMM (+RoPE, KV append) -> attention -> o GEMM (+x)
//   -> RMSNorm_2 -> gate/up GEMM (+SiLU*up) -> down GEMM (+h)
// on the caller's stream ("Full Llama 3 transformer block", How it works).
#include "llama_block.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <atomic>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "launch.h"

using lb::Elem;

// Packed weights of one block: for bf16 blocks one copy, in the operand type
// and the k-step tiled layout (lb_device.h) that both the prefill and the
// decode GEMMs read; for fp32 blocks row-major fp32.
struct LayerW {
    void* w_qkv = nullptr;   // [Wq; Wk; Wv]
    void* w_o = nullptr;
    void* w_gu = nullptr;    // gate/up interleaved in groups of four rows
    void* w_down = nullptr;
    float* g1 = nullptr;
    float* g2 = nullptr;
};

struct lb_block {
    lb_config cfg;
    Elem dt = Elem::F32;  // dtype of x, out, cache
    Elem op = Elem::F32;  // matrix-product operand type
    int dev = 0;
    int qd = 0, kvd = 0, nqkv = 0;
    LayerW lw;  // this block's weights
    float2* rope = nullptr;
    // workspace
    void* n1 = nullptr;
    void* n2 = nullptr;
    void* q = nullptr;
    void* o = nullptr;
    void* z = nullptr;
    float* h = nullptr;
    void* kws = nullptr;
    void* vws = nullptr;
    size_t ws_rows = 0;  // token rows the k/v workspace copies hold
    float* part = nullptr;       // decode attention partials
    float* gpart = nullptr;      // split-K decode GEMM partials
    size_t gpart_cap = 0;        // floats
    unsigned* gcnt = nullptr;    // arrival counts of the two-way split decode GEMM (zeroed at init)
    // decode activations (<= kDecodeRows token rows) in the k-step tiled layout
    void* at_n1 = nullptr;
    void* at_o = nullptr;
    void* at_n2 = nullptr;
    void* at_z = nullptr;
    int last_mt = 0;             // row tiles of the last forward's tiled activations (0: none)
    int last_ffn_mt = 0;         // the same for n2 and z (MoE blocks keep them row-major)
    int last_m = 0;
    // mixture-of-experts FFN (moe_E > 0); the dense FFN above is the shared expert
    int moe_E = 0, moe_K = 0, moe_fe = 0;
    void* w_router = nullptr;    // [E][d] operand type
    void* w_egu = nullptr;       // [E][2 fe][d] gate/up packed per expert
    void* w_edown = nullptr;     // [E][d][fe]
    float* m_logits = nullptr;   // [T][E]
    int* m_sel = nullptr;        // [T][K]
    float* m_wts = nullptr;      // [T][K]
    int* m_row_off = nullptr;    // [E+1]
    int* m_tile_off = nullptr;   // [E+1]
    int* m_src = nullptr;        // [T*K]
    int* m_slot = nullptr;       // [T*K]
    void* m_a = nullptr;         // [T*K][d] normalised rows in expert order
    void* m_z = nullptr;         // [T*K][fe]
    float* m_r = nullptr;        // [T*K][d] expert outputs
    float* m_hs = nullptr;       // [T][d] h plus the shared expert
    std::vector<void*> allocs;
    uint64_t device_bytes = 0;   // sum of the sizes in allocs
    std::string err;
    // per-stage timing: a ring of event sets, LB_NUM_STAGES + 1 events each
    bool profiling = false;
    uint32_t profile_mask = 0;
    std::vector<hipEvent_t> events;
    std::vector<int> pending;      // ring slots recorded but not yet summed
    int next_slot = 0;
    double stage_ms[LB_NUM_STAGES] = {};
    int64_t profiled_calls = 0;
};

// The scratch buffers one forward writes and reads: the handle's workspace,
// or (llama_block_forward_decode_static) pieces of the library's static array.
struct Workspace {
    void* n1 = nullptr;
    void* n2 = nullptr;
    void* q = nullptr;
    void* o = nullptr;
    void* z = nullptr;
    float* h = nullptr;
    void* kws = nullptr;
    void* vws = nullptr;
    float* part = nullptr;
    float* gpart = nullptr;
    size_t gpart_cap = 0;
    unsigned* gcnt = nullptr;
    void* at_n1 = nullptr;
    void* at_o = nullptr;
    void* at_n2 = nullptr;
    void* at_z = nullptr;
};

static Workspace handle_workspace(const lb_block* blk) {
    Workspace w;
    w.n1 = blk->n1;
    w.n2 = blk->n2;
    w.q = blk->q;
    w.o = blk->o;
    w.z = blk->z;
    w.h = blk->h;
    w.kws = blk->kws;
    w.vws = blk->vws;
    w.part = blk->part;
    w.gpart = blk->gpart;
    w.gpart_cap = blk->gpart_cap;
    w.gcnt = blk->gcnt;
    w.at_n1 = blk->at_n1;
    w.at_o = blk->at_o;
    w.at_n2 = blk->at_n2;
    w.at_z = blk->at_z;
    return w;
}

static constexpr int kProfileSlots = 256;
static constexpr int kDecodeRows = 64;  // largest decode batch that runs on the tiled GEMMs

// ---- static scratch of llama_block_forward_decode_static ---------------------------
// One array per GPU in the library's device code; that entry point carves its
// scratch buffers out of it and so allocates nothing.  Host code never uses
// the array's name as an address: each device's copy sits at its own address,
// looked up once per device (set up by init) and kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[LB_STATIC_SCRATCH_BYTES];
static constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch[kMaxDevices];
static std::mutex g_scratch_lock;

// Look up the current device's copy of `scratch` (dev must be current).
static void setup_static_scratch(int dev) {
    if (dev < 0 || dev >= kMaxDevices || g_scratch[dev].load(std::memory_order_acquire)) return;
    std::lock_guard<std::mutex> guard(g_scratch_lock);
    if (g_scratch[dev].load(std::memory_order_relaxed)) return;
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess && p) {
        g_scratch[dev].store(p, std::memory_order_release);
    } else {
        (void)hipGetLastError();
    }
}

static void profile_release(lb_block* blk) {
    for (hipEvent_t e : blk->events) hipEventDestroy(e);
    blk->events.clear();
    blk->pending.clear();
    blk->profiling = false;
}

// Sum one recorded slot into the per-stage totals (waits for its events).
// event i is recorded when stage i or stage i-1 is timed
static bool mark_needed(uint32_t mask, int i) {
    return ((mask >> i) & 1u) || (i > 0 && ((mask >> (i - 1)) & 1u));
}

static hipError_t profile_collect(lb_block* blk, int slot) {
    hipEvent_t* ev = &blk->events[(size_t)slot * (LB_NUM_STAGES + 1)];
    int last = LB_NUM_STAGES;
    while (last > 0 && !mark_needed(blk->profile_mask, last)) --last;
    hipError_t e = hipEventSynchronize(ev[last]);
    if (e != hipSuccess) return e;
    for (int i = 0; i < LB_NUM_STAGES; ++i) {
        if (!((blk->profile_mask >> i) & 1u)) continue;
        float ms = 0.0f;
        e = hipEventElapsedTime(&ms, ev[i], ev[i + 1]);
        if (e != hipSuccess) return e;
        blk->stage_ms[i] += ms;
    }
    blk->profiled_calls += 1;
    return hipSuccess;
}

static thread_local std::string g_init_error;

static lb_status fail(lb_block* blk, lb_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    if (blk) blk->err = buf;
    else g_init_error = buf;
    return st;
}

static void free_all(lb_block* blk) {
    for (void* p : blk->allocs) hipFree(p);
    blk->allocs.clear();
}

template <typename P>
static bool dalloc(lb_block* blk, P** out, size_t bytes) {
    void* p = nullptr;
    if (bytes == 0) bytes = 256;
    if (hipMalloc(&p, bytes) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    blk->allocs.push_back(p);
    blk->device_bytes += bytes;
    *out = static_cast<P*>(p);
    return true;
}

static size_t esz(Elem e) { return lb::elem_bytes(e); }

extern "C" const char* llama_block_status_string(lb_status s) {
    switch (s) {
        case LB_OK: return "ok";
        case LB_ERR_INVALID_ARG: return "invalid argument";
        case LB_ERR_UNSUPPORTED: return "unsupported configuration";
        case LB_ERR_OOM: return "device out of memory";
        case LB_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

extern "C" const char* llama_block_last_error(const lb_block* blk) {
    return blk ? blk->err.c_str() : g_init_error.c_str();
}

static lb_status validate_config(const lb_config* c) {
    if (c->d_model <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->d_head <= 0 || c->d_ff <= 0)
        return fail(nullptr, LB_ERR_INVALID_ARG, "d_model, n_heads, n_kv_heads, d_head and d_ff must be > 0");
    if ((long)c->n_heads * c->d_head != c->d_model)
        return fail(nullptr, LB_ERR_INVALID_ARG, "d_model (%d) != n_heads (%d) * d_head (%d)", c->d_model,
                    c->n_heads, c->d_head);
    if (c->n_heads % c->n_kv_heads != 0)
        return fail(nullptr, LB_ERR_INVALID_ARG, "n_heads (%d) is not a multiple of n_kv_heads (%d)",
                    c->n_heads, c->n_kv_heads);
    if (c->d_head % 2 != 0) return fail(nullptr, LB_ERR_INVALID_ARG, "d_head (%d) must be even", c->d_head);
    if (c->max_tokens <= 0 || c->max_seq_len <= 0)
        return fail(nullptr, LB_ERR_INVALID_ARG, "max_tokens and max_seq_len must be > 0");
    if (!(c->rope_theta > 0.0) || !std::isfinite(c->rope_theta) || !(c->norm_eps > 0.0) ||
        !std::isfinite(c->norm_eps))
        return fail(nullptr, LB_ERR_INVALID_ARG, "rope_theta and norm_eps must be finite and > 0");
    if (c->dtype != LB_F32 && c->dtype != LB_BF16)
        return fail(nullptr, LB_ERR_INVALID_ARG, "unknown dtype %d", (int)c->dtype);
    if (c->operands != LB_OPERANDS_AUTO && c->operands != LB_OPERANDS_F16 && c->operands != LB_OPERANDS_BF16)
        return fail(nullptr, LB_ERR_INVALID_ARG, "unknown operands %d", (int)c->operands);
    if (c->rope_layout != LB_ROPE_INTERLEAVED && c->rope_layout != LB_ROPE_HALF)
        return fail(nullptr, LB_ERR_INVALID_ARG, "unknown rope_layout %d", (int)c->rope_layout);
    if (c->rope_scale_factor > 1.0 &&
        !(c->rope_low_freq_factor > 0.0 && c->rope_high_freq_factor > c->rope_low_freq_factor &&
          c->rope_original_max_pos > 0.0 && std::isfinite(c->rope_scale_factor) &&
          std::isfinite(c->rope_high_freq_factor) && std::isfinite(c->rope_original_max_pos)))
        return fail(nullptr, LB_ERR_INVALID_ARG,
                    "rope scaling needs 0 < low_freq_factor < high_freq_factor and original_max_pos > 0");
    if (c->d_model > 16384)
        return fail(nullptr, LB_ERR_UNSUPPORTED, "d_model > 16384 is not supported (got %d)", c->d_model);
    if (c->dtype == LB_BF16) {
        if (c->d_head != 64 && c->d_head != 128)
            return fail(nullptr, LB_ERR_UNSUPPORTED, "bf16 blocks need d_head 64 or 128 (got %d)", c->d_head);
        if (c->d_model % 64 != 0 || c->d_ff % 64 != 0)
            return fail(nullptr, LB_ERR_UNSUPPORTED, "bf16 blocks need d_model and d_ff multiples of 64");
        if (c->n_heads / c->n_kv_heads > 16)
            return fail(nullptr, LB_ERR_UNSUPPORTED, "bf16 blocks need n_heads / n_kv_heads <= 16");
    } else {
        if (c->d_head % 8 != 0 || c->d_head > 256)
            return fail(nullptr, LB_ERR_UNSUPPORTED, "fp32 blocks need d_head a multiple of 8 and <= 256");
        if (c->d_model % 8 != 0 || c->d_ff % 4 != 0)
            return fail(nullptr, LB_ERR_UNSUPPORTED, "fp32 blocks need d_model % 8 == 0 and d_ff % 4 == 0");
    }
    return LB_OK;
}

// Bytes of every device buffer of a dense block, from its (validated) config
// alone: create_core, alloc_layer and llama_stack_init allocate exactly these,
// and llama_block_footprint adds them up.  Operands take 2 bytes in bf16
// blocks (fp16 or bf16) and 4 in fp32 blocks.
struct Sizes {
    size_t rope, n1, n2, q, o, z, h;                         // every block
    size_t kws, vws, part, gpart, gcnt, at_n1, at_o, at_n2, at_z;  // bf16 blocks only (else 0)
    size_t ws_rows, gpart_floats;
    size_t w_qkv, w_o, w_gu, w_down, g1, g2;                 // the weights of one block
    size_t staging;                                          // held while init packs (bf16)
    size_t g_final, act;                                     // a stack's final gain, activations

    uint64_t workspace() const {
        return (uint64_t)rope + n1 + n2 + q + o + z + h + kws + vws + part + gpart + gcnt + at_n1 + at_o + at_n2 +
               at_z;
    }
    uint64_t layer() const { return (uint64_t)w_qkv + w_o + w_gu + w_down + g1 + g2; }
};

static Sizes sizes_of(const lb_config& c) {
    Sizes z = {};
    const bool bf = c.dtype == LB_BF16;
    const size_t eo = bf ? 2 : 4, eio = bf ? 2 : 4;
    const size_t T = (size_t)c.max_tokens, d = (size_t)c.d_model, dh = (size_t)c.d_head, dff = (size_t)c.d_ff;
    const size_t qd = (size_t)c.n_heads * dh, kvd = (size_t)c.n_kv_heads * dh, nqkv = qd + 2 * kvd;
    z.rope = (size_t)c.max_seq_len * (dh / 2) * sizeof(float2);
    z.n1 = z.n2 = T * d * eo;
    z.q = z.o = T * qd * eo;
    z.z = T * dff * eo;
    z.h = T * d * 4;
    if (bf) {
        // prefill from position 0 keeps k and v^T in the operand type with the
        // sequence stride rounded up to 8: B * round8(S) <= T + 7 * T / 2 rows.
        z.ws_rows = T + 7 * (T / 2) + 8;
        z.kws = z.vws = z.ws_rows * kvd * eo;
        z.part = lb::decode_partials_floats(c.max_tokens, c.n_heads, c.d_head, c.max_seq_len) * sizeof(float);
        z.gpart_floats = lb::skinny_partials_floats(c.max_tokens < 64 ? c.max_tokens : 64,
                                                    (int)std::max(std::max(nqkv, d), 2 * dff));
        z.gpart = z.gpart_floats * sizeof(float);
        z.gcnt = (size_t)lb::kSplitCounters * sizeof(unsigned);
        z.at_n1 = z.at_n2 = (size_t)kDecodeRows * d * eo;
        z.at_o = (size_t)kDecodeRows * qd * eo;
        z.at_z = (size_t)kDecodeRows * dff * eo;
        z.staging = std::max(std::max(nqkv * d, d * qd), 2 * dff * d) * eo;
    }
    z.w_qkv = nqkv * d * eo;
    z.w_o = d * qd * eo;
    z.w_gu = 2 * dff * d * eo;
    z.w_down = d * dff * eo;
    z.g1 = z.g2 = d * 4;
    z.g_final = d * 4;
    z.act = T * d * eio;
    return z;
}

// Allocate one block's packed weights (owned by blk's allocation list).
static bool alloc_layer(lb_block* blk, LayerW* L) {
    const Sizes z = sizes_of(blk->cfg);
    return dalloc(blk, &L->w_qkv, z.w_qkv) && dalloc(blk, &L->w_o, z.w_o) && dalloc(blk, &L->w_gu, z.w_gu) &&
           dalloc(blk, &L->w_down, z.w_down) && dalloc(blk, &L->g1, z.g1) && dalloc(blk, &L->g2, z.g2);
}

static bool weights_complete(const lb_weights* w) {
    const void* wp[9] = {w->attn_norm, w->wq, w->wk, w->wv, w->wo, w->ffn_norm, w->w_gate, w->w_up, w->w_down};
    for (const void* p : wp)
        if (!p) return false;
    return true;
}

// Enqueue the packing of one block's weights from the caller's tensors.  For
// bf16 blocks each matrix is converted row-major into `stage` (device scratch
// of Sizes::staging bytes) and then tiled into its place.
static hipError_t pack_layer(const lb_block* blk, const lb_weights* w, const LayerW& L, void* stage,
                             hipStream_t s) {
    const lb_config& c = blk->cfg;
    const int d = c.d_model, dh = c.d_head, dff = c.d_ff;
    const Elem op = blk->op, dt = blk->dt;
    const bool tiled = dt == Elem::BF16;
    const size_t eo_row = (size_t)d * esz(op);
    // row-major destination of a matrix: its final place (fp32) or the stage
    auto dst = [&](void* final_place) { return tiled ? stage : final_place; };
    auto tile = [&](void* final_place, int rows, int K) {
        return tiled ? lb::launch_tile_weights(op, stage, final_place, rows, K, s) : hipSuccess;
    };
    // rotate_half layout: the rows of each q and k head are reordered so that
    // the projection puts dimensions i and i + d_head/2 side by side, where the
    // epilogue turns adjacent pairs; it stores them back in natural order
    const int perm_dh = c.rope_layout == LB_ROPE_HALF ? dh : 0;
    void* qkv = dst(L.w_qkv);
    hipError_t e = lb::launch_convert_rows(dt, op, w->wq, qkv, blk->qd, d, perm_dh, s);
    if (e == hipSuccess)
        e = lb::launch_convert_rows(dt, op, w->wk, (char*)qkv + (size_t)blk->qd * eo_row, blk->kvd, d, perm_dh, s);
    if (e == hipSuccess)
        e = lb::launch_convert(dt, op, w->wv, (char*)qkv + (size_t)(blk->qd + blk->kvd) * eo_row,
                               (size_t)blk->kvd * d, s);
    if (e == hipSuccess) e = tile(L.w_qkv, blk->nqkv, d);
    if (e == hipSuccess) e = lb::launch_convert(dt, op, w->wo, dst(L.w_o), (size_t)d * blk->qd, s);
    if (e == hipSuccess) e = tile(L.w_o, d, blk->qd);
    if (e == hipSuccess) e = lb::launch_pack_gate_up(dt, op, w->w_gate, w->w_up, dst(L.w_gu), dff, d, s);
    if (e == hipSuccess) e = tile(L.w_gu, 2 * dff, d);
    if (e == hipSuccess) e = lb::launch_convert(dt, op, w->w_down, dst(L.w_down), (size_t)d * dff, s);
    if (e == hipSuccess) e = tile(L.w_down, d, dff);
    if (e == hipSuccess) e = lb::launch_convert(dt, Elem::F32, w->attn_norm, L.g1, (size_t)d, s);
    if (e == hipSuccess) e = lb::launch_convert(dt, Elem::F32, w->ffn_norm, L.g2, (size_t)d, s);
    return e;
}

// A handle with the config, the RoPE table and the workspace, but no weights
// yet.  Synchronous.  On error *out stays NULL and the message is in
// g_init_error.
static lb_status create_core(const lb_config* cfg, Elem op_type, lb_block** out) {
    *out = nullptr;
    lb_status st = validate_config(cfg);
    if (st != LB_OK) return st;

    lb_block* blk = new lb_block();
    blk->cfg = *cfg;
    const lb_config& c = blk->cfg;
    blk->dt = c.dtype == LB_BF16 ? Elem::BF16 : Elem::F32;
    blk->op = op_type;
    if (hipGetDevice(&blk->dev) != hipSuccess) {
        delete blk;
        return fail(nullptr, LB_ERR_HIP, "hipGetDevice failed");
    }
    setup_static_scratch(blk->dev);
    const int d = c.d_model, dh = c.d_head, dff = c.d_ff;
    blk->qd = c.n_heads * dh;
    blk->kvd = c.n_kv_heads * dh;
    blk->nqkv = blk->qd + 2 * blk->kvd;
    const Elem op = blk->op, dt = blk->dt;
    const size_t eo = esz(op);
    const Sizes z = sizes_of(c);

    bool ok = dalloc(blk, &blk->rope, z.rope) && dalloc(blk, &blk->n1, z.n1) && dalloc(blk, &blk->n2, z.n2) &&
              dalloc(blk, &blk->q, z.q) && dalloc(blk, &blk->o, z.o) && dalloc(blk, &blk->z, z.z) &&
              dalloc(blk, &blk->h, z.h);
    if (ok && dt == Elem::BF16) {
        blk->ws_rows = z.ws_rows;
        blk->gpart_cap = z.gpart_floats;
        ok = dalloc(blk, &blk->kws, z.kws) && dalloc(blk, &blk->vws, z.vws) && dalloc(blk, &blk->part, z.part) &&
             dalloc(blk, &blk->gpart, z.gpart) && dalloc(blk, &blk->gcnt, z.gcnt) &&
             dalloc(blk, &blk->at_n1, z.at_n1) && dalloc(blk, &blk->at_o, z.at_o) && dalloc(blk, &blk->at_n2, z.at_n2) &&
             dalloc(blk, &blk->at_z, z.at_z);
        ok = ok && hipMemset(blk->gcnt, 0, z.gcnt) == hipSuccess;
    }
    if (!ok) {
        free_all(blk);
        delete blk;
        return fail(nullptr, LB_ERR_OOM, "device allocation failed");
    }

    // RoPE table: (cos, sin) of pos * speed_i, angles in fp64, speed_i =
    // theta^(-2i/d_head) ("The Evolving Transformer 04 LLaMA", 02 RoPE),
    // stretched as in Llama 3.1 when a scale factor is given ("From GPT-2 to
    // Llama", Positions become a rotation; the rule is stated in the header).
    std::vector<float2> table((size_t)c.max_seq_len * (dh / 2));
    for (int i = 0; i < dh / 2; ++i) {
        double freq = std::pow(c.rope_theta, -2.0 * (double)i / (double)dh);
        if (c.rope_scale_factor > 1.0) {
            const double wavelen = 2.0 * M_PI / freq;
            const double orig = c.rope_original_max_pos, lo = c.rope_low_freq_factor,
                         hi = c.rope_high_freq_factor, f = c.rope_scale_factor;
            if (wavelen > orig / lo) {
                freq /= f;
            } else if (wavelen >= orig / hi) {
                const double t = (orig / wavelen - lo) / (hi - lo);
                freq = (1.0 - t) * freq / f + t * freq;
            }
        }
        for (long pos = 0; pos < c.max_seq_len; ++pos) {
            const double a = (double)pos * freq;
            table[(size_t)pos * (dh / 2) + i] = make_float2((float)std::cos(a), (float)std::sin(a));
        }
    }

    hipStream_t s = nullptr;
    hipError_t e = hipStreamCreate(&s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(blk->rope, table.data(), table.size() * sizeof(float2), hipMemcpyHostToDevice, s);
    if (e == hipSuccess && dt == Elem::BF16) {
        // rows past a decode batch are read by the GEMMs (their results are
        // dropped): start them at zero
        e = hipMemsetAsync(blk->at_n1, 0, (size_t)kDecodeRows * d * eo, s);
        if (e == hipSuccess) e = hipMemsetAsync(blk->at_o, 0, (size_t)kDecodeRows * blk->qd * eo, s);
        if (e == hipSuccess) e = hipMemsetAsync(blk->at_n2, 0, (size_t)kDecodeRows * d * eo, s);
        if (e == hipSuccess) e = hipMemsetAsync(blk->at_z, 0, (size_t)kDecodeRows * dff * eo, s);
    }
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (s) hipStreamDestroy(s);
    if (e != hipSuccess) {
        const char* msg = hipGetErrorString(e);
        free_all(blk);
        delete blk;
        return fail(nullptr, LB_ERR_HIP, "workspace set-up failed: %s", msg);
    }
    *out = blk;
    return LB_OK;
}

// ---- range of the fp16 operand path ----------------------------------------------
// A bf16 weight widens to fp16 exactly from 2^-17 up to 65504 in magnitude
// (8 significant bits fit fp16's subnormal spacing 2^-24 from 2^-17 up), and
// every activation that a bf16 block rounds to an fp16 operand is bounded by
// its weights and gains:
//   |n1_k| <= sqrt(d) max|g1|, |n2_k| <= sqrt(d) max|g2|: the row divided by
//     its root mean square has Euclidean norm at most sqrt(d);
//   |q_j|, |k_j| <= sqrt(2) sqrt(d) ||g1 . Wq_j||: Cauchy-Schwarz, and RoPE
//     turns each pair within its norm; |v_j| <= sqrt(d) ||g1 . Wv_j||;
//   |o| <= max |v|: each output is a convex combination of value rows;
//   |z_j| <= |a_j| |u_j| <= d ||g2 . Wgate_j|| ||g2 . Wup_j||, as |SiLU(a)| <= |a|
//     (the same for every routed expert of a MoE block).
// AUTO and F16 take fp16 operands when every bound and every |w| stays below
// fp16's largest finite value and each weight row changes by at most 2^-11 of
// its norm in the conversion (fp16's own relative rounding); otherwise AUTO
// takes bf16 operands and F16 is refused.
static hipError_t row_stats(float* dev, const void* w, const void* g, int rows, int K, std::vector<float>& out) {
    out.assign((size_t)rows * 4, 0.0f);
    hipError_t e = lb::launch_weight_row_stats(w, g, rows, K, dev, nullptr);
    if (e == hipSuccess) e = hipMemcpy(out.data(), dev, out.size() * sizeof(float), hipMemcpyDeviceToHost);
    return e;
}

struct RangeCheck {
    bool fits = true;
    char why[256] = {0};
    void fail(const char* fmt, ...) {
        if (!fits) return;
        fits = false;
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(why, sizeof(why), fmt, ap);
        va_end(ap);
    }
    // fp16 limit with a margin for the rounding of the bounds themselves
    static constexpr double kLimit = 65504.0 * (1.0 - 1.0 / 256.0);
    void bound(const char* what, int layer, double v) {
        if (!(v <= kLimit)) fail("block %d: %s can reach %.6g, beyond fp16's range", layer, what, v);
    }
    // every weight in fp16 range and every row widened closely enough
    void weights(const char* name, int layer, const std::vector<float>& st, int rows) {
        for (int r = 0; r < rows && fits; ++r) {
            const float* p = &st[(size_t)r * 4];
            if (!(p[2] <= 65504.0f)) fail("block %d: |%s| reaches %.6g, beyond fp16's range", layer, name, p[2]);
            else if (!(p[1] <= std::ldexp(p[3], -22)))
                fail("block %d: row %d of %s loses more than 2^-11 of its norm in fp16", layer, r, name);
        }
    }
    // max over rows of sqrt(sum (g w)^2)
    static double max_gnorm(const std::vector<float>& st, int rows) {
        double m = 0.0;
        for (int r = 0; r < rows; ++r) m = std::max(m, std::sqrt((double)st[(size_t)r * 4]));
        return m;
    }
};

static lb_status check_f16_range(const lb_config& c, const lb_weights* ws, int n_layers, const lb_moe_config* moe,
                                 const lb_moe_weights* ew, RangeCheck* rc) {
    const int d = c.d_model, dh = c.d_head, dff = c.d_ff, qd = c.n_heads * dh, kvd = c.n_kv_heads * dh;
    long rows_max = std::max(std::max(qd, d), std::max(dff, 1));
    if (moe) rows_max = std::max(rows_max, (long)moe->n_experts * std::max(moe->d_ff_expert, d));
    float* dev = nullptr;
    if (hipMalloc(&dev, (size_t)rows_max * 4 * sizeof(float)) != hipSuccess) {
        (void)hipGetLastError();
        return fail(nullptr, LB_ERR_OOM, "device allocation failed (range check)");
    }
    const double sd = std::sqrt((double)d);
    std::vector<float> g1, g2, a, b;
    hipError_t e = hipSuccess;
    for (int l = 0; l < n_layers && e == hipSuccess && rc->fits; ++l) {
        const lb_weights& w = ws[l];
        e = row_stats(dev, w.attn_norm, nullptr, 1, d, g1);
        if (e == hipSuccess) e = row_stats(dev, w.ffn_norm, nullptr, 1, d, g2);
        if (e != hipSuccess) break;
        rc->bound("RMSNorm_1 output", l, sd * g1[2]);
        rc->bound("RMSNorm_2 output", l, sd * g2[2]);
        const struct { const char* name; const void* w; int rows; double f; } proj[3] = {
            {"wq", w.wq, qd, std::sqrt(2.0)}, {"wk", w.wk, kvd, std::sqrt(2.0)}, {"wv", w.wv, kvd, 1.0}};
        for (const auto& p : proj) {
            if ((e = row_stats(dev, p.w, w.attn_norm, p.rows, d, a)) != hipSuccess) break;
            rc->weights(p.name, l, a, p.rows);
            rc->bound(p.name[1] == 'q' ? "q" : (p.name[1] == 'k' ? "k" : "v (and the attention output)"), l,
                      p.f * sd * RangeCheck::max_gnorm(a, p.rows));
        }
        if (e != hipSuccess) break;
        if ((e = row_stats(dev, w.wo, nullptr, d, qd, a)) != hipSuccess) break;
        rc->weights("wo", l, a, d);
        if ((e = row_stats(dev, w.w_down, nullptr, d, dff, a)) != hipSuccess) break;
        rc->weights("w_down", l, a, d);
        // gate and up rows pair up in z
        auto ffn = [&](const char* what, const void* gate, const void* up, int rows) -> hipError_t {
            hipError_t er = row_stats(dev, gate, w.ffn_norm, rows, d, a);
            if (er == hipSuccess) er = row_stats(dev, up, w.ffn_norm, rows, d, b);
            if (er != hipSuccess) return er;
            rc->weights(what, l, a, rows);
            rc->weights(what, l, b, rows);
            double m = 0.0;
            for (int r = 0; r < rows; ++r)
                m = std::max(m, std::sqrt((double)a[(size_t)r * 4]) * std::sqrt((double)b[(size_t)r * 4]));
            rc->bound(what, l, (double)d * m);
            return hipSuccess;
        };
        if ((e = ffn("SwiGLU output z (w_gate, w_up)", w.w_gate, w.w_up, dff)) != hipSuccess) break;
        if (moe) {
            const int E = moe->n_experts, fe = moe->d_ff_expert;
            if ((e = row_stats(dev, ew->router, nullptr, E, d, a)) != hipSuccess) break;
            rc->weights("router", l, a, E);
            if ((e = ffn("expert SwiGLU output z", ew->w_gate, ew->w_up, E * fe)) != hipSuccess) break;
            if ((e = row_stats(dev, ew->w_down, nullptr, E * d, fe, a)) != hipSuccess) break;
            rc->weights("expert w_down", l, a, E * d);
        }
    }
    hipFree(dev);
    if (e != hipSuccess) return fail(nullptr, LB_ERR_HIP, "range check: %s", hipGetErrorString(e));
    return LB_OK;
}

// Operand type of the matrix products of a new handle (see above).
static lb_status choose_operands(const lb_config* cfg, const lb_weights* ws, int n_layers, const lb_moe_config* moe,
                                 const lb_moe_weights* ew, Elem* op) {
    lb_status st = validate_config(cfg);
    if (st != LB_OK) return st;
    if (cfg->dtype == LB_F32) {
        *op = Elem::F32;
        return LB_OK;
    }
    if (cfg->operands == LB_OPERANDS_BF16) {
        *op = Elem::BF16;
        return LB_OK;
    }
    RangeCheck rc;
    st = check_f16_range(*cfg, ws, n_layers, moe, ew, &rc);
    if (st != LB_OK) return st;
    if (rc.fits) {
        *op = Elem::F16;
        return LB_OK;
    }
    if (cfg->operands == LB_OPERANDS_F16) return fail(nullptr, LB_ERR_UNSUPPORTED, "fp16 operands: %s", rc.why);
    *op = Elem::BF16;
    return LB_OK;
}

// Allocate and pack n layers of weights into ls[0..n) (synchronous).
static lb_status load_layers(lb_block* blk, const lb_weights* w, int n, LayerW* ls) {
    for (int l = 0; l < n; ++l)
        if (!alloc_layer(blk, &ls[l])) return fail(nullptr, LB_ERR_OOM, "device allocation failed (weights of block %d)", l);
    // staging buffer of the tiling (bf16 blocks), freed before returning
    void* stage = nullptr;
    if (blk->dt == Elem::BF16 && hipMalloc(&stage, sizes_of(blk->cfg).staging) != hipSuccess) {
        (void)hipGetLastError();
        return fail(nullptr, LB_ERR_OOM, "device allocation failed (weight staging)");
    }
    hipStream_t s = nullptr;
    hipError_t e = hipStreamCreate(&s);
    for (int l = 0; l < n && e == hipSuccess; ++l) e = pack_layer(blk, &w[l], ls[l], stage, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (s) hipStreamDestroy(s);
    if (stage) hipFree(stage);
    if (e != hipSuccess) return fail(nullptr, LB_ERR_HIP, "weight packing failed: %s", hipGetErrorString(e));
    return LB_OK;
}

extern "C" lb_status llama_block_init(const lb_config* cfg, const lb_weights* w, lb_block** out) {
    g_init_error.clear();
    if (!out) return fail(nullptr, LB_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!cfg || !w) return fail(nullptr, LB_ERR_INVALID_ARG, "cfg or weights is NULL");
    if (!weights_complete(w)) return fail(nullptr, LB_ERR_INVALID_ARG, "a weight pointer is NULL");
    Elem op = Elem::F32;
    lb_status st = choose_operands(cfg, w, 1, nullptr, nullptr, &op);
    if (st != LB_OK) return st;
    lb_block* blk = nullptr;
    st = create_core(cfg, op, &blk);
    if (st != LB_OK) return st;
    st = load_layers(blk, w, 1, &blk->lw);
    if (st != LB_OK) {
        free_all(blk);
        delete blk;
        return st;
    }
    *out = blk;
    return LB_OK;
}

extern "C" lb_status llama_moe_block_init(const lb_config* cfg, const lb_weights* w, const lb_moe_config* moe,
                                          const lb_moe_weights* ew, lb_block** out) {
    g_init_error.clear();
    if (!out) return fail(nullptr, LB_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!cfg || !w || !moe || !ew) return fail(nullptr, LB_ERR_INVALID_ARG, "cfg, weights, moe or experts is NULL");
    if (!weights_complete(w) || !ew->router || !ew->w_gate || !ew->w_up || !ew->w_down)
        return fail(nullptr, LB_ERR_INVALID_ARG, "a weight pointer is NULL");
    const int E = moe->n_experts, K = moe->top_k, fe = moe->d_ff_expert;
    if (E < 1 || E > lb::kMoeMaxExperts)
        return fail(nullptr, LB_ERR_INVALID_ARG, "n_experts (%d) must be in [1, %d]", E, lb::kMoeMaxExperts);
    if (K < 1 || K > E || K > lb::kMoeMaxTopK)
        return fail(nullptr, LB_ERR_INVALID_ARG, "top_k (%d) must be in [1, min(n_experts, %d)]", K, lb::kMoeMaxTopK);
    if (fe < 1) return fail(nullptr, LB_ERR_INVALID_ARG, "d_ff_expert (%d) must be >= 1", fe);
    lb_status st = validate_config(cfg);
    if (st != LB_OK) return st;
    if (cfg->dtype != LB_BF16) return fail(nullptr, LB_ERR_UNSUPPORTED, "MoE blocks run in bf16 only");
    if (fe % 64 != 0) return fail(nullptr, LB_ERR_UNSUPPORTED, "d_ff_expert (%d) must be a multiple of 64", fe);
    if ((long)cfg->max_tokens * K > (1L << 24))
        return fail(nullptr, LB_ERR_UNSUPPORTED, "max_tokens * top_k exceeds 2^24");
    Elem op = Elem::F32;
    st = choose_operands(cfg, w, 1, moe, ew, &op);
    if (st != LB_OK) return st;
    lb_block* blk = nullptr;
    st = create_core(cfg, op, &blk);
    if (st != LB_OK) return st;
    blk->moe_E = E;
    blk->moe_K = K;
    blk->moe_fe = fe;
    const lb_config& c = blk->cfg;
    const size_t d = (size_t)c.d_model, T = (size_t)c.max_tokens, eo = esz(blk->op);
    bool ok = dalloc(blk, &blk->w_router, (size_t)E * d * eo) &&
              dalloc(blk, &blk->w_egu, (size_t)E * 2 * fe * d * eo) &&
              dalloc(blk, &blk->w_edown, (size_t)E * d * fe * eo) &&
              dalloc(blk, &blk->m_logits, T * E * 4) && dalloc(blk, &blk->m_sel, T * K * 4) &&
              dalloc(blk, &blk->m_wts, T * K * 4) && dalloc(blk, &blk->m_row_off, (size_t)(E + 1) * 4) &&
              dalloc(blk, &blk->m_tile_off, (size_t)(E + 1) * 4) && dalloc(blk, &blk->m_src, T * K * 4) &&
              dalloc(blk, &blk->m_slot, T * K * 4) && dalloc(blk, &blk->m_a, T * K * d * eo) &&
              dalloc(blk, &blk->m_z, T * K * fe * eo) && dalloc(blk, &blk->m_r, T * K * d * 4) &&
              dalloc(blk, &blk->m_hs, T * d * 4);
    if (!ok) st = fail(nullptr, LB_ERR_OOM, "device allocation failed (experts)");
    if (st == LB_OK) st = load_layers(blk, w, 1, &blk->lw);
    if (st == LB_OK) {
        hipStream_t s = nullptr;
        hipError_t e = hipStreamCreate(&s);
        const Elem dt = blk->dt, op = blk->op;
        const size_t ebytes = esz(dt);
        if (e == hipSuccess) e = lb::launch_convert(dt, op, ew->router, blk->w_router, (size_t)E * d, s);
        for (int x = 0; x < E && e == hipSuccess; ++x) {
            const size_t off = (size_t)x * fe * d;
            e = lb::launch_pack_gate_up(dt, op, (const char*)ew->w_gate + off * ebytes,
                                        (const char*)ew->w_up + off * ebytes,
                                        (char*)blk->w_egu + 2 * off * eo, fe, (int)d, s);
        }
        if (e == hipSuccess) e = lb::launch_convert(dt, op, ew->w_down, blk->w_edown, (size_t)E * d * fe, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (s) hipStreamDestroy(s);
        if (e != hipSuccess) st = fail(nullptr, LB_ERR_HIP, "expert weight packing failed: %s", hipGetErrorString(e));
    }
    if (st != LB_OK) {
        free_all(blk);
        delete blk;
        return st;
    }
    *out = blk;
    return LB_OK;
}

extern "C" lb_status llama_block_copy_routing(lb_block* blk, int32_t* sel, float* weights, float* logits,
                                              void* stream) {
    if (!blk) return LB_ERR_INVALID_ARG;
    blk->err.clear();
    if (blk->moe_E == 0) return fail(blk, LB_ERR_INVALID_ARG, "not a MoE block");
    const size_t M = (size_t)blk->last_m, K = (size_t)blk->moe_K, E = (size_t)blk->moe_E;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    if (sel) e = hipMemcpyAsync(sel, blk->m_sel, M * K * 4, hipMemcpyDefault, s);
    if (e == hipSuccess && weights) e = hipMemcpyAsync(weights, blk->m_wts, M * K * 4, hipMemcpyDefault, s);
    if (e == hipSuccess && logits) e = hipMemcpyAsync(logits, blk->m_logits, M * E * 4, hipMemcpyDefault, s);
    if (e != hipSuccess) return fail(blk, LB_ERR_HIP, "copy_routing: %s", hipGetErrorString(e));
    return LB_OK;
}

extern "C" void llama_block_destroy(lb_block* blk) {
    if (!blk) return;
    int cur = 0;
    hipGetDevice(&cur);
    hipSetDevice(blk->dev);
    hipDeviceSynchronize();
    profile_release(blk);
    free_all(blk);
    hipSetDevice(cur);
    delete blk;
}

static bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const char* pa = (const char*)a;
    const char* pb = (const char*)b;
    return pa < pb + nb && pb < pa + na;
}

// The MoE FFN after RMSNorm_2 ("Llama 4 From Scratch", The idea): the shared
// expert (the block's dense FFN) adds into h, the router picks each row's
// experts, the rows are grouped by expert, the experts run as grouped GEMMs,
// and the combine writes y = h + shared + sum of weighted expert outputs.
template <typename Mark>
static lb_status run_moe_ffn(lb_block* blk, const LayerW& L, const void* n2, void* z, int M, void* out,
                             const lb::SplitWs& ws, hipStream_t s, Mark& mark) {
    const lb_config& c = blk->cfg;
    const int d = c.d_model, dff = c.d_ff, E = blk->moe_E, K = blk->moe_K, fe = blk->moe_fe;
    const Elem op = blk->op;
    const int MK = M * K;
    mark(5);
    hipError_t e = lb::gemm_swiglu(op, n2, L.w_gu, M, 2 * dff, d, z, ws, s);
    if (e == hipSuccess) e = lb::launch_moe_router(op, n2, blk->w_router, M, d, E, K, blk->m_logits, blk->m_sel,
                                                   blk->m_wts, s);
    if (e == hipSuccess) e = lb::launch_moe_route(blk->m_sel, MK, E, blk->m_row_off, blk->m_tile_off, blk->m_src,
                                                  blk->m_slot, s);
    if (e == hipSuccess) e = lb::launch_moe_gather(op, n2, blk->m_src, MK, K, d, blk->m_a, s);
    if (e == hipSuccess) e = lb::launch_moe_grouped_swiglu(op, blk->m_a, blk->w_egu, blk->m_row_off,
                                                           blk->m_tile_off, E, MK, 2 * fe, d, blk->m_z, s);
    if (e != hipSuccess) return fail(blk, LB_ERR_HIP, "MoE gate/up: %s", hipGetErrorString(e));
    mark(6);
    e = lb::gemm_resid(op, Elem::F32, z, L.w_down, M, d, dff, blk->h, blk->m_hs, ws, s);
    if (e == hipSuccess) e = lb::launch_moe_grouped_down(op, blk->m_z, blk->w_edown, blk->m_row_off, blk->m_tile_off,
                                                         E, MK, d, fe, blk->m_r, s);
    if (e == hipSuccess) e = lb::launch_moe_combine(blk->dt, blk->m_hs, blk->m_r, blk->m_slot, blk->m_wts, M, K, d,
                                                    out, s);
    if (e != hipSuccess) return fail(blk, LB_ERR_HIP, "MoE down: %s", hipGetErrorString(e));
    return LB_OK;
}

// sp: start position of every sequence (validated by the caller).  wk: the
// scratch buffers; stage_state: record the layout of this call's stage
// buffers for llama_block_copy_stage (calls on the handle's own workspace).
static lb_status run_forward(lb_block* blk, const LayerW& L, const void* x, int B, int S,
                             const lb::SeqPos& sp, const lb_kv_cache* kv, void* out, hipStream_t s,
                             const Workspace& wk, bool stage_state = true) {
    const lb_config& c = blk->cfg;
    const int M = B * S, d = c.d_model, dh = c.d_head, nkv = c.n_kv_heads, dff = c.d_ff;
    const int cap = kv->max_seq_len;
    const Elem op = blk->op, dt = blk->dt;
    hipError_t e;
    hipEvent_t* ev = nullptr;
    if (blk->profiling) {
        const int slot = blk->next_slot;
        for (size_t i = 0; i < blk->pending.size(); ++i) {
            if (blk->pending[i] == slot) {  // ring full: fold the oldest use of this slot in first
                e = profile_collect(blk, slot);
                if (e != hipSuccess) return fail(blk, LB_ERR_HIP, "profiling: %s", hipGetErrorString(e));
                blk->pending.erase(blk->pending.begin() + i);
                break;
            }
        }
        ev = &blk->events[(size_t)slot * (LB_NUM_STAGES + 1)];
        blk->pending.push_back(slot);
        blk->next_slot = (slot + 1) % kProfileSlots;
    }
    const uint32_t pmask = blk->profile_mask;
    auto mark = [&](int i) {
        if (ev && mark_needed(pmask, i)) hipEventRecord(ev[i], s);
    };

    // decode batches of <= kDecodeRows sequences run the weight-streaming
    // GEMMs on k-step tiled activations and weights
    const bool dec = dt == Elem::BF16 && S == 1 && M <= kDecodeRows;
    const int mt = dec ? lb::decode_row_tiles(M) : 0;
    const lb::SplitWs ws{wk.gpart, wk.gpart_cap, wk.gcnt, wk.gcnt ? lb::kSplitCounters : 0};
    void* n1 = dec ? wk.at_n1 : wk.n1;
    void* o = dec ? wk.at_o : wk.o;
    const bool moe = blk->moe_E > 0;
    // MoE blocks keep n2 and z row-major: the router and the grouping read n2 by rows
    const bool dec_ffn = dec && !moe;
    void* n2 = dec_ffn ? wk.at_n2 : wk.n2;
    void* z = dec_ffn ? wk.at_z : wk.z;

    mark(0);
    e = lb::launch_rmsnorm(dt, op, x, L.g1, n1, M, d, (float)c.norm_eps, mt, s);
    if (e != hipSuccess) return fail(blk, LB_ERR_HIP, "rmsnorm_1: %s", hipGetErrorString(e));

    // device-held positions: shape the launches for the largest start the
    // kernels can read (they clamp to it)
    int max_start = sp.dev ? sp.lim : sp.base, all_zero = !sp.dev && sp.base == 0;
    if (!sp.dev && sp.ragged) {
        max_start = 0;
        all_zero = 1;
        for (int b = 0; b < B; ++b) {
            max_start = std::max(max_start, sp.pos[b]);
            all_zero &= sp.pos[b] == 0;
        }
    }
    const bool ws_kv = (dt == Elem::BF16) && S > 1 && all_zero;
    const int s_stride = (S + 7) & ~7;
    lb::QkvEpi qe;
    qe.q = wk.q;
    qe.kws = ws_kv ? wk.kws : nullptr;
    qe.vws = ws_kv ? wk.vws : nullptr;
    qe.kc = kv->k;
    qe.vc = kv->v;
    qe.rope = blk->rope;
    qe.S = S;
    qe.sp = sp;
    qe.cap = cap;
    qe.s_stride = s_stride;
    qe.nkv = nkv;
    qe.dh = dh;
    qe.qd = blk->qd;
    qe.rope_half = c.rope_layout == LB_ROPE_HALF;
    mark(1);
    if (dec) e = lb::decode_qkv(op, dt, n1, L.w_qkv, M, blk->nqkv, d, qe, ws, s);
    else e = lb::gemm_qkv(op, dt, n1, L.w_qkv, M, blk->nqkv, d, qe, ws, s);
    if (e != hipSuccess) return fail(blk, LB_ERR_HIP, "qkv projection: %s", hipGetErrorString(e));

    lb::AttnArgs a;
    a.q = wk.q;
    a.o = o;
    a.B = B;
    a.S = S;
    a.sp = sp;
    a.max_start = max_start;
    a.H = c.n_heads;
    a.nkv = nkv;
    a.dh = dh;
    if (ws_kv) {
        a.k = wk.kws;
        a.v = wk.vws;
        a.kv_bg = (long)s_stride * dh;
    } else {
        a.k = kv->k;
        a.v = kv->v;
        a.kv_bg = (long)cap * dh;
    }
    mark(2);
    if (dt == Elem::F32) e = lb::attn_simple(a, s);
    else if (S == 1) e = lb::attn_decode(op, dt, a, wk.part, mt, s);
    else e = lb::attn_prefill(op, ws_kv ? op : dt, a, s);
    if (e != hipSuccess) return fail(blk, LB_ERR_HIP, "attention: %s", hipGetErrorString(e));

    mark(3);
    if (dec) e = lb::decode_resid(op, dt, o, L.w_o, M, d, blk->qd, x, wk.h, ws, s);
    else e = lb::gemm_resid(op, dt, o, L.w_o, M, d, blk->qd, x, wk.h, ws, s);
    if (e != hipSuccess) return fail(blk, LB_ERR_HIP, "o projection: %s", hipGetErrorString(e));
    mark(4);
    e = lb::launch_rmsnorm(Elem::F32, op, wk.h, L.g2, n2, M, d, (float)c.norm_eps, dec_ffn ? mt : 0, s);
    if (e != hipSuccess) return fail(blk, LB_ERR_HIP, "rmsnorm_2: %s", hipGetErrorString(e));
    if (stage_state) {
        blk->last_mt = mt;
        blk->last_ffn_mt = dec_ffn ? mt : 0;
        blk->last_m = M;
    }
    if (moe) {
        lb_status st = run_moe_ffn(blk, L, n2, z, B * S, out, ws, s, mark);
        if (st == LB_OK) mark(7);
        return st;
    }
    mark(5);
    if (dec) e = lb::decode_swiglu(op, n2, L.w_gu, M, 2 * dff, d, z, ws, s);
    else e = lb::gemm_swiglu(op, n2, L.w_gu, M, 2 * dff, d, z, ws, s);
    if (e != hipSuccess) return fail(blk, LB_ERR_HIP, "gate/up projection: %s", hipGetErrorString(e));
    mark(6);
    if (dec) e = lb::decode_out(op, dt, z, L.w_down, M, d, dff, wk.h, out, ws, s);
    else e = lb::gemm_out(op, dt, z, L.w_down, M, d, dff, wk.h, out, ws, s);
    if (e != hipSuccess) return fail(blk, LB_ERR_HIP, "down projection: %s", hipGetErrorString(e));
    mark(7);
    return LB_OK;
}

// Checks every forward shares: pointers, sizes, the cache and overlap.
static lb_status check_call(lb_block* blk, const void* x, int32_t batch, int32_t seq_len,
                            const lb_kv_cache* kv, void* out) {
    const lb_config& c = blk->cfg;
    if (!x || !out || !kv || !kv->k || !kv->v)
        return fail(blk, LB_ERR_INVALID_ARG, "x, out, kv, kv->k and kv->v must be non-NULL");
    if (batch < 1 || seq_len < 1)
        return fail(blk, LB_ERR_INVALID_ARG, "batch (%d) and seq_len (%d) must be >= 1", batch, seq_len);
    if ((long)batch * seq_len > c.max_tokens)
        return fail(blk, LB_ERR_INVALID_ARG, "batch*seq_len (%ld) exceeds max_tokens (%d)",
                    (long)batch * seq_len, c.max_tokens);
    if (batch > kv->batch)
        return fail(blk, LB_ERR_INVALID_ARG, "batch (%d) exceeds the cache's batch (%d)", batch, kv->batch);
    if (kv->max_seq_len < 1)
        return fail(blk, LB_ERR_INVALID_ARG, "the cache's max_seq_len (%d) must be >= 1", kv->max_seq_len);
    if (blk->dt == Elem::BF16 && kv->max_seq_len % 8 != 0)
        return fail(blk, LB_ERR_UNSUPPORTED, "bf16 caches need max_seq_len % 8 == 0 (got %d)", kv->max_seq_len);
    const size_t act = (size_t)batch * seq_len * c.d_model * esz(blk->dt);
    if (overlap(x, act, out, act)) return fail(blk, LB_ERR_INVALID_ARG, "out overlaps x");
    return LB_OK;
}

// Start positions of a call: host values (starts == nullptr: every sequence
// at start_pos), each checked against cap (the smallest capacity of the
// caches the call writes), or (dev != nullptr) a device array read by the
// kernels, clamped there to the last start that fits.
static lb_status make_positions(lb_block* blk, int32_t batch, int32_t seq_len, int32_t start_pos,
                                const int32_t* starts, const int32_t* dev, int cap, lb::SeqPos* sp) {
    const lb_config& c = blk->cfg;
    sp->base = start_pos;
    sp->ragged = starts != nullptr;
    for (int b = 0; b < lb::kMaxRagged; ++b) sp->pos[b] = 0;
    sp->dev = dev;
    sp->lim = std::min(c.max_seq_len, cap) - seq_len;
    if (dev) {
        if (sp->lim < 0)
            return fail(blk, LB_ERR_INVALID_ARG, "seq_len (%d) exceeds max_seq_len (config %d, cache %d)", seq_len,
                        c.max_seq_len, cap);
        return LB_OK;
    }
    if (starts && batch > lb::kMaxRagged)
        return fail(blk, LB_ERR_INVALID_ARG, "a ragged forward takes at most %d sequences (got %d)",
                    lb::kMaxRagged, batch);
    for (int b = 0; b < (starts ? batch : 1); ++b) {
        const int32_t p = starts ? starts[b] : start_pos;
        if (p < 0) return fail(blk, LB_ERR_INVALID_ARG, "start_pos of sequence %d (%d) < 0", b, p);
        if ((long)p + seq_len > c.max_seq_len || (long)p + seq_len > cap)
            return fail(blk, LB_ERR_INVALID_ARG,
                        "start_pos+seq_len of sequence %d (%ld) exceeds max_seq_len (config %d, cache %d)",
                        b, (long)p + seq_len, c.max_seq_len, cap);
        if (starts) sp->pos[b] = p;
    }
    return LB_OK;
}

// Runs fn() with blk's device current, restoring the caller's afterwards.
template <typename F>
static lb_status on_device(lb_block* blk, F fn) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return fail(blk, LB_ERR_HIP, "hipGetDevice failed");
    if (cur != blk->dev) hipSetDevice(blk->dev);
    lb_status st = fn();
    if (cur != blk->dev) hipSetDevice(cur);
    return st;
}

// Validation and launch shared by the uniform and the ragged entry points;
// starts == nullptr: every sequence at start_pos.
static lb_status forward_checked(lb_block* blk, const void* x, int32_t batch, int32_t seq_len,
                                 int32_t start_pos, const int32_t* starts, const lb_kv_cache* kv,
                                 void* out, void* stream) {
    if (!blk) return LB_ERR_INVALID_ARG;
    blk->err.clear();
    lb_status st = check_call(blk, x, batch, seq_len, kv, out);
    if (st != LB_OK) return st;
    lb::SeqPos sp;
    st = make_positions(blk, batch, seq_len, start_pos, starts, nullptr, kv->max_seq_len, &sp);
    if (st != LB_OK) return st;
    return on_device(blk, [&] {
        return run_forward(blk, blk->lw, x, batch, seq_len, sp, kv, out, (hipStream_t)stream, handle_workspace(blk));
    });
}

extern "C" lb_status llama_block_forward(lb_block* blk, const void* x, int32_t batch, int32_t seq_len,
                                         int32_t start_pos, const lb_kv_cache* kv, void* out,
                                         void* stream) {
    return forward_checked(blk, x, batch, seq_len, start_pos, nullptr, kv, out, stream);
}

extern "C" lb_status llama_block_forward_ragged(lb_block* blk, const void* x, int32_t batch,
                                                int32_t seq_len, const int32_t* start_pos,
                                                const lb_kv_cache* kv, void* out, void* stream) {
    if (blk && !start_pos) {
        blk->err.clear();
        return fail(blk, LB_ERR_INVALID_ARG, "start_pos must be non-NULL");
    }
    return forward_checked(blk, x, batch, seq_len, 0, start_pos, kv, out, stream);
}

// Decode forward on the static scratch: the buffers of a decode step of at most
// kDecodeRows tokens, each 256-byte aligned, then the split-K partials in what
// is left.
extern "C" lb_status llama_block_forward_decode_static(lb_block* blk, const void* x, int32_t batch,
                                                       int32_t start_pos, const lb_kv_cache* kv, void* out,
                                                       void* stream) {
    if (!blk) return LB_ERR_INVALID_ARG;
    blk->err.clear();
    if (blk->dt != Elem::BF16 || blk->moe_E > 0)
        return fail(blk, LB_ERR_UNSUPPORTED, "the static-scratch decode runs dense bf16 blocks only");
    lb_status st = check_call(blk, x, batch, 1, kv, out);
    if (st != LB_OK) return st;
    if (batch > kDecodeRows)
        return fail(blk, LB_ERR_UNSUPPORTED, "the static-scratch decode takes at most %d sequences (got %d)",
                    kDecodeRows, batch);
    lb::SeqPos sp;
    st = make_positions(blk, batch, 1, start_pos, nullptr, nullptr, kv->max_seq_len, &sp);
    if (st != LB_OK) return st;
    const lb_config& c = blk->cfg;
    const size_t eo = esz(blk->op), R = kDecodeRows;
    auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
    const size_t sz[7] = {al(R * c.d_model * eo), al(R * blk->qd * eo), al(R * blk->qd * eo),
                          al(R * c.d_model * 4), al(R * c.d_model * eo), al(R * c.d_ff * eo),
                          al(lb::decode_partials_floats(batch, c.n_heads, c.d_head, c.max_seq_len) * 4)};
    size_t need = 0;
    for (size_t b : sz) need += b;
    if (need > (size_t)LB_STATIC_SCRATCH_BYTES)
        return fail(blk, LB_ERR_UNSUPPORTED,
                    "a decode step of this block needs %zu bytes of scratch, more than the static %zu", need,
                    (size_t)LB_STATIC_SCRATCH_BYTES);
    char* base = (char*)(blk->dev >= 0 && blk->dev < kMaxDevices ? g_scratch[blk->dev].load(std::memory_order_acquire)
                                                                 : nullptr);
    if (!base) return fail(blk, LB_ERR_HIP, "the static scratch of device %d is not available", blk->dev);
    Workspace w;
    char* p = base;
    w.at_n1 = p, p += sz[0];
    w.q = p, p += sz[1];
    w.at_o = p, p += sz[2];
    w.h = (float*)p, p += sz[3];
    w.at_n2 = p, p += sz[4];
    w.at_z = p, p += sz[5];
    w.part = (float*)p, p += sz[6];
    w.gpart = (float*)p;
    w.gpart_cap = ((size_t)LB_STATIC_SCRATCH_BYTES - need) / sizeof(float);
    return on_device(blk, [&] {
        return run_forward(blk, blk->lw, x, batch, 1, sp, kv, out, (hipStream_t)stream, w, false);
    });
}

// ---- stacks of blocks ------------------------------------------------------------
// N blocks sharing one workspace and RoPE table, each with its own weights and
// cache, then the final RMSNorm ("The Evolving Transformer 04 LLaMA", 07
// ASSEMBLE LLAMA).  Block outputs pass between blocks in the config's dtype,
// as the block's own interface hands them over.
struct lb_stack {
    lb_block* core = nullptr;  // config, workspace, RoPE table; owns every allocation
    std::vector<LayerW> layers;
    float* g_final = nullptr;
    void* act[2] = {nullptr, nullptr};  // block outputs when the caller keeps none
};

struct lb_stack_graph {
    lb_stack* st = nullptr;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
};

extern "C" lb_status llama_stack_init(const lb_config* cfg, int32_t n_layers, const lb_weights* layers,
                                      const void* final_norm, lb_stack** out) {
    g_init_error.clear();
    if (!out) return fail(nullptr, LB_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!cfg || !layers || !final_norm) return fail(nullptr, LB_ERR_INVALID_ARG, "cfg, layers or final_norm is NULL");
    if (n_layers < 1 || n_layers > LB_MAX_STACK_LAYERS)
        return fail(nullptr, LB_ERR_INVALID_ARG, "n_layers (%d) must be in [1, %d]", n_layers, LB_MAX_STACK_LAYERS);
    for (int l = 0; l < n_layers; ++l)
        if (!weights_complete(&layers[l]))
            return fail(nullptr, LB_ERR_INVALID_ARG, "a weight pointer of block %d is NULL", l);
    Elem op = Elem::F32;
    lb_status st = choose_operands(cfg, layers, n_layers, nullptr, nullptr, &op);
    if (st != LB_OK) return st;
    lb_block* blk = nullptr;
    st = create_core(cfg, op, &blk);
    if (st != LB_OK) return st;
    lb_stack* sk = new lb_stack();
    sk->core = blk;
    sk->layers.resize((size_t)n_layers);
    const Sizes z = sizes_of(blk->cfg);
    bool ok = dalloc(blk, &sk->g_final, z.g_final) && dalloc(blk, &sk->act[0], z.act) &&
              dalloc(blk, &sk->act[1], z.act);
    st = ok ? load_layers(blk, layers, n_layers, sk->layers.data())
            : fail(nullptr, LB_ERR_OOM, "device allocation failed");
    if (st == LB_OK) {
        hipError_t e = lb::launch_convert(blk->dt, Elem::F32, final_norm, sk->g_final, (size_t)blk->cfg.d_model, nullptr);
        if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
        if (e != hipSuccess) st = fail(nullptr, LB_ERR_HIP, "final norm gain: %s", hipGetErrorString(e));
    }
    if (st != LB_OK) {
        free_all(blk);
        delete blk;
        delete sk;
        return st;
    }
    *out = sk;
    return LB_OK;
}

extern "C" void llama_stack_destroy(lb_stack* sk) {
    if (!sk) return;
    llama_block_destroy(sk->core);
    delete sk;
}

extern "C" int32_t llama_stack_num_layers(const lb_stack* sk) { return sk ? (int32_t)sk->layers.size() : 0; }

extern "C" const char* llama_stack_last_error(const lb_stack* sk) {
    return llama_block_last_error(sk ? sk->core : nullptr);
}

// Checks of a stack call; *cap receives the smallest capacity of the caches.
static lb_status check_stack_call(lb_stack* sk, const void* x, int32_t batch, int32_t seq_len,
                                  const lb_kv_cache* kv, void* out, void* hidden, int* cap) {
    lb_block* blk = sk->core;
    if (!kv) return fail(blk, LB_ERR_INVALID_ARG, "kv must be non-NULL");
    const int L = (int)sk->layers.size();
    *cap = INT32_MAX;
    for (int l = 0; l < L; ++l) {
        lb_status st = check_call(blk, x, batch, seq_len, &kv[l], out);
        if (st != LB_OK) return st;
        *cap = std::min(*cap, kv[l].max_seq_len);
    }
    const size_t act = (size_t)batch * seq_len * blk->cfg.d_model * esz(blk->dt);
    if (hidden && (overlap(hidden, act * L, x, act) || overlap(hidden, act * L, out, act)))
        return fail(blk, LB_ERR_INVALID_ARG, "hidden overlaps x or out");
    return LB_OK;
}

// Enqueue every block and the final norm (arguments validated).
static lb_status stack_run(lb_stack* sk, const void* x, int B, int S, const lb::SeqPos& sp,
                           const lb_kv_cache* kv, void* out, void* hidden, hipStream_t s) {
    lb_block* blk = sk->core;
    const lb_config& c = blk->cfg;
    const size_t act = (size_t)B * S * c.d_model * esz(blk->dt);
    const void* in = x;
    for (size_t l = 0; l < sk->layers.size(); ++l) {
        void* o = hidden ? (char*)hidden + l * act : sk->act[l & 1];
        lb_status st = run_forward(blk, sk->layers[l], in, B, S, sp, &kv[l], o, s, handle_workspace(blk));
        if (st != LB_OK) return st;
        in = o;
    }
    hipError_t e = lb::launch_rmsnorm(blk->dt, blk->dt, in, sk->g_final, out, B * S, c.d_model,
                                      (float)c.norm_eps, 0, s);
    if (e != hipSuccess) return fail(blk, LB_ERR_HIP, "final norm: %s", hipGetErrorString(e));
    return LB_OK;
}

extern "C" lb_status llama_stack_forward(lb_stack* sk, const void* x, int32_t batch, int32_t seq_len,
                                         int32_t start_pos, const int32_t* starts, const lb_kv_cache* kv,
                                         void* out, void* hidden, void* stream) {
    if (!sk) return LB_ERR_INVALID_ARG;
    lb_block* blk = sk->core;
    blk->err.clear();
    int cap = 0;
    lb_status st = check_stack_call(sk, x, batch, seq_len, kv, out, hidden, &cap);
    if (st != LB_OK) return st;
    lb::SeqPos sp;
    st = make_positions(blk, batch, seq_len, start_pos, starts, nullptr, cap, &sp);
    if (st != LB_OK) return st;
    return on_device(blk, [&] { return stack_run(sk, x, batch, seq_len, sp, kv, out, hidden, (hipStream_t)stream); });
}

static lb_status stack_device_pos(lb_stack* sk, const void* x, int32_t batch, int32_t seq_len, int32_t* positions,
                                  int32_t advance, const lb_kv_cache* kv, void* out, void* hidden, hipStream_t s) {
    lb_block* blk = sk->core;
    if (!positions) return fail(blk, LB_ERR_INVALID_ARG, "positions must be non-NULL");
    int cap = 0;
    lb_status st = check_stack_call(sk, x, batch, seq_len, kv, out, hidden, &cap);
    if (st != LB_OK) return st;
    lb::SeqPos sp;
    st = make_positions(blk, batch, seq_len, 0, nullptr, positions, cap, &sp);
    if (st != LB_OK) return st;
    st = stack_run(sk, x, batch, seq_len, sp, kv, out, hidden, s);
    if (st != LB_OK || !advance) return st;
    hipError_t e = lb::launch_advance_positions(positions, batch, seq_len, s);
    if (e != hipSuccess) return fail(blk, LB_ERR_HIP, "advance positions: %s", hipGetErrorString(e));
    return LB_OK;
}

extern "C" lb_status llama_stack_forward_device_pos(lb_stack* sk, const void* x, int32_t batch, int32_t seq_len,
                                                    int32_t* positions, int32_t advance, const lb_kv_cache* kv,
                                                    void* out, void* hidden, void* stream) {
    if (!sk) return LB_ERR_INVALID_ARG;
    sk->core->err.clear();
    return on_device(sk->core, [&] {
        return stack_device_pos(sk, x, batch, seq_len, positions, advance, kv, out, hidden, (hipStream_t)stream);
    });
}

extern "C" lb_status llama_stack_graph_create(lb_stack* sk, const void* x, int32_t batch, int32_t seq_len,
                                              int32_t* positions, const lb_kv_cache* kv, void* out,
                                              lb_stack_graph** g) {
    if (!sk) return LB_ERR_INVALID_ARG;
    lb_block* blk = sk->core;
    blk->err.clear();
    if (!g) return fail(blk, LB_ERR_INVALID_ARG, "g is NULL");
    *g = nullptr;
    if (blk->profiling) return fail(blk, LB_ERR_INVALID_ARG, "stage profiling is on");
    // the same checks the capture would run, before anything is captured
    int cap = 0;
    lb_status st = check_stack_call(sk, x, batch, seq_len, kv, out, nullptr, &cap);
    if (st != LB_OK) return st;
    if (!positions) return fail(blk, LB_ERR_INVALID_ARG, "positions must be non-NULL");
    lb::SeqPos probe;
    st = make_positions(blk, batch, seq_len, 0, nullptr, positions, cap, &probe);
    if (st != LB_OK) return st;
    return on_device(blk, [&]() -> lb_status {
        hipStream_t s = nullptr;
        if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess)
            return fail(blk, LB_ERR_HIP, "hipStreamCreate failed");
        hipGraph_t graph = nullptr;
        hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeRelaxed);
        lb_status rs = LB_OK;
        if (e == hipSuccess) {
            rs = stack_device_pos(sk, x, batch, seq_len, positions, 1, kv, out, nullptr, s);
            e = hipStreamEndCapture(s, &graph);  // ends the capture whatever happened in it
        }
        hipStreamDestroy(s);
        if (rs != LB_OK) {
            if (graph) hipGraphDestroy(graph);
            return rs;
        }
        if (e != hipSuccess) {
            if (graph) hipGraphDestroy(graph);
            return fail(blk, LB_ERR_HIP, "graph capture: %s", hipGetErrorString(e));
        }
        hipGraphExec_t exec = nullptr;
        e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
        if (e != hipSuccess) {
            hipGraphDestroy(graph);
            return fail(blk, LB_ERR_HIP, "graph instantiate: %s", hipGetErrorString(e));
        }
        lb_stack_graph* sg = new lb_stack_graph();
        sg->st = sk;
        sg->graph = graph;
        sg->exec = exec;
        *g = sg;
        return LB_OK;
    });
}

extern "C" lb_status llama_stack_graph_launch(lb_stack_graph* g, void* stream) {
    if (!g) return LB_ERR_INVALID_ARG;
    lb_block* blk = g->st->core;
    blk->err.clear();
    return on_device(blk, [&]() -> lb_status {
        hipError_t e = hipGraphLaunch(g->exec, (hipStream_t)stream);
        if (e != hipSuccess) return fail(blk, LB_ERR_HIP, "graph launch: %s", hipGetErrorString(e));
        return LB_OK;
    });
}

extern "C" void llama_stack_graph_destroy(lb_stack_graph* g) {
    if (!g) return;
    int cur = 0;
    hipGetDevice(&cur);
    hipSetDevice(g->st->core->dev);
    hipDeviceSynchronize();
    if (g->exec) hipGraphExecDestroy(g->exec);
    if (g->graph) hipGraphDestroy(g->graph);
    hipSetDevice(cur);
    delete g;
}

static bool stage_buffer(const lb_block* blk, lb_stage which, const void** ptr, Elem* elem, int64_t* cols) {
    const lb_config& c = blk->cfg;
    switch (which) {
        case LB_STAGE_N1: *ptr = blk->n1; *elem = blk->op; *cols = c.d_model; return true;
        case LB_STAGE_Q: *ptr = blk->q; *elem = blk->op; *cols = blk->qd; return true;
        case LB_STAGE_O: *ptr = blk->o; *elem = blk->op; *cols = blk->qd; return true;
        case LB_STAGE_H: *ptr = blk->h; *elem = Elem::F32; *cols = c.d_model; return true;
        case LB_STAGE_N2: *ptr = blk->n2; *elem = blk->op; *cols = c.d_model; return true;
        case LB_STAGE_Z: *ptr = blk->z; *elem = blk->op; *cols = c.d_ff; return true;
        case LB_STAGE_ROUTED:
            if (blk->moe_E == 0) return false;
            *ptr = blk->m_r; *elem = Elem::F32; *cols = c.d_model; return true;
    }
    return false;
}

static lb_elem to_abi(Elem e) {
    return e == Elem::F32 ? LB_ELEM_F32 : (e == Elem::BF16 ? LB_ELEM_BF16 : LB_ELEM_F16);
}

extern "C" lb_elem llama_block_operand_type(const lb_block* blk) {
    return blk ? to_abi(blk->op) : LB_ELEM_F32;
}

extern "C" lb_elem llama_stack_operand_type(const lb_stack* sk) {
    return sk ? to_abi(sk->core->op) : LB_ELEM_F32;
}

extern "C" lb_status llama_block_footprint(const lb_config* cfg, int32_t n_layers, lb_footprint* out) {
    if (!cfg || !out) return fail(nullptr, LB_ERR_INVALID_ARG, "cfg or out is NULL");
    if (n_layers < 0 || n_layers > LB_MAX_STACK_LAYERS)
        return fail(nullptr, LB_ERR_INVALID_ARG, "n_layers (%d) must be in [0, %d]", n_layers, LB_MAX_STACK_LAYERS);
    lb_status st = validate_config(cfg);
    if (st != LB_OK) return st;
    const Sizes z = sizes_of(*cfg);
    out->weights = z.layer() * (uint64_t)(n_layers > 0 ? n_layers : 1);
    out->workspace = z.workspace() + (n_layers > 0 ? (uint64_t)z.g_final + 2 * (uint64_t)z.act : 0);
    out->init_staging = z.staging;
    return LB_OK;
}

extern "C" uint64_t llama_block_device_bytes(const lb_block* blk) { return blk ? blk->device_bytes : 0; }

extern "C" uint64_t llama_stack_device_bytes(const lb_stack* sk) { return sk ? sk->core->device_bytes : 0; }

extern "C" lb_status llama_block_stage_info(const lb_block* blk, lb_stage which, lb_elem* elem, int64_t* cols) {
    if (!blk || !elem || !cols) return LB_ERR_INVALID_ARG;
    const void* p;
    Elem e;
    if (!stage_buffer(blk, which, &p, &e, cols)) return LB_ERR_INVALID_ARG;
    *elem = to_abi(e);
    return LB_OK;
}

extern "C" lb_status llama_block_copy_stage(lb_block* blk, lb_stage which, void* dst, size_t bytes, void* stream) {
    if (!blk) return LB_ERR_INVALID_ARG;
    const void* p;
    Elem e;
    int64_t cols;
    if (!dst || !stage_buffer(blk, which, &p, &e, &cols))
        return fail(blk, LB_ERR_INVALID_ARG, "bad stage or NULL destination");
    const size_t rows_per_token = which == LB_STAGE_ROUTED ? (size_t)blk->moe_K : 1;
    const size_t cap = (size_t)blk->cfg.max_tokens * rows_per_token * (size_t)cols * esz(e);
    if (bytes > cap) return fail(blk, LB_ERR_INVALID_ARG, "%zu bytes exceed the stage buffer (%zu)", bytes, cap);
    if (which == LB_STAGE_ROUTED) {
        // expert rows are stored grouped by expert: row slot[t*K + j] holds
        // pair (t, j); gather whole rows (16-byte pieces) into pair order
        hipPointerAttribute_t attr{};
        if (hipPointerGetAttributes(&attr, dst) != hipSuccess || attr.type != hipMemoryTypeDevice) {
            (void)hipGetLastError();
            return fail(blk, LB_ERR_INVALID_ARG, "the routed stage is copied to device memory only");
        }
        const size_t row_bytes = (size_t)cols * 4;
        if (bytes % row_bytes != 0 || bytes / row_bytes > (size_t)blk->last_m * rows_per_token)
            return fail(blk, LB_ERR_INVALID_ARG, "copy_stage: the routed stage copies whole rows of the last forward");
        const int rows = (int)(bytes / row_bytes);
        hipError_t err = lb::launch_moe_gather(Elem::F16, blk->m_r, blk->m_slot, rows, 1, (int)cols * 2, dst,
                                               (hipStream_t)stream);
        if (err != hipSuccess) return fail(blk, LB_ERR_HIP, "copy_stage: %s", hipGetErrorString(err));
        return LB_OK;
    }
    const int tiled_mt = (which == LB_STAGE_N2 || which == LB_STAGE_Z) ? blk->last_ffn_mt : blk->last_mt;
    if (tiled_mt > 0 && which != LB_STAGE_Q && which != LB_STAGE_H) {
        // the last forward was a decode: this stage lives in the tiled layout;
        // lay it out row-major in the (idle) prefill buffer first
        const void* t = which == LB_STAGE_N1 ? blk->at_n1
                        : which == LB_STAGE_O ? blk->at_o
                        : which == LB_STAGE_N2 ? blk->at_n2 : blk->at_z;
        hipError_t err = lb::launch_untile(e, t, const_cast<void*>(p), blk->last_m, (int)cols, tiled_mt,
                                           (hipStream_t)stream);
        if (err != hipSuccess) return fail(blk, LB_ERR_HIP, "copy_stage: %s", hipGetErrorString(err));
    }
    hipError_t err = hipMemcpyAsync(dst, p, bytes, hipMemcpyDefault, (hipStream_t)stream);
    if (err != hipSuccess) return fail(blk, LB_ERR_HIP, "copy_stage: %s", hipGetErrorString(err));
    return LB_OK;
}

extern "C" lb_status llama_block_profile(lb_block* blk, uint32_t stage_mask) {
    if (!blk) return LB_ERR_INVALID_ARG;
    profile_release(blk);
    for (double& v : blk->stage_ms) v = 0.0;
    blk->profiled_calls = 0;
    blk->next_slot = 0;
    stage_mask &= LB_PROFILE_ALL;
    blk->profile_mask = stage_mask;
    if (!stage_mask) return LB_OK;
    blk->events.resize((size_t)kProfileSlots * (LB_NUM_STAGES + 1));
    for (size_t i = 0; i < blk->events.size(); ++i) {
        // timing-only events: no system-scope fence (cache writeback and
        // invalidate) when they are recorded, so they barely perturb the
        // kernels between them
        if (hipEventCreateWithFlags(&blk->events[i], hipEventDisableSystemFence) != hipSuccess) {
            blk->events.resize(i);
            profile_release(blk);
            return fail(blk, LB_ERR_HIP, "hipEventCreate failed");
        }
    }
    blk->profiling = true;
    return LB_OK;
}

extern "C" lb_status llama_block_profile_read(lb_block* blk, double* stage_ms, int n, int64_t* calls) {
    if (!blk || !stage_ms || !calls || n < 0 || n > LB_NUM_STAGES) return LB_ERR_INVALID_ARG;
    for (int slot : blk->pending) {
        hipError_t e = profile_collect(blk, slot);
        if (e != hipSuccess) return fail(blk, LB_ERR_HIP, "profiling: %s", hipGetErrorString(e));
    }
    blk->pending.clear();
    for (int i = 0; i < n; ++i) stage_ms[i] = blk->stage_ms[i];
    *calls = blk->profiled_calls;
    return LB_OK;
}
