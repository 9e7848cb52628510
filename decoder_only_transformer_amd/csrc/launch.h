// Host-side launch interface between the block executor and the kernel
// translation units.  All pointers are device pointers; every launcher only
// enqueues work on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lb_device.h"

namespace lb {

enum class Elem : int { F32 = 0, BF16 = 1, F16 = 2 };

inline size_t elem_bytes(Elem e) { return e == Elem::F32 ? 4 : 2; }

// ---- small kernels ------------------------------------------------------------
// out[m][:] = x[m][:] / sqrt(mean(x[m]^2) + eps) * g  (fp32 arithmetic, one rounding);
// out_mt > 0 writes out in the decode (k-step tiled) layout with out_mt row tiles.
hipError_t launch_rmsnorm(Elem in_t, Elem out_t, const void* x, const float* g, void* out, int M,
                          int d, float eps, int out_mt, hipStream_t s);
// Weights [N][K] (16-bit) -> the decode (k-step tiled) layout; N % 16 == 0, K % 32 == 0.
hipError_t launch_tile_weights(Elem t, const void* src, void* dst, int N, int K, hipStream_t s);
// Activations in the decode layout (mt row tiles) -> [M][K] row-major.
hipError_t launch_untile(Elem t, const void* src, void* dst, int M, int K, int mt, hipStream_t s);
// dst[i] = src[i] converted (round to nearest even)
hipError_t launch_convert(Elem src_t, Elem dst_t, const void* src, void* dst, size_t n,
                          hipStream_t s);
// Row-wise conversion of a [rows][K] weight; with perm_dh > 0 the rows of each
// block of perm_dh (one head) are reordered: dst row 2i <- src row i,
// dst row 2i+1 <- src row i + perm_dh/2.
hipError_t launch_convert_rows(Elem src_t, Elem dst_t, const void* src, void* dst, int rows, int K,
                               int perm_dh, hipStream_t s);
// Per-row statistics of a bf16 weight w [rows][K] (gain g [K] or null for
// ones), four floats per row into out [rows][4]: sum (g w)^2, sum of the
// squared change of a bf16 -> fp16 conversion, max |w|, sum w^2.  K % 8 == 0.
hipError_t launch_weight_row_stats(const void* w, const void* g, int rows, int K, float* out, hipStream_t s);
// pos[b] += S for b < B (device array)
hipError_t launch_advance_positions(int* pos, int B, int S, hipStream_t s);
// dst [2*dff][d]: row groups of 8 = four gate rows then the same four up rows
hipError_t launch_pack_gate_up(Elem src_t, Elem dst_t, const void* gate, const void* up, void* dst,
                               int dff, int d, hipStream_t s);

// ---- GEMMs: C[M][N] = A[M][K] . W[N][K]^T, fp32 accumulation ---------------------
// For 16-bit operands W is in the k-step tiled layout (lb_device.h) in every
// GEMM below, prefill and decode; for fp32 blocks it is row-major [N][K].
struct QkvEpi {
    void* q;          // [M][qd]           operand type
    void* kws;        // [B][nkv][s_stride][dh] operand type, or nullptr
    void* vws;        // [B][nkv][s_stride][dh] operand type, or nullptr
    void* kc;         // [Bc][nkv][cap][dh] cache type
    void* vc;         // [Bc][nkv][cap][dh] cache type
    const float2* rope;
    SeqPos sp;        // start position of each sequence
    int S, cap, s_stride, nkv, dh, qd;
    int rope_half;    // q/k columns of a head come pair-interleaved; store them in natural order
};
// op: operand type of A and W (F32 selects the plain fp32 kernels); cache: cache type.
// part: fp32 workspace for the split-K decode GEMMs (M <= 64), cap floats;
// skinny_partials_floats(max M, max N) is enough for any split the launcher
// picks, and the launcher lowers the split until [split][M][N] fits cap.
constexpr int kSkinnyMaxSplit = 8;
size_t skinny_partials_floats(int max_m, int max_n);
struct SplitWs {
    float* part;
    size_t cap;                // floats at part
    unsigned* cnt = nullptr;   // zeroed words: a two-way split decode GEMM finishes itself
    int ncnt = 0;
};
// words of SplitWs::cnt a block's workspace holds (one per block column of a
// split decode GEMM)
constexpr int kSplitCounters = 4096;
hipError_t gemm_qkv(Elem op, Elem cache, const void* A, const void* W, int M, int N, int K,
                    const QkvEpi& e, const SplitWs& part, hipStream_t s);
// out(fp32) = resid + A W^T
hipError_t gemm_resid(Elem op, Elem resid_t, const void* A, const void* W, int M, int N, int K,
                      const void* resid, float* out, const SplitWs& part, hipStream_t s);
// z[M][dff] = SiLU(gate) * up from the interleaved gate/up product (N = 2*dff)
hipError_t gemm_swiglu(Elem op, const void* A, const void* W, int M, int N, int K, void* z,
                       const SplitWs& part, hipStream_t s);
// y = h + A W^T, y in out_t
hipError_t gemm_out(Elem op, Elem out_t, const void* A, const void* W, int M, int N, int K,
                    const float* h, void* y, const SplitWs& part, hipStream_t s);

// ---- decode GEMMs: M <= 64 token rows, A and W in the k-step tiled layout ---------
// (lb_device.h).  A has decode_row_tiles(M) row tiles.
int decode_row_tiles(int M);
hipError_t decode_qkv(Elem op, Elem cache, const void* At, const void* Wt, int M, int N, int K,
                      const QkvEpi& e, const SplitWs& part, hipStream_t s);
hipError_t decode_resid(Elem op, Elem resid_t, const void* At, const void* Wt, int M, int N, int K,
                        const void* resid, float* out, const SplitWs& part, hipStream_t s);
// z is written in the tiled layout (decode_row_tiles(M) row tiles, dff = N / 2 columns)
hipError_t decode_swiglu(Elem op, const void* At, const void* Wt, int M, int N, int K, void* zt,
                         const SplitWs& part, hipStream_t s);
hipError_t decode_out(Elem op, Elem out_t, const void* At, const void* Wt, int M, int N, int K,
                      const float* h, void* y, const SplitWs& part, hipStream_t s);

// ---- attention --------------------------------------------------------------------
struct AttnArgs {
    const void* q;   // [B*S][H*dh] operand type (fp32 for fp32 blocks)
    const void* k;   // element (bg, t, d) at k[bg*kv_bg + t*dh + d]
    const void* v;   // element (bg, t, d) at v[bg*kv_bg + t*dh + d]
    void* o;         // [B*S][H*dh] operand type
    long kv_bg;      // elements per (sequence, KV head): positions * dh
    SeqPos sp;       // start position of each sequence
    int B, S, max_start, H, nkv, dh;  // max_start: the largest start position
};
// Causal prefill attention (seq_len > 1).  op: q/o type; kv_t: K/V storage type.
hipError_t attn_prefill(Elem op, Elem kv_t, const AttnArgs& a, hipStream_t s);

// Split-K decode attention (seq_len == 1) over a bf16/fp16 cache, then the
// merge of the splits into o.  part: workspace of decode_partials_floats().
size_t decode_partials_floats(int max_batch, int H, int dh, int max_kv);
// o_mt > 0 writes o in the decode (k-step tiled) layout with o_mt row tiles.
hipError_t attn_decode(Elem op, Elem kv_t, const AttnArgs& a, float* part, int o_mt, hipStream_t s);

// Plain fp32 attention (fp32 blocks, any seq_len).
hipError_t attn_simple(const AttnArgs& a, hipStream_t s);

// ---- mixture-of-experts FFN (k_moe.hip) --------------------------------------------
constexpr int kMoeMaxExperts = 256;
constexpr int kMoeMaxTopK = 8;
constexpr int kMoeMaxWidth = 16384;  // d_model the router stages in LDS
constexpr int kMoeTileM = 128;       // row tile of the grouped expert GEMMs
// logits [M][E] fp32; sel / wts [M][K]: the top K experts, larger logit first
// (lower index among equal logits), and the softmax of their logits
hipError_t launch_moe_router(Elem op, const void* n, const void* wr, int M, int d, int E, int K,
                             float* logits, int* sel, float* wts, hipStream_t s);
// row_off / tile_off [E+1]; src [MK]: pair of each sorted row; slot [MK]:
// sorted row of each pair (pair i = token i / K, choice i % K)
hipError_t launch_moe_route(const int* sel, int MK, int E, int* row_off, int* tile_off, int* src, int* slot,
                            hipStream_t s);
hipError_t launch_moe_gather(Elem op, const void* n, const int* src, int MK, int K, int d, void* a,
                             hipStream_t s);
// expert e: z rows [row_off[e], row_off[e+1]) = SwiGLU(A rows . W_e^T), W_e = W + e*N*K (gate/up packed)
hipError_t launch_moe_grouped_swiglu(Elem op, const void* A, const void* W, const int* row_off, const int* tile_off,
                                     int E, int MK, int N, int K, void* z, hipStream_t s);
// expert e: r rows = A rows . W_e^T in fp32
hipError_t launch_moe_grouped_down(Elem op, const void* A, const void* W, const int* row_off, const int* tile_off,
                                   int E, int MK, int N, int K, float* r, hipStream_t s);
hipError_t launch_moe_combine(Elem out_t, const float* hs, const float* r, const int* slot, const float* wts,
                              int M, int K, int d, void* y, hipStream_t s);

}  // namespace lb
