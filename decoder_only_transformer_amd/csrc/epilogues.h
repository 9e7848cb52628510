// GEMM epilogues of the block.  Every GEMM kernel hands its fp32 results to
// an epilogue in chunks of 8 consecutive output columns of one token row:
// row8(m, n, v) with n % 8 == 0.  The epilogue owns the fusion that follows
// the product and the stores.
//
// What an epilogue reads from memory besides the product (a residual) it
// can fetch ahead: load(m, n, aux) fills an Aux for the chunk,
// row8(m, n, v, aux) finishes it.  The tiled GEMMs issue the loads of all of
// a thread's chunks of an epilogue pass first and then finish them, so the
// loads overlap one another; the compiler cannot do that reordering itself,
// since the stores of one chunk might alias the loads of the next.
// row8(m, n, v) is load and finish of one chunk.
#pragma once

#include "lb_device.h"

namespace lb {

// q/k/v projection epilogue: RoPE on q and k, KV-cache append, q (and, for a
// prefill from position 0, a k/v copy in the operand type) to the workspace.
//
// RoPE ("The Evolving Transformer 04 LLaMA", 02 RoPE; "Mini Llama 2
// Implementation", Rotary positional embeddings): the pair (2i, 2i+1) of a
// head is turned by the angle pos * theta^(-2i/d_head) with
// pos = start_pos(b) + s ("Full Llama 3 transformer block", How it works).  The
// (cos, sin) table is built in fp64 on the host and stored as fp32 pairs.
//
// Column ranges of the packed projection: [0, qd) q heads, [qd, qd+kvd) k
// heads, [qd+kvd, qd+2kvd) v heads, each head d_head wide.
template <typename TO, typename TC>
struct EpiQKV {
    TO* q;              // [M][qd]
    TO* kws;            // [B][nkv][s_stride][dh] or nullptr
    TO* vws;            // [B][nkv][s_stride][dh] or nullptr
    TC* kc;             // [B][nkv][cap][dh]
    TC* vc;             // [B][nkv][cap][dh]
    const float2* rope; // [max_seq][dh/2] (cos, sin)
    SeqPos sp;
    int S, cap, s_stride, nkv, dh, qd;
    int rope_half;      // columns of a q/k head arrive pair-interleaved (rotate_half weights)

    // 8 rotated values of head columns [j, j+8) to the head that starts at
    // `head`: as they are, or (rotate_half) slot 2i back to dimension i and
    // slot 2i+1 back to dimension i + dh/2
    template <typename T>
    __device__ __forceinline__ void put(T* head, int j, const float (&v)[8]) const {
        if (!rope_half) {
            store8(head + j, v);
            return;
        }
        const float lo[4] = {v[0], v[2], v[4], v[6]}, hi[4] = {v[1], v[3], v[5], v[7]};
        store4(head + j / 2, lo);
        store4(head + j / 2 + dh / 2, hi);
    }

    // RoPE angles are read in the finishing step: fetching them ahead for a
    // whole pass measured slower (the registers outweigh the overlap).
    struct Aux {};
    __device__ __forceinline__ void load(int, int, Aux&) const {}
    __device__ __forceinline__ void row8(int m, int n, float (&v)[8], const Aux&) const { row8(m, n, v); }
    __device__ __forceinline__ void row8(int m, int n, float (&v)[8]) const {
        const int b = m / S, s = m - b * S, pos = LB_SEQ_START(sp, b) + s;
        const int kvd = nkv * dh;
        if (n < qd + kvd) {
            const int j = (n < qd ? n : n - qd) % dh;
            const float2* cs = rope + (size_t)pos * (dh / 2) + (j >> 1);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float2 t = cs[e];
                const float u = v[2 * e], w = v[2 * e + 1];
                v[2 * e] = u * t.x - w * t.y;
                v[2 * e + 1] = u * t.y + w * t.x;
            }
            if (n < qd) {
                put(q + (size_t)m * qd + (n - j), j, v);
            } else {
                const int g = (n - qd) / dh;
                const size_t bg = (size_t)b * nkv + g;
                put(kc + (bg * cap + pos) * dh, j, v);
                if (kws) put(kws + (bg * s_stride + s) * dh, j, v);
            }
        } else {
            const int nn = n - qd - kvd;
            const int g = nn / dh, j = nn % dh;
            const size_t bg = (size_t)b * nkv + g;
            store8(vc + (bg * cap + pos) * dh + j, v);
            if (vws) store8(vws + (bg * s_stride + s) * dh + j, v);
        }
    }
};

// h = x + o Wo^T, kept in fp32 ("Full Llama 3 transformer block", How it works).
template <typename TR>
struct EpiResid {
    const TR* resid;  // [M][N]
    float* out;       // [M][N]
    int N;
    using Aux = Raw8<TR>;
    __device__ __forceinline__ void load(int m, int n, Aux& a) const { fetch8(resid + (size_t)m * N + n, a); }
    __device__ __forceinline__ void row8(int m, int n, float (&v)[8], const Aux& a) const {
        float r[8];
        widen8(a, r);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = r[e] + v[e];
        store8(out + (size_t)m * N + n, v);
    }
    __device__ __forceinline__ void row8(int m, int n, float (&v)[8]) const {
        Aux a;
        load(m, n, a);
        row8(m, n, v, a);
    }
};

// z = SiLU(gate) * up ("The Evolving Transformer 04 LLaMA", 04 SWIGLU), with
// SiLU(a) = a / (1 + e^-a).  The packed weight interleaves groups of four rows:
// packed columns [8c, 8c+4) are gate features [4c, 4c+4), [8c+4, 8c+8) the
// up features of the same four.
template <typename TO>
struct EpiSwiGLU {
    TO* z;    // [M][dff], or k-step tiled with mt row tiles when mt > 0
    int dff;
    int mt;
    struct Aux {};
    __device__ __forceinline__ void load(int, int, Aux&) const {}
    __device__ __forceinline__ void row8(int m, int n, float (&v)[8], const Aux&) const { row8(m, n, v); }
    __device__ __forceinline__ void row8(int m, int n, float (&v)[8]) const {
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = v[e];
            // e^-a as 2^(-a log2 e); 1 / (1 + e^-a) by the hardware reciprocal
            r[e] = a * __builtin_amdgcn_rcpf(1.0f + exp2_hw(-a * 1.4426950408889634f)) * v[4 + e];
        }
        const int j = n >> 1;
        store4(z + (mt > 0 ? ktile_act_off(m, j, mt) : (size_t)m * dff + j), r);
    }
};

// y = h + z W_down^T, stored in the block's dtype.
template <typename TY>
struct EpiOut {
    const float* h;  // [M][N]
    TY* y;           // [M][N]
    int N;
    using Aux = Raw8<float>;
    __device__ __forceinline__ void load(int m, int n, Aux& a) const { fetch8(h + (size_t)m * N + n, a); }
    __device__ __forceinline__ void row8(int m, int n, float (&v)[8], const Aux& a) const {
        float r[8];
        widen8(a, r);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = r[e] + v[e];
        store8(y + (size_t)m * N + n, v);
    }
    __device__ __forceinline__ void row8(int m, int n, float (&v)[8]) const {
        Aux a;
        load(m, n, a);
        row8(m, n, v, a);
    }
};

// Any epilogue applied to a launch that covers the output columns from
// n_off on (the launch sees column n, the output column is n + n_off).
template <class Epi>
struct EpiShift {
    Epi e;
    int n_off;
    using Aux = typename Epi::Aux;
    __device__ __forceinline__ void load(int m, int n, Aux& a) const { e.load(m, n + n_off, a); }
    __device__ __forceinline__ void row8(int m, int n, float (&v)[8], const Aux& a) const { e.row8(m, n + n_off, v, a); }
    __device__ __forceinline__ void row8(int m, int n, float (&v)[8]) const { e.row8(m, n + n_off, v); }
};

}  // namespace lb
