// Causal grouped-query attention ("The Evolving Transformer 04 LLaMA", 05 GQA:
// softmax(Q K^T / sqrt(d_head)) V with a lower-triangular mask; query head h
// reads key/value head floor(h / n_rep); "Full Llama 3 transformer block",
// How it works: queries sit at absolute positions start_pos + s and see every
// cached key at a position <= their own).
//
// All three kernels evaluate the softmax online (running maximum, rescaled
// running sum and output) in base 2: scores are multiplied by
// log2(e)/sqrt(d_head) and exponentiated with exp2.
#include <math.h>

#include <type_traits>

#include "launch.h"
#include "lb_device.h"

namespace lb {

constexpr int kDecodeMaxSplit = 256;  // decode blocks per (sequence, KV group)

template <typename T, typename S> __device__ __forceinline__ u32x4 to_operand(const u32x4& raw);
template <> __device__ __forceinline__ u32x4 to_operand<f16, f16>(const u32x4& raw) { return raw; }
template <> __device__ __forceinline__ u32x4 to_operand<bf16, bf16>(const u32x4& raw) { return raw; }
template <> __device__ __forceinline__ u32x4 to_operand<f16, bf16>(const u32x4& raw) {
    bf16x8 s;
    __builtin_memcpy(&s, &raw, 16);
    f16x8 d;
#pragma unroll
    for (int e = 0; e < 8; ++e) d[e] = (f16)(float)s[e];
    u32x4 r;
    __builtin_memcpy(&r, &d, 16);
    return r;
}

// Row order of the key tile fed to the S^T = K Q^T product: MFMA row i holds
// key pi(i) (bits 2 and 3 of i swapped), so that after the product each lane
// holds 8 consecutive keys per 16-key step -- the order the P V product needs
// for its operand, with V^T read as contiguous 16-byte runs.
__device__ __forceinline__ int key_perm(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }
// LDS chunk swizzle of the key tile, conflict-free for the permuted read.
__device__ __forceinline__ int kswz(int row) { return (row & 3) | ((row >> 1) & 4); }
// LDS chunk swizzle of a value tile ([key][d] rows): the 16 lanes of a
// transpose read cover 4 consecutive keys x 2 chunks, which land on 8
// different bank groups.
__device__ __forceinline__ int vswz(int row) { return (row & 3) << 1; }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;
typedef __attribute__((address_space(3))) void* lds_void_ptr;

// Transpose read (ds_read_b64_tr_b16) of a V^T operand from a [key][DH]
// value tile in LDS.  Within each 16-lane group, lane s reads 4 values of
// key k0 + s/4 at d0 + 4*(s%4); the hardware hands lane j the 4 values of
// column d0 + j at keys k0 .. k0+3.  Two reads (keys k0.. and k0+4..) give the
// 8 k-slots of one MFMA operand: slot e <-> key k0 + e, column d0 + j.
template <typename T, int DH>
__device__ __forceinline__ typename vec8<T>::type vt_fragment(const T* tile, int k0, int d0, int lane) {
    const int s = lane & 15;
    const int d = d0 + 4 * (s & 3);
    const int ka = k0 + (s >> 2), kb = ka + 4;
    const T* pa = tile + ka * DH + ((((d >> 3) ^ vswz(ka)) << 3) | (d & 7));
    const T* pb = tile + kb * DH + ((((d >> 3) ^ vswz(kb)) << 3) | (d & 7));
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)pa);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)pb);
    typename vec8<T>::type r;
    __builtin_memcpy(&r, &lo, 8);
    __builtin_memcpy(reinterpret_cast<char*>(&r) + 8, &hi, 8);
    return r;
}

// ------------------------------------------------------------------------------------
// Prefill.  Grid (B*n_kv*n_hb, ceil(S/32)), NW wavefronts per block: the
// block owns 32 consecutive queries of one sequence and NW query heads of one
// KV group; every wavefront is one head and all of them share each K / V
// tile staged in LDS.  Per 64-key tile a wavefront computes S^T (64 keys x
// 32 queries) with 32x32x16 MFMAs, masks, updates the softmax state of its
// lane's query (lane = query, so rescaling is lane-local) and accumulates
// O^T += V^T P^T, the V^T operands read from the [key][d] tile with transpose
// reads.  Tiles are prefetched into registers during the MFMAs.  Heavier
// (later) query blocks of every head group are launched first.
// ------------------------------------------------------------------------------------
template <typename T, typename KVT, int DH, int NW>
__global__ void __launch_bounds__(NW * 64) attn_prefill_kernel(
    const T* __restrict__ q, const KVT* __restrict__ kbase, const KVT* __restrict__ vbase,
    T* __restrict__ o, long kv_bg, int S, SeqPos sp, int H, int nkv, int n_rep, int n_hb,
    float c) {
    typedef typename vec8<T>::type V8;
    constexpr int KT = 64;
    constexpr int NT = NW * 64;
    constexpr int KCH = DH / 8;
    constexpr int KCHUNKS = KT * KCH;
    constexpr int KPT = (KCHUNKS + NT - 1) / NT;
    __shared__ __attribute__((aligned(16))) T ks[KT * DH];
    __shared__ __attribute__((aligned(16))) T vs[KT * DH];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int qb = gridDim.y - 1 - blockIdx.y;
    const int hb = blockIdx.x % n_hb;
    const int bg = blockIdx.x / n_hb;
    const int g = bg % nkv, b = bg / nkv;
    const int start_pos = LB_SEQ_START(sp, b);
    const int hl = hb * NW + wave;
    const bool head_ok = hl < n_rep;
    const int h = g * n_rep + (head_ok ? hl : n_rep - 1);
    const int q0 = qb * 32;
    const int qi = q0 + (lane & 31);
    const int qrow = min(qi, S - 1);
    const int qpos = start_pos + qrow;
    const int qd = H * DH;

    V8 qf[DH / 16];
    {
        const T* qp = q + (size_t)(b * S + qrow) * qd + h * DH + 8 * (lane >> 5);
#pragma unroll
        for (int kk = 0; kk < DH / 16; ++kk) qf[kk] = *reinterpret_cast<const V8*>(qp + 16 * kk);
    }
    const int kv_len = start_pos + min(q0 + 32, S);
    const int ntiles = (kv_len + KT - 1) / KT;
    const KVT* kp = kbase + (size_t)bg * kv_bg;
    const KVT* vp = vbase + (size_t)bg * kv_bg;

    // rows past kv_len are zero in both tiles (masked keys must not bring
    // non-finite cache contents into the products)
    u32x4 kreg[KPT], vreg[KPT];
    auto gload = [&](int tile) {
        const int t0 = tile * KT;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int cidx = tid + i * NT;
            if (cidx < KCHUNKS) {
                const int row = cidx / KCH, ch = cidx % KCH, key = t0 + row;
                if (key < kv_len) {
                    kreg[i] = *reinterpret_cast<const u32x4*>(kp + (size_t)key * DH + ch * 8);
                    vreg[i] = *reinterpret_cast<const u32x4*>(vp + (size_t)key * DH + ch * 8);
                } else {
                    kreg[i] = u32x4{0u, 0u, 0u, 0u};
                    vreg[i] = u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int cidx = tid + i * NT;
            if (cidx < KCHUNKS) {
                const int row = cidx / KCH, ch = cidx % KCH;
                *reinterpret_cast<u32x4*>(ks + row * DH + ((ch ^ kswz(row)) << 3)) = to_operand<T, KVT>(kreg[i]);
                *reinterpret_cast<u32x4*>(vs + row * DH + ((ch ^ vswz(row)) << 3)) = to_operand<T, KVT>(vreg[i]);
            }
        }
    };

    f32x16 oacc[DH / 32];
#pragma unroll
    for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;
    const int prow = key_perm(lane & 31);

    gload(0);
    for (int tile = 0; tile < ntiles; ++tile) {
        __syncthreads();
        lstore();
        __syncthreads();
        if (tile + 1 < ntiles) gload(tile + 1);

        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
            const int row = kb * 32 + prow;
#pragma unroll
            for (int kk = 0; kk < DH / 16; ++kk) {
                const int ch = 2 * kk + (lane >> 5);
                const V8 kf = *reinterpret_cast<const V8*>(ks + row * DH + ((ch ^ kswz(row)) << 3));
                sacc[kb] = mfma32(kf, qf[kk], sacc[kb]);
            }
        }
        const int t0 = tile * KT;
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = t0 + kb * 32 + 16 * (r >> 3) + 8 * (lane >> 5) + (r & 7);
                float sv = sacc[kb][r] * c;
                if (key > qpos) sv = -INFINITY;
                sacc[kb][r] = sv;
                mx = fmaxf(mx, sv);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2_hw(m_run - m_new);
        float ls = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = exp2_hw(sacc[kb][r] - m_new);
                sacc[kb][r] = p;
                ls += p;
            }
        l_run = l_run * alpha + ls;
        m_run = m_new;
#pragma unroll
        for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
        V8 pf[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                for (int e = 0; e < 8; ++e) pf[kb][cc][e] = from_f32<T>(sacc[kb][8 * cc + e]);
#pragma unroll
        for (int dt = 0; dt < DH / 32; ++dt) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    // slot e <-> key 32kb + 16cc + 8*(lane/32) + e, column 32dt + lane%32
                    const V8 vf = vt_fragment<T, DH>(vs, 32 * kb + 16 * cc + 8 * (lane >> 5),
                                                     32 * dt + 16 * ((lane >> 4) & 1), lane);
                    oacc[dt] = mfma32(vf, pf[kb][cc], oacc[dt]);
                }
        }
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = 1.0f / l_tot;
    if (head_ok && qi < S) {
        T* op = o + (size_t)(b * S + qi) * qd + h * DH;
#pragma unroll
        for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                float vv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) vv[e] = oacc[dt][4 * a + e] * inv;
                store4(op + dt * 32 + 8 * a + 4 * (lane >> 5), vv);
            }
    }
}

// ------------------------------------------------------------------------------------
// Prefill, d_head 128, q and K/V in the same 16-bit type (a prefill from
// position 0 reads the workspace copies of k and v).  Same block shape and
// products as attn_prefill_kernel, reorganised for the chip:
//  * the K and V tiles of 64 keys go from global memory straight into a
//    two-stage LDS ring (direct-to-LDS loads issued from inline assembly,
//    one barrier per tile); the next tile loads under the current one;
//  * LDS swizzles for 64 four-byte banks: key rows XOR their chunk index by
//    row % 16 (16 rows per ds_read_b128 phase), value rows by
//    4*(row % 4) ^ 2*(row / 8 % 2) (the 32 lanes of a transpose read cover
//    4 keys x 4 chunks or 8 keys x 2 chunks);
//  * the mask is applied only on tiles that reach past the block's first
//    query; the softmax scale is folded into exp2(s*c - m);
//  * the running maximum used for the exponentials is raised only when a
//    tile's maximum exceeds it by more than 8 (factor 256), so the output
//    rescale is skipped on most tiles (probabilities stay below 256, far
//    inside fp16 range);
//  * a block is NWH heads of one KV group x QB consecutive query blocks of
//    32 (eight wavefronts in use), all sharing each staged tile; a
//    wavefront whose queries end before the block's last tile skips the
//    products of that tile but keeps loading and syncing.
// Keys past kv_len load the last valid row (finite) and are masked.
// ------------------------------------------------------------------------------------
__device__ __forceinline__ int kswz128(int row) { return row & 15; }
__device__ __forceinline__ int vswz128(int row) { return ((row & 3) << 2) ^ ((row & 8) >> 2); }

template <typename T, int NWH, int QB>
__global__ void __launch_bounds__(NWH * QB * 64, 8 / (NWH * QB)) attn_prefill_fa_kernel(
    const T* __restrict__ q, const T* __restrict__ kbase, const T* __restrict__ vbase,
    T* __restrict__ o, long kv_bg, int S, SeqPos sp, int H, int nkv, int n_rep, int n_hb,
    float c) {
    typedef typename vec8<T>::type V8;
    constexpr int NW = NWH * QB;
    constexpr int DH = 128, KT = 64, NT = NW * 64;
    constexpr int TILE = KT * DH;                 // elements of one K or V tile
    constexpr int ND = 2 * TILE / 8 / NT;          // 16-byte loads per thread per stage
    static_assert(ND * NT * 8 == 2 * TILE, "whole load instructions");
    __shared__ __attribute__((aligned(16))) T lds[2 * 2 * TILE];  // stage s: K at 2sTILE, V after

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hw = wave % NWH, qs = wave / NWH;   // head and query block of this wavefront
    const int qblk = gridDim.y - 1 - blockIdx.y;
    const int hb = blockIdx.x % n_hb;
    const int bg = blockIdx.x / n_hb;
    const int g = bg % nkv, b = bg / nkv;
    const int start_pos = LB_SEQ_START(sp, b);
    const int hl = hb * NWH + hw;
    const bool head_ok = hl < n_rep;
    const int h = g * n_rep + (head_ok ? hl : n_rep - 1);
    const int q0 = (qblk * QB + qs) * 32;
    const int qi = q0 + (lane & 31);
    const int qrow = min(qi, S - 1);
    const int qpos = start_pos + qrow;
    const int qd = H * DH;

    V8 qf[DH / 16];
    {
        const T* qp = q + (size_t)(b * S + qrow) * qd + h * DH + 8 * (lane >> 5);
#pragma unroll
        for (int kk = 0; kk < DH / 16; ++kk) qf[kk] = *reinterpret_cast<const V8*>(qp + 16 * kk);
        // consume q here: the compiler then waits for these loads once, before
        // the tile loop.  Left to itself it waits for them at the first use in
        // every tile, with counters that also cover the next tile's
        // direct-to-LDS loads (invisible to it), so every tile would wait for
        // the next one to land before its fifth product.
#pragma unroll
        for (int kk = 0; kk < DH / 16; ++kk) asm volatile("" ::"v"(qf[kk]));
    }
    // keys the block loads: up to its last query; keys this wavefront uses:
    // up to its own last query (none past S)
    const int kv_len = start_pos + min((qblk + 1) * QB * 32, S);
    const int ntiles = (kv_len + KT - 1) / KT;
    const int my_tiles = q0 < S ? (start_pos + min(q0 + 32, S) + KT - 1) / KT : 0;
    const int first_masked = start_pos + q0;     // keys above this need the mask
    const T* kp = kbase + (size_t)bg * kv_bg;
    const T* vp = vbase + (size_t)bg * kv_bg;

    // load d: 64 consecutive 16-byte slots (d*NW + wave)*64 ..; slots 0..1023
    // are the K tile (row = slot/16), 1024..2047 the V tile
    int src_off[ND];
    unsigned dst_off[ND];
    const unsigned lds0 = (unsigned)(size_t)(lds_void_ptr)lds;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
        const int slot = (d * NW + wave) * 64 + lane;
        const bool isk = slot < TILE / 8;
        const int sl = isk ? slot : slot - TILE / 8;
        const int row = sl >> 4, pc = sl & 15;
        const int ch = pc ^ (isk ? kswz128(row) : vswz128(row));
        src_off[d] = (isk ? 0 : (1 << 30)) | (row * DH + ch * 8);   // bit 30 tags V
        dst_off[d] = lds0 + (unsigned)(((d * NW + wave) * 64 * 8) * (int)sizeof(T));
    }
    auto issue = [&](int tile) {
        const int t0 = tile * KT;
        const unsigned stage = (unsigned)((tile & 1) * 2 * TILE * (int)sizeof(T));
#pragma unroll
        for (int d = 0; d < ND; ++d) {
            const bool isv = src_off[d] >> 30;
            const int off = src_off[d] & ((1 << 30) - 1);
            const int row = off / DH;
            const int key = min(t0 + row, kv_len - 1);
            const T* src = (isv ? vp : kp) + (size_t)key * DH + (off - row * DH);
            lds_dma16(src, dst_off[d] + stage);
        }
    };

    f32x16 oacc[DH / 32];
#pragma unroll
    for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.0f;
    float m_used = -INFINITY, l_run = 0.0f;
    const int prow = key_perm(lane & 31);

    issue(0);
    for (int tile = 0; tile < ntiles; ++tile) {
        wait_vm<0>();
        lds_barrier();  // tile landed everywhere; every wave is done with the other stage
        if (tile + 1 < ntiles) issue(tile + 1);
        if (tile >= my_tiles) continue;  // past this wavefront's queries (it keeps loading and syncing)
        const T* ks = lds + (tile & 1) * 2 * TILE;
        const T* vs = ks + TILE;

        // the matrix-core sections run at raised wavefront priority, so the
        // SIMD prefers the wavefront that feeds the MFMA unit while the other
        // one runs its softmax
        __builtin_amdgcn_s_setprio(1);
        f32x16 sacc[2];
        // K fragments: the first key block's eight go out together, then
        // each product of the first block is followed by the read of the
        // second block's fragment for the same registers
        auto kread = [&](int kb, int kk) -> V8 {
            const int row = kb * 32 + prow;
            const int ch = 2 * kk + (lane >> 5);
            return *reinterpret_cast<const V8*>(ks + row * DH + ((ch ^ kswz128(row)) << 3));
        };
        V8 kf[DH / 16];
#pragma unroll
        for (int kk = 0; kk < DH / 16; ++kk) kf[kk] = kread(0, kk);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < DH / 16; ++kk) {
            sacc[0] = mfma32(kf[kk], qf[kk], sacc[0]);
            kf[kk] = kread(1, kk);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int kk = 0; kk < DH / 16; ++kk) sacc[1] = mfma32(kf[kk], qf[kk], sacc[1]);
        __builtin_amdgcn_s_setprio(0);
        const int t0 = tile * KT;
        float mx = -INFINITY;
        if (t0 + KT - 1 > first_masked) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = t0 + kb * 32 + 16 * (r >> 3) + 8 * (lane >> 5) + (r & 7);
                    if (key > qpos) sacc[kb][r] = -INFINITY;
                    mx = fmaxf(mx, sacc[kb][r]);
                }
        } else {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
        }
        {
            // the other half of the wavefront holds the same queries' other
            // keys: swap halves in registers (no LDS round trip)
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c;
        }
        const bool raise = mx > m_used + 8.0f;
        if (__builtin_amdgcn_ballot_w64(raise)) {
            const float m_new = raise ? mx : m_used;
            const float alpha = exp2_hw(m_used - m_new);
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
            m_used = m_new;
        }
        V8 pf[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float p = exp2_hw(fmaf(sacc[kb][8 * cc + e], c, -m_used));
                    l_run += p;
                    pf[kb][cc][e] = from_f32<T>(p);
                }
        __builtin_amdgcn_s_setprio(1);
        // V^T fragments of column block dt (four, from two transpose reads
        // each), read one column block ahead of its products
        auto vread = [&](int dt, V8 (&vf)[4]) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    // slot e <-> key 32kb + 16cc + 8*(lane/32) + e, column 32dt + lane%32
                    const int k0 = 32 * kb + 16 * cc + 8 * (lane >> 5);
                    const int sg = lane & 15;
                    const int dcol = 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (sg & 3);
                    const int ka = k0 + (sg >> 2), kb2 = ka + 4;
                    const T* pa = vs + ka * DH + ((((dcol >> 3) ^ vswz128(ka)) << 3) | (dcol & 7));
                    const T* pb = vs + kb2 * DH + ((((dcol >> 3) ^ vswz128(kb2)) << 3) | (dcol & 7));
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)pa);
                    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)pb);
                    __builtin_memcpy(&vf[kb * 2 + cc], &lo, 8);
                    __builtin_memcpy(reinterpret_cast<char*>(&vf[kb * 2 + cc]) + 8, &hi, 8);
                }
        };
        V8 vfb[2][4];
        vread(0, vfb[0]);
#pragma unroll
        for (int dt = 0; dt < DH / 32; ++dt) {
            if (dt + 1 < DH / 32) vread(dt + 1, vfb[(dt + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) oacc[dt] = mfma32(vfb[dt & 1][kb * 2 + cc], pf[kb][cc], oacc[dt]);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = 1.0f / l_tot;
    if (head_ok && qi < S) {
        T* op = o + (size_t)(b * S + qi) * qd + h * DH;
#pragma unroll
        for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                float vv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) vv[e] = oacc[dt][4 * a + e] * inv;
                store4(op + dt * 32 + 8 * a + 4 * (lane >> 5), vv);
            }
    }
}

// ------------------------------------------------------------------------------------
// Decode (one new token per sequence).  Grid (nsplit, B*n_kv), 4 wavefronts
// per block; the block owns 4*CH consecutive keys of one (sequence, KV group),
// each wavefront CH of them in steps of 32, and all n_rep query heads of the
// group (heads are the 16 columns of a 16x16x32 MFMA; columns >= n_rep are
// zero).  K rows go straight from HBM into MFMA operand registers with
// 16-byte loads; each step's 32 V rows (one contiguous run) go from HBM into
// the wavefront's own LDS slab (two per wavefront, alternating) with
// direct-to-LDS loads and come back as V^T operands through transpose reads.
// Software pipeline without extra registers: as soon as the QK^T MFMAs of
// step s have consumed the K registers, the K loads and V slab loads of step
// s+1 are issued into them, so HBM stays busy during step s's softmax and PV.
// The cache is bf16; q and the probabilities enter the bf16 MFMAs as a hi +
// lo pair of bf16 values (16 mantissa bits), so only the cache itself is
// bf16.  The block merges its wavefronts in LDS and writes one partial
// (unnormalised output, running max, running sum) per head;
// attn_combine_kernel merges the splits.
// ------------------------------------------------------------------------------------
template <int N> __device__ __forceinline__ void wait_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Cache policy of the K/V streams: every cache byte is read once per step, so
// the loads carry the non-temporal hint (the nt bit, cache-policy value 2 of
// the direct-to-LDS builtin).  Measured on the 8B decode caches (two 537 MB
// tensors): 7.0 TB/s for non-temporal grid-stride reads against 6.3 TB/s
// plain, and 6.5 against 5.7 TB/s in this kernel's own read order.
constexpr int kNonTemporal = 2;

template <typename T, int DH, int NW, bool DIRECT>
__global__ void __launch_bounds__(NW * 64) attn_decode_kernel(
    const T* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc,
    float* __restrict__ part, T* __restrict__ o, int o_mt, long kv_bg, int H, int nkv, int n_rep,
    SeqPos sp, int CH, int nsplit, float c) {
    constexpr int KCH = DH / 8;              // 16-byte chunks per row
    constexpr int VLOADS = 32 * KCH / 64;    // direct-to-LDS instructions per step
    constexpr int KLOADS = 2 * (DH / 32);    // K operand loads per step
    constexpr int SLAB = 32 * DH;            // bf16 elements per slab
    __shared__ float sm[NW][16], sl[NW][16];
    // Two V slabs per wavefront, one in each array, so that every LDS access
    // names its array statically and the compiler's wait for the
    // direct-to-LDS loads of one slab never covers the other.  slab_a is the
    // merge buffer after the loop.
    __shared__ __attribute__((aligned(16))) bf16 slab_a[NW * SLAB];
    __shared__ __attribute__((aligned(16))) bf16 slab_b[NW * SLAB];
    static_assert(NW * 16 * DH * 4 <= NW * SLAB * 2, "merge buffer fits a slab array");
    float (*so)[16][DH] = reinterpret_cast<float (*)[16][DH]>(slab_a);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int split = blockIdx.x, bg = blockIdx.y;
    const int b = bg / nkv, g = bg % nkv;
    const int kv_len = LB_SEQ_START(sp, b) + 1;  // keys of this sequence, its new one included
    const int hl = lane & 15, grp = lane >> 4;
    bf16* my_a = slab_a + wave * SLAB;
    bf16* my_b = slab_b + wave * SLAB;

    const bf16* kp = kc + (size_t)bg * kv_bg;
    const bf16* vp = vc + (size_t)bg * kv_bg;
    const int k_begin = (split * NW + wave) * CH;
    int nsteps = (kv_len - k_begin + 31) / 32;
    nsteps = nsteps < 0 ? 0 : (nsteps > CH / 32 ? CH / 32 : nsteps);
    // Each wavefront walks its steps from its own starting step, wrapping
    // around (the online softmax takes the keys in any order): with every
    // stream at the same offset of its region the reads measured 6.6 TB/s,
    // with the start rotated by block and by wavefront 7.0 TB/s.
    const int rot = nsteps > 0 ? (7 * (int)(blockIdx.y * gridDim.x + blockIdx.x) + 3 * wave) % nsteps : 0;
    auto key0 = [&](int st) { return k_begin + 32 * (st + rot < nsteps ? st + rot : st + rot - nsteps); };
    bf16x8 kf[2][DH / 32];
    // K operands of step st into kf; V rows of step st into slab (rows past
    // kv_len repeat the last valid row: finite values that meet zero
    // probabilities)
    auto issue = [&](int st, bf16* slab) {
        const int kb0 = key0(st);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int key = kb0 + 8 * ((lane & 15) >> 2) + 4 * t + (lane & 3);
            const bf16* p = kp + (size_t)min(key, kv_len - 1) * DH + 8 * grp;
#pragma unroll
            for (int kk = 0; kk < DH / 32; ++kk)
                kf[t][kk] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p + 32 * kk));
        }
#pragma unroll
        for (int i = 0; i < VLOADS; ++i) {
            const int p = i * 64 + lane, row = p / KCH, pc = p % KCH, ch = pc ^ vswz(row);
            const bf16* src = vp + (size_t)min(kb0 + row, kv_len - 1) * DH + ch * 8;
            __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_ptr)(slab + i * 64 * 8), 16, 0, kNonTemporal);
        }
    };
    // the first step's loads go out before q's, which the first step needs
    // only after they have landed anyway
    if (nsteps > 0) issue(0, my_a);

    // q of head hl (heads >= n_rep read head 0 and are zeroed)
    bf16x8 qh[DH / 32], ql[DH / 32];
    {
        const T* qp = q + (size_t)b * H * DH + (size_t)(g * n_rep + (hl < n_rep ? hl : 0)) * DH + 8 * grp;
        float v[DH / 32][8];
#pragma unroll
        for (int kk = 0; kk < DH / 32; ++kk) load8(qp + 32 * kk, v[kk]);
        const float keep = hl < n_rep ? 1.0f : 0.0f;
#pragma unroll
        for (int kk = 0; kk < DH / 32; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = v[kk][e] * keep;
                const bf16 hi = (bf16)x;
                qh[kk][e] = hi;
                ql[kk][e] = (bf16)(x - (float)hi);
            }
    }

    f32x4 oacc[DH / 16];
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    // one 32-key step whose V rows are in cur; the next step goes to nxt
    auto step = [&](int st, const bf16* cur, bf16* nxt) {
        const int kb0 = key0(st);
        f32x4 sc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < DH / 32; ++kk) {
                sc[t] = mfma16(kf[t][kk], qh[kk], sc[t]);
                sc[t] = mfma16(kf[t][kk], ql[kk], sc[t]);
            }
        }
        const bool more = st + 1 < nsteps;
        if (more) issue(st + 1, nxt);
        // lane: head hl, register r of tile t: key kb0 + 8*grp + 4t + r
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = kb0 + 8 * grp + 4 * t + r;
                float sv = sc[t][r] * c;
                if (key >= kv_len) sv = -INFINITY;
                sc[t][r] = sv;
                mx = fmaxf(mx, sv);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2_hw(m_run - m_new);
        float pv[8], ls = 0.0f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = exp2_hw(sc[t][r] - m_new);
                pv[4 * t + r] = p;
                ls += p;
            }
        l_run = l_run * alpha + ls;
        m_run = m_new;
        bf16x8 ph, pl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const bf16 hi = (bf16)pv[e];
            ph[e] = hi;
            pl[e] = (bf16)(pv[e] - (float)hi);
        }
        // cur has landed once at most the next step's loads are pending
        // (loads retire in order)
        if (more) wait_vmcnt<KLOADS + VLOADS>();
        else wait_vmcnt<0>();
#pragma unroll
        for (int dt = 0; dt < DH / 16; ++dt) {
            // slot e <-> key 8*grp + e of the step, column 16dt + lane%16
            const bf16x8 vf = vt_fragment<bf16, DH>(cur, 8 * grp, 16 * dt, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) oacc[dt][r] *= alpha;
            oacc[dt] = mfma16(vf, ph, oacc[dt]);
            oacc[dt] = mfma16(vf, pl, oacc[dt]);
        }
        // cur's transpose reads have returned before the step after next
        // loads into it
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    };
    for (int st = 0; st < nsteps; st += 2) {
        step(st, my_a, my_b);
        if (st + 1 < nsteps) step(st + 1, my_b, my_a);
    }

    float lt = l_run + __shfl_xor(l_run, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    __syncthreads();  // all slabs are done before the merge buffer is written
    if (grp == 0) {
        sm[wave][hl] = m_run;
        sl[wave][hl] = lt;
    }
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) so[wave][hl][16 * dt + 4 * grp + r] = oacc[dt][r];
    __syncthreads();
    for (int idx = tid; idx < n_rep * DH; idx += NW * 64) {
        const int hh = idx / DH, d = idx % DH;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, sm[w][hh]);
        float L = 0.0f, O = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            if (sm[w][hh] != -INFINITY) {
                const float f = exp2_hw(sm[w][hh] - M);
                L += sl[w][hh] * f;
                O += so[w][hh][d] * f;
            }
        }
        if (DIRECT) {
            // one block covers every key of the group: the normalised output
            const int col = (g * n_rep + hh) * DH + d;
            o[o_mt > 0 ? ktile_act_off(b, col, o_mt) : (size_t)b * H * DH + col] = from_f32<T>(O / L);
        } else {
            float* pp = part + (((size_t)b * H + g * n_rep + hh) * nsplit + split) * (DH + 2);
            pp[d] = O;
            if (d == 0) {
                pp[DH] = M;
                pp[DH + 1] = L;
            }
        }
    }
}

// Merge the decode splits of one (sequence, KV group): grid B*n_kv, 256
// threads.  A wavefront per head reduces the running maxima and sums over the
// splits (lanes across splits) and leaves the per-split weights
// exp2(m_s - M) / L in LDS; then every thread accumulates output elements over
// the splits, four independent partial sums in flight.  nsplit <= 256.
template <typename T, int DH>
__global__ void __launch_bounds__(256) attn_combine_kernel(const float* __restrict__ part,
                                                           T* __restrict__ o, int H, int nkv,
                                                           int n_rep, int nsplit, int o_mt) {
    __shared__ float wt[16][kDecodeMaxSplit];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int bg = blockIdx.x, b = bg / nkv, g = bg % nkv;
    const size_t head0 = (size_t)b * H + (size_t)g * n_rep;
    for (int hh = wave; hh < n_rep; hh += 4) {
        const float* pp = part + (head0 + hh) * nsplit * (DH + 2);
        float m = -INFINITY;
        for (int s = lane; s < nsplit; s += 64) m = fmaxf(m, pp[(size_t)s * (DH + 2) + DH]);
        const float M = wave_max(m);
        float l = 0.0f;
        for (int s = lane; s < nsplit; s += 64) {
            const float f = exp2_hw(pp[(size_t)s * (DH + 2) + DH] - M);
            wt[hh][s] = f;
            l += pp[(size_t)s * (DH + 2) + DH + 1] * f;
        }
        const float inv = 1.0f / wave_sum(l);
        for (int s = lane; s < nsplit; s += 64) wt[hh][s] *= inv;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < n_rep * DH; idx += 256) {
        const int hh = idx / DH, d = idx % DH;
        const float* pp = part + (head0 + hh) * nsplit * (DH + 2) + d;
        float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
        int s = 0;
        for (; s + 4 <= nsplit; s += 4) {
            o0 += pp[(size_t)s * (DH + 2)] * wt[hh][s];
            o1 += pp[(size_t)(s + 1) * (DH + 2)] * wt[hh][s + 1];
            o2 += pp[(size_t)(s + 2) * (DH + 2)] * wt[hh][s + 2];
            o3 += pp[(size_t)(s + 3) * (DH + 2)] * wt[hh][s + 3];
        }
        for (; s < nsplit; ++s) o0 += pp[(size_t)s * (DH + 2)] * wt[hh][s];
        const int col = (g * n_rep + hh) * DH + d;
        o[o_mt > 0 ? ktile_act_off(b, col, o_mt) : (size_t)b * H * DH + col] =
            from_f32<T>((o0 + o1) + (o2 + o3));
    }
}

// ------------------------------------------------------------------------------------
// fp32 attention for fp32 blocks.  Grid (S, H, B), one wavefront per query:
// lanes score 64 keys at a time (fp32 dot products), the block of
// probabilities goes through LDS and each lane accumulates up to 4 output
// dimensions.  Any d_head <= 256, any length.
// ------------------------------------------------------------------------------------
__global__ void __launch_bounds__(64) attn_simple_kernel(const float* __restrict__ q,
                                                         const float* __restrict__ kc,
                                                         const float* __restrict__ vc,
                                                         float* __restrict__ o, long kv_bg, int S,
                                                         SeqPos sp, int H, int nkv, int dh,
                                                         float c) {
    __shared__ float qs[256];
    __shared__ float ps[64];
    const int lane = threadIdx.x;
    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int g = h / (H / nkv);
    const int n = LB_SEQ_START(sp, b) + s + 1;
    const size_t bg = (size_t)b * nkv + g;
    const float* qp = q + ((size_t)b * S + s) * H * dh + (size_t)h * dh;
    for (int d = lane; d < dh; d += 64) qs[d] = qp[d];
    __syncthreads();
    float oa[4] = {0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;
    for (int t0 = 0; t0 < n; t0 += 64) {
        const int t = t0 + lane;
        float sv = -INFINITY;
        if (t < n) {
            const float* kr = kc + bg * kv_bg + (size_t)t * dh;
            float acc = 0.0f;
            for (int d = 0; d < dh; ++d) acc = fmaf(qs[d], kr[d], acc);
            sv = acc * c;
        }
        const float m_new = fmaxf(m_run, wave_max(sv));
        const float alpha = exp2f(m_run - m_new);
        const float p = (t < n) ? exp2f(sv - m_new) : 0.0f;
        l_run = l_run * alpha + wave_sum(p);
        m_run = m_new;
        ps[lane] = p;
        __syncthreads();
        const int cnt = min(64, n - t0);
        for (int j = 0; j < 4; ++j) {
            const int d = lane + 64 * j;
            if (d < dh) {
                float a = oa[j] * alpha;
                const float* vr = vc + bg * kv_bg + (size_t)t0 * dh + d;
                for (int u = 0; u < cnt; ++u) a = fmaf(ps[u], vr[(size_t)u * dh], a);
                oa[j] = a;
            }
        }
        __syncthreads();
    }
    float* op = o + ((size_t)b * S + s) * H * dh + (size_t)h * dh;
    for (int j = 0; j < 4; ++j) {
        const int d = lane + 64 * j;
        if (d < dh) op[d] = oa[j] / l_run;
    }
}

// ---- dispatch ---------------------------------------------------------------------------

template <typename T, typename KVT, int DH, int NW>
static hipError_t prefill_t(const AttnArgs& a, hipStream_t s) {
    const int n_rep = a.H / a.nkv;
    const int n_hb = n_rep / NW;
    // blocks are dispatched x-fastest: every (sequence, head group) of the
    // last query block first, so the longest blocks (causal: the most key
    // tiles) start first and the short ones fill the tail
    const dim3 grid(a.B * a.nkv * n_hb, (a.S + 31) / 32);
    const float c = kLog2e / sqrtf((float)DH);
    attn_prefill_kernel<T, KVT, DH, NW><<<grid, NW * 64, 0, s>>>(
        (const T*)a.q, (const KVT*)a.k, (const KVT*)a.v, (T*)a.o, a.kv_bg, a.S, a.sp, a.H,
        a.nkv, n_rep, n_hb, c);
    return hipGetLastError();
}

template <typename T, int NWH, int QB>
static hipError_t prefill_fa_t(const AttnArgs& a, hipStream_t s) {
    const int n_rep = a.H / a.nkv;
    const int n_hb = n_rep / NWH;
    // blocks are dispatched x-fastest: every (sequence, head group) of the
    // last query block first, so the longest blocks (causal: the most key
    // tiles) start first and the short ones fill the tail
    const dim3 grid(a.B * a.nkv * n_hb, (a.S + 32 * QB - 1) / (32 * QB));
    const float c = kLog2e / sqrtf(128.0f);
    attn_prefill_fa_kernel<T, NWH, QB><<<grid, NWH * QB * 64, 0, s>>>(
        (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.o, a.kv_bg, a.S, a.sp, a.H,
        a.nkv, n_rep, n_hb, c);
    return hipGetLastError();
}

template <typename T, typename KVT, int DH>
static hipError_t prefill_nw(const AttnArgs& a, hipStream_t s) {
    const int n_rep = a.H / a.nkv;
    if constexpr (DH == 128 && std::is_same<T, KVT>::value) {
        // eight wavefronts per block, 2 heads of the group x 4 query blocks,
        // share every staged K / V tile: measured 2.5-3 % faster than 4 x 2
        // heads x blocks with 4 heads per group (8B) and 2 % faster than 8 x 1
        // with 8 (70B)
        if (n_rep % 2 == 0) return prefill_fa_t<T, 2, 4>(a, s);
    }
    if (n_rep % 8 == 0) return prefill_t<T, KVT, DH, 8>(a, s);
    if (n_rep % 4 == 0) return prefill_t<T, KVT, DH, 4>(a, s);
    if (n_rep % 3 == 0) return prefill_t<T, KVT, DH, 3>(a, s);
    if (n_rep % 2 == 0) return prefill_t<T, KVT, DH, 2>(a, s);
    return prefill_t<T, KVT, DH, 1>(a, s);
}

template <typename T, typename KVT>
static hipError_t prefill_dh(const AttnArgs& a, hipStream_t s) {
    if (a.dh == 128) return prefill_nw<T, KVT, 128>(a, s);
    if (a.dh == 64) return prefill_nw<T, KVT, 64>(a, s);
    return hipErrorInvalidValue;
}

hipError_t attn_prefill(Elem op, Elem kv_t, const AttnArgs& a, hipStream_t s) {
    if (a.B <= 0 || a.S <= 0) return hipSuccess;
    if (op == Elem::F16 && kv_t == Elem::F16) return prefill_dh<f16, f16>(a, s);
    if (op == Elem::F16 && kv_t == Elem::BF16) return prefill_dh<f16, bf16>(a, s);
    if (op == Elem::BF16 && kv_t == Elem::BF16) return prefill_dh<bf16, bf16>(a, s);
    return hipErrorInvalidValue;
}

// Launch shape of the split-KV decode: 8 wavefronts per block and about one
// block per CU.  With at least 256 (sequence, KV group) pairs every block
// takes all keys of one pair and writes the output itself; otherwise the keys
// of a pair are split so that about 256 blocks run, and a merge kernel
// combines the splits.  Keys per wavefront are a multiple of 32.
constexpr int kDecodeWaves = 8;
struct DecodeShape {
    int nsplit, ch;
};
static DecodeShape decode_shape(int bgs, int kv_len) {
    int nsplit = (256 + bgs - 1) / bgs;
    const int max_split = (kv_len + kDecodeWaves * 32 - 1) / (kDecodeWaves * 32);  // >= 32 keys per wave
    if (nsplit > max_split) nsplit = max_split;
    if (nsplit > kDecodeMaxSplit) nsplit = kDecodeMaxSplit;
    if (nsplit < 1) nsplit = 1;
    int ch = (kv_len + nsplit * kDecodeWaves - 1) / (nsplit * kDecodeWaves);
    ch = (ch + 31) / 32 * 32;
    nsplit = (kv_len + kDecodeWaves * ch - 1) / (kDecodeWaves * ch);
    return {nsplit, ch};
}

// Partials for any batch <= max_batch: B * nsplit <= B + 256 / n_kv blocks'
// worth of (sequence, head) rows.
size_t decode_partials_floats(int max_batch, int H, int dh, int max_kv) {
    (void)max_kv;
    return (size_t)(max_batch + 256) * H * (dh + 2);
}

template <typename T, int DH>
static hipError_t decode_t(const AttnArgs& a, float* part, int o_mt, hipStream_t s) {
    const int n_rep = a.H / a.nkv;
    // shaped for the longest sequence; in a ragged batch the blocks of shorter
    // ones finish early (splitting every group further and combining was
    // measured slower: 140 against 130 us for 32 sequences at 1024..8191)
    const DecodeShape sh = decode_shape(a.B * a.nkv, a.max_start + 1);
    const float c = kLog2e / sqrtf((float)DH);
    const dim3 grid(sh.nsplit, a.B * a.nkv);
    constexpr int NW = kDecodeWaves;
    if (sh.nsplit == 1) {
        attn_decode_kernel<T, DH, NW, true><<<grid, NW * 64, 0, s>>>(
            (const T*)a.q, (const bf16*)a.k, (const bf16*)a.v, part, (T*)a.o, o_mt, a.kv_bg, a.H,
            a.nkv, n_rep, a.sp, sh.ch, 1, c);
        return hipGetLastError();
    }
    attn_decode_kernel<T, DH, NW, false><<<grid, NW * 64, 0, s>>>(
        (const T*)a.q, (const bf16*)a.k, (const bf16*)a.v, part, (T*)a.o, o_mt, a.kv_bg, a.H,
        a.nkv, n_rep, a.sp, sh.ch, sh.nsplit, c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    attn_combine_kernel<T, DH><<<a.B * a.nkv, 256, 0, s>>>(part, (T*)a.o, a.H, a.nkv, n_rep, sh.nsplit, o_mt);
    return hipGetLastError();
}

hipError_t attn_decode(Elem op, Elem kv_t, const AttnArgs& a, float* part, int o_mt, hipStream_t s) {
    if (a.B <= 0) return hipSuccess;
    if (kv_t != Elem::BF16 || a.S != 1 || a.H / a.nkv > 16) return hipErrorInvalidValue;
    if (o_mt > 0 && a.B > 16 * o_mt) return hipErrorInvalidValue;
    if (op == Elem::F16 && a.dh == 128) return decode_t<f16, 128>(a, part, o_mt, s);
    if (op == Elem::F16 && a.dh == 64) return decode_t<f16, 64>(a, part, o_mt, s);
    if (op == Elem::BF16 && a.dh == 128) return decode_t<bf16, 128>(a, part, o_mt, s);
    if (op == Elem::BF16 && a.dh == 64) return decode_t<bf16, 64>(a, part, o_mt, s);
    return hipErrorInvalidValue;
}

hipError_t attn_simple(const AttnArgs& a, hipStream_t s) {
    if (a.B <= 0 || a.S <= 0) return hipSuccess;
    if (a.dh > 256) return hipErrorInvalidValue;
    const float c = kLog2e / sqrtf((float)a.dh);
    attn_simple_kernel<<<dim3(a.S, a.H, a.B), 64, 0, s>>>(
        (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.kv_bg, a.S,
        a.sp, a.H, a.nkv, a.dh, c);
    return hipGetLastError();
}

}  // namespace lb
