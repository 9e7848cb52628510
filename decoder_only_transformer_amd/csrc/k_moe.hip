// Mixture-of-experts FFN ("Llama 4 From Scratch", The idea: N expert FFNs, a
// router that sends each token to its top k, one always-on shared expert).
//
//   router      moe_router_kernel: logits = n2 . router^T (fp32 sums of exact
//               fp16 or bf16 products, 16 tokens per block), the top k
//               (larger first, the lower index among equal logits) and the
//               softmax of their logits
//   grouping    moe_route_kernel: a counting sort of the (token, choice)
//               pairs by expert: row_off / tile_off per expert, the sorted
//               row of every pair and the pair of every sorted row
//   gather      moe_gather_kernel: the normalised rows in expert order
//   experts     gemm_grouped_kernel twice: gate/up with the SwiGLU epilogue,
//               then down into fp32 rows
//   combine     moe_combine_kernel: y = (h + shared expert) + sum_j w_j r_j
//
// The shared expert is the block's dense FFN (its down projection adds into
// h).  Values do not depend on where a pair lands inside its expert's rows:
// each output row of a GEMM tile is computed from its own input row alone.
#include "epilogues.h"
#include "gemm_kernels.h"
#include "launch.h"

namespace lb {

// ---- router and top k ------------------------------------------------------------
// One block per 16 tokens: the logits of the 16 tokens and 16*NE16 experts
// come from 16x16x32 MFMAs (tokens x experts tiles; products exact, fp32
// sums), d split over the four wavefronts in contiguous k ranges and their
// partial sums added in LDS in wavefront order, so the result is fixed.  The
// router matrix is read once per 16 tokens (one block per token read it once
// per token: 67 us of an 8B-width MoE prefill step for 16 experts).  Then
// each wavefront picks the top k of four tokens: k rounds of a wavefront
// argmax over the experts not yet taken (lane l holds experts l, l+64,
// l+128, l+192); NaN counts as -inf so that every comparison is a total order
// and every lane agrees; the lower index wins among equal logits.
template <typename T, int NE16>
__global__ void __launch_bounds__(256) moe_router_kernel(const T* __restrict__ n, const T* __restrict__ wr, int M,
                                                         int d, int E, int K, float* __restrict__ logits,
                                                         int* __restrict__ sel, float* __restrict__ wts) {
    typedef typename vec8<T>::type V8;
    __shared__ float part[4][16][NE16 * 16 + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.x * 16;
    // operand fragments: lane -> row lane % 16 (token, or expert), 8
    // consecutive k at 8 * (lane / 16) of each 32-wide k step
    const int nks = (d + 31) / 32;
    const int kb = wave * nks / 4, ke = (wave + 1) * nks / 4;
    const int kl = 8 * (lane >> 4);
    const T* arow = n + (size_t)min(t0 + (lane & 15), M - 1) * d + kl;
    const T* brow[NE16];
#pragma unroll
    for (int c = 0; c < NE16; ++c) brow[c] = wr + (size_t)min(c * 16 + (lane & 15), E - 1) * d + kl;
    f32x4 acc[NE16];
#pragma unroll
    for (int c = 0; c < NE16; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    // U k steps per group, all their loads issued before their products
    // (about 16 loads in flight per lane at any NE16)
    constexpr int U = NE16 >= 8 ? 1 : 8 / NE16;
    for (int k0 = kb; k0 < ke; k0 += U) {
        V8 a[U], b[U][NE16];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = (k0 + u) * 32;
            // d % 8 == 0: a lane's 8 values are all inside or all past d
            const bool in = k0 + u < ke && k + kl < d;
            a[u] = in ? *reinterpret_cast<const V8*>(arow + k) : V8{};
#pragma unroll
            for (int c = 0; c < NE16; ++c) b[u][c] = in ? *reinterpret_cast<const V8*>(brow[c] + k) : V8{};
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int c = 0; c < NE16; ++c) acc[c] = mfma16(a[u], b[u][c], acc[c]);
    }
    // lane holds token 4 * (lane / 16) + r, expert c * 16 + lane % 16
#pragma unroll
    for (int c = 0; c < NE16; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) part[wave][4 * (lane >> 4) + r][c * 16 + (lane & 15)] = acc[c][r];
    __syncthreads();
    for (int q4 = 0; q4 < 4; ++q4) {
        const int tl = wave * 4 + q4, t = t0 + tl;
        if (t >= M) break;  // whole wavefronts leave together
        float lv[kMoeMaxExperts / 64];
#pragma unroll
        for (int q = 0; q < kMoeMaxExperts / 64; ++q) {
            const int e = lane + 64 * q;
            lv[q] = -INFINITY;
            if (e < E) {
                lv[q] = (part[0][tl][e] + part[1][tl][e]) + (part[2][tl][e] + part[3][tl][e]);
                logits[(size_t)t * E + e] = lv[q];
            }
        }
        float top[kMoeMaxTopK];
        int idx[kMoeMaxTopK];
        unsigned taken = 0;
#pragma unroll
        for (int j = 0; j < kMoeMaxTopK; ++j) {
            top[j] = -INFINITY;
            idx[j] = 0;
            if (j < K) {
                float bv = -INFINITY;
                int bi = INT_MAX;
#pragma unroll
                for (int q = 0; q < kMoeMaxExperts / 64; ++q) {
                    const int e = lane + 64 * q;
                    if (e < E && !((taken >> q) & 1u)) {
                        float v = lv[q];
                        v = v != v ? -INFINITY : v;
                        if (bi == INT_MAX || v > bv) {
                            bv = v;
                            bi = e;
                        }
                    }
                }
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) {
                    const float ov = __shfl_xor(bv, o, 64);
                    const int oi = __shfl_xor(bi, o, 64);
                    if (ov > bv || (ov == bv && oi < bi)) {
                        bv = ov;
                        bi = oi;
                    }
                }
                top[j] = bv;
                idx[j] = bi;
                if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
            }
        }
        if (lane == 0) {
            // softmax over the chosen logits; top[0] is the largest
            float p[kMoeMaxTopK], sum = 0.0f;
#pragma unroll
            for (int j = 0; j < kMoeMaxTopK; ++j) {
                p[j] = j < K ? exp2_hw((top[j] - top[0]) * kLog2e) : 0.0f;
                sum += p[j];
            }
            const float inv = 1.0f / sum;
#pragma unroll
            for (int j = 0; j < kMoeMaxTopK; ++j) {
                if (j < K) {
                    sel[(size_t)t * K + j] = idx[j];
                    wts[(size_t)t * K + j] = p[j] * inv;
                }
            }
        }
    }
}

// ---- grouping ------------------------------------------------------------------------
// One block: counts per expert (LDS atomics give each pair its rank inside its
// expert), prefix sums into row_off / tile_off (row tiles of tile_m), then
// every pair's sorted row (slot) and every sorted row's pair (src).  The same
// thread handles pair i in both passes.
__global__ void __launch_bounds__(1024) moe_route_kernel(const int* __restrict__ sel, int MK, int E, int tile_m,
                                                         int* __restrict__ row_off, int* __restrict__ tile_off,
                                                         int* __restrict__ src, int* __restrict__ slot) {
    __shared__ int cnt[kMoeMaxExperts];
    __shared__ int base[kMoeMaxExperts];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += 1024) cnt[e] = 0;
    __syncthreads();
    for (int i = tid; i < MK; i += 1024) {
        const int e = min(max(sel[i], 0), E - 1);
        slot[i] = atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    if (tid == 0) {
        int r = 0, tl = 0;
        for (int e = 0; e < E; ++e) {
            base[e] = r;
            row_off[e] = r;
            tile_off[e] = tl;
            r += cnt[e];
            tl += (cnt[e] + tile_m - 1) / tile_m;
        }
        row_off[E] = r;
        tile_off[E] = tl;
    }
    __syncthreads();
    for (int i = tid; i < MK; i += 1024) {
        const int e = min(max(sel[i], 0), E - 1);
        const int r = base[e] + slot[i];
        slot[i] = r;
        src[r] = i;
    }
}

// Row r of a gets row src[r] / K of n (16-byte copies).
template <typename T>
__global__ void __launch_bounds__(256) moe_gather_kernel(const T* __restrict__ n, const int* __restrict__ src,
                                                         int K, int d, T* __restrict__ a) {
    const int r = blockIdx.x;
    const int tok = src[r] / K;
    const u32x4* s = reinterpret_cast<const u32x4*>(n + (size_t)tok * d);
    u32x4* o = reinterpret_cast<u32x4*>(a + (size_t)r * d);
    for (int i = threadIdx.x; i < d / 8; i += 256) o[i] = s[i];
}

// y[t] = hs[t] + sum_j wts[t][j] * r[slot[t][j]], in the order of the choices;
// hs = h plus the shared expert.
template <typename TO>
__global__ void __launch_bounds__(256) moe_combine_kernel(const float* __restrict__ hs, const float* __restrict__ r,
                                                          const int* __restrict__ slot,
                                                          const float* __restrict__ wts, int K, int d,
                                                          TO* __restrict__ y) {
    const int t = blockIdx.x;
    for (int i = threadIdx.x * 8; i < d; i += 256 * 8) {
        float v[8];
        load8(hs + (size_t)t * d + i, v);
        for (int j = 0; j < K; ++j) {
            const float w = wts[(size_t)t * K + j];
            float u[8];
            load8(r + (size_t)slot[(size_t)t * K + j] * d + i, u);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] += w * u[e];
        }
        store8(y + (size_t)t * d + i, v);
    }
}

// Plain fp32 rows.
struct EpiStoreF32 {
    float* out;
    int N;
    struct Aux {};
    __device__ __forceinline__ void load(int, int, Aux&) const {}
    __device__ __forceinline__ void row8(int m, int n, float (&v)[8], const Aux&) const { row8(m, n, v); }
    __device__ __forceinline__ void row8(int m, int n, float (&v)[8]) const { store8(out + (size_t)m * N + n, v); }
};

// ---- launchers -------------------------------------------------------------------------

// experts in tiles of 16: 1, 2, 4, 8 or 16 of them (E <= 256)
template <typename T>
static hipError_t router_t(const T* n, const T* wr, int M, int d, int E, int K, float* logits, int* sel, float* wts,
                           hipStream_t s) {
    const unsigned grid = (unsigned)((M + 15) / 16);
    const int ne = (E + 15) / 16;
    if (ne <= 1) moe_router_kernel<T, 1><<<grid, 256, 0, s>>>(n, wr, M, d, E, K, logits, sel, wts);
    else if (ne <= 2) moe_router_kernel<T, 2><<<grid, 256, 0, s>>>(n, wr, M, d, E, K, logits, sel, wts);
    else if (ne <= 4) moe_router_kernel<T, 4><<<grid, 256, 0, s>>>(n, wr, M, d, E, K, logits, sel, wts);
    else if (ne <= 8) moe_router_kernel<T, 8><<<grid, 256, 0, s>>>(n, wr, M, d, E, K, logits, sel, wts);
    else moe_router_kernel<T, 16><<<grid, 256, 0, s>>>(n, wr, M, d, E, K, logits, sel, wts);
    return hipGetLastError();
}

hipError_t launch_moe_router(Elem op, const void* n, const void* wr, int M, int d, int E, int K,
                             float* logits, int* sel, float* wts, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    if (d % 8 != 0 || d > kMoeMaxWidth || E < 1 || E > kMoeMaxExperts || K < 1 || K > kMoeMaxTopK || K > E)
        return hipErrorInvalidValue;
    if (op == Elem::F16) return router_t<f16>((const f16*)n, (const f16*)wr, M, d, E, K, logits, sel, wts, s);
    if (op == Elem::BF16) return router_t<bf16>((const bf16*)n, (const bf16*)wr, M, d, E, K, logits, sel, wts, s);
    return hipErrorInvalidValue;
}

// Row-tile height of the grouped GEMMs: 256-row tiles of the large kernel
// when the experts average at least one full such tile; 32-row tiles when
// they average at most 32 rows (decode: the A tile is then mostly real rows
// and the LDS ring small enough for two blocks per CU); else 128-row tiles.
constexpr int kMoeSmallTileM = 32;
int moe_tile_m(int MK, int E) {
    return MK >= 256 * E ? 256 : (MK <= kMoeSmallTileM * E ? kMoeSmallTileM : kMoeTileM);
}

hipError_t launch_moe_route(const int* sel, int MK, int E, int* row_off, int* tile_off, int* src, int* slot,
                            hipStream_t s) {
    if (E < 1 || E > kMoeMaxExperts || MK < 0) return hipErrorInvalidValue;
    moe_route_kernel<<<1, 1024, 0, s>>>(sel, MK, E, moe_tile_m(MK, E), row_off, tile_off, src, slot);
    return hipGetLastError();
}

hipError_t launch_moe_gather(Elem op, const void* n, const int* src, int MK, int K, int d, void* a,
                             hipStream_t s) {
    if (MK <= 0) return hipSuccess;
    if (d % 8 != 0 || op == Elem::F32) return hipErrorInvalidValue;
    moe_gather_kernel<f16><<<MK, 256, 0, s>>>((const f16*)n, src, K, d, (f16*)a);
    return hipGetLastError();
}

// Row-tile bound of the grouped GEMMs over MK sorted rows and E experts: each
// expert's last tile is the only partial one.
static int grouped_tiles_m(int MK, int E, int tile_m) {
    return (MK + tile_m - 1) / tile_m + (E < MK ? E : MK);
}

// At most one row tile per expert on average (decode-sized calls): each
// expert's weights are read by one row tile, so they stream non-temporally.
static bool stream_experts(int MK, int E) { return MK <= E * kMoeTileM; }

template <typename T>
static hipError_t grouped_swiglu_t(const void* A, const void* W, const int* row_off, const int* tile_off, int E,
                                   int MK, int N, int K, void* z, hipStream_t s) {
    const EpiSwiGLU<T> epi{(T*)z, N / 2, 0};
    if (moe_tile_m(MK, E) == 256) {
        const int tm = grouped_tiles_m(MK, E, 256), tn = (N + 255) / 256;
        gemm_big_grouped_kernel<T, EpiSwiGLU<T>><<<(unsigned)tm * tn, 256, 0, s>>>(
            (const T*)A, (const T*)W, row_off, tile_off, E, N, K, tm, epi);
        return hipGetLastError();
    }
    if (moe_tile_m(MK, E) == kMoeSmallTileM) {
        const int tm = grouped_tiles_m(MK, E, kMoeSmallTileM), tn = (N + 127) / 128;
        gemm_grouped_kernel<T, kMoeSmallTileM, 128, 32, 32, 4, EpiSwiGLU<T>, true><<<(unsigned)tm * tn, 256, 0, s>>>(
            (const T*)A, (const T*)W, row_off, tile_off, E, N, K, tm, epi);
        return hipGetLastError();
    }
    const int tm = grouped_tiles_m(MK, E, kMoeTileM), tn = (N + 127) / 128;
    if (stream_experts(MK, E))
        gemm_grouped_kernel<T, kMoeTileM, 128, 64, 64, 4, EpiSwiGLU<T>, true><<<(unsigned)tm * tn, 256, 0, s>>>(
            (const T*)A, (const T*)W, row_off, tile_off, E, N, K, tm, epi);
    else
        gemm_grouped_kernel<T, kMoeTileM, 128, 64, 64, 4, EpiSwiGLU<T>, false><<<(unsigned)tm * tn, 256, 0, s>>>(
            (const T*)A, (const T*)W, row_off, tile_off, E, N, K, tm, epi);
    return hipGetLastError();
}

hipError_t launch_moe_grouped_swiglu(Elem op, const void* A, const void* W, const int* row_off, const int* tile_off,
                                     int E, int MK, int N, int K, void* z, hipStream_t s) {
    if (MK <= 0) return hipSuccess;
    if (K % 64 != 0 || N % 16 != 0) return hipErrorInvalidValue;
    if (op == Elem::F16) return grouped_swiglu_t<f16>(A, W, row_off, tile_off, E, MK, N, K, z, s);
    if (op == Elem::BF16) return grouped_swiglu_t<bf16>(A, W, row_off, tile_off, E, MK, N, K, z, s);
    return hipErrorInvalidValue;
}

template <typename T>
static hipError_t grouped_down_t(const void* A, const void* W, const int* row_off, const int* tile_off, int E,
                                 int MK, int N, int K, float* r, hipStream_t s) {
    if (moe_tile_m(MK, E) == 256) {
        const int tm = grouped_tiles_m(MK, E, 256), tn = (N + 255) / 256;
        gemm_big_grouped_kernel<T, EpiStoreF32><<<(unsigned)tm * tn, 256, 0, s>>>(
            (const T*)A, (const T*)W, row_off, tile_off, E, N, K, tm, EpiStoreF32{r, N});
        return hipGetLastError();
    }
    if (moe_tile_m(MK, E) == kMoeSmallTileM) {
        const int tm = grouped_tiles_m(MK, E, kMoeSmallTileM), tn = (N + 127) / 128;
        gemm_grouped_kernel<T, kMoeSmallTileM, 128, 32, 32, 4, EpiStoreF32, true><<<(unsigned)tm * tn, 256, 0, s>>>(
            (const T*)A, (const T*)W, row_off, tile_off, E, N, K, tm, EpiStoreF32{r, N});
        return hipGetLastError();
    }
    const int tm = grouped_tiles_m(MK, E, kMoeTileM), tn = (N + 127) / 128;
    if (stream_experts(MK, E))
        gemm_grouped_kernel<T, kMoeTileM, 128, 64, 64, 4, EpiStoreF32, true><<<(unsigned)tm * tn, 256, 0, s>>>(
            (const T*)A, (const T*)W, row_off, tile_off, E, N, K, tm, EpiStoreF32{r, N});
    else
        gemm_grouped_kernel<T, kMoeTileM, 128, 64, 64, 4, EpiStoreF32, false><<<(unsigned)tm * tn, 256, 0, s>>>(
            (const T*)A, (const T*)W, row_off, tile_off, E, N, K, tm, EpiStoreF32{r, N});
    return hipGetLastError();
}

hipError_t launch_moe_grouped_down(Elem op, const void* A, const void* W, const int* row_off, const int* tile_off,
                                   int E, int MK, int N, int K, float* r, hipStream_t s) {
    if (MK <= 0) return hipSuccess;
    if (K % 64 != 0 || N % 8 != 0) return hipErrorInvalidValue;
    if (op == Elem::F16) return grouped_down_t<f16>(A, W, row_off, tile_off, E, MK, N, K, r, s);
    if (op == Elem::BF16) return grouped_down_t<bf16>(A, W, row_off, tile_off, E, MK, N, K, r, s);
    return hipErrorInvalidValue;
}

hipError_t launch_moe_combine(Elem out_t, const float* hs, const float* r, const int* slot, const float* wts,
                              int M, int K, int d, void* y, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    if (d % 8 != 0) return hipErrorInvalidValue;
    if (out_t == Elem::BF16)
        moe_combine_kernel<bf16><<<M, 256, 0, s>>>(hs, r, slot, wts, K, d, (bf16*)y);
    else if (out_t == Elem::F32)
        moe_combine_kernel<float><<<M, 256, 0, s>>>(hs, r, slot, wts, K, d, (float*)y);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace lb
