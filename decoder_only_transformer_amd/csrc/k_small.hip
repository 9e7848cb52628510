// RMSNorm, dtype conversion and weight packing kernels.
#include "launch.h"
#include "lb_device.h"

namespace lb {

// RMSNorm ("The Evolving Transformer 04 LLaMA", 03 RMSNORM; "Full Llama 3
// transformer block", How it works): out = x / sqrt(mean(x^2) + eps) * g.
// One 256-thread block per token row, so even a 32-row decode batch spreads
// over 32 CUs.  Each thread keeps its (up to 8) 8-element chunks in
// registers; the sum of squares is accumulated in fp32 and reduced across
// wavefronts (butterfly) and then across the block in a fixed order, so
// results are deterministic.  d <= 16384 (d % 8 == 0).  out_mt > 0 stores
// the row in the decode (k-step tiled) layout with out_mt row tiles.
template <typename TI, typename TO>
__global__ void __launch_bounds__(256) rmsnorm_kernel(const TI* __restrict__ x,
                                                      const float* __restrict__ g,
                                                      TO* __restrict__ out, int M, int d, float eps,
                                                      int out_mt) {
    __shared__ float part[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = blockIdx.x;
    const TI* xr = x + (size_t)row * d;
    TO* orow = out + (size_t)row * d;
    float v[8][8], gg[8][8];
    float ss = 0.0f;
    // the gains are loaded with the row so that one memory round trip
    // precedes the reduction
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = (threadIdx.x + 256 * i) * 8;
        if (c < d) {
            load8(xr + c, v[i]);
            load8(g + c, gg[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = (threadIdx.x + 256 * i) * 8;
        if (c < d) {
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += v[i][e] * v[i][e];
        }
    }
    ss = wave_sum(ss);
    if (lane == 0) part[wave] = ss;
    __syncthreads();
    ss = (part[0] + part[1]) + (part[2] + part[3]);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = (threadIdx.x + 256 * i) * 8;
        if (c < d) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[i][e] = v[i][e] * r * gg[i][e];
            store8(out_mt > 0 ? out + ktile_act_off(row, c, out_mt) : orow + c, v[i]);
        }
    }
}

// Same RMSNorm for many rows (prefill): one wavefront per row, four rows per
// block, the row in registers (CPL 8-element chunks per lane, d <= 512*CPL),
// the sum of squares reduced by a butterfly inside the wavefront, no LDS and
// no block barrier.  Deterministic (fixed order).
template <typename TI, typename TO, int CPL, bool FULL>
__device__ __forceinline__ void rmsnorm_row(const TI* __restrict__ xr, const float* __restrict__ g,
                                            TO* __restrict__ orow, int d, float eps, int lane) {
    // FULL: the row fills all CPL chunks of every lane, so no load is
    // predicated and all of them go out before the first wait
    auto in_row = [&](int c) { return FULL || c < d; };
    float v[CPL][8];
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = (lane + 64 * i) * 8;
        if (in_row(c)) load8(xr + c, v[i]);
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = (lane + 64 * i) * 8;
        if (in_row(c)) {
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += v[i][e] * v[i][e];
        }
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = (lane + 64 * i) * 8;
        if (in_row(c)) {
            float gg[8];
            load8(g + c, gg);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[i][e] = v[i][e] * r * gg[e];
            store8(orow + c, v[i]);
        }
    }
}

template <typename TI, typename TO, int CPL>
__global__ void __launch_bounds__(256) rmsnorm_rows_kernel(const TI* __restrict__ x,
                                                           const float* __restrict__ g,
                                                           TO* __restrict__ out, int M, int d,
                                                           float eps) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;  // whole wavefronts leave together
    const TI* xr = x + (size_t)row * d;
    TO* orow = out + (size_t)row * d;
    // all loads of a full row at once: measured faster for 16-bit rows
    // (8B width 18.2 -> 15.3 us) and for 16 chunks per lane (70B width:
    // 41.7 -> 30.6 us, fp32 rows 40.9 -> 38.6 us), slower for fp32 rows of
    // 8 chunks (19.6 -> 20.7 us), where more wavefronts per SIMD already
    // overlap the loads
    constexpr bool batch = sizeof(TI) == 2 || CPL >= 16;
    if (batch && d == 512 * CPL) rmsnorm_row<TI, TO, CPL, true>(xr, g, orow, d, eps, lane);
    else rmsnorm_row<TI, TO, CPL, false>(xr, g, orow, d, eps, lane);
}

// One 16-byte chunk per thread: chunk q of the tiled layout comes from row
// 16 * (piece / (K/32)) + q % 16, columns 32 * (piece % (K/32)) + 8 * (q % 64 / 16).
template <typename T>
__global__ void tile_weights_kernel(const T* __restrict__ src, T* __restrict__ dst, int N, int K) {
    const size_t nch = (size_t)N * K / 8;
    const int nks = K / 32;
    for (size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x; q < nch; q += (size_t)gridDim.x * blockDim.x) {
        const int l = (int)(q & 63);
        const size_t piece = q >> 6;
        const size_t n = (piece / nks) * 16 + (l & 15);
        const size_t k = (piece % nks) * 32 + 8 * (l >> 4);
        *reinterpret_cast<u32x4*>(dst + q * 8) = *reinterpret_cast<const u32x4*>(src + n * K + k);
    }
}

template <typename T>
__global__ void untile_kernel(const T* __restrict__ src, T* __restrict__ dst, int M, int K, int mt) {
    const size_t nch = (size_t)M * K / 8;
    for (size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x; q < nch; q += (size_t)gridDim.x * blockDim.x) {
        const int m = (int)(q / (K / 8)), k = (int)(q % (K / 8)) * 8;
        *reinterpret_cast<u32x4*>(dst + (size_t)m * K + k) =
            *reinterpret_cast<const u32x4*>(src + ktile_act_off(m, k, mt));
    }
}

template <typename TI, typename TO>
__global__ void convert_kernel(const TI* __restrict__ src, TO* __restrict__ dst, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        dst[i] = from_f32<TO>(to_f32(src[i]));
}

// One block per destination row r of a [rows][K] weight; with perm_dh > 0,
// inside each block of perm_dh rows, row 2i takes source row i and row 2i+1
// source row i + perm_dh/2.
template <typename TI, typename TO>
__global__ void convert_rows_kernel(const TI* __restrict__ src, TO* __restrict__ dst, int K,
                                    int perm_dh) {
    const int r = blockIdx.x;
    int sr = r;
    if (perm_dh > 0) {
        const int h = r / perm_dh, j = r % perm_dh;
        sr = h * perm_dh + (j & 1 ? j / 2 + perm_dh / 2 : j / 2);
    }
    const TI* in = src + (size_t)sr * K;
    TO* out = dst + (size_t)r * K;
    for (int k = threadIdx.x; k < K; k += blockDim.x) out[k] = from_f32<TO>(to_f32(in[k]));
}

// Packed row p: group c = p / 8; rows 8c..8c+3 = gate rows 4c..4c+3,
// rows 8c+4..8c+7 = up rows 4c..4c+3.
template <typename TI, typename TO>
__global__ void pack_gate_up_kernel(const TI* __restrict__ gate, const TI* __restrict__ up,
                                    TO* __restrict__ dst, int dff, int d) {
    const int p = blockIdx.x;
    const int c = p >> 3, e = p & 7;
    const TI* src = (e < 4) ? gate + (size_t)(4 * c + e) * d : up + (size_t)(4 * c + e - 4) * d;
    TO* out = dst + (size_t)p * d;
    for (int k = threadIdx.x; k < d; k += blockDim.x) out[k] = from_f32<TO>(to_f32(src[k]));
}

template <typename TI, typename TO>
static hipError_t rmsnorm_t(const void* x, const float* g, void* out, int M, int d, float eps,
                            int out_mt, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    if (d > 16384) return hipErrorInvalidValue;
    if (out_mt > 0 && (d % 32 != 0 || M > 16 * out_mt)) return hipErrorInvalidValue;
    if (out_mt == 0 && M >= 256 && d <= 512 * 16) {
        const unsigned blocks = (unsigned)((M + 3) / 4);
        if (d <= 512 * 8)
            rmsnorm_rows_kernel<TI, TO, 8><<<blocks, 256, 0, s>>>((const TI*)x, g, (TO*)out, M, d, eps);
        else
            rmsnorm_rows_kernel<TI, TO, 16><<<blocks, 256, 0, s>>>((const TI*)x, g, (TO*)out, M, d, eps);
        return hipGetLastError();
    }
    rmsnorm_kernel<TI, TO><<<M, 256, 0, s>>>((const TI*)x, g, (TO*)out, M, d, eps, out_mt);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(Elem in_t, Elem out_t, const void* x, const float* g, void* out, int M,
                          int d, float eps, int out_mt, hipStream_t s) {
    if (out_mt > 0 && out_t == Elem::F32) return hipErrorInvalidValue;
#define RN(TI, TO) return rmsnorm_t<TI, TO>(x, g, out, M, d, eps, out_mt, s)
    if (in_t == Elem::F32 && out_t == Elem::F32) RN(float, float);
    if (in_t == Elem::F32 && out_t == Elem::F16) RN(float, f16);
    if (in_t == Elem::F32 && out_t == Elem::BF16) RN(float, bf16);
    if (in_t == Elem::BF16 && out_t == Elem::F16) RN(bf16, f16);
    if (in_t == Elem::BF16 && out_t == Elem::BF16) RN(bf16, bf16);
#undef RN
    return hipErrorInvalidValue;
}

hipError_t launch_tile_weights(Elem t, const void* src, void* dst, int N, int K, hipStream_t s) {
    if (t == Elem::F32 || N % 16 != 0 || K % 32 != 0) return hipErrorInvalidValue;
    if (N <= 0) return hipSuccess;
    size_t blocks = ((size_t)N * K / 8 + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    tile_weights_kernel<f16><<<(unsigned)blocks, 256, 0, s>>>((const f16*)src, (f16*)dst, N, K);
    return hipGetLastError();
}

hipError_t launch_untile(Elem t, const void* src, void* dst, int M, int K, int mt, hipStream_t s) {
    if (t == Elem::F32 || K % 32 != 0 || mt <= 0 || M > 16 * mt) return hipErrorInvalidValue;
    if (M <= 0) return hipSuccess;
    const size_t blocks = ((size_t)M * K / 8 + 255) / 256;
    untile_kernel<f16><<<(unsigned)blocks, 256, 0, s>>>((const f16*)src, (f16*)dst, M, K, mt);
    return hipGetLastError();
}

template <typename TI, typename TO>
static hipError_t convert_t(const void* src, void* dst, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    convert_kernel<TI, TO><<<(unsigned)blocks, 256, 0, s>>>((const TI*)src, (TO*)dst, n);
    return hipGetLastError();
}

hipError_t launch_convert(Elem src_t, Elem dst_t, const void* src, void* dst, size_t n,
                          hipStream_t s) {
#define CV(TI, TO) return convert_t<TI, TO>(src, dst, n, s)
    if (src_t == Elem::F32 && dst_t == Elem::F32) CV(float, float);
    if (src_t == Elem::BF16 && dst_t == Elem::F32) CV(bf16, float);
    if (src_t == Elem::BF16 && dst_t == Elem::F16) CV(bf16, f16);
    if (src_t == Elem::BF16 && dst_t == Elem::BF16) CV(bf16, bf16);
    if (src_t == Elem::F32 && dst_t == Elem::BF16) CV(float, bf16);
    if (src_t == Elem::F32 && dst_t == Elem::F16) CV(float, f16);
#undef CV
    return hipErrorInvalidValue;
}

template <typename TI, typename TO>
static hipError_t convert_rows_t(const void* src, void* dst, int rows, int K, int perm_dh,
                                 hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    convert_rows_kernel<TI, TO><<<rows, 256, 0, s>>>((const TI*)src, (TO*)dst, K, perm_dh);
    return hipGetLastError();
}

hipError_t launch_convert_rows(Elem src_t, Elem dst_t, const void* src, void* dst, int rows, int K,
                               int perm_dh, hipStream_t s) {
    if (perm_dh < 0 || (perm_dh > 0 && (perm_dh % 2 != 0 || rows % perm_dh != 0)))
        return hipErrorInvalidValue;
#define CR(TI, TO) return convert_rows_t<TI, TO>(src, dst, rows, K, perm_dh, s)
    if (src_t == Elem::F32 && dst_t == Elem::F32) CR(float, float);
    if (src_t == Elem::BF16 && dst_t == Elem::F16) CR(bf16, f16);
    if (src_t == Elem::BF16 && dst_t == Elem::BF16) CR(bf16, bf16);
#undef CR
    return hipErrorInvalidValue;
}

template <typename TI, typename TO>
static hipError_t pack_t(const void* gate, const void* up, void* dst, int dff, int d,
                         hipStream_t s) {
    pack_gate_up_kernel<TI, TO><<<2 * dff, 256, 0, s>>>((const TI*)gate, (const TI*)up, (TO*)dst,
                                                        dff, d);
    return hipGetLastError();
}

hipError_t launch_pack_gate_up(Elem src_t, Elem dst_t, const void* gate, const void* up, void* dst,
                               int dff, int d, hipStream_t s) {
#define PK(TI, TO) return pack_t<TI, TO>(gate, up, dst, dff, d, s)
    if (src_t == Elem::F32 && dst_t == Elem::F32) PK(float, float);
    if (src_t == Elem::BF16 && dst_t == Elem::F16) PK(bf16, f16);
    if (src_t == Elem::BF16 && dst_t == Elem::BF16) PK(bf16, bf16);
#undef PK
    return hipErrorInvalidValue;
}

// Per-row statistics of a bf16 weight [rows][K] for the range check of the
// fp16 operand path: out[row] = (sum_k (g_k w_k)^2, sum_k (w_k - fp16(w_k))^2,
// max_k |w_k|, sum_k w_k^2), with g_k = 1 when g is null.  One wavefront per
// row, four rows per block; K % 8 == 0.
__global__ void __launch_bounds__(256) weight_row_stats_kernel(const bf16* __restrict__ w,
                                                               const bf16* __restrict__ g, int rows,
                                                               int K, f32x4* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const bf16* wr = w + (size_t)row * K;
    float sg = 0.0f, se = 0.0f, mx = 0.0f, sw = 0.0f;
    for (int c = lane * 8; c < K; c += 512) {
        float v[8], gg[8];
        load8(wr + c, v);
        if (g) {
            load8(g + c, gg);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) gg[e] = 1.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float gw = gg[e] * v[e];
            const float dv = v[e] - (float)(f16)v[e];
            sg += gw * gw;
            se += dv * dv;
            mx = fmaxf(mx, fabsf(v[e]));
            sw += v[e] * v[e];
        }
    }
    sg = wave_sum(sg);
    se = wave_sum(se);
    sw = wave_sum(sw);
    mx = wave_max(mx);
    if (lane == 0) out[row] = f32x4{sg, se, mx, sw};
}

hipError_t launch_weight_row_stats(const void* w, const void* g, int rows, int K, float* out, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if (K % 8 != 0) return hipErrorInvalidValue;
    weight_row_stats_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, s>>>((const bf16*)w, (const bf16*)g, rows, K,
                                                                      (f32x4*)out);
    return hipGetLastError();
}

// Device-held start positions move on by the tokens of the step that read
// them; queued after that step's last kernel on the same stream.
__global__ void __launch_bounds__(256) advance_positions_kernel(int* __restrict__ pos, int B, int S) {
    const int b = blockIdx.x * 256 + threadIdx.x;
    if (b < B) pos[b] += S;
}

hipError_t launch_advance_positions(int* pos, int B, int S, hipStream_t s) {
    if (B <= 0) return hipSuccess;
    advance_positions_kernel<<<(B + 255) / 256, 256, 0, s>>>(pos, B, S);
    return hipGetLastError();
}

}  // namespace lb
