// GEMM kernels: C[M][N] = A[M][K] . W[N][K]^T with fp32 accumulation, results
// handed to an epilogue (epilogues.h) in 8-column chunks.
//
//  gemm_mfma_kernel   prefill: 32x32x16 MFMA tiles, LDS double buffering
//  gemm_skinny_kernel decode (M <= 64): 16x16x32 MFMA, split-K over waves,
//                     weights streamed from HBM straight into MFMA operands
//  gemm_simple_kernel fp32 blocks: plain LDS-tiled fp32 FMA
#pragma once

#include "lb_device.h"

namespace lb {

// ------------------------------------------------------------------------------------
// Prefill GEMM.  Block tile BM x BN x 64, 256 threads = 4 wavefronts in a
// (BM/WM) x (BN/WN) grid, each computing WM x WN with (WM/32)*(WN/32)
// accumulator tiles.  A and W tiles live in LDS as [rows][64] with the 16-byte
// chunk index XORed by (row & 7): the 8 lanes of one ds_read_b128 phase read
// 8 different rows at one logical chunk and hit 8 different bank groups.
// One barrier per K step: global loads for step k+1 are issued before the
// MFMAs of step k and written to the other LDS buffer after them.
// Rows of A beyond M and of W beyond N are clamped to the last valid row (they
// only feed outputs that the epilogue discards).  K % 64 == 0.
// ------------------------------------------------------------------------------------
template <typename T, int BM, int BN, int WM, int WN, class Epi>
__global__ void __launch_bounds__(256) gemm_mfma_kernel(const T* __restrict__ A,
                                                        const T* __restrict__ W, int M, int N,
                                                        int K, Epi epi) {
    typedef typename vec8<T>::type V8;
    constexpr int BK = 64;
    constexpr int NWN = BN / WN;
    static_assert((BM / WM) * NWN == 4, "4 wavefronts per block");
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int ACH = BM * BK / 8 / 256;  // 16-byte chunks per thread and stage
    constexpr int BCH = BN * BK / 8 / 256;
    constexpr int EPR = 64;                 // epilogue rows per pass
    constexpr int CPAD = BN + 8;            // fp32 row pitch of the epilogue stage
    static_assert(EPR * CPAD * 4 <= 2 * (BM + BN) * BK * (int)sizeof(T), "epilogue stage fits");
    __shared__ __attribute__((aligned(16))) T lds[2 * (BM + BN) * BK];

    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    // Workgroups are dealt round-robin to the 8 XCDs: renumber so that each
    // XCD runs a contiguous range of tiles, then walk tiles in groups of 8
    // tile-rows (column-major inside a group) so neighbours share A and W panels.
    int bid = blockIdx.x;
    const int nb = gridDim.x;
    if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
    constexpr int GM = 8;
    const int per_group = GM * tiles_n;
    const int first_m = (bid / per_group) * GM;
    const int gsize = min(tiles_m - first_m, GM);
    const int in_group = bid % per_group;
    const int tm = first_m + in_group % gsize;
    const int tn = in_group / gsize;
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / NWN, wn = wave % NWN;

    u32x4 ra[ACH], rb[BCH];
    const T* abase[ACH];
    const T* bbase[BCH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        const int c = tid + i * 256, row = c >> 3, kc = c & 7;
        abase[i] = A + (size_t)min(m0 + row, M - 1) * K + kc * 8;
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
        const int c = tid + i * 256, row = c >> 3, kc = c & 7;
        bbase[i] = W + (size_t)min(n0 + row, N - 1) * K + kc * 8;
    }
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < ACH; ++i) ra[i] = *reinterpret_cast<const u32x4*>(abase[i] + k0);
#pragma unroll
        for (int i = 0; i < BCH; ++i) rb[i] = *reinterpret_cast<const u32x4*>(bbase[i] + k0);
    };
    auto lstore = [&](int buf) {
        T* la = lds + buf * (BM + BN) * BK;
        T* lb = la + BM * BK;
#pragma unroll
        for (int i = 0; i < ACH; ++i) {
            const int c = tid + i * 256, row = c >> 3, kc = c & 7;
            *reinterpret_cast<u32x4*>(la + row * BK + ((kc ^ (row & 7)) << 3)) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < BCH; ++i) {
            const int c = tid + i * 256, row = c >> 3, kc = c & 7;
            *reinterpret_cast<u32x4*>(lb + row * BK + ((kc ^ (row & 7)) << 3)) = rb[i];
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = K / BK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
        const T* la = lds + buf * (BM + BN) * BK;
        const T* lb = la + BM * BK;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            V8 af[TM], bfr[TN];
            const int kc = ks * 2 + (lane >> 5);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wm * WM + i * 32 + (lane & 31);
                af[i] = *reinterpret_cast<const V8*>(la + row * BK + ((kc ^ (row & 7)) << 3));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = wn * WN + j * 32 + (lane & 31);
                bfr[j] = *reinterpret_cast<const V8*>(lb + row * BK + ((kc ^ (row & 7)) << 3));
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
        }
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: stage EPR rows of the fp32 tile through LDS, then hand
    // contiguous 8-column chunks to the epilogue.
    float* cst = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int p = 0; p < BM / EPR; ++p) {
        if (wm == (p * EPR) / WM) {
            constexpr int IPP = EPR / 32;
#pragma unroll
            for (int ii = 0; ii < IPP; ++ii) {
                const int i = ((p * EPR) % WM) / 32 + ii;
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = ii * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                        const int col = wn * WN + j * 32 + (lane & 31);
                        cst[row * CPAD + col] = acc[i][j][r];
                    }
            }
        }
        __syncthreads();
        for (int c = tid; c < EPR * (BN / 8); c += 256) {
            const int row = c / (BN / 8), c8 = c % (BN / 8);
            const int m = m0 + p * EPR + row, n = n0 + c8 * 8;
            if (m < M && n < N) {
                float v[8];
                const f32x4 a = *reinterpret_cast<const f32x4*>(cst + row * CPAD + c8 * 8);
                const f32x4 b = *reinterpret_cast<const f32x4*>(cst + row * CPAD + c8 * 8 + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
                epi.row8(m, n, v);
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------------------------
// Decode GEMM for M <= 16*MT token rows.  One block owns 16 output columns;
// its KW wavefronts split K (k-steps of 32 dealt round-robin), each keeping
// U k-steps of weight loads in flight.  Per k-step a lane loads 16 bytes of
// one weight row (the MFMA B operand) and 16 bytes of each token tile (A, hot
// in L2).  Partial sums meet in LDS in a fixed order (deterministic).
// K % 32 == 0.
// ------------------------------------------------------------------------------------
template <typename T, int MT, int KW, class Epi>
__global__ void __launch_bounds__(KW * 64) gemm_skinny_kernel(const T* __restrict__ A,
                                                              const T* __restrict__ W, int M,
                                                              int N, int K, Epi epi) {
    typedef typename vec8<T>::type V8;
    constexpr int U = 8;
    __shared__ float red[KW][MT][16][17];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n0 = blockIdx.x * 16;
    const int nks = K / 32;
    const T* wp = W + (size_t)min(n0 + (lane & 15), N - 1) * K + 8 * (lane >> 4);
    const T* ap[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) ap[t] = A + (size_t)min(t * 16 + (lane & 15), M - 1) * K + 8 * (lane >> 4);

    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int ks0 = wave; ks0 < nks; ks0 += KW * U) {
        V8 bw[U], aa[U][MT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int ks = ks0 + u * KW;
            if (ks < nks) {
                bw[u] = *reinterpret_cast<const V8*>(wp + ks * 32);
#pragma unroll
                for (int t = 0; t < MT; ++t) aa[u][t] = *reinterpret_cast<const V8*>(ap[t] + ks * 32);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int ks = ks0 + u * KW;
            if (ks < nks) {
#pragma unroll
                for (int t = 0; t < MT; ++t) acc[t] = mfma16(aa[u][t], bw[u], acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][t][4 * (lane >> 4) + r][lane & 15] = acc[t][r];
    __syncthreads();
    for (int c = threadIdx.x; c < MT * 16 * 2; c += KW * 64) {
        const int row = c >> 1, half = c & 1;
        const int n = n0 + half * 8;
        if (row < M && n < N) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float s = 0.0f;
                for (int w = 0; w < KW; ++w) s += red[w][row >> 4][row & 15][half * 8 + e];
                v[e] = s;
            }
            epi.row8(row, n, v);
        }
    }
}

// ------------------------------------------------------------------------------------
// fp32 GEMM for fp32 blocks: 32 x 64 output tile per block, each thread one
// row and 8 consecutive columns, K in steps of 32 through LDS.  Any M, N
// (N % 8 == 0) and K.
// ------------------------------------------------------------------------------------
template <class Epi>
__global__ void __launch_bounds__(256) gemm_simple_kernel(const float* __restrict__ A,
                                                          const float* __restrict__ W, int M,
                                                          int N, int K, Epi epi) {
    __shared__ float As[32][33];
    __shared__ float Ws[64][33];
    const int tid = threadIdx.x;
    const int row = tid >> 3, c8 = tid & 7;
    const int m0 = blockIdx.y * 32, n0 = blockIdx.x * 64;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    for (int k0 = 0; k0 < K; k0 += 32) {
        for (int i = tid; i < 32 * 32; i += 256) {
            const int r = i >> 5, kk = i & 31;
            As[r][kk] = (m0 + r < M && k0 + kk < K) ? A[(size_t)(m0 + r) * K + k0 + kk] : 0.0f;
        }
        for (int i = tid; i < 64 * 32; i += 256) {
            const int r = i >> 5, kk = i & 31;
            Ws[r][kk] = (n0 + r < N && k0 + kk < K) ? W[(size_t)(n0 + r) * K + k0 + kk] : 0.0f;
        }
        __syncthreads();
        for (int kk = 0; kk < 32; ++kk) {
            const float a = As[row][kk];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = fmaf(a, Ws[c8 * 8 + e][kk], acc[e]);
        }
        __syncthreads();
    }
    const int m = m0 + row, n = n0 + c8 * 8;
    if (m < M && n < N) epi.row8(m, n, acc);
}

}  // namespace lb
