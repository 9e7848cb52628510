// GEMM kernels: C[M][N] = A[M][K] . W[N][K]^T with fp32 accumulation, results
// handed to an epilogue (epilogues.h) in 8-column chunks.
//
//  gemm_big2_kernel   prefill, large: 256 x 256 (or 256 x 192) tiles,
//                     64-deep k-steps, 16x16x32 MFMA, two LDS stages,
//                     weights in the k-step tiled layout
//  gemm_big_grouped_kernel  grouped expert GEMMs: the same tile body on
//                     row-major expert weights
//  gemm_mfma_kernel   prefill, small: 32x32x16 MFMA tiles, direct-to-LDS
//                     loads, LDS double buffering
//  gemm_skinny_kernel row-major activations of M <= 64 rows (prefill-path
//                     calls with few tokens): 16x16x32 MFMA, split-K over
//                     waves and blocks, weights streamed from HBM straight
//                     into MFMA operands (+ reduce_epilogue_kernel)
//  gemm_decode_kernel decode (one token per sequence, <= 64 sequences):
//                     activations and weights both k-step tiled, every
//                     operand load one contiguous 1 KB piece, K split over
//                     waves and, for long K, two blocks that finish the tile
//                     themselves (or + reduce_epilogue_kernel)
//  gemm_decode_wide_kernel  decode, very wide outputs (gate/up): the 7 or 8
//                     column tiles of a block share the activations through LDS
//  gemm_simple_kernel fp32 blocks: plain LDS-tiled fp32 FMA
//
// The M <= 64 kernels read each weight byte once per call.  With NT their
// weight loads carry the non-temporal hint (streamed reads of hundreds of MB
// measured 7.0 TB/s with it against 6.3 TB/s without); the launchers set it
// for matrices of 40 MB and more, so that the weights of a small model can
// stay in the 256 MB MALL from one call to the next.  Activations, shared by
// every block, are read plainly.
#pragma once

#include <type_traits>

#include "lb_device.h"

namespace lb {

// One epilogue pass of a tiled GEMM: rows [mp, mp + EPR) x columns
// [n0, n0 + BN) of the tile, staged in LDS (row stride CPAD floats), handed
// to the epilogue as 8-column chunks, chunk c = tid + i * NT of the pass to
// thread tid.  When the epilogue reads memory (a non-empty Aux), fetch()
// issues those loads for all of the thread's chunks before the staging, so
// that they overlap one another and it; the loads are not predicated (a
// branch would keep each load's wait beside it): a chunk past the tile's edge
// loads the last chunk inside it, unused.  Epilogues that read nothing run
// the plain strided loop.
template <class Epi, int EPR, int BN, int NT, int CPAD>
struct EpiPass {
    static constexpr int IT = EPR * (BN / 8) / NT;
    static_assert(IT * NT == EPR * (BN / 8), "whole chunks per thread");
    static constexpr bool kReads = !std::is_empty<typename Epi::Aux>::value;
    typename Epi::Aux aux[kReads ? IT : 1];

    __device__ __forceinline__ void fetch(const Epi& epi, int tid, int mp, int n0, int M, int N) {
        if constexpr (kReads) {
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int c = tid + it * NT, row = c / (BN / 8), c8 = c % (BN / 8);
                epi.load(min(mp + row, M - 1), min(n0 + c8 * 8, N - 8), aux[it]);
            }
        }
    }
    __device__ __forceinline__ static void chunk(const Epi& epi, const float* cst, int c, int mp, int n0, int M,
                                                 int N, const typename Epi::Aux& a) {
        const int row = c / (BN / 8), c8 = c % (BN / 8);
        const int m = mp + row, n = n0 + c8 * 8;
        if (m < M && n < N) {
            float v[8];
            const f32x4 lo = *reinterpret_cast<const f32x4*>(cst + row * CPAD + c8 * 8);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(cst + row * CPAD + c8 * 8 + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[e] = lo[e];
                v[4 + e] = hi[e];
            }
            epi.row8(m, n, v, a);
        }
    }
    __device__ __forceinline__ void finish(const Epi& epi, const float* cst, int tid, int mp, int n0, int M,
                                           int N) const {
        if constexpr (kReads) {
#pragma unroll
            for (int it = 0; it < IT; ++it) chunk(epi, cst, tid + it * NT, mp, n0, M, N, aux[it]);
        } else {
            for (int c = tid; c < EPR * (BN / 8); c += NT) chunk(epi, cst, c, mp, n0, M, N, aux[0]);
        }
    }
};

// ------------------------------------------------------------------------------------
// Prefill GEMM.  Block tile BM x BN x 64, NW wavefronts in a (BM/WM) x (BN/WN)
// grid, each computing WM x WN with (WM/32)*(WN/32) accumulator tiles.
// A and W tiles live in LDS as [rows][64] with the 16-byte chunk index XORed
// by (row / 2) & 7: the 16 lanes of one ds_read_b128 phase (64 banks of 4
// bytes) read 16 consecutive rows at one logical chunk and hit 16 different
// 16-byte bank groups.  Tiles are fetched
// straight from global memory into LDS (global_load_lds_dwordx4, no VGPR
// staging): instruction i of wavefront w fills the 64 consecutive 16-byte
// LDS slots starting at (i*NW + w)*64, lane l the slot l, so every lane loads
// the global chunk whose swizzled home is that slot.  An LDS ring of STAGES
// k-steps (two for prefill, where two blocks share a CU; four for the
// weight-streaming expert GEMM): the loads for step k + STAGES - 1 are
// issued before the MFMAs of step k, the kernel waits for its own loads
// (vmcnt) and one barrier closes each step.  Rows of A beyond M and of W
// beyond N are clamped to the last valid
// row (they only feed outputs that the epilogue discards).  K % 64 == 0.
// ------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One BM x BN output tile at (m0, n0); lds holds STAGES * (BM + BN) * 64
// elements.
// NTW: the W loads carry the non-temporal hint (weights read by one row
// tile only).
// WT: W is in the k-step tiled layout (lb_device.h; N % 16 == 0): the W
// stage is BN/16 row tiles x 2 pieces of 1 KB, each one direct-to-LDS load,
// kept in LDS in piece order (piece rt * 2 + h), whose 16-lane groups read 256
// contiguous bytes for the MFMA operand.
template <typename T, int BM, int BN, int WM, int WN, int NW, class Epi, bool NTW = false, int STAGES = 2,
          bool WT = false>
__device__ __forceinline__ void gemm_mfma_tile(const T* __restrict__ A, const T* __restrict__ W, int M,
                                               int N, int K, Epi epi, int m0, int n0, T* lds) {
    typedef typename vec8<T>::type V8;
    constexpr int NT = NW * 64;
    constexpr int BK = 64;
    constexpr int NWN = BN / WN;
    static_assert((BM / WM) * NWN == NW, "wavefront grid covers the tile");
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int ACH = BM * BK / 8 / NT;   // direct-load instructions per thread and stage
    constexpr int BCH = BN * BK / 8 / NT;
    static_assert(ACH * NT * 8 == BM * BK && BCH * NT * 8 == BN * BK, "whole instructions");
    constexpr int EPR = BM < 64 ? BM : 64;  // epilogue rows per pass
    constexpr int CPAD = BN + 8;            // fp32 row pitch of the epilogue stage
    static_assert(EPR * CPAD * 4 <= 2 * (BM + BN) * BK * (int)sizeof(T), "epilogue stage fits");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / NWN, wn = wave % NWN;

    // load i of a stage fills the 64 consecutive 16-byte slots from
    // (i*NW + wave)*64; lane l the slot l.  Addresses are the tile's first A
    // (or W) row, wave-uniform, plus a per-lane byte offset.
    constexpr int ND = ACH + BCH;
    unsigned aoff[ACH], boff[BCH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        const int p = (i * NW + wave) * 64 + lane, row = p >> 3, c = (p & 7) ^ ((row >> 1) & 7);
        aoff[i] = (unsigned)(((size_t)(min(m0 + row, M - 1) - m0) * K + c * 8) * sizeof(T));
    }
    const int nks32 = K / 32;
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
        if constexpr (WT) {
            // piece q = i*NW + wave of the stage: row tile q/2, k half q%2
            const int q = i * NW + wave, rt = min((n0 >> 4) + (q >> 1), (N >> 4) - 1) - (n0 >> 4);
            boff[i] = (unsigned)((((size_t)rt * nks32 + (q & 1)) * 512 + lane * 8) * sizeof(T));
        } else {
            const int p = (i * NW + wave) * 64 + lane, row = p >> 3, c = (p & 7) ^ ((row >> 1) & 7);
            boff[i] = (unsigned)(((size_t)(min(n0 + row, N - 1) - n0) * K + c * 8) * sizeof(T));
        }
    }
    const T* a0 = A + (size_t)m0 * K;
    const T* w0 = WT ? W + (size_t)(n0 >> 4) * nks32 * 512 : W + (size_t)n0 * K;
    constexpr int WSTEP = WT ? 2 * 512 : BK;  // elements from one k-step of W to the next
    const unsigned lds0 = (unsigned)(size_t)(lds_ptr_t)lds;
    const int nk = K / BK;
    // k-steps past the end reload the last one into a stage nobody reads
    auto gload = [&](int kstep) {
        const int ks = kstep < nk ? kstep : nk - 1;
        const unsigned la = lds0 + (unsigned)((kstep % STAGES) * (BM + BN) * BK * (int)sizeof(T));
        const unsigned lb = la + (unsigned)(BM * BK * (int)sizeof(T));
#pragma unroll
        for (int i = 0; i < ACH; ++i)
            lds_dma16_s(a0 + ks * BK, aoff[i], la + (unsigned)((i * NW + wave) * 64 * 8 * (int)sizeof(T)));
#pragma unroll
        for (int i = 0; i < BCH; ++i)
            lds_dma16_s<NTW>(w0 + (size_t)ks * WSTEP, boff[i], lb + (unsigned)((i * NW + wave) * 64 * 8 * (int)sizeof(T)));
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // an LDS ring of STAGES k-steps: the loads of step k + STAGES - 1 go out
    // as step k starts, into the stage of step k - 1, which every wavefront
    // finished reading before the barrier that closed step k - 1
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st) gload(st);
    wait_vm<(STAGES - 2) * ND>();  // step 0 has landed
    lds_barrier();
    for (int kt = 0; kt < nk; ++kt) {
        gload(kt + STAGES - 1);
        const T* la = lds + (kt % STAGES) * (BM + BN) * BK;
        const T* lb = la + BM * BK;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            V8 af[TM], bfr[TN];
            const int kc = ks * 2 + (lane >> 5);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wm * WM + i * 32 + (lane & 31);
                af[i] = *reinterpret_cast<const V8*>(la + row * BK + ((kc ^ ((row >> 1) & 7)) << 3));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = wn * WN + j * 32 + (lane & 31);
                if constexpr (WT)
                    bfr[j] = *reinterpret_cast<const V8*>(lb + ((row >> 4) * 2 + (kc >> 2)) * 512 +
                                                          ((kc & 3) * 16 + (row & 15)) * 8);
                else
                    bfr[j] = *reinterpret_cast<const V8*>(lb + row * BK + ((kc ^ ((row >> 1) & 7)) << 3));
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
        }
        // step k+1 has landed for this wavefront (later steps may fly); the
        // barrier makes it so for all and closes the reads of step k
        wait_vm<(STAGES - 2) * ND>();
        lds_barrier();
    }
    wait_vm<0>();
    __syncthreads();

    // Epilogue: stage EPR rows of the fp32 tile through LDS, then hand
    // contiguous 8-column chunks to the epilogue.
    float* cst = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int p = 0; p < BM / EPR; ++p) {
        EpiPass<Epi, EPR, BN, NT, CPAD> pass;
        pass.fetch(epi, tid, m0 + p * EPR, n0, M, N);
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
        pass.finish(epi, cst, tid, m0 + p * EPR, n0, M, N);
        __syncthreads();
    }
}

template <typename T, int BM, int BN, int WM, int WN, int NW, class Epi, bool WT = false>
__global__ void __launch_bounds__(NW * 64) gemm_mfma_kernel(const T* __restrict__ A,
                                                            const T* __restrict__ W, int M, int N,
                                                            int K, Epi epi) {
    __shared__ __attribute__((aligned(16))) T lds[2 * (BM + BN) * 64];
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
    gemm_mfma_tile<T, BM, BN, WM, WN, NW, Epi, false, 2, WT>(A, W, M, N, K, epi, tm * BM, tn * BN, lds);
}

// Any epilogue applied to rows counted from m_off (the tile sees row m, the
// output row is m + m_off).
template <class Epi>
struct EpiRowOff {
    Epi e;
    int m_off;
    using Aux = typename Epi::Aux;
    __device__ __forceinline__ void load(int m, int n, Aux& a) const { e.load(m + m_off, n, a); }
    __device__ __forceinline__ void row8(int m, int n, float (&v)[8], const Aux& a) const { e.row8(m + m_off, n, v, a); }
    __device__ __forceinline__ void row8(int m, int n, float (&v)[8]) const { e.row8(m + m_off, n, v); }
};

// ------------------------------------------------------------------------------------
// Grouped GEMM over experts: group e multiplies the rows [row_off[e],
// row_off[e+1]) of A by its own W_e = W + e * N * K (N x K, the layout of
// gemm_mfma_kernel).  The groups' BM-row tiles are numbered consecutively
// (group e owns tiles [tile_off[e], tile_off[e+1])); the grid holds
// tiles_m_max x tiles_n blocks, a bound the host knows without reading the
// group sizes, and blocks past the last tile return at once.  Consecutive
// blocks take consecutive row tiles of one column tile, so the tiles of a
// group share its W panel.
// ------------------------------------------------------------------------------------
template <typename T, int BM, int BN, int WM, int WN, int NW, class Epi, bool NTW = false>
__global__ void __launch_bounds__(NW * 64) gemm_grouped_kernel(const T* __restrict__ A,
                                                               const T* __restrict__ W,
                                                               const int* __restrict__ row_off,
                                                               const int* __restrict__ tile_off, int E,
                                                               int N, int K, int tiles_m_max, Epi epi) {
    // decode-sized calls (NTW) stream the expert weights: a four-step LDS
    // ring keeps three steps of loads in flight per block
    constexpr int STAGES = NTW ? 4 : 2;
    __shared__ __attribute__((aligned(16))) T lds[STAGES * (BM + BN) * 64];
    // workgroups are dealt round-robin to the 8 XCDs: renumber so that each
    // XCD runs a contiguous range, whose row tiles of one column tile then
    // share the expert's weight panel in that XCD's L2.  With NTW every panel
    // has one row tile and nothing to share; the plain round-robin order
    // measured faster there (MoE decode 0.76 against 0.79 ms).
    int bid = blockIdx.x;
    const int nb = gridDim.x;
    if (!NTW && (nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
    const int tn = bid / tiles_m_max, tmg = bid - tn * tiles_m_max;
    if (tmg >= tile_off[E]) return;
    // the group of this row tile: the last e with tile_off[e] <= tmg (empty
    // groups own no tile, so that e is the one whose range holds tmg)
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tile_off[mid] <= tmg) lo = mid;
        else hi = mid - 1;
    }
    const int r0 = row_off[lo], rows = row_off[lo + 1] - r0;
    gemm_mfma_tile<T, BM, BN, WM, WN, NW, EpiRowOff<Epi>, NTW, STAGES>(
        A + (size_t)r0 * K, W + (size_t)lo * N * K, rows, N, K, EpiRowOff<Epi>{epi, r0}, (tmg - tile_off[lo]) * BM,
        tn * BN, lds);
}

// ------------------------------------------------------------------------------------
// Large prefill GEMM with 64-deep k-steps: 256 x BN tiles (BN 256 or 192),
// four wavefronts in a 2 x 2 grid (128 x BN/2 each, 16x16x32 MFMAs,
// accumulators in AGPRs), two LDS stages of (256 + BN) x 128 bytes.  A stage
// of A is 256 rows x 128 bytes, loaded by direct-to-LDS loads of whole cache
// lines (eight 128-byte rows per wavefront instruction; chunk index XORed by
// (row / 2) & 7 in LDS, free of bank conflicts for the operand read).  With
// WT, W is in the k-step tiled layout (lb_device.h; N % 16 == 0): a stage is
// BN / 16 row tiles x 2 pieces of 1 KB, one load each, kept in piece order,
// whose operand reads are 1 KB contiguous.  Each k-step is two sub-steps of
// TI x TJ MFMAs, accumulating in place (AGPRs).  Operands are double-buffered
// in registers: during one sub-step the wavefront reads the next sub-step's
// operands into the other buffer, one read after every few products.  One
// barrier per k-step, between its sub-steps: every wavefront's reads of
// stage kt are complete (sub-step 1's operands are in registers) and stage
// kt+1 has landed; sub-step 1 then reads stage kt+1 and issues the loads of
// stage kt+2 into stage kt's buffer, one after every NM / ND products.  Rows beyond
// M / N are clamped to the last valid row.  K % 64 == 0.
// ------------------------------------------------------------------------------------
template <typename T, int BN>
constexpr int big2_tile_lds() { return 2 * (256 + BN) * 64; }

template <typename T, class Epi, bool WT, int BN>
__device__ __forceinline__ void gemm_big2_tile(const T* __restrict__ A, const T* __restrict__ W, int M, int N,
                                               int K, Epi epi, int m0, int n0, T* lds) {
    typedef typename vec8<T>::type V8;
    static_assert(BN == 256 || BN == 192, "tile width");
    constexpr int BM = 256, BK = 64, NW = 4, NT = 256, WM = 128, WN = BN / 2;
    constexpr int TI = WM / 16, TJ = WN / 16, NIT = TI + TJ;
    constexpr int SA = BM * BK, SB = BN * BK, STG = SA + SB;   // elements per stage
    constexpr int NA = SA / 8 / NT, NB = SB / 8 / NT;          // loads per thread per stage (8 + BN / 32)
    constexpr int ND = NA + NB;
    constexpr int EPR = 64, CPAD = BN + 4;
    static_assert(2 * STG == big2_tile_lds<T, BN>(), "LDS size");
    static_assert(EPR * CPAD * 4 <= 2 * STG * (int)sizeof(T), "epilogue stage fits");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int nks32 = K / 32;
    // load d: the wavefront's instruction d of a stage fills 64 consecutive
    // 16-byte slots ((d % NA) * NW + wave) * 64 of its operand, lane l the slot l
    unsigned voff[ND], ldst[ND];
    const unsigned lds0 = (unsigned)(size_t)(lds_ptr_t)lds;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
        const bool isa = d < NA;
        const int slot0 = ((isa ? d : d - NA) * NW + wave) * 64;
        if (isa || !WT) {
            const int p = slot0 + lane, row = p >> 3, c = (p & 7) ^ ((row >> 1) & 7);
            const int r = isa ? min(m0 + row, M - 1) - m0 : min(n0 + row, N - 1) - n0;
            voff[d] = (unsigned)(((size_t)r * K + c * 8) * sizeof(T));
        } else {
            // piece q = slot0 / 64 of the stage: row tile q / 2, k half q % 2
            const int q = slot0 >> 6, rt = min((n0 >> 4) + (q >> 1), (N >> 4) - 1) - (n0 >> 4);
            voff[d] = (unsigned)((((size_t)rt * nks32 + (q & 1)) * 512 + lane * 8) * sizeof(T));
        }
        ldst[d] = lds0 + (unsigned)(((isa ? 0 : SA) + slot0 * 8) * (int)sizeof(T));
    }
    const T* abase = A + (size_t)m0 * K;
    const T* wbase = WT ? W + (size_t)(n0 >> 4) * nks32 * 512 : W + (size_t)n0 * K;
    constexpr int WSTEP = WT ? 2 * 512 : BK;  // elements from one k-step of W to the next
    const int nk = K / BK;
    // k-steps past the end reload the last one into a stage nobody reads
    auto dma = [&](int kstep, int d) {
        const size_t ks = (size_t)(kstep < nk ? kstep : nk - 1);
        lds_dma16_s(d < NA ? abase + ks * BK : wbase + ks * WSTEP, voff[d],
                    ldst[d] + (unsigned)((kstep & 1) * STG * (int)sizeof(T)));
    };
    f32x4 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    V8 af[2][TI], bf[2][TJ];
    // operand item it (0..7: A row tile, 8..15: W column tile) of sub-step s
    // (0/1) of stage kstep, into register buffer fb
    auto rd = [&](int kstep, int s, int fb, int it) {
        const T* st = lds + (kstep & 1) * STG;
        const int f = it < TI ? it : it - TI;
        const int kc = s * 4 + (lane >> 4);
        if (it < TI) {
            const int row = wm * WM + f * 16 + (lane & 15);
            af[fb][f] = *reinterpret_cast<const V8*>(st + row * BK + ((kc ^ ((row >> 1) & 7)) << 3));
        } else if constexpr (WT) {
            bf[fb][f] = *reinterpret_cast<const V8*>(st + SA + ((wn * TJ + f) * 2 + s) * 512 + lane * 8);
        } else {
            const int row = wn * WN + f * 16 + (lane & 15);
            bf[fb][f] = *reinterpret_cast<const V8*>(st + SA + row * BK + ((kc ^ ((row >> 1) & 7)) << 3));
        }
    };
    // prologue: stages 0 and 1 in flight, stage 0 landed
#pragma unroll
    for (int d = 0; d < ND; ++d) dma(0, d);
#pragma unroll
    for (int d = 0; d < ND; ++d) dma(1, d);
    wait_vm<ND>();
    lds_barrier();
#pragma unroll
    for (int it = 0; it < NIT; ++it) rd(0, 0, 0, it);
    // one sub-step: NM = TI * TJ MFMAs on buffer fb, each followed by at
    // most one load and one operand read, spread evenly: with loads, load d
    // of stage kd after MFMA d * NM / ND + 1; the next sub-step's operand
    // item it (stage nstage, sub-step ns, into buffer fb^1) after MFMA
    // it * (NM - 16) / NIT + 2, so the last read lands 14 products before
    // the sub-step ends.  Issuing the loads four at a time after whole rows
    // of products instead left the matrix cores idle while they went out
    // (8B gate/up 778 -> 741 us, down 400 -> 364 us, A/B on one box).
    auto sub = [&](const int fb, const int nstage, const int ns, const bool loads, const int kd) {
        constexpr int NM = TI * TJ, RM = NM - 16;
#pragma unroll
        for (int i = 0; i < TI; ++i) {
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
                const int m = i * TJ + j;
                mfma16_tied(acc[i][j], af[fb][i], bf[fb][j]);
                __builtin_amdgcn_sched_barrier(0);
                if (loads) {
#pragma unroll
                    for (int d = 0; d < ND; ++d)
                        if (m == d * NM / ND + 1) dma(kd, d);
                }
#pragma unroll
                for (int it = 0; it < NIT; ++it)
                    if (m == it * RM / NIT + 2) rd(nstage, ns, fb ^ 1, it);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    for (int kt = 0; kt < nk; ++kt) {
        sub(0, kt, 1, false, 0);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        wait_vm<0>();
        lds_barrier();
        sub(1, kt + 1, 0, true, kt + 2);
    }
    wait_vm<0>();
    mfma_drain();
    __syncthreads();

    // Epilogue: stage EPR rows of the fp32 tile through LDS, then hand
    // contiguous 8-column chunks to the epilogue.
    float* cst = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int p = 0; p < BM / EPR; ++p) {
        EpiPass<Epi, EPR, BN, NT, CPAD> pass;
        pass.fetch(epi, tid, m0 + p * EPR, n0, M, N);
        if (wm == (p * EPR) / WM) {
#pragma unroll
            for (int ii = 0; ii < EPR / 16; ++ii) {
                const int i = ((p * EPR) % WM) / 16 + ii;
#pragma unroll
                for (int j = 0; j < TJ; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        cst[(ii * 16 + 4 * (lane >> 4) + r) * CPAD + wn * WN + j * 16 + (lane & 15)] = acc[i][j][r];
            }
        }
        __syncthreads();
        pass.finish(epi, cst, tid, m0 + p * EPR, n0, M, N);
        __syncthreads();
    }
}

template <typename T, class Epi, bool WT, int BN = 256>
__global__ void __launch_bounds__(256) gemm_big2_kernel(const T* __restrict__ A, const T* __restrict__ W, int M,
                                                       int N, int K, Epi epi) {
    constexpr int BM = 256;
    __shared__ __attribute__((aligned(16))) T lds[big2_tile_lds<T, BN>()];
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    // workgroups are dealt round-robin to the 8 XCDs: renumber so that each
    // XCD runs a contiguous range of tiles, walked in groups of 8 tile-rows
    // (column-major inside a group) so that neighbours share A and W panels
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
    gemm_big2_tile<T, Epi, WT, BN>(A, W, M, N, K, epi, tm * BM, tn * BN, lds);
}

// Grouped GEMM over experts with the 256 x 256 tile body of gemm_big2_tile
// on row-major expert weights: as gemm_grouped_kernel (row tiles of height
// 256 numbered per group by tile_off, a host-side bound tiles_m_max, idle
// blocks return at once).  The 64-deep body measured 2.29 ms per MoE prefill
// step against 2.32 ms with a 32-deep four-stage one (A/B on one box).
template <typename T, class Epi>
__global__ void __launch_bounds__(256) gemm_big_grouped_kernel(const T* __restrict__ A, const T* __restrict__ W,
                                                              const int* __restrict__ row_off,
                                                              const int* __restrict__ tile_off, int E, int N,
                                                              int K, int tiles_m_max, Epi epi) {
    __shared__ __attribute__((aligned(16))) T lds[big2_tile_lds<T, 256>()];
    int bid = blockIdx.x;
    const int nb = gridDim.x;
    if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
    const int tn = bid / tiles_m_max, tmg = bid - tn * tiles_m_max;
    if (tmg >= tile_off[E]) return;
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tile_off[mid] <= tmg) lo = mid;
        else hi = mid - 1;
    }
    const int r0 = row_off[lo], rows = row_off[lo + 1] - r0;
    gemm_big2_tile<T, EpiRowOff<Epi>, false, 256>(A + (size_t)r0 * K, W + (size_t)lo * N * K, rows, N, K,
                                                  EpiRowOff<Epi>{epi, r0}, (tmg - tile_off[lo]) * 256, tn * 256, lds);
}

// ------------------------------------------------------------------------------------
// GEMM for M <= 16*MT rows of row-major activations (calls through the
// prefill path with few tokens): a weight-streaming kernel.  Grid
// (N / (16*CT), KS), KW wavefronts per block.  Every wavefront owns the block's
// 16*CT output columns (CT 16x16x32 MFMA column tiles); the KS blocks of a
// column tile split K into contiguous ranges and a block deals its k-steps of
// 32 round-robin to its wavefronts, U steps per chunk, two chunks in flight
// (register double buffering).  Per k-step a
// lane loads 16 bytes of each of its CT weight rows (MFMA B operands) straight
// from HBM and 16 bytes of each token tile (A, hot in L2); CT column tiles per
// A load keep the activation re-reads at 2*MT/CT of the weight traffic.  The
// block sums its wavefronts in LDS in a fixed order; with KS == 1 it runs the
// epilogue, otherwise it stores an fp32 partial [ks][M][N] and
// reduce_epilogue_kernel adds the KS partials in order (deterministic).
// K % 32 == 0.
// ------------------------------------------------------------------------------------
template <typename T, int MT, int KW, int U, int CT, bool PARTIAL, class Epi, bool NT = false, bool WT = false>
__global__ void __launch_bounds__(KW * 64) gemm_skinny_kernel(const T* __restrict__ A,
                                                              const T* __restrict__ W, int M,
                                                              int N, int K, int KS,
                                                              float* __restrict__ part, Epi epi) {
    typedef typename vec8<T>::type V8;
    constexpr int COLS = 16 * CT;
    __shared__ float red[KW][MT * 16][COLS + 1];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = blockIdx.x * COLS, ks = blockIdx.y;
    const int nks = K / 32;
    // block ks owns the contiguous k-steps [ks*nks/KS, (ks+1)*nks/KS); inside
    // the block they are dealt round-robin to the wavefronts, so at any moment
    // the block sweeps each weight row through one contiguous run
    const int kfirst = (int)((long)ks * nks / KS);
    const int kcount = (int)((long)(ks + 1) * nks / KS) - kfirst;
    const int n_my = wave < kcount ? (kcount - wave + KW - 1) / KW : 0;
    const int nchunk = (n_my + U - 1) / U;
    // WT: W in the k-step tiled layout (N % 16 == 0), lane l's 16 bytes of a
    // k-step are l * 8 elements into the row tile's 1 KB piece
    const T* wp[CT];
    constexpr int WSTEP = WT ? 512 : 32;  // elements from one k-step of a lane's weights to the next
#pragma unroll
    for (int c = 0; c < CT; ++c) {
        if constexpr (WT) wp[c] = W + (size_t)min((n0 >> 4) + c, (N >> 4) - 1) * nks * 512 + lane * 8;
        else wp[c] = W + (size_t)min(n0 + 16 * c + (lane & 15), N - 1) * K + 8 * (lane >> 4);
    }
    const T* ap[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) ap[t] = A + (size_t)min(t * 16 + (lane & 15), M - 1) * K + 8 * (lane >> 4);
    f32x4 acc[MT][CT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    V8 bw[2][U][CT], aa[2][U][MT];
    // steps past this wavefront's share load a clamped (valid) address and
    // contribute nothing: their A operand is zeroed
    auto load = [&](int chunk, int s) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kstep = min(kfirst + wave + (chunk * U + u) * KW, nks - 1);
#pragma unroll
            for (int c = 0; c < CT; ++c) bw[s][u][c] = load_w<NT>(reinterpret_cast<const V8*>(wp[c] + (size_t)kstep * WSTEP));
#pragma unroll
            for (int t = 0; t < MT; ++t) aa[s][u][t] = *reinterpret_cast<const V8*>(ap[t] + kstep * 32);
        }
    };
    auto compute = [&](int chunk, int s) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = chunk * U + u < n_my;
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                V8 a = aa[s][u][t];
                if (!ok) a = V8{};
#pragma unroll
                for (int c = 0; c < CT; ++c) acc[t][c] = mfma16(a, bw[s][u][c], acc[t][c]);
            }
        }
    };
    if (nchunk > 0) load(0, 0);
    int c = 0;
    for (; c + 1 < nchunk; c += 2) {
        load(c + 1, 1);
        compute(c, 0);
        load(c + 2, 0);  // unconditional: a branch here would make every wait a full drain
        compute(c + 1, 1);
    }
    if (c < nchunk) compute(c, 0);
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int cc = 0; cc < CT; ++cc)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                red[wave][t * 16 + 4 * (lane >> 4) + r][cc * 16 + (lane & 15)] = acc[t][cc][r];
    __syncthreads();
    for (int q = threadIdx.x; q < MT * 16 * (COLS / 8); q += KW * 64) {
        const int row = q / (COLS / 8), c8 = q % (COLS / 8);
        const int n = n0 + c8 * 8;
        if (row < M && n < N) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float sacc = 0.0f;
                for (int w = 0; w < KW; ++w) sacc += red[w][row][c8 * 8 + e];
                v[e] = sacc;
            }
            if (PARTIAL) store8(part + ((size_t)ks * M + row) * N + n, v);
            else epi.row8(row, n, v);
        }
    }
}

// ------------------------------------------------------------------------------------
// Decode GEMM over k-step-tiled operands (lb_device.h): A [MT row tiles][K],
// W [N][K], both tiled, so every operand load of a wavefront is one contiguous
// 1 KB piece (8 full cache lines).  Grid (N / (16*CT), KS), NW wavefronts per
// block: the block owns CT 16-column tiles and the KS-th part of K; its
// k-steps are cut into NW contiguous runs, one per wavefront, and every
// wavefront streams its run of each of the CT weight tiles, U k-steps per
// chunk with the next chunk's loads in flight (register double buffering).
// Loads past the end of a run repeat a valid k-step and are discarded.  The
// block sums its wavefronts in LDS in a fixed order; with KS == 1 it runs the
// epilogue on rows < M, otherwise it stores an fp32 partial [ks][M][N] for
// reduce_epilogue_kernel.  With `cnt` (KS == 2, one zeroed word per block
// column) the pair finishes itself instead: both blocks store their partial,
// each then counts itself in cnt[blockIdx.x], and the one that counts second
// adds the other's partial, runs the epilogue and clears the word.  Nobody
// waits; the partials and the count move with agent-coherent accesses
// (sc1), and the sum part0 + part1 has the same bits as the reduction
// kernel's.  N % (16*CT) == 0, K % 32 == 0.
// ------------------------------------------------------------------------------------
template <typename T, int MT, int CT, int U, int NW, bool PARTIAL, class Epi, bool NT = false>
__global__ void __launch_bounds__(NW * 64) gemm_decode_kernel(const T* __restrict__ At,
                                                              const T* __restrict__ Wt, int M,
                                                              int N, int K, int KS,
                                                              float* __restrict__ part, Epi epi,
                                                              unsigned* cnt = nullptr) {
    typedef typename vec8<T>::type V8;
    constexpr int COLS = 16 * CT;
    __shared__ float red[NW][MT * 16][COLS + 1];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nt0 = blockIdx.x * CT, ksp = blockIdx.y;
    const int nks = K / 32;
    const int kb0 = (int)((long)ksp * nks / KS), kb1 = (int)((long)(ksp + 1) * nks / KS);
    const int w0 = kb0 + wave * (kb1 - kb0) / NW, w1 = kb0 + (wave + 1) * (kb1 - kb0) / NW;
    const int n_my = w1 - w0;
    const int nchunk = (n_my + U - 1) / U;
    const T* wp[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) wp[c] = Wt + (size_t)(nt0 + c) * nks * 512 + lane * 8;
    const T* ap = At + lane * 8;
    f32x4 acc[MT][CT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    V8 bw[2][U][CT], aa[2][U][MT];
    auto load = [&](int chunk, int s) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kstep = min(w0 + chunk * U + u, nks - 1);
#pragma unroll
            for (int c = 0; c < CT; ++c) bw[s][u][c] = load_w<NT>(reinterpret_cast<const V8*>(wp[c] + (size_t)kstep * 512));
#pragma unroll
            for (int t = 0; t < MT; ++t)
                aa[s][u][t] = *reinterpret_cast<const V8*>(ap + ((size_t)kstep * MT + t) * 512);
        }
    };
    auto compute = [&](int chunk, int s) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = chunk * U + u < n_my;
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                V8 a = aa[s][u][t];
                if (!ok) a = V8{};
#pragma unroll
                for (int c = 0; c < CT; ++c) acc[t][c] = mfma16(a, bw[s][u][c], acc[t][c]);
            }
        }
    };
    if (nchunk > 0) load(0, 0);
    int c = 0;
    for (; c + 1 < nchunk; c += 2) {
        load(c + 1, 1);
        compute(c, 0);
        load(c + 2, 0);  // unconditional: a branch here would make every wait a full drain
        compute(c + 1, 1);
    }
    if (c < nchunk) compute(c, 0);
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int cc = 0; cc < CT; ++cc)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                red[wave][t * 16 + 4 * (lane >> 4) + r][cc * 16 + (lane & 15)] = acc[t][cc][r];
    __syncthreads();
    const int n0 = nt0 * 16;
    // this block's sum of chunk q (8 columns of one row), waves in order
    auto block_sum = [&](int row, int c8, float (&v)[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float sacc = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) sacc += red[w][row][c8 * 8 + e];
            v[e] = sacc;
        }
    };
    if (PARTIAL && cnt) {
        __shared__ unsigned arrived;
        const __amdgpu_buffer_rsrc_t r = agent_rsrc(part);
        auto off = [&](int ks, int row, int c8) { return (unsigned)((((size_t)ks * M + row) * N + n0 + c8 * 8) * 4); };
        for (int q = threadIdx.x; q < MT * 16 * (COLS / 8); q += NW * 64) {
            const int row = q / (COLS / 8), c8 = q % (COLS / 8);
            if (row < M) {
                float v[8];
                block_sum(row, c8, v);
                store16_agent(r, off(ksp, row, c8), f32x4{v[0], v[1], v[2], v[3]});
                store16_agent(r, off(ksp, row, c8) + 16, f32x4{v[4], v[5], v[6], v[7]});
            }
        }
        wait_vm<0>();  // the partial is stored before the block counts itself
        __syncthreads();
        if (threadIdx.x == 0)
            arrived = __hip_atomic_fetch_add(cnt + blockIdx.x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (arrived == 0) return;  // the other block finishes the tile
        if (threadIdx.x == 0) __hip_atomic_store(cnt + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int q = threadIdx.x; q < MT * 16 * (COLS / 8); q += NW * 64) {
            const int row = q / (COLS / 8), c8 = q % (COLS / 8);
            if (row < M) {
                float v[8];
                block_sum(row, c8, v);
                const f32x4 a = load16_agent(r, off(ksp ^ 1, row, c8)), b = load16_agent(r, off(ksp ^ 1, row, c8) + 16);
                const float o[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = ksp == 0 ? v[e] + o[e] : o[e] + v[e];
                epi.row8(row, n0 + c8 * 8, v);
            }
        }
        return;
    }
    for (int q = threadIdx.x; q < MT * 16 * (COLS / 8); q += NW * 64) {
        const int row = q / (COLS / 8), c8 = q % (COLS / 8);
        if (row < M) {
            float v[8];
            block_sum(row, c8, v);
            if (PARTIAL) store8(part + ((size_t)ksp * M + row) * N + n0 + c8 * 8, v);
            else epi.row8(row, n0 + c8 * 8, v);
        }
    }
}

// ------------------------------------------------------------------------------------
// Decode GEMM for wide outputs: the NW wavefronts of a block own NW different
// 16-column weight tiles and all of K, and share the activations: chunks of AC
// k-steps of the (k-step tiled) activation rows go from global memory into
// LDS once per block (direct-to-LDS loads issued from inline assembly, two
// buffers) and every wavefront reads its MFMA operands from there, so the
// activation traffic per weight byte drops by NW.  Each wavefront streams its
// weight tile with U k-steps in flight in registers.  The output tile of a
// wavefront goes through LDS to form the 8-column chunks of the epilogue.
// Grid N / (16*NW).  N % (16*NW) == 0, K % 32 == 0.
// ------------------------------------------------------------------------------------
template <typename T, int MT, int U, int NW, int AC, class Epi, bool NT = false>
__global__ void __launch_bounds__(NW * 64) gemm_decode_wide_kernel(const T* __restrict__ At,
                                                                   const T* __restrict__ Wt, int M,
                                                                   int N, int K, Epi epi) {
    typedef typename vec8<T>::type V8;
    constexpr int APC = AC * MT;  // 1 KB activation pieces per chunk
    static_assert(APC % NW == 0 && AC % U == 0, "chunk shape");
    __shared__ __attribute__((aligned(16))) T abuf[2 * APC * 512];
    __shared__ float ost[NW][MT * 16][17];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nks = K / 32;
    const int nchunk = (nks + AC - 1) / AC;
    const int nt = blockIdx.x * NW + wave;
    const T* wp = Wt + (size_t)nt * nks * 512 + lane * 8;
    const unsigned lds0 = (unsigned)(size_t)(lds_ptr_t)abuf;
    // pieces past the last k-step reload the last one (never used)
    auto dma_chunk = [&](int chunk) {
#pragma unroll
        for (int i = 0; i < APC / NW; ++i) {
            const int pc = i * NW + wave;
            const int ks = min(chunk * AC + pc / MT, nks - 1);
            lds_dma16(At + ((size_t)ks * MT + pc % MT) * 512 + lane * 8,
                      lds0 + (unsigned)((((chunk & 1) * APC + pc) * 512) * (int)sizeof(T)));
        }
    };
    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    V8 bw[U];
    auto wload = [&](int step, int slot) {
        bw[slot] = load_w<NT>(reinterpret_cast<const V8*>(wp + (size_t)min(step, nks - 1) * 512));
    };
#pragma unroll
    for (int u = 0; u < U; ++u) wload(u, u);
    dma_chunk(0);
    wait_vm<0>();
    __syncthreads();
    for (int ch = 0; ch < nchunk; ++ch) {
        dma_chunk(ch + 1);
        const T* ab = abuf + (ch & 1) * APC * 512;
        for (int s0 = 0; s0 < AC; s0 += U) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int step = ch * AC + s0 + u;
                V8 a[MT];
#pragma unroll
                for (int t = 0; t < MT; ++t) a[t] = *reinterpret_cast<const V8*>(ab + ((s0 + u) * MT + t) * 512 + lane * 8);
                if (step >= nks) {
#pragma unroll
                    for (int t = 0; t < MT; ++t) a[t] = V8{};
                }
#pragma unroll
                for (int t = 0; t < MT; ++t) acc[t] = mfma16(a[t], bw[u], acc[t]);
                wload(step + U, u);
            }
        }
        // chunk ch+1 has landed: only this chunk's AC weight loads may still fly
        wait_vm<AC>();
        __syncthreads();
    }
    wait_vm<0>();
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) ost[wave][t * 16 + 4 * (lane >> 4) + r][lane & 15] = acc[t][r];
    __syncthreads();
    // lane -> (row, 8-column half) of this wavefront's tile
    for (int q = lane; q < MT * 16 * 2; q += 64) {
        const int row = q >> 1, h = q & 1;
        if (row < M) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = ost[wave][row][8 * h + e];
            epi.row8(row, nt * 16 + 8 * h, v);
        }
    }
}

// Sum the KS fp32 partials of a split-K decode GEMM (in split order) and run
// the epilogue: one thread per 8-column chunk.
template <class Epi>
__global__ void __launch_bounds__(256) reduce_epilogue_kernel(const float* __restrict__ part, int M,
                                                              int N, int KS, Epi epi) {
    const int q = blockIdx.x * 256 + threadIdx.x;
    const int n8 = N / 8;
    if (q >= M * n8) return;
    const int row = q / n8, n = (q % n8) * 8;
    float v[8];
    load8(part + (size_t)row * N + n, v);
    for (int k = 1; k < KS; ++k) {
        float w[8];
        load8(part + ((size_t)k * M + row) * N + n, w);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] += w[e];
    }
    epi.row8(row, n, v);
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
