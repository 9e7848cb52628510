// GEMM dispatch for the four projections of the block.
#include <atomic>

#include "epilogues.h"
#include "gemm_kernels.h"
#include "launch.h"

namespace lb {

size_t skinny_partials_floats(int max_m, int max_n) { return (size_t)kSkinnyMaxSplit * max_m * max_n; }

// Decode GEMM launch: CT column tiles per wavefront, split-K over KS blocks
// so that a launch has >= ~256 blocks even for narrow outputs.
// Weight matrices from this size up are streamed with the non-temporal hint;
// smaller ones are read plainly.  Measured at 32 tokens with every call on
// fresh weights: the hint wins from the 50 MB q/k/v matrix up (13.4 against
// 13.7 us; down 24.4 against 25.3; gate/up 40 against 45) and loses on the
// 34 MB o matrix (11.1 against 10.0 us); a small model's whole weight set
// fits in the 256 MB MALL, where plain loads let it stay between calls.
constexpr size_t kStreamMinBytes = size_t(40) << 20;

// W is in the k-step tiled layout (N % 16 == 0, K % 32 == 0).
template <typename T, int MT, bool NT, class Epi>
static hipError_t run_skinny(const T* A, const T* W, int M, int N, int K, const Epi& epi,
                             float* part, size_t part_cap, hipStream_t s) {
    if constexpr (MT <= 2) {
        if (N >= 128 * 192) {  // wide outputs: 128 columns per wavefront, no split
            const dim3 grid((N + 127) / 128, 1);
            gemm_skinny_kernel<T, MT, 8, 1, 8, false, Epi, NT, true><<<grid, 512, 0, s>>>(A, W, M, N, K, 1, part, epi);
            return hipGetLastError();
        }
    }
    const int tiles = (N + 63) / 64;
    int ks = (256 + tiles / 2) / tiles;
    ks = ks < 1 ? 1 : (ks > kSkinnyMaxSplit ? kSkinnyMaxSplit : ks);
    if (ks > K / 32) ks = K / 32;
    // the partials [ks][M][N] must fit the workspace
    while (ks > 1 && (size_t)ks * M * N > part_cap) --ks;
    const dim3 grid(tiles, ks);
    if (ks == 1) {
        gemm_skinny_kernel<T, MT, 4, 2, 4, false, Epi, NT, true><<<grid, 256, 0, s>>>(A, W, M, N, K, 1, part, epi);
        return hipGetLastError();
    }
    gemm_skinny_kernel<T, MT, 4, 2, 4, true, Epi, NT, true><<<grid, 256, 0, s>>>(A, W, M, N, K, ks, part, epi);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    reduce_epilogue_kernel<Epi><<<(M * (N / 8) + 255) / 256, 256, 0, s>>>(part, M, N, ks, epi);
    return hipGetLastError();
}

// Decode GEMM over k-step-tiled operands.  Very wide outputs (>= 1536
// 16-column tiles) share the activations of a block through LDS; wide ones
// (>= 384 tiles) take two column tiles per wavefront, so a wavefront's activation
// loads feed twice the weight bytes; narrower ones take one and split K
// across blocks when there are fewer than 192 column tiles.
int decode_row_tiles(int M) { return M <= 16 ? 1 : (M <= 32 ? 2 : 4); }

constexpr size_t kSplitMinBytes = size_t(4) << 20;

template <typename T, int MT, bool NT, class Epi>
static hipError_t run_decode_mt(const T* At, const T* Wt, int M, int N, int K, const Epi& epi,
                                const SplitWs& ws, hipStream_t s) {
    const int tiles = N / 16, nks = K / 32;
    // very wide outputs (gate/up): blocks of 7 or 8 column tiles sharing the
    // activations through LDS.  Seven when they divide the tiles: the Llama
    // gate/up widths (2 d_ff / 16 = 1792 tiles at d_ff 14336, 3584 at 28672)
    // are multiples of 7 * 256, so every CU gets the same number of blocks,
    // where blocks of 8 leave 32 of the 256 CUs idle.  Measured at the
    // 8B width: one token 46.0 -> 40.6 us, 32 tokens 41.5 us either way
    // (28 activation k-steps per LDS refill, 7 k-steps in flight).
    if (tiles >= 8 * 192 && tiles % 7 == 0) {
        constexpr int AC = MT == 4 ? 14 : 28, U = 7;
        gemm_decode_wide_kernel<T, MT, U, 7, AC, Epi, NT><<<tiles / 7, 448, 0, s>>>(At, Wt, M, N, K, epi);
        return hipGetLastError();
    }
    if (tiles >= 8 * 192 && tiles % 8 == 0) {
        // k-steps in flight per wavefront and activation k-steps per LDS
        // refill (measured at 32 tokens: U 4 with AC 16, 39.4 us, against
        // 40.2 with U 8)
        constexpr int AC = MT == 4 ? 8 : 16, U = MT == 4 ? 8 : 4;
        gemm_decode_wide_kernel<T, MT, U, 8, AC, Epi, NT><<<tiles / 8, 512, 0, s>>>(At, Wt, M, N, K, epi);
        return hipGetLastError();
    }
    if (tiles >= 384 && tiles % 2 == 0) {
        gemm_decode_kernel<T, MT, 2, 2, 4, false, Epi, NT><<<dim3(tiles / 2, 1), 256, 0, s>>>(At, Wt, M, N, K, 1, ws.part, epi);
        return hipGetLastError();
    }
    // long K at mid widths (the down projection): two column tiles per
    // wavefront halve the activation loads per weight byte; a two-way K
    // split keeps one block per CU (measured faster than one split, despite
    // the extra reduction launch, from K = 8192 up)
    if (tiles >= 192 && tiles % 2 == 0 && nks >= 256 && (size_t)2 * M * N <= ws.cap) {
        if (ws.cnt && ws.ncnt >= tiles / 2) {
            // the pair of blocks of a column tile adds its halves itself
            gemm_decode_kernel<T, MT, 2, 2, 4, true, Epi, NT><<<dim3(tiles / 2, 2), 256, 0, s>>>(
                At, Wt, M, N, K, 2, ws.part, epi, ws.cnt);
            return hipGetLastError();
        }
        gemm_decode_kernel<T, MT, 2, 2, 4, true, Epi, NT><<<dim3(tiles / 2, 2), 256, 0, s>>>(At, Wt, M, N, K, 2, ws.part, epi);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        reduce_epilogue_kernel<Epi><<<(M * (N / 8) + 255) / 256, 256, 0, s>>>(ws.part, M, N, 2, epi);
        return hipGetLastError();
    }
    int ks = 1;
    // narrow outputs: split K so that about 256 blocks stream the weights,
    // unless the whole matrix is small enough (a few MB, the small-model
    // widths) that the reduction's extra launch costs more than the split saves
    if (tiles < 192 && (size_t)N * K * sizeof(T) >= kSplitMinBytes) {
        ks = (256 + tiles - 1) / tiles;
        if (ks > kSkinnyMaxSplit) ks = kSkinnyMaxSplit;
        if (ks > nks / 4) ks = nks / 4;  // at least one k-step per wavefront
        while (ks > 1 && (size_t)ks * M * N > ws.cap) --ks;
        if (ks < 1) ks = 1;
    }
    if (ks == 1) {
        gemm_decode_kernel<T, MT, 1, 4, 4, false, Epi, NT><<<dim3(tiles, 1), 256, 0, s>>>(At, Wt, M, N, K, 1, ws.part, epi);
        return hipGetLastError();
    }
    gemm_decode_kernel<T, MT, 1, 4, 4, true, Epi, NT><<<dim3(tiles, ks), 256, 0, s>>>(At, Wt, M, N, K, ks, ws.part, epi);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    reduce_epilogue_kernel<Epi><<<(M * (N / 8) + 255) / 256, 256, 0, s>>>(ws.part, M, N, ks, epi);
    return hipGetLastError();
}

template <typename T, class Epi>
static hipError_t run_decode(const T* At, const T* Wt, int M, int N, int K, const Epi& epi,
                             const SplitWs& ws, hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if (M > 64 || N % 16 != 0 || K % 32 != 0) return hipErrorInvalidValue;
    const bool nt = (size_t)N * K * sizeof(T) >= kStreamMinBytes;
    switch (decode_row_tiles(M)) {
        case 1: return nt ? run_decode_mt<T, 1, true>(At, Wt, M, N, K, epi, ws, s)
                          : run_decode_mt<T, 1, false>(At, Wt, M, N, K, epi, ws, s);
        case 2: return nt ? run_decode_mt<T, 2, true>(At, Wt, M, N, K, epi, ws, s)
                          : run_decode_mt<T, 2, false>(At, Wt, M, N, K, epi, ws, s);
        default: return nt ? run_decode_mt<T, 4, true>(At, Wt, M, N, K, epi, ws, s)
                           : run_decode_mt<T, 4, false>(At, Wt, M, N, K, epi, ws, s);
    }
}

// compute units of the current device, cached per device (threads that race
// to fill an entry store the same value)
static int device_cus() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Prefill GEMM: A [M][K] row-major, W in the k-step tiled layout.
template <typename T, class Epi>
static hipError_t run_gemm(const T* A, const T* W, int M, int N, int K, const Epi& epi,
                           const SplitWs& ws, hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if (N % 16 != 0 || K % 64 != 0) return hipErrorInvalidValue;
    if (M <= 64) {
        const bool nt = (size_t)N * K * sizeof(T) >= kStreamMinBytes;
        if (M <= 16) return nt ? run_skinny<T, 1, true>(A, W, M, N, K, epi, ws.part, ws.cap, s)
                               : run_skinny<T, 1, false>(A, W, M, N, K, epi, ws.part, ws.cap, s);
        if (M <= 32) return nt ? run_skinny<T, 2, true>(A, W, M, N, K, epi, ws.part, ws.cap, s)
                               : run_skinny<T, 2, false>(A, W, M, N, K, epi, ws.part, ws.cap, s);
        return nt ? run_skinny<T, 4, true>(A, W, M, N, K, epi, ws.part, ws.cap, s)
                  : run_skinny<T, 4, false>(A, W, M, N, K, epi, ws.part, ws.cap, s);
    }
    const long tm = (M + 255) / 256, tn = (N + 255) / 256, t256 = tm * tn;
    if (t256 >= 192 && N % 192 == 0) {
        // A CU runs one tile at a time, so a launch takes ceil(tiles / CUs)
        // rounds of tile time ~ BN.  256 x 192 tiles when their rounds cost
        // less (the 8B q/k/v product: 512 tiles in 2 rounds of 192 columns
        // against 384 in 2 of 256), the 192-wide tile taken 5 % slower per
        // column.
        const long cus = device_cus();
        const long t192 = tm * (N / 192);
        if ((t192 + cus - 1) / cus * 192 * 105 < (t256 + cus - 1) / cus * 256 * 100) {
            gemm_big2_kernel<T, Epi, true, 192><<<(unsigned)t192, 256, 0, s>>>(A, W, M, N, K, epi);
            return hipGetLastError();
        }
    }
    if (t256 >= 192) {
        // When the last round of 256 x 256 tiles would be at most
        // half full and made of whole tile columns (the 8B q/k/v product:
        // 384 tiles), those columns go to the 128 x 128 kernel instead, two
        // blocks per CU: measured 82 us for them there against a 113 us round.
        const long cus = device_cus();
        const long rem = t256 % cus;
        if (rem > 0 && 2 * rem <= cus && rem % tm == 0 && rem / tm < tn) {
            const int n1 = (int)(tn - rem / tm) * 256, nt = N - n1;
            gemm_big2_kernel<T, Epi, true><<<(unsigned)(tm * (tn - rem / tm)), 256, 0, s>>>(A, W, M, n1, K, epi);
            const long t = (long)((M + 127) / 128) * ((nt + 127) / 128);
            // the tiled weight rows from n1 on: row tile n1 / 16 onward
            gemm_mfma_kernel<T, 128, 128, 64, 64, 4, EpiShift<Epi>, true><<<(unsigned)t, 256, 0, s>>>(
                A, W + (size_t)(n1 / 16) * (K / 32) * 512, M, nt, K, EpiShift<Epi>{epi, n1});
        } else {
            gemm_big2_kernel<T, Epi, true><<<(unsigned)t256, 256, 0, s>>>(A, W, M, N, K, epi);
        }
    } else {
        const long t = (long)((M + 127) / 128) * ((N + 127) / 128);
        gemm_mfma_kernel<T, 128, 128, 64, 64, 4, Epi, true><<<(unsigned)t, 256, 0, s>>>(A, W, M, N, K, epi);
    }
    return hipGetLastError();
}

template <class Epi>
static hipError_t run_gemm_f32(const float* A, const float* W, int M, int N, int K, const Epi& epi,
                               hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const dim3 grid((N + 63) / 64, (M + 31) / 32);
    gemm_simple_kernel<Epi><<<grid, 256, 0, s>>>(A, W, M, N, K, epi);
    return hipGetLastError();
}

template <typename TO, typename TC>
static EpiQKV<TO, TC> make_qkv(const QkvEpi& e) {
    EpiQKV<TO, TC> r;
    r.q = (TO*)e.q;
    r.kws = (TO*)e.kws;
    r.vws = (TO*)e.vws;
    r.kc = (TC*)e.kc;
    r.vc = (TC*)e.vc;
    r.rope = e.rope;
    r.S = e.S;
    r.sp = e.sp;
    r.rope_half = e.rope_half;
    r.cap = e.cap;
    r.s_stride = e.s_stride;
    r.nkv = e.nkv;
    r.dh = e.dh;
    r.qd = e.qd;
    return r;
}

hipError_t gemm_qkv(Elem op, Elem cache, const void* A, const void* W, int M, int N, int K,
                    const QkvEpi& e, const SplitWs& part, hipStream_t s) {
    if (op == Elem::F32 && cache == Elem::F32)
        return run_gemm_f32((const float*)A, (const float*)W, M, N, K, make_qkv<float, float>(e), s);
    if (op == Elem::F16 && cache == Elem::BF16)
        return run_gemm((const f16*)A, (const f16*)W, M, N, K, make_qkv<f16, bf16>(e), part, s);
    if (op == Elem::BF16 && cache == Elem::BF16)
        return run_gemm((const bf16*)A, (const bf16*)W, M, N, K, make_qkv<bf16, bf16>(e), part, s);
    return hipErrorInvalidValue;
}

hipError_t gemm_resid(Elem op, Elem resid_t, const void* A, const void* W, int M, int N, int K,
                      const void* resid, float* out, const SplitWs& part, hipStream_t s) {
    if (op == Elem::F32 && resid_t == Elem::F32)
        return run_gemm_f32((const float*)A, (const float*)W, M, N, K,
                            EpiResid<float>{(const float*)resid, out, N}, s);
    if (op == Elem::F16 && resid_t == Elem::BF16)
        return run_gemm((const f16*)A, (const f16*)W, M, N, K, EpiResid<bf16>{(const bf16*)resid, out, N}, part, s);
    if (op == Elem::BF16 && resid_t == Elem::BF16)
        return run_gemm((const bf16*)A, (const bf16*)W, M, N, K, EpiResid<bf16>{(const bf16*)resid, out, N}, part, s);
    // fp32 residual (out may be resid itself: each element is read, then
    // written, by one thread)
    if (op == Elem::F16 && resid_t == Elem::F32)
        return run_gemm((const f16*)A, (const f16*)W, M, N, K, EpiResid<float>{(const float*)resid, out, N}, part, s);
    if (op == Elem::BF16 && resid_t == Elem::F32)
        return run_gemm((const bf16*)A, (const bf16*)W, M, N, K, EpiResid<float>{(const float*)resid, out, N}, part, s);
    return hipErrorInvalidValue;
}

hipError_t gemm_swiglu(Elem op, const void* A, const void* W, int M, int N, int K, void* z,
                       const SplitWs& part, hipStream_t s) {
    const int dff = N / 2;
    if (op == Elem::F32)
        return run_gemm_f32((const float*)A, (const float*)W, M, N, K, EpiSwiGLU<float>{(float*)z, dff}, s);
    if (op == Elem::F16)
        return run_gemm((const f16*)A, (const f16*)W, M, N, K, EpiSwiGLU<f16>{(f16*)z, dff}, part, s);
    if (op == Elem::BF16)
        return run_gemm((const bf16*)A, (const bf16*)W, M, N, K, EpiSwiGLU<bf16>{(bf16*)z, dff}, part, s);
    return hipErrorInvalidValue;
}

hipError_t gemm_out(Elem op, Elem out_t, const void* A, const void* W, int M, int N, int K,
                    const float* h, void* y, const SplitWs& part, hipStream_t s) {
    if (op == Elem::F32 && out_t == Elem::F32)
        return run_gemm_f32((const float*)A, (const float*)W, M, N, K, EpiOut<float>{h, (float*)y, N}, s);
    if (op == Elem::F16 && out_t == Elem::BF16)
        return run_gemm((const f16*)A, (const f16*)W, M, N, K, EpiOut<bf16>{h, (bf16*)y, N}, part, s);
    if (op == Elem::BF16 && out_t == Elem::BF16)
        return run_gemm((const bf16*)A, (const bf16*)W, M, N, K, EpiOut<bf16>{h, (bf16*)y, N}, part, s);
    return hipErrorInvalidValue;
}

hipError_t decode_qkv(Elem op, Elem cache, const void* At, const void* Wt, int M, int N, int K,
                      const QkvEpi& e, const SplitWs& part, hipStream_t s) {
    if (op == Elem::F16 && cache == Elem::BF16)
        return run_decode((const f16*)At, (const f16*)Wt, M, N, K, make_qkv<f16, bf16>(e), part, s);
    if (op == Elem::BF16 && cache == Elem::BF16)
        return run_decode((const bf16*)At, (const bf16*)Wt, M, N, K, make_qkv<bf16, bf16>(e), part, s);
    return hipErrorInvalidValue;
}

hipError_t decode_resid(Elem op, Elem resid_t, const void* At, const void* Wt, int M, int N, int K,
                        const void* resid, float* out, const SplitWs& part, hipStream_t s) {
    if (resid_t != Elem::BF16) return hipErrorInvalidValue;
    if (op == Elem::F16)
        return run_decode((const f16*)At, (const f16*)Wt, M, N, K, EpiResid<bf16>{(const bf16*)resid, out, N}, part, s);
    if (op == Elem::BF16)
        return run_decode((const bf16*)At, (const bf16*)Wt, M, N, K, EpiResid<bf16>{(const bf16*)resid, out, N}, part, s);
    return hipErrorInvalidValue;
}

hipError_t decode_swiglu(Elem op, const void* At, const void* Wt, int M, int N, int K, void* zt,
                         const SplitWs& part, hipStream_t s) {
    const int dff = N / 2, mt = decode_row_tiles(M);
    if (op == Elem::F16)
        return run_decode((const f16*)At, (const f16*)Wt, M, N, K, EpiSwiGLU<f16>{(f16*)zt, dff, mt}, part, s);
    if (op == Elem::BF16)
        return run_decode((const bf16*)At, (const bf16*)Wt, M, N, K, EpiSwiGLU<bf16>{(bf16*)zt, dff, mt}, part, s);
    return hipErrorInvalidValue;
}

hipError_t decode_out(Elem op, Elem out_t, const void* At, const void* Wt, int M, int N, int K,
                      const float* h, void* y, const SplitWs& part, hipStream_t s) {
    if (out_t != Elem::BF16) return hipErrorInvalidValue;
    if (op == Elem::F16)
        return run_decode((const f16*)At, (const f16*)Wt, M, N, K, EpiOut<bf16>{h, (bf16*)y, N}, part, s);
    if (op == Elem::BF16)
        return run_decode((const bf16*)At, (const bf16*)Wt, M, N, K, EpiOut<bf16>{h, (bf16*)y, N}, part, s);
    return hipErrorInvalidValue;
}

}  // namespace lb
