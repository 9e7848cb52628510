// GEMM dispatch for the four projections of the block.
#include "epilogues.h"
#include "gemm_kernels.h"
#include "launch.h"

namespace lb {

size_t skinny_partials_floats(int max_m, int max_n) { return (size_t)kSkinnyMaxSplit * max_m * max_n; }

// Decode GEMM launch: CT column tiles per wavefront, split-K over KS blocks
// so that a launch has >= ~256 blocks even for narrow outputs.
template <typename T, int MT, class Epi>
static hipError_t run_skinny(const T* A, const T* W, int M, int N, int K, const Epi& epi,
                             float* part, size_t part_cap, hipStream_t s) {
    if constexpr (MT <= 2) {
        if (N >= 128 * 192) {  // wide outputs: 128 columns per wavefront, no split
            const dim3 grid((N + 127) / 128, 1);
            gemm_skinny_kernel<T, MT, 8, 1, 8, false, Epi><<<grid, 512, 0, s>>>(A, W, M, N, K, 1, part, epi);
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
        gemm_skinny_kernel<T, MT, 4, 2, 4, false, Epi><<<grid, 256, 0, s>>>(A, W, M, N, K, 1, part, epi);
        return hipGetLastError();
    }
    gemm_skinny_kernel<T, MT, 4, 2, 4, true, Epi><<<grid, 256, 0, s>>>(A, W, M, N, K, ks, part, epi);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    reduce_epilogue_kernel<Epi><<<(M * (N / 8) + 255) / 256, 256, 0, s>>>(part, M, N, ks, epi);
    return hipGetLastError();
}

template <typename T, class Epi>
static hipError_t run_gemm(const T* A, const T* W, int M, int N, int K, const Epi& epi,
                           const SplitWs& ws, hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if (M <= 16) return run_skinny<T, 1>(A, W, M, N, K, epi, ws.part, ws.cap, s);
    if (M <= 32) return run_skinny<T, 2>(A, W, M, N, K, epi, ws.part, ws.cap, s);
    if (M <= 64) return run_skinny<T, 4>(A, W, M, N, K, epi, ws.part, ws.cap, s);
    const long big_tiles = (long)((M + 255) / 256) * ((N + 255) / 256);
    if (big_tiles >= 192) {
        gemm_mfma_kernel<T, 256, 256, 128, 64, 8, Epi><<<(unsigned)big_tiles, 512, 0, s>>>(A, W, M, N, K, epi);
    } else {
        const long t = (long)((M + 127) / 128) * ((N + 127) / 128);
        gemm_mfma_kernel<T, 128, 128, 64, 64, 4, Epi><<<(unsigned)t, 256, 0, s>>>(A, W, M, N, K, epi);
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
    r.start_pos = e.start_pos;
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

}  // namespace lb
