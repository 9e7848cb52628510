// GEMM dispatch for the four projections of the block.
#include "epilogues.h"
#include "gemm_kernels.h"
#include "launch.h"

namespace lb {

template <typename T, class Epi>
static hipError_t run_gemm(const T* A, const T* W, int M, int N, int K, const Epi& epi,
                           hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if (M <= 64) {
        const dim3 grid((N + 15) / 16);
        if (M <= 16) gemm_skinny_kernel<T, 1, 8, Epi><<<grid, 512, 0, s>>>(A, W, M, N, K, epi);
        else if (M <= 32) gemm_skinny_kernel<T, 2, 8, Epi><<<grid, 512, 0, s>>>(A, W, M, N, K, epi);
        else gemm_skinny_kernel<T, 4, 8, Epi><<<grid, 512, 0, s>>>(A, W, M, N, K, epi);
        return hipGetLastError();
    }
    const long big_tiles = (long)((M + 255) / 256) * ((N + 255) / 256);
    if (big_tiles >= 192) {
        gemm_mfma_kernel<T, 256, 256, 128, 128, Epi><<<(unsigned)big_tiles, 256, 0, s>>>(A, W, M, N, K, epi);
    } else {
        const long t = (long)((M + 127) / 128) * ((N + 127) / 128);
        gemm_mfma_kernel<T, 128, 128, 64, 64, Epi><<<(unsigned)t, 256, 0, s>>>(A, W, M, N, K, epi);
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
                    const QkvEpi& e, hipStream_t s) {
    if (op == Elem::F32 && cache == Elem::F32)
        return run_gemm_f32((const float*)A, (const float*)W, M, N, K, make_qkv<float, float>(e), s);
    if (op == Elem::F16 && cache == Elem::BF16)
        return run_gemm((const f16*)A, (const f16*)W, M, N, K, make_qkv<f16, bf16>(e), s);
    if (op == Elem::BF16 && cache == Elem::BF16)
        return run_gemm((const bf16*)A, (const bf16*)W, M, N, K, make_qkv<bf16, bf16>(e), s);
    return hipErrorInvalidValue;
}

hipError_t gemm_resid(Elem op, Elem resid_t, const void* A, const void* W, int M, int N, int K,
                      const void* resid, float* out, hipStream_t s) {
    if (op == Elem::F32 && resid_t == Elem::F32)
        return run_gemm_f32((const float*)A, (const float*)W, M, N, K,
                            EpiResid<float>{(const float*)resid, out, N}, s);
    if (op == Elem::F16 && resid_t == Elem::BF16)
        return run_gemm((const f16*)A, (const f16*)W, M, N, K, EpiResid<bf16>{(const bf16*)resid, out, N}, s);
    if (op == Elem::BF16 && resid_t == Elem::BF16)
        return run_gemm((const bf16*)A, (const bf16*)W, M, N, K, EpiResid<bf16>{(const bf16*)resid, out, N}, s);
    return hipErrorInvalidValue;
}

hipError_t gemm_swiglu(Elem op, const void* A, const void* W, int M, int N, int K, void* z,
                       hipStream_t s) {
    const int dff = N / 2;
    if (op == Elem::F32)
        return run_gemm_f32((const float*)A, (const float*)W, M, N, K, EpiSwiGLU<float>{(float*)z, dff}, s);
    if (op == Elem::F16)
        return run_gemm((const f16*)A, (const f16*)W, M, N, K, EpiSwiGLU<f16>{(f16*)z, dff}, s);
    if (op == Elem::BF16)
        return run_gemm((const bf16*)A, (const bf16*)W, M, N, K, EpiSwiGLU<bf16>{(bf16*)z, dff}, s);
    return hipErrorInvalidValue;
}

hipError_t gemm_out(Elem op, Elem out_t, const void* A, const void* W, int M, int N, int K,
                    const float* h, void* y, hipStream_t s) {
    if (op == Elem::F32 && out_t == Elem::F32)
        return run_gemm_f32((const float*)A, (const float*)W, M, N, K, EpiOut<float>{h, (float*)y, N}, s);
    if (op == Elem::F16 && out_t == Elem::BF16)
        return run_gemm((const f16*)A, (const f16*)W, M, N, K, EpiOut<bf16>{h, (bf16*)y, N}, s);
    if (op == Elem::BF16 && out_t == Elem::BF16)
        return run_gemm((const bf16*)A, (const bf16*)W, M, N, K, EpiOut<bf16>{h, (bf16*)y, N}, s);
    return hipErrorInvalidValue;
}

}  // namespace lb
