// Device-side types and helpers shared by the block's HIP kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lb {

typedef _Float16 f16;
typedef __bf16 bf16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// Start position of every sequence of one forward: all at `base`, (ragged)
// sequence b at pos[b], b < kMaxRagged, or (dev != nullptr) read at run time
// from the device array dev[b] and clamped to [0, lim], so that no value in
// that array can take an access out of the cache or the RoPE table.  Passed by
// value in kernel arguments; device code reads it through LB_SEQ_START, which
// names the members of the argument itself (a member function taking `this`
// would copy the argument to scratch memory).
constexpr int kMaxRagged = 64;
struct SeqPos {
    int base;
    int ragged;
    int pos[kMaxRagged];
    const int* dev;
    int lim;
};
#define LB_SEQ_START(sp, b)                                                  \
    ((sp).dev ? min(max((sp).dev[(b)], 0), (sp).lim)                        \
              : ((sp).ragged ? (sp).pos[(b)] : (sp).base))

// ---- scalar conversions (fp32 <-> storage types, round to nearest even) ----
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(f16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ f16 from_f32<f16>(float v) { return (f16)v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// ---- 8-element vector loads/stores through fp32 ------------------------------
// 16-bit types move as one 16-byte access, fp32 as two.  Pointers must be
// aligned to the access size.
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
}
__device__ __forceinline__ void load8(const f16* p, float (&v)[8]) {
    f16x8 a = *reinterpret_cast<const f16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)a[i];
}
__device__ __forceinline__ void load8(const bf16* p, float (&v)[8]) {
    bf16x8 a = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)a[i];
}

// The same loads split in two: fetch8 issues the access into a Raw8 holding
// the stored type, widen8 converts it once the data is needed, so that several
// fetches can be in flight before the first conversion waits on one.
template <typename T> struct Raw8;
template <> struct Raw8<float> { f32x4 a, b; };
template <> struct Raw8<f16> { f16x8 a; };
template <> struct Raw8<bf16> { bf16x8 a; };
__device__ __forceinline__ void fetch8(const float* p, Raw8<float>& r) {
    r.a = *reinterpret_cast<const f32x4*>(p);
    r.b = *reinterpret_cast<const f32x4*>(p + 4);
}
__device__ __forceinline__ void fetch8(const f16* p, Raw8<f16>& r) { r.a = *reinterpret_cast<const f16x8*>(p); }
__device__ __forceinline__ void fetch8(const bf16* p, Raw8<bf16>& r) { r.a = *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ void widen8(const Raw8<float>& r, float (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = r.a[i]; v[4 + i] = r.b[i]; }
}
template <typename T> __device__ __forceinline__ void widen8(const Raw8<T>& r, float (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)r.a[i];
}

__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] = v[i]; b[i] = v[4 + i]; }
    *reinterpret_cast<f32x4*>(p) = a;
    *reinterpret_cast<f32x4*>(p + 4) = b;
}
__device__ __forceinline__ void store8(f16* p, const float (&v)[8]) {
    f16x8 a;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = (f16)v[i];
    *reinterpret_cast<f16x8*>(p) = a;
}
__device__ __forceinline__ void store8(bf16* p, const float (&v)[8]) {
    bf16x8 a;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = (bf16)v[i];
    *reinterpret_cast<bf16x8*>(p) = a;
}

// 4-element stores (8 bytes for 16-bit types, 16 for fp32).
template <typename T> __device__ __forceinline__ void store4(T* p, const float* v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = from_f32<T>(v[i]);
}

// 2^x from the hardware base-2 exponential (about 1 ulp; -inf gives 0 and
// results below the smallest normal flush toward zero).  Used where the result
// only ever meets a sum that is at least one: softmax weights and SiLU.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// A 16-byte operand load, with the non-temporal hint when NT (data read once
// per call that should not displace reusable lines).
template <bool NT, typename V>
__device__ __forceinline__ V load_w(const V* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

// ---- wavefront reductions (64 lanes, fixed butterfly order) ----------------
// Each step combines a lane with its partner in a group twice the size of the
// last: quad permutes (groups of 2 and 4), the row half-mirror (8) and row
// mirror (16) of DPP, then the 16- and 32-lane half swaps.  Every step runs in
// the vector ALU (no LDS round trip), and partners add the same two values,
// so every lane ends with the same, deterministic result.
template <int CTRL> __device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <class Op> __device__ __forceinline__ float wave_reduce(float v, Op op) {
    v = op(v, dpp_mov<0xB1>(v));   // quad_perm [1,0,3,2]
    v = op(v, dpp_mov<0x4E>(v));   // quad_perm [2,3,0,1]
    v = op(v, dpp_mov<0x141>(v));  // row_half_mirror
    v = op(v, dpp_mov<0x140>(v));  // row_mirror
    const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = op(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
    const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return op(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
}
__device__ __forceinline__ float wave_sum(float v) {
    return wave_reduce(v, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ float wave_max(float v) {
    return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}

// ---- MFMA wrappers -------------------------------------------------------------
// 32x32x16: A lane l holds row (l%32) and 8 k values, B lane l holds column
// (l%32) and the same 8 k slots; D lane l, register r holds
// row 8*(r/4) + 4*(l/32) + r%4, column l%32.
__device__ __forceinline__ f32x16 mfma32(const f16x8& a, const f16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 16x16x32: A lane l holds row (l%16) and 8 k values, B lane l column (l%16);
// D lane l, register r holds row 4*(l/16) + r, column l%16.
__device__ __forceinline__ f32x4 mfma16(const f16x8& a, const f16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The same products accumulating in place: the accumulator is one AGPR tuple
// that the instruction reads and writes (the builtins above may get a
// destination apart from the accumulator, which makes the register allocator
// shuffle accumulators through other registers when every AGPR holds one).
// The compiler does not see these as matrix instructions and inserts none of
// the wait states they need: after the last one, call mfma_drain() before
// any other instruction reads the accumulators, and feed them only operands
// that come straight from memory loads (which the compiler waits for as for
// any inline-asm input) -- an operand written by a vector ALU instruction
// just before (a select, a move) can be read stale.
__device__ __forceinline__ void mfma16_tied(f32x4& c, const f16x8& a, const f16x8& b) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16_tied(f32x4& c, const bf16x8& a, const bf16x8& b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// 24 wait states: more than the result latency of a 16x16x32 product
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// ---- decode operand layout -------------------------------------------------------
// Token-batch GEMMs of the decode path read their operands in "k-step tiles":
// for an operand with rows r (tokens or weight rows) and K columns, the 16
// rows of row tile rt and the 32 columns of k-step ks form one contiguous
// 1 KB piece whose 16-byte chunk l (l = 16 * (k % 32 / 8) + r % 16) is
// exactly what lane l of a 16x16x32 MFMA operand needs.
//   activations [M rows, MT row tiles]: piece (ks * MT + rt)
//   weights     [N rows]:               piece (rt * (K / 32) + ks)
// Element offset of (r, k) inside its piece:
__host__ __device__ __forceinline__ int ktile_in_piece(int r, int k) {
    return ((((k >> 3) & 3) << 4) + (r & 15)) * 8 + (k & 7);
}
__host__ __device__ __forceinline__ size_t ktile_act_off(int m, int k, int mt) {
    return ((size_t)(k >> 5) * mt + (m >> 4)) * 512 + ktile_in_piece(m, k);
}
__host__ __device__ __forceinline__ size_t ktile_w_off(int n, int k, int K) {
    return ((size_t)(n >> 4) * (K >> 5) + (k >> 5)) * 512 + ktile_in_piece(n, k);
}

// ---- direct-to-LDS loads issued from inline assembly -------------------------------
// One global_load_lds_dwordx4: lane l copies 16 bytes from g (its own
// address) to LDS byte address lds_byte_addr + 16 * l (M0 holds the
// wave-uniform base).  The compiler does not see these loads, so its waits
// for ordinary LDS reads stay exact; the caller waits for them with wait_vm
// (they are the only vector-memory loads in flight where it does) before a
// barrier that publishes the data.
__device__ __forceinline__ void lds_dma16(const void* g, unsigned lds_byte_addr) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_byte_addr)
                 : "memory", "m0");
}
// The same load from a wave-uniform base address (in SGPRs) plus a per-lane
// 32-bit byte offset: no per-lane 64-bit address arithmetic.  NT adds the
// non-temporal hint (data read once).
template <bool NT = false>
__device__ __forceinline__ void lds_dma16_s(const void* sbase, unsigned voff, unsigned lds_byte_addr) {
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase),
                     "s"(lds_byte_addr)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
                     "s"(lds_byte_addr)
                     : "memory", "m0");
}
// 16-byte accesses through a buffer resource with the agent-scope coherence
// bit (sc1), the cache policy of relaxed device-scope atomics: a store is
// visible to a later sc1 load from any XCD once it has completed (vmcnt), with
// no cache-wide write-back or invalidate.  Offsets in bytes; accesses beyond
// 2 GiB from the base are dropped by the range check.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t agent_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ void store16_agent(__amdgpu_buffer_rsrc_t r, unsigned off, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 16);
}
__device__ __forceinline__ f32x4 load16_agent(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16));
}

template <int N> __device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// 8-element operand vector of a 16-bit type.
template <typename T> struct vec8;
template <> struct vec8<f16> { typedef f16x8 type; };
template <> struct vec8<bf16> { typedef bf16x8 type; };

}  // namespace lb
