// Device-side building blocks shared by the chunked gated delta-rule kernels.
//
// Matrix-core conventions (CDNA4 / gfx950, 64-lane wavefronts; lane l = 16*qd + r):
//
//  * Accumulator tile: a 16x16 fp32 block Y; lane l holds Y[4*qd + j][r], j = 0..3.
//    This is the result layout of v_mfma_f32_16x16x32_bf16 and v_mfma_f32_16x16x4_f32.
//
//  * Pair fragment: one operand of a 16x16 (rows) by 32 (contraction) product.
//    Lane l holds 8 values X[r][m(qd, e)] with
//        m(qd, e) = 4*qd + e            for e < 4
//        m(qd, e) = 16 + 4*qd + e - 4   for e >= 4.
//    The contraction order is a permutation of 0..31 that only has to agree
//    between the two operands of a product. It is chosen so that two
//    accumulator tiles stacked along the contraction index (rows 0..15 and
//    16..31) ARE a pair fragment of the transposed block, element for
//    element: an MFMA result feeds the next MFMA as an operand without any
//    data movement between lanes. Loading a pair fragment from a row-major
//    row costs two 4-element vector loads.
//
//  * bf16 pairs use one v_mfma_f32_16x16x32_bf16 (lane element e sits in
//    instruction slot 8*qd + e). fp32 pairs use eight v_mfma_f32_16x16x4_f32,
//    element e of every lane forming the e-th 4-deep slice.
//
// Precision: inputs (q, k, v) are exact in the compute type T. Every operand
// derived inside the method (A, W, U, the state, V_new, the score block) is an
// fp32 value; when T is bf16 it enters a product as an unevaluated sum
// hi + lo of two bf16 values (hi = rne(x), lo = rne(x - hi)), which carries
// about 16 significant bits. A product with one exact input operand then takes
// two MFMA passes, a product of two derived operands three (hi*hi, hi*lo,
// lo*hi); the dropped lo*lo term is below fp32 rounding of the sum. When T is
// fp32 every operand is exact and each product is a single pass.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <typename T> struct Vec;
template <> struct Vec<bf16> {
    typedef bf16 v8 __attribute__((ext_vector_type(8)));
    typedef bf16 v4 __attribute__((ext_vector_type(4)));
};
template <> struct Vec<float> {
    typedef float v8 __attribute__((ext_vector_type(8)));
    typedef float v4 __attribute__((ext_vector_type(4)));
};

constexpr int kChunk = 64;     // chunk length C
constexpr int kWave = 64;      // wavefront size

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ---------------------------------------------------------------- conversions
template <typename T> __device__ __forceinline__ T to_t(float x);
template <> __device__ __forceinline__ bf16 to_t<bf16>(float x) { return (bf16)x; }   // RNE
template <> __device__ __forceinline__ float to_t<float>(float x) { return x; }

template <typename T> __device__ __forceinline__ float to_f(T x) { return (float)x; }

// ---------------------------------------------------------------- MFMA wrappers
__device__ __forceinline__ f32x4 mfma_pair(const Vec<bf16>::v8& a, const Vec<bf16>::v8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_pair(const Vec<float>::v8& a, const Vec<float>::v8& b, f32x4 c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
}

// ---------------------------------------------------------------- fragments
template <typename T>
__device__ __forceinline__ typename Vec<T>::v8 concat(const typename Vec<T>::v4& lo, const typename Vec<T>::v4& hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <typename T>
__device__ __forceinline__ typename Vec<T>::v8 zero_pair() {
    typename Vec<T>::v8 z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = to_t<T>(0.f);
    return z;
}

// Pair fragment of a row-major row: p points at contraction index 0 of the
// 32-block; needs 4-element alignment of p.
template <typename T>
__device__ __forceinline__ typename Vec<T>::v8 load_pair_row(const T* p, int qd) {
    typedef typename Vec<T>::v4 v4;
    v4 lo = *reinterpret_cast<const v4*>(p + 4 * qd);
    v4 hi = *reinterpret_cast<const v4*>(p + 16 + 4 * qd);
    return concat<T>(lo, hi);
}

// Same, from an fp32 row (LDS), converted to T.
template <typename T>
__device__ __forceinline__ typename Vec<T>::v8 load_pair_row_f32(const float* p, int qd) {
    typename Vec<T>::v8 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[e] = to_t<T>(p[4 * qd + e]);
        v[4 + e] = to_t<T>(p[16 + 4 * qd + e]);
    }
    return v;
}

// Two accumulator tiles (contraction rows 0..15 and 16..31) as a pair fragment.
template <typename T>
__device__ __forceinline__ typename Vec<T>::v8 acc_to_pair(const f32x4& a0, const f32x4& a1) {
    typename Vec<T>::v8 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[j] = to_t<T>(a0[j]);
        v[4 + j] = to_t<T>(a1[j]);
    }
    return v;
}

// Fragment-major storage: a pair fragment occupies 64 lanes x 8 values, an
// accumulator tile 64 lanes x 4 values, lane-contiguous.
template <typename T>
__device__ __forceinline__ typename Vec<T>::v8 load_frag(const T* base, int lane) {
    return *reinterpret_cast<const typename Vec<T>::v8*>(base + lane * 8);
}
template <typename T>
__device__ __forceinline__ void store_frag(T* base, int lane, const typename Vec<T>::v8& v) {
    *reinterpret_cast<typename Vec<T>::v8*>(base + lane * 8) = v;
}
template <typename T>
__device__ __forceinline__ f32x4 load_tile(const T* base, int lane) {
    typename Vec<T>::v4 v = *reinterpret_cast<const typename Vec<T>::v4*>(base + lane * 4);
    f32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = to_f(v[j]);
    return r;
}
template <typename T>
__device__ __forceinline__ void store_tile(T* base, int lane, const f32x4& x) {
    typename Vec<T>::v4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = to_t<T>(x[j]);
    *reinterpret_cast<typename Vec<T>::v4*>(base + lane * 4) = v;
}
// Half of a pair fragment (elements 4*half .. 4*half+3) from one accumulator tile.
template <typename T>
__device__ __forceinline__ void store_pair_half(T* base, int lane, int half, const f32x4& x) {
    typename Vec<T>::v4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = to_t<T>(x[j]);
    *reinterpret_cast<typename Vec<T>::v4*>(base + lane * 8 + 4 * half) = v;
}

// ---------------------------------------------------------------- split operands
template <typename T> struct Split {
    typename Vec<T>::v8 hi, lo;
};
template <typename T> inline constexpr bool kSplitNeeded = false;
template <> inline constexpr bool kSplitNeeded<bf16> = true;

// fp32 values -> hi/lo pair fragment (lo unused for fp32)
template <typename T>
__device__ __forceinline__ Split<T> split8(const float (&x)[8]) {
    Split<T> s;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        s.hi[e] = to_t<T>(x[e]);
        if constexpr (kSplitNeeded<T>) s.lo[e] = to_t<T>(x[e] - to_f(s.hi[e]));
    }
    return s;
}
template <typename T>
__device__ __forceinline__ Split<T> split_acc_pair(const f32x4& a0, const f32x4& a1) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[j] = a0[j];
        x[4 + j] = a1[j];
    }
    return split8<T>(x);
}
template <typename T>
__device__ __forceinline__ Split<T> split_v8(const typename Vec<float>::v8& v) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = v[e];
    return split8<T>(x);
}
// Row-major fp32 row (global or LDS) -> split pair fragment.
template <typename T>
__device__ __forceinline__ Split<T> load_split_row(const float* p, int qd) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[e] = p[4 * qd + e];
        x[4 + e] = p[16 + 4 * qd + e];
    }
    return split8<T>(x);
}

// exact (a) times derived (b): 2 passes for bf16
template <typename T>
__device__ __forceinline__ f32x4 mfma_xd(const typename Vec<T>::v8& a, const Split<T>& b, f32x4 c) {
    if constexpr (kSplitNeeded<T>) c = mfma_pair(a, b.lo, c);
    return mfma_pair(a, b.hi, c);
}
// derived (a) times exact (b)
template <typename T>
__device__ __forceinline__ f32x4 mfma_dx(const Split<T>& a, const typename Vec<T>::v8& b, f32x4 c) {
    if constexpr (kSplitNeeded<T>) c = mfma_pair(a.lo, b, c);
    return mfma_pair(a.hi, b, c);
}
// derived times derived: 3 passes for bf16
template <typename T>
__device__ __forceinline__ f32x4 mfma_dd(const Split<T>& a, const Split<T>& b, f32x4 c) {
    if constexpr (kSplitNeeded<T>) {
        c = mfma_pair(a.lo, b.hi, c);
        c = mfma_pair(a.hi, b.lo, c);
    }
    return mfma_pair(a.hi, b.hi, c);
}

// fp32 fragment-major storage (8 floats per lane for a pair, 4 for a tile)
__device__ __forceinline__ typename Vec<float>::v8 load_frag_f32(const float* base, int lane) {
    return *reinterpret_cast<const typename Vec<float>::v8*>(base + lane * 8);
}
__device__ __forceinline__ void store_frag_f32(float* base, int lane, const typename Vec<float>::v8& v) {
    *reinterpret_cast<typename Vec<float>::v8*>(base + lane * 8) = v;
}
__device__ __forceinline__ f32x4 load_tile_f32(const float* base, int lane) {
    return *reinterpret_cast<const f32x4*>(base + lane * 4);
}
__device__ __forceinline__ void store_tile_f32(float* base, int lane, const f32x4& x) {
    *reinterpret_cast<f32x4*>(base + lane * 4) = x;
}
__device__ __forceinline__ void store_pair_half_f32(float* base, int lane, int half, const f32x4& x) {
    *reinterpret_cast<f32x4*>(base + lane * 8 + 4 * half) = x;
}

// Global -> LDS copies without registers: lane l's 16 (or 4) bytes at byte
// offset voffset of the buffer land at lds_dst + 16 l (or 4 l); lds_dst is
// wave-uniform. Completion is tracked by the issuing wave's vector memory counter.
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t rs, const void* lds_dst, int voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_dst, 16, voffset, 0, 0, 0);
}
__device__ __forceinline__ void buffer_to_lds4(__amdgpu_buffer_rsrc_t rs, const void* lds_dst, int voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_dst, 4, voffset, 0, 0, 0);
}

// Range-checked loads: a buffer of `bytes` bytes at `base`; an access at or past
// its end reads zero. A load whose invalid lanes fall outside the range needs
// no select on the loaded value, so the wave does not wait for the load until
// the value is used.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ f32x4 buf_ld_f32x4(__amdgpu_buffer_rsrc_t rs, int voffset) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voffset, 0, 0));
}
__device__ __forceinline__ float buf_ld_f32(__amdgpu_buffer_rsrc_t rs, int voffset) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, voffset, 0, 0));
}

// Workgroup barrier for LDS traffic: this wave's LDS operations complete, then
// all waves of the workgroup meet. Unlike __syncthreads() it does not wait for
// the wave's outstanding global loads, stores or global-to-LDS copies; a copy
// whose data the other waves read after the barrier needs an explicit
// vector-memory wait first (wait_vmem()).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N of this wave's vector memory operations are outstanding
// (they complete in issue order, so every older one has finished).
template <int N>
__device__ __forceinline__ void wait_vmem_but() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ float load_beta(const void* beta, int64_t idx, int beta_f32) {
    return beta_f32 ? reinterpret_cast<const float*>(beta)[idx]
                    : (float)reinterpret_cast<const bf16*>(beta)[idx];
}

}  // namespace gdr
