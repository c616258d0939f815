// Measured peaks of the two rooflines the forward is reported against: a
// streaming copy (HBM bandwidth) and a loop of independent bf16 matrix-core
// products (dense MFMA throughput). They compute nothing of the method; the
// benchmark divides the forward's algorithmic bytes and flops by these rates
// as well as by the published ones.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdr_peaks.h"

namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;      // 16-byte loads in flight per lane

// Grid-stride copy of n16 16-byte units: each lane keeps kCopyUnroll loads in
// flight before it stores them.
__global__ __launch_bounds__(kCopyThreads) void k_peak_copy(const u4* __restrict__ src, u4* __restrict__ dst,
                                                            int64_t n16) {
    const int64_t step = (int64_t)gridDim.x * kCopyThreads * kCopyUnroll;
    int64_t i = (int64_t)blockIdx.x * kCopyThreads * kCopyUnroll + threadIdx.x;
    for (; i + (kCopyUnroll - 1) * kCopyThreads < n16; i += step) {
        u4 x[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) x[u] = __builtin_nontemporal_load(src + i + u * kCopyThreads);
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) __builtin_nontemporal_store(x[u], dst + i + u * kCopyThreads);
    }
    for (; i < n16; i += kCopyThreads) dst[i] = src[i];
}

constexpr int kMfmaChains = 8;      // independent accumulators per wave

// Each wave issues iters x kMfmaChains v_mfma_f32_16x16x32_bf16 on operands
// held in registers; one value per lane is stored so that nothing is dropped.
__global__ __launch_bounds__(256) void k_peak_mfma(float* __restrict__ out, int32_t iters) {
    const int tid = threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(1.0f + 0.001f * (float)((tid + e) & 7));
        b[e] = (__bf16)(0.5f - 0.001f * (float)((tid * 3 + e) & 7));
    }
    f32x4 acc[kMfmaChains];
#pragma unroll
    for (int j = 0; j < kMfmaChains; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kMfmaChains; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kMfmaChains; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    out[(int64_t)blockIdx.x * blockDim.x + tid] = s;
}

}  // namespace

extern "C" int gdr_peak_copy(const void* src, void* dst, size_t bytes, int32_t blocks, void* stream) {
    if (!src || !dst || bytes % 16 != 0 || blocks <= 0 || (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16)
        return 1;
    k_peak_copy<<<blocks, kCopyThreads, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u4*>(src), static_cast<u4*>(dst), (int64_t)(bytes / 16));
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int gdr_peak_mfma(float* out, int32_t blocks, int32_t iters, void* stream) {
    if (!out || blocks <= 0 || iters <= 0) return 1;
    k_peak_mfma<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(out, iters);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" double gdr_peak_mfma_flops(int32_t blocks, int32_t iters) {
    return (double)blocks * 4.0 * iters * kMfmaChains * (2.0 * 16 * 16 * 32);
}
