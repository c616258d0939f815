// Token-by-token (fused recurrent) forward of the gated delta rule for gfx950:
// the form for decoding and short inputs, where a chunk would be mostly empty
// (FLA notes page, "fused recurrent fwd": one program per sequence and head
// walks the tokens and keeps the state on chip; the model layer takes this
// path when the query is at most 64 tokens long, FLA notes RetNet section).
//
// Per token t of a sequence, for every value head h (q/k head kh = h / (Nv/Nk)):
//   S   <- exp(g_t) S                                   decay first
//   u    = beta_t (v_t - S^T k_t)                       delta read from the decayed state
//   S   <- S + k_t u^T
//   o_t  = scale S^T q_t
// (ChunkGatedDeltaRule page, section 1, with the delta read from the decayed
// state; FLA DeltaNet article, section 1, for the loop order: write, then read.)
// With use_qk_l2norm, q_t and k_t are first divided by sqrt(sum of squares +
// 1e-6) inside the kernel (FLA DeltaNet article, section 5, the in-kernel L2
// normalisation option).
//
// Mapping: one workgroup per (sequence, value head), one wavefront per 256 / RQ
// columns of dv (RQ = dk / 16; at most four wavefronts). Lane l = RQ cg + rq
// owns columns 4 cg .. 4 cg + 3 of its wavefront's column block over rows
// 16 rq .. 16 rq + 15: 64 state values in registers, so that four wavefronts
// fit on a SIMD. S^T k and S^T q are sums over the lane's rows followed by a
// butterfly over the RQ lanes of a group. Each lane reads its 16 elements of
// q_t and k_t straight from global memory (the lanes of one row range read the
// same bytes); beta and g are wave-uniform scalar loads. The state moves in
// and out with 16-byte non-temporal accesses (it is read and written once),
// four columns of one row per access. The arithmetic is fp32 throughout; o is
// rounded once, at the store.
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {

namespace {

constexpr int kRowsPerLane = 16;

// 16 consecutive elements of a q/k row -> fp32 (16-byte loads; the offset is a
// multiple of 16 elements)
__device__ __forceinline__ void load_part(const bf16* p, float* x) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const uint4 w = *reinterpret_cast<const uint4*>(p + 8 * c);
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[8 * c + 2 * e] = __uint_as_float(u[e] << 16);
            x[8 * c + 2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
        }
    }
}
__device__ __forceinline__ void load_part(const float* p, float* x) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float4 w = *reinterpret_cast<const float4*>(p + 4 * c);
        x[4 * c] = w.x;
        x[4 * c + 1] = w.y;
        x[4 * c + 2] = w.z;
        x[4 * c + 3] = w.w;
    }
}
// sum over the RQ adjacent lanes of a group
template <int RQ>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int m = 1; m < RQ; m <<= 1) x += __shfl_xor(x, m, 64);
    return x;
}

template <typename T, int DK>
__global__ __launch_bounds__(256, 4) void k_recurrent(const T* __restrict__ q, const T* __restrict__ k,
                                                   const T* __restrict__ v, const void* __restrict__ beta,
                                                   int beta_f32, const float* __restrict__ g,
                                                   const float* __restrict__ S0, const int32_t* __restrict__ cu,
                                                   int64_t T_row, int64_t Ttot, int32_t Nk, int32_t Nv, int32_t DV,
                                                   float scale, int l2norm, int out_f32, void* __restrict__ o,
                                                   float* __restrict__ ST) {
    constexpr int RPL = kRowsPerLane;
    constexpr int RQ = DK / RPL;                 // lanes per column group (2, 4 or 8)
    constexpr int COLS = 4 * 64 / RQ;            // state columns per wavefront
    static_assert(DK % RPL == 0 && RQ >= 2 && RQ <= 8, "dk");
    const int n = blockIdx.x, h = blockIdx.y;
    const int lane = threadIdx.x & 63, rq = lane % RQ, cg = lane / RQ;
    const int j0 = (threadIdx.x >> 6) * COLS + 4 * cg;   // this lane's first state column (wavefront = column block)
    const bool active = j0 < DV;                 // DV is a multiple of 32: all four columns or none
    const int r0 = rq * RPL;                     // this lane's first state row
    const int kh = h / (Nv / Nk);
    int64_t s = cu ? (int64_t)cu[n] : (int64_t)n * T_row;
    int64_t e = cu ? (int64_t)cu[n + 1] : (int64_t)(n + 1) * T_row;
    s = s < 0 ? 0 : (s > Ttot ? Ttot : s);       // offsets clamped to the token range
    e = e < s ? s : (e > Ttot ? Ttot : e);

    const int64_t sbase = ((int64_t)n * Nv + h) * DK * DV;
    f32x4 S[RPL];                                // S[i][c]: row r0 + i, column j0 + c
#pragma unroll
    for (int i = 0; i < RPL; ++i)
        S[i] = (S0 && active)
                   ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(&S0[sbase + (int64_t)(r0 + i) * DV + j0]))
                   : f32x4{0.f, 0.f, 0.f, 0.f};

    for (int64_t t = s; t < e; ++t) {
        const int64_t row = t * Nk + kh, th = t * Nv + h;
        float kx[RPL], qx[RPL];
        load_part(k + row * DK + r0, kx);
        load_part(q + row * DK + r0, qx);
        const float b = load_beta(beta, th, beta_f32);
        const float a = g ? __expf(g[th]) : 1.f;
        f32x4 vv = {0.f, 0.f, 0.f, 0.f};
        if (active) {
#pragma unroll
            for (int c = 0; c < 4; ++c) vv[c] = to_f(v[th * DV + j0 + c]);
        }
        float rk = 1.f, rqn = 1.f;
        if (l2norm) {                            // 1 / |x| of the whole vector: sums over the group's rows
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                sk += kx[i] * kx[i];
                sq += qx[i] * qx[i];
            }
            rk = 1.f / sqrtf(group_sum<RQ>(sk) + 1e-6f);
            rqn = 1.f / sqrtf(group_sum<RQ>(sq) + 1e-6f);
        }
        // u = beta (v - exp(g) S_old^T k); S = exp(g) S_old + k u, with k = kx rk
        f32x4 ks = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < RPL; ++i) ks += kx[i] * S[i];
        f32x4 u;
#pragma unroll
        for (int c = 0; c < 4; ++c) u[c] = b * (vv[c] - a * (rk * group_sum<RQ>(ks[c])));
        u = u * rk;
#pragma unroll
        for (int i = 0; i < RPL; ++i) S[i] = S[i] * a + kx[i] * u;
        f32x4 os = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < RPL; ++i) os += qx[i] * S[i];
        // every lane of the group holds the four sums; lane rq stores the
        // columns c with c % RQ == rq
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float x = scale * rqn * group_sum<RQ>(os[c]);
            if (active && c % RQ == rq) {
                if (out_f32) reinterpret_cast<float*>(o)[th * DV + j0 + c] = x;
                else reinterpret_cast<T*>(o)[th * DV + j0 + c] = to_t<T>(x);
            }
        }
    }
    if (ST && active) {
#pragma unroll
        for (int i = 0; i < RPL; ++i)
            __builtin_nontemporal_store(S[i], reinterpret_cast<f32x4*>(&ST[sbase + (int64_t)(r0 + i) * DV + j0]));
    }
}

template <typename T>
hipError_t dispatch(const RecurrentArgs& a) {
    const int cols = 4 * 64 * kRowsPerLane / a.dk;     // state columns per wavefront
    const dim3 grid(a.N, a.Nv);
    const int threads = 64 * ((a.dv + cols - 1) / cols);   // one wavefront per column block (at most 4)
#define GDR_REC(DKv)                                                                                              \
    if (a.dk == DKv) {                                                                                            \
        k_recurrent<T, DKv><<<grid, threads, 0, a.stream>>>((const T*)a.q, (const T*)a.k, (const T*)a.v, a.beta,      \
                                                       a.beta_f32, a.g, a.S0, a.cu_dev, a.T_row, a.Ttot, a.Nk,   \
                                                       a.Nv, a.dv, a.scale, a.l2norm, a.out_f32, a.o, a.ST);      \
        return hipGetLastError();                                                                                 \
    }
    GDR_REC(32) GDR_REC(64) GDR_REC(128)
#undef GDR_REC
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_recurrent(const RecurrentArgs& a) {
    if (a.N == 0) return hipSuccess;
    return a.bf16 ? dispatch<bf16>(a) : dispatch<float>(a);
}

}  // namespace gdr
