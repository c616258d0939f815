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
// Mapping: one wavefront per (sequence, value head, 64 columns of dv). Lane j
// owns column j of the state slice with all dk rows in registers, so neither
// S^T k nor S^T q needs a reduction across lanes. Blocks of 16 tokens of q and
// k (normalised if asked, in fp32) are staged in LDS and read back as
// broadcasts; beta and g are wave-uniform scalar loads. The arithmetic is fp32
// throughout; o is rounded once, at the store.
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {

namespace {

constexpr int kTokBlock = 16;   // tokens of q and k staged per LDS block

template <typename T, int DK>
__global__ __launch_bounds__(64) void k_recurrent(const T* __restrict__ q, const T* __restrict__ k,
                                                   const T* __restrict__ v, const void* __restrict__ beta,
                                                   int beta_f32, const float* __restrict__ g,
                                                   const float* __restrict__ S0, const int32_t* __restrict__ cu,
                                                   int64_t T_row, int64_t Ttot, int32_t Nk, int32_t Nv, int32_t DV,
                                                   float scale, int l2norm, int out_f32, void* __restrict__ o,
                                                   float* __restrict__ ST) {
    static_assert(DK <= 128 && DK % 32 == 0, "dk");
    constexpr int EPL = (DK + 63) / 64;          // q/k elements staged per lane per token
    __shared__ __attribute__((aligned(16))) float kq[2][kTokBlock][DK];

    const int n = blockIdx.x, h = blockIdx.y;
    const int lane = threadIdx.x;
    const int j = blockIdx.z * 64 + lane;        // this lane's state column
    const bool active = j < DV;
    const int kh = h / (Nv / Nk);
    int64_t s = cu ? (int64_t)cu[n] : (int64_t)n * T_row;
    int64_t e = cu ? (int64_t)cu[n + 1] : (int64_t)(n + 1) * T_row;
    s = s < 0 ? 0 : (s > Ttot ? Ttot : s);       // offsets clamped to the token range
    e = e < s ? s : (e > Ttot ? Ttot : e);

    const int64_t sbase = ((int64_t)n * Nv + h) * DK * DV;
    float S[DK];
#pragma unroll
    for (int i = 0; i < DK; ++i) S[i] = (S0 && active) ? S0[sbase + (int64_t)i * DV + j] : 0.f;

    for (int64_t t0 = s; t0 < e; t0 += kTokBlock) {
        const int nt = (int)min((int64_t)kTokBlock, e - t0);
        // stage q and k of tokens t0 .. t0+nt-1 (lane holds elements lane, lane + 64)
        for (int tt = 0; tt < nt; ++tt) {
            const int64_t row = (t0 + tt) * Nk + kh;
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                const T* src = (w == 0 ? k : q) + row * DK;
                float x[EPL];
                float ss = 0.f;
#pragma unroll
                for (int c = 0; c < EPL; ++c) {
                    const int i = lane + 64 * c;
                    x[c] = i < DK ? to_f(src[i]) : 0.f;
                    ss += x[c] * x[c];
                }
                if (l2norm) {
#pragma unroll
                    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
                    const float rn = 1.f / sqrtf(ss + 1e-6f);
#pragma unroll
                    for (int c = 0; c < EPL; ++c) x[c] *= rn;
                }
#pragma unroll
                for (int c = 0; c < EPL; ++c) {
                    const int i = lane + 64 * c;
                    if (i < DK) kq[w][tt][i] = x[c];
                }
            }
        }
        __syncthreads();
        for (int tt = 0; tt < nt; ++tt) {
            const int64_t t = t0 + tt;
            const int64_t th = t * Nv + h;
            const float b = load_beta(beta, th, beta_f32);
            const float a = g ? __expf(g[th]) : 1.f;
            const float vj = active ? to_f(v[th * DV + j]) : 0.f;
            // u = beta (v - exp(g) S_old^T k); S = exp(g) S_old + k u
            float ks0 = 0.f, ks1 = 0.f;
#pragma unroll
            for (int i = 0; i < DK; i += 2) {
                ks0 += kq[0][tt][i] * S[i];
                ks1 += kq[0][tt][i + 1] * S[i + 1];
            }
            const float u = b * (vj - a * (ks0 + ks1));
#pragma unroll
            for (int i = 0; i < DK; ++i) S[i] = S[i] * a + kq[0][tt][i] * u;
            float o0 = 0.f, o1 = 0.f;
#pragma unroll
            for (int i = 0; i < DK; i += 2) {
                o0 += kq[1][tt][i] * S[i];
                o1 += kq[1][tt][i + 1] * S[i + 1];
            }
            const float val = scale * (o0 + o1);
            if (active) {
                if (out_f32) reinterpret_cast<float*>(o)[th * DV + j] = val;
                else reinterpret_cast<T*>(o)[th * DV + j] = to_t<T>(val);
            }
        }
        __syncthreads();                          // the block is consumed before it is overwritten
    }
    if (ST && active) {
#pragma unroll
        for (int i = 0; i < DK; ++i) ST[sbase + (int64_t)i * DV + j] = S[i];
    }
}

template <typename T>
hipError_t dispatch(const RecurrentArgs& a) {
    const dim3 grid(a.N, a.Nv, (a.dv + 63) / 64);
#define GDR_REC(DKv)                                                                                              \
    if (a.dk == DKv) {                                                                                            \
        k_recurrent<T, DKv><<<grid, 64, 0, a.stream>>>((const T*)a.q, (const T*)a.k, (const T*)a.v, a.beta,      \
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
