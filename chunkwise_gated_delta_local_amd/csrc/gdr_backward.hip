// Backward pass of the chunked gated delta rule for gfx950.
//
// Given dO (the loss gradient with respect to o) and dS_T (with respect to the
// final state), computes dq, dk, dv, dbeta, dg and the initial state's
// gradient. The structure follows the chunked backward of the pages (GLA
// notes, backward steps 1-7: recompute the gate sums and the chunk states,
// run the state gradient backwards over the chunks, then form the per-chunk
// gradients of V, of the intra-chunk score block and of Q, K and the gate),
// extended through the delta rule's WY products (ChunkGatedDeltaRule page,
// formulas (1)-(6); FLA DeltaNet article, sections 2.3-2.4).
//
// Per chunk (positions i < L, chunk-local gate sums G, G_last = G_{L-1},
// D_ij = exp(G_i - G_j) for j <= i, P = (Q K^T) (.) D, h = the entering state,
// V_new = U - W h, dS = the gradient with respect to the state leaving the
// chunk):
//   reverse state pass:
//     dV_new = scale P^T dO + diag(exp(G_last - G)) K dS
//     dS_in  = exp(G_last) dS + scale Q^T diag(exp(G)) dO - W^T dV_new
//   per chunk:
//     dQ  = scale diag(exp(G)) dO h^T + dM K,   dP = scale dO V_new^T (j <= i), dM = dP (.) D
//     dW  = -dV_new h^T,  dU = dV_new
//     dV  = diag(beta) A^T dU
//     dA  = dU (diag(beta) V)^T + dW (diag(beta exp(G)) K)^T,  dL = -A^T dA A^T (strictly lower part F)
//     dK  = dM^T Q + diag(exp(G_last - G)) V_new dS^T + diag(beta exp(G)) A^T dW
//           + diag(beta) (F (.) D) K + (F (.) D)^T diag(beta) K
//     dbeta_i = v_i . (A^T dU)_i + exp(G_i) k_i . (A^T dW)_i + sum_j F_ij (k_i . k_j) D_ij
//     dG_i from exp(G) in the inter-chunk output, D in P and L, exp(G_last - G)
//     and exp(G_last) in the state update and exp(G) in W; dg = the reverse
//     prefix sum of dG inside the chunk.
// dq and dk are formed per value head and summed over the heads that share a
// q/k head. All arithmetic is fp32: the products run on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32) with operands staged through LDS, the rest on the
// vector units. The forward values are recomputed by the five-kernel forward
// path.
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

#include <type_traits>

namespace gdr {

namespace {

// offset of element (row r < 16, contraction index m < 32) inside a pair fragment
__device__ __forceinline__ int pair_off(int r, int m) {
    const int mm = m & 15;
    return (16 * (mm >> 2) + r) * 8 + (mm & 3) + (m >= 16 ? 4 : 0);
}

__device__ __forceinline__ float load_any(const void* p, int64_t idx, int is_f32) {
    return is_f32 ? reinterpret_cast<const float*>(p)[idx] : (float)reinterpret_cast<const bf16*>(p)[idx];
}

constexpr int kStageK = 16;                     // K-tile of the staged products

// LDS pitches of a staged operand tile (rows x KT contraction indices). An
// operand read from memory along k is kept row by row with a pitch of 17
// (mod 32) words; one read along its rows is kept k by k with a pitch of 16
// (mod 32) words. Either way the stores of consecutive threads and the
// matrix-core fragment reads (16 rows x 4 k per instruction) spread over the
// LDS banks.
constexpr int stage_kpitch(int KT) { return KT == 16 ? 17 : KT + 17; }
constexpr int stage_rpitch(int R) { return R % 32 == 0 ? R + 16 : R + 32; }
constexpr int stage_floats(int R, int KT) {
    return R * stage_kpitch(KT) > KT * stage_rpitch(R) ? R * stage_kpitch(KT) : KT * stage_rpitch(R);
}

// Operands of a staged product. A global operand (kGlobal) loads raw 32-bit
// words with range-checked buffer loads when a tile is fetched (an element
// outside its matrix reads zero, so no select touches the loaded value) and
// converts and scales them when the tile is committed to LDS: its loads stay
// in flight while the previous tile's products run. Any other operand is a
// function of (row, k) evaluated at commit (values in LDS).
//
// Matrix in global memory: element (row, col) at row * rstride + col
// elements from the base; ES = 2 (bf16) or 4 (fp32) bytes, 0 when the
// element size is the wave-uniform `es` (a tensor whose type is a runtime
// argument: then every load reads the aligned 32-bit word that holds the
// element, and the conversion picks its half). Rows at or past `rows` read as
// zero.
template <int ES>
struct GMat {
    __amdgpu_buffer_rsrc_t rs;
    int rstride;
    int es;
    __device__ __forceinline__ static GMat make(const void* base, int64_t rstride, int rows, int cols, int es_rt = ES) {
        GMat m;
        const uint32_t bytes = rows > 0 ? (uint32_t)(((int64_t)(rows - 1) * rstride + cols) * es_rt) : 0u;
        m.rs = buf_rsrc(base, bytes);
        m.rstride = (int)rstride;
        m.es = es_rt;
        return m;
    }
    __device__ __forceinline__ uint32_t load(int row, int col, bool ok) const {
        if constexpr (ES == 2) {
            const int off = ok ? (row * rstride + col) * 2 : 0x7ffffff0;
            return (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0);
        } else {
            const int off = ok ? ((row * rstride + col) * (ES ? ES : es)) & ~3 : 0x7ffffff0;
            return __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
        }
    }
    __device__ __forceinline__ float conv(uint32_t raw, int row, int col) const {
        if constexpr (ES == 2) return __uint_as_float(raw << 16);
        if constexpr (ES == 4) return __uint_as_float(raw);
        if (es == 4) return __uint_as_float(raw);
        return __uint_as_float(((row * rstride + col) & 1) ? (raw & 0xffff0000u) : (raw << 16));
    }
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    // four elements adjacent in memory from (row, col) (the caller knows they
    // are), one load: their raw words (fp32), or two words of bf16 pairs
    __device__ __forceinline__ u32x4 load4(int row, int col, bool ok) const {
        const int esz = ES ? ES : es;
        const int off = ok ? (row * rstride + col) * esz : 0x7ffffff0;
        if (esz == 4) return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0));
        return u32x4{w[0], w[1], 0u, 0u};
    }
    __device__ __forceinline__ f32x4 conv4(u32x4 raw) const {
        if ((ES ? ES : es) == 4) return __builtin_bit_cast(f32x4, raw);
        return f32x4{__uint_as_float(raw[0] << 16), __uint_as_float(raw[0] & 0xffff0000u),
                     __uint_as_float(raw[1] << 16), __uint_as_float(raw[1] & 0xffff0000u)};
    }
};
template <typename T>
constexpr int es_of() { return (int)sizeof(T); }

// The operands below take the contraction index as k0 + kk, k0 being the
// tile's first index (wave-uniform).
// global operand x(row, k) = fin(row, k, M(row, k)), or M(k, row) when TR
template <bool TR, int ES, typename Fin>
struct GOp {
    static constexpr bool kGlobal = true;
    typedef uint32_t raw_t;
    GMat<ES> m;
    Fin fin;
    __device__ __forceinline__ uint32_t load(int row, int k0, int kk, bool ok) const {
        return TR ? m.load(k0 + kk, row, ok) : m.load(row, k0 + kk, ok);
    }
    __device__ __forceinline__ float value(uint32_t raw, int row, int k0, int kk) const {
        return fin(row, k0 + kk, TR ? m.conv(raw, k0 + kk, row) : m.conv(raw, row, k0 + kk));
    }
    // a group of four: (row, k0 + kk + u) when KC, else (row + u, k0 + kk);
    // one vector load when the four are adjacent in memory (KC != TR)
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    template <bool KC>
    __device__ __forceinline__ u32x4 load4(int row, int k0, int kk, bool ok) const {
        if constexpr (KC != TR) return TR ? m.load4(k0 + kk, row, ok) : m.load4(row, k0 + kk, ok);
        u32x4 r;
#pragma unroll
        for (int u = 0; u < 4; ++u) r[u] = KC ? load(row, k0, kk + u, ok) : load(row + u, k0, kk, ok);
        return r;
    }
    template <bool KC>
    __device__ __forceinline__ f32x4 value4(u32x4 raw, int row, int k0, int kk) const {
        f32x4 v;
        if constexpr (KC != TR) {
            const f32x4 x = m.conv4(raw);
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = KC ? fin(row, k0 + kk + u, x[u]) : fin(row + u, k0 + kk, x[u]);
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = KC ? value(raw[u], row, k0, kk + u) : value(raw[u], row + u, k0, kk);
        }
        return v;
    }
};
struct Ident {
    __device__ __forceinline__ float operator()(int, int, float x) const { return x; }
};
template <bool TR, int ES, typename Fin = Ident>
__device__ __forceinline__ GOp<TR, ES, Fin> gop(const GMat<ES>& m, Fin fin = Fin{}) {
    return GOp<TR, ES, Fin>{m, fin};
}
// two global operands along k: x(row, k) = x0(row, k) for k < kc, else
// x1(row, k - kc); kc is a multiple of the tile depth, so each tile reads one
// of them (a wave-uniform branch with one load on either side)
template <typename X0, typename X1>
struct GCat {
    static constexpr bool kGlobal = true;
    X0 x0;
    X1 x1;
    int kc;
    __device__ __forceinline__ uint32_t load(int row, int k0, int kk, bool ok) const {
        if (k0 < kc) return x0.load(row, k0, kk, ok);
        return x1.load(row, k0 - kc, kk, ok);
    }
    __device__ __forceinline__ float value(uint32_t raw, int row, int k0, int kk) const {
        if (k0 < kc) return x0.value(raw, row, k0, kk);
        return x1.value(raw, row, k0 - kc, kk);
    }
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    template <bool KC>
    __device__ __forceinline__ u32x4 load4(int row, int k0, int kk, bool ok) const {
        if (k0 < kc) return x0.template load4<KC>(row, k0, kk, ok);
        return x1.template load4<KC>(row, k0 - kc, kk, ok);
    }
    template <bool KC>
    __device__ __forceinline__ f32x4 value4(u32x4 raw, int row, int k0, int kk) const {
        if (k0 < kc) return x0.template value4<KC>(raw, row, k0, kk);
        return x1.template value4<KC>(raw, row, k0 - kc, kk);
    }
};
template <typename X0, typename X1>
__device__ __forceinline__ GCat<X0, X1> gcat(const X0& x0, const X1& x1, int kc) {
    return GCat<X0, X1>{x0, x1, kc};
}
// operand evaluated at commit
template <typename F>
struct LOp {
    static constexpr bool kGlobal = false;
    F f;
    __device__ __forceinline__ uint32_t load(int, int, int, bool) const { return 0u; }
    __device__ __forceinline__ float value(uint32_t, int row, int k0, int kk) const { return f(row, k0 + kk); }
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    template <bool KC>
    __device__ __forceinline__ f32x4 value4(u32x4, int row, int k0, int kk) const {
        f32x4 v;
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = KC ? f(row, k0 + kk + u) : f(row + u, k0 + kk);
        return v;
    }
};
template <typename F>
__device__ __forceinline__ LOp<F> lop(F f) { return LOp<F>{f}; }
// One operand of a staged product: R rows by KT contraction indices, element
// x(row, k). KC: consecutive k are adjacent in LDS (else consecutive rows).
// Each thread moves groups of 4 elements.
template <int R, int KT, bool KC>
struct StageOp {
    static constexpr int NG4 = R * KT / 4, NE = (NG4 + 255) / 256;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    static __device__ __forceinline__ int off(int row, int k) {
        return KC ? row * stage_kpitch(KT) + k : k * stage_rpitch(R) + row;
    }
    static __device__ __forceinline__ bool coords(int e, int& row, int& k) {
        const int g4 = 4 * ((int)threadIdx.x + 256 * e);
        row = KC ? g4 / KT : g4 % R;
        k = KC ? g4 % KT : g4 / R;
        return NG4 % 256 == 0 || g4 < 4 * NG4;
    }
    template <typename X>
    static __device__ __forceinline__ void fetch(u32x4 (&r)[NE], const X& x, int k0) {
        if constexpr (X::kGlobal) {
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                int row, k;
                const bool ok = coords(e, row, k);
                r[e] = x.template load4<KC>(row, k0, k, ok);
            }
        }
    }
    template <typename X>
    static __device__ __forceinline__ void commit(float* S, const u32x4 (&r)[NE], const X& x, int k0) {
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            int row, k;
            if (coords(e, row, k)) {
                const f32x4 v = x.template value4<KC>(r[e], row, k0, k);
                if (KC) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) S[off(row, k + u)] = v[u];
                } else {
                    *reinterpret_cast<f32x4*>(&S[off(row, k)]) = v;
                }
            }
        }
    }
};

// Wave layout of a staged product with TM x TN output tiles of 16 x 16 over
// four wavefronts: WM x WN waves, each owning a block of (TM/WM) x (TN/WN)
// tiles, the split with the fewest fragment reads per step (with fewer than
// four tiles, some waves only stage operands).
constexpr int stage_wm(int TM, int TN) {
    if (TM * TN < 4) return TM;
    int best = 0, cost = 1 << 30;
    for (int wm = 1; wm <= 4; wm *= 2) {
        const int wn = 4 / wm;
        if (TM % wm == 0 && TN % wn == 0 && TM / wm + TN / wn < cost) {
            cost = TM / wm + TN / wn;
            best = wm;
        }
    }
    return best;
}

template <int M, int N>
struct StageGrid {
    static constexpr int TM = M / 16, TN = N / 16;
    static constexpr int WM = stage_wm(TM, TN), WN = TM * TN < 4 ? TN : 4 / WM;
    static constexpr int RM = TM / WM, RN = TN / WN;
};

// Staged product: out(i, j) = sum over k < K of a(i, k) b(j, k) for i < M,
// j < N (b is given transposed; M, N multiples of 16; K a multiple of KT, 16
// or 32), on the fp32 matrix cores (v_mfma_f32_16x16x4_f32: products and sums
// in fp32). a and b are operands as above. Tiles of KT contraction indices of
// both go through LDS: the raw words of a global operand's next tile are
// loaded while the current one is multiplied, and converted when it is
// committed; consecutive threads take consecutive addresses of the operand
// (AK: a(i, k) is contiguous in k, else in i; BJ: b(j, k) is contiguous in j,
// else in k). Each wave accumulates its block of 16 x 16 tiles; lane 16 qd + r
// holds rows 4 qd + 0..3 of column r of each tile. As and Bs hold
// stage_floats(M, KT) and stage_floats(N, KT) floats. The product starts with
// a barrier, so its operands may be LDS or memory written by the phase
// before; store(i, j, x) is called once per output element, and for a given
// (M, N) always by the same thread.
// Row sums: when store returns a float (a contribution of element (i, j) to a
// sum over j), the sums of each row are formed in a fixed order (per lane over
// its tiles, then a butterfly over the 16 lanes of a row) and wave column wn
// writes its part to Red[wn * M + i]; the caller adds the StageGrid<M, N>::WN
// parts after a barrier. No atomics: the result is the same on every run.
// no epilogue operand
struct NoEp {
    static constexpr bool kGlobal = false;
    typedef uint32_t raw_t;
};
// two epilogue operands: store receives a float2 (x0(i, j), x1(i, j))
template <typename X0, typename X1>
struct EpPair {
    static constexpr bool kGlobal = true;
    typedef uint32_t raw_t __attribute__((ext_vector_type(2)));
    X0 x0;
    X1 x1;
    __device__ __forceinline__ raw_t load(int i, int k0, int j, bool ok) const {
        return raw_t{x0.load(i, k0, j, ok), x1.load(i, k0, j, ok)};
    }
    __device__ __forceinline__ float2 value(raw_t raw, int i, int k0, int j) const {
        return make_float2(x0.value(raw[0], i, k0, j), x1.value(raw[1], i, k0, j));
    }
};
template <typename X0, typename X1>
__device__ __forceinline__ EpPair<X0, X1> ep_pair(const X0& x0, const X1& x1) {
    return EpPair<X0, X1>{x0, x1};
}
// gemm_lds_e: as gemm_lds, with an epilogue operand ep (a global operand of
// the output's shape): its elements are loaded together once the products are
// issued and passed to store(i, j, x, ep(i, j)).
template <int M, int N, bool AK, bool BJ, int KT, typename FA, typename FB, typename EP, typename FS>
__device__ __forceinline__ void gemm_lds_e(int K, float* As, float* Bs, const FA& a, const FB& b, const EP& ep,
                                           FS&& store, float* Red);
template <int M, int N, bool AK, bool BJ, int KT = kStageK, typename FA, typename FB, typename FS>
__device__ __forceinline__ void gemm_lds(int K, float* As, float* Bs, const FA& a, const FB& b, FS&& store,
                                         float* Red = nullptr) {
    gemm_lds_e<M, N, AK, BJ, KT>(K, As, Bs, a, b, NoEp{}, store, Red);
}
template <int M, int N, bool AK, bool BJ, int KT, typename FA, typename FB, typename EP, typename FS>
__device__ __forceinline__ void gemm_lds_e(int K, float* As, float* Bs, const FA& a, const FB& b, const EP& ep,
                                           FS&& store, float* Red) {
    static_assert(M % 16 == 0 && N % 16 == 0 && KT % 4 == 0, "16 x 16 tiles");
    using OA = StageOp<M, KT, AK>;
    using OB = StageOp<N, KT, !BJ>;
    using SG = StageGrid<M, N>;
    constexpr int WM = SG::WM, WN = SG::WN, RM = SG::RM, RN = SG::RN;
    constexpr bool kEp = !std::is_same<EP, NoEp>::value;
    typedef typename EP::raw_t raw_t;
    auto st = [&](int i, int j, float x, raw_t e) {
        if constexpr (kEp) return store(i, j, x, ep.value(e, i, 0, j));
        else return store(i, j, x);
    };
    constexpr bool kRowSum = !std::is_void<decltype(st(0, 0, 0.f, raw_t{}))>::value;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const bool active = w < WM * WN;
    const int tm0 = (w / WN) * RM, tn0 = (w % WN) * RN;
    const int r = lane & 15, qd = lane >> 4;
    f32x4 acc[RM][RN];
#pragma unroll
    for (int x = 0; x < RM; ++x)
#pragma unroll
        for (int y = 0; y < RN; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
    typename OA::u32x4 ra[OA::NE];
    typename OB::u32x4 rb[OB::NE];
    __syncthreads();                                   // operands written by the previous phase are visible
    OA::fetch(ra, a, 0);
    OB::fetch(rb, b, 0);
    for (int k0 = 0; k0 < K; k0 += KT) {
        lds_barrier();                                 // the previous tile is consumed (LDS only:
        OA::commit(As, ra, a, k0);                     // the prefetched loads stay in flight)
        OB::commit(Bs, rb, b, k0);
        lds_barrier();
        if (k0 + KT < K) {                             // in flight during this tile's products
            OA::fetch(ra, a, k0 + KT);
            OB::fetch(rb, b, k0 + KT);
        }
        if (active) {
#pragma unroll
            for (int k4 = 0; k4 < KT; k4 += 4) {
                float af[RM], bf[RN];
#pragma unroll
                for (int x = 0; x < RM; ++x) af[x] = As[OA::off(16 * (tm0 + x) + r, k4 + qd)];
#pragma unroll
                for (int y = 0; y < RN; ++y) bf[y] = Bs[OB::off(16 * (tn0 + y) + r, k4 + qd)];
#pragma unroll
                for (int x = 0; x < RM; ++x)
#pragma unroll
                    for (int y = 0; y < RN; ++y)
                        acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[x], bf[y], acc[x][y], 0, 0, 0);
            }
        }
    }
    if (active) {
        raw_t ev[RM][4][RN];
#pragma unroll
        for (int x = 0; x < RM; ++x)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                for (int y = 0; y < RN; ++y) {
                    if constexpr (kEp) ev[x][jj][y] = ep.load(16 * (tm0 + x) + 4 * qd + jj, 0, 16 * (tn0 + y) + r, true);
                    else ev[x][jj][y] = raw_t{};
                }
#pragma unroll
        for (int x = 0; x < RM; ++x)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int i = 16 * (tm0 + x) + 4 * qd + jj;
                if constexpr (kRowSum) {
                    float part = 0.f;
#pragma unroll
                    for (int y = 0; y < RN; ++y) part += st(i, 16 * (tn0 + y) + r, acc[x][y][jj], ev[x][jj][y]);
#pragma unroll
                    for (int o = 8; o > 0; o >>= 1) part += __shfl_xor(part, o);
                    if (r == 0) Red[(w % WN) * M + i] = part;
                } else {
#pragma unroll
                    for (int y = 0; y < RN; ++y) st(i, 16 * (tn0 + y) + r, acc[x][y][jj], ev[x][jj][y]);
                }
            }
    }
}

// ------------------------------------------------------------ preparation
// One workgroup per (chunk, value head): the forward intermediates in plain
// row-major layouts (the chunk's entering state transposed, h^T [dv][dk], V_new by token
// row, W^T [dk][C] per chunk), the score block P = (Q K^T) (.) D [C][C] (zero above the
// diagonal and past the chunk end), and the two parts of the reverse state
// pass that do not depend on the state gradient:
//   X  = scale P^T dO                                   (into the dV_new buffer)
//   Y' = Q^T diag(scale exp(G)) dO - W^T X  (into the dS buffer, as Y'^T [dv][dk])
// so that the serial pass only forms Z = diag(exp(G_last - G)) K dS,
// dV_new = X + Z and dS <- exp(G_last) dS + Y' - W^T Z.
// h_done: the entering states are already in Hn (written there as H^T by the
// fp16 chunk pass); otherwise Hn is formed here from the five-kernel path's
// fragments.
template <typename T, int DK, int DV, int C>
__global__ __launch_bounds__(256) void k_bwd_prep(const T* __restrict__ q, const T* __restrict__ k,
                                                   const float* __restrict__ G, const float* __restrict__ Hf,
                                                   const float* __restrict__ VNf, const float* __restrict__ Wf,
                                                   const void* __restrict__ d_o, int do_f32, float scale,
                                                   const int32_t* __restrict__ chunk_start,
                                                   const int32_t* __restrict__ chunk_len, int32_t Nk, int32_t Nv,
                                                   float* __restrict__ Hn, float* __restrict__ Vn,
                                                   float* __restrict__ WT, float* __restrict__ P,
                                                   float* __restrict__ X, float* __restrict__ Yp, int h_done) {
    constexpr int NKP = DK / 32, NNB = DV / 16, NTB = C / 16, NTP = C < 32 ? 1 : C / 32;
    constexpr int NMAX = (DK > DV ? DK : DV) > C ? (DK > DV ? DK : DV) : C;
    constexpr int KT = 32;                       // deeper tiles: this kernel's LDS has room
    __shared__ float Pm[C * C];
    __shared__ __attribute__((aligned(16))) float As[stage_floats(DK > C ? DK : C, KT)];
    __shared__ __attribute__((aligned(16))) float Bs[stage_floats(NMAX, KT)];
    __shared__ float gs[C], se[C];
    const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    const int kh = h / (Nv / Nk);
    const int64_t s = chunk_start[c];
    const int L = chunk_len[c];
    if (L <= 0) return;
    if (tid < C) {
        gs[tid] = tid < L ? G[(s + tid) * Nv + h] : 0.f;
        se[tid] = tid < L ? scale * __expf(gs[tid]) : 0.f;
    }
    const int64_t ch = (int64_t)c * Nv + h;
    // element-wise copies in batches: 16 loads per thread in flight, then their stores
    auto batched = [&](auto n_t, auto&& ld, auto&& st) {
        constexpr int N = decltype(n_t)::value, PER = (N + 255) / 256, B = PER < 16 ? PER : 16;
        static_assert(PER % B == 0, "batch");
#pragma unroll
        for (int b0 = 0; b0 < PER; b0 += B) {
            float x[B];
#pragma unroll
            for (int e = 0; e < B; ++e) {
                const int idx = tid + 256 * (b0 + e);
                x[e] = (N % 256 == 0 || idx < N) ? ld(idx) : 0.f;
            }
#pragma unroll
            for (int e = 0; e < B; ++e) {
                const int idx = tid + 256 * (b0 + e);
                if (N % 256 == 0 || idx < N) st(idx, x[e]);
            }
        }
    };
    if (!h_done)                               // H^T [dv][dk] from the fragments
        batched(std::integral_constant<int, DK * DV>{},
                [&](int idx) { const int j = idx / DK, i = idx % DK;
                               return Hf[((ch * NNB + j / 16) * NKP + i / 32) * 512 + pair_off(j % 16, i % 32)]; },
                [&](int idx, float x) { Hn[ch * DK * DV + idx] = x; });
    batched(std::integral_constant<int, C * DV>{},
            [&](int idx) { const int p = idx / DV, j = idx % DV;
                           return VNf[((ch * NNB + j / 16) * NTP + p / 32) * 512 + pair_off(j % 16, p % 32)]; },
            [&](int idx, float x) { const int p = idx / DV, j = idx % DV;
                                    if (p < L) Vn[((s + p) * Nv + h) * DV + j] = x; });
    batched(std::integral_constant<int, DK * C>{},              // W^T of the chunk, zero past its end
            [&](int idx) { const int i = idx / C, p = idx % C;
                           return Wf[((ch * NTB + p / 16) * NKP + i / 32) * 512 + pair_off(p % 16, i % 32)]; },
            [&](int idx, float x) { const int i = idx / C, p = idx % C; WT[(ch * DK + i) * C + p] = p < L ? x : 0.f; });
    constexpr int EI = es_of<T>();
    const int esd = do_f32 ? 4 : 2;
    const auto Qm = GMat<EI>::make(q + (s * Nk + kh) * DK, (int64_t)Nk * DK, L, DK);
    const auto Km = GMat<EI>::make(k + (s * Nk + kh) * DK, (int64_t)Nk * DK, L, DK);
    const auto dOm = GMat<0>::make(static_cast<const char*>(d_o) + (s * Nv + h) * DV * esd, (int64_t)Nv * DV, L, DV, esd);
    const auto Xm = GMat<4>::make(X + (s * Nv + h) * DV, (int64_t)Nv * DV, L, DV);
    const auto WTm = GMat<4>::make(WT + ch * DK * C, C, DK, C);
    float* Pc = P + ch * C * C;
    // P = (Q K^T) (.) D
    gemm_lds<C, C, true, false, KT>(DK, As, Bs, gop<false>(Qm), gop<false>(Km),
        [&](int i, int j, float x) {
            const float pv = (i < L && j <= i) ? x * __expf(gs[i] - gs[j]) : 0.f;
            Pm[i * C + j] = pv;
            Pc[i * C + j] = pv;
        });
    // X = scale P^T dO
    gemm_lds<C, DV, false, true, (C % 32 == 0 ? KT : 16)>(C, As, Bs, lop([&](int i, int t) { return Pm[t * C + i]; }),
                                 gop<true>(dOm),
                                 [&](int i, int j, float x) { if (i < L) X[((s + i) * Nv + h) * DV + j] = scale * x; });
    // Y' = Q^T diag(scale exp(G)) dO - W^T X (contraction over [Q rows | W^T columns])
    // (tiles of 16 when C = 16: a tile must not straddle the two parts)
    gemm_lds<DK, DV, false, true, (C % 32 == 0 ? KT : 16)>(2 * C, As, Bs,
        gcat(gop<true>(Qm), gop<false>(WTm, [](int, int, float x) { return -x; }), C),
        gcat(gop<true>(dOm, [&](int, int t, float x) { return se[t] * x; }), gop<true>(Xm), C),
        [&](int m, int j, float x) { Yp[(ch * DV + j) * DK + m] = x; });
}

// ------------------------------------------------------------ reverse state pass
// One workgroup of four wavefronts per (sequence, value head, 16 columns of
// dv) walks the chunks backwards with the 16-column slice of the state
// gradient dS in fp32 accumulators. Per chunk, with X and Y' from the
// preparation kernel:
//   Z = diag(exp(G_last - G)) K dS;  dV_new = X + Z   (overwrites X)
//   the chunk's outgoing-state gradient dS is stored (over Y', after reading it)
//   dS <- exp(G_last) dS + Y' - W^T Z
// Wavefront w forms rows 16 w .. 16 w + 15 of Z (contraction over dk) and
// the dk row blocks w, w + 4, ... of W^T Z (contraction over the chunk's
// positions); K, W^T, Z^T and dS^T go through LDS. For bf16 inputs (C a
// multiple of 32) both products run on v_mfma_f32_16x16x32_bf16 with K as it
// is and dS, W^T and Z split into hi + lo bf16 (three or two products per
// tile; about 16 bits of each value kept, so the result matches the fp32
// products to about 1e-5, and scaling the inputs by 2 scales every gradient
// by exactly 2), lane (qd, r) holding the contraction indices 32 t + 8 qd ..
// + 7 (one 16-byte read per operand). For fp32 inputs they run on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32) with fp32 tiles, lane (qd, r) taking the
// contraction indices 16 t + 4 qd + u, u = 0..3, in each group of four
// products. The next chunk's K rows, W^T, X, Y' and gate sums are loaded into
// registers while the current chunk is computed.
template <typename T, int DK, int DV, int C>
__global__ __launch_bounds__(256) void k_bwd_state(const T* __restrict__ k, const float* __restrict__ G,
                                                    const float* __restrict__ WT, const float* __restrict__ dST,
                                                    const int32_t* __restrict__ chunk_start,
                                                    const int32_t* __restrict__ chunk_len,
                                                    const int32_t* __restrict__ seq_first, int32_t Nk, int32_t Nv,
                                                    float* __restrict__ dSY, float* __restrict__ dVX,
                                                    float* __restrict__ dS0) {
    typedef typename Vec<T>::v8 v8;
    constexpr int NB = DK / 16;                 // dk row blocks of dS
    constexpr int NBW = (NB + 3) / 4;           // row blocks per wavefront
    constexpr int KP = DK + 4, CP = C + 4;      // LDS pitches (floats)
    constexpr int NSEG = C * DK / 8;            // 8-element pieces of the K rows
    constexpr int NK8 = (NSEG + 255) / 256;
    constexpr int NW4 = DK * C / 4;             // 4-float pieces of W^T
    constexpr int NWT = (NW4 + 255) / 256;
    // bf16 inputs (C a multiple of 32): bf16 tiles on v_mfma_f32_16x16x32_bf16,
    // K as it is (exact) and dS, W^T and Z as hi + lo bf16 pairs (products
    // K dS_hi + K dS_lo and W_hi Z_hi + W_hi Z_lo + W_lo Z_hi, fp32 sums);
    // fp32 inputs: fp32 tiles on v_mfma_f32_16x16x4_f32
    constexpr bool kHalf = sizeof(T) == 2 && C % 32 == 0;
    constexpr int KPH = DK + 8, CPH = C + 8;    // bf16 pitches (elements)
    typedef Vec<bf16>::v8 b8;
    typedef Vec<bf16>::v4 b4;
    __shared__ __attribute__((aligned(16))) float Ks[kHalf ? 1 : C][KP];
    __shared__ __attribute__((aligned(16))) float Wt[kHalf ? 1 : DK][CP];
    __shared__ __attribute__((aligned(16))) float dSt[kHalf ? 1 : 16][KP];
    __shared__ __attribute__((aligned(16))) float Zt[kHalf ? 1 : 16][CP];
    __shared__ __attribute__((aligned(16))) bf16 Kb[kHalf ? C : 1][KPH];
    __shared__ __attribute__((aligned(16))) bf16 Wb[kHalf ? 2 : 1][kHalf ? DK : 1][CPH];     // hi, lo
    __shared__ __attribute__((aligned(16))) bf16 dSb[kHalf ? 2 : 1][kHalf ? 16 : 1][KPH];
    __shared__ __attribute__((aligned(16))) bf16 Zb[kHalf ? 2 : 1][kHalf ? 16 : 1][CPH];
    // four fp32 values -> hi and lo bf16 (x = hi + lo to about 16 bits)
    auto put_split4 = [](bf16* hi, bf16* lo, const f32x4& x) {
        b4 h, l;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            h[j] = (bf16)x[j];
            l[j] = (bf16)(x[j] - (float)h[j]);
        }
        *reinterpret_cast<b4*>(hi) = h;
        *reinterpret_cast<b4*>(lo) = l;
    };
    __shared__ float gs[256];                   // gate sums (one per thread; C used)
    const int n = blockIdx.x, h = blockIdx.y, nb = blockIdx.z, tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, r = lane & 15, qd = lane >> 4;
    const int kh = h / (Nv / Nk);
    const int64_t hb = (int64_t)n * Nv + h;
    // dS rows 16 m + 4 qd + v, column r, for the blocks m = w + 4 i
    f32x4 dS[NBW];
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
        const int m = w + 4 * i;
#pragma unroll
        for (int v = 0; v < 4; ++v)
            dS[i][v] = (m < NB && dST) ? dST[(hb * DK + 16 * m + 4 * qd + v) * DV + nb * 16 + r] : 0.f;
    }
    // K rows and W^T of a chunk, loaded two chunks ahead into one of two
    // register sets; X, Y' and the gate sums one chunk ahead
    v8 kr[2][NK8];
    f32x4 wr[2][NWT], xr, yr[NBW];
    float gr = 0.f;
    auto fetch_tiles = [&](int c, auto set_t) {
        constexpr int SET = decltype(set_t)::value;
        const int64_t s = chunk_start[c];
        const int L = chunk_len[c];
        // rows past the chunk's end fall outside the buffer and read as zero
        const auto rk = buf_rsrc(k + (s * Nk + kh) * DK, L > 0 ? (uint32_t)(((L - 1) * Nk + 1) * DK * sizeof(T)) : 0u);
#pragma unroll
        for (int e = 0; e < NK8; ++e) {
            const int idx = tid + 256 * e, i = idx / (DK / 8), seg = idx % (DK / 8);
            const int off = idx < NSEG ? (int)((i * Nk * DK + seg * 8) * sizeof(T)) : 0x7fffffff;
            if constexpr (sizeof(T) == 2) {
                kr[SET][e] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
            } else {
                const f32x4 lo = buf_ld_f32x4(rk, off), hi = buf_ld_f32x4(rk, off + 16);
                kr[SET][e] = __builtin_bit_cast(v8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        }
        const auto rw = buf_rsrc(WT + ((int64_t)c * Nv + h) * DK * C, DK * C * 4);
#pragma unroll
        for (int e = 0; e < NWT; ++e) wr[SET][e] = buf_ld_f32x4(rw, 16 * (tid + 256 * e));
    };
    auto fetch_small = [&](int c) {
        const int64_t s = chunk_start[c];
        const int L = chunk_len[c];
        const auto rx = buf_rsrc(dVX + (s * Nv + h) * DV + nb * 16, L > 0 ? (uint32_t)(((L - 1) * Nv * DV + 16) * 4) : 0u);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = 16 * w + 4 * qd + v;    // rows past the end (or past C) read as zero
            xr[v] = buf_ld_f32(rx, (i * Nv * DV + r) * 4);
        }
        // Y' (and later dS) of the chunk as dS^T [dv][dk]: rows 16 m + 4 qd .. + 3 of
        // column 16 nb + r are 16 contiguous bytes
        const auto ry = buf_rsrc(dSY + (((int64_t)c * Nv + h) * DV + nb * 16) * DK, 16 * DK * 4);
#pragma unroll
        for (int i = 0; i < NBW; ++i) {
            const int m = w + 4 * i;
            yr[i] = buf_ld_f32x4(ry, m < NB ? (r * DK + 16 * m + 4 * qd) * 4 : 0x7ffffff0);
        }
        const auto rg = buf_rsrc(G + s * Nv + h, L > 0 ? (uint32_t)(((L - 1) * Nv + 1) * 4) : 0u);
        gr = buf_ld_f32(rg, tid * Nv * 4);
    };
    auto put_dS = [&]() {                          // dS^T -> LDS
#pragma unroll
        for (int i = 0; i < NBW; ++i) {
            const int m = w + 4 * i;
            if (m < NB) {
                if constexpr (kHalf)
                    put_split4(&dSb[0][r][16 * m + 4 * qd], &dSb[1][r][16 * m + 4 * qd], dS[i]);
                else
                    *reinterpret_cast<f32x4*>(&dSt[r][16 * m + 4 * qd]) = dS[i];
            }
        }
    };
    typedef std::integral_constant<int, 0> S0_t;
    typedef std::integral_constant<int, 1> S1_t;
    put_dS();
    const int c0 = seq_first[n], c1 = seq_first[n + 1];
    if (c1 <= c0) {
        if (dS0) {                                  // no chunks: the gradient passes through
#pragma unroll
            for (int i = 0; i < NBW; ++i) {
                const int m = w + 4 * i;
                if (m < NB) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) dS0[(hb * DK + 16 * m + 4 * qd + v) * DV + nb * 16 + r] = dS[i][v];
                }
            }
        }
        return;
    }
    // every step issues its loads unconditionally (chunks before the first
    // re-read chunk c0, unused), so that the compiler's waits count the same
    // loads on every path
    fetch_small(c1 - 1);
    fetch_tiles(c1 - 1, S0_t{});
    fetch_tiles(max(c1 - 2, c0), S1_t{});
    auto step = [&](int c, auto set_t) {
        constexpr int SET = decltype(set_t)::value;
        const int64_t s = chunk_start[c];
        const int L = chunk_len[c];
        lds_barrier();                                // the previous chunk's reads are done
#pragma unroll
        for (int e = 0; e < NK8; ++e) {               // K rows and W^T -> LDS
            const int idx = tid + 256 * e, i = idx / (DK / 8), seg = idx % (DK / 8);
            if (NSEG % 256 == 0 || idx < NSEG) {
                if constexpr (kHalf) {
                    *reinterpret_cast<b8*>(&Kb[i][seg * 8]) = __builtin_bit_cast(b8, kr[SET][e]);
                } else {
                    f32x4 a, b;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        a[t] = to_f(kr[SET][e][t]);
                        b[t] = to_f(kr[SET][e][4 + t]);
                    }
                    *reinterpret_cast<f32x4*>(&Ks[i][seg * 8]) = a;
                    *reinterpret_cast<f32x4*>(&Ks[i][seg * 8 + 4]) = b;
                }
            }
        }
#pragma unroll
        for (int e = 0; e < NWT; ++e) {
            const int idx = tid + 256 * e;
            if (NW4 % 256 == 0 || idx < NW4) {
                const f32x4 x4 = wr[SET][e];
                if constexpr (kHalf)
                    put_split4(&Wb[0][idx / (C / 4)][4 * (idx % (C / 4))], &Wb[1][idx / (C / 4)][4 * (idx % (C / 4))], x4);
                else
                    *reinterpret_cast<f32x4*>(&Wt[idx / (C / 4)][4 * (idx % (C / 4))]) = x4;
            }
        }
        gs[tid] = gr;
        const f32x4 x = xr;
        f32x4 y[NBW];
#pragma unroll
        for (int i = 0; i < NBW; ++i) y[i] = yr[i];
        lds_barrier();
        // the small loads first: they are waited for at the next step's start,
        // and loads complete in issue order
        fetch_small(max(c - 1, c0));
        fetch_tiles(max(c - 2, c0), set_t);          // in flight during this chunk and the next
        const float gL = gs[L - 1];
        // Z rows 16 w + 4 qd + v, column r; dV_new = X + Z
        if (16 * w < C) {
            f32x4 z;
            if constexpr (kHalf) {                    // lane (qd, r): contraction indices 32 t + 8 qd .. + 7
                f32x4 zu[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};   // K dS_hi, K dS_lo
#pragma unroll
                for (int t = 0; t < DK / 32; ++t) {
                    const b8 a = *reinterpret_cast<const b8*>(&Kb[16 * w + r][32 * t + 8 * qd]);
                    const b8 bh = *reinterpret_cast<const b8*>(&dSb[0][r][32 * t + 8 * qd]);
                    const b8 bl = *reinterpret_cast<const b8*>(&dSb[1][r][32 * t + 8 * qd]);
                    zu[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, zu[0], 0, 0, 0);
                    zu[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, zu[1], 0, 0, 0);
                }
                z = zu[0] + zu[1];
            } else {
                f32x4 zu[4];                          // four independent sums (u), added at the end
#pragma unroll
                for (int u = 0; u < 4; ++u) zu[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < DK / 16; ++t) {
                    const f32x4 a = *reinterpret_cast<const f32x4*>(&Ks[16 * w + r][16 * t + 4 * qd]);
                    const f32x4 b = *reinterpret_cast<const f32x4*>(&dSt[r][16 * t + 4 * qd]);
#pragma unroll
                    for (int u = 0; u < 4; ++u) zu[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u], b[u], zu[u], 0, 0, 0);
                }
                z = (zu[0] + zu[1]) + (zu[2] + zu[3]);
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int i = 16 * w + 4 * qd + v;
                z[v] = i < L ? __expf(gL - gs[i]) * z[v] : 0.f;
                if (i < L) dVX[((s + i) * Nv + h) * DV + nb * 16 + r] = x[v] + z[v];
            }
            if constexpr (kHalf)
                put_split4(&Zb[0][r][16 * w + 4 * qd], &Zb[1][r][16 * w + 4 * qd], z);
            else
                *reinterpret_cast<f32x4*>(&Zt[r][16 * w + 4 * qd]) = z;
        }
        lds_barrier();
        // the outgoing-state gradient of this chunk, then dS <- exp(G_last) dS + Y' - W^T Z
        const float eL = __expf(gL);
#pragma unroll
        for (int i = 0; i < NBW; ++i) {
            const int m = w + 4 * i;
            if (m < NB) {
                f32x4 au[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};   // two independent sums
                if constexpr (kHalf) {
#pragma unroll
                    for (int t = 0; t < C / 32; ++t) {
                        const b8 ah = *reinterpret_cast<const b8*>(&Wb[0][16 * m + r][32 * t + 8 * qd]);
                        const b8 al = *reinterpret_cast<const b8*>(&Wb[1][16 * m + r][32 * t + 8 * qd]);
                        const b8 bh = *reinterpret_cast<const b8*>(&Zb[0][r][32 * t + 8 * qd]);
                        const b8 bl = *reinterpret_cast<const b8*>(&Zb[1][r][32 * t + 8 * qd]);
                        au[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, au[0], 0, 0, 0);
                        au[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, au[1], 0, 0, 0);
                        au[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, au[1], 0, 0, 0);
                    }
                } else {
#pragma unroll
                    for (int t = 0; t < C / 16; ++t) {
                        const f32x4 a = *reinterpret_cast<const f32x4*>(&Wt[16 * m + r][16 * t + 4 * qd]);
                        const f32x4 b = *reinterpret_cast<const f32x4*>(&Zt[r][16 * t + 4 * qd]);
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            au[u & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u], b[u], au[u & 1], 0, 0, 0);
                    }
                }
                const f32x4 acc = au[0] + au[1];
                *reinterpret_cast<f32x4*>(&dSY[(((int64_t)c * Nv + h) * DV + nb * 16 + r) * DK + 16 * m + 4 * qd]) = dS[i];
                dS[i] = eL * dS[i] + y[i] - acc;
            }
        }
        put_dS();
    };
    int c = c1 - 1;
    for (; c - 1 >= c0; c -= 2) {
        step(c, S0_t{});
        step(c - 1, S1_t{});
    }
    if (c >= c0) step(c, S0_t{});
    if (dS0) {
#pragma unroll
        for (int i = 0; i < NBW; ++i) {
            const int m = w + 4 * i;
            if (m < NB) {
#pragma unroll
                for (int v = 0; v < 4; ++v) dS0[(hb * DK + 16 * m + 4 * qd + v) * DV + nb * 16 + r] = dS[i][v];
            }
        }
    }
}

// ------------------------------------------------------------ per-chunk gradients
// One workgroup per (chunk, value head). Four C x C matrices sit in LDS (A;
// dM = dP (.) D; dA, then F, then F (.) D; A^T dA, then K K^T) with the
// staging tiles of the products, about 79 KB for C = 64, so that two
// workgroups share a compute unit; D is recomputed from the gate sums where
// it is needed. Writes dq and dk of this value head (summed over the group
// later), dv, dbeta and dg, and uses a per-token scratch for dW.
template <typename T, int DK, int DV, int C>
__global__ __launch_bounds__(256, 2) void k_bwd_chunk(const T* __restrict__ q, const T* __restrict__ k,
                                                    const T* __restrict__ v, const void* __restrict__ beta,
                                                    int beta_f32, const float* __restrict__ G,
                                                    const float* __restrict__ A, const float* __restrict__ P,
                                                    const float* __restrict__ Hn, const float* __restrict__ Vn,
                                                    const float* __restrict__ dSout, const float* __restrict__ dVn,
                                                    const void* __restrict__ d_o, int do_f32,
                                                    const int32_t* __restrict__ chunk_start,
                                                    const int32_t* __restrict__ chunk_len, int32_t Nk, int32_t Nv,
                                                    float scale, float* __restrict__ dW, float* __restrict__ dqv,
                                                    float* __restrict__ dkv, float* __restrict__ dv,
                                                    float* __restrict__ dbeta, float* __restrict__ dg) {
    constexpr int NMAX = (DK > DV ? DK : DV) > C ? (DK > DV ? DK : DV) : C;
    __shared__ float Am[C * C], dMm[C * C], dAm[C * C], Xm[C * C];
    __shared__ __attribute__((aligned(16))) float As[stage_floats(C, kStageK)];
    __shared__ __attribute__((aligned(16))) float Bs[stage_floats(NMAX, kStageK)];
    __shared__ float gs[C], eg[C], elg[C], bs[C], dGs[C], dBs[C], cv[C];
    __shared__ float wsum[4];
    const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    const int kh = h / (Nv / Nk);
    const int64_t s = chunk_start[c];
    const int L = chunk_len[c];
    if (L <= 0) return;
    const int64_t ch = (int64_t)c * Nv + h;
    const float* Hc = Hn + ch * DK * DV;          // entering state, transposed: [dv][dk]
    const float* dSc = dSout + ch * DK * DV;      // gradient of the outgoing state, transposed: [dv][dk]
    const float* Pc = P + ch * C * C;

    auto row_dk = [&](int i) { return ((s + i) * Nv + h) * DK; };
    auto Dv = [&](int i, int j) { return (i < L && j <= i) ? __expf(gs[i] - gs[j]) : 0.f; };
    // the same matrices as operands of the staged products (rows past the chunk end read zero)
    constexpr int EI = es_of<T>();
    const int esd = do_f32 ? 4 : 2;
    const auto Qm = GMat<EI>::make(q + (s * Nk + kh) * DK, (int64_t)Nk * DK, L, DK);
    const auto Km = GMat<EI>::make(k + (s * Nk + kh) * DK, (int64_t)Nk * DK, L, DK);
    const auto Vm = GMat<EI>::make(v + (s * Nv + h) * DV, (int64_t)Nv * DV, L, DV);
    const auto dOm = GMat<0>::make(static_cast<const char*>(d_o) + (s * Nv + h) * DV * esd, (int64_t)Nv * DV, L, DV, esd);
    const auto Vnm = GMat<4>::make(Vn + (s * Nv + h) * DV, (int64_t)Nv * DV, L, DV);
    const auto dVnm = GMat<4>::make(dVn + (s * Nv + h) * DV, (int64_t)Nv * DV, L, DV);
    const auto dWm = GMat<4>::make(dW + (s * Nv + h) * DK, (int64_t)Nv * DK, L, DK);
    const auto Hm = GMat<4>::make(Hc, DK, DV, DK);      // Hm(j, m) = h[m][j]
    const auto dSm = GMat<4>::make(dSc, DK, DV, DK);
    const auto dqvm = GMat<4>::make(dqv + (s * Nv + h) * DK, (int64_t)Nv * DK, L, DK);
    const auto dkvm = GMat<4>::make(dkv + (s * Nv + h) * DK, (int64_t)Nv * DK, L, DK);

    if (tid < C) {
        const bool ok = tid < L;
        gs[tid] = ok ? G[(s + tid) * Nv + h] : 0.f;
        bs[tid] = ok ? load_beta(beta, (s + tid) * Nv + h, beta_f32) : 0.f;
        dGs[tid] = 0.f;
        dBs[tid] = 0.f;
    }
    {   // A of the chunk: all loads first (rows past the end read zero), then the mask
        constexpr int NA = (C * C + 255) / 256;
        const auto rA = buf_rsrc(A + (s * Nv + h) * C, (uint32_t)(((L - 1) * Nv + 1) * C * 4));
        float av[NA];
#pragma unroll
        for (int e = 0; e < NA; ++e) {
            const int idx = tid + 256 * e;
            av[e] = buf_ld_f32(rA, idx < C * C ? ((idx / C) * Nv * C + idx % C) * 4 : 0x7ffffff0);
        }
#pragma unroll
        for (int e = 0; e < NA; ++e) {
            const int idx = tid + 256 * e, i = idx / C, j = idx % C;
            if (idx < C * C) Am[idx] = j <= i ? av[e] : 0.f;
        }
    }
    __syncthreads();
    const float gL = gs[L - 1];
    if (tid < C) {
        eg[tid] = tid < L ? __expf(gs[tid]) : 0.f;
        elg[tid] = tid < L ? __expf(gL - gs[tid]) : 0.f;
    }

    // dP = scale dO V_new^T on and below the diagonal; dM = dP (.) D, and the gate
    // gradient through D in P: E = dP (.) P (kept in Xm) adds its row sums to dG
    // and subtracts its column sums
    gemm_lds_e<C, C, true, false, kStageK>(DV, As, Bs, gop<false>(dOm), gop<false>(Vnm),
        gop<false>(GMat<4>::make(Pc, C, C, C)),
        [&](int i, int j, float x, float p) {
            const float dp = (i < L && j <= i) ? scale * x : 0.f;
            dMm[i * C + j] = dp * Dv(i, j);
            Xm[i * C + j] = dp * p;
        }, nullptr);
    // dQ = scale diag(exp(G)) dO h^T + dM K (the same thread owns each element in both products)
    gemm_lds<C, DK, true, true>(DV, As, Bs, gop<false>(dOm, [&](int i, int, float x) { return scale * eg[i] * x; }),
                                gop<true>(Hm),
                                 [&](int i, int m, float x) { if (i < L) dqv[row_dk(i) + m] = x; });
    {   // row and column sums of E, 256 / C threads per position, in a fixed order
        constexpr int TPR = 256 / C;
        const int i = tid / TPR, part = tid % TPR;
        float rs = 0.f, cs = 0.f;
        for (int j = part; j < C; j += TPR) {
            rs += Xm[i * C + j];
            cs += Xm[j * C + i];
        }
#pragma unroll
        for (int o = TPR / 2; o > 0; o >>= 1) {
            rs += __shfl_xor(rs, o);
            cs += __shfl_xor(cs, o);
        }
        if (part == 0) dGs[i] += rs - cs;
    }
    gemm_lds_e<C, DK, true, true, kStageK>(C, As, Bs, lop([&](int i, int kk) { return dMm[i * C + kk]; }), gop<true>(Km),
                                           gop<false>(dqvm),
                                           [&](int i, int m, float x, float old) { if (i < L) dqv[row_dk(i) + m] = old + x; },
                                           nullptr);
    // dW = -dV_new h^T
    gemm_lds<C, DK, true, true>(DV, As, Bs, gop<false>(dVnm), gop<true>(Hm),
                                 [&](int i, int m, float x) { if (i < L) dW[row_dk(i) + m] = -x; });
    // dV = diag(beta) A^T dU (dU = dV_new); dbeta += v . (A^T dU)  (row sums in dAm, free until dA)
    float* const red1 = dAm;
    float* const red2 = dAm + 4 * C;
    gemm_lds_e<C, DV, false, true, kStageK>(C, As, Bs, lop([&](int i, int kk) { return Am[kk * C + i]; }), gop<true>(dVnm),
        gop<false>(Vm),
        [&](int i, int j, float x, float vij) {
            if (i >= L) return 0.f;
            dv[((s + i) * Nv + h) * DV + j] = bs[i] * x;
            return vij * x;
        }, red1);
    // A^T dW: dK = diag(beta exp(G)) A^T dW; dbeta, dG through exp(G) in W
    gemm_lds_e<C, DK, false, true, kStageK>(C, As, Bs, lop([&](int i, int kk) { return Am[kk * C + i]; }), gop<true>(dWm),
        gop<false>(Km),
        [&](int i, int m, float x, float kim) {
            if (i >= L) return 0.f;
            dkv[row_dk(i) + m] = bs[i] * eg[i] * x;
            return kim * x * eg[i];
        }, red2);
    __syncthreads();
    if (tid < C) {
        float r1 = 0.f, r2 = 0.f;
#pragma unroll
        for (int wn = 0; wn < StageGrid<C, DV>::WN; ++wn) r1 += red1[wn * C + tid];
#pragma unroll
        for (int wn = 0; wn < StageGrid<C, DK>::WN; ++wn) r2 += red2[wn * C + tid];
        dBs[tid] += r1 + r2;
        dGs[tid] += bs[tid] * r2;
    }
    // dA = dU (diag(beta) V)^T + dW (diag(beta exp(G)) K)^T
    gemm_lds<C, C, true, false>(DV, As, Bs, gop<false>(dVnm), gop<false>(Vm, [&](int j, int, float x) { return bs[j] * x; }),
                                [&](int i, int j, float x) { dAm[i * C + j] = x; });
    gemm_lds<C, C, true, false>(DK, As, Bs, gop<false>(dWm),
                                gop<false>(Km, [&](int j, int, float x) { return bs[j] * eg[j] * x; }),
                                [&](int i, int j, float x) { dAm[i * C + j] += x; });
    // A^T dA, then F = strictly lower part of dL = -(A^T dA) A^T
    gemm_lds<C, C, false, true>(C, As, Bs, lop([&](int i, int kk) { return Am[kk * C + i]; }),
                                lop([&](int j, int kk) { return dAm[kk * C + j]; }),
                                [&](int i, int j, float x) { Xm[i * C + j] = x; });
    gemm_lds<C, C, true, false>(C, As, Bs, lop([&](int i, int kk) { return Xm[i * C + kk]; }),
                                lop([&](int j, int kk) { return Am[j * C + kk]; }),
                                [&](int i, int j, float x) { dAm[i * C + j] = (i < L && j < i) ? -x : 0.f; });
    // K K^T
    gemm_lds<C, C, true, false>(DK, As, Bs, gop<false>(Km), gop<false>(Km),
                                [&](int i, int j, float x) { Xm[i * C + j] = x; });
    __syncthreads();
    // dbeta and dG through L_ij = beta_i (k_i . k_j) D_ij
    if (tid < C) {
        float db = 0.f, dgr = 0.f;
        for (int j = 0; j < C; ++j) {
            const float fd = dAm[tid * C + j] * Xm[tid * C + j] * Dv(tid, j);
            db += fd;
            dgr += fd * bs[tid] - dAm[j * C + tid] * bs[j] * Xm[j * C + tid] * Dv(j, tid);
        }
        dBs[tid] += db;
        dGs[tid] += dgr;
    }
    __syncthreads();
    for (int idx = tid; idx < C * C; idx += 256) dAm[idx] *= Dv(idx / C, idx % C);   // F (.) D
    // dK += diag(beta) (F (.) D) K + (F (.) D)^T diag(beta) K + dM^T Q
    gemm_lds_e<C, DK, false, true, kStageK>(3 * C, As, Bs,
        lop([&](int i, int kk) {
            return kk < C ? bs[i] * dAm[i * C + kk]
                          : (kk < 2 * C ? bs[kk - C] * dAm[(kk - C) * C + i] : dMm[(kk - 2 * C) * C + i]);
        }),
        gcat(gop<true>(Km), gcat(gop<true>(Km), gop<true>(Qm), C), C), gop<false>(dkvm),
        [&](int i, int m, float x, float old) { if (i < L) dkv[row_dk(i) + m] = old + x; }, nullptr);
    // dK += diag(exp(G_last - G)) V_new dS^T; the same term's gate gradient (row sums
    // in Xm, free after the dK product above)
    float* const red3 = Xm;
    float* const red4 = Xm + 4 * C;
    gemm_lds_e<C, DK, true, true, kStageK>(DV, As, Bs, gop<false>(Vnm), gop<true>(dSm), ep_pair(gop<false>(dkvm), gop<false>(Km)),
        [&](int i, int m, float x, float2 e) {
            if (i >= L) return 0.f;
            const float y = elg[i] * x;
            dkv[row_dk(i) + m] = e.x + y;
            return e.y * y;
        }, red3);
    // dG through exp(G) in the inter-chunk output: dG_i += dO_i . (scale exp(G_i) h^T q_i)
    gemm_lds_e<C, DV, true, false, kStageK>(DK, As, Bs, gop<false>(Qm), gop<false>(Hm), gop<false>(dOm),
        [&](int i, int j, float x, float d) { return i < L ? scale * eg[i] * d * x : 0.f; }, red4);
    // exp(G_last) h in the state update: sum(dS (.) h), per wave then over the waves
    {
        float part = 0.f;
        constexpr int N4 = DK * DV / 4 / 256, NBATCH = N4 < 8 ? N4 : 8;   // 16-byte pieces per thread
        static_assert(N4 % NBATCH == 0, "dk dv");
#pragma unroll
        for (int b0 = 0; b0 < N4; b0 += NBATCH) {      // a batch of loads, then their products
            f32x4 xs[NBATCH], xh[NBATCH];
#pragma unroll
            for (int e = 0; e < NBATCH; ++e) {
                xs[e] = *reinterpret_cast<const f32x4*>(dSc + 4 * (tid + 256 * (b0 + e)));
                xh[e] = *reinterpret_cast<const f32x4*>(Hc + 4 * (tid + 256 * (b0 + e)));
            }
#pragma unroll
            for (int e = 0; e < NBATCH; ++e) part += (xs[e][0] * xh[e][0] + xs[e][1] * xh[e][1]) + (xs[e][2] * xh[e][2] + xs[e][3] * xh[e][3]);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
        if ((tid & 63) == 0) wsum[tid >> 6] = part;
    }
    __syncthreads();
    if (tid < C) {
        float c3 = 0.f, r4 = 0.f;
#pragma unroll
        for (int wn = 0; wn < StageGrid<C, DK>::WN; ++wn) c3 += red3[wn * C + tid];
#pragma unroll
        for (int wn = 0; wn < StageGrid<C, DV>::WN; ++wn) r4 += red4[wn * C + tid];
        cv[tid] = c3;
        dGs[tid] += r4 - c3;
    }
    __syncthreads();
    if (tid == 0) {
        float tot = 0.f;
        for (int i = 0; i < L; ++i) tot += cv[i];
        const float sum_sh = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
        dGs[L - 1] += tot + __expf(gL) * sum_sh;
        float acc = 0.f;                             // dg = reverse prefix sum of dG in the chunk
        for (int i = L - 1; i >= 0; --i) {
            acc += dGs[i];
            if (dg) dg[(s + i) * Nv + h] = acc;
        }
    }
    if (tid < L) dbeta[(s + tid) * Nv + h] = dBs[tid];
}

// dq and dk of each q/k head: the sum over the value heads that share it.
template <int DK>
__global__ __launch_bounds__(256) void k_bwd_reduce_qk(const float* __restrict__ dqv, const float* __restrict__ dkv,
                                                        int64_t Ttot, int32_t Nk, int32_t Nv,
                                                        float* __restrict__ dq, float* __restrict__ dk) {
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (p >= Ttot * Nk * DK) return;
    const int64_t t = p / ((int64_t)Nk * DK);
    const int kh = (int)((p / DK) % Nk), m = (int)(p % DK);
    const int group = Nv / Nk;
    float aq = 0.f, ak = 0.f;
    for (int hh = 0; hh < group; ++hh) {
        const int64_t src = (t * Nv + kh * group + hh) * DK + m;
        aq += dqv[src];
        ak += dkv[src];
    }
    dq[p] = aq;
    dk[p] = ak;
}

template <typename T, int DK, int DV, int C>
hipError_t launch_bwd(const BackwardArgs& b) {
    const LaunchArgs& a = b.fwd;
    hipStream_t st = a.stream;
    auto mark = [&](int i) { if (b.events && b.events[i]) (void)hipEventRecord(b.events[i], st); };
    mark(0);
    LaunchArgs f = a;
    if (!f.states16) f.T16 = nullptr;            // the fp16 path's T, score block and decay rows are not needed
    else f.H = b.Hn;                             // the fp16 chunk pass writes the states as H^T directly
    hipError_t e = launch_forward(f, nullptr);   // recompute: G, A, W, U, K^T, h, V_new
    if (e != hipSuccess) return e;
    mark(1);
    const int32_t NT = a.nt;
    if (NT > 0) {
        k_bwd_prep<T, DK, DV, C><<<dim3(NT, a.Nv), 256, 0, st>>>(
            (const T*)a.q, (const T*)a.k, a.G, (const float*)a.H, (const float*)a.VN, (const float*)a.W, b.d_o,
            b.do_f32, a.scale, a.chunk_start, a.chunk_len, a.Nk, a.Nv, b.Hn, b.Vn, b.WT, b.P, b.dVn, b.dSout,
            (int)a.states16);
    }
    mark(2);
    if (a.N > 0) {
        k_bwd_state<T, DK, DV, C><<<dim3(a.N, a.Nv, DV / 16), 256, 0, st>>>(
            (const T*)a.k, a.G, b.WT, b.dST, a.chunk_start, a.chunk_len, a.seq_first, a.Nk, a.Nv, b.dSout, b.dVn,
            b.dS0);
    }
    mark(3);
    if (NT > 0) {
        k_bwd_chunk<T, DK, DV, C><<<dim3(NT, a.Nv), 256, 0, st>>>(
            (const T*)a.q, (const T*)a.k, (const T*)a.v, a.beta, a.beta_f32, a.G, (const float*)a.A, b.P, b.Hn,
            b.Vn, b.dSout, b.dVn, b.d_o, b.do_f32, a.chunk_start, a.chunk_len, a.Nk, a.Nv, a.scale, b.dWs,
            b.dqv, b.dkv, b.dv, b.dbeta, b.dg);
    }
    mark(4);
    const int64_t nq = a.Ttot * a.Nk * DK;
    if (nq > 0)
        k_bwd_reduce_qk<DK><<<(unsigned)((nq + 255) / 256), 256, 0, st>>>(b.dqv, b.dkv, a.Ttot, a.Nk, a.Nv, b.dq,
                                                                          b.dk);
    mark(5);
    return hipGetLastError();
}

template <typename T, int C>
hipError_t bwd_dims(const BackwardArgs& b) {
#define GDR_BCASE(DKv, DVv) \
    if (b.fwd.dk == DKv && b.fwd.dv == DVv) return launch_bwd<T, DKv, DVv, C>(b);
    GDR_BCASE(32, 32) GDR_BCASE(32, 64) GDR_BCASE(32, 128)
    GDR_BCASE(64, 32) GDR_BCASE(64, 64) GDR_BCASE(64, 128)
    GDR_BCASE(128, 32) GDR_BCASE(128, 64) GDR_BCASE(128, 128)
#undef GDR_BCASE
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t bwd_chunk(const BackwardArgs& b) {
    if (b.fwd.C == 64) return bwd_dims<T, 64>(b);
    if (b.fwd.C == 32) return bwd_dims<T, 32>(b);
    if (b.fwd.C == 16) return bwd_dims<T, 16>(b);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_backward(const BackwardArgs& b) {
    return b.fwd.bf16 ? bwd_chunk<bf16>(b) : bwd_chunk<float>(b);
}

}  // namespace gdr
