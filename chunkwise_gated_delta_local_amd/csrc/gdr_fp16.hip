// Production path of the chunked gated delta-rule forward for bf16 inputs
// with C = 64, on the fp16 matrix cores of gfx950.
//
// Method (FLA DeltaNet article on pnsm.cn, sections 2.3-2.4 and 3.1-3.4;
// ChunkGatedDeltaRule math page, section 3, formulas (1)-(6)); per chunk of
// 64 tokens and value head h (q/k head kh = h / (Nv/Nk)):
//   G      chunk-local inclusive prefix sum of g
//   L      strictly lower beta_i (k_i . k_j) exp(G_i - G_j);   A = (I + L)^-1
//   T      A diag(beta)                        (the article's T, section 2.3)
//   P      (Q K^T) (.) D,  D_ij = exp(G_i - G_j) for j <= i    (formula (5))
//   Y      K S_in,   Z = V - diag(exp(G)) Y,   V_new = T Z     (= U - W S_in, formula (3))
//   S_out  exp(G_last) S_in + K^T diag(exp(G_last - G)) V_new (formula (6))
//   O      scale [diag(exp(G)) Q S_in + P V_new]               (formulas (4), (5))
//
// Two kernels:
//   k_prep     one workgroup per (chunk, q/k head), fully parallel over chunks:
//              gate sums and decay rows, K K^T and Q K^T on exact bf16
//              products, the triangular solve in fp32, then T and P rounded
//              once to fp16 matrix-core fragments.
//   k_chunk16  one workgroup per (sequence, value head, 16 columns of dv): the
//              chunk-serial pass. One "chain" wavefront keeps the dk x 16 state
//              slice in registers and runs the whole per-chunk dependency
//              Y -> Z -> V_new -> S on the matrix cores without touching LDS
//              for it: every product's result is, lane for lane, an operand of
//              the next (two stacked accumulator tiles are a pair fragment of
//              the transposed block). Three helper wavefronts form O from the
//              fp16 Q rows, the P pairs and exp(G) (loaded straight into
//              registers) and from the state and V_new the chain publishes in
//              LDS; they also copy the fp16 K tiles and the V slices of later
//              chunks into LDS with buffer-to-LDS loads.
//
// Number formats: q, k, v are exact in bf16 and exact in fp16 (an fp16 has
// more significant bits; values below 2^-14 become fp16 subnormals, absolute
// error below 2^-25). Every value derived inside the method (T, P, the state
// operand, Z, V_new) is rounded once to fp16 (11 significant bits) where it
// enters a product; every product accumulates in fp32 and the state itself is
// carried in fp32. fp16 range: derived values must stay below 65504 in
// magnitude, which holds for L2-normalised keys and gates g <= 0.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gdr_device.hpp"
#include "gdr_fp16.hpp"
#include "gdr_launch.hpp"

namespace gdr {

typedef _Float16 f16;
typedef f16 h8 __attribute__((ext_vector_type(8)));
typedef f16 h4 __attribute__((ext_vector_type(4)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef s4 __attribute__((address_space(3))) * lds_s4;
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

namespace {

constexpr int kPairs = 6;      // lower-triangular (16-row block, 32-position block) pairs of a 64 x 64 block
// pair p = 0..5 covers row block tb(p) = 0, 1, 2, 2, 3, 3 and position block
// tp(p) = 0, 0, 0, 1, 0, 1 (formed arithmetically: a table indexed by a
// run-time p would be a memory load on the critical path)
__device__ __forceinline__ int pair_tb(int p) { return p < 2 ? p : (p + 2) >> 1; }
__device__ __forceinline__ int pair_tp(int p) { return p < 2 ? 0 : (p - 2) & 1; }
constexpr int kFrag = 512;     // elements of one pair fragment (64 lanes x 8)
// In global memory the six pairs of one (chunk, value head) are packed
// (kPackedPairs values): pairs 0 and 3 sit on the diagonal of an even row
// block, so their positions 16..31 (lane elements 4..7) lie above the
// diagonal and are zero; each keeps only elements 0..3 of every lane (lane l
// at values 4 l .. 4 l + 3). Pair p starts at value pair_off(p).
__host__ __device__ constexpr bool pair_half(int p) { return p == 0 || p == 3; }
__host__ __device__ constexpr int pair_off(int p) { return 512 * p - (p >= 1 ? 256 : 0) - (p >= 4 ? 256 : 0); }
static_assert(pair_off(kPairs - 1) + kFrag == kPackedPairs, "packed pair layout");
constexpr int kRsrc = 0x00020000;   // buffer descriptor word 3: raw 32-bit access

__device__ __forceinline__ f32x4 mfma16(const h8& a, const h8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// two fp32 values -> packed fp16 pair, round to nearest even (v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t pk16(float x, float y) {
    typedef f16 h2 __attribute__((ext_vector_type(2)));
    h2 v;
    v[0] = (f16)x;
    v[1] = (f16)y;
    return __builtin_bit_cast(uint32_t, v);
}
// two accumulator tiles (contraction rows 0..15 and 16..31) -> fp16 pair fragment
__device__ __forceinline__ h8 pack_pair(const f32x4& a0, const f32x4& a1) {
    u4 w = {pk16(a0[0], a0[1]), pk16(a0[2], a0[3]), pk16(a1[0], a1[1]), pk16(a1[2], a1[3])};
    return __builtin_bit_cast(h8, w);
}
__device__ __forceinline__ u2 pack4(const f32x4& a) { return u2{pk16(a[0], a[1]), pk16(a[2], a[3])}; }
// eight bf16 (one 16-byte load) -> eight fp16; exact for normal values (bf16 has 8 significant bits)
__device__ __forceinline__ h8 bf16x8_to_f16(const u4& w) {
    u4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = __builtin_bit_cast(float, w[i] << 16);
        const float hi = __builtin_bit_cast(float, w[i] & 0xffff0000u);
        r[i] = pk16(lo, hi);
    }
    return __builtin_bit_cast(h8, r);
}
__device__ __forceinline__ f32x4 bf16x4_to_f32(const s4& v) {
    f32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = __builtin_bit_cast(float, ((uint32_t)(uint16_t)v[j]) << 16);
    return r;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base, int64_t byte_off, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(reinterpret_cast<const char*>(base)) + byte_off,
                                             (short)0, (int)bytes, kRsrc);
}
__device__ __forceinline__ u4 buf_load16(__amdgpu_buffer_rsrc_t rs, int voff) {
    return __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0));
}
__device__ __forceinline__ u2 buf_load8(__amdgpu_buffer_rsrc_t rs, int voff) {
    return __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(rs, voff, 0, 0));
}
// a packed half pair's four values per lane -> the lane's pair fragment (elements 4..7 zero)
__device__ __forceinline__ h8 half_pair(u2 lo) { return __builtin_bit_cast(h8, u4{lo[0], lo[1], 0u, 0u}); }

// fp16 K and Q tiles (64 rows of DK values per chunk and q/k head): the 16-byte
// unit u of row `row` sits at unit u ^ tile_swz(row), in global memory as in
// LDS, so that a tile is copied verbatim and the chunk pass's operand reads
// (16-byte row reads and transposing K^T reads) spread over the LDS banks.
template <int DK>
__device__ __forceinline__ int tile_swz(int row) {
    return ((((row & 3) << 1) | ((row >> 2) & 1) | (row & 8))) & (DK / 8 - 1);
}

}  // namespace

// ============================================================ k_prep
// One workgroup (four wavefronts) per (chunk, q/k head); it serves the value
// heads that share the key head (ChunkGatedDeltaRule page, section 1: GQA).
//   1. K and Q rows of the chunk -> LDS (zero past the chunk end), and as fp16
//      tiles for the chunk pass.
//   2. K K^T and the transposed score tiles K Q^T of block row `wave` on bf16
//      matrix cores: exact products of the inputs, fp32 sums (FLA DeltaNet
//      article, section 3.1).
//   3. Per value head (the gates of up to four heads are loaded, scanned and
//      placed in LDS together, so the per-head phases issue no global load and
//      their barriers wait for LDS only):
//      a. G = inclusive prefix sum of g over the chunk (one lane per position,
//         a shuffle scan in fp32); the decay rows R = (exp(G), exp(G_last - G))
//         (zero past the chunk end) for the state pass.
//      b. L = tril(beta_i (k_i . k_j) exp(G_i - G_j), -1) in fp32 (LDS).
//      c. The four 16 x 16 diagonal blocks of A = (I + L)^-1 by forward
//         substitution in fp32, then the off-diagonal blocks by block
//         substitution, 16 -> 32 -> 64, on split-bf16 matrix cores (three
//         passes, fp32-level accuracy) (ChunkGatedDeltaRule page, section 3.1;
//         FLA DeltaNet article, section 3.2).
//      d. T = A diag(beta) and P_ij = (q_i . k_j) exp(G_i - G_j) (j <= i < L)
//         rounded to fp16 pair fragments of the six lower blocks.
// WITH_P false (the backward's recompute of the chunk states, which forms no
// output): no Q rows, Q tiles or score block.
template <int DK, bool WITH_P>
__global__ __launch_bounds__(256, 4) void k_prep(const bf16* __restrict__ k, const bf16* __restrict__ q,
                                                  const void* __restrict__ beta, int beta_f32,
                                                  const float* __restrict__ g,
                                                  const int32_t* __restrict__ chunk_start,
                                                  const int32_t* __restrict__ chunk_len, int32_t Nk, int32_t Nv,
                                                  f16* __restrict__ Tf, f16* __restrict__ Pf,
                                                  float* __restrict__ R, f16* __restrict__ K16,
                                                  f16* __restrict__ Q16) {
    constexpr int C = 64, NTHR = 256;
    constexpr int KP = DK + 8;                 // padded LDS row (elements)
    constexpr int SEGS = C * (DK / 8) / NTHR;  // 16-byte row segments per thread (>= 1 for DK >= 32)
    constexpr int TILE_BYTES = 2 * C * KP * 2;
    constexpr int LP = C + 4;                  // L and A row pitch (floats)
    constexpr int LA_BYTES = 2 * C * LP * 4;
    static_assert(SEGS >= 1, "dk");
    __shared__ __attribute__((aligned(16))) char smem[TILE_BYTES > LA_BYTES ? TILE_BYTES : LA_BYTES];
    constexpr int HB = 4;                      // value heads whose gates are prepared together
    __shared__ __attribute__((aligned(16))) float bsa[HB][C], gsa[HB][C];
    bf16* Ks = reinterpret_cast<bf16*>(smem);
    bf16* Qs = Ks + C * KP;
    float (*Lf)[LP] = reinterpret_cast<float (*)[LP]>(smem);
    float (*Af)[LP] = Lf + C;
    typedef Vec<bf16>::v8 v8;

    const int c = blockIdx.x, kh = blockIdx.y;
    const int64_t s = chunk_start[c];
    const int L = chunk_len[c];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 15, qd = lane >> 4;
    const int group = Nv / Nk;

    // beta and g of up to HB value heads go through registers of wave 0, as
    // raw bits (no arithmetic on a freshly loaded value): the first batch's are
    // loaded with the tiles; each batch's prefix sums, decay rows and LDS rows
    // are formed before its heads are processed, so the per-head phases issue
    // no global load (and no wait that would drain their stores)
    uint32_t b_raw[HB];
    float g_raw[HB];
    auto fetch_gates = [&](int hb) {           // heads hb .. hb + HB - 1 of the group
        const int64_t idx = (s + tid) * Nv + kh * group + hb;
#pragma unroll
        for (int u = 0; u < HB; ++u) {
            b_raw[u] = 0;
            g_raw[u] = 0.f;
            if (tid < L && hb + u < group) {
                if (beta_f32) b_raw[u] = reinterpret_cast<const uint32_t*>(beta)[idx + u];
                else b_raw[u] = reinterpret_cast<const uint16_t*>(beta)[idx + u];
                if (g) g_raw[u] = g[idx + u];
            }
        }
    };
    // prefix sums over the 64 positions (wave 0, one lane per position), decay
    // rows R = (exp(G), exp(G_last - G)) for the chunk pass, and the LDS rows
    auto prepare_gates = [&](int hb) {
#pragma unroll
        for (int u = 0; u < HB; ++u) {
            if (hb + u >= group) break;
            float x = g_raw[u];
#pragma unroll
            for (int off = 1; off < C; off <<= 1) {
                const float y = __shfl_up(x, off, C);
                if (lane >= off) x += y;
            }
            const float g_last = __shfl(x, L > 0 ? L - 1 : 0, C);
            const bool on = lane < L;
            gsa[u][lane] = on ? x : 0.f;
            bsa[u][lane] = __uint_as_float(beta_f32 ? b_raw[u] : b_raw[u] << 16);
            float* Rh = R + ((int64_t)c * Nv + kh * group + hb + u) * 2 * C;
            Rh[lane] = on ? __expf(x) : 0.f;
            Rh[C + lane] = on ? __expf(g_last - x) : 0.f;
        }
    };

    // 1. K and Q rows (all loads first)
    {
        v8 kv[SEGS], qv[SEGS];
#pragma unroll
        for (int i = 0; i < SEGS; ++i) {
            const int idx = tid + NTHR * i, row = idx / (DK / 8), seg = idx % (DK / 8);
            kv[i] = zero_pair<bf16>();
            qv[i] = zero_pair<bf16>();
            if (row < L) {
                kv[i] = *reinterpret_cast<const v8*>(k + ((s + row) * Nk + kh) * DK + seg * 8);
                if constexpr (WITH_P) qv[i] = *reinterpret_cast<const v8*>(q + ((s + row) * Nk + kh) * DK + seg * 8);
            }
        }
        if (wave == 0) fetch_gates(0);
        f16* kt16 = K16 + ((int64_t)c * Nk + kh) * C * DK;
        f16* qt16 = Q16 + ((int64_t)c * Nk + kh) * C * DK;
#pragma unroll
        for (int i = 0; i < SEGS; ++i) {
            const int idx = tid + NTHR * i, row = idx / (DK / 8), seg = idx % (DK / 8);
            *reinterpret_cast<v8*>(&Ks[row * KP + seg * 8]) = kv[i];
            *reinterpret_cast<v8*>(&Qs[row * KP + seg * 8]) = qv[i];
            // the fp16 tiles of the chunk pass (exact: bf16 values are fp16 values
            // down to fp16's subnormal range)
            const int u = (seg ^ tile_swz<DK>(row)) * 8;
            *reinterpret_cast<h8*>(&kt16[row * DK + u]) = bf16x8_to_f16(__builtin_bit_cast(u4, kv[i]));
            if constexpr (WITH_P) *reinterpret_cast<h8*>(&qt16[row * DK + u]) = bf16x8_to_f16(__builtin_bit_cast(u4, qv[i]));
        }
    }
    lds_barrier();

    // 2. kk[j]: K K^T rows 16 wave + 4 qd + jj, column 16 j + r.
    //    qk[j]: k_{16 j + 4 qd + jj} . q_{16 wave + r} (the score block transposed).
    f32x4 kk[4], qk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        kk[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        qk[j] = kk[j];
        if (j <= wave) {
#pragma unroll
            for (int kp = 0; kp < DK / 32; ++kp) {
                const v8 kw = load_pair_row<bf16>(&Ks[(wave * 16 + r) * KP + kp * 32], qd);
                const v8 kj = load_pair_row<bf16>(&Ks[(j * 16 + r) * KP + kp * 32], qd);
                const v8 qw = load_pair_row<bf16>(&Qs[(wave * 16 + r) * KP + kp * 32], qd);
                kk[j] = mfma_pair(kw, kj, kk[j]);
                if constexpr (WITH_P) qk[j] = mfma_pair(kj, qw, qk[j]);
            }
        }
    }
    lds_barrier();                           // tiles consumed: the LDS now holds L and A
    for (int idx = tid; idx < 2 * 256; idx += NTHR) {   // the two strictly-upper blocks the merges read
        const int blk = idx >> 8, e = idx & 255, row = blk * 32 + (e >> 4), col = blk * 32 + 16 + (e & 15);
        Af[row][col] = 0.f;
    }

    for (int hh = 0; hh < group; ++hh) {
        const int h = kh * group + hh;
        // 3a. the gates of heads hh .. hh + HB - 1 (wave 0)
        if (hh % HB == 0) {
            if (wave == 0) {
                if (hh > 0) fetch_gates(hh);
                prepare_gates(hh);
            }
            lds_barrier();
        }
        const float* gs = gsa[hh % HB];
        const float* bs = bsa[hh % HB];

        // 3b. strictly lower L
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j <= wave) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int i = wave * 16 + 4 * qd + jj, col = j * 16 + r;
                    float val = 0.f;
                    if (i > col && i < L) val = bs[i] * kk[j][jj] * __expf(gs[i] - gs[col]);
                    Lf[i][col] = val;
                }
            }
        }
        lds_barrier();

        // 3c. diagonal block `wave`: lane r < 16 owns column r of the block's
        //     inverse; each substitution step reads row i of L with broadcast reads
        {
            const int b0 = wave * 16;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = (i == lane) ? 1.f : 0.f;
#pragma unroll
            for (int i = 1; i < 16; ++i) {
                const float* lr = &Lf[b0 + i][b0];
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < i; ++m) acc += lr[m] * x[m];
                if (i > lane) x[i] = -acc;
            }
            if (lane < 16) {
#pragma unroll
                for (int i = 0; i < 16; ++i) Af[b0 + i][b0 + lane] = x[i];
            }
        }
        lds_barrier();
        // A_ij = -A_ii (L_ij A_jj) for (i, j) = (1, 0) [wave 0] and (3, 2) [wave 1]
        if (wave < 2) {
            const int bi = 2 * wave + 1, bj = 2 * wave;
            float la[8], db[8], ai[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                la[e] = Lf[bi * 16 + r][bj * 16 + 4 * qd + e];
                db[e] = Af[bj * 16 + 4 * qd + e][bj * 16 + r];
                ai[e] = Af[bi * 16 + r][bi * 16 + 4 * qd + e];
                la[4 + e] = db[4 + e] = ai[4 + e] = 0.f;
            }
            const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
            const f32x4 t1 = mfma_dd<bf16>(split8<bf16>(la), split8<bf16>(db), zero4);
            const f32x4 t2 = mfma_dd<bf16>(split8<bf16>(ai), split_acc_pair<bf16>(t1, zero4), zero4);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) Af[bi * 16 + 4 * qd + jj][bj * 16 + r] = -t2[jj];
        }
        lds_barrier();
        // lower-left 32 x 32 block = -A_bot (L_bl A_top); wave w < 2 takes column block w
        if (wave < 2) {
            const int ct = wave;
            float bt[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                bt[e] = Af[4 * qd + e][ct * 16 + r];
                bt[4 + e] = Af[16 + 4 * qd + e][ct * 16 + r];
            }
            const Split<bf16> b = split8<bf16>(bt);
            f32x4 t1[2];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
                t1[rb] = mfma_dd<bf16>(load_split_row<bf16>(&Lf[32 + 16 * rb + r][0], qd), b,
                                       f32x4{0.f, 0.f, 0.f, 0.f});
            const Split<bf16> b2 = split_acc_pair<bf16>(t1[0], t1[1]);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const f32x4 t2 = mfma_dd<bf16>(load_split_row<bf16>(&Af[32 + 16 * rb + r][32], qd), b2,
                                               f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) Af[32 + 16 * rb + 4 * qd + jj][ct * 16 + r] = -t2[jj];
            }
        }
        lds_barrier();

        // 3d. T = A diag(beta): pair p covers rows 16 tb + r and positions
        //     32 tp + m(qd, e) (m = 4 qd + e, or 16 + 4 qd + e - 4); rows past the end are zero
        for (int p = wave; p < kPairs; p += 4) {
            const int tb = pair_tb(p), tp = pair_tp(p);
            const int row = tb * 16 + r;
            const int m0 = tp * 32 + 4 * qd;
            const f32x4 a0 = *reinterpret_cast<const f32x4*>(&Af[row][m0]);
            const f32x4 a1 = *reinterpret_cast<const f32x4*>(&Af[row][m0 + 16]);
            const f32x4 b0 = *reinterpret_cast<const f32x4*>(&bs[m0]);
            const f32x4 b1 = *reinterpret_cast<const f32x4*>(&bs[m0 + 16]);
            f32x4 x0, x1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x0[e] = (row < L && m0 + e <= row) ? a0[e] * b0[e] : 0.f;
                x1[e] = (row < L && m0 + 16 + e <= row) ? a1[e] * b1[e] : 0.f;
            }
            f16* dst = Tf + ((int64_t)c * Nv + h) * kPackedPairs + pair_off(p);
            if (pair_half(p))
                *reinterpret_cast<u2*>(dst + lane * 4) = pack4(x0);
            else
                *reinterpret_cast<h8*>(dst + lane * 8) = pack_pair(x0, x1);
        }
        if constexpr (WITH_P) {
            //     P pairs of block row `wave` (rows i = 16 wave + r): the transposed
            //     tiles qk[j] are, stacked two at a time, the pair fragments of P
            {
                const int i = wave * 16 + r;
                f32x4 pt[4];
    #pragma unroll
                for (int j = 0; j < 4; ++j) {
    #pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int col = j * 16 + 4 * qd + jj;
                        pt[j][jj] = (j <= wave && col <= i && i < L) ? qk[j][jj] * __expf(gs[i] - gs[col]) : 0.f;
                    }
                }
                const int pbase = (wave == 0) ? 0 : (wave == 1 ? 1 : (wave == 2 ? 2 : 4));
    #pragma unroll
                for (int tp = 0; tp < 2; ++tp) {
                    if (2 * tp <= wave) {
                        const int p = pbase + tp;
                        f16* dst = Pf + ((int64_t)c * Nv + h) * kPackedPairs + pair_off(p);
                        if (pair_half(p))
                            *reinterpret_cast<u2*>(dst + lane * 4) = pack4(pt[2 * tp]);
                        else
                            *reinterpret_cast<h8*>(dst + lane * 8) = pack_pair(pt[2 * tp], pt[2 * tp + 1]);
                    }
                }
            }
        }
        lds_barrier();
    }
}

// ============================================================ k_chunk16
// Modes: kFull16 (state and output from S0, or from the segment entering
// states) and kSegment16 (state only: a workgroup with blockIdx.z < dv/16
// forms the end state of its run of chunks from a zero state; one with a
// larger blockIdx.z forms the map the run applies to its entering state, the
// end state from S = I over dk columns with V read as zero). Both serve
// segment-parallel state passing; the full mode also serves the serial pass.
//
// One workgroup of four wavefronts (one per SIMD, up to 512 registers each)
// per (sequence, value head, 16 columns of dv). Per chunk c the chain
// wavefront runs the serial dependency
//     Y = K S,  Z = V - exp(G) Y,  V_new = T Z,  S = exp(G_last) S + K^T (exp(G_last - G) V_new)
// on the matrix cores with the dk x 16 state slice in registers: every
// product's accumulators are, lane for lane, an operand of the next (two
// stacked accumulator tiles are a pair fragment of the transposed block).
// All of its operands are in registers when the step starts: the K operand
// of Y, the V rows, the T pairs and the decay rows of chunk c + 1 are read
// from LDS during step c; the chain issues no vector-memory operation. The other three
// wavefronts form the output, transposed (O^T = S^T Q^T + V_new^T P^T, so that
// each lane holds four adjacent columns of one row), for the row blocks
// {0, 1}, {2} and {3}: chunk c's output in step c + 1, from the entering state
// and V_new the chain published in step c and from the Q rows, score pairs and
// exp(G) they loaded from global memory in step c - 1. Wavefront 1 also copies
// the V slice and the decay rows of chunk c + 3 into LDS (16-byte
// buffer-to-LDS loads); wavefronts 2 and 3 copy the two halves (rows 0..31
// and 32..63) of chunk c + 3's fp16 K tile and half of its T pairs each. One
// LDS-only barrier per chunk step. K tiles, V slices, T pairs and decay rows
// are quadruple-buffered, the published state and V_new double-buffered.
//
// LDS layout of a K tile: row-major, 64 rows of dk fp16 values, the 16-byte
// units of row `row` permuted by an XOR with swz(row), so that the chain's
// operand reads and its transposing K^T reads hit distinct banks.
template <int DK, int DV, int MODE>
__global__ __launch_bounds__(256) void k_chunk16(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                 const bf16* __restrict__ v, const float* __restrict__ R,
                                                 const f16* __restrict__ Tf, const f16* __restrict__ Pf,
                                                 const f16* __restrict__ K16, const f16* __restrict__ Q16,
                                                 const float* __restrict__ S0,
                                                 const int32_t* __restrict__ chunk_start,
                                                 const int32_t* __restrict__ chunk_len,
                                                 const int32_t* __restrict__ first, int32_t Nk, int32_t Nv,
                                                 float scale, int out_f32, void* __restrict__ o,
                                                 float* __restrict__ ST, float* __restrict__ ST2,
                                                 float* __restrict__ Hout, float* __restrict__ VNout) {
    constexpr int C = 64;
    constexpr int NKP = DK / 32, NDB = DK / 16;
    constexpr bool want_o = MODE == kFull16;
    constexpr bool want_h = MODE == kStates16;   // entering states and V_new out (fp32)
    __shared__ __attribute__((aligned(16))) f16 Ks[4][C * DK];
    __shared__ __attribute__((aligned(16))) bf16 Vs[4][C * 16];
    __shared__ __attribute__((aligned(16))) f16 Ts[4][kPairs * kFrag];  // T pairs of a chunk
    __shared__ __attribute__((aligned(16))) float Rs[4][256];           // decay rows (128 used)
    __shared__ __attribute__((aligned(16))) f16 Sx[2][NKP][kFrag];     // entering state, natural dk order
    __shared__ __attribute__((aligned(16))) f16 VNx[2][2][kFrag];      // V_new pairs (stacked positions)
    // kStates16: the entering state's and V_new's fp32 accumulator tiles, lane-contiguous
    __shared__ __attribute__((aligned(16))) float Hx[want_h ? 2 : 1][want_h ? NDB : 1][want_h ? 256 : 4];
    __shared__ __attribute__((aligned(16))) float VNx32[want_h ? 2 : 1][want_h ? 4 : 1][want_h ? 256 : 4];
    __shared__ uint32_t pf_sink[64];                                     // checksum of the L2 warm-up loads (never read)

    // XCD-aware placement. Workgroups go to the eight XCDs round-robin by
    // linear id. A unit is the (sequence, q/k head) pair whose workgroups (the
    // group's value heads x the column tiles) read the same K and Q tiles; the
    // workgroups of a unit go to one XCD, consecutively, so they share its L2.
    // Units are dealt to the XCDs in snake order (0..7, 7..0, ...) over
    // (sequence, q/k head), so every XCD gets the same share of every
    // sequence's heads and sequences of different lengths do not leave one
    // XCD with the longest ones. Otherwise (a unit count not a multiple of 8)
    // each XCD takes a contiguous run of (sequence, head, column tile) triples.
    int bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
    {
        const int64_t W = (int64_t)gridDim.x * gridDim.y * gridDim.z;
        const int64_t lin = bx + (int64_t)gridDim.x * (by + (int64_t)gridDim.y * bz);
        const int G = Nv / Nk;
        const int per_unit = G * gridDim.z;                   // workgroups of a unit
        const int64_t units = (int64_t)gridDim.x * Nk;
        if (units % 8 == 0) {
            const int x = (int)(lin % 8);
            const int64_t i = lin / 8;                        // position in the XCD's list
            const int64_t lu = i / per_unit;                  // the XCD's lu-th unit
            const int j = (int)(i % per_unit);
            const int64_t rank = lu * 8 + ((lu & 1) ? 7 - x : x);
            bx = (int)(rank / Nk);
            const int kh_u = (int)(rank % Nk);
            by = kh_u * G + j / gridDim.z;
            bz = j % gridDim.z;
        } else if (W % 8 == 0) {
            const int64_t work = (lin % 8) * (W / 8) + lin / 8;
            bz = (int)(work % gridDim.z);
            by = (int)((work / gridDim.z) % gridDim.y);
            bx = (int)(work / ((int64_t)gridDim.z * gridDim.y));
        }
    }
    const int n = bx, h = by;
    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, r = lane & 15, qd = lane >> 4;
    const int kh = h / (Nv / Nk);
    const bool trans = MODE == kSegment16 && bz >= DV / 16;   // transition workgroup
    const int nb = trans ? bz - DV / 16 : bz;
    const int NC = trans ? DK : DV;
    float* const STo = trans ? ST2 : ST;
    const int c0 = __builtin_amdgcn_readfirstlane(first[n]), c1 = __builtin_amdgcn_readfirstlane(first[n + 1]);
    auto slot4 = [&](int c) { return (c - c0) & 3; };      // K tiles; V, decay rows and T
    // chunk start and length in scalar registers (uniform buffer descriptors),
    // formed from the run's first chunk and its end: the chunks of a run are
    // consecutive C-token pieces of one sequence (the last may be shorter), so
    // no step waits for a table load; a chunk past the run's last reads as empty
    const int64_t run_s = c0 < c1 ? (int64_t)__builtin_amdgcn_readfirstlane(chunk_start[c0]) : 0;
    const int64_t run_e = c0 < c1 ? (int64_t)__builtin_amdgcn_readfirstlane(chunk_start[c1 - 1]) +
                                        __builtin_amdgcn_readfirstlane(chunk_len[c1 - 1])
                                  : 0;
    auto chunk_s = [&](int c) { return c < c1 ? run_s + (int64_t)(c - c0) * C : (int64_t)0; };
    auto chunk_L = [&](int c) { return c < c1 ? max(0, min(C, (int)(run_e - chunk_s(c)))) : 0; };
    auto swz = [](int row) { return tile_swz<DK>(row); };
    const int64_t sbase = ((int64_t)n * Nv + h) * DK * NC;
    typedef std::integral_constant<int, 0> P0;
    typedef std::integral_constant<int, 1> P1;
    // V slice of a chunk -> LDS: 2 buffer-to-LDS loads of 16 bytes per lane
    // (a chunk past the sequence's last reads as zero)
    auto copy_v = [&](int c) {
        const int sl = slot4(c);
        const int64_t s = chunk_s(c);
        const int L = chunk_L(c);
        const uint32_t vbytes = (trans || L <= 0) ? 0u : (uint32_t)((L - 1) * Nv * DV + 16) * 2u;
        const auto rv = rsrc_of(v, ((s * Nv + h) * DV + nb * 16) * 2, vbytes);
#pragma unroll
        for (int vh = 0; vh < 2; ++vh)                    // rows 32 vh .. 32 vh + 31, 16 columns
            buffer_to_lds16(rv, &Vs[sl][vh * 512], ((32 * vh + (lane >> 1)) * Nv * DV + 8 * (lane & 1)) * 2);
    };

    if (wv == 0) {
        // ======================================================== chain
        // State tile t, accumulator row 4 qd + j holds dk row srow(t, 4 qd + j) =
        // 32 (t / 2) + 8 qd + 4 (t % 2) + j: then the two tiles 2 kp, 2 kp + 1,
        // stacked, are the state's operand for dk 32 kp .. 32 kp + 31 in the
        // natural order (lane (qd, r) element e = dk 32 kp + 8 qd + e), the order
        // in which a 16-byte read of a K row is that row's operand.
        auto srow = [&](int t, int j) { return 32 * (t >> 1) + 8 * qd + 4 * (t & 1) + j; };
        f32x4 S[NDB];
#pragma unroll
        for (int t = 0; t < NDB; ++t) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = srow(t, j), col = nb * 16 + r;
                S[t][j] = trans ? (row == col ? 1.f : 0.f) : (S0 ? S0[sbase + (int64_t)row * NC + col] : 0.f);
            }
        }
        h8 Sp[NKP];
        // state pairs for Y; the output waves take the same fragments (published
        // at the start of the chunk's step, read in the next step)
        auto make_pairs = [&]() {
#pragma unroll
            for (int kp = 0; kp < NKP; ++kp) Sp[kp] = pack_pair(S[2 * kp], S[2 * kp + 1]);
        };
        // K operand of Y: row 16 b + r, dk 32 kp + 8 qd .. + 7 (one 16-byte read)
        h8 ka[4][NKP];
        auto read_ka = [&](int c) {
            const f16* Kb = Ks[slot4(c)];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int row = 16 * b + r;
#pragma unroll
                for (int kp = 0; kp < NKP; ++kp)
                    ka[b][kp] = *reinterpret_cast<const h8*>(&Kb[row * DK + ((4 * kp + qd) ^ swz(row)) * 8]);
            }
        };
        // V rows 16 b + 4 qd + j of column r (transposing reads of the bf16 tile)
        struct VR {
            s4 v[4];
        };
        auto read_vr = [&](int c) {
            VR x;
            const int sl = slot4(c);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int row = 16 * b + 4 * qd + (r >> 2);
                x.v[b] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)&Vs[sl][row * 16 + 4 * (r & 3)]);
            }
            return x;
        };
        // T pairs and decay rows of a chunk, read from LDS a step ahead:
        // exp(G) and exp(G_last - G) of rows 16 b + 4 qd + j, and exp(G_last) =
        // exp(G_0) exp(G_last - G_0) from the rows themselves
        struct TR {
            h8 tf[kPairs];
            f32x4 eg[4], ed[4];
            float a0, a1;
        };
        auto read_tr = [&](int c) {
            TR x;
            const int sl = slot4(c);
#pragma unroll
            for (int p = 0; p < kPairs; ++p)
                x.tf[p] = pair_half(p) ? half_pair(*reinterpret_cast<const u2*>(&Ts[sl][p * kFrag + lane * 4]))
                                       : *reinterpret_cast<const h8*>(&Ts[sl][p * kFrag + lane * 8]);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                x.eg[b] = *reinterpret_cast<const f32x4*>(&Rs[sl][16 * b + 4 * qd]);
                x.ed[b] = *reinterpret_cast<const f32x4*>(&Rs[sl][C + 16 * b + 4 * qd]);
            }
            x.a0 = Rs[sl][0];
            x.a1 = Rs[sl][C];
            return x;
        };
        // L2 warm-up. Each chunk's tiles (K16, Q16 per q/k head; T and P pairs,
        // decay rows and the V rows per value head) are read by every column
        // tile of a head (and by both value heads of a GQA pair), each time as
        // an L2 miss if none of them has touched the lines yet. At step c the
        // chain loads one dword per 128-byte line of chunk c + kAhead, the
        // lines split over the workgroups that share them (about 45 lines per
        // workgroup and chunk at dk = dv = 128): the helpers' copies and
        // loads, issued three and one steps ahead, then hit the L2. The loads
        // for two chunks are issued at the start of an even step and folded
        // into a checksum at the end of the odd step after it (the chain's
        // only wait for them, two steps after the loads); the checksum goes to
        // an LDS word that is never read, which keeps the loads. Four to six
        // steps ahead measured best (eight: 1.5 % slower, twelve: 5 %).
        constexpr int kAhead = 6;
        // (the serial pass and the backward's state pass; the latter reads no Q16 or P)
        constexpr bool want_pf = want_o || want_h;
        constexpr int NKT = want_o ? 2 : 1, NPT = want_o ? 2 : 1;         // K16 (and Q16); T (and P)
        const char* pf_base = nullptr;           // the tensor; byte offset of chunk cp's line: pf_off + cp pf_stride
        int64_t pf_off = 0, pf_stride = 0;
        int pf_row = -1;                         // V lines: the row, valid only below the chunk's length
        bool pf_on = false;
        if constexpr (want_pf) {
            constexpr int NB = DV / 16, LT = C * DK * 2 / 128;                  // column tiles; lines of a K/Q tile
            constexpr int LTP = kPackedPairs * 2 / 128, LR = 2 * C * 4 / 128;    // lines of T (and P); of R
            constexpr int VL = DV * 2 >= 128 ? DV * 2 / 128 : 1;                 // lines of a V row
            constexpr int NVL = NPT * LTP + LR + C * VL;                         // lines per value head
            const int G = Nv / Nk, U = G * NB, u = (h % G) * NB + nb;
            const int cnt_k = u < NKT * LT ? (NKT * LT - u + U - 1) / U : 0;
            const int cnt_v = (NVL - nb + NB - 1) / NB;
            int idx = lane;
            if (idx < cnt_k) {
                const int i = u + U * idx;
                const f16* t = i < LT ? K16 : Q16;
                pf_base = reinterpret_cast<const char*>(t);
                pf_off = (int64_t)kh * C * DK * 2 + (int64_t)(i % LT) * 128;
                pf_stride = (int64_t)Nk * C * DK * 2;
                pf_on = true;
            } else if ((idx -= cnt_k) < cnt_v) {
                const int j = nb + NB * idx;
                if (j < NPT * LTP) {
                    const f16* t = j < LTP ? Tf : Pf;
                    pf_base = reinterpret_cast<const char*>(t);
                    pf_off = (int64_t)h * kPackedPairs * 2 + (int64_t)(j % LTP) * 128;
                    pf_stride = (int64_t)Nv * kPackedPairs * 2;
                } else if (j < NPT * LTP + LR) {
                    pf_base = reinterpret_cast<const char*>(R);
                    pf_off = (int64_t)h * 2 * C * 4 + (int64_t)(j - NPT * LTP) * 128;
                    pf_stride = (int64_t)Nv * 2 * C * 4;
                } else {                         // V row `row` of the chunk: token run_s + (cp - c0) C + row
                    const int jj = j - NPT * LTP - LR;
                    pf_row = jj / VL;
                    pf_base = reinterpret_cast<const char*>(v);
                    pf_off = (((run_s - (int64_t)c0 * C + pf_row) * Nv + h) * DV) * 2 + (int64_t)(jj % VL) * 128;
                    pf_stride = (int64_t)C * Nv * DV * 2;
                }
                pf_on = true;
            }
        }
        // the lane's line in chunk c0 + kAhead as an address, advanced two chunks
        // per call; only the run's last chunk can be shorter than C
        uint64_t pf_addr = (uint64_t)pf_base + (uint64_t)(pf_off + (int64_t)(c0 + kAhead) * pf_stride);
        const bool pf_last = pf_on && pf_row < chunk_L(c1 - 1);
        typedef const __attribute__((address_space(1))) float* gptr;   // global loads (not flat: no LDS counter)
        auto prefetch2 = [&](int c, float& x0, float& x1) {     // chunks c + kAhead and c + kAhead + 1
            const int cp = c + kAhead;
            if (want_pf && cp < c1 && (cp < c1 - 1 ? pf_on : pf_last)) x0 = *(gptr)pf_addr;
            if (want_pf && cp + 1 < c1 && (cp + 1 < c1 - 1 ? pf_on : pf_last))
                x1 = *(gptr)(pf_addr + (uint64_t)pf_stride);
            pf_addr += 2 * (uint64_t)pf_stride;
        };
        uint32_t pf_sum = 0;
        auto consume = [&](float x) { pf_sum ^= __float_as_uint(x); };
        VR vr;
        TR tr;
        make_pairs();
        lds_barrier();                                                            // prologue barrier
        if (c0 < c1) {
            read_ka(c0);
            vr = read_vr(c0);
            tr = read_tr(c0);
        }
        auto step = [&](int c, auto&& at_start, auto&& at_end) {
            const int s4l = slot4(c);
            const f16* Kb = Ks[s4l];
            at_start();
            // ---- region 1: S_in's pairs published; Y = K S_in (operands read in the
            //      previous step) with the reads of this chunk's K^T operands and the
            //      scaling of S by exp(G_last) interleaved
            if constexpr (want_o) {
#pragma unroll
                for (int kp = 0; kp < NKP; ++kp) *reinterpret_cast<h8*>(&Sx[(c - c0) & 1][kp][lane * 8]) = Sp[kp];
            }
            if constexpr (want_h) {
#pragma unroll
                for (int t = 0; t < NDB; ++t) *reinterpret_cast<f32x4*>(&Hx[(c - c0) & 1][t][lane * 4]) = S[t];
            }
            f32x4 Y[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) Y[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kp = 0; kp < NKP; ++kp)
#pragma unroll
                for (int b = 0; b < 4; ++b) Y[b] = mfma16(ka[b][kp], Sp[kp], Y[b]);
            const h8* tf = tr.tf;
            const f32x4* ed = tr.ed;
            // K^T for state tile t: lane (qd, j) fetches the 4 dk values from
            // 32 (t / 2) + 8 (j & 3) + 4 (t % 2) of position 16 (2 tp + hh) + 4 qd + (j >> 2);
            // the transposing read hands lane (qd, r') the values of dk row
            // srow(t, r') at positions 32 tp + m(qd, e)
            h8 kt[NDB][2];
#pragma unroll
            for (int t = 0; t < NDB; ++t) {
#pragma unroll
                for (int tp = 0; tp < 2; ++tp) {
                    s4 part[2];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int row = 16 * (2 * tp + hh) + 4 * qd + (r >> 2);
                        const int unit = 4 * (t >> 1) + (r & 3);
                        const f16* p = &Kb[row * DK + (unit ^ swz(row)) * 8 + 4 * (t & 1)];
                        part[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)p);
                    }
                    kt[t][tp] = __builtin_bit_cast(h8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
                }
            }
            const float al = tr.a0 * tr.a1;
#pragma unroll
            for (int db = 0; db < NDB; ++db) S[db] = S[db] * al;
#pragma unroll
            for (int i = 0; i < 4 * NKP; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // one product
                __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);       // three LDS reads
                __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);       // two vector ops
            }
            __builtin_amdgcn_sched_barrier(0);
            // ---- region 2: Z = V - exp(G) Y, V_new = T Z, VD = exp(G_last - G) V_new,
            //      with the next chunk's K operand read (past the sequence's last
            //      chunk it reads a stale slot and is not used)
            f32x4 Z[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const f32x4 vv = bf16x4_to_f32(vr.v[b]);
#pragma unroll
                for (int j = 0; j < 4; ++j) Z[b][j] = vv[j] - tr.eg[b][j] * Y[b][j];
            }
            const h8 zp0 = pack_pair(Z[0], Z[1]), zp1 = pack_pair(Z[2], Z[3]);
            const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
            f32x4 VN[4];
            VN[0] = mfma16(tf[0], zp0, zero4);
            VN[1] = mfma16(tf[1], zp0, zero4);
            VN[2] = mfma16(tf[3], zp1, mfma16(tf[2], zp0, zero4));
            VN[3] = mfma16(tf[5], zp1, mfma16(tf[4], zp0, zero4));
            read_ka(c + 1);
            if constexpr (want_o) {
                *reinterpret_cast<h8*>(&VNx[(c - c0) & 1][0][lane * 8]) = pack_pair(VN[0], VN[1]);
                *reinterpret_cast<h8*>(&VNx[(c - c0) & 1][1][lane * 8]) = pack_pair(VN[2], VN[3]);
            }
            if constexpr (want_h) {
#pragma unroll
                for (int b = 0; b < 4; ++b) *reinterpret_cast<f32x4*>(&VNx32[(c - c0) & 1][b][lane * 4]) = VN[b];
            }
            f32x4 VD[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) VD[b] = VN[b] * ed[b];
            const h8 vd0 = pack_pair(VD[0], VD[1]), vd1 = pack_pair(VD[2], VD[3]);
            __builtin_amdgcn_sched_barrier(0);
            // ---- region 3: S_out = exp(G_last) S_in + K^T VD, with the next chunk's
            //      V and decay rows read
#pragma unroll
            for (int t = 0; t < NDB; ++t) S[t] = mfma16(kt[t][1], vd1, mfma16(kt[t][0], vd0, S[t]));
            vr = read_vr(c + 1);
            const TR tr_next = read_tr(c + 1);
            __builtin_amdgcn_sched_barrier(0);
            make_pairs();
            tr = tr_next;
            at_end();
            lds_barrier();                                                        // end of step c
        };
        // two steps per iteration: no warm-up value is live across iterations
        const auto none = [] {};
        int c = c0;
        for (; c + 1 < c1; c += 2) {
            float x0 = 0.f, x1 = 0.f;
            step(c, [&] { prefetch2(c, x0, x1); }, none);
            step(c + 1, none, [&] { consume(x0); consume(x1); });
        }
        if (c < c1) step(c, none, none);
        pf_sink[lane] = pf_sum;
        if (STo) {
#pragma unroll
            for (int t = 0; t < NDB; ++t) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    STo[sbase + (int64_t)srow(t, j) * NC + nb * 16 + r] = S[t][j];
            }
        }
        return;
    }

    // ============================================================ helper waves
    // wavefront 1: output rows 0..31 (blocks 0, 1) and the copies of the V slice
    // and the decay rows; wavefront 2: output block 2 and the copies of K rows
    // 0..31 and T pairs 0..2; wavefront 3: output block 3 and the copies of K
    // rows 32..63 and T pairs 3..5. A
    // helper reads no LDS array it copies into (the compiler would otherwise wait
    // for the copies before each such read). Every copy is a 16-byte buffer-to-LDS load
    // of chunk c + 3 issued at the start of step c; the wave waits for the
    // previous step's copies (all of its vector memory operations issued after
    // them may still be in flight) before the step's closing barrier.
    auto helper = [&](auto nblk_t, auto role_t) {
        constexpr int NBL = decltype(nblk_t)::value;       // output row blocks of this wave
        constexpr int ROLE = decltype(role_t)::value;       // 1: V; 2: K rows 0..31; 3: K rows 32..63
        int blk[NBL];
        if constexpr (NBL == 2) {
            blk[0] = 0;
            blk[1] = 1;
        } else {
            blk[0] = wv;
        }
        const int ob = out_f32 ? 4 : 2;
        // ---- K rows of a chunk (half of the fp16 tile: DK / 16 loads) -> LDS
        auto copy_k = [&](int c) {
            const int half = wv - 2;
            const auto rk = rsrc_of(K16, (c < c1 ? (int64_t)c * Nk + kh : 0) * C * DK * 2, c < c1 ? C * DK * 2 : 0u);
#pragma unroll
            for (int i = 0; i < DK / 16; ++i) {
                const int off = (half * (DK / 16) + i) * 1024;
                buffer_to_lds16(rk, reinterpret_cast<const char*>(Ks[slot4(c)]) + off, off + lane * 16);
            }
        };
        // ---- decay rows of a chunk -> LDS (wavefront 1): one load (the rows are
        //      512 bytes; lanes 32..63 read past them and write zeros)
        auto copy_r = [&](int c) {
            const bool ok = c < c1;
            const auto rr = rsrc_of(R, (ok ? (int64_t)c * Nv + h : 0) * 2 * C * 4, ok ? 2 * C * 4 : 0u);
            buffer_to_lds16(rr, &Rs[slot4(c)][0], lane * 16);
        };
        // ---- T pairs of a chunk -> LDS: pairs 0..2 (wavefront 2) or 3..5 (wavefront 3),
        //      each into its own 1024-byte slot; a packed half pair (512 bytes)
        //      comes from lanes 0..31, and lanes 32..63 read past the buffer and
        //      write zeros to the slot's second half, which nothing reads
        auto copy_t = [&](int c) {
            const bool ok = c < c1;
            const auto rt = rsrc_of(Tf, (ok ? (int64_t)c * Nv + h : 0) * kPackedPairs * 2, ok ? kPackedPairs * 2 : 0u);
            constexpr int p0 = ROLE == 3 ? kPairs / 2 : 0;
#pragma unroll
            for (int p = p0; p < p0 + kPairs / 2; ++p) {
                const int voff = (pair_half(p) && lane >= 32) ? kPackedPairs * 2 : pair_off(p) * 2 + lane * 16;
                buffer_to_lds16(rt, &Ts[slot4(c)][p * kFrag], voff);
            }
        };
        constexpr int NDMA = ROLE == 1 ? 2 + 1 : DK / 16 + kPairs / 2;    // copies per step
        // ---- output operands: the Q rows (fp16 tile) and score pairs of chunk c,
        //      loaded in step c - 1 and used in step c + 1, when the chunk's
        //      entering state and V_new (published in step c) are in LDS
        h8 qraw[2][NBL][NKP];
        h8 praw[2][2];
        float egraw[2][NBL];                                // exp(G) of this lane's output row
        auto load_eg = [&](int c, float* dst) {
            const auto rr = rsrc_of(R, (c < c1 ? (int64_t)c * Nv + h : 0) * 2 * C * 4, c < c1 ? C * 4 : 0u);
#pragma unroll
            for (int i = 0; i < NBL; ++i)
                dst[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rr, (16 * blk[i] + r) * 4, 0, 0));
        };
        auto load_q = [&](int c, h8 (*dst)[NKP]) {
            const auto rq = rsrc_of(Q16, (c < c1 ? (int64_t)c * Nk + kh : 0) * C * DK * 2, c < c1 ? C * DK * 2 : 0u);
#pragma unroll
            for (int i = 0; i < NBL; ++i) {
                const int row = 16 * blk[i] + r;
#pragma unroll
                for (int kp = 0; kp < NKP; ++kp)
                    dst[i][kp] = __builtin_bit_cast(h8, buf_load16(rq, (row * DK + ((4 * kp + qd) ^ tile_swz<DK>(row)) * 8) * 2));
            }
        };
        // the two score pairs this wave needs: blocks 0 and 1 (pairs 0, 1) or
        // block b >= 2 (pairs 2 b - 2, 2 b - 1)
        constexpr int pbase = ROLE == 1 ? 0 : 2 * ROLE - 2;
        auto load_p = [&](int c, h8* dst) {
            const auto rp = rsrc_of(Pf, (c < c1 ? (int64_t)c * Nv + h : 0) * kPackedPairs * 2,
                                    c < c1 ? kPackedPairs * 2 : 0u);
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                dst[p] = pair_half(pbase + p) ? half_pair(buf_load8(rp, pair_off(pbase + p) * 2 + lane * 8))
                                              : __builtin_bit_cast(h8, buf_load16(rp, pair_off(pbase + p) * 2 + lane * 16));
            }
        };
        // kStates16: chunk cc's entering state (wavefronts 2, 3: state tiles of
        // their half) as H^T [dv][dk] per chunk and head, and V_new (wavefront 1)
        // as fp32 pair fragments, from LDS to global memory (stored only when cc
        // is one of this sequence's chunks)
        auto store_states = [&](int cc, auto parc) {
            constexpr int PC = decltype(parc)::value;
            if (cc < c0 || cc >= c1) return;
            const int64_t unit = ((int64_t)cc * Nv + h) * (DV / 16) + nb;
            if constexpr (ROLE == 1) {
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    *reinterpret_cast<f32x4*>(&VNout[(unit * 2 + (b >> 1)) * kFrag + lane * 8 + (b & 1) * 4]) =
                        *reinterpret_cast<const f32x4*>(&VNx32[PC][b][lane * 4]);
            } else {
                constexpr int T0 = ROLE == 2 ? 0 : NDB / 2;
                // tile t holds dk rows 32 (t / 2) + 8 qd + 4 (t % 2) + j, j = 0..3, of column 16 nb + r
                float* hc = Hout + (((int64_t)cc * Nv + h) * DV + nb * 16 + r) * DK + 8 * qd;
#pragma unroll
                for (int t = T0; t < T0 + NDB / 2; ++t)
                    *reinterpret_cast<f32x4*>(&hc[32 * (t >> 1) + 4 * (t & 1)]) =
                        *reinterpret_cast<const f32x4*>(&Hx[PC][t][lane * 4]);
            }
        };
        // O of chunk cc = scale [exp(G) (Q S_in) + P V_new], formed transposed
        // (stored only when cc is one of this sequence's chunks)
        auto finish = [&](int cc, auto parc) {
            constexpr int PC = decltype(parc)::value;       // parity of chunk cc
            const bool valid = cc >= c0 && cc < c1;
            const int64_t s = valid ? chunk_s(cc) : 0;
            const int L = valid ? chunk_L(cc) : 0;
            const auto ro = rsrc_of(o, ((s * Nv + h) * DV + nb * 16) * ob,
                                    L > 0 ? (uint32_t)(((L - 1) * Nv * DV + 16) * ob) : 0u);
            h8 sx[NKP];
#pragma unroll
            for (int kp = 0; kp < NKP; ++kp) sx[kp] = *reinterpret_cast<const h8*>(&Sx[PC][kp][lane * 8]);
            const h8 vn0 = *reinterpret_cast<const h8*>(&VNx[PC][0][lane * 8]);
            const h8 vn1 = *reinterpret_cast<const h8*>(&VNx[PC][1][lane * 8]);
#pragma unroll
            for (int i = 0; i < NBL; ++i) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kp = 0; kp < NKP; ++kp) acc = mfma16(sx[kp], qraw[PC][i][kp], acc);
                acc = acc * egraw[PC][i];
                if constexpr (NBL == 2) {
                    acc = mfma16(vn0, praw[PC][i], acc);
                } else {
                    acc = mfma16(vn1, praw[PC][1], mfma16(vn0, praw[PC][0], acc));
                }
                const f32x4 x = acc * scale;
                const int off = ((16 * blk[i] + r) * Nv * DV + 4 * qd) * ob;   // rows past the end fall outside ro
                if (out_f32) {
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, x), ro, off, 0, 0);
                } else {
                    typedef bf16 b4 __attribute__((ext_vector_type(4)));
                    const b4 y = {(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, y), ro, off, 0, 0);
                }
            }
        };
#pragma unroll
        for (int i = 0; i < NBL; ++i)
#pragma unroll
            for (int kp = 0; kp < NKP; ++kp) qraw[1][i][kp] = h8{};
        praw[1][0] = praw[1][1] = h8{};
#pragma unroll
        for (int i = 0; i < NBL; ++i) egraw[1][i] = 0.f;
        // prologue: the copies of the first three chunks landed
        auto copy = [&](int c) {
            if constexpr (ROLE == 1) {
                copy_v(c);
                copy_r(c);
            } else {
                copy_k(c);
                copy_t(c);
            }
        };
        copy(c0);
        copy(c0 + 1);
        copy(c0 + 2);
        wait_vmem();
        if constexpr (want_o) {
            load_q(c0, qraw[0]);
            load_p(c0, praw[0]);
            load_eg(c0, egraw[0]);
        }
        lds_barrier();                                                            // prologue barrier
        auto step = [&](int c, auto par) {
            constexpr int PAR = decltype(par)::value;
            copy(c + 3);
            if constexpr (want_o) {
                finish(c - 1, std::integral_constant<int, PAR ^ 1>{});
                load_p(c + 1, praw[PAR ^ 1]);
                load_q(c + 1, qraw[PAR ^ 1]);
                load_eg(c + 1, egraw[PAR ^ 1]);
            }
            if constexpr (want_h) store_states(c - 1, std::integral_constant<int, PAR ^ 1>{});
            // the copies of chunk c + 2 (issued in step c - 1) have landed
            constexpr int after = want_o ? NBL + 2 + NBL * NKP + NBL
                                         : (want_h ? (ROLE == 1 ? 4 : NDB / 2) : 0);   // operations per step after the copies
            if constexpr (NDMA > 0) wait_vmem_but<2 * after + NDMA>();
            lds_barrier();                                                        // end of step c
        };
        // both steps of a pair in the loop body on every path, so that the
        // compiler's waits for loads issued two steps earlier count both steps
        int c = c0;
        for (; c + 1 < c1; c += 2) {
            step(c, P0{});
            step(c + 1, P1{});
        }
        if (c < c1) step(c, P0{});
        if constexpr (want_o) {                             // the last chunk's output
            if (c1 > c0) {
                if ((c1 - 1 - c0) & 1) finish(c1 - 1, P1{});
                else finish(c1 - 1, P0{});
            }
        }
        if constexpr (want_h) {                             // the last chunk's states
            if (c1 > c0) {
                if ((c1 - 1 - c0) & 1) store_states(c1 - 1, P1{});
                else store_states(c1 - 1, P0{});
            }
        }
        wait_vmem();
    };
    if (wv == 1) helper(std::integral_constant<int, 2>{}, std::integral_constant<int, 1>{});
    else if (wv == 2) helper(std::integral_constant<int, 1>{}, std::integral_constant<int, 2>{});
    else helper(std::integral_constant<int, 1>{}, std::integral_constant<int, 3>{});
}

// ============================================================ launch
template <int DK, int DV>
static hipError_t launch_dims(const LaunchArgs& a, hipEvent_t* ev) {
    hipStream_t st = a.stream;
    auto mark = [&](int i) { if (ev && ev[i]) (void)hipEventRecord(ev[i], st); };
    const int32_t NT = a.nt;
    const bf16 *q = (const bf16*)a.q, *k = (const bf16*)a.k, *v = (const bf16*)a.v;
    f16* Tf = (f16*)a.T16;
    f16* Pf = (f16*)a.P16;
    float* R = a.R16;
    mark(2);
    if (NT > 0)
        k_prep<DK, true><<<dim3(NT, a.Nk), 256, 0, st>>>(k, q, a.beta, a.beta_f32, a.g, a.chunk_start, a.chunk_len,
                                                           a.Nk, a.Nv, Tf, Pf, R, (f16*)a.K16, (f16*)a.Q16);
    mark(3);
    mark(4);
    if (a.N > 0 && !a.prep_only) {
        if (a.nseg > 0) {
            k_chunk16<DK, DV, kSegment16><<<dim3(a.nseg, a.Nv, DV / 16 + DK / 16), 256, 0, st>>>(
                q, k, v, R, Tf, Pf, (const f16*)a.K16, (const f16*)a.Q16, nullptr, a.chunk_start, a.chunk_len,
                a.seg_first, a.Nk, a.Nv, a.scale, a.out_f32, nullptr, a.Sloc, a.Mseg, nullptr, nullptr);
            const hipError_t e = launch_segment_scan(a);
            if (e != hipSuccess) return e;
            k_chunk16<DK, DV, kFull16><<<dim3(a.nseg, a.Nv, DV / 16), 256, 0, st>>>(
                q, k, v, R, Tf, Pf, (const f16*)a.K16, (const f16*)a.Q16, a.Sstart, a.chunk_start, a.chunk_len,
                a.seg_first, a.Nk, a.Nv, a.scale, a.out_f32, a.o, nullptr, nullptr, nullptr, nullptr);
        } else {
            k_chunk16<DK, DV, kFull16><<<dim3(a.N, a.Nv, DV / 16), 256, 0, st>>>(
                q, k, v, R, Tf, Pf, (const f16*)a.K16, (const f16*)a.Q16, a.S0, a.chunk_start, a.chunk_len,
                a.seq_first, a.Nk, a.Nv, a.scale, a.out_f32, a.o, a.ST, nullptr, nullptr, nullptr);
        }
    }
    mark(5);
    mark(6);
    return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_states_dims(const LaunchArgs& a) {
    hipStream_t st = a.stream;
    const int32_t NT = a.nt;
    const bf16 *q = (const bf16*)a.q, *k = (const bf16*)a.k, *v = (const bf16*)a.v;
    if (NT > 0)
        k_prep<DK, false><<<dim3(NT, a.Nk), 256, 0, st>>>(k, q, a.beta, a.beta_f32, a.g, a.chunk_start, a.chunk_len,
                                                            a.Nk, a.Nv, (f16*)a.T16, (f16*)a.P16, a.R16, (f16*)a.K16,
                                                            (f16*)a.Q16);
    if (a.N > 0)
        k_chunk16<DK, DV, kStates16><<<dim3(a.N, a.Nv, DV / 16), 256, 0, st>>>(
            q, k, v, a.R16, (const f16*)a.T16, (const f16*)a.P16, (const f16*)a.K16, (const f16*)a.Q16, a.S0,
            a.chunk_start, a.chunk_len, a.seq_first, a.Nk, a.Nv, a.scale, 0, nullptr, nullptr, nullptr,
            (float*)a.H, (float*)a.VN);
    return hipGetLastError();
}

hipError_t launch_fp16_states(const LaunchArgs& a) {
#define GDR_CASE(DKv, DVv) \
    if (a.dk == DKv && a.dv == DVv) return launch_states_dims<DKv, DVv>(a);
    GDR_CASE(32, 32) GDR_CASE(32, 64) GDR_CASE(32, 128)
    GDR_CASE(64, 32) GDR_CASE(64, 64) GDR_CASE(64, 128)
    GDR_CASE(128, 32) GDR_CASE(128, 64) GDR_CASE(128, 128)
#undef GDR_CASE
    return hipErrorInvalidValue;
}

// debug copies: packed pair sets -> six 512-value fragments per set, one
// 16-byte lane unit per thread
__global__ __launch_bounds__(256) void k_unpack_pairs(const f16* __restrict__ packed, f16* __restrict__ dense,
                                                      int64_t units) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= units) return;
    const int64_t set = i / (kPairs * 64);
    const int rem = (int)(i % (kPairs * 64)), p = rem / 64, l = rem % 64;
    const f16* src = packed + set * kPackedPairs + pair_off(p);
    const u4 x = pair_half(p) ? __builtin_bit_cast(u4, half_pair(*reinterpret_cast<const u2*>(src + l * 4)))
                              : *reinterpret_cast<const u4*>(src + l * 8);
    *reinterpret_cast<u4*>(dense + (set * kPairs + p) * kFrag + l * 8) = x;
}

hipError_t unpack_pairs16(const void* packed, void* dense, int64_t sets, hipStream_t stream) {
    const int64_t units = sets * kPairs * 64;
    if (units <= 0) return hipSuccess;
    k_unpack_pairs<<<dim3((unsigned)((units + 255) / 256)), 256, 0, stream>>>((const f16*)packed, (f16*)dense, units);
    return hipGetLastError();
}

hipError_t launch_fp16_path(const LaunchArgs& a, hipEvent_t* ev) {
#define GDR_CASE(DKv, DVv) \
    if (a.dk == DKv && a.dv == DVv) return launch_dims<DKv, DVv>(a, ev);
    GDR_CASE(32, 32) GDR_CASE(32, 64) GDR_CASE(32, 128)
    GDR_CASE(64, 32) GDR_CASE(64, 64) GDR_CASE(64, 128)
    GDR_CASE(128, 32) GDR_CASE(128, 64) GDR_CASE(128, 128)
#undef GDR_CASE
    return hipErrorInvalidValue;
}

}  // namespace gdr
