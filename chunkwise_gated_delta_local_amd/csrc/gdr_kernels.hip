// HIP kernels of the chunked gated delta-rule forward for gfx950.
//
// Method (FLA DeltaNet article on pnsm.cn, sections 2.3-2.4 and 3.1-3.4;
// ChunkGatedDeltaRule math page, section 3, formulas (1)-(6)). Per chunk of
// C tokens (C = 64; the five-kernel path also takes C = 16 and 32, the chunk
// sizes the FLA article's tests sweep, section 6) and value head h (q/k head
// kh = h / (Nv/Nk)):
//   G     = chunk-local inclusive prefix sum of g                       (K1)
//   L_ij  = beta_i (k_i . k_j) exp(G_i - G_j), i > j;  A = (I + L)^-1    (K2)
//   W     = A diag(beta exp(G)) K,  U = A diag(beta) V                   (K3)
//   h_c   = S;  V_new = U - W S;
//   S    <- exp(G_last) S + (diag(exp(G_last - G)) K)^T V_new            (K4, sequential)
//   O     = scale [diag(exp(G)) Q h_c + (Q K^T (.) D) V_new],
//           D_ij = exp(G_i - G_j) for i >= j else 0                      (K5)
// Intermediates live in the caller's workspace in fragment-major layouts
// (gdr_device.hpp) chosen so that every matrix-core operand is read with
// lane-contiguous vector loads and MFMA results feed later products in place.
#include <type_traits>

#include "gdr_device.hpp"
#include "gdr_fp16.hpp"
#include "gdr_launch.hpp"

namespace gdr {

// ============================================================ chunk table
// Builds, from the sequence offsets, the list of chunks of C tokens (sequence
// id, first token, length) numbered sequence by sequence, and the first chunk
// of each sequence. One block; sequences are scanned 1024 at a time. Offsets are
// clamped to [0, Ttot] and chunk indices to the table capacity, so inconsistent
// offsets can never send a later kernel outside its buffers.
__global__ __launch_bounds__(1024) void k_chunk_table(const int32_t* __restrict__ cu, int64_t T_row,
                                                       int32_t N, int64_t Ttot, int32_t cap, int32_t C,
                                                       int32_t* __restrict__ chunk_seq,
                                                       int32_t* __restrict__ chunk_start,
                                                       int32_t* __restrict__ chunk_len,
                                                       int32_t* __restrict__ seq_first) {
    __shared__ int32_t scan[1024];
    const int tid = threadIdx.x;
    for (int32_t c = tid; c < cap; c += 1024) {       // entries no sequence reaches stay empty
        chunk_seq[c] = 0;
        chunk_start[c] = 0;
        chunk_len[c] = 0;
    }
    __syncthreads();
    int32_t base = 0;
    for (int32_t n0 = 0; n0 < N; n0 += 1024) {
        const int32_t n = n0 + tid;
        int64_t s = 0, e = 0;
        if (n < N) {
            s = cu ? (int64_t)cu[n] : (int64_t)n * T_row;
            e = cu ? (int64_t)cu[n + 1] : (int64_t)(n + 1) * T_row;
            s = s < 0 ? 0 : (s > Ttot ? Ttot : s);
            e = e < s ? s : (e > Ttot ? Ttot : e);
        }
        const int32_t nch = (int32_t)((e - s + C - 1) / C);
        scan[tid] = nch;   // chunks of sequence n
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {         // inclusive Hillis-Steele scan
            int32_t add = tid >= off ? scan[tid - off] : 0;
            __syncthreads();
            scan[tid] += add;
            __syncthreads();
        }
        const int32_t first = base + scan[tid] - nch;
        if (n < N) seq_first[n] = first < cap ? first : cap;
        base += scan[1023];
        __syncthreads();
    }
    if (tid == 0) seq_first[N] = base < cap ? base : cap;
    __syncthreads();
    // Entries: chunk c belongs to the last sequence whose first chunk is <= c.
    const int32_t total = base < cap ? base : cap;
    for (int32_t c = tid; c < total; c += 1024) {
        int32_t lo = 0, hi = N - 1;                       // seq_first is non-decreasing
        while (lo < hi) {
            const int32_t mid = (lo + hi + 1) >> 1;
            if (seq_first[mid] <= c) lo = mid; else hi = mid - 1;
        }
        const int32_t n = lo;
        int64_t s = cu ? (int64_t)cu[n] : (int64_t)n * T_row;
        int64_t e = cu ? (int64_t)cu[n + 1] : (int64_t)(n + 1) * T_row;
        s = s < 0 ? 0 : (s > Ttot ? Ttot : s);
        e = e < s ? s : (e > Ttot ? Ttot : e);
        const int64_t cs = s + (int64_t)(c - seq_first[n]) * C;
        const int64_t ce = cs + C < e ? cs + C : e;
        const bool empty = !(ce > cs);
        chunk_seq[c] = n;
        chunk_start[c] = empty ? 0 : (int32_t)cs;          // empty entries point at token 0
        chunk_len[c] = empty ? 0 : (int32_t)(ce - cs);
    }
}

// ============================================================ K1: gate prefix sums
// G[t, h] = sum of g over the tokens of t's chunk up to and including t, in
// fp32 (ChunkGatedDeltaRule page, section 3, "G_i"; GLA notes, forward step 1,
// chunk-local cumulative log gate). One workgroup per (chunk, 256 / C heads):
// lane i of each C-lane group takes position i of one head, and the prefix sum
// runs across the group with shuffles (log2 C steps, always in the same
// order). g == NULL writes zeros (ungated rule).
template <int C>
__global__ __launch_bounds__(256) void k_gate_cumsum(const float* __restrict__ g,
                                                      const int32_t* __restrict__ chunk_start,
                                                      const int32_t* __restrict__ chunk_len,
                                                      int32_t NT, int32_t Nv, float* __restrict__ G) {
    constexpr int HB = 256 / C;                   // heads per workgroup
    const int c = blockIdx.x;
    const int i = threadIdx.x % C, h = blockIdx.y * HB + threadIdx.x / C;
    const bool on = h < Nv;
    const int64_t s = chunk_start[c];
    const int L = chunk_len[c];
    float x = (g && on && i < L) ? g[(s + i) * Nv + h] : 0.f;
#pragma unroll
    for (int off = 1; off < C; off <<= 1) {       // inclusive scan over the group (every lane takes part)
        const float y = __shfl_up(x, off, C);
        if (i >= off) x += y;
    }
    if (on && i < L) G[(s + i) * Nv + h] = x;
}

// ============================================================ K2: A-build + solve
// One workgroup (C/16 wavefronts) per (chunk, q/k head); it serves the Nv/Nk
// value heads that share the key head, computing K K^T once (FLA DeltaNet
// article, section 3.1: beta-scaled K K^T, strictly lower part).
//   1. K chunk -> LDS; wave w forms the K K^T tiles of block row w on MFMA.
//   2. Per value head: L = tril(beta_i (k_i.k_j) exp(G_i - G_j), -1) -> LDS (fp32).
//   3. The C/16 16x16 diagonal blocks of A = (I + L)^-1 by forward substitution
//      in fp32, one column per lane (ChunkGatedDeltaRule page, section 3.1,
//      row-recursive correction; FLA DeltaNet article, section 3.2, 16x16
//      blocks).
//   4. Off-diagonal blocks by block substitution on MFMA, merging
//      16 -> 32 -> 64 as far as C reaches (FLA DeltaNet article, section 3.2):
//        A_ij = -A_ii L_ij A_jj for the two 16-blocks below the diagonal of each
//        32-block, then the lower-left 32x32 block = -A_bot L_bl A_top.
//      Both operands are derived values, so each product takes the split
//      (three-pass) form.
//   5. A rows (fp32) -> global, zero above the diagonal and past the chunk end.
template <typename T, int DK, int C>
__global__ __launch_bounds__(256, 4) void k_build_solve(const T* __restrict__ k,
                                                         const void* __restrict__ beta, int beta_f32,
                                                         const float* __restrict__ G,
                                                         const int32_t* __restrict__ chunk_start,
                                                         const int32_t* __restrict__ chunk_len,
                                                         int32_t Nk, int32_t Nv, float* __restrict__ A_out) {
    static_assert(C == 16 || C == 32 || C == 64, "chunk size");
    constexpr int NTB = C / 16;                // 16-row blocks of the chunk, one wavefront each
    constexpr int NTHR = 64 * NTB;
    constexpr int KP = DK + 8;                 // padded LDS row (elements)
    constexpr int SEGS = C * (DK / 8) / NTHR;  // 16-byte row segments per thread
    // The K tile is only needed until the K K^T tiles are in registers; L and A
    // reuse its LDS afterwards.
    constexpr int TILE_BYTES = C * KP * (int)sizeof(T);
    constexpr int LP = C + 4;                  // L and A row pitch (floats): 16-byte aligned rows
    constexpr int LA_BYTES = 2 * C * LP * 4;
    __shared__ __attribute__((aligned(16))) char smem[TILE_BYTES > LA_BYTES ? TILE_BYTES : LA_BYTES];
    __shared__ __attribute__((aligned(16))) float bs[C], gs[C];
    T* Ks = reinterpret_cast<T*>(smem);
    float (*Lf)[LP] = reinterpret_cast<float (*)[LP]>(smem);
    float (*Af)[LP] = Lf + C;

    const int c = blockIdx.x, kh = blockIdx.y;
    const int64_t s = chunk_start[c];
    const int L = chunk_len[c];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 15, qd = lane >> 4;
    typedef typename Vec<T>::v8 v8;

    const int group = Nv / Nk;
    // beta and G of a value head go through registers: head 0's are fetched with
    // the tiles, each next head's while the current one is processed
    float b_nx = 0.f, g_nx = 0.f;
    auto fetch_gates = [&](int hh) {
        const int h = kh * group + hh;
        if (tid < C && tid < L) {
            b_nx = load_beta(beta, (s + tid) * Nv + h, beta_f32);
            g_nx = G[(s + tid) * Nv + h];
        } else {
            b_nx = 0.f;
            g_nx = 0.f;
        }
    };

    // 1. K rows of the chunk (zero past the chunk end): all loads first
    {
        v8 kv[SEGS];
#pragma unroll
        for (int i = 0; i < SEGS; ++i) {
            const int idx = tid + NTHR * i, row = idx / (DK / 8), seg = idx % (DK / 8);
            kv[i] = zero_pair<T>();
            if (row < L) kv[i] = *reinterpret_cast<const v8*>(k + ((s + row) * Nk + kh) * DK + seg * 8);
        }
        fetch_gates(0);
#pragma unroll
        for (int i = 0; i < SEGS; ++i) {
            const int idx = tid + NTHR * i, row = idx / (DK / 8), seg = idx % (DK / 8);
            *reinterpret_cast<v8*>(&Ks[row * KP + seg * 8]) = kv[i];
        }
    }
    __syncthreads();

    // K K^T tiles of block row `wave`: kk[j] holds rows 16*wave + 4*qd + jj, column 16*j + r.
    f32x4 kk[NTB];
#pragma unroll
    for (int j = 0; j < NTB; ++j) {
        kk[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (j <= wave) {
#pragma unroll
            for (int kp = 0; kp < DK / 32; ++kp) {
                v8 a = load_pair_row<T>(&Ks[(wave * 16 + r) * KP + kp * 32], qd);
                v8 b = load_pair_row<T>(&Ks[(j * 16 + r) * KP + kp * 32], qd);
                kk[j] = mfma_pair(a, b, kk[j]);
            }
        }
    }
    __syncthreads();                           // tiles consumed: the LDS now holds L and A
    // the two strictly-upper 16x16 blocks of A that the block merges read are zero
    for (int idx = tid; idx < (NTB / 2) * 256; idx += NTHR) {
        const int blk = idx >> 8, e = idx & 255, row = blk * 32 + (e >> 4), col = blk * 32 + 16 + (e & 15);
        Af[row][col] = 0.f;
    }

    for (int hh = 0; hh < group; ++hh) {
        const int h = kh * group + hh;
        if (tid < C) {
            bs[tid] = b_nx;
            gs[tid] = g_nx;
        }
        __syncthreads();
        if (hh + 1 < group) fetch_gates(hh + 1);

        // 2. strictly lower L (every entry of the blocks on and below the diagonal)
#pragma unroll
        for (int j = 0; j < NTB; ++j) {
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
        __syncthreads();

        // 3. diagonal block `wave`: lane r < 16 owns column r of the block. Each
        //    substitution step reads row i of the block's L with LDS reads whose
        //    address is the same in every lane (broadcast, no bank conflicts),
        //    so the recursion spends its vector instructions on the FMAs only.
        {
            const int b0 = wave * 16;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = (i == lane) ? 1.f : 0.f;
#pragma unroll
            for (int i = 1; i < 16; ++i) {
                const float* lr = &Lf[b0 + i][b0];     // the same address in every lane: broadcast reads
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
        __syncthreads();

        // 4a. A_ij = -A_ii (L_ij A_jj) for (i, j) = (1, 0) [wave 0] and (3, 2) [wave 1];
        //     contraction depth 16: pair elements 4..7 are zero.
        if (wave < NTB / 2) {
            const int bi = 2 * wave + 1, bj = 2 * wave;
            float la[8], db[8], ai[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                la[e] = Lf[bi * 16 + r][bj * 16 + 4 * qd + e];
                db[e] = Af[bj * 16 + 4 * qd + e][bj * 16 + r];
                ai[e] = Af[bi * 16 + r][bi * 16 + 4 * qd + e];
                la[4 + e] = db[4 + e] = ai[4 + e] = 0.f;
            }
            f32x4 t1 = mfma_dd<T>(split8<T>(la), split8<T>(db), f32x4{0.f, 0.f, 0.f, 0.f});   // L_ij A_jj
            f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
            f32x4 t2 = mfma_dd<T>(split8<T>(ai), split_acc_pair<T>(t1, zero4), zero4);          // A_ii (L_ij A_jj)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) Af[bi * 16 + 4 * qd + jj][bj * 16 + r] = -t2[jj];
        }
        __syncthreads();

        // 4b. lower-left 32x32 block = -A_bot (L_bl A_top); wave w < 2 takes column block w.
        if constexpr (C == 64) {
            if (wave < 2) {
                const int ct = wave;
                float bt[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bt[e] = Af[4 * qd + e][ct * 16 + r];
                    bt[4 + e] = Af[16 + 4 * qd + e][ct * 16 + r];
                }
                const Split<T> b = split8<T>(bt);
                f32x4 t1[2];
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
                    t1[rb] = mfma_dd<T>(load_split_row<T>(&Lf[32 + 16 * rb + r][0], qd), b, f32x4{0.f, 0.f, 0.f, 0.f});
                const Split<T> b2 = split_acc_pair<T>(t1[0], t1[1]);
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    f32x4 t2 = mfma_dd<T>(load_split_row<T>(&Af[32 + 16 * rb + r][32], qd), b2, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) Af[32 + 16 * rb + 4 * qd + jj][ct * 16 + r] = -t2[jj];
                }
            }
        }
        __syncthreads();

        // 5. rows of A for the valid tokens (fp32)
        for (int idx = tid; A_out && idx < C * (C / 4); idx += NTHR) {
            const int row = idx / (C / 4), seg = idx % (C / 4);
            if (row < L) {
                f32x4 val;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int col = seg * 4 + e;
                    val[e] = (col <= row) ? Af[row][col] : 0.f;
                }
                *reinterpret_cast<f32x4*>(A_out + ((s + row) * Nv + h) * C + seg * 4) = val;
            }
        }
        __syncthreads();
    }
}

// ============================================================ K3: w/u products
// One workgroup (C/16 wavefronts) per (chunk, q/k head). Formulas (1) and (2) of
// the ChunkGatedDeltaRule page (FLA DeltaNet article, section 3.3, where
// diag(beta) is absorbed into one operand):
//   W = (A diag(beta exp(G))) K  -> stored as W^T tiles, which in accumulator
//       layout are exactly the pair fragments the state pass reads;
//   U = (A diag(beta)) V         -> stored as accumulator tiles.
// The scaled A rows are derived (split operands); K and V are exact inputs.
// K^T and V^T are staged in LDS so that the contraction over chunk positions
// reads contiguous LDS rows; the key head's K^T is also written out once, as
// pair fragments, for the state pass. W and U are stored in fp32.
// Wavefront w owns chunk positions 16w..16w+15 (C / 16 wavefronts). Products
// over positions take them in 32-position pairs; for C = 16 the second half
// of the one pair is zero.
template <typename T, int DK, int DV, int C>
__global__ __launch_bounds__(256) void k_wu(const T* __restrict__ k, const T* __restrict__ v,
                                             const void* __restrict__ beta, int beta_f32,
                                             const float* __restrict__ G, const float* __restrict__ A,
                                             const int32_t* __restrict__ chunk_start,
                                             const int32_t* __restrict__ chunk_len, int32_t Nk, int32_t Nv,
                                             float* __restrict__ Wf, float* __restrict__ Uf, T* __restrict__ KTf,
                                             int w_only) {
    constexpr int NTB = C / 16, NTHR = 64 * NTB;
    constexpr int CP = C < 32 ? 32 : C;        // positions padded to whole pairs
    constexpr int NTP = CP / 32;
    constexpr int MP = CP + 8;                 // padded LDS row over chunk positions
    __shared__ __attribute__((aligned(16))) T KTs[DK * MP];
    __shared__ __attribute__((aligned(16))) T VTs[DV * MP];
    __shared__ float bs[CP], sc[CP];

    const int c = blockIdx.x, kh = blockIdx.y;
    const int64_t s = chunk_start[c];
    const int L = chunk_len[c];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 15, qd = lane >> 4;
    typedef typename Vec<T>::v8 v8;

    // K^T of the chunk (zero past the chunk end); consecutive threads take consecutive positions.
    for (int idx = tid; idx < CP * (DK / 8); idx += NTHR) {
        const int m = idx % CP, seg = idx / CP;
        v8 val = zero_pair<T>();
        if (m < L) val = *reinterpret_cast<const v8*>(k + ((s + m) * Nk + kh) * DK + seg * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) KTs[(seg * 8 + e) * MP + m] = val[e];
    }
    __syncthreads();

    // K^T pair fragments for the state pass: [c][kh][db][tp] (w_only: W alone is wanted)
    for (int f = wave; f < (w_only ? 0 : (DK / 16) * NTP); f += NTB) {
        const int db = f / NTP, tp = f % NTP;
        v8 val = load_pair_row<T>(&KTs[(db * 16 + r) * MP + tp * 32], qd);
        store_frag<T>(KTf + (((int64_t)c * Nk + kh) * (DK / 16) * NTP + f) * 512, lane, val);
    }

    const int group = Nv / Nk;
    const int tb = wave;                       // wave w owns chunk positions 16w..16w+15
    const int i = tb * 16 + r;
    for (int hh = 0; hh < group; ++hh) {
        const int h = kh * group + hh;
        __syncthreads();                       // previous head's readers are done with VTs / sc
        if (tid < CP) {
            const float bm = tid < L ? load_beta(beta, (s + tid) * Nv + h, beta_f32) : 0.f;
            bs[tid] = bm;
            sc[tid] = tid < L ? bm * __expf(G[(s + tid) * Nv + h]) : 0.f;
        }
        for (int idx = tid; idx < (w_only ? 0 : CP * (DV / 8)); idx += NTHR) {
            const int m = idx % CP, seg = idx / CP;
            v8 val = zero_pair<T>();
            if (m < L) val = *reinterpret_cast<const v8*>(v + ((s + m) * Nv + h) * DV + seg * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) VTs[(seg * 8 + e) * MP + m] = val[e];
        }
        __syncthreads();

        // Row i of A over positions m, scaled by beta_m (for U) and beta_m exp(G_m) (for W).
        Split<T> aU[NTP], aW[NTP];
#pragma unroll
        for (int tp = 0; tp < NTP; ++tp) {
            float xa[8], xu[8], xw[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) xa[e] = 0.f;
            if (i < L) {
                const float* row = A + ((s + i) * Nv + h) * C + tp * 32;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    xa[e] = row[4 * qd + e];
                    if (C > 16) xa[4 + e] = row[16 + 4 * qd + e];
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int m = tp * 32 + (e < 4 ? 4 * qd + e : 16 + 4 * qd + e - 4);
                xu[e] = xa[e] * bs[m];
                xw[e] = xa[e] * sc[m];
            }
            aU[tp] = split8<T>(xu);
            aW[tp] = split8<T>(xw);
        }
        // W^T tiles (db, tb): rows dk, columns i
#pragma unroll
        for (int db = 0; db < DK / 16; ++db) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int tp = 0; tp < NTP; ++tp)
                acc = mfma_xd<T>(load_pair_row<T>(&KTs[(db * 16 + r) * MP + tp * 32], qd), aW[tp], acc);
            float* dst = Wf + ((((int64_t)c * Nv + h) * NTB + tb) * (DK / 32) + (db >> 1)) * 512;
            store_pair_half_f32(dst, lane, db & 1, acc);
        }
        // U tiles (tb, nb): rows i, columns dv
        if (w_only) continue;
#pragma unroll
        for (int nb = 0; nb < DV / 16; ++nb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int tp = 0; tp < NTP; ++tp)
                acc = mfma_dx<T>(aU[tp], load_pair_row<T>(&VTs[(nb * 16 + r) * MP + tp * 32], qd), acc);
            store_tile_f32(Uf + ((((int64_t)c * Nv + h) * NTB + tb) * (DV / 16) + nb) * 256, lane, acc);
        }
    }
}

// ============================================================ K4: state pass
// One wavefront per (sequence, value head, 16 columns of dv); it keeps its
// dk x 16 slice of the state in fp32 accumulator registers for the whole
// sequence and walks the chunks in order (FLA DeltaNet article, section 3.4,
// chunk-serial state update; ChunkGatedDeltaRule page, formulas (3) and (6)):
//   H     <- S (the state entering the chunk, fp32, for the output kernel)
//   V_new  = U - W S
//   S      = exp(G_last) S + K^T diag(exp(G_last - G)) V_new
// S in accumulator layout is already the pair-fragment operand of W S, and
// V_new in accumulator layout is already the operand of K^T V_new.
// For segment-parallel state passing: the state may start as I
// (init_identity; the grid then covers dk columns), U == NULL stands for
// U = 0, and H and V_new are written only when their pointers are given.
template <typename T, int DK, int DV, int C>
__global__ __launch_bounds__(64) void k_state(const float* __restrict__ Wf, const float* __restrict__ Uf,
                                               const T* __restrict__ KTf, const float* __restrict__ G,
                                               const float* __restrict__ S0, int init_identity,
                                               const int32_t* __restrict__ chunk_start,
                                               const int32_t* __restrict__ chunk_len,
                                               const int32_t* __restrict__ seq_first, int32_t Nk, int32_t Nv,
                                               float* __restrict__ Hf, float* __restrict__ VNf, float* __restrict__ ST) {
    constexpr int NDB = DK / 16, NKP = DK / 32, NNB = DV / 16;
    constexpr int NTB = C / 16, NTP = C < 32 ? 1 : C / 32;   // 16-row blocks, 32-position pairs
    const int n = blockIdx.x, h = blockIdx.y, nb = blockIdx.z;
    const int lane = threadIdx.x, r = lane & 15, qd = lane >> 4;
    const int kh = h / (Nv / Nk);
    typedef typename Vec<float>::v8 f8;

    f32x4 S[NDB];
    const int64_t sbase = ((int64_t)n * Nv + h) * DK * DV;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = db * 16 + 4 * qd + j, col = nb * 16 + r;
            S[db][j] = init_identity ? (row == col ? 1.f : 0.f) : S0 ? S0[sbase + (int64_t)row * DV + col] : 0.f;
        }

    const int c0 = seq_first[n], c1 = seq_first[n + 1];
    for (int c = c0; c < c1; ++c) {
        const int64_t s = chunk_start[c];
        const int L = chunk_len[c];
        if (L <= 0) continue;
        const float g_last = G[(s + L - 1) * Nv + h];

        // state entering the chunk, stored in fp32 and split for the products
        Split<T> sb[NKP];
        float* hdst = Hf + (((int64_t)c * Nv + h) * NNB + nb) * NKP * 512;
#pragma unroll
        for (int kp = 0; kp < NKP; ++kp) {
            f8 raw = __builtin_shufflevector(S[2 * kp], S[2 * kp + 1], 0, 1, 2, 3, 4, 5, 6, 7);
            if (Hf) store_frag_f32(hdst + kp * 512, lane, raw);
            sb[kp] = split_acc_pair<T>(S[2 * kp], S[2 * kp + 1]);
        }

        // V_new = U - W S for the blocks of 16 chunk positions (zero in the padding of C = 16)
        f32x4 vn[2 * NTP];
        const float* wsrc = Wf + ((int64_t)c * Nv + h) * NTB * NKP * 512;
        const float* usrc = Uf + ((int64_t)c * Nv + h) * NTB * NNB * 256;
#pragma unroll
        for (int tb = NTB; tb < 2 * NTP; ++tb) vn[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kp = 0; kp < NKP; ++kp)
                x = mfma_dd<T>(split_v8<T>(load_frag_f32(wsrc + (tb * NKP + kp) * 512, lane)), sb[kp], x);
            vn[tb] = (Uf ? load_tile_f32(usrc + (tb * NNB + nb) * 256, lane) : f32x4{0.f, 0.f, 0.f, 0.f}) - x;
        }
        float* vdst = VNf + (((int64_t)c * Nv + h) * NNB + nb) * NTP * 512;
#pragma unroll
        for (int tb = 0; tb < 2 * NTP && VNf; ++tb)
            store_pair_half_f32(vdst + (tb >> 1) * 512, lane, tb & 1, vn[tb]);

        // decay each position to the chunk end; positions past the end contribute nothing
        f32x4 vd[2 * NTP];
#pragma unroll
        for (int tb = 0; tb < 2 * NTP; ++tb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = tb * 16 + 4 * qd + j;
                vd[tb][j] = row < L ? vn[tb][j] * __expf(g_last - G[(s + row) * Nv + h]) : 0.f;
            }
        Split<T> vb[NTP];
#pragma unroll
        for (int tp = 0; tp < NTP; ++tp) vb[tp] = split_acc_pair<T>(vd[2 * tp], vd[2 * tp + 1]);

        const float a_last = __expf(g_last);
        const T* ksrc = KTf + ((int64_t)c * Nk + kh) * NDB * NTP * 512;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            f32x4 acc = S[db] * a_last;
#pragma unroll
            for (int tp = 0; tp < NTP; ++tp)
                acc = mfma_xd<T>(load_frag<T>(ksrc + (db * NTP + tp) * 512, lane), vb[tp], acc);
            S[db] = acc;
        }
    }
    if (ST) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) ST[sbase + (int64_t)(db * 16 + 4 * qd + j) * DV + nb * 16 + r] = S[db][j];
    }
}

// ============================================================ K5: output
// One workgroup (C/16 wavefronts) per (chunk, value head); wave w produces the
// output rows 16w..16w+15 for all dv (ChunkGatedDeltaRule page, formulas (4)
// and (5); FLA DeltaNet article, section 3.4 "chunk_fwd_o"):
//   O = scale [ diag(exp(G)) Q H + (Q K^T (.) D) V_new ],  D_ij = exp(G_i - G_j), j <= i.
// The score block is formed transposed (K Q^T) so that its accumulator tiles
// are the pair-fragment operand of the product with V_new; the upper
// triangle and positions past the chunk end are masked explicitly.
template <typename T, int DK, int DV, int C>
__global__ __launch_bounds__(256) void k_output(const T* __restrict__ q, const T* __restrict__ k,
                                                 const float* __restrict__ G, const float* __restrict__ Hf,
                                                 const float* __restrict__ VNf, const int32_t* __restrict__ chunk_start,
                                                 const int32_t* __restrict__ chunk_len, int32_t Nk, int32_t Nv,
                                                 float scale, int out_f32, void* __restrict__ o) {
    constexpr int NKP = DK / 32, NNB = DV / 16;
    constexpr int NTB = C / 16, NTP = C < 32 ? 1 : C / 32;   // wavefronts (16-row blocks), 32-position pairs
    const int c = blockIdx.x, h = blockIdx.y;
    const int64_t s = chunk_start[c];
    const int L = chunk_len[c];
    const int tid = threadIdx.x, tb = tid >> 6, lane = tid & 63, r = lane & 15, qd = lane >> 4;
    if (tb * 16 >= L) return;                  // no valid rows in this wave's block
    const int kh = h / (Nv / Nk);
    typedef typename Vec<T>::v8 v8;

    // Q rows 16*tb + r as pair fragments over dk (zero past the chunk end)
    const int i = tb * 16 + r;
    v8 qf[NKP];
#pragma unroll
    for (int kp = 0; kp < NKP; ++kp) {
        qf[kp] = zero_pair<T>();
        if (i < L) qf[kp] = load_pair_row<T>(q + ((s + i) * Nk + kh) * DK + kp * 32, qd);
    }
    const float g_i = i < L ? G[(s + i) * Nv + h] : 0.f;
    float g_rows[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = tb * 16 + 4 * qd + j;
        g_rows[j] = row < L ? G[(s + row) * Nv + h] : 0.f;
    }

    // inter-chunk part: Q H, rows scaled by exp(G_i)
    f32x4 out[NNB];
    const float* hsrc = Hf + ((int64_t)c * Nv + h) * NNB * NKP * 512;
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kp = 0; kp < NKP; ++kp)
            acc = mfma_xd<T>(qf[kp], split_v8<T>(load_frag_f32(hsrc + (nb * NKP + kp) * 512, lane)), acc);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] *= __expf(g_rows[j]);
        out[nb] = acc;
    }

    // scores, transposed: pt[tj] rows j = 16*tj + 4*qd + jj, column i
    f32x4 pt[2 * NTP];
#pragma unroll
    for (int tj = 0; tj < 2 * NTP; ++tj) {
        pt[tj] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (tj < NTB && tj <= tb) {
            const int jr = tj * 16 + r;
#pragma unroll
            for (int kp = 0; kp < NKP; ++kp) {
                v8 kf = zero_pair<T>();
                if (jr < L) kf = load_pair_row<T>(k + ((s + jr) * Nk + kh) * DK + kp * 32, qd);
                pt[tj] = mfma_pair(kf, qf[kp], pt[tj]);
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int j = tj * 16 + 4 * qd + jj;
                float gj = j < L ? G[(s + j) * Nv + h] : 0.f;
                pt[tj][jj] = (j <= i && i < L) ? pt[tj][jj] * __expf(g_i - gj) : 0.f;
            }
        }
    }
    Split<T> pa[NTP];
#pragma unroll
    for (int tp = 0; tp < NTP; ++tp) pa[tp] = split_acc_pair<T>(pt[2 * tp], pt[2 * tp + 1]);

    // intra-chunk part: (Q K^T (.) D) V_new
    const float* vsrc = VNf + ((int64_t)c * Nv + h) * NNB * NTP * 512;
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) {
#pragma unroll
        for (int tp = 0; tp < NTP; ++tp)
            if (2 * tp <= tb)
                out[nb] = mfma_dd<T>(pa[tp], split_v8<T>(load_frag_f32(vsrc + (nb * NTP + tp) * 512, lane)), out[nb]);
    }

#pragma unroll
    for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = tb * 16 + 4 * qd + j;
            if (row < L) {
                const int64_t idx = ((s + row) * Nv + h) * DV + nb * 16 + r;
                if (out_f32) reinterpret_cast<float*>(o)[idx] = scale * out[nb][j];
                else reinterpret_cast<T*>(o)[idx] = to_t<T>(scale * out[nb][j]);
            }
        }
}

// ============================================================ K4 + K5 fused: state pass with output
// ============================================================ segment-parallel state passing
// The state recursion is affine in the state: over any run of chunks,
//   S_end = M S_start + S_loc,
// where S_loc is the end state reached from a zero state and M (dk x dk) is the
// end state reached from S_start = I with V = 0 (the per-chunk map
// S -> exp(G_last) S + K^T diag(exp(G_last - G)) T (V - diag(exp(G)) K S),
// ChunkGatedDeltaRule page formulas (3) and (6), composed over the run). So a
// long sequence can be cut into segments of whole chunks whose local states and
// transitions are formed side by side; one short scan over the segments then
// gives each segment's true entering state, and a last pass from those states
// writes the output (FLA DeltaNet article, section 2.4: the chunk states form
// a linear recurrence, here composed segment by segment instead of chunk by
// chunk).
//
// Segment table: segment j of the batch covers chunks seg_first[j] ..
// seg_first[j + 1] - 1, at most `seg_chunks` consecutive chunks of one
// sequence; seq_seg[n] is the first segment of sequence n (seq_seg[N] = the
// segment count). Entries are clamped to the capacity `cap` sized on the host,
// and entries no sequence reaches are empty, so a table built from offsets
// that disagree with the host's copy still stays inside every buffer.
__global__ __launch_bounds__(1024) void k_segment_table(const int32_t* __restrict__ seq_first, int32_t N,
                                                         int32_t seg_chunks, int32_t cap,
                                                         int32_t* __restrict__ seg_first,
                                                         int32_t* __restrict__ seq_seg) {
    __shared__ int32_t scan[1024];
    const int tid = threadIdx.x;
    const int32_t end = seq_first[N];
    for (int32_t j = tid; j <= cap; j += 1024) seg_first[j] = end;
    __syncthreads();
    int32_t base = 0;
    for (int32_t n0 = 0; n0 < N; n0 += 1024) {
        const int32_t n = n0 + tid;
        const int32_t f = n < N ? seq_first[n] : 0;
        const int32_t nch = n < N ? seq_first[n + 1] - f : 0;
        const int32_t nseg = (nch + seg_chunks - 1) / seg_chunks;
        scan[tid] = nseg;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {         // inclusive Hillis-Steele scan
            int32_t add = tid >= off ? scan[tid - off] : 0;
            __syncthreads();
            scan[tid] += add;
            __syncthreads();
        }
        const int32_t first = base + scan[tid] - nseg;
        if (n < N) {
            seq_seg[n] = first < cap ? first : cap;
            for (int32_t i = 0; i < nseg && first + i < cap; ++i) seg_first[first + i] = f + i * seg_chunks;
            // the sequence that holds the last kept segment ends it: when the
            // offsets give more segments than the capacity, that segment takes
            // the rest of its own sequence and never runs into the next one
            if (first < cap && first + nseg >= cap) seg_first[cap] = f + nch;
        }
        base += scan[1023];
        __syncthreads();
    }
    if (tid == 0) seq_seg[N] = base < cap ? base : cap;
}

// Scan over the segments of each sequence, per (sequence, value head, 16
// columns of dv): S = S0; for each segment j in order, S_start[j] = S, then
// S = M_j S + S_loc[j]; the last S is the sequence's final state. fp32 FMA
// throughout. Thread u < 2 dk owns row u / 2 and columns 8 (u % 2) .. + 7 of
// the slice; the slice itself sits in LDS, so every step reads the rows of M_j
// from memory once and the slice as LDS broadcasts.
// Layouts: S_loc, S_start [segments][Nv][dk][dv], M [segments][Nv][dk][dk],
// S0 and ST [N][Nv][dk][dv], all fp32.
template <int DK, int DV>
__global__ __launch_bounds__(256) void k_segment_scan(const int32_t* __restrict__ seq_seg,
                                                       const float* __restrict__ S0, const float* __restrict__ Sloc,
                                                       const float* __restrict__ M, int32_t Nv,
                                                       float* __restrict__ Sstart, float* __restrict__ ST) {
    static_assert(2 * DK <= 256, "one row half per thread");
    __shared__ __attribute__((aligned(16))) float Ss[DK][16];
    const int n = blockIdx.x, h = blockIdx.y, nb = blockIdx.z;
    const int tid = threadIdx.x;
    const bool own = tid < 2 * DK;
    const int i = tid >> 1, c8 = 8 * (tid & 1);
    const int64_t col = (int64_t)nb * 16 + c8;
    f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = x0;
    if (own && S0) {
        const float* src = S0 + (((int64_t)n * Nv + h) * DK + i) * DV + col;
        x0 = *reinterpret_cast<const f32x4*>(src);
        x1 = *reinterpret_cast<const f32x4*>(src + 4);
    }
    const int32_t j0 = seq_seg[n], j1 = seq_seg[n + 1];
    for (int32_t j = j0; j < j1; ++j) {
        const int64_t sb = (((int64_t)j * Nv + h) * DK + i) * DV + col;
        if (own) {
            *reinterpret_cast<f32x4*>(&Ss[i][c8]) = x0;
            *reinterpret_cast<f32x4*>(&Ss[i][c8 + 4]) = x1;
            *reinterpret_cast<f32x4*>(Sstart + sb) = x0;
            *reinterpret_cast<f32x4*>(Sstart + sb + 4) = x1;
        }
        __syncthreads();
        if (own) {
            x0 = *reinterpret_cast<const f32x4*>(Sloc + sb);
            x1 = *reinterpret_cast<const f32x4*>(Sloc + sb + 4);
            const float* mrow = M + (((int64_t)j * Nv + h) * DK + i) * DK;
#pragma unroll 4
            for (int m4 = 0; m4 < DK; m4 += 4) {
                const f32x4 mv = *reinterpret_cast<const f32x4*>(mrow + m4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const f32x4 s0 = *reinterpret_cast<const f32x4*>(&Ss[m4 + e][c8]);
                    const f32x4 s1 = *reinterpret_cast<const f32x4*>(&Ss[m4 + e][c8 + 4]);
                    x0 += mv[e] * s0;
                    x1 += mv[e] * s1;
                }
            }
        }
        __syncthreads();                         // the slice is read before it is overwritten
    }
    if (own && ST) {
        float* dst = ST + (((int64_t)n * Nv + h) * DK + i) * DV + col;
        *reinterpret_cast<f32x4*>(dst) = x0;
        *reinterpret_cast<f32x4*>(dst + 4) = x1;
    }
}

// ============================================================ launchers
template <int DK, int DV>
static hipError_t scan_dims(const LaunchArgs& a) {
    k_segment_scan<DK, DV><<<dim3(a.N, a.Nv, DV / 16), 256, 0, a.stream>>>(a.seq_seg, a.S0, a.Sloc, a.Mseg, a.Nv,
                                                                       a.Sstart, a.ST);
    return hipGetLastError();
}

hipError_t launch_segment_scan(const LaunchArgs& a) {
#define GDR_CASE(DKv, DVv) \
    if (a.dk == DKv && a.dv == DVv) return scan_dims<DKv, DVv>(a);
    GDR_CASE(32, 32) GDR_CASE(32, 64) GDR_CASE(32, 128)
    GDR_CASE(64, 32) GDR_CASE(64, 64) GDR_CASE(64, 128)
    GDR_CASE(128, 32) GDR_CASE(128, 64) GDR_CASE(128, 128)
#undef GDR_CASE
    return hipErrorInvalidValue;
}

// bf16 inputs with C = 64 take the fp16 path (gdr_fp16.hip) after the chunk
// and segment tables; everything else, and the debug entry point, runs the
// five kernels. For the debug entry point on a bf16 C = 64 problem, k_prep
// runs as well, so that its T, score block and decay rows can be copied out.
template <typename T, int DK, int DV, int C>
static hipError_t launch_pipeline(const LaunchArgs& a, hipEvent_t* ev) {
    hipStream_t st = a.stream;
    auto mark = [&](int i) { if (ev && ev[i]) (void)hipEventRecord(ev[i], st); };
    const int32_t cap = a.nt_cap;
    const int32_t NT = a.nt;
    constexpr bool kFp16 = std::is_same<T, bf16>::value && C == 64;
    constexpr int NTHR = 64 * (C / 16);        // one wavefront per 16-row block of a chunk
    mark(0);
    k_chunk_table<<<1, 1024, 0, st>>>(a.cu_dev, a.T_row, a.N, a.Ttot, cap, C, a.chunk_seq, a.chunk_start,
                                      a.chunk_len, a.seq_first);
    const bool segmented = a.nseg > 0 && a.N > 0;
    if (segmented)
        k_segment_table<<<1, 1024, 0, st>>>(a.seq_first, a.N, a.seg_chunks, a.nseg, a.seg_first, a.seq_seg);
    mark(1);
    if constexpr (kFp16) {
        if (!a.reference) return launch_fp16_path(a, ev);
        if (a.T16 && !a.states16) {
            LaunchArgs b = a;
            b.prep_only = true;
            b.nseg = 0;
            const hipError_t e = launch_fp16_path(b, nullptr);
            if (e != hipSuccess) return e;
        }
    }
    if (NT > 0) {
        k_gate_cumsum<C><<<dim3(NT, (a.Nv + 256 / C - 1) / (256 / C)), 256, 0, st>>>(a.g, a.chunk_start, a.chunk_len,
                                                                                   NT, a.Nv, a.G);
    }
    mark(2);
    if (NT > 0)
        k_build_solve<T, DK, C><<<dim3(NT, a.Nk), NTHR, 0, st>>>((const T*)a.k, a.beta, a.beta_f32, a.G,
                                                                  a.chunk_start, a.chunk_len, a.Nk, a.Nv,
                                                                  (float*)a.A);
    mark(3);
    if (NT > 0)
        k_wu<T, DK, DV, C><<<dim3(NT, a.Nk), NTHR, 0, st>>>((const T*)a.k, (const T*)a.v, a.beta, a.beta_f32, a.G,
                                                       (const float*)a.A, a.chunk_start, a.chunk_len, a.Nk, a.Nv,
                                                       (float*)a.W, (float*)a.U, (T*)a.KT, (int)a.states16);
    mark(4);
    if (kFp16 && a.states16) {
        // backward recompute: H and V_new from the fp16 chunk pass (k_prep and
        // the chunk pass in kStates16 mode); G, A and W above stay fp32
        const hipError_t e = launch_fp16_states(a);
        if (e != hipSuccess) return e;
    } else if (segmented) {
        // local end states from zero, transitions from I with V = 0, the scan,
        // then the pass from the entering states that writes H and V_new
        const dim3 gs(a.nseg, a.Nv, DV / 16), gm(a.nseg, a.Nv, DK / 16);
        const float *W = (const float*)a.W, *U = (const float*)a.U;
        const T* KT = (const T*)a.KT;
        k_state<T, DK, DV, C><<<gs, 64, 0, st>>>(W, U, KT, a.G, nullptr, 0, a.chunk_start, a.chunk_len, a.seg_first,
                                              a.Nk, a.Nv, nullptr, nullptr, a.Sloc);
        k_state<T, DK, DK, C><<<gm, 64, 0, st>>>(W, nullptr, KT, a.G, nullptr, 1, a.chunk_start, a.chunk_len,
                                              a.seg_first, a.Nk, a.Nv, nullptr, nullptr, a.Mseg);
        const hipError_t e = launch_segment_scan(a);
        if (e != hipSuccess) return e;
        k_state<T, DK, DV, C><<<gs, 64, 0, st>>>(W, U, KT, a.G, a.Sstart, 0, a.chunk_start, a.chunk_len,
                                              a.seg_first, a.Nk, a.Nv, (float*)a.H, (float*)a.VN, nullptr);
    } else if (a.N > 0) {
        k_state<T, DK, DV, C><<<dim3(a.N, a.Nv, DV / 16), 64, 0, st>>>((const float*)a.W, (const float*)a.U,
                                                                   (const T*)a.KT, a.G, a.S0, 0, a.chunk_start,
                                                                   a.chunk_len, a.seq_first, a.Nk, a.Nv,
                                                                   (float*)a.H, (float*)a.VN, a.ST);
    }
    mark(5);
    if (NT > 0 && a.o)
        k_output<T, DK, DV, C><<<dim3(NT, a.Nv), NTHR, 0, st>>>((const T*)a.q, (const T*)a.k, a.G, (const float*)a.H,
                                                           (const float*)a.VN, a.chunk_start, a.chunk_len, a.Nk, a.Nv,
                                                           a.scale, a.out_f32, a.o);
    mark(6);
    return hipGetLastError();
}

template <typename T, int C>
static hipError_t dispatch_dims(const LaunchArgs& a, hipEvent_t* ev) {
#define GDR_CASE(DKv, DVv) \
    if (a.dk == DKv && a.dv == DVv) return launch_pipeline<T, DKv, DVv, C>(a, ev);
    GDR_CASE(32, 32) GDR_CASE(32, 64) GDR_CASE(32, 128)
    GDR_CASE(64, 32) GDR_CASE(64, 64) GDR_CASE(64, 128)
    GDR_CASE(128, 32) GDR_CASE(128, 64) GDR_CASE(128, 128)
#undef GDR_CASE
    return hipErrorInvalidValue;
}

template <typename T>
static hipError_t dispatch_chunk(const LaunchArgs& a, hipEvent_t* ev) {
    if (a.C == 64) return dispatch_dims<T, 64>(a, ev);
    if (a.C == 32) return dispatch_dims<T, 32>(a, ev);
    if (a.C == 16) return dispatch_dims<T, 16>(a, ev);
    return hipErrorInvalidValue;
}

hipError_t launch_forward(const LaunchArgs& a, hipEvent_t* events) {
    if (a.bf16) return dispatch_chunk<bf16>(a, events);
    return dispatch_chunk<float>(a, events);
}

}  // namespace gdr
