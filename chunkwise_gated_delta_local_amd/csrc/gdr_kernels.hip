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
#include "gdr_launch.hpp"

namespace gdr {

// Lower-triangular pair fragments of T (16-row block tb, 32-position block tp).
constexpr int kTPairs = 6;
__constant__ int kTPairTb[kTPairs] = {0, 1, 2, 2, 3, 3};
__constant__ int kTPairTp[kTPairs] = {0, 0, 0, 1, 0, 1};

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
// When R is given, the two decay factors the fused state pass needs are
// written per token too:
//   R.x = exp(G_t)                      decay from the chunk start
//   R.y = exp(G_last - G_t)             decay to the chunk end
// chunk-major, [chunk][head][C positions] with zeros past the chunk end, so
// that the sequential pass reads the factors of one (chunk, head) as one
// contiguous block.
template <int C>
__global__ __launch_bounds__(256) void k_gate_cumsum(const float* __restrict__ g,
                                                      const int32_t* __restrict__ chunk_start,
                                                      const int32_t* __restrict__ chunk_len,
                                                      int32_t NT, int32_t Nv, float* __restrict__ G,
                                                      f32x2* __restrict__ R) {
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
    const float g_last = __shfl(x, L > 0 ? L - 1 : 0, C);
    if (on && i < L) G[(s + i) * Nv + h] = x;
    if (R && on)
        R[((int64_t)c * Nv + h) * C + i] = i < L ? f32x2{__expf(x), __expf(g_last - x)} : f32x2{0.f, 0.f};
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
//   5. A rows (fp32) -> global, zero above the diagonal and past the chunk end
//      (when A_out is given), and/or T = A diag(beta) (FLA DeltaNet article,
//      section 2.3: T absorbs diag(beta)) as split (hi, lo) pair fragments of
//      its lower-triangular 16 x 32 blocks for the fused state pass (C = 64,
//      when Tf is given).
//   6. When Pf is given (fused pipeline, C = 64): the intra-chunk score block
//      P = (Q K^T) (.) D, D_ij = exp(G_i - G_j) for j <= i (ChunkGatedDeltaRule
//      page, formula (5); FLA DeltaNet article, section 2.4), as split pair
//      fragments in the same six-block layout as T, so that the state pass
//      does not recompute it for every dv tile. Q K^T is formed once per key
//      head; the decay is applied per value head.
template <typename T, int DK, int C>
__global__ __launch_bounds__(256, 4) void k_build_solve(const T* __restrict__ k, const T* __restrict__ q,
                                                         const void* __restrict__ beta, int beta_f32,
                                                         const float* __restrict__ G,
                                                         const int32_t* __restrict__ chunk_start,
                                                         const int32_t* __restrict__ chunk_len,
                                                         int32_t Nk, int32_t Nv, float* __restrict__ A_out,
                                                         T* __restrict__ Tf, T* __restrict__ Pf) {
    static_assert(C == 16 || C == 32 || C == 64, "chunk size");
    constexpr int NTB = C / 16;                // 16-row blocks of the chunk, one wavefront each
    constexpr int NTHR = 64 * NTB;
    constexpr int KP = DK + 8;                 // padded LDS row (elements)
    constexpr int SEGS = C * (DK / 8) / NTHR;  // 16-byte row segments per thread
    // The K and Q tiles are only needed until the K K^T and Q K^T tiles are in
    // registers; L and A reuse their LDS afterwards.
    constexpr int TILE_BYTES = 2 * C * KP * (int)sizeof(T);
    constexpr int LP = C + 4;                  // L and A row pitch (floats): 16-byte aligned rows
    constexpr int LA_BYTES = 2 * C * LP * 4;
    __shared__ __attribute__((aligned(16))) char smem[TILE_BYTES > LA_BYTES ? TILE_BYTES : LA_BYTES];
    __shared__ __attribute__((aligned(16))) float bs[C], gs[C];
    T* Ks = reinterpret_cast<T*>(smem);
    T* Qs = Ks + C * KP;
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

    // 1. K (and Q) rows of the chunk (zero past the chunk end): all loads first
    {
        v8 kv[SEGS], qv[SEGS];
#pragma unroll
        for (int i = 0; i < SEGS; ++i) {
            const int idx = tid + NTHR * i, row = idx / (DK / 8), seg = idx % (DK / 8);
            kv[i] = zero_pair<T>();
            qv[i] = zero_pair<T>();
            if (row < L) {
                kv[i] = *reinterpret_cast<const v8*>(k + ((s + row) * Nk + kh) * DK + seg * 8);
                if (Pf) qv[i] = *reinterpret_cast<const v8*>(q + ((s + row) * Nk + kh) * DK + seg * 8);
            }
        }
        fetch_gates(0);
#pragma unroll
        for (int i = 0; i < SEGS; ++i) {
            const int idx = tid + NTHR * i, row = idx / (DK / 8), seg = idx % (DK / 8);
            *reinterpret_cast<v8*>(&Ks[row * KP + seg * 8]) = kv[i];
            if (Pf) *reinterpret_cast<v8*>(&Qs[row * KP + seg * 8]) = qv[i];
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
    // transposed score tiles of block row `wave`: qk[j] holds k_{16j+4qd+jj} . q_{16*wave+r}
    f32x4 qk[NTB];
#pragma unroll
    for (int j = 0; j < NTB; ++j) {
        qk[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (Pf && j <= wave) {
#pragma unroll
            for (int kp = 0; kp < DK / 32; ++kp) {
                v8 a = load_pair_row<T>(&Ks[(j * 16 + r) * KP + kp * 32], qd);
                v8 b = load_pair_row<T>(&Qs[(wave * 16 + r) * KP + kp * 32], qd);
                qk[j] = mfma_pair(a, b, qk[j]);
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
        // T = A diag(beta) pair fragments: pair p covers rows 16*tb + r and positions 32*tp + m(qd, e)
        // for (tb, tp) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1); rows past the chunk end are zero.
        if constexpr (C == 64) {
            if (Tf) {
                for (int p = wave; p < kTPairs; p += 4) {
                    const int tb = kTPairTb[p], tp = kTPairTp[p];
                    const int row = tb * 16 + r;
                    const int m0 = tp * 32 + 4 * qd;           // positions m0..m0+3 and m0+16..m0+19
                    const f32x4 a0 = *reinterpret_cast<const f32x4*>(&Af[row][m0]);
                    const f32x4 a1 = *reinterpret_cast<const f32x4*>(&Af[row][m0 + 16]);
                    const f32x4 b0 = *reinterpret_cast<const f32x4*>(&bs[m0]);
                    const f32x4 b1 = *reinterpret_cast<const f32x4*>(&bs[m0 + 16]);
                    float x[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[e] = (row < L && m0 + e <= row) ? a0[e] * b0[e] : 0.f;
                        x[4 + e] = (row < L && m0 + 16 + e <= row) ? a1[e] * b1[e] : 0.f;
                    }
                    const Split<T> sp = split8<T>(x);
                    T* dst = Tf + (((int64_t)c * Nv + h) * kTPairs + p) * 2 * 512;
                    store_frag<T>(dst, lane, sp.hi);
                    if constexpr (kSplitNeeded<T>) store_frag<T>(dst + 512, lane, sp.lo);
                }
            }
        }
        // 6. score pairs of block row `wave`: P_ij = (q_i . k_j) exp(G_i - G_j), j <= i < L
        if constexpr (C == 64) {
            if (Pf) {
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
                        const Split<T> sp = split_acc_pair<T>(pt[2 * tp], pt[2 * tp + 1]);
                        T* dst = Pf + (((int64_t)c * Nv + h) * kTPairs + pbase + tp) * 2 * 512;
                        store_frag<T>(dst, lane, sp.hi);
                        if constexpr (kSplitNeeded<T>) store_frag<T>(dst + 512, lane, sp.lo);
                    }
                }
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
                                             float* __restrict__ Wf, float* __restrict__ Uf, T* __restrict__ KTf) {
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

    // K^T pair fragments for the state pass: [c][kh][db][tp]
    for (int f = wave; f < (DK / 16) * NTP; f += NTB) {
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
        for (int idx = tid; idx < CP * (DV / 8); idx += NTHR) {
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
// Modes of the fused pass: kFull (state and output, from S0; twelve
// wavefronts) and kSegment (eight wavefronts: state and copy roles only, no
// output work). A kSegment workgroup with blockIdx.z < dv/16 forms the end
// state of its run of chunks from a zero state; one with a larger blockIdx.z
// forms the map a run of chunks applies to its entering state: the end state
// from S = I (dk columns, written to ST2) with V read as zero. Both serve
// segment-parallel state passing (below) and run in one launch, two
// workgroups to a compute unit.
constexpr int kFull = 0, kSegment = 1;
// Production path for bf16 inputs. One workgroup of twelve wavefronts per
// (sequence, value head, 16 columns of dv) walks the sequence's chunks in
// order with the state slice S (dk x 16, fp32) on chip, and produces the output
// of each chunk as it goes, so neither the per-chunk states nor V_new reach HBM.
// Per chunk (ChunkGatedDeltaRule page, formulas (3)-(6); FLA DeltaNet article,
// sections 2.3-2.4), with T = A diag(beta) and the score block
// P = (Q K^T) (.) D from the A-build kernel:
//   Y     = K S_in,  Z = V - diag(exp(G)) Y      so that V_new = U - W S_in = T Z
//   V_new = T Z                                  (T lower triangular)
//   S_out = exp(G_last) S_in + K^T diag(exp(G_last - G)) V_new
//   O     = scale [diag(exp(G)) Q S_in + P V_new]
// The wavefronts split into three roles that run side by side, one of each on
// every SIMD:
//   state waves  (0..3):  wave w owns positions 16w..16w+15 for Y, Z, Q S_in and
//                         V_new, and dk tiles of S for the update. This is the
//                         sequential chain.
//   output waves (4..7):  wave 4+w forms the output of positions 16w..16w+15.
//   copy waves   (8..11): move the coming chunks' K, Q, score, V and R tiles
//                         from global memory straight into LDS (16-byte buffer
//                         loads to LDS, rows past the chunk end read as zero)
//                         and do nothing else, so no wave that reads LDS ever
//                         waits for a copy.
// The state waves load their T fragments for the next chunk straight into
// registers once T Z has used the current ones (they issue no global stores,
// so waiting for those loads never waits for a store).
// Each chunk step has three phases separated by barriers that wait for LDS
// traffic only (never for global loads or stores):
//   A  state:  S_in (split) from LDS, Y, Z -> LDS; every read of the chunk's
//              K and Q tiles happens here
//      output: O of the previous chunk, in registers
//   B  state:  Q S_in -> LDS, V_new = T Z -> LDS (T pairs from LDS)
//      output: this chunk's score pairs and exp(G) from LDS
//   C  state:  S update, S_out (split) -> LDS
//      output: the previous chunk's O -> global
// K and Q tiles sit in LDS row-major with the 16-byte units of each row
// XOR-permuted by the row (swz): every matrix-core operand is one 16-byte LDS
// read, K^T operands come from the same tile through transposing LDS reads,
// both without bank conflicts, and each 1 KB copy moves whole rows (strided
// half-line copies of 16 rows each ran the state pass about 15 % slower).
//
// Contraction orders: products over dk (K S, Q S) take the 32 indices of a
// block as 8 qd + e for lane quarter qd and element e (so that a fragment is 16
// contiguous bytes of a row); products over positions (T Z, K^T V, P V_new) use
// the stacked-accumulator order of gdr_device.hpp. The state is written to LDS
// in the first order by the wave that updates it.
template <int DK, int DV, int MODE>
__global__ __launch_bounds__(MODE == kFull ? 768 : 512) void k_state_output(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                       const bf16* __restrict__ v, const f32x2* __restrict__ R, const bf16* __restrict__ Tf,
                                                       const bf16* __restrict__ Pf, const float* __restrict__ S0,
                                                       const int32_t* __restrict__ chunk_start,
                                                       const int32_t* __restrict__ chunk_len,
                                                       const int32_t* __restrict__ seq_first, int32_t Nk, int32_t Nv,
                                                       float scale, int out_f32, void* __restrict__ o,
                                                       float* __restrict__ ST, float* __restrict__ ST2) {
    typedef bf16 T;
    typedef Vec<T>::v8 v8;
    typedef Vec<T>::v4 v4;
    typedef short s4 __attribute__((ext_vector_type(4)));
    typedef s4 __attribute__((address_space(3))) * lds_s4;
    constexpr int NKP = DK / 32, NDB = DK / 16;
    constexpr int TPW = (NDB + 3) / 4;          // state tiles owned per state wave
    constexpr int FRAG = 512;                   // elements of one fragment block (64 lanes x 8)
    constexpr int TFRAG = kTPairs * 2 * 512;    // T elements per (chunk, head)
    constexpr int NTCP = TFRAG * 2 / 1024;      // 1 KB copies of T per chunk
    constexpr int MCE = 2 * NKP;                // early-list copies per copy wave per chunk
    constexpr int RSRC = 0x00020000;            // buffer descriptor word 3 (raw 32-bit access)
    static_assert(NTCP % 4 == 0, "fragment count");
    // chunk tiles, double-buffered; each half is its own array so that the
    // compiler can tell reads of one half from copies into the other
    __shared__ __attribute__((aligned(16))) T Ks0[4 * NKP * FRAG], Ks1[4 * NKP * FRAG];
    __shared__ __attribute__((aligned(16))) T Qs0[4 * NKP * FRAG], Qs1[4 * NKP * FRAG];
    __shared__ __attribute__((aligned(16))) T Pb0[TFRAG], Pb1[TFRAG];
    // with output (twelve waves) the T pairs also come through LDS, so that the
    // state waves issue no global loads: a load of theirs would queue behind
    // the copy waves' tile loads in the compute unit's memory pipeline
    constexpr int TLDS = MODE == kFull ? TFRAG : 1;
    __shared__ __attribute__((aligned(16))) T Tb0[TLDS], Tb1[TLDS];
    __shared__ __attribute__((aligned(16))) T Vs0[kChunk * 16], Vs1[kChunk * 16];
    __shared__ __attribute__((aligned(16))) f32x2 Rs0[kChunk], Rs1[kChunk];
    __shared__ __attribute__((aligned(16))) T Sb[NKP][2][FRAG];
    __shared__ __attribute__((aligned(16))) T Zb[2][2][FRAG];
    __shared__ __attribute__((aligned(16))) T Vb[2][2][FRAG];
    __shared__ __attribute__((aligned(16))) T Vtb[2][2][FRAG];
    __shared__ __attribute__((aligned(16))) f32x4 QSx[4][64];

    // XCD-aware placement: workgroups are dealt to the 8 XCDs round-robin by
    // linear id, so the grid is renumbered for every XCD to take a contiguous
    // run of (unit, head, column tile) triples, column tile fastest: the
    // workgroups that read the same K and Q tiles (all column tiles of the
    // value heads of one key head) then share one XCD's L2.
    int bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
    {
        const int64_t W = (int64_t)gridDim.x * gridDim.y * gridDim.z;
        if (W % 8 == 0) {
            const int64_t lin = bx + (int64_t)gridDim.x * (by + (int64_t)gridDim.y * bz);
            const int64_t work = (lin % 8) * (W / 8) + lin / 8;
            bz = (int)(work % gridDim.z);
            by = (int)((work / gridDim.z) % gridDim.y);
            bx = (int)(work / ((int64_t)gridDim.z * gridDim.y));
        }
    }
    const int n = bx, h = by;
    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);     // wave index, uniform
    const int lane = tid & 63, r = lane & 15, qd = lane >> 4;
    const int kh = h / (Nv / Nk);
    constexpr bool want_o = MODE == kFull;       // else state only: no Q, score or output work
    constexpr int kCopy0 = want_o ? 8 : 4;       // first copy wave
    const bool trans = MODE != kFull && bz >= DV / 16;   // transition workgroup
    const int nb = trans ? bz - DV / 16 : bz;
    const int NC = trans ? DK : DV;              // columns of the state written
    float* const STo = trans ? ST2 : ST;
    const int c0 = seq_first[n], c1 = seq_first[n + 1];
    // The chunks of a sequence are consecutive 64-token pieces of its token
    // range, so their start and length follow from the range.
    const int64_t seq_s = c0 < c1 ? (int64_t)chunk_start[c0] : 0;
    const int64_t seq_e = c0 < c1 ? (int64_t)chunk_start[c1 - 1] + chunk_len[c1 - 1] : 0;
    auto chunk_s = [&](int c) { return seq_s + (int64_t)(c - c0) * kChunk; };
    // (clamped to [0, C]: a segment table built from offsets that disagree with
    // the host's copy can never produce a negative length or a range past the
    // chunk; an empty chunk copies nothing, leaves the state and writes no rows)
    auto chunk_L = [&](int c) { return (int)max((int64_t)0, min((int64_t)kChunk, seq_e - chunk_s(c))); };
    auto rsrc = [&](const void* base, int64_t elem_off, int elem_bytes, uint32_t bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(reinterpret_cast<const char*>(base)) + elem_off * elem_bytes, (short)0, (int)bytes, RSRC);
    };
    // K and Q chunk tiles sit in LDS row-major (64 rows of dk values), the
    // 16-byte units of each row permuted by an XOR with swz(row): the MFMA
    // operand reads (rows 16 tb + r, unit 4 kp + qd) and the transposing K^T
    // reads then hit distinct banks, and each tile copy moves whole rows.
    constexpr int UPR = DK / 8;                  // 16-byte units per row
    auto swz = [](int row) { return ((((row & 3) << 1) | ((row >> 2) & 1) | (row & 8))) & (UPR - 1); };
    auto frag = [&](const T* tile, int tb, int kp) {
        const int row = 16 * tb + r;
        return *reinterpret_cast<const v8*>(&tile[row * DK + ((4 * kp + qd) ^ swz(row)) * 8]);
    };
    // Exchange buffers hold split pair fragments as two lane-linear half blocks
    // (elements 0..3 of every lane, then elements 4..7), so that the wave that
    // produces one half writes 8 contiguous bytes per lane.
    auto store_split_half = [&](T (*buf)[2][FRAG], int tp, int half, const f32x4& x) {
        float xx[8] = {x[0], x[1], x[2], x[3], 0.f, 0.f, 0.f, 0.f};
        const Split<T> sp = split8<T>(xx);
        v4 hi4 = {sp.hi[0], sp.hi[1], sp.hi[2], sp.hi[3]};
        v4 lo4 = {sp.lo[0], sp.lo[1], sp.lo[2], sp.lo[3]};
        *reinterpret_cast<v4*>(&buf[tp][0][half * 256 + lane * 4]) = hi4;
        *reinterpret_cast<v4*>(&buf[tp][1][half * 256 + lane * 4]) = lo4;
    };
    auto load_split = [&](T (*buf)[2][FRAG], int tp) {
        Split<T> sp;
        sp.hi = concat<T>(*reinterpret_cast<const v4*>(&buf[tp][0][lane * 4]),
                          *reinterpret_cast<const v4*>(&buf[tp][0][256 + lane * 4]));
        sp.lo = concat<T>(*reinterpret_cast<const v4*>(&buf[tp][1][lane * 4]),
                          *reinterpret_cast<const v4*>(&buf[tp][1][256 + lane * 4]));
        return sp;
    };
    const int64_t sbase = ((int64_t)n * Nv + h) * DK * NC;
    // split pair fragment p (hi, lo) of a six-pair set (T or the score block) of
    // chunk c, straight into registers (16 bytes per lane per half)
    auto load_pair_set = [&](const T* base, int c, int p) {
        typedef int i4 __attribute__((ext_vector_type(4)));
        const auto rs = rsrc(base, ((int64_t)c * Nv + h) * TFRAG, 2, TFRAG * 2);
        Split<T> sp;
        sp.hi = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(rs, (p * 2 * FRAG) * 2 + lane * 16, 0, 0));
        sp.lo = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(rs, (p * 2 * FRAG + FRAG) * 2 + lane * 16,
                                                                             0, 0));
        return sp;
    };

    if (wv < 4) {
        // ======================================================== state waves
        const int w = wv;
        const int ntp = (w >> 1) + 1;                       // T pairs of block w: positions < 32 * ntp
        const int pbase = (w == 0) ? 0 : (w == 1 ? 1 : (w == 2 ? 2 : 4));
        f32x4 S[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int db = w * TPW + t;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = db * 16 + 4 * qd + j, col = nb * 16 + r;
                S[t][j] = db >= NDB ? 0.f
                          : trans ? (row == col ? 1.f : 0.f)
                          : S0 ? S0[sbase + (int64_t)row * NC + col] : 0.f;
            }
        }
        // S tile db (rows 16 db + 4 qd + j of this lane's column r) -> B fragments of
        // contraction block db / 2 in the 8 qd + e order
        auto publish_state = [&]() {
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const int db = w * TPW + t;
                if (db < NDB) {
                    float xx[8] = {S[t][0], S[t][1], S[t][2], S[t][3], 0.f, 0.f, 0.f, 0.f};
                    const Split<T> sp = split8<T>(xx);
                    v4 hi4 = {sp.hi[0], sp.hi[1], sp.hi[2], sp.hi[3]};
                    v4 lo4 = {sp.lo[0], sp.lo[1], sp.lo[2], sp.lo[3]};
                    const int dst = (qd & 1) * 256 + (16 * (2 * (db & 1) + (qd >> 1)) + r) * 4;
                    *reinterpret_cast<v4*>(&Sb[db >> 1][0][dst]) = hi4;
                    *reinterpret_cast<v4*>(&Sb[db >> 1][1][dst]) = lo4;
                }
            }
        };
        // transposed K operand: K^T rows 16 db.., positions of pair tp (stacked order)
        // (the transposing read gives lane (qd, r') element e = element (r' & 3)
        // of lane (qd, 4 e + (r' >> 2)), so lane (qd, j) fetches the four dk
        // values 16 db + 4 (j & 3) .. of position 16 (2 tp + hh) + 4 qd + (j >> 2))
        auto kt_frag = [&](const T* Kb, int db, int tp) {
            const int j = lane & 15;
            const int unit = 2 * db + ((j & 3) >> 1);
            const int e0 = 4 * (j & 1);
            v4 part[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int row = 16 * (2 * tp + hh) + 4 * qd + (j >> 2);
                const T* p = &Kb[row * DK + (unit ^ swz(row)) * 8 + e0];
                part[hh] = __builtin_bit_cast(v4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)p));
            }
            return concat<T>(part[0], part[1]);
        };
        if (c0 < c1) {
            // T pairs of block w for the current chunk, in registers; the next
            // chunk's are loaded once T Z has used them
            constexpr bool t_lds = MODE == kFull;
            Split<T> tf[2];
            if constexpr (!t_lds) {
#pragma unroll
                for (int tp = 0; tp < 2; ++tp)
                    if (tp < ntp) tf[tp] = load_pair_set(Tf, c0, pbase + tp);
            }
            publish_state();
            lds_barrier();
            for (int c = c0; c < c1; ++c) {
                const bool odd = (c - c0) & 1;
                const int L = chunk_L(c);
                const T* Kb = odd ? Ks1 : Ks0;
                const T* Qb = odd ? Qs1 : Qs0;
                const T* Vsb = odd ? Vs1 : Vs0;
                const f32x2* Rsb = odd ? Rs1 : Rs0;

                // ---- A: Y = K S_in (hi and lo passes), Z = V - exp(G) Y -> LDS
                Split<T> BS[NKP];
                v8 ka[NKP], qa[NKP];
#pragma unroll
                for (int kp = 0; kp < NKP; ++kp) {
                    BS[kp] = load_split(Sb, kp);
                    ka[kp] = frag(Kb, w, kp);
                }
                f32x2 rrow[4];
                float vrow[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    rrow[j] = Rsb[w * 16 + 4 * qd + j];
                    vrow[j] = to_f(Vsb[(w * 16 + 4 * qd + j) * 16 + r]);
                }
#pragma unroll
                for (int kp = 0; kp < NKP; ++kp) qa[kp] = want_o ? frag(Qb, w, kp) : v8{};
                v8 kt[TPW][2];                          // K^T operands of phase C
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
                    const int db = min(w * TPW + t, NDB - 1);
#pragma unroll
                    for (int tp = 0; tp < 2; ++tp) kt[t][tp] = kt_frag(Kb, db, tp);
                }
                f32x4 Yh = {0.f, 0.f, 0.f, 0.f}, Yl = Yh;
#pragma unroll
                for (int kp = 0; kp < NKP; ++kp) {
                    Yh = mfma_pair(ka[kp], BS[kp].hi, Yh);
                    Yl = mfma_pair(ka[kp], BS[kp].lo, Yl);
                }
                f32x4 Z;
#pragma unroll
                for (int j = 0; j < 4; ++j) Z[j] = vrow[j] - rrow[j].x * (Yh[j] + Yl[j]);
                store_split_half(Zb, w >> 1, w & 1, Z);
                lds_barrier();                                                    // barrier 1

                // ---- B: Q S_in for the output waves; V_new = T Z -> LDS
                Split<T> zf[2];
#pragma unroll
                for (int tp = 0; tp < 2; ++tp)
                    if (tp < ntp) zf[tp] = load_split(Zb, tp);
                if constexpr (t_lds) {
                    const T* Tbb = odd ? Tb1 : Tb0;
#pragma unroll
                    for (int tp = 0; tp < 2; ++tp) {
                        if (tp < ntp) {
                            tf[tp].hi = load_frag<T>(&Tbb[(pbase + tp) * 2 * FRAG], lane);
                            tf[tp].lo = load_frag<T>(&Tbb[(pbase + tp) * 2 * FRAG + FRAG], lane);
                        }
                    }
                }
                f32x4 Qh = {0.f, 0.f, 0.f, 0.f}, Ql = Qh;
                if constexpr (want_o) {
#pragma unroll
                    for (int kp = 0; kp < NKP; ++kp) {
                        Qh = mfma_pair(qa[kp], BS[kp].hi, Qh);
                        Ql = mfma_pair(qa[kp], BS[kp].lo, Ql);
                    }
                }
                f32x4 Va = {0.f, 0.f, 0.f, 0.f}, Vl = Va;
#pragma unroll
                for (int tp = 0; tp < 2; ++tp) {
                    if (tp < ntp) {
                        Va = mfma_pair(tf[tp].hi, zf[tp].hi, Va);
                        Vl = mfma_pair(tf[tp].lo, zf[tp].hi, Vl);
                        Vl = mfma_pair(tf[tp].hi, zf[tp].lo, Vl);
                    }
                }
                f32x4 VN, VD;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    VN[j] = Va[j] + Vl[j];
                    VD[j] = VN[j] * rrow[j].y;
                }
                store_split_half(Vtb, w >> 1, w & 1, VD);
                store_split_half(Vb, w >> 1, w & 1, VN);
                if constexpr (want_o) QSx[w][lane] = Qh + Ql;
                if (!t_lds && c + 1 < c1) {
#pragma unroll
                    for (int tp = 0; tp < 2; ++tp)
                        if (tp < ntp) tf[tp] = load_pair_set(Tf, c + 1, pbase + tp);
                }
                lds_barrier();                                                    // barrier 2

                // ---- C: S_out = exp(G_last) S_in + K^T V_decayed for the dk tiles of this wave
                const Split<T> vt[2] = {load_split(Vtb, 0), load_split(Vtb, 1)};
                const float a_last = L > 0 ? Rsb[L - 1].x : 1.f;
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
                    const int db = w * TPW + t;
                    if (db < NDB) {
                        f32x4 acc = S[t] * a_last, lo = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int tp = 0; tp < 2; ++tp) {
                            acc = mfma_pair(kt[t][tp], vt[tp].hi, acc);
                            lo = mfma_pair(kt[t][tp], vt[tp].lo, lo);
                        }
                        S[t] = acc + lo;
                    }
                }
                publish_state();
                lds_barrier();                                                    // barrier 3
            }
        }
        if (STo) {
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const int db = w * TPW + t;
                if (db < NDB) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        STo[sbase + (int64_t)(db * 16 + 4 * qd + j) * NC + nb * 16 + r] = S[t][j];
                }
            }
        }
        return;
    }

    if (c0 >= c1) return;
    if (wv >= kCopy0) {
        // ======================================================== copy waves
        // Wave 8+w moves its share of each chunk's tiles into LDS. A chunk's
        // early list (K and Q blocks: read only in phase A) is issued during
        // phases B and C two steps ahead, once the state waves have finished
        // reading the half it overwrites; its late list (score pieces, V
        // halves, R: read until phase C) during phase A one step ahead. (T goes
        // straight into the state waves' registers.) Before the last barrier of step c the wave waits for everything
        // but the early list of chunk c+2, which may still be in flight (vector
        // memory operations complete in order).
        const int w = wv - kCopy0;
        // copy u of a tile moves rows 512/DK * u .. (a whole number of rows per 1 KB)
        constexpr int RPI = 512 / DK;
        auto kq_off = [&](int u) {
            const int row = RPI * u + lane / UPR;
            return (row * Nk * DK + 8 * ((lane % UPR) ^ swz(row))) * 2;
        };
        auto copy_early = [&](int c, bool odd, int m0, int m1) {
            T* Kd = odd ? Ks1 : Ks0;
            T* Qd = odd ? Qs1 : Qs0;
            const int64_t s = chunk_s(c);
            const int L = chunk_L(c);
            const uint32_t kq_bytes = L > 0 ? (uint32_t)((L - 1) * Nk * DK + DK) * 2u : 0u;
            const auto rk = rsrc(k, (s * Nk + kh) * DK, 2, kq_bytes);
            const auto rq = rsrc(q, (s * Nk + kh) * DK, 2, kq_bytes);
#pragma unroll
            for (int m = 0; m < MCE; ++m) {
                const int u = w + 4 * m;
                if (m < m0 || m >= m1 || (m >= NKP && !want_o)) continue;
                if (m < NKP) {                               // K rows
                    buffer_to_lds16(rk, Kd + u * FRAG, kq_off(u));
                } else {                                     // Q rows
                    const int f = u - 4 * NKP;
                    buffer_to_lds16(rq, Qd + f * FRAG, kq_off(f));
                }
            }
        };
        auto copy_late = [&](int c, bool odd) {
            T* Vd = odd ? Vs1 : Vs0;
            f32x2* Rd = odd ? Rs1 : Rs0;
            const int64_t s = chunk_s(c);
            const int L = chunk_L(c);
            T* Pd = odd ? Pb1 : Pb0;
            T* Td = odd ? Tb1 : Tb0;
            const auto rp = rsrc(Pf, ((int64_t)c * Nv + h) * TFRAG, 2, TFRAG * 2);
            const auto rt = rsrc(Tf, ((int64_t)c * Nv + h) * TFRAG, 2, TFRAG * 2);
            constexpr int NTP = MODE == kFull ? NTCP : 0;    // T pieces through LDS
#pragma unroll
            for (int m = 0; m < (NTCP + NTP + 3 + 3) / 4; ++m) {
                const int u = w + 4 * m;
                if (u < NTCP) {                              // score piece
                    if constexpr (want_o) buffer_to_lds16(rp, Pd + u * FRAG, (u * 64 + lane) * 16);
                } else if (u < NTCP + NTP) {                 // T piece
                    buffer_to_lds16(rt, Td + (u - NTCP) * FRAG, ((u - NTCP) * 64 + lane) * 16);
                } else if (u < NTCP + NTP + 2) {             // V rows 32 vh .. 32 vh + 31 (16 columns)
                    // transition pass: an empty range, so every row reads as zero
                    const int vh = u - NTCP - NTP;
                    const uint32_t vbytes = (trans || L <= 0) ? 0u : (uint32_t)((L - 1) * Nv * DV + 16) * 2u;
                    buffer_to_lds16(rsrc(trans ? k : v, trans ? 0 : (s * Nv + h) * DV + nb * 16, 2, vbytes),
                                    Vd + vh * 512, ((32 * vh + (lane >> 1)) * Nv * DV + 8 * (lane & 1)) * 2);
                } else if (u == NTCP + NTP + 2 && lane < 32) {   // R (512 bytes: two positions per lane)
                    buffer_to_lds16(rsrc(R, ((int64_t)c * Nv + h) * kChunk, 8, kChunk * 8), Rd, lane * 16);
                }
            }
        };
        constexpr int MEB = MCE / 2;                     // early copies issued in phase B (rest in C)
        copy_early(c0, false, 0, MCE);
        copy_late(c0, false);
        wait_vmem();
        if (c0 + 1 < c1) copy_early(c0 + 1, true, 0, MCE);
        lds_barrier();
        for (int c = c0; c < c1; ++c) {
            const bool odd = (c - c0) & 1;
            if (c + 1 < c1) copy_late(c + 1, !odd);
            lds_barrier();                                                          // barrier 1
            if (c + 2 < c1) copy_early(c + 2, odd, 0, MEB);
            lds_barrier();                                                          // barrier 2
            if (c + 2 < c1) {
                copy_early(c + 2, odd, MEB, MCE);
                // chunk c+1 has landed; chunk c+2's early list (its K blocks only, without o) may be in flight
                if constexpr (want_o) wait_vmem_but<MCE>();
                else wait_vmem_but<MEB>();
            } else {
                wait_vmem();
            }
            lds_barrier();                                                          // barrier 3
        }
        return;
    }

    // ============================================================ output waves
    // The output of chunk c is formed in phase A of step c+1 (after the loop for
    // the last chunk): its operands V_new and Q S_in stay in the exchange buffers
    // until phase B of step c+1, and the score pairs and exp(G) are taken into
    // registers in phase B of step c, before the copy waves overwrite that LDS
    // half with chunk c+2.
    if constexpr (!want_o) return;                   // (no output waves in this mode)
    const int w = wv - 4;
    const int ntp = (w >> 1) + 1;
    const int ob = out_f32 ? 4 : 2;
    int o_off[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) o_off[j] = ((w * 16 + 4 * qd + j) * Nv * DV + r) * ob;
    const int pbase = (w == 0) ? 0 : (w == 1 ? 1 : (w == 2 ? 2 : 4));
    Split<T> pa[2];                                  // score pairs of the pending chunk
    float ex[4];                                     // exp(G) of its rows
    f32x4 ofin;                                      // finished output rows, held until phase C
    auto output = [&](int c) {                       // O = scale [exp(G) Q S_in + P V_new], positions 16w..
        Split<T> vn[2];
#pragma unroll
        for (int tp = 0; tp < 2; ++tp)
            if (tp < ntp) vn[tp] = load_split(Vb, tp);
        const f32x4 qs = QSx[w][lane];
        f32x4 out, ol = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) out[j] = ex[j] * qs[j];
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
            if (tp < ntp) {
                out = mfma_pair(pa[tp].hi, vn[tp].hi, out);
                ol = mfma_pair(pa[tp].lo, vn[tp].hi, ol);
                ol = mfma_pair(pa[tp].hi, vn[tp].lo, ol);
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) ofin[j] = scale * (out[j] + ol[j]);
    };
    auto store_out = [&](int c) {
        const int64_t s = chunk_s(c);
        const int L = chunk_L(c);
        const auto ro = rsrc(o, (s * Nv + h) * DV + nb * 16, ob, L > 0 ? (uint32_t)(((L - 1) * Nv * DV + 16) * ob) : 0u);
#pragma unroll
        for (int j = 0; j < 4; ++j) {                   // rows past the chunk end fall outside ro
            const float val = ofin[j];
            if (out_f32) __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, val), ro, o_off[j], 0, 0);
            else __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, to_t<T>(val)), ro,
                                                       o_off[j], 0, 0);
        }
    };
    lds_barrier();
    for (int c = c0; c < c1; ++c) {
        const bool odd = (c - c0) & 1;

        // ---- A: output of the previous chunk
        if (c > c0) output(c - 1);
        lds_barrier();                                                              // barrier 1

        // ---- B: this chunk's score pairs and exp(G) into registers
        const T* Pbb = odd ? Pb1 : Pb0;
        const f32x2* Rsb = odd ? Rs1 : Rs0;
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
            if (tp < ntp) {
                pa[tp].hi = load_frag<T>(&Pbb[(pbase + tp) * 2 * FRAG], lane);
                pa[tp].lo = load_frag<T>(&Pbb[(pbase + tp) * 2 * FRAG + FRAG], lane);
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) ex[j] = Rsb[w * 16 + 4 * qd + j].x;
        lds_barrier();                                                              // barrier 2

        // ---- C: store the previous chunk's output. Phase C is the output waves'
        // idlest phase; issued in phase A the stores queue behind the copy
        // waves' tile loads and lengthen that phase.
        if (c > c0) store_out(c - 1);
        lds_barrier();                                                              // barrier 3
    }
    output(c1 - 1);
    store_out(c1 - 1);
}
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
template <typename T, int DK, int DV, int C>
static hipError_t launch_pipeline(const LaunchArgs& a, hipEvent_t* ev) {
    hipStream_t st = a.stream;
    auto mark = [&](int i) { if (ev) (void)hipEventRecord(ev[i], st); };
    const int32_t cap = a.nt_cap;
    const int32_t NT = a.nt;
    constexpr bool kFused = std::is_same<T, bf16>::value && C == 64;
    constexpr int NTHR = 64 * (C / 16);        // one wavefront per 16-row block of a chunk
    const bool fused = kFused && !a.reference;
    mark(0);
    k_chunk_table<<<1, 1024, 0, st>>>(a.cu_dev, a.T_row, a.N, a.Ttot, cap, C, a.chunk_seq, a.chunk_start,
                                      a.chunk_len, a.seq_first);
    const bool segmented = a.nseg > 0 && a.N > 0;
    if (segmented)
        k_segment_table<<<1, 1024, 0, st>>>(a.seq_first, a.N, a.seg_chunks, a.nseg, a.seg_first, a.seq_seg);
    mark(1);
    if (NT > 0) {
        k_gate_cumsum<C><<<dim3(NT, (a.Nv + 256 / C - 1) / (256 / C)), 256, 0, st>>>(
            a.g, a.chunk_start, a.chunk_len, NT, a.Nv, a.G, fused ? (f32x2*)a.R : nullptr);
    }
    mark(2);
    if (NT > 0)
        k_build_solve<T, DK, C><<<dim3(NT, a.Nk), NTHR, 0, st>>>((const T*)a.k, (const T*)a.q, a.beta, a.beta_f32, a.G,
                                                            a.chunk_start, a.chunk_len, a.Nk, a.Nv,
                                                            fused ? nullptr : (float*)a.A, (T*)a.Tf,
                                                            fused ? (T*)a.Pf : nullptr);
    mark(3);
    if (NT > 0 && !fused)
        k_wu<T, DK, DV, C><<<dim3(NT, a.Nk), NTHR, 0, st>>>((const T*)a.k, (const T*)a.v, a.beta, a.beta_f32, a.G,
                                                       (const float*)a.A, a.chunk_start, a.chunk_len, a.Nk, a.Nv,
                                                       (float*)a.W, (float*)a.U, (T*)a.KT);
    mark(4);
    if (segmented) {
        // local end states from zero, transitions from I with V = 0, the scan,
        // then the pass from the entering states that writes the output
        const dim3 gs(a.nseg, a.Nv, DV / 16), gm(a.nseg, a.Nv, DK / 16), gn(a.N, a.Nv, DV / 16);
        if constexpr (kFused) {
            if (fused) {
                const bf16 *q = (const bf16*)a.q, *k = (const bf16*)a.k, *v = (const bf16*)a.v;
                const bf16 *Tf = (const bf16*)a.Tf, *Pf = (const bf16*)a.Pf;
                const f32x2* R = (const f32x2*)a.R;
                k_state_output<DK, DV, kSegment><<<dim3(a.nseg, a.Nv, DV / 16 + DK / 16), 512, 0, st>>>(
                    q, k, v, R, Tf, Pf, nullptr, a.chunk_start, a.chunk_len, a.seg_first, a.Nk, a.Nv, a.scale,
                    a.out_f32, nullptr, a.Sloc, a.Mseg);
                k_segment_scan<DK, DV><<<gn, 256, 0, st>>>(a.seq_seg, a.S0, a.Sloc, a.Mseg, a.Nv, a.Sstart, a.ST);
                k_state_output<DK, DV, kFull><<<gs, 768, 0, st>>>(
                    q, k, v, R, Tf, Pf, a.Sstart, a.chunk_start, a.chunk_len, a.seg_first, a.Nk, a.Nv, a.scale,
                    a.out_f32, a.o, nullptr, nullptr);
            }
        }
        if (!fused) {
            const float *W = (const float*)a.W, *U = (const float*)a.U;
            const T* KT = (const T*)a.KT;
            k_state<T, DK, DV, C><<<gs, 64, 0, st>>>(W, U, KT, a.G, nullptr, 0, a.chunk_start, a.chunk_len, a.seg_first,
                                                  a.Nk, a.Nv, nullptr, nullptr, a.Sloc);
            k_state<T, DK, DK, C><<<gm, 64, 0, st>>>(W, nullptr, KT, a.G, nullptr, 1, a.chunk_start, a.chunk_len,
                                                  a.seg_first, a.Nk, a.Nv, nullptr, nullptr, a.Mseg);
            k_segment_scan<DK, DV><<<gn, 256, 0, st>>>(a.seq_seg, a.S0, a.Sloc, a.Mseg, a.Nv, a.Sstart, a.ST);
            k_state<T, DK, DV, C><<<gs, 64, 0, st>>>(W, U, KT, a.G, a.Sstart, 0, a.chunk_start, a.chunk_len,
                                                  a.seg_first, a.Nk, a.Nv, (float*)a.H, (float*)a.VN, nullptr);
        }
    } else if (a.N > 0) {
        if constexpr (kFused) {
            if (fused) {
                k_state_output<DK, DV, kFull><<<dim3(a.N, a.Nv, DV / 16), 768, 0, st>>>(
                    (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const f32x2*)a.R,
                    (const bf16*)a.Tf, (const bf16*)a.Pf, a.S0,
                    a.chunk_start, a.chunk_len, a.seq_first, a.Nk, a.Nv, a.scale, a.out_f32, a.o, a.ST, nullptr);
            }
        }
        if (!fused)
            k_state<T, DK, DV, C><<<dim3(a.N, a.Nv, DV / 16), 64, 0, st>>>((const float*)a.W, (const float*)a.U,
                                                                       (const T*)a.KT, a.G, a.S0, 0, a.chunk_start,
                                                                       a.chunk_len, a.seq_first, a.Nk, a.Nv,
                                                                       (float*)a.H, (float*)a.VN, a.ST);
    }
    mark(5);
    if (NT > 0 && !fused && a.o)
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
