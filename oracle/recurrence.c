/*
 * Oracle: token-by-token gated delta-rule recurrence in fp64 on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library. The HIP product path never calls it
 * and shares no code with it.
 *
 * What it computes is the plain definition of the method, one token at a time.
 * Sources:
 *   - ChunkGatedDeltaRule math page ("01 · 数学原理"), section 1: the gated
 *     recurrence S_t = a_t S_{t-1} + b_t k_t (v_t - k_t^T S_{t-1})^T with
 *     a_t = exp(g_t), and the prose order of one step: read, form the delta,
 *     forget first, then write with strength beta.
 *   - FLA DeltaNet article (pnsm.cn), section 1: the reference token loop
 *     (subtract the read, scale by beta, rank-1 update, then read the output
 *     from the UPDATED state).
 *   - Same article, section 5: default scale 1/sqrt(dk); shapes q,k [T,H,K],
 *     v [T,H,V], state [N,H,K,V]; varlen via cumulative sequence offsets.
 *   - ChunkGatedDeltaRule page, section 1: GQA, V-head h reads q/k head
 *     h / (Nv/Nk); beta and g are per V-head.
 *
 * Reading of the decay placement (the printed formula reads k^T S_{t-1}
 * undecayed, the prose forgets first): by default the delta is read from the
 * decayed state, i.e.
 *     Sd    = exp(g_t) * S_{t-1}
 *     delta = beta_t * (v_t - Sd^T k_t)
 *     S_t   = Sd + k_t delta^T
 *     o_t   = scale * S_t^T q_t
 * which is the only reading under which the page's chunk formulas (3) and (6)
 * reproduce the token loop when g != 0. literal_undecayed_read = 1 selects the
 * literal printed form (delta read from the undecayed S_{t-1}) so a test can
 * show that it disagrees with the chunked form when g != 0.
 *
 * Layouts (row-major, token axis flattened over batch rows):
 *   q, k [Ttot, Nk, dk]; v, o [Ttot, Nv, dv]; g, beta [Ttot, Nv];
 *   S0, S_T [N, Nv, dk, dv]; cu_seqlens [N+1] (int64, non-decreasing,
 *   cu_seqlens[0] = 0, cu_seqlens[N] = Ttot).
 * g == NULL means the ungated rule (factor 1); S0 == NULL means zeros.
 * unit_mask (may be NULL) has N*Nv bytes; units (n, h) with mask 0 are skipped
 * and their o rows / S_T blocks are left untouched.
 * num_threads > 0 fixes the OpenMP team size (0: the runtime default); the
 * team size actually used is stored in *threads_used when that is not NULL.
 * Returns 0 on success, -1 on a bad argument.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

int gdr_oracle_recurrence(int64_t Ttot, int32_t Nk, int32_t Nv, int32_t dk, int32_t dv,
                          int32_t N, const int64_t* cu_seqlens,
                          const double* q, const double* k, const double* v,
                          const double* g, const double* beta, double scale,
                          const double* S0, int32_t literal_undecayed_read,
                          const uint8_t* unit_mask, double* o, double* S_T,
                          int32_t num_threads, int32_t* threads_used)
{
    if (Nk <= 0 || Nv <= 0 || dk <= 0 || dv <= 0 || N < 0 || Nv % Nk != 0) return -1;
    if (!cu_seqlens || !q || !k || !v || !beta || !o || !S_T) return -1;
    if (cu_seqlens[0] != 0 || cu_seqlens[N] != Ttot) return -1;
    for (int32_t n = 0; n < N; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;

    const int32_t group = Nv / Nk;
    const int64_t units = (int64_t)N * Nv;

    const int team = num_threads > 0 ? num_threads : omp_get_max_threads();
    if (threads_used) *threads_used = team;

#pragma omp parallel for schedule(dynamic, 1) num_threads(team)
    for (int64_t unit = 0; unit < units; ++unit) {
        const int32_t n = (int32_t)(unit / Nv);
        const int32_t h = (int32_t)(unit % Nv);
        if (unit_mask && !unit_mask[unit]) continue;
        const int32_t kh = h / group;               /* q/k head shared by this V-head */

        double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
        double* read = (double*)malloc(sizeof(double) * (size_t)dv);
        if (!S || !read) { free(S); free(read); continue; }

        const size_t sbase = ((size_t)n * Nv + h) * (size_t)dk * dv;
        if (S0) memcpy(S, S0 + sbase, sizeof(double) * (size_t)dk * dv);
        else memset(S, 0, sizeof(double) * (size_t)dk * dv);

        for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
            const double* qt = q + ((size_t)t * Nk + kh) * dk;
            const double* kt = k + ((size_t)t * Nk + kh) * dk;
            const double* vt = v + ((size_t)t * Nv + h) * dv;
            const double bt = beta[(size_t)t * Nv + h];
            const double at = g ? exp(g[(size_t)t * Nv + h]) : 1.0;

            /* read = S_{t-1}^T k_t, taken before the forget step */
            for (int32_t j = 0; j < dv; ++j) read[j] = 0.0;
            for (int32_t i = 0; i < dk; ++i)
                for (int32_t j = 0; j < dv; ++j)
                    read[j] += kt[i] * S[(size_t)i * dv + j];

            /* forget: S <- a_t S_{t-1}; the decayed read is a_t * read */
            for (size_t e = 0; e < (size_t)dk * dv; ++e) S[e] *= at;
            const double read_factor = literal_undecayed_read ? 1.0 : at;

            /* delta = beta_t (v_t - read); write S += k_t delta^T */
            for (int32_t j = 0; j < dv; ++j) read[j] = bt * (vt[j] - read_factor * read[j]);
            for (int32_t i = 0; i < dk; ++i)
                for (int32_t j = 0; j < dv; ++j)
                    S[(size_t)i * dv + j] += kt[i] * read[j];

            /* output from the updated state: o_t = scale * S_t^T q_t */
            double* ot = o + ((size_t)t * Nv + h) * dv;
            for (int32_t j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int32_t i = 0; i < dk; ++i) acc += qt[i] * S[(size_t)i * dv + j];
                ot[j] = scale * acc;
            }
        }
        memcpy(S_T + sbase, S, sizeof(double) * (size_t)dk * dv);
        free(S);
        free(read);
    }
    return 0;
}
