/*
 * gdr.h — C ABI of the chunked gated delta-rule forward for AMD MI355X (gfx950).
 *
 * The operation (FLA DeltaNet article on pnsm.cn, section 1 and sections
 * 2.3–2.4; ChunkGatedDeltaRule math page "01 · 数学原理", sections 1 and 3):
 * for every sequence n and value head h, with q/k head kh = h / (Nv / Nk),
 *
 *     S_t = exp(g_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t                      (read after the write)
 *
 * starting from S_0 = initial_state[n, h] (zeros when absent); the state after
 * the last token is returned as final_state[n, h]. The library computes this
 * with the chunkwise WY/UT algorithm (chunk size C = 64, 32 or 16). For bf16
 * inputs with C = 64, gdr_chunk_fwd runs two kernels after the chunk table: a
 * chunk-parallel preparation (gate prefix sums, decay rows, the triangular
 * solve, T = A diag(beta) and the score block (Q K^T) (.) D) and the
 * chunk-serial pass, which forms U - W S as T (V - diag(exp(G)) K S) and the
 * output in the same kernel; every derived operand of its matrix-core
 * products is rounded once to fp16 and every product accumulates in fp32.
 * fp32 inputs, C = 16 or 32, and gdr_chunk_fwd_debug run five kernels as
 * separate launches (gate prefix sums, A-build + solve, w/u products, the
 * state pass, the output) with every derived value in fp32. The chunk size
 * changes only the rounding
 * order of the result (FLA DeltaNet article, section 6, tests the chunked
 * form at several chunk sizes against the recurrence); it trades the serial
 * depth T / C of the state pass against the C x C work of the solve.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers except cu_seqlens_host. Tensors
 *   are dense row-major with 16-byte aligned base addresses; anything else is
 *   GDR_ERR_SHAPE.
 * - The caller owns every buffer (inputs, outputs, workspace). The library
 *   never allocates or frees device memory and keeps no global state apart
 *   from a thread-local error string.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *   the call returns without synchronising. Argument errors are detected on
 *   the host BEFORE any device work is enqueued. Launch failures return
 *   GDR_ERR_HIP; faults during execution surface at the caller's next
 *   synchronisation.
 * - Ttot = batch * seq_len is the total token count. Token row t of a
 *   [Ttot, H, D] tensor holds token t of the flattened (batch, time) axis.
 * - NaN/Inf in the inputs are not checked and propagate.
 * - Calls that share a workspace must not overlap in time.
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDR_F32 = 0,   /* IEEE binary32 */
    GDR_BF16 = 1   /* bfloat16; conversions from fp32 round to nearest even */
} gdr_dtype_t;

typedef enum {
    GDR_OK = 0,
    GDR_ERR_NULL = 1,        /* a required pointer is NULL                        */
    GDR_ERR_SHAPE = 2,       /* inconsistent or out-of-range sizes, misalignment  */
    GDR_ERR_DTYPE = 3,       /* unknown dtype or a dtype combination not allowed  */
    GDR_ERR_UNSUPPORTED = 4, /* valid problem outside this build (head dims, C)   */
    GDR_ERR_SEQLENS = 5,     /* cu_seqlens malformed or inconsistent with sizes   */
    GDR_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required           */
    GDR_ERR_HIP = 7          /* a HIP runtime call or kernel launch failed        */
} gdr_status_t;

/*
 * Problem description. Shapes follow the pages' statement of the problem
 * (FLA DeltaNet article, section 5; ChunkGatedDeltaRule page, section 1 I/O
 * table; FLA notes on note.zhuruihan.top, "fused recurrent fwd" shapes):
 *   q, k   [batch, seq_len, num_qk_heads, head_dim_qk]   io_dtype
 *   v      [batch, seq_len, num_v_heads,  head_dim_v]    io_dtype
 *   o      [batch, seq_len, num_v_heads,  head_dim_v]    out_dtype
 *   beta   [batch, seq_len, num_v_heads]                 beta_dtype
 *   g      [batch, seq_len, num_v_heads]                 fp32, log-domain gate (<= 0)
 *   state  [num_seqs, num_v_heads, head_dim_qk, head_dim_v]  fp32
 * Variable-length batches: batch = 1, seq_len = total tokens, and
 * cu_seqlens (int32, num_seqs + 1 entries, cu[0] = 0, non-decreasing,
 * cu[num_seqs] = seq_len) marks sequence n as tokens [cu[n], cu[n+1]).
 * Zero-length sequences are allowed (their final state equals the initial).
 * Without cu_seqlens each batch row is one sequence and num_seqs = batch.
 * The state and every sum are fp32 whatever the input type; the bf16 C = 64
 * path rounds the derived operands of its products (T, the score block, the
 * state, V - diag(exp(G)) K S, V_new) once to fp16, the other paths keep them
 * in fp32. out_dtype = GDR_F32 returns o without a final bf16 rounding.
 */
typedef struct {
    int64_t batch;          /* B >= 1; must be 1 when cu_seqlens is given          */
    int64_t seq_len;        /* T >= 0 per batch row (total tokens when varlen)     */
    int32_t num_qk_heads;   /* Nk >= 1                                             */
    int32_t num_v_heads;    /* Nv >= 1, Nv % Nk == 0; V-head h reads q/k head h/(Nv/Nk) */
    int32_t head_dim_qk;    /* dk: 32, 64 or 128 in this build                     */
    int32_t head_dim_v;     /* dv: 32, 64 or 128 in this build                     */
    int32_t chunk_size;     /* C: 64, 32 or 16                                     */
    int32_t num_seqs;       /* N: batch, or len(cu_seqlens) - 1                    */
    int32_t io_dtype;       /* gdr_dtype_t of q, k and v                           */
    int32_t beta_dtype;     /* gdr_dtype_t of beta: io_dtype or GDR_F32            */
    int32_t out_dtype;      /* gdr_dtype_t of o: io_dtype or GDR_F32               */
} gdr_problem_t;

/*
 * Host-only check of a problem description (and of cu_seqlens_host when not
 * NULL). Touches no device memory. Returns the first error found. The checks
 * are those the chunked API states for its arguments (FLA DeltaNet article,
 * section 5, parameter table): q, k, v of one dtype with the stated shapes,
 * beta [B, T, H], the state [N, H, dk, dv] with N = batch or
 * len(cu_seqlens) - 1, batch 1 when cu_seqlens is given, and a chunk size of
 * 16, 32 or 64. Two differences from that table: fp32 q, k, v are accepted,
 * and Nv may be a multiple of Nk (grouped value heads, ChunkGatedDeltaRule
 * page, section 1). Sizes outside this build (head dims other than 32, 64 or
 * 128) are GDR_ERR_UNSUPPORTED.
 */
gdr_status_t gdr_validate(const gdr_problem_t* problem, const int32_t* cu_seqlens_host);

/*
 * Workspace bytes needed by gdr_chunk_fwd (and gdr_chunk_fwd_timed) for this
 * problem: an upper bound that holds for every cu_seqlens with the same
 * num_seqs and total length. The workspace must be 256-byte aligned. It holds
 * the per-chunk values that do not depend on the state (FLA DeltaNet article,
 * section 3.1-3.3: the products and the solve that precede the state pass):
 * the chunk table and, for bf16 inputs with C = 64, the decay rows, T and the
 * score block (12.5 KB per chunk and value head) and the fp16 K and Q tiles
 * (256 dk bytes per chunk and q/k head); the five-kernel path (fp32 inputs,
 * C = 16 or 32) keeps all of its intermediates there. Validation errors as
 * for gdr_validate.
 */
gdr_status_t gdr_chunk_fwd_workspace_size(const gdr_problem_t* problem, size_t* bytes);

/*
 * Workspace bytes needed by gdr_chunk_fwd_debug, which runs the five kernels
 * as separate launches and keeps every intermediate: G, A, W, U, K^T, the
 * chunk-entering states and V_new (FLA DeltaNet article, section 3.4: the
 * three-stage pipeline whose intermediates these are), much larger than the
 * production workspace. Validation errors as for gdr_validate.
 */
gdr_status_t gdr_chunk_fwd_debug_workspace_size(const gdr_problem_t* problem, size_t* bytes);

/*
 * Token-by-token (fused recurrent) gated delta-rule forward: the same result
 * as gdr_chunk_fwd, computed one token at a time with the state on chip, for
 * decoding and short inputs (FLA notes page, "fused recurrent fwd"; the model
 * layer there takes this path for queries of at most 64 tokens).
 *   Arguments as for gdr_chunk_fwd; problem->chunk_size is ignored and no
 *   workspace is needed.
 *   use_qk_l2norm  nonzero: q and k of every token are divided by
 *                  sqrt(sum of squares + 1e-6) inside the kernel before use
 *                  (the in-kernel L2 normalisation option of the FLA
 *                  DeltaNet article, section 5); the caller's tensors are not
 *                  modified.
 * Errors as for gdr_chunk_fwd. Asynchronous on `stream`.
 */
gdr_status_t gdr_recurrent_fwd(const gdr_problem_t* problem,
                               const void* q, const void* k, const void* v,
                               const float* g, const void* beta, float scale,
                               const float* initial_state,
                               const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                               int use_qk_l2norm,
                               void* o, float* final_state, void* stream);

/*
 * Chunked gated delta-rule forward.
 *   q, k, v, beta  required inputs (layouts above).
 *   g              NULL for the ungated rule (identical to g == 0).
 *   scale          multiplies the output; callers usually pass dk^-0.5 (the
 *                  FLA article's default, section 5).
 *   initial_state  NULL means zeros.
 *   cu_seqlens_dev, cu_seqlens_host: both NULL (fixed length), or both point
 *                  to the same num_seqs + 1 offsets (device and host copies;
 *                  the host copy sizes the launch without a device sync).
 *                  If the two copies differ the results are unspecified, but
 *                  every kernel still stays inside its buffers.
 *   o              output, written for every token.
 *   final_state    NULL to skip; else written for every sequence.
 *   workspace      device scratch of at least gdr_chunk_fwd_workspace_size.
 */
gdr_status_t gdr_chunk_fwd(const gdr_problem_t* problem,
                           const void* q, const void* k, const void* v,
                           const float* g, const void* beta, float scale,
                           const float* initial_state,
                           const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                           void* o, float* final_state,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdr_chunk_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and results as gdr_chunk_fwd, with the workspace taken
 * from a scratch array the library holds on every GPU it runs on (256 MiB per
 * GPU, kept until the process ends). The caller passes inputs and outputs only.
 *   Arguments and layouts as for gdr_chunk_fwd; the buffers and `stream`
 *   belong to the current device.
 *   Returns GDR_ERR_WORKSPACE (nothing enqueued) when the problem needs more
 *   than gdr_chunk_fwd_noalloc_max_workspace() bytes of workspace (what
 *   gdr_chunk_fwd_workspace_size reports); GDR_ERR_HIP when the scratch
 *   array's address cannot be obtained. Allocates nothing (no hipMalloc or
 *   hipFree, on the first call either).
 *   Every call on one GPU uses the same scratch: calls that overlap on one GPU
 *   (on different streams, or from different threads without ordering) race,
 *   and the caller must order them. Nothing in the scratch has to start at zero.
 */
gdr_status_t gdr_chunk_fwd_noalloc(const gdr_problem_t* problem,
                                   const void* q, const void* k, const void* v,
                                   const float* g, const void* beta, float scale,
                                   const float* initial_state,
                                   const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                                   void* o, float* final_state, void* stream);

/* Bytes of scratch gdr_chunk_fwd_noalloc holds per GPU (its largest workspace). */
size_t gdr_chunk_fwd_noalloc_max_workspace(void);

/*
 * Segment-parallel state passing on one GPU: the same result as gdr_chunk_fwd
 * (up to rounding order), for inputs whose serial state pass would leave most
 * compute units idle: few sequences times value heads, and long sequences.
 *
 * The chunk-to-chunk state map S -> exp(G_last) S + K^T diag(exp(G_last - G))
 * V_new, with V_new = T (V - diag(exp(G)) K S) (ChunkGatedDeltaRule page,
 * section 3.2, formulas (3) and (6); FLA DeltaNet article, section 2.4), is
 * affine in S. Each sequence is cut into segments of `segment_chunks` whole
 * 64-token chunks (the last one shorter). For every segment, side by side:
 * its end state from a zero state (S_loc) and its dk x dk transition M (the
 * end state from S = I with V = 0). One scan per (sequence, value head) then
 * forms the entering states S_start[j+1] = M_j S_start[j] + S_loc[j] from
 * initial_state, and a last pass from those states writes o. final_state is
 * the scan's last value. All of these are fp32.
 *   segment_chunks  > 0: chunks per segment. 0: the library chooses. It cuts
 *                   each sequence into up to 256 / W segments when the serial
 *                   pass has W < 64 workgroups (W = num_seqs * num_v_heads *
 *                   head_dim_v / 16); otherwise it runs the serial pass.
 *                   When no sequence spans more than one segment, the serial
 *                   pass runs too. Negative: GDR_ERR_SHAPE.
 *   stage_events    NULL, or GDR_NUM_STAGES + 1 events (NULL entries
 *                   skipped) recorded as for gdr_chunk_fwd_timed; stage [5] covers all four segment
 *                   launches (the two side-by-side passes, the scan, the
 *                   output pass).
 *   workspace       at least gdr_chunk_fwd_segmented_workspace_size bytes for
 *                   the same segment_chunks. That is the production workspace
 *                   plus, per segment, 4 * num_v_heads * dk * (2 dv + dk)
 *                   bytes.
 * Other arguments and errors as for gdr_chunk_fwd. Asynchronous on `stream`.
 */
gdr_status_t gdr_chunk_fwd_segmented_workspace_size(const gdr_problem_t* problem, int32_t segment_chunks,
                                                    size_t* bytes);
gdr_status_t gdr_chunk_fwd_segmented(const gdr_problem_t* problem,
                                     const void* q, const void* k, const void* v,
                                     const float* g, const void* beta, float scale,
                                     const float* initial_state,
                                     const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                                     void* o, float* final_state, int32_t segment_chunks,
                                     void* workspace, size_t workspace_bytes, void* stream,
                                     void* const* stage_events);

/*
 * Backward pass: the gradients of a loss L with respect to every input of
 * gdr_chunk_fwd, given dL/do and dL/dS_T. The chunked backward of the pages
 * (GLA notes, backward steps 1-7: recompute the gate sums and chunk states,
 * run the state gradient backwards over the chunks, then the per-chunk
 * gradients of V, the score block, Q, K and the gate), carried through the
 * delta rule's WY products (ChunkGatedDeltaRule page, formulas (1)-(6); FLA
 * DeltaNet article, sections 2.3-2.4). The pages' tests compare dq, dk, dv,
 * dbeta and dh0 against the token recurrence (FLA DeltaNet article, section
 * 6); dg completes the gated form.
 *   Forward arguments (problem, q, k, v, g, beta, scale, initial_state,
 *   cu_seqlens) exactly as given to gdr_chunk_fwd; the forward is recomputed.
 *   d_o            [Ttot][Nv][dv] in problem->out_dtype: dL/do. Required.
 *   d_final_state  [N][Nv][dk][dv] fp32, dL/dS_T; NULL means zeros.
 *   dq, dk         [Ttot][Nk][dk] fp32 out (summed over the value heads that
 *                  share a q/k head). Required.
 *   dv             [Ttot][Nv][dv] fp32 out. Required.
 *   dbeta          [Ttot][Nv] fp32 out. Required.
 *   dg             [Ttot][Nv] fp32 out, or NULL to skip. With g == NULL it
 *                  receives the gradient at g = 0.
 *   d_initial_state [N][Nv][dk][dv] fp32 out, or NULL to skip.
 *   workspace      at least gdr_chunk_bwd_workspace_size bytes, 256-byte aligned.
 *   stage_events   NULL, or GDR_BWD_NUM_STAGES + 1 caller-created events
 *                  (NULL entries skipped) recorded on `stream`: [0] before the first kernel and [i]
 *                  after stage i: [1] forward recompute (five kernels), [2]
 *                  preparation (layouts, score block), [3] reverse state
 *                  pass, [4] per-chunk gradients, [5] sum of dq and dk over
 *                  the value heads of each q/k head.
 * The forward recompute runs the five-kernel path; for bf16 inputs at C = 64
 * with at least 128 (sequence, value head, 16 dv columns) units its chunk
 * states and V_new come from the fp16 chunk pass instead (fp16 operands, fp32
 * sums, as in gdr_chunk_fwd). The backward's own arithmetic is fp32 (products
 * on the fp32 matrix cores), and every sum runs in a fixed order: the same
 * inputs give the same bits on every run.
 * Errors as for gdr_chunk_fwd. Asynchronous on `stream`.
 */
#define GDR_BWD_NUM_STAGES 5
gdr_status_t gdr_chunk_bwd_workspace_size(const gdr_problem_t* problem, size_t* bytes);
gdr_status_t gdr_chunk_bwd(const gdr_problem_t* problem,
                           const void* q, const void* k, const void* v,
                           const float* g, const void* beta, float scale,
                           const float* initial_state,
                           const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                           const void* d_o, const float* d_final_state,
                           float* dq, float* dk, float* dv, float* dbeta, float* dg,
                           float* d_initial_state,
                           void* workspace, size_t workspace_bytes, void* stream,
                           void* const* stage_events);

/*
 * Intermediates of the five kernels, for per-kernel parity checks. Each
 * pointer is a caller-owned device buffer (NULL to skip) that receives a copy
 * of the workspace region in the layout the kernels use; sizes follow from
 * the problem and NT, the number of chunks (sum over sequences of
 * ceil(len / C), numbered sequence by sequence in token order). T below is
 * the input type: bf16 when io_dtype is bf16, fp32 when it is fp32. Values
 * derived inside the method are kept in fp32.
 *
 * Fragment conventions (64-lane wavefront, lane l = 16 * qd + r):
 *   a "pair fragment" holds, for each lane, 8 values of a 16 x 32 block X
 *   (rows r, contraction index m in [0, 32)) with element e of lane l equal to
 *   X[r][m(qd, e)], where m(qd, e) = 4*qd + e for e < 4 and 16 + 4*qd + e - 4
 *   for e >= 4. An "accumulator tile" holds 4 values of a 16 x 16 block Y per
 *   lane, element j of lane l equal to Y[4*qd + j][r].
 *
 * Layouts (Nv = num_v_heads, Nk = num_qk_heads, c = chunk, i/j = position in
 * the chunk, tb = i / 16 (C / 16 blocks), db/kp = 16/32-blocks of dk, nb =
 * 16-block of dv, tp = 32-block of chunk positions (NTP = max(1, C / 32)
 * blocks; with C = 16 the one block's positions 16..31 hold zeros)):
 *   G    [Ttot][Nv] fp32                  chunk-local inclusive prefix sum of g
 *   A    [Ttot][Nv][C] fp32               row i of (I + L)^-1 for the token's chunk;
 *                                         zero above the diagonal and past the chunk end
 *   W    [NT][Nv][C/16 tb][dk/32 kp] fp32 pair fragments (rows i, m = dk index)
 *   U    [NT][Nv][C/16 tb][dv/16 nb] fp32 accumulator tiles (rows i, columns dv)
 *   KT   [NT][Nk][dk/16 db][NTP tp] T pair fragments of K^T (rows dk, m = position)
 *   H    [NT][Nv][dv/16 nb][dk/32 kp] fp32 pair fragments of the chunk's
 *                                     entering state transposed (rows dv, m = dk)
 *   VN   [NT][Nv][dv/16 nb][NTP tp] fp32 pair fragments of V_new^T (rows dv, m = position)
 *   T    [NT][Nv][6 pairs] fp16 pair fragments of T = A diag(beta) (rows i,
 *        m = position) for the blocks (tb, tp) = (0,0) (1,0) (2,0) (2,1)
 *        (3,0) (3,1), each value rounded once from fp32 (the operand of the
 *        production pass). bf16 inputs with C = 64 only (NULL otherwise).
 *        The buffer must be 16-byte aligned (else GDR_ERR_SHAPE before
 *        anything runs); so must P's.
 *   P    [NT][Nv][6 pairs] fp16 pair fragments of the score block
 *        P = (Q K^T) (.) D, D_ij = exp(G_i - G_j) for j <= i (rows i, m = j),
 *        same blocks and conditions as T.
 *   R    [NT][Nv][2][C] fp32: exp(G_i) and exp(G_last - G_i) per chunk
 *        position (zero past the chunk end); same conditions as T.
 * Chunk positions past the end of a sequence hold zeros in W, U, KT, VN, T,
 * P and R. The decay matrix D itself is not copied out: it is a function of
 * G alone (ChunkGatedDeltaRule page, formula (5)), so a test forms it from G.
 */
typedef struct {
    float* G;
    void* A;
    void* W;
    void* U;
    void* KT;
    void* H;
    void* VN;
    void* T;
    void* P;
    float* R;
    int64_t num_chunks;     /* out: NT */
} gdr_intermediates_t;

/* Same result as gdr_chunk_fwd up to rounding, computed by the five kernels as
 * separate launches with every derived value in fp32 (the stages of the FLA
 * DeltaNet article, sections 3.1-3.4: K K^T, the solve, W and U, the state
 * pass, the output); then copies the intermediates (asynchronously, on the
 * same stream) into the buffers of `dbg`. For bf16 inputs with C = 64 it also
 * runs the production preparation kernel and copies its T, P and R. The
 * workspace must hold gdr_chunk_fwd_debug_workspace_size bytes; errors as for
 * gdr_chunk_fwd (GDR_ERR_WORKSPACE when it is smaller). */
gdr_status_t gdr_chunk_fwd_debug(const gdr_problem_t* problem,
                                 const void* q, const void* k, const void* v,
                                 const float* g, const void* beta, float scale,
                                 const float* initial_state,
                                 const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                                 void* o, float* final_state,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 gdr_intermediates_t* dbg);

/* Number of kernel stages of one forward call. */
#define GDR_NUM_STAGES 6

/*
 * As gdr_chunk_fwd, and also records the caller-created HIP events
 * stage_events[0 .. GDR_NUM_STAGES] (hipEvent_t handles) on `stream`: [0]
 * before the first kernel and [i] after stage i, the stages being [1] chunk
 * table, [2] gate prefix sums, [3] A-build + solve, [4] w/u, [5] state pass,
 * [6] output. On the bf16 C = 64 path stages [2], [4] and [6] launch nothing:
 * [3] is the preparation kernel (gate sums included) and [5] the chunk-serial
 * pass with the w/u products and the output. A NULL entry is skipped (that
 * event is not recorded), so a timed loop can bracket one stage alone: each
 * recorded event puts a few microseconds between two launches. Nothing is
 * synchronised; the caller reads the elapsed times once the stream has passed
 * the last event. Used to time each kernel inside a benchmark's timed region.
 */
gdr_status_t gdr_chunk_fwd_timed(const gdr_problem_t* problem,
                                 const void* q, const void* k, const void* v,
                                 const float* g, const void* beta, float scale,
                                 const float* initial_state,
                                 const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                                 void* o, float* final_state,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 void* const* stage_events);

/* Static description of a status code. */
const char* gdr_status_string(gdr_status_t status);

/* Detail message of the last error reported on the calling thread ("" if none). */
const char* gdr_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
