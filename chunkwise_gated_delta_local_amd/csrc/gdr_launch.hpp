// Internal interface between the host API (gdr_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

struct LaunchArgs {
    bool bf16;                 // compute/io type: bf16 (true) or fp32
    int dk, dv;
    int C;                     // chunk size: 64, or 16 / 32 (five-kernel path)
    int32_t Nk, Nv, N;         // q/k heads, v heads, sequences
    int64_t T_row, Ttot;       // tokens per batch row (fixed length), total tokens
    int32_t nt, nt_cap;        // chunks used, chunk-table capacity
    const void *q, *k, *v, *beta;
    int beta_f32;
    int out_f32;               // o in fp32 (else in the io type)
    const float* g;            // NULL: ungated
    const float* S0;           // NULL: zeros
    float scale;
    const int32_t* cu_dev;     // NULL: fixed length
    void* o;                   // NULL on the five-kernel path: no output kernel (the backward's recompute)
    float* ST;                 // NULL: not written
    // workspace regions
    int32_t *chunk_seq, *chunk_start, *chunk_len, *seq_first;
    float* G;
    void *A, *W, *U, *KT, *H, *VN;   // reference-pipeline intermediates
    void* T16;                       // T = A diag(beta), fp16 pair fragments [cap][Nv][6][64][8] (fp16 path)
    void* P16;                       // score block (Q K^T) (.) D, same layout (fp16 path)
    float* R16;                      // decay rows exp(G), exp(G_last - G): [cap][Nv][2][64] (fp16 path)
    void* K16;                       // K rows in fp16, [cap][Nk][64][dk], 16-byte units swizzled (fp16 path)
    void* Q16;                       // Q rows, same layout (fp16 path)
    bool reference;                  // run the five separate kernels even for bf16
    bool prep_only;                  // fp16 path: run k_prep only (debug copies of T, P, R)
    bool states16;                   // five-kernel run whose state pass is the fp16 chunk pass
                                     // (backward recompute, bf16 with C = 64): H and VN from it
    // segment-parallel state passing (nseg == 0: one serial pass per sequence)
    int32_t nseg;                    // segment-table capacity: the host's count of segments
    int32_t seg_chunks;              // chunks per segment
    int32_t *seg_first, *seq_seg;    // [nseg + 1], [N + 1]
    float *Sloc, *Mseg, *Sstart;     // local end states, transitions, entering states (fp32)
    hipStream_t stream;
};

// Enqueues the whole forward on a.stream. bf16 inputs with C = 64 take the
// fused path (state pass and output in one kernel) unless a.reference is set;
// fp32 inputs and C = 16 or 32 take the five-kernel path. events: NULL, or 7 events recorded
// before the first and after every one of the six stages.
hipError_t launch_forward(const LaunchArgs& a, hipEvent_t* events);

// Backward pass (gdr_backward.hip): recomputes the forward on the five-kernel
// path (fwd.reference must be set; fwd.o is a scratch output), then the
// reverse state pass and the per-chunk gradients.
struct BackwardArgs {
    LaunchArgs fwd;
    const void* d_o;           // [Ttot][Nv][dv], fp32 (do_f32) or bf16
    int do_f32;
    const float* dST;          // [N][Nv][dk][dv] or NULL (zeros)
    float *dq, *dk;            // [Ttot][Nk][dk]
    float *dv;                 // [Ttot][Nv][dv]
    float *dbeta, *dg;         // [Ttot][Nv]; dg may be NULL
    float* dS0;                // [N][Nv][dk][dv] or NULL
    // workspace (fp32, natural row-major layouts)
    float *P;                  // [NT][Nv][C][C] score block (Q K^T) (.) D
    float *Hn;                 // [NT][Nv][dv][dk] entering states, transposed
    float *Vn, *dVn;           // [Ttot][Nv][dv] V_new and its gradient
    float *WT;                 // [NT][Nv][dk][C] W^T per chunk (zero past the chunk end)
    float *dWs;                // [Ttot][Nv][dk] the gradient of W
    float *dSout;              // [NT][Nv][dv][dk] gradients of the outgoing states, transposed
    float *dqv, *dkv;          // [Ttot][Nv][dk] dq, dk per value head
    hipEvent_t* events;        // NULL, or 6 events: before the forward recompute and after
                               // it, the preparation, the state pass, the per-chunk pass, the sum
};
hipError_t launch_backward(const BackwardArgs& b);

// Token-by-token forward (gdr_recurrent.hip): no workspace.
struct RecurrentArgs {
    bool bf16;
    int dk, dv;
    int32_t Nk, Nv, N;
    int64_t T_row, Ttot;
    const void *q, *k, *v, *beta;
    int beta_f32, out_f32, l2norm;
    const float* g;
    const float* S0;
    float scale;
    const int32_t* cu_dev;     // NULL: fixed length T_row per sequence
    void* o;
    float* ST;
    hipStream_t stream;
};
hipError_t launch_recurrent(const RecurrentArgs& a);

}  // namespace gdr
