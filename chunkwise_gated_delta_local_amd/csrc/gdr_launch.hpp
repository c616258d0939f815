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
    void* o;
    float* ST;                 // NULL: not written
    // workspace regions
    int32_t *chunk_seq, *chunk_start, *chunk_len, *seq_first;
    float* G;
    void *A, *W, *U, *KT, *H, *VN;   // reference-pipeline intermediates
    void* Tf;                        // T = A diag(beta) fragments (fused pipeline)
    void* Pf;                        // score block (Q K^T) (.) D fragments (fused pipeline)
    void* R;                         // decay factors exp(G), exp(G_last - G), chunk-major (fused pipeline)
    bool reference;                  // run the five separate kernels even for bf16
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
