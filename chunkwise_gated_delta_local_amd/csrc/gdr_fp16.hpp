// Internal interface of the fp16 production path (gdr_fp16.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "gdr_launch.hpp"

namespace gdr {

// Modes of the fp16 chunk pass: state and output (serial pass, or the last
// pass of segment-parallel state passing), or state only (segment passes).
// kStates16: state only, for the backward's recompute: every chunk's entering
// state and V_new are written (fp32) instead of the output.
constexpr int kFull16 = 0, kSegment16 = 1, kStates16 = 2;

// fp16 values of the six T (or score-block) pair fragments of one (chunk,
// value head) as the workspace holds them: the two pairs whose second half
// lies above the diagonal keep only their first half (2 x 256 + 4 x 512).
constexpr int kPackedPairs = 2560;

// Expands `sets` packed pair sets into the six-fragment layout of the debug
// intermediates (6 x 512 fp16 values per set, the dropped halves zero).
hipError_t unpack_pairs16(const void* packed, void* dense, int64_t sets, hipStream_t stream);

// Enqueues stages 2..6 of the forward for bf16 inputs with C = 64 (the chunk
// and segment tables are built by the caller): k_prep, then the chunk pass (or
// the two segment passes, the scan and the output pass). Records events
// [2] .. [6] when `ev` is given. With a.prep_only set, only k_prep runs (the
// debug entry point's copy of T, P and the decay rows).
hipError_t launch_fp16_path(const LaunchArgs& a, hipEvent_t* ev);

// The backward's recompute of the chunk states on this path (bf16, C = 64):
// k_prep, then the chunk pass in kStates16 mode, writing into a.H the
// chunk-entering states transposed ([NT][Nv][dv][dk] fp32) and into a.VN
// V_new ([NT][Nv][dv/16][2] fp32 pair fragments of V_new^T, the five-kernel
// path's layout).
hipError_t launch_fp16_states(const LaunchArgs& a);

// Segment scan over the segments of every (sequence, value head, 16 columns)
// (gdr_kernels.hip): S_start[j] and the final state from S0, M and S_loc.
hipError_t launch_segment_scan(const LaunchArgs& a);

}  // namespace gdr
