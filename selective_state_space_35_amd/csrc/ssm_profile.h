// Opt-in per-kernel timing with HIP events (benchmark support).
#pragma once

#include <hip/hip_runtime.h>

namespace ssm {

// Kinds of kernels the library launches; indices of ssm_profile_read().
enum : int {
  kKindAgg = 0,         // per-chunk aggregates
  kKindCarry = 1,       // carries across chunk boundaries
  kKindMain = 2,        // main scan pass
  kKindFill = 3,        // last_state of an empty sequence (L == 0)
  kKindUpdate = 4,      // single-token state update
  kKindConv = 5,        // causal depthwise convolution over a sequence
  kKindConvUpdate = 6,  // single-token convolution-state update
  kKindBwdRows = 7,     // backward: B / C rows padded to 16 states
  kKindBwdAgg = 8,      // backward: per-chunk maps (reverse in time; without saved states also the forward ones)
  kKindBwdCarry = 9,    // backward: chain of the state gradient across chunks
  kKindBwdMain = 10,    // backward: recompute states, gradients of every input
  kKindBwdReduce = 11,  // backward: sums of the per-chunk / per-block partial gradients
  kKindSsdState = 12,   // scalar-per-head scan: chunk states (matrix products)
  kKindSsdCarry = 13,   // scalar-per-head scan: chain of chunk states
  kKindSsdScan = 14,    // scalar-per-head scan: chunk outputs (matrix products)
  kKindFused = 15,      // single-pass scan: chunks of a block joined through LDS
  kKindWiden = 16,      // bf16 -> f32 copy of the B / C rows of a cut scan
  kNumKinds = 17
};

// When profiling is on, creates and records the start event on `s` and returns true.
bool profile_begin(hipStream_t s, hipEvent_t* ev0, hipEvent_t* ev1);
// Records the stop event and files the pair under `kind`.
void profile_end(int kind, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);

}  // namespace ssm
