// Opt-in per-kernel timing with HIP events (benchmark support).
#pragma once

#include <hip/hip_runtime.h>

namespace ssm {

// Kinds of kernels the library launches; indices of ssm_profile_read().
enum : int {
  kKindWiden = 0,   // bf16 -> f32 copy of the B / C rows
  kKindAgg = 1,     // per-chunk aggregates
  kKindCarry = 2,   // carries across chunk boundaries
  kKindMain = 3,    // main scan pass
  kKindFill = 4,    // last_state of an empty sequence (L == 0)
  kKindUpdate = 5,  // single-token state update
  kKindConv = 6,    // causal depthwise convolution over a sequence
  kKindConvUpdate = 7,  // single-token convolution-state update
  kKindBwdRows = 8,     // backward: B / C rows padded to 16 states
  kKindBwdAgg = 9,      // backward: per-chunk aggregate of the state gradient (reverse in time)
  kKindBwdCarry = 10,   // backward: chain of the state gradient across chunks
  kKindBwdMain = 11,    // backward: recompute states, gradients of every input
  kKindBwdReduce = 12,  // backward: sums of the per-chunk / per-block partial gradients
  kKindSsdState = 13,   // scalar-per-head scan: chunk states (matrix products)
  kKindSsdCarry = 14,   // scalar-per-head scan: chain of chunk states
  kKindSsdScan = 15,    // scalar-per-head scan: chunk outputs (matrix products)
  kKindFused = 16,      // single-pass scan: chunks of a block joined through LDS
  kNumKinds = 17
};

// When profiling is on, creates and records the start event on `s` and returns true.
bool profile_begin(hipStream_t s, hipEvent_t* ev0, hipEvent_t* ev1);
// Records the stop event and files the pair under `kind`.
void profile_end(int kind, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);

}  // namespace ssm
