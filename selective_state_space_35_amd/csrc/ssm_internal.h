// Internal interface between the C-ABI layer (ssm_api.hip) and the kernel
// launchers (ssm_kernels.hip).  Arguments have already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

struct ScanArgs {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;      // nullable
  const void* z;       // nullable
  const float* bias;   // nullable
  int softplus;
  void* y;
  float* last_state;   // nullable
  const float* h0;     // nullable: incoming state [b, E, N] (zero when null)
  float* saved;        // nullable: the state after every kSaveEvery-th step, [b, K, E, N], K = ceil(L / kSaveEvery) - 1
  int64_t b, L, E, N;
  int dtype;           // 0 = f32, 1 = bf16
  hipStream_t stream;
};
constexpr int64_t kSaveEvery = 64;  // interval of the saved states (the backward's chunk)

struct UpdateArgs {
  float* state;
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;      // nullable
  const void* z;       // nullable
  const float* bias;   // nullable
  int softplus;
  void* y;
  int64_t b, E, N;
  int dtype;
  hipStream_t stream;
};

// Causal depthwise convolution (sequence form and token form).
struct ConvArgs {
  const void* v;         // [b, L, E] (sequence) or [b, E] (token)
  const float* q;        // [E, K]
  const float* cb;       // [E], nullable
  const void* state_in;  // [b, E, K], nullable (sequence form)
  void* x;               // output, same shape as v
  void* state_out;       // [b, E, K]: written (sequence form, nullable) / updated in place (token form)
  int64_t b, L, E, K;
  int dtype;
  hipStream_t stream;
};

constexpr int kMaxConvK = 8;
int64_t conv_chunk_steps();  // steps per wave of the sequence kernel
hipError_t launch_conv_fwd(const ConvArgs& a);
hipError_t launch_conv_update(const ConvArgs& a);

// How a scan is split along the sequence: n_chunks chunks of chunk_len steps.
struct ScanPlan {
  int64_t chunk_len;
  int n_chunks;
  int e_blocks;  // ceil(E / 64): one 64-lane wave covers 64 channels
};

// elem_bytes: size of the streamed element type (4 for f32, 2 for bf16).
// chunk_len == 0 means the row size is too large to address (rejected).
ScanPlan plan_scan(int64_t b, int64_t L, int64_t E, int elem_bytes);

// State slots per channel in the chunk-state buffers (N, or 16 when N is not 4, 8 or 16).
int chunk_state_slots(int64_t N);
// Incoming state of every chunk of the scan described by `a` cut as `pl` says:
// afterwards carry[(b * n_chunks + c) * E + e][slots] holds the state at the end
// of chunk c (c < n_chunks - 1) and csum the sum of steps of chunk c.  `rows`
// (2 * b * L * N floats) is scratch for widened bf16 rows.  y / last_state are
// not touched.
hipError_t launch_chunk_states(const ScanArgs& a, const ScanPlan& pl, float* rows, float* carry, float* csum);

// Backward of the scan (gradients of every input).
struct BwdArgs {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;      // nullable
  const void* z;       // nullable
  const float* bias;   // nullable
  int softplus;
  const float* h0;     // nullable
  const void* dy;
  const float* dlast;  // nullable
  void* du;
  void* ddelta;
  float* dA;
  float* dB;
  float* dC;
  float* dD;           // nullable
  void* dz;            // required when z is given
  float* dbias;        // nullable
  float* dh0;          // nullable
  const float* saved;  // nullable: the forward's states every kSaveEvery steps (ScanArgs::saved)
  int64_t b, L, E, N;
  int dtype;
  hipStream_t stream;
};
int64_t bwd_chunk_steps();  // steps per chunk of the backward
hipError_t launch_scan_bwd(const BwdArgs& a);

// The scan with a scalar transition per head, in chunks of matrix products (bf16 I/O).
struct SsdArgs {
  const void* x;       // [b, L, H * P]
  const void* delta;   // [b, L, H]
  const float* A;      // [H]
  const void* B;       // [b, L, N]
  const void* C;       // [b, L, N]
  const float* D;      // [H], nullable
  const void* z;       // [b, L, H * P], nullable
  const float* bias;   // [H], nullable
  int softplus;
  const float* h0;     // [b, H * P, N], nullable
  void* y;             // [b, L, H * P]
  float* last_state;   // [b, H * P, N], nullable
  int64_t b, L, H, N;
  hipStream_t stream;
};
int64_t ssd_chunk_steps();  // steps per chunk
int64_t ssd_head_dim();     // channels per head (P)
int64_t ssd_max_channels(); // largest H * P the chunk kernels address with 32-bit offsets
hipError_t launch_ssd(const SsdArgs& a);

// Both return hipSuccess or the first HIP error met while enqueueing.
hipError_t launch_scan(const ScanArgs& a);
hipError_t launch_state_update(const UpdateArgs& a);

}  // namespace ssm
