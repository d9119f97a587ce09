// Internal interface between the C-ABI layer (ssm_api.hip) and the kernel
// launchers (ssm_kernels.hip).  Arguments have already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

// Forms of the forward scan.
constexpr int kPathAuto = 0;        // chosen from the sizes
constexpr int kPathChunked = 1;     // one pass per chunk of the sequence (with aggregate + carry passes when cut)
constexpr int kPathSinglePass = 2;  // the single-pass form (ssm_fused.hip)

// Explicit plan choices of a forward scan; zero fields leave the choice to the sizes.
struct ScanTuning {
  int path = kPathAuto;
  int min_chunk = 0;     // chunked form: shortest chunk (steps)
  int target_waves = 0;  // chunked form: waves the cut aims for
};

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
  ScanTuning tune;
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
ScanPlan plan_scan(int64_t b, int64_t L, int64_t E, int elem_bytes, const ScanTuning& tune = ScanTuning{});

// State slots per channel in the chunk-state buffers (N, or 16 when N is not 4, 8 or 16).
int chunk_state_slots(int64_t N);

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

// The single-pass scan (ssm_fused.hip): a workgroup walks the whole sequence for a
// slice of channels, in blocks of W chunks of 8 steps joined through LDS.
constexpr int kFusedMaxWaves = 16;
struct FusedPlan {
  int lpc;         // lanes per channel (4 states each): 1, 2 or 4
  int cg;          // channels per workgroup (of one batch row)
  int W;           // chunks per block
  int BT;          // steps per block (W * 8)
  int groups_row;  // workgroups per batch row
  int n_wg;        // workgroups
  int lanes;       // compute lanes: W * lpc * cg
  int n_cmp;       // compute waves (the first ones); the lanes of chunk 0 chain the block's chunks
  int n_prod;      // producer waves after them: global <-> LDS tiles
  int n_threads;   // 64 * (n_cmp + n_prod)
  int nblk;        // blocks over the sequence
  int ux, ub;      // bytes one producer lane moves per access: rows of u, delta, z, y / rows of B, C
  int xR, xM;      // u, delta, z, y tiles: rows per producer pass, passes per block
  int bR, bM;      // B, C tiles: rows per producer pass, passes per block
  int xrows, brows;  // rows of an LDS tile (xR * xM, bR * bM >= BT: the last pass may run past BT)
  int o_x[3], o_bc[3], o_agg, o_hin, o_y[2], o_junk;  // LDS byte offsets (tiles triple / double buffered)
  int lds_bytes;
};
// Most chunks per block the single-pass form takes (the chain of their maps is serial).
constexpr int kFusedMaxChunks = 16;
// Most chunks per block it takes when the form is chosen from the sizes: at 4
// chunks (b8 L2048 E1536 bf16) it ran 18% faster than the chunked form, at 11
// (b1 L65536 E5120 bf16, 20 channels per CU) 17% slower.
constexpr int kFusedChainMax = 8;
// Plans the single-pass scan for this call with at most max_w chunks per block;
// false when it does not apply (too few channels to fill the chip, rows that
// are not whole 8-byte units, or tiles that do not fit in LDS).
bool plan_fused(const ScanArgs& a, int n_cu, int max_w, FusedPlan* p);
hipError_t launch_fused(const ScanArgs& a, const FusedPlan& p);

// The form a forward scan takes: kPathChunked or kPathSinglePass (then *fp is
// its plan), or -1 when a.tune asks for the single pass and it does not apply.
int choose_path(const ScanArgs& a, const ScanPlan& pl, int n_cu, FusedPlan* fp);
// Compute units of the current device.
hipError_t device_cu_count(int* n_cu);
// Bytes of workspace the chunked form of this scan needs (0 for one chunk).
size_t chunked_workspace_bytes(const ScanArgs& a, const ScanPlan& pl);

// Size of the fixed device buffer of ssm_scan_fwd_noalloc (ssm_noalloc.hip).
constexpr size_t kScratchBytes = size_t(128) << 20;
// Device address of the current device's copy of that buffer (taken once per device).
hipError_t scratch_address(void** out);

// Both return hipSuccess or the first HIP error met while enqueueing.  A cut
// chunked scan takes its workspace from `workspace` when given (at least
// chunked_workspace_bytes), else from the stream-ordered pool.
hipError_t launch_scan(const ScanArgs& a, void* workspace = nullptr, size_t workspace_bytes = 0);
hipError_t launch_state_update(const UpdateArgs& a);

}  // namespace ssm
