// ssm_calib.hip -- issue-rate calibration kernels for the ALU roofline of the
// scan kernels (libssm_calib.so, benchmark support; not part of libssm.so).
//
// The scan's inner step needs, per (step, channel, state), one exp2 on the
// transcendental unit and a handful of plain fp32 VALU operations (two
// products and two fused multiply-adds).  The kernels below time exactly
// those instruction kinds in isolation and mixed, built with the library's
// own flags (gfx950, packed-FP32 selection off), so the ALU ceiling quoted for
// the scan kernels rests on measured rates of this chip and toolchain:
//
//   kind 0  v_fma_f32 only        4 independent FMAs per chain step, 8 chains per lane
//   kind 1  v_exp_f32 only        1 exp per chain step, 8 chains per lane
//   kind 2  4 FMA + 1 exp         per chain step (the scan's per-state mix)
//   kind 3  2 FMA + 1 exp         per chain step
//   kind 4  v_mul_f32 with a DPP quad broadcast operand, 4 per chain step
//   kind 5  v_add_f32 only        4 per chain step (a second plain VALU opcode)
//
// Every operand is a runtime value (loaded from memory), so nothing folds;
// each lane runs 8 independent dependency chains so a few waves per SIMD
// cover the pipeline latency.  The counted work is in lane-operations:
// (FMA/add/mul instructions) x 64 lanes, and transcendentals likewise.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kChains = 8;
constexpr int kThreads = 256;  // 4 waves: one per SIMD of a CU

// the value of quad lane j in every lane of the quad (DPP quad_perm [j, j, j, j]); j folds to a constant
__device__ __forceinline__ float quad_lane(float v, int j) {
  const int b = __float_as_int(v);
  switch (j) {
    case 0: return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x00, 0xF, 0xF, false));
    case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x55, 0xF, 0xF, false));
    case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0xAA, 0xF, 0xF, false));
    default: return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0xFF, 0xF, 0xF, false));
  }
}

template <int NF, int NE, int KIND>
__global__ __launch_bounds__(kThreads) void alu_probe(const float* __restrict__ in, float* __restrict__ out,
                                                      int iters) {
  const float c0 = in[0];  // 1.0 at run time
  const float c1 = in[1];  // a small increment
  float f[kChains], e[kChains];
#pragma unroll
  for (int k = 0; k < kChains; k++) {
    f[k] = in[2 + k] + float(threadIdx.x) * 1e-7f;
    e[k] = in[2 + kChains + k];
  }
  for (int i = 0; i < iters; i++) {
#pragma unroll
    for (int r = 0; r < NF; r++) {
#pragma unroll
      for (int k = 0; k < kChains; k++) {
        if constexpr (KIND == 4) {
          // product with a value broadcast from quad lane r % 4 (DPP quad_perm folded into the multiply)
          f[k] = f[k] * quad_lane(f[(k + 1) % kChains], r % 4);
        } else if constexpr (KIND == 5) {
          f[k] = f[k] + c1;
        } else {
          f[k] = fmaf(f[k], c0, c1);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < NE; r++) {
#pragma unroll
      for (int k = 0; k < kChains; k++) e[k] = __builtin_amdgcn_exp2f(-e[k]);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; k++) s += f[k] + e[k];
  out[int64_t(blockIdx.x) * kThreads + threadIdx.x] = s;
}

float* g_in = nullptr;
float* g_out = nullptr;
int64_t g_out_blocks = 0;

template <int NF, int NE, int KIND>
hipError_t run(int blocks, int iters, int reps, double* ms, double* valu_lane_ops, double* trans_lane_ops) {
  const int64_t threads = int64_t(blocks) * kThreads;
  *valu_lane_ops = double(threads) * iters * kChains * NF * reps;
  *trans_lane_ops = double(threads) * iters * kChains * NE * reps;
  hipLaunchKernelGGL((alu_probe<NF, NE, KIND>), dim3(blocks), dim3(kThreads), 0, 0, g_in, g_out, iters);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipEvent_t e0, e1;
  if ((err = hipEventCreate(&e0)) != hipSuccess) return err;
  if ((err = hipEventCreate(&e1)) != hipSuccess) return err;
  (void)hipEventRecord(e0, 0);
  for (int r = 0; r < reps; r++)
    hipLaunchKernelGGL((alu_probe<NF, NE, KIND>), dim3(blocks), dim3(kThreads), 0, 0, g_in, g_out, iters);
  (void)hipEventRecord(e1, 0);
  err = hipEventSynchronize(e1);
  float t = 0.f;
  (void)hipEventElapsedTime(&t, e0, e1);
  *ms = double(t);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return err == hipSuccess ? hipGetLastError() : err;
}

}  // namespace

extern "C" {

// Runs probe `kind` (0..5) on `blocks` workgroups of 256 threads, `iters`
// chain steps per thread, `reps` timed launches after one untimed launch.
// Writes the total time of the timed launches and the VALU and
// transcendental lane-operations they executed.  Returns 0, -1 for a bad
// argument, or the HIP error code.  Allocates its own small buffers on first
// use (calibration only).
__attribute__((visibility("default"))) int ssm_calib_alu(int kind, int blocks, int iters, int reps, double* ms,
                                                         double* valu_lane_ops, double* trans_lane_ops) {
  if (blocks <= 0 || blocks > (1 << 20) || iters <= 0 || reps <= 0 || !ms || !valu_lane_ops || !trans_lane_ops)
    return -1;
  if (!g_in) {
    float h[2 + 2 * kChains];
    h[0] = 1.0f;
    h[1] = 1e-7f;
    for (int k = 0; k < kChains; k++) {
      h[2 + k] = 0.5f + 0.01f * k;
      h[2 + kChains + k] = 0.3f + 0.05f * k;
    }
    if (hipMalloc(&g_in, sizeof(h)) != hipSuccess) return -2;
    if (hipMemcpy(g_in, h, sizeof(h), hipMemcpyHostToDevice) != hipSuccess) return -2;
  }
  if (blocks > g_out_blocks) {
    if (g_out) (void)hipFree(g_out);
    if (hipMalloc(&g_out, size_t(blocks) * kThreads * sizeof(float)) != hipSuccess) return -2;
    g_out_blocks = blocks;
  }
  hipError_t err;
  switch (kind) {
    case 0: err = run<4, 0, 0>(blocks, iters, reps, ms, valu_lane_ops, trans_lane_ops); break;
    case 1: err = run<0, 1, 1>(blocks, iters, reps, ms, valu_lane_ops, trans_lane_ops); break;
    case 2: err = run<4, 1, 2>(blocks, iters, reps, ms, valu_lane_ops, trans_lane_ops); break;
    case 3: err = run<2, 1, 3>(blocks, iters, reps, ms, valu_lane_ops, trans_lane_ops); break;
    case 4: err = run<4, 0, 4>(blocks, iters, reps, ms, valu_lane_ops, trans_lane_ops); break;
    case 5: err = run<4, 0, 5>(blocks, iters, reps, ms, valu_lane_ops, trans_lane_ops); break;
    default: return -1;
  }
  return err == hipSuccess ? 0 : int(err);
}

}  // extern "C"
