// Device helpers shared by the library's kernel files (bf16 access, buffer
// resources, the scalar functions of the method) and the launch wrapper.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssm_profile.h"

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

typedef uint16_t bf16_bits;  // bfloat16 values are passed around as their raw 16 bits

__device__ __forceinline__ float load_elem(const float* p) { return *p; }
__device__ __forceinline__ float load_elem(const bf16_bits* p) { return __uint_as_float(uint32_t(*p) << 16); }
__device__ __forceinline__ void store_elem(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_elem(bf16_bits* p, float v) {
  *p = __builtin_bit_cast(bf16_bits, static_cast<__bf16>(v));  // v_cvt_pk_bf16_f32: round to nearest even
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// softplus(x) = log(1 + e^x) = max(x, 0) + log(1 + e^{-|x|}); both terms finite for every finite x.
__device__ __forceinline__ float softplus(float x) {
  const float e = exp2_fast(-fabsf(x) * kLog2e);
  return fmaxf(x, 0.f) + __builtin_amdgcn_logf(1.f + e) * kLn2;
}

// silu(z) = z * sigmoid(z) = z / (1 + e^{-z})   ([AB] row 5)
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.f + exp2_fast(-z * kLog2e));
}

__device__ __forceinline__ float sigmoid(float x) { return __builtin_amdgcn_rcpf(1.f + exp2_fast(-x * kLog2e)); }

// Cross-lane reads inside a quad of lanes (DPP quad_perm).
__device__ __forceinline__ float quad_xor1(float v) {  // value of lane ^ 1 within the quad
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_xor2(float v) {  // value of lane ^ 2 within the quad
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
}
// value of quad lane j, for every lane of the quad (DPP quad_perm [j, j, j, j]);
// j is a constant once the calling loop is unrolled, so the switch folds away
__device__ __forceinline__ float quad_bcast(float v, int j) {
  const int b = __float_as_int(v);
  switch (j) {
    case 0: return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x00, 0xF, 0xF, false));
    case 1: return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x55, 0xF, 0xF, false));
    case 2: return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0xAA, 0xF, 0xF, false));
    default: return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0xFF, 0xF, 0xF, false));
  }
}

// Raw buffer resource over a tensor region (CDNA buffer descriptor: 48-bit
// base, no stride, 2 GiB range, dword3 as used for gfx9-family buffer ops).
// Per-step loads then need one lane-offset VGPR shared by every stream and a
// wave-uniform row offset in an SGPR, instead of one 64-bit address per load.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ float buf_load(__amdgpu_buffer_rsrc_t r, int voff, int soff, float*) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ float buf_load(__amdgpu_buffer_rsrc_t r, int voff, int soff, bf16_bits*) {
  return __uint_as_float(uint32_t(__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0)) << 16);
}
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, int voff, int soff, float v, float*) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff, soff, 0);
}
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, int voff, int soff, float v, bf16_bits*) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(bf16_bits, static_cast<__bf16>(v)), r, voff, soff, 0);
}

// Every launch goes through here.  With profiling on, it is bracketed by two
// HIP events on the launch stream (see ssm_profile_enable in ssm.h).
template <typename Kern, typename... Args>
hipError_t launch_kind(int kind, Kern k, int64_t blocks, int threads, hipStream_t s, Args... args) {
  if (blocks <= 0) return hipSuccess;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  const bool prof = profile_begin(s, &ev0, &ev1);
  hipLaunchKernelGGL(k, dim3(unsigned(blocks)), dim3(threads), 0, s, args...);
  hipError_t err = hipGetLastError();
  if (prof) profile_end(kind, s, ev0, ev1);
  return err;
}

}  // namespace ssm
