// ssm_kernels.hip -- gfx950 (CDNA4) kernels of the S6 selective scan and of
// the single-token state update, plus their host-side launchers.
//
// Pages that define the arithmetic (title, site):
//   [KK] "mamba, from scratch" (khushi keswani)
//   [AB] "Mamba: Linear-Time Sequence Modeling with Selective State Spaces" (abhik.ai)
//
// Per step t, channel e, state n (float32 throughout):
//   d   = softplus(delta + bias)            [KK] "from ssm to selective ssm"
//   h_n = exp(d*A_n) * h_n + (d*u) * B_n    [AB] "Original paper, equations and
//                                           runnable CPU code", row 2
//   y   = (sum_n C_n h_n + D*u) * silu(z)   same row 2; [AB] row 5
//
// Layout on the GPU
// -----------------
// One lane owns one channel and keeps all N (<= 16) states of it in VGPRs.
// A 64-lane wave covers 64 consecutive channels, so every per-step load of
// u/delta/z and store of y is one contiguous 128-byte (bf16) or 256-byte
// (fp32) row segment.  B_t and C_t are shared by all channels of a batch
// row, hence wave-uniform: they are fetched with scalar loads into SGPRs and
// (bf16) widened on the scalar ALU, costing no VALU and no LDS.
//
// Splitting the sequence
// ----------------------
// The recurrence is an associative affine map per (channel, state)
// ([KK] "the scan": (a2, b2) o (a1, b1) = (a2 a1, a2 b1 + b2); [AB] "Compose
// the updates instead of waiting for every state").  When the batch x channel
// count alone cannot fill the GPU (the long-sequence case has only 80 waves of
// channels), the sequence is cut into chunks and processed in three launches:
//   1. scan_chunk_agg_kernel: per chunk, the state reached from zero and the
//      sum of the steps d (the product of the retentions over the chunk is
//      exp(A_n * sum d), so its "a" half needs no per-state work);
//   2. chain_kernel (ssm_chain.h): the chain of the chunk aggregates, giving
//      every chunk its incoming state;
//   3. scan_main_kernel: every chunk rescans from its incoming state and
//      writes y (and the last chunk writes last_state).
// Only y and last_state are written to HBM besides the small per-chunk
// workspace (b * chunks * E * (N + 1) floats).  Nothing here is a dense
// contraction, so no MFMA is used.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "ssm_chain.h"
#include "ssm_device.h"
#include "ssm_internal.h"
#include "ssm_profile.h"

namespace ssm {
namespace {

// Row of NS coefficients of B or C at one (batch, step).  The row address is
// wave-uniform, so a row is fetched with scalar loads into SGPRs one step
// ahead (RowBuf) and unpacked to floats when the step uses it (unpack_row).
// EXACT means N == NS; otherwise entries n >= N read as zero, which keeps
// padded states at zero.
//
// A bf16 row is fetched as the 32-bit words that cover it and split on the
// scalar ALU.  `odd` says that the row starts in the upper half of a word (odd
// N, or a tensor that starts 2 bytes into a word); the caller tracks it from
// the element index (a pointer turned into an integer here would keep the
// loads off the scalar unit).  Every word read lies inside the aligned words
// that hold the row's own values.
template <typename T, int NS>
struct RowBuf;
template <int NS>
struct RowBuf<float, NS> {
  float v[NS];
};
template <int NS>
struct RowBuf<bf16_bits, NS> {
  uint32_t w[NS / 2 + 1];
  int odd;
};

template <int NS, bool EXACT>
__device__ __forceinline__ void fetch_row(const float* __restrict__ row, int /*odd*/, int N, RowBuf<float, NS>& r) {
#pragma unroll
  for (int n = 0; n < NS; n++) r.v[n] = (EXACT || n < N) ? row[n] : 0.f;
}

template <int NS, bool EXACT>
__device__ __forceinline__ void fetch_row(const bf16_bits* __restrict__ row, int odd, int N,
                                          RowBuf<bf16_bits, NS>& r) {
  const uint32_t* __restrict__ w = reinterpret_cast<const uint32_t*>(row - odd);
  r.odd = odd;
#pragma unroll
  for (int k = 0; k < NS / 2; k++) r.w[k] = (EXACT || 2 * k < N + odd) ? w[k] : 0u;  // word k holds a value
  r.w[NS / 2] = (NS < N + odd) ? w[NS / 2] : 0u;
}

template <int NS, bool EXACT>
__device__ __forceinline__ void unpack_row(const RowBuf<float, NS>& r, int /*N*/, float (&out)[NS]) {
#pragma unroll
  for (int n = 0; n < NS; n++) out[n] = r.v[n];
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

template <int NS, bool EXACT>
__device__ __forceinline__ void unpack_row(const RowBuf<bf16_bits, NS>& r, int N, float (&out)[NS]) {
  if (r.odd == 0) {  // value 2k is the low half of word k, value 2k + 1 its high half
#pragma unroll
    for (int k = 0; k < NS / 2; k++) {
      out[2 * k] = (EXACT || 2 * k < N) ? bf16_lo(r.w[k]) : 0.f;
      out[2 * k + 1] = (EXACT || 2 * k + 1 < N) ? bf16_hi(r.w[k]) : 0.f;
    }
  } else {  // value 2k is the high half of word k, value 2k + 1 the low half of word k + 1
#pragma unroll
    for (int k = 0; k < NS / 2; k++) {
      out[2 * k] = (EXACT || 2 * k < N) ? bf16_hi(r.w[k]) : 0.f;
      out[2 * k + 1] = (EXACT || 2 * k + 1 < N) ? bf16_lo(r.w[k + 1]) : 0.f;
    }
  }
}

// bf16 -> f32 copy of the B and C rows (b*L*N values each), for a scan cut
// into chunks.
__global__ __launch_bounds__(256) void widen_rows_kernel(const bf16_bits* __restrict__ B,
                                                         const bf16_bits* __restrict__ C, float* __restrict__ Bf,
                                                         float* __restrict__ Cf, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) {
    Bf[i] = load_elem(B + i);
    Cf[i] = load_elem(C + i);
  }
}

// Steps per software-pipelined group: the inputs of the next group are in
// flight while the current group computes.
#ifndef SSM_KGROUP
#define SSM_KGROUP 4
#endif
constexpr int kGroup = SSM_KGROUP;

// Optional occupancy hint for the scan kernels (waves per SIMD the register
// allocation must allow); 0 leaves the choice to the compiler.
#ifndef SSM_SCAN_WAVES_PER_EU
#define SSM_SCAN_WAVES_PER_EU 0
#endif
#if SSM_SCAN_WAVES_PER_EU > 0
#define SSM_SCAN_OCCUPANCY __attribute__((amdgpu_waves_per_eu(SSM_SCAN_WAVES_PER_EU)))
#else
#define SSM_SCAN_OCCUPANCY
#endif

struct BlockPos {
  int64_t bi, e, ec, t0, t1, row0;  // row0: element index of (bi, t0, first channel of the block)
  int c;
  int lane_ld;                        // channel offset inside the block used for loads (clamped)
  bool active;
};

// blockIdx.x enumerates (batch, chunk, channel block) with the channel block fastest,
// so consecutive workgroups read neighbouring channels of the same rows.
__device__ __forceinline__ BlockPos block_pos(int n_chunks, int e_blocks, int64_t E, int64_t L, int64_t chunk_len) {
  BlockPos p;
  const int eb = blockIdx.x % e_blocks;
  const int rest = blockIdx.x / e_blocks;
  p.c = rest % n_chunks;
  p.bi = rest / n_chunks;
  p.e = int64_t(eb) * kWave + threadIdx.x;
  p.active = p.e < E;
  p.ec = p.active ? p.e : E - 1;  // inactive lanes read a valid channel and store nothing
  p.lane_ld = int(p.ec - int64_t(eb) * kWave);
  p.t0 = int64_t(p.c) * chunk_len;
  p.t1 = (p.t0 + chunk_len < L) ? p.t0 + chunk_len : L;
  p.row0 = (p.bi * L + p.t0) * E + int64_t(eb) * kWave;
  return p;
}

// ---------------------------------------------------------------------------
// 1. chunk aggregates: state reached from zero over the chunk, and sum of d
// ---------------------------------------------------------------------------
template <typename T, typename R, int NS, bool EXACT, bool SOFTPLUS>
__global__ __launch_bounds__(kWave) SSM_SCAN_OCCUPANCY void scan_chunk_agg_kernel(
    const T* __restrict__ u, const T* __restrict__ delta, const float* __restrict__ A,
    const R* __restrict__ B, const float* __restrict__ bias, float* __restrict__ carry,
    float* __restrict__ chunk_sum, int64_t L, int64_t E, int N, int64_t chunk_len, int n_chunks,
    int agg_chunks, int e_blocks, int rows_odd) {
  // grid covers chunks 0 .. agg_chunks-1 (the last chunk's aggregate is never needed)
  const BlockPos p = block_pos(agg_chunks, e_blocks, E, L, chunk_len);
  float A2[NS];
#pragma unroll
  for (int n = 0; n < NS; n++) A2[n] = (EXACT || n < N) ? A[p.ec * N + n] * kLog2e : 0.f;
  const float bv = bias ? bias[p.ec] : 0.f;
  float h[NS];
#pragma unroll
  for (int n = 0; n < NS; n++) h[n] = 0.f;
  double dsum = 0.0;  // sum of steps, kept in double so long chunks do not drift

  const __amdgpu_buffer_rsrc_t ru = make_rsrc(u + p.row0);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(delta + p.row0);
  const int voff = p.lane_ld * int(sizeof(T));
  const int row_bytes = int(E * int64_t(sizeof(T)));  // the plan keeps chunk_len * row_bytes < 2^31
  const R* brow = B + (p.bi * L + p.t0) * int64_t(N);
  int bodd = int(((p.bi * L + p.t0) * int64_t(N) + rows_odd) & 1);  // the row starts in a word's upper half
  RowBuf<R, NS> bn;
  fetch_row<NS, EXACT>(brow, bodd, N, bn);

  int ks = 0;  // step index inside the chunk
  const int n_steps = int(p.t1 - p.t0);
  auto step = [&](float d, float x) {
    d += bv;
    if (SOFTPLUS) d = softplus(d);
    float bcur[NS];
    unpack_row<NS, EXACT>(bn, N, bcur);
    if (++ks < n_steps) {  // the last step re-reads its own row: never past the end of B
      brow += N;
      bodd ^= N & 1;
    }
    fetch_row<NS, EXACT>(brow, bodd, N, bn);  // next step's row, fetched while this step computes
    const float dx = d * x;
#pragma unroll
    for (int n = 0; n < NS; n++) h[n] = fmaf(exp2_fast(d * A2[n]), h[n], dx * bcur[n]);
    dsum += double(d);
  };
  const int n_groups = n_steps / kGroup;
  float cu[kGroup], cd[kGroup];
  int soff = 0;
  if (n_groups > 0) {
#pragma unroll
    for (int k = 0; k < kGroup; k++) {
      cu[k] = buf_load(ru, voff, k * row_bytes, (T*)nullptr);
      cd[k] = buf_load(rd, voff, k * row_bytes, (T*)nullptr);
    }
  }
  for (int g = 0; g < n_groups; ++g) {
    const int nxt = (g + 1 < n_groups) ? soff + kGroup * row_bytes : soff;  // last group re-reads itself
    float nu[kGroup], nd[kGroup];
#pragma unroll
    for (int k = 0; k < kGroup; k++) {
      nu[k] = buf_load(ru, voff, nxt + k * row_bytes, (T*)nullptr);
      nd[k] = buf_load(rd, voff, nxt + k * row_bytes, (T*)nullptr);
    }
#pragma unroll
    for (int k = 0; k < kGroup; k++) step(cd[k], cu[k]);
#pragma unroll
    for (int k = 0; k < kGroup; k++) { cu[k] = nu[k]; cd[k] = nd[k]; }
    soff += kGroup * row_bytes;
  }
  for (int k = n_groups * kGroup; k < n_steps; ++k) {
    step(buf_load(rd, voff, soff, (T*)nullptr), buf_load(ru, voff, soff, (T*)nullptr));
    soff += row_bytes;
  }
  if (p.active) {
    float* dst = carry + ((p.bi * n_chunks + p.c) * E + p.e) * NS;
#pragma unroll
    for (int n = 0; n < NS; n++) dst[n] = h[n];
    chunk_sum[(p.bi * n_chunks + p.c) * E + p.e] = float(dsum);
  }
}

// ---------------------------------------------------------------------------
// 3. main pass: rescan each chunk from its incoming state, write y
// ---------------------------------------------------------------------------
// FULL: every lane of every block is a real channel (E % 64 == 0), so the
// per-step store needs no exec-mask branch.
template <typename T, typename R, int NS, bool EXACT, bool SOFTPLUS, bool HAS_Z, bool FULL, bool SAVE>
__global__ __launch_bounds__(kWave) SSM_SCAN_OCCUPANCY void scan_main_kernel(
    const T* __restrict__ u, const T* __restrict__ delta, const float* __restrict__ A,
    const R* __restrict__ B, const R* __restrict__ C, const float* __restrict__ D,
    const T* __restrict__ z, const float* __restrict__ bias, T* __restrict__ y,
    float* __restrict__ last_state, const float* __restrict__ carry, const float* __restrict__ h0,
    float* __restrict__ saved, int64_t L, int64_t E, int N, int64_t chunk_len, int n_chunks, int e_blocks,
    int rows_odd) {
  const BlockPos p = block_pos(n_chunks, e_blocks, E, L, chunk_len);
  const int64_t n_saved = (L + kSaveEvery - 1) / kSaveEvery - 1;
  float A2[NS];
#pragma unroll
  for (int n = 0; n < NS; n++) A2[n] = (EXACT || n < N) ? A[p.ec * N + n] * kLog2e : 0.f;
  const float Dv = D ? D[p.ec] : 0.f;
  const float bv = bias ? bias[p.ec] : 0.f;
  float h[NS];
  if (p.c == 0) {  // the incoming state of the sequence: given, or zero
    const float* src = h0 ? h0 + (p.bi * E + p.ec) * N : nullptr;
#pragma unroll
    for (int n = 0; n < NS; n++) h[n] = (src && (EXACT || n < N)) ? src[n] : 0.f;
  } else {
    const float* src = carry + ((p.bi * n_chunks + p.c - 1) * E + p.ec) * NS;
#pragma unroll
    for (int n = 0; n < NS; n++) h[n] = src[n];
  }

  const __amdgpu_buffer_rsrc_t ru = make_rsrc(u + p.row0);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(delta + p.row0);
  const __amdgpu_buffer_rsrc_t rz = make_rsrc((HAS_Z ? z : u) + p.row0);
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(y + p.row0);
  const int voff = p.lane_ld * int(sizeof(T));
  const int row_bytes = int(E * int64_t(sizeof(T)));  // the plan keeps chunk_len * row_bytes < 2^31
  const R* brow = B + (p.bi * L + p.t0) * int64_t(N);
  const R* crow = C + (p.bi * L + p.t0) * int64_t(N);
  const int rodd = int(((p.bi * L + p.t0) * int64_t(N)) & 1);  // rows starting in a word's upper half
  int bodd = rodd ^ (rows_odd & 1), codd = rodd ^ (rows_odd >> 1);
  RowBuf<R, NS> bn, cn;
  fetch_row<NS, EXACT>(brow, bodd, N, bn);
  fetch_row<NS, EXACT>(crow, codd, N, cn);
  int soff = 0;  // byte offset of the current step's row inside the chunk
  int ks = 0;    // step index inside the chunk
  const int n_steps = int(p.t1 - p.t0);

  auto step = [&](float d, float x, float zz) {
    d += bv;
    if (SOFTPLUS) d = softplus(d);
    float bcur[NS], ccur[NS];
    unpack_row<NS, EXACT>(bn, N, bcur);
    unpack_row<NS, EXACT>(cn, N, ccur);
    if (++ks < n_steps) {  // the last step re-reads its own rows: never past the end of B / C
      brow += N;
      crow += N;
      bodd ^= N & 1;
      codd ^= N & 1;
    }
    fetch_row<NS, EXACT>(brow, bodd, N, bn);  // next step's rows are fetched while this step computes
    fetch_row<NS, EXACT>(crow, codd, N, cn);
    const float dx = d * x;
    float acc0 = 0.f, acc1 = 0.f;  // two chains halve the dependent-FMA depth of the readout
#pragma unroll
    for (int n = 0; n < NS; n++) {
      h[n] = fmaf(exp2_fast(d * A2[n]), h[n], dx * bcur[n]);
      if (n % 2 == 0) acc0 = fmaf(ccur[n], h[n], acc0);
      else acc1 = fmaf(ccur[n], h[n], acc1);
    }
    float out = fmaf(Dv, x, acc0 + acc1);
    if (HAS_Z) out *= silu(zz);
    if (FULL || p.active) buf_store(ry, voff, soff, out, (T*)nullptr);
    soff += row_bytes;
    // the state after every kSaveEvery-th step of the sequence, for the backward (a uniform
    // test; a variant of its own, so that the kernel without it compiles as before)
    if (SAVE && (p.t0 + ks) % kSaveEvery == 0 && (p.t0 + ks) < L && p.active) {
      float* dst = saved + ((p.bi * n_saved + (p.t0 + ks) / kSaveEvery - 1) * E + p.e) * N;
#pragma unroll
      for (int n = 0; n < NS; n++)
        if (EXACT || n < N) dst[n] = h[n];
    }
  };
  const int n_groups = n_steps / kGroup;
  float cu[kGroup], cd[kGroup], cz[kGroup];
  if (n_groups > 0) {
#pragma unroll
    for (int k = 0; k < kGroup; k++) {
      cu[k] = buf_load(ru, voff, k * row_bytes, (T*)nullptr);
      cd[k] = buf_load(rd, voff, k * row_bytes, (T*)nullptr);
      cz[k] = HAS_Z ? buf_load(rz, voff, k * row_bytes, (T*)nullptr) : 0.f;
    }
  }
  for (int g = 0; g < n_groups; ++g) {
    const int nxt = (g + 1 < n_groups) ? soff + kGroup * row_bytes : soff;  // last group re-reads itself
    float nu[kGroup], nd[kGroup], nz[kGroup];
#pragma unroll
    for (int k = 0; k < kGroup; k++) {
      nu[k] = buf_load(ru, voff, nxt + k * row_bytes, (T*)nullptr);
      nd[k] = buf_load(rd, voff, nxt + k * row_bytes, (T*)nullptr);
      nz[k] = HAS_Z ? buf_load(rz, voff, nxt + k * row_bytes, (T*)nullptr) : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kGroup; k++) step(cd[k], cu[k], cz[k]);
#pragma unroll
    for (int k = 0; k < kGroup; k++) { cu[k] = nu[k]; cd[k] = nd[k]; cz[k] = nz[k]; }
  }
  for (int k = n_groups * kGroup; k < n_steps; ++k) {
    const float x = buf_load(ru, voff, soff, (T*)nullptr);
    const float d = buf_load(rd, voff, soff, (T*)nullptr);
    const float zz = HAS_Z ? buf_load(rz, voff, soff, (T*)nullptr) : 0.f;
    step(d, x, zz);
  }
  if (last_state && p.c == n_chunks - 1 && p.active) {
    float* dst = last_state + (p.bi * E + p.e) * N;
#pragma unroll
    for (int n = 0; n < NS; n++)
      if (EXACT || n < N) dst[n] = h[n];
  }
}

// last_state of an empty sequence: a copy of the incoming state, or zeros
__global__ __launch_bounds__(256) void fill_state_kernel(float* __restrict__ p, const float* __restrict__ src,
                                                         int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = src ? src[i] : 0.f;
}

// ---------------------------------------------------------------------------
// single-token state update ([AB] row 6, the SSM half of `step`)
// ---------------------------------------------------------------------------
// LPC = NS / 4 lanes share one channel, each holding 4 consecutive states, so
// a wave reads and writes the fp32 state as one contiguous 1 KiB block per
// instruction.  Workgroups are laid out per group of kRows batch rows
// (row_blocks of them per group), so the rows are per-workgroup scalars and
// the lane's channel is plain 32-bit arithmetic.  The partial readouts of the LPC lanes are summed
// with DPP quad permutes (no LDS traffic).

#ifndef SSM_UPDATE_ROWS
#define SSM_UPDATE_ROWS 4
#endif
// Each thread updates the same 4 states of one channel in kRows consecutive
// batch rows: the channel's A slice and bias / D are loaded once and reused,
// and all rows' state loads are issued before any arithmetic.  When four
// lanes share a channel (N of 9 to 16) and there are four rows, lane q also
// works out row q's step and gate: the quad shares step and step * x through
// DPP broadcasts, and lane q writes row q's output, so the softplus and silu
// are not repeated in every lane.  STAGE (that layout, E a multiple of 64,
// 16-byte aligned rows): the workgroup's 64 channels x 4 rows of x, step and
// z come in through LDS as 16-byte pieces and y goes out the same way,
// instead of 2- or 4-byte accesses per lane; with VEC the 4 rows of B and C
// come in the same way (the decode workload: 37.4 -> 32.7 us per call with
// events around each call).
constexpr int kRows = SSM_UPDATE_ROWS;

template <typename T, int NS, bool VEC, bool SOFTPLUS, bool HAS_Z, bool STAGE>
__global__ __launch_bounds__(256) void state_update_kernel(
    float* __restrict__ state, const T* __restrict__ x, const T* __restrict__ delta,
    const float* __restrict__ A, const T* __restrict__ B, const T* __restrict__ C,
    const float* __restrict__ D, const T* __restrict__ z, const float* __restrict__ bias,
    T* __restrict__ y, int b, int E, int N, int row_blocks) {
  constexpr int LPC = NS / 4;
  constexpr bool SHARED = LPC == 4 && kRows == 4;  // lane q owns row q's per-channel scalars
  static_assert(!STAGE || SHARED, "staging goes with the shared-scalar layout (64 channels per workgroup)");
  constexpr int kEpp = 16 / int(sizeof(T));  // elements per 16-byte piece
  constexpr int kPieces = 64 / kEpp;         // pieces per 64-channel row
  __shared__ __attribute__((aligned(16))) T xs[3][4][64];  // x, step, z of the workgroup (STAGE)
  __shared__ __attribute__((aligned(16))) T ys[4][64];     // y of the workgroup (STAGE)
  __shared__ __attribute__((aligned(16))) T bcs[2][4][NS];  // B and C rows of the 4 batch rows (STAGE and VEC)
  const int rb = blockIdx.x / row_blocks;  // group of kRows batch rows: uniform per workgroup
  const int r = (blockIdx.x - rb * row_blocks) * 256 + threadIdx.x;
  const int e_raw = r / LPC;
  const int q = r % LPC;
  const bool active = e_raw < E;
  const int e = active ? e_raw : E - 1;
  const int n0 = 4 * q;

  float a[4];
  if constexpr (VEC) {
    const float4 av = *reinterpret_cast<const float4*>(A + int64_t(e) * NS + n0);
    a[0] = av.x; a[1] = av.y; a[2] = av.z; a[3] = av.w;
  } else {
#pragma unroll
    for (int k = 0; k < 4; k++) a[k] = (n0 + k < N) ? A[int64_t(e) * N + n0 + k] : 0.f;
  }
#pragma unroll
  for (int k = 0; k < 4; k++) a[k] *= kLog2e;
  const float bv = bias ? bias[e] : 0.f;
  const float Dv = D ? D[e] : 0.f;
  const int e0 = (blockIdx.x - rb * row_blocks) * 64;  // the workgroup's first channel (STAGE)
  if constexpr (STAGE) {
    constexpr int kArr = HAS_Z ? 3 : 2;
    if (threadIdx.x < kArr * 4 * kPieces) {
      const int arr = threadIdx.x / (4 * kPieces), row = (threadIdx.x / kPieces) % 4, piece = threadIdx.x % kPieces;
      const T* src = arr == 0 ? x : arr == 1 ? delta : z;
      const int bi_raw = rb * kRows + row;
      const int bi = bi_raw < b ? bi_raw : b - 1;
      *reinterpret_cast<uint4*>(&xs[arr][row][piece * kEpp]) =
          *reinterpret_cast<const uint4*>(src + int64_t(bi) * E + e0 + piece * kEpp);
    }
    if constexpr (VEC) {  // B and C rows (NS elements each) by the threads of the workgroup's last two waves
      constexpr int kBcPieces = NS / kEpp;
      const int t = int(threadIdx.x) - 128;
      if (t >= 0 && t < 2 * 4 * kBcPieces) {
        const int arr = t / (4 * kBcPieces), row = (t / kBcPieces) % 4, piece = t % kBcPieces;
        const int bi_raw = rb * kRows + row;
        const int bi = bi_raw < b ? bi_raw : b - 1;
        *reinterpret_cast<uint4*>(&bcs[arr][row][piece * kEpp]) =
            *reinterpret_cast<const uint4*>((arr ? C : B) + int64_t(bi) * NS + piece * kEpp);
      }
    }
    __syncthreads();
  }

  float s[kRows][4], bn[kRows][4], cn[kRows][4];
  float xv[kRows], dr[kRows], zz[kRows];
  int64_t cc[kRows];
  bool row_ok[kRows];
#pragma unroll
  for (int j = 0; j < kRows; j++) {
    const int bi_raw = rb * kRows + j;
    row_ok[j] = bi_raw < b;
    const int bi = row_ok[j] ? bi_raw : b - 1;
    cc[j] = int64_t(bi) * E + e;
    if constexpr (VEC) {  // N == NS, state / B / C rows aligned for vector access
      const float4 sv = *reinterpret_cast<const float4*>(state + cc[j] * NS + n0);
      s[j][0] = sv.x; s[j][1] = sv.y; s[j][2] = sv.z; s[j][3] = sv.w;
      if constexpr (STAGE) {
#pragma unroll
        for (int kk = 0; kk < 4; kk++) {
          bn[j][kk] = load_elem(&bcs[0][j][n0 + kk]);
          cn[j][kk] = load_elem(&bcs[1][j][n0 + kk]);
        }
      } else if constexpr (std::is_same<T, float>::value) {
        const float4 b4 = *reinterpret_cast<const float4*>(B + int64_t(bi) * NS + n0);
        const float4 c4 = *reinterpret_cast<const float4*>(C + int64_t(bi) * NS + n0);
        bn[j][0] = b4.x; bn[j][1] = b4.y; bn[j][2] = b4.z; bn[j][3] = b4.w;
        cn[j][0] = c4.x; cn[j][1] = c4.y; cn[j][2] = c4.z; cn[j][3] = c4.w;
      } else {
        const uint2 b2 = *reinterpret_cast<const uint2*>(B + int64_t(bi) * NS + n0);
        const uint2 c2 = *reinterpret_cast<const uint2*>(C + int64_t(bi) * NS + n0);
        bn[j][0] = __uint_as_float(b2.x << 16); bn[j][1] = __uint_as_float(b2.x & 0xffff0000u);
        bn[j][2] = __uint_as_float(b2.y << 16); bn[j][3] = __uint_as_float(b2.y & 0xffff0000u);
        cn[j][0] = __uint_as_float(c2.x << 16); cn[j][1] = __uint_as_float(c2.x & 0xffff0000u);
        cn[j][2] = __uint_as_float(c2.y << 16); cn[j][3] = __uint_as_float(c2.y & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const int n = n0 + k;
        const bool in = n < N;
        s[j][k] = in ? state[cc[j] * N + n] : 0.f;
        bn[j][k] = in ? load_elem(B + int64_t(bi) * N + n) : 0.f;
        cn[j][k] = in ? load_elem(C + int64_t(bi) * N + n) : 0.f;
      }
    }
    if constexpr (!SHARED) {
      xv[j] = load_elem(x + cc[j]);
      dr[j] = load_elem(delta + cc[j]);
      zz[j] = HAS_Z ? load_elem(z + cc[j]) : 0.f;
    }
  }
  // this lane's own row (SHARED): row q of the group
  const int bo_raw = rb * kRows + q;
  const bool own_ok = bo_raw < b;
  const int64_t co = int64_t(own_ok ? bo_raw : b - 1) * E + e;
  float xo = 0.f, d_own = 0.f, dx_own = 0.f, zo = 0.f, acc_own = 0.f;
  if constexpr (SHARED) {
    float raw;
    if constexpr (STAGE) {
      const int chl = threadIdx.x / 4;  // the lane's channel inside the workgroup
      xo = load_elem(&xs[0][q][chl]);
      raw = load_elem(&xs[1][q][chl]) + bv;
      zo = HAS_Z ? load_elem(&xs[2][q][chl]) : 0.f;
    } else {
      xo = load_elem(x + co);
      raw = load_elem(delta + co) + bv;
      zo = HAS_Z ? load_elem(z + co) : 0.f;
    }
    d_own = SOFTPLUS ? softplus(raw) : raw;
    dx_own = d_own * xo;
  }
#pragma unroll
  for (int j = 0; j < kRows; j++) {
    float d, dx;
    if constexpr (SHARED) {
      d = quad_bcast(d_own, j);
      dx = quad_bcast(dx_own, j);
    } else {
      d = dr[j] + bv;
      if (SOFTPLUS) d = softplus(d);
      dx = d * xv[j];
    }
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < 4; k++) {
      s[j][k] = fmaf(exp2_fast(d * a[k]), s[j][k], dx * bn[j][k]);
      acc = fmaf(cn[j][k], s[j][k], acc);
    }
    if constexpr (LPC >= 2) acc += quad_xor1(acc);
    if constexpr (LPC >= 4) acc += quad_xor2(acc);
    if constexpr (SHARED) acc_own = (q == j) ? acc : acc_own;
    if (active && row_ok[j]) {
      if constexpr (VEC) {
        *reinterpret_cast<float4*>(state + cc[j] * NS + n0) = make_float4(s[j][0], s[j][1], s[j][2], s[j][3]);
      } else {
#pragma unroll
        for (int k = 0; k < 4; k++)
          if (n0 + k < N) state[cc[j] * N + n0 + k] = s[j][k];
      }
      if (!SHARED && q == 0) {
        float out = fmaf(Dv, xv[j], acc);
        if (HAS_Z) out *= silu(zz[j]);
        store_elem(y + cc[j], out);
      }
    }
  }
  // every lane of the quad holds the same sums: lane q produces row q's output
  if constexpr (STAGE) {
    float out = fmaf(Dv, xo, acc_own);
    if (HAS_Z) out *= silu(zo);
    store_elem(&ys[q][threadIdx.x / 4], out);
    __syncthreads();
    if (threadIdx.x < 4 * kPieces) {
      const int row = threadIdx.x / kPieces, piece = threadIdx.x % kPieces;
      if (rb * kRows + row < b)
        *reinterpret_cast<uint4*>(y + int64_t(rb * kRows + row) * E + e0 + piece * kEpp) =
            *reinterpret_cast<const uint4*>(&ys[row][piece * kEpp]);
    }
  } else if (SHARED && active && own_ok) {
    float out = fmaf(Dv, xo, acc_own);
    if (HAS_Z) out *= silu(zo);
    store_elem(y + co, out);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// 1 when a bf16 tensor starts 2 bytes into a 32-bit word.
int bf16_rows_odd(const void* p) { return int((reinterpret_cast<uintptr_t>(p) >> 1) & 1); }

// Rows of B and C as the kernels read them (the caller's arrays, or float
// copies of bf16 ones) and the per-chunk workspace of a cut scan.
struct ScanBufs {
  const void* B;
  const void* C;
  int rows_odd;  // bf16 rows: bit 0 / bit 1 set when B / C starts 2 bytes into a 32-bit word
  float* carry;  // [b][n_chunks][E][NS] chunk aggregates, then incoming states
  float* csum;   // [b][n_chunks][E] sum of steps per chunk
};

// Chunk aggregates, then the carry chain: afterwards carry slot c holds the
// state at the end of chunk c (the incoming state of chunk c + 1).
template <typename T, typename R, int NS, bool EXACT, bool SOFTPLUS>
hipError_t run_carries(const ScanArgs& a, const ScanPlan& pl, const ScanBufs& w) {
  if (pl.n_chunks <= 1) return hipSuccess;
  const int N = int(a.N);
  const int agg = pl.n_chunks - 1;
  hipError_t err = launch_kind(kKindAgg, scan_chunk_agg_kernel<T, R, NS, EXACT, SOFTPLUS>, a.b * agg * pl.e_blocks,
                               kWave, a.stream, static_cast<const T*>(a.u), static_cast<const T*>(a.delta), a.A,
                               static_cast<const R*>(w.B), a.bias, w.carry, w.csum, a.L, a.E, N, pl.chunk_len,
                               pl.n_chunks, agg, pl.e_blocks, w.rows_odd & 1);
  if (err != hipSuccess) return err;
  // the state at the end of chunk c (forward, inclusive), from the incoming state of the sequence
  const ChainArgs c{w.carry, w.csum, a.A, a.h0, nullptr, a.b, a.E, NS, N, pl.n_chunks, pl.n_chunks - 1};
  return launch_chain<false, false, false>(kKindCarry, c, a.stream);
}

template <typename T, typename R, int NS, bool EXACT, bool SOFTPLUS, bool HAS_Z, bool FULL>
hipError_t run_scan(const ScanArgs& a, const ScanPlan& pl, const ScanBufs& w) {
  const T* u = static_cast<const T*>(a.u);
  const T* dl = static_cast<const T*>(a.delta);
  const T* z = static_cast<const T*>(a.z);
  const R* B = static_cast<const R*>(w.B);
  const R* C = static_cast<const R*>(w.C);
  T* y = static_cast<T*>(a.y);
  const int N = int(a.N);
  hipError_t err = run_carries<T, R, NS, EXACT, SOFTPLUS>(a, pl, w);
  if (err != hipSuccess) return err;
  const int64_t blocks = a.b * pl.n_chunks * pl.e_blocks;
  if (a.saved)  // the saving variant exists for the general channel count only
    return launch_kind(kKindMain, scan_main_kernel<T, R, NS, EXACT, SOFTPLUS, HAS_Z, false, true>, blocks, kWave, a.stream,
                       u, dl, a.A, B, C, a.D, z, a.bias, y, a.last_state, (const float*)w.carry, a.h0, a.saved, a.L,
                       a.E, N, pl.chunk_len, pl.n_chunks, pl.e_blocks, w.rows_odd);
  return launch_kind(kKindMain, scan_main_kernel<T, R, NS, EXACT, SOFTPLUS, HAS_Z, FULL, false>, blocks, kWave, a.stream,
                     u, dl, a.A, B, C, a.D, z, a.bias, y, a.last_state, (const float*)w.carry, a.h0,
                     (float*)nullptr, a.L, a.E, N, pl.chunk_len, pl.n_chunks, pl.e_blocks, w.rows_odd);
}

template <typename T, typename R, int NS, bool EXACT, bool FULL>
hipError_t scan_flags(const ScanArgs& a, const ScanPlan& pl, const ScanBufs& w) {
  const bool z = a.z != nullptr;
  if (a.softplus) {
    return z ? run_scan<T, R, NS, EXACT, true, true, FULL>(a, pl, w)
             : run_scan<T, R, NS, EXACT, true, false, FULL>(a, pl, w);
  }
  return z ? run_scan<T, R, NS, EXACT, false, true, FULL>(a, pl, w)
           : run_scan<T, R, NS, EXACT, false, false, FULL>(a, pl, w);
}

template <typename T, typename R, int NS, bool EXACT>
hipError_t scan_full(const ScanArgs& a, const ScanPlan& pl, const ScanBufs& w) {
  return (a.E % kWave == 0) ? scan_flags<T, R, NS, EXACT, true>(a, pl, w) : scan_flags<T, R, NS, EXACT, false>(a, pl, w);
}

// state slots per channel in the workspace: N for the exact-size kernels, 16 for the padded one
int scan_states(int64_t N) { return (N == 4 || N == 8 || N == 16) ? int(N) : 16; }

template <typename T, typename R>
hipError_t scan_typed(const ScanArgs& a, const ScanPlan& pl, const ScanBufs& w) {
  if (a.N == 16) return scan_full<T, R, 16, true>(a, pl, w);
  if (a.N == 8) return scan_full<T, R, 8, true>(a, pl, w);
  if (a.N == 4) return scan_full<T, R, 4, true>(a, pl, w);
  return scan_full<T, R, 16, false>(a, pl, w);
}

template <typename T, int NS, bool VEC, bool STAGE>
hipError_t update_launch(const UpdateArgs& a) {
  const T* x = static_cast<const T*>(a.x);
  const T* dl = static_cast<const T*>(a.delta);
  const T* B = static_cast<const T*>(a.B);
  const T* C = static_cast<const T*>(a.C);
  const T* z = static_cast<const T*>(a.z);
  T* y = static_cast<T*>(a.y);
  const int row_blocks = int((a.E * (NS / 4) + 255) / 256);
  const int64_t blocks = (a.b + kRows - 1) / kRows * row_blocks;
  const int N = int(a.N), E = int(a.E);
#define SSM_UPDATE_LAUNCH(SP, HZ)                                                                                      \
  return launch_kind(kKindUpdate, state_update_kernel<T, NS, VEC, SP, HZ, STAGE>, blocks, 256, a.stream, a.state, x, \
                     dl, a.A, B, C, a.D, z, a.bias, y, int(a.b), E, N, row_blocks)
  if (a.softplus) {
    if (z) { SSM_UPDATE_LAUNCH(true, true); }
    SSM_UPDATE_LAUNCH(true, false);
  }
  if (z) { SSM_UPDATE_LAUNCH(false, true); }
  SSM_UPDATE_LAUNCH(false, false);
#undef SSM_UPDATE_LAUNCH
}

template <typename T, int NS, bool VEC>
hipError_t update_flags(const UpdateArgs& a) {
  if constexpr (NS == 16 && kRows == 4) {
    // x, step, z and y move through LDS in 16-byte pieces: whole 64-channel blocks, aligned rows
    auto al16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
    if (a.E % 64 == 0 && al16(a.x) && al16(a.delta) && al16(a.y) && (!a.z || al16(a.z)) &&
        (!VEC || (al16(a.B) && al16(a.C))))
      return update_launch<T, NS, VEC, true>(a);
  }
  return update_launch<T, NS, VEC, false>(a);
}

template <typename T>
hipError_t update_typed(const UpdateArgs& a) {
  const size_t row_align = std::is_same<T, float>::value ? 16 : 8;
  const bool vec = (a.N == 4 || a.N == 8 || a.N == 16) && reinterpret_cast<uintptr_t>(a.state) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(a.A) % 16 == 0 && reinterpret_cast<uintptr_t>(a.B) % row_align == 0 &&
                   reinterpret_cast<uintptr_t>(a.C) % row_align == 0;
  if (vec) {
    if (a.N == 16) return update_flags<T, 16, true>(a);
    if (a.N == 8) return update_flags<T, 8, true>(a);
    return update_flags<T, 4, true>(a);
  }
  if (a.N <= 4) return update_flags<T, 4, false>(a);
  if (a.N <= 8) return update_flags<T, 8, false>(a);
  return update_flags<T, 16, false>(a);
}

}  // namespace

ScanPlan plan_scan(int64_t b, int64_t L, int64_t E, int elem_bytes, const ScanTuning& tune) {
  ScanPlan pl;
  pl.e_blocks = int((E + kWave - 1) / kWave);
  // Enough waves that every SIMD of the 256 CUs sees several rounds of them
  // (the two passes hold 6 and 7 waves per SIMD).  20480 measured best on the
  // long sequence among targets of 12288 to 30720: 256 chunks of 256 steps,
  // 1.871 ms against 1.896 for 16384 and 1.93 for 22528 (means of repeated
  // runs).  The sequence is cut only when batch x channel blocks alone cannot
  // provide them.
  const int64_t target = tune.target_waves > 0 ? tune.target_waves : 20480;
  const int64_t base = b * pl.e_blocks;
  // Chunks of at least 64 steps, or of 32 when 64-step chunks give fewer than
  // 4096 waves (4 per SIMD) and the sequence has 256 steps or more (shorter
  // ones are launch-bound): b32 L512 E512 takes 96 us in 16 chunks of 32 steps
  // against 114 us in 8 of 64.
  int64_t min_chunk = (L >= 256 && base * ((L + 63) / 64) < 4096) ? 32 : 64;
  if (tune.min_chunk > 0) min_chunk = tune.min_chunk;
  pl.chunk_len = std::max<int64_t>(L, 1);
  pl.n_chunks = 1;
  if (base > 0 && base * 2 < target && L > min_chunk) {
    const int64_t want = (target + base - 1) / base;
    int64_t len = std::max<int64_t>(min_chunk, (L + want - 1) / want);
    len = (len + 7) / 8 * 8;
    pl.chunk_len = len;
  }
  // a chunk's rows are addressed with 32-bit buffer offsets: keep them below 2^31
  const int64_t row_bytes = std::max<int64_t>(E, 1) * elem_bytes;
  const int64_t max_len = (int64_t(0x7fffffff) - kWave * elem_bytes) / row_bytes;
  if (max_len >= 1 && pl.chunk_len > max_len) pl.chunk_len = max_len;
  if (max_len < 1) pl.chunk_len = 0;  // rejected by the caller
  pl.n_chunks = pl.chunk_len > 0 ? int((std::max<int64_t>(L, 1) + pl.chunk_len - 1) / pl.chunk_len) : 0;
  return pl;
}

// Workspace of a cut scan, in floats: [chunk aggregates | chunk step sums | float
// rows of B | of C].  A cut bf16 scan reads float copies of its B / C rows: the
// rows are taken once per step by every wave of a chunk, and unpacking bf16 on
// the scalar ALU made the long b1 L65536 E5120 scan 4-8% slower.  One chunk
// reads the bf16 rows directly and takes no workspace.
struct WsLayout {
  size_t carry, csum, rows, total;  // offsets and size in floats
};
WsLayout ws_layout(const ScanArgs& a, const ScanPlan& pl) {
  WsLayout l{0, 0, 0, 0};
  if (pl.n_chunks <= 1) return l;
  const size_t slots = size_t(a.b) * size_t(pl.n_chunks) * size_t(a.E);
  l.csum = slots * size_t(scan_states(a.N));
  l.rows = l.csum + slots;
  const size_t n_rows = a.dtype == 0 ? 0 : size_t(a.b) * size_t(a.L) * size_t(a.N);
  l.total = l.rows + 2 * n_rows;
  return l;
}

size_t chunked_workspace_bytes(const ScanArgs& a, const ScanPlan& pl) { return ws_layout(a, pl).total * sizeof(float); }

int choose_path(const ScanArgs& a, const ScanPlan& pl, int n_cu, FusedPlan* fp) {
  if (a.tune.path == kPathChunked) return kPathChunked;
  if (a.tune.path == kPathSinglePass) return plan_fused(a, n_cu, kFusedMaxChunks, fp) ? kPathSinglePass : -1;
  // by default the single pass runs where the sequence has to be cut and its
  // chain of chunk maps per block stays short
  if (pl.n_chunks > 1 && plan_fused(a, n_cu, kFusedChainMax, fp)) return kPathSinglePass;
  return kPathChunked;
}

hipError_t device_cu_count(int* n_cu) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  return err;
}

hipError_t launch_scan(const ScanArgs& a, void* workspace, size_t workspace_bytes) {
  if (a.b == 0 || a.E == 0) return hipSuccess;
  if (a.L == 0) {  // no step: the last state is the incoming one
    if (!a.last_state) return hipSuccess;
    const int64_t n = a.b * a.E * a.N;
    return launch_kind(kKindFill, fill_state_kernel, (n + 255) / 256, 256, a.stream, a.last_state, a.h0, n);
  }
  const ScanPlan pl = plan_scan(a.b, a.L, a.E, a.dtype == 0 ? 4 : 2, a.tune);
  int n_cu = 0;
  hipError_t err = device_cu_count(&n_cu);
  if (err != hipSuccess) return err;
  FusedPlan fp;
  const int path = choose_path(a, pl, n_cu, &fp);
  if (path < 0) return hipErrorInvalidConfiguration;  // the caller checked this before
  if (path == kPathSinglePass) return launch_fused(a, fp);
  // workspace, taken from the caller or from the stream's pool
  const WsLayout lay = ws_layout(a, pl);
  const size_t need = lay.total * sizeof(float);
  void* ws = nullptr;
  bool own = false;
  if (need > 0) {
    if (workspace) {
      if (workspace_bytes < need) return hipErrorInvalidValue;
      ws = workspace;
    } else {
      err = hipMallocAsync(&ws, need, a.stream);
      if (err != hipSuccess) return err;
      own = true;
    }
  }
  float* const f = static_cast<float*>(ws);
  ScanBufs w;
  w.carry = need ? f + lay.carry : nullptr;
  w.csum = need ? f + lay.csum : nullptr;
  w.B = a.B;
  w.C = a.C;
  w.rows_odd = 0;
  if (a.dtype == 0) {
    err = scan_typed<float, float>(a, pl, w);
  } else if (need) {  // cut: float copies of the rows
    const size_t n_rows = size_t(a.b) * size_t(a.L) * size_t(a.N);
    float* const Bf = f + lay.rows;
    float* const Cf = Bf + n_rows;
    err = launch_kind(kKindWiden, widen_rows_kernel, int64_t((n_rows + 255) / 256), 256, a.stream,
                      static_cast<const bf16_bits*>(a.B), static_cast<const bf16_bits*>(a.C), Bf, Cf,
                      int64_t(n_rows));
    w.B = Bf;
    w.C = Cf;
    if (err == hipSuccess) err = scan_typed<bf16_bits, float>(a, pl, w);
  } else {
    w.rows_odd = bf16_rows_odd(a.B) | (bf16_rows_odd(a.C) << 1);
    err = scan_typed<bf16_bits, bf16_bits>(a, pl, w);
  }
  if (own) {
    hipError_t ferr = hipFreeAsync(ws, a.stream);
    if (err == hipSuccess) err = ferr;
  }
  return err;
}

int chunk_state_slots(int64_t N) { return scan_states(N); }

hipError_t launch_state_update(const UpdateArgs& a) {
  if (a.b == 0 || a.E == 0) return hipSuccess;
  return a.dtype == 0 ? update_typed<float>(a) : update_typed<bf16_bits>(a);
}

}  // namespace ssm
