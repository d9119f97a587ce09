// ssm_bwd.hip -- backward of the selective scan: the gradient of a scalar loss
// with respect to u, delta, A, B, C, D, z, the step bias and the initial state,
// given dloss/dy and (optionally) dloss/dlast_state.  States are recomputed,
// never stored for the whole sequence (pages: "Mamba: Linear-Time Sequence
// Modeling with Selective State Spaces", nadeemcite summary, "Core Idea": the
// backward pass recomputes the states; abhik.ai page, "Compose the updates
// instead of waiting for every state": the affine composition that lets the
// sequence be cut into chunks, used here in both time directions).
//
// Per chain, with G_t = dloss/dh_t and X the gradient arriving from later steps:
//   dq_t = dy_t * silu(z_t);  G_t = X + dq_t * C_t;  X <- a_t * G_t  (dloss/dh_{t-1})
//   dB_t += G_t * d_t * u_t;  dC_t += dq_t * h_t;  dA += G_t * a_t * h_{t-1} * d_t
//   du_t = dq_t * D + d_t * sum_n G_t B_t;  dd_t = u_t * sum_n G_t B_t + sum_n G_t a_t h_{t-1} A
//   ddelta_t = dd_t * sigmoid(delta_t + bias) (softplus) ;  dz_t = dy_t * q_t * silu'(z_t)
//
// Passes (one call):
//   1. forward chunk states: per chunk of kBwdChunk steps the state reached
//      from zero, then the forward chain of those maps gives the state entering
//      every chunk (with saved states these are the saved states instead);
//   2. per chunk, the state gradient its own steps send to its first step (the
//      reverse-time aggregate).  Without saved states 1 and 2 come from one walk
//      over each chunk (bwd_chunk_maps_kernel); with them, 2 alone
//      (bwd_chunk_agg_kernel, walking the chunk backwards);
//   3. chain_kernel (ssm_chain.h), in reverse: the chain of those aggregates
//      from the last chunk to the first, started from dlast: the gradient
//      entering every chunk from its end (the decay of a chunk is
//      exp(A * sum of its steps), as forward);
//   4. bwd_main_kernel: per chunk, states recomputed from the chunk's incoming
//      state (checkpoints every kSub steps, then each sub-block's states in
//      registers), the reverse walk, every gradient;
//   5. bwd_reduce_*: sums of the partial gradients over channel blocks (dB, dC)
//      and over batch rows and chunks (dA, dD, dbias), in a fixed order.
//
// Layout of the main kernel: a quad of lanes per channel, 4 state coordinates
// per lane (N padded to 16), 16 channels per wave, 4 waves per workgroup.  The
// sums over channels for dB and dC go through lane swaps and DPP inside the
// wave, then through LDS across the workgroup's 4 waves.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "ssm_chain.h"
#include "ssm_device.h"
#include "ssm_internal.h"
#include "ssm_profile.h"

namespace ssm {
namespace {

constexpr int kBwdChunk = 64;                          // steps per chunk
constexpr int kSub = 8;                                // steps whose states a sub-block keeps in registers
constexpr int kNSub = kBwdChunk / kSub;                // checkpoints per chunk
constexpr int kBwdWaves = 4;                           // waves per workgroup of the main kernel
constexpr int kChPerWave = kWave / 4;                  // a quad of lanes per channel
constexpr int kChPerBlock = kBwdWaves * kChPerWave;    // 64 channels per workgroup
constexpr int kS = 16;                                 // state slots per channel (N padded)
constexpr int kRed = 2 * kS;                           // dB and dC values per (step, channel block)

// B and C rows as float, padded with zeros to 16 states: [b, L, 16].
template <typename T>
__global__ __launch_bounds__(256) void bwd_rows_kernel(const T* __restrict__ B, const T* __restrict__ C,
                                                       float* __restrict__ B16, float* __restrict__ C16, int64_t rows,
                                                       int N) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows * kS) return;
  const int64_t r = i / kS;
  const int n = int(i % kS);
  B16[i] = n < N ? load_elem(B + r * N + n) : 0.f;
  C16[i] = n < N ? load_elem(C + r * N + n) : 0.f;
}

// ---------------------------------------------------------------------------
// 2. reverse-time chunk aggregate: walking chunk c (c >= 1) from its last step
//    to its first with X = 0 at the end, X <- a_t * (X + dq_t * C_t); also the
//    chunk's sum of steps.  One lane per channel, 16 states in registers.
// ---------------------------------------------------------------------------
template <typename T, bool SOFTPLUS, bool HAS_Z>
__global__ __launch_bounds__(kWave) void bwd_chunk_agg_kernel(
    const T* __restrict__ delta, const T* __restrict__ dy, const T* __restrict__ z, const float* __restrict__ A,
    const float* __restrict__ C16, const float* __restrict__ bias, float* __restrict__ xagg,
    float* __restrict__ xsum, int64_t L, int64_t E, int N, int n_chunks, int e_blocks) {
  const int eb = blockIdx.x % e_blocks;
  const int rest = blockIdx.x / e_blocks;
  const int c = 1 + rest % (n_chunks - 1);
  const int64_t bi = rest / (n_chunks - 1);
  const int64_t e = int64_t(eb) * kWave + threadIdx.x;
  const bool active = e < E;
  const int64_t ec = active ? e : E - 1;
  const int64_t t0 = int64_t(c) * kBwdChunk;
  const int n_steps = int(std::min<int64_t>(L - t0, kBwdChunk));

  float A2[kS];
#pragma unroll
  for (int n = 0; n < kS; n++) A2[n] = n < N ? A[ec * N + n] * kLog2e : 0.f;
  const float bv = bias ? bias[ec] : 0.f;
  float X[kS];
#pragma unroll
  for (int n = 0; n < kS; n++) X[n] = 0.f;
  double dsum = 0.0;

  const int64_t row0 = (bi * L + t0) * E + int64_t(eb) * kWave;
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(delta + row0);
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(dy + row0);
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(HAS_Z ? z + row0 : delta + row0);
  const int voff = int(ec - int64_t(eb) * kWave) * int(sizeof(T));
  const int row_bytes = int(E * int64_t(sizeof(T)));  // kBwdChunk * row_bytes < 2^31 is checked by the caller
  const float* crow0 = C16 + (bi * L + t0) * kS;

  for (int k = n_steps - 1; k >= 0; --k) {
    const int so = k * row_bytes;
    float d = buf_load(rd, voff, so, (T*)nullptr) + bv;
    float dq = buf_load(ry, voff, so, (T*)nullptr);
    if (HAS_Z) dq *= silu(buf_load(rz, voff, so, (T*)nullptr));
    if (SOFTPLUS) d = softplus(d);
    const float* crow = crow0 + k * kS;  // wave-uniform: scalar loads
#pragma unroll
    for (int n = 0; n < kS; n++) X[n] = exp2_fast(d * A2[n]) * fmaf(dq, crow[n], X[n]);
    dsum += double(d);
  }
  if (active) {
    float* dst = xagg + ((bi * n_chunks + c) * E + e) * kS;
#pragma unroll
    for (int n = 0; n < kS; n++) dst[n] = X[n];
    xsum[(bi * n_chunks + c) * E + e] = float(dsum);
  }
}

// ---------------------------------------------------------------------------
// 1 and 2 in one walk (no saved states): chunk c walked once, first step to
// last, gives both of its maps and its sum of steps, which both chains use:
//   forward  h <- a_t * h + d_t * u_t * B_t from zero: the state leaving the
//            chunk when it is entered with zero (written for c < n_chunks - 1);
//   reverse  X = sum_t (a_t0 * .. * a_t) * dq_t * C_t: the state gradient that
//            the chunk's own steps send to its first step, the same sum as the
//            backward walk X <- a_t * (X + dq_t * C_t) above, with the running
//            product of the retentions in place of the walk's order (written
//            for c >= 1).
// Each retention exp2(d * A * log2 e) is evaluated once for both maps and u,
// delta, dy, z are read once.  One lane per channel, 16 states in registers;
// the float B and C rows are wave-uniform (scalar loads).
// ---------------------------------------------------------------------------
template <typename T, bool SOFTPLUS, bool HAS_Z>
__global__ __launch_bounds__(kWave) void bwd_chunk_maps_kernel(
    const T* __restrict__ u, const T* __restrict__ delta, const T* __restrict__ dy, const T* __restrict__ z,
    const float* __restrict__ A, const float* __restrict__ B16, const float* __restrict__ C16,
    const float* __restrict__ bias, float* __restrict__ fagg, int fslots, float* __restrict__ xagg,
    float* __restrict__ sums, int64_t L, int64_t E, int N, int n_chunks, int e_blocks) {
  constexpr int kG = 4;  // steps whose loads are issued together
  const int eb = blockIdx.x % e_blocks;
  const int rest = blockIdx.x / e_blocks;
  const int c = rest % n_chunks;
  const int64_t bi = rest / n_chunks;
  const int64_t e = int64_t(eb) * kWave + threadIdx.x;
  const bool active = e < E;
  const int64_t ec = active ? e : E - 1;
  const int64_t t0 = int64_t(c) * kBwdChunk;
  const int n_steps = int(std::min<int64_t>(L - t0, kBwdChunk));

  float A2[kS];
#pragma unroll
  for (int n = 0; n < kS; n++) A2[n] = n < N ? A[ec * N + n] * kLog2e : 0.f;
  const float bv = bias ? bias[ec] : 0.f;
  float h[kS], X[kS], R[kS];
#pragma unroll
  for (int n = 0; n < kS; n++) {
    h[n] = 0.f;
    X[n] = 0.f;
    R[n] = 1.f;
  }
  double dsum = 0.0;

  const int64_t row0 = (bi * L + t0) * E + int64_t(eb) * kWave;
  const __amdgpu_buffer_rsrc_t ru = make_rsrc(u + row0);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(delta + row0);
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(dy + row0);
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(HAS_Z ? z + row0 : delta + row0);
  const int voff = int(ec - int64_t(eb) * kWave) * int(sizeof(T));
  const int row_bytes = int(E * int64_t(sizeof(T)));  // kBwdChunk * row_bytes < 2^31 is checked by the caller
  const float* brow0 = B16 + (bi * L + t0) * kS;
  const float* crow0 = C16 + (bi * L + t0) * kS;

  for (int k0 = 0; k0 < n_steps; k0 += kG) {
    float rd_[kG], ru_[kG], ry_[kG], rz_[kG];
#pragma unroll
    for (int g = 0; g < kG; g++) {  // rows past the chunk's end re-read its last row, unused
      const int so = std::min(k0 + g, n_steps - 1) * row_bytes;
      rd_[g] = buf_load(rd, voff, so, (T*)nullptr);
      ru_[g] = buf_load(ru, voff, so, (T*)nullptr);
      ry_[g] = buf_load(ry, voff, so, (T*)nullptr);
      rz_[g] = HAS_Z ? buf_load(rz, voff, so, (T*)nullptr) : 0.f;
    }
#pragma unroll
    for (int g = 0; g < kG; g++) {
      const int k = k0 + g;
      if (k < n_steps) {
        float d = rd_[g] + bv;
        if (SOFTPLUS) d = softplus(d);
        const float dx = d * ru_[g];
        const float dq = HAS_Z ? ry_[g] * silu(rz_[g]) : ry_[g];
        const float* br = brow0 + k * kS;  // wave-uniform: scalar loads
        const float* cr = crow0 + k * kS;
#pragma unroll
        for (int n = 0; n < kS; n++) {
          const float a = exp2_fast(d * A2[n]);
          h[n] = fmaf(a, h[n], dx * br[n]);
          R[n] *= a;
          X[n] = fmaf(R[n], dq * cr[n], X[n]);
        }
        dsum += double(d);
      }
    }
  }
  if (active) {
    const int64_t slot = (bi * n_chunks + c) * E + e;
    if (c < n_chunks - 1) {
#pragma unroll
      for (int n = 0; n < kS; n++)
        if (n < fslots) fagg[slot * fslots + n] = h[n];
    }
    if (c >= 1) {
#pragma unroll
      for (int n = 0; n < kS; n++) xagg[slot * kS + n] = X[n];
    }
    sums[slot] = float(dsum);
  }
}

// Sum over the 16 channels of a wave (lane = 4 * channel + quarter) of four
// values per lane, one per state of the lane's quarter; the 16 sums of the
// wave (state 4 * quarter + k) are written to dst[4 * quarter + k] by 16 lanes.
// Lane swaps across the wave halves and rows, then DPP rotations inside rows.
__device__ __forceinline__ void sum_channels(float v0, float v1, float v2, float v3, float* dst) {
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v0), __float_as_uint(v1), false, false);
  const float w01 = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);  // lanes < 32: v0, else v1
  sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v2), __float_as_uint(v3), false, false);
  const float w23 = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);  // lanes < 32: v2, else v3
  sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(w01), __float_as_uint(w23), false, false);
  float x = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);  // rows 0..3 hold v0, v2, v1, v3
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));  // row_ror:8
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xF, 0xF, false));  // row_ror:4
  const int l = threadIdx.x & (kWave - 1);
  if ((l & 12) == 4) {  // complete in lanes 4..7 of each row
    const int r = l >> 4;
    const int k = (r == 0) ? 0 : (r == 1) ? 2 : (r == 2) ? 1 : 3;
    dst[4 * (l & 3) + k] = x;
  }
}

// Streams of one chunk staged in LDS: [stream][step][channel of the block].
// Slots u, delta and z receive du, ddelta and dz once their inputs are dead.
enum { kSu = 0, kSd = 1, kSy = 2, kSz = 3 };

// ---------------------------------------------------------------------------
// 4. main backward pass over one chunk of one 64-channel block
// ---------------------------------------------------------------------------
// Occupancy: three workgroups per CU with bf16 streams; with fp32 streams the
// staged chunk doubles and LDS holds two.
template <typename T, bool SOFTPLUS, bool HAS_Z, bool HAS_D>
__global__ __launch_bounds__(kBwdWaves * kWave) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 3 : 2))) void bwd_main_kernel(
    const T* __restrict__ u, const T* __restrict__ delta, const float* __restrict__ A,
    const float* __restrict__ B16, const float* __restrict__ C16, const float* __restrict__ D,
    const T* __restrict__ z, const float* __restrict__ bias, const T* __restrict__ dy, const float* __restrict__ h0,
    const float* __restrict__ fcarry, int fslots, int fchunks, const float* __restrict__ xin, T* __restrict__ du,
    T* __restrict__ ddelta, T* __restrict__ dz, float* __restrict__ dh0, float* __restrict__ dA_part,
    float* __restrict__ dDb_part, float* __restrict__ dbc_part, int64_t L, int64_t E, int N, int n_chunks,
    int e_blocks) {
  constexpr int kStreams = HAS_Z ? 4 : 3;
  // rows padded by one 32-bit word so that the four lanes of a quad, reading four
  // different steps of one channel, fall into different LDS banks
  constexpr int kRowPad = kChPerBlock + 4 / int(sizeof(T));
  __shared__ T sio[kStreams][kBwdChunk][kRowPad];
  __shared__ float4 srow[2][kBwdChunk][kS / 4];  // B and C rows of the chunk
  __shared__ float red[kBwdWaves][kSub][kRed];
  const int eb = blockIdx.x % e_blocks;
  const int rest = blockIdx.x / e_blocks;
  const int c = rest % n_chunks;
  const int64_t bi = rest / n_chunks;
  const int wv = threadIdx.x / kWave;
  const int l = threadIdx.x % kWave;
  const int q = l & 3;
  const int chl = wv * kChPerWave + (l >> 2);  // channel inside the block
  const int64_t e = int64_t(eb) * kChPerBlock + chl;
  const bool active = e < E;
  const int64_t ec = active ? e : E - 1;
  const int64_t t0 = int64_t(c) * kBwdChunk;
  const int n_steps = int(std::min<int64_t>(L - t0, kBwdChunk));
  const bool lead = (q == 0) && active;  // the lane that writes the channel's per-step gradients

  // stage the chunk: thread (row group g, channel k) moves rows g, g + 4, ... of every stream
  const int64_t row0 = (bi * L + t0) * E + int64_t(eb) * kChPerBlock;
  const int row_bytes = int(E * int64_t(sizeof(T)));  // kBwdChunk * row_bytes < 2^31 is checked by the caller
  {
    const int k = threadIdx.x % kChPerBlock, g = threadIdx.x / kChPerBlock;
    const bool col_ok = int64_t(eb) * kChPerBlock + k < E;
    const int voff = (col_ok ? k : 0) * int(sizeof(T));
    const __amdgpu_buffer_rsrc_t rs[4] = {make_rsrc(u + row0), make_rsrc(delta + row0), make_rsrc(dy + row0),
                                          make_rsrc(HAS_Z ? z + row0 : u + row0)};
#pragma unroll
    for (int st = 0; st < kStreams; st++) {
      float v[kBwdChunk / kBwdWaves];
#pragma unroll
      for (int j = 0; j < kBwdChunk / kBwdWaves; j++) {
        const int r = g + kBwdWaves * j;
        // the row term goes into the lane offset: g is per wave but not provably uniform
        v[j] = buf_load(rs[st], voff + std::min(r, n_steps - 1) * row_bytes, 0, (T*)nullptr);
      }
      // a column past the last channel keeps the block's first channel's step (so its
      // retentions stay those of a real channel) and zero u and dy (so it adds nothing)
      const bool keep = st == kSd || st == kSz || col_ok;
#pragma unroll
      for (int j = 0; j < kBwdChunk / kBwdWaves; j++) {
        const int r = g + kBwdWaves * j;
        store_elem(&sio[st][r][k], (keep && r < n_steps) ? v[j] : 0.f);
      }
    }
    // B and C rows: 2 * 64 rows of 4 float4 = 512 float4, two per thread
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int idx = threadIdx.x + j * kBwdWaves * kWave;  // 0 .. 511
      const int which = idx / (kBwdChunk * 4), r = (idx / 4) % kBwdChunk, p = idx % 4;
      const float* src = (which ? C16 : B16) + (bi * L + t0 + std::min(r, n_steps - 1)) * kS + 4 * p;
      srow[which][r][p] = *reinterpret_cast<const float4*>(src);
    }
  }

  float Ar[4], A2[4];
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const int n = 4 * q + k;
    Ar[k] = n < N ? A[ec * N + n] : 0.f;
    A2[k] = Ar[k] * kLog2e;
  }
  const float bv = bias ? bias[ec] : 0.f;
  const float Dv = HAS_D ? D[ec] : 0.f;

  float h[4], X[4];
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const int n = 4 * q + k;
    if (c == 0)
      h[k] = (h0 && n < N) ? h0[(bi * E + ec) * N + n] : 0.f;
    else
      h[k] = n < N ? fcarry[((bi * fchunks + c - 1) * E + ec) * fslots + n] : 0.f;
    X[k] = xin[((bi * n_chunks + c) * E + ec) * kS + n];
  }
  __syncthreads();

  // Per-step scalars (step, gate and their derivatives) are computed once per
  // channel: in a group of four steps, quad lane q works out step g0 + q and the
  // quad shares the results through DPP broadcasts.  Lanes past the last
  // channel read u = dy = 0, so they add nothing to dB and dC.
  struct Scal {
    float d, x, dq, sg, gz;
  };
  auto own_scalars = [&](int i, bool with_grad) {  // i: this lane's step (rows past the end hold zeros)
    Scal r;
    r.x = load_elem(&sio[kSu][i][chl]);
    const float raw = load_elem(&sio[kSd][i][chl]) + bv;
    r.d = SOFTPLUS ? softplus(raw) : raw;
    r.sg = 1.f;
    r.dq = 0.f;
    r.gz = 0.f;
    if (with_grad) {
      if (SOFTPLUS) r.sg = sigmoid(raw);
      const float dyv = load_elem(&sio[kSy][i][chl]);
      r.dq = dyv;
      if (HAS_Z) {
        const float zv = load_elem(&sio[HAS_Z ? kSz : kSu][i][chl]);
        const float zs = sigmoid(zv);
        r.dq = dyv * zv * zs;                         // dy * silu(z)
        r.gz = dyv * zs * fmaf(zv, 1.f - zs, 1.f);   // dz = q * gz
      }
    }
    return r;
  };
  auto brow = [&](int i) {
    const float4 v = srow[0][i][q];
    return v;
  };
  auto crow = [&](int i) {
    const float4 v = srow[1][i][q];
    return v;
  };

  // pass A: checkpoints (state entering each sub-block).  The sub-block loops
  // stay rolled so the kernel's code fits the instruction cache; the
  // checkpoint slot (a wave-uniform index) is picked by comparison.
  typedef float ck_vec __attribute__((ext_vector_type(kNSub)));
  ck_vec ck[4];  // ck[k][sb]: state coordinate k entering sub-block sb
  auto ck_put = [&](int sb) {
#pragma unroll
    for (int k = 0; k < 4; k++) ck[k][sb] = h[k];
  };
  auto ck_get = [&](int sb, float (&out)[4]) {
#pragma unroll
    for (int k = 0; k < 4; k++) out[k] = ck[k][sb];
  };
  const int n_sub = (n_steps + kSub - 1) / kSub;
#pragma unroll 1
  for (int sb = 0; sb < n_sub; sb++) {
    ck_put(sb);
    if (sb < n_sub - 1) {  // a full sub-block
#pragma unroll
      for (int g0 = sb * kSub; g0 < (sb + 1) * kSub; g0 += 4) {
        const Scal own = own_scalars(g0 + q, false);
        const float own_dx = own.d * own.x;
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const float d = quad_bcast(own.d, j), dx = quad_bcast(own_dx, j);
          const float4 b4 = brow(g0 + j);
          const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
          for (int k = 0; k < 4; k++) h[k] = fmaf(exp2_fast(d * A2[k]), h[k], dx * bb[k]);
        }
      }
    }
  }

  // pass B: sub-blocks from the last to the first
  float dAacc[4] = {0.f, 0.f, 0.f, 0.f};
  float dDacc = 0.f, dbacc = 0.f;
  float* redw = &red[wv][0][0];
#pragma unroll 1
  for (int sb = n_sub - 1; sb >= 0; sb--) {
    const int base = sb * kSub;
    const int cnt = std::min(kSub, n_steps - base);
    float hs[kSub][4];
    float cd[kSub], cx[kSub], cq[kSub], cs[kSub];
    float h_in[4];
    ck_get(sb, h_in);
#pragma unroll
    for (int k = 0; k < 4; k++) h[k] = h_in[k];
    // forward over the sub-block: states, readout (for dz), dC
#pragma unroll
    for (int g = 0; g < kSub; g += 4) {
      if (g < cnt) {
        const Scal own = own_scalars(base + g + q, true);
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int i = g + j;
          if (i < cnt) {
            const float d = quad_bcast(own.d, j), x = quad_bcast(own.x, j), dq = quad_bcast(own.dq, j);
            const float4 b4 = brow(base + i);
            const float4 c4 = crow(base + i);
            const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
            const float cc[4] = {c4.x, c4.y, c4.z, c4.w};
            const float dx = d * x;
            float qp = 0.f;
#pragma unroll
            for (int k = 0; k < 4; k++) {
              h[k] = fmaf(exp2_fast(d * A2[k]), h[k], dx * bb[k]);
              hs[i][k] = h[k];
              qp = fmaf(cc[k], h[k], qp);
            }
            if (HAS_Z) {
              qp += quad_xor1(qp);
              qp += quad_xor2(qp);
              const float qt = HAS_D ? fmaf(Dv, x, qp) : qp;
              const float dzv = qt * quad_bcast(own.gz, j);
              if (lead) store_elem(&sio[HAS_Z ? kSz : kSu][base + i][chl], dzv);  // z of this step is dead now
            }
            if (HAS_D) dDacc = fmaf(dq, x, dDacc);
            sum_channels(dq * h[0], dq * h[1], dq * h[2], dq * h[3], redw + i * kRed + kS);
            cd[i] = d;
            cx[i] = x;
            cq[i] = dq;
            cs[i] = SOFTPLUS ? quad_bcast(own.sg, j) : 1.f;
          }
        }
      }
    }
    // reverse over the sub-block
#pragma unroll
    for (int i = kSub - 1; i >= 0; i--) {
      if (i < cnt) {
        const float4 b4 = brow(base + i);
        const float4 c4 = crow(base + i);
        const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
        const float cc[4] = {c4.x, c4.y, c4.z, c4.w};
        const float d = cd[i], x = cx[i], dq = cq[i];
        const float dx = d * x;
        float s1 = 0.f, ddp = 0.f, gb[4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
          const float G = fmaf(dq, cc[k], X[k]);
          const float a = exp2_fast(d * A2[k]);
          const float hp = (i > 0) ? hs[i > 0 ? i - 1 : 0][k] : h_in[k];
          const float gha = G * a * hp;
          dAacc[k] = fmaf(gha, d, dAacc[k]);
          ddp = fmaf(gha, Ar[k], ddp);
          s1 = fmaf(G, bb[k], s1);
          gb[k] = G * dx;
          X[k] = a * G;
        }
        s1 += quad_xor1(s1);
        s1 += quad_xor2(s1);
        ddp += quad_xor1(ddp);
        ddp += quad_xor2(ddp);
        const float dut = fmaf(s1, d, HAS_D ? dq * Dv : 0.f);
        const float ddv = fmaf(s1, x, ddp) * cs[i];
        if (lead) {  // u and delta of this step are dead now
          store_elem(&sio[kSu][base + i][chl], dut);
          store_elem(&sio[kSd][base + i][chl], ddv);
        }
        dbacc += ddv;
        sum_channels(gb[0], gb[1], gb[2], gb[3], redw + i * kRed);
      }
    }
    // dB / dC of the sub-block: the four waves' sums added in a fixed order
    __syncthreads();
    {
      const int i = threadIdx.x / kRed, v = threadIdx.x % kRed;  // 256 threads = kSub * kRed
      if (i < cnt)
        dbc_part[((bi * L + t0 + base + i) * e_blocks + eb) * kRed + v] =
            red[0][i][v] + red[1][i][v] + red[2][i][v] + red[3][i][v];
    }
    __syncthreads();
  }

  // per-step gradients of the chunk, from LDS to HBM in whole rows
  {
    const int k = threadIdx.x % kChPerBlock, g = threadIdx.x / kChPerBlock;
    const bool col_ok = int64_t(eb) * kChPerBlock + k < E;
    T* outs[3] = {du, ddelta, dz};
    const int slots[3] = {kSu, kSd, HAS_Z ? kSz : kSu};
#pragma unroll
    for (int o = 0; o < (HAS_Z ? 3 : 2); o++) {
      const __amdgpu_buffer_rsrc_t ro = make_rsrc(outs[o] + row0);
#pragma unroll
      for (int j = 0; j < kBwdChunk / kBwdWaves; j++) {
        const int r = g + kBwdWaves * j;
        if (col_ok && r < n_steps)
          buf_store(ro, k * int(sizeof(T)) + r * row_bytes, 0, load_elem(&sio[slots[o]][r][k]), (T*)nullptr);
      }
    }
  }

  if (active) {
    float* pa = dA_part + ((bi * n_chunks + c) * E + e) * kS + 4 * q;
#pragma unroll
    for (int k = 0; k < 4; k++) pa[k] = dAacc[k];
    if (q == 0) {
      dDb_part[((bi * n_chunks + c) * E + e) * 2 + 0] = dDacc;
      dDb_part[((bi * n_chunks + c) * E + e) * 2 + 1] = dbacc;
    }
    if (c == 0 && dh0) {
#pragma unroll
      for (int k = 0; k < 4; k++)
        if (4 * q + k < N) dh0[(bi * E + e) * N + 4 * q + k] = X[k];
    }
  }
}

// ---------------------------------------------------------------------------
// 5. sums of the partials, each in a fixed order
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_reduce_bc_kernel(const float* __restrict__ part, float* __restrict__ dB,
                                                            float* __restrict__ dC, int64_t rows, int e_blocks,
                                                            int N) {
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= rows * kRed) return;
  const int64_t r = gid / kRed;
  const int v = int(gid % kRed);
  const float* p = part + r * e_blocks * kRed + v;
  constexpr int U = 8;  // independent partial sums, added in a fixed order at the end
  float acc[U];
#pragma unroll
  for (int k = 0; k < U; k++) acc[k] = 0.f;
  int k0 = 0;
  for (; k0 + U <= e_blocks; k0 += U) {
#pragma unroll
    for (int k = 0; k < U; k++) acc[k] += p[int64_t(k0 + k) * kRed];
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < U; k++) s += acc[k];
  for (; k0 < e_blocks; k0++) s += p[int64_t(k0) * kRed];
  const int n = v % kS;
  if (n < N) (v < kS ? dB : dC)[r * N + n] = s;
}

// Per channel: slots 0..15 sum dA over (batch, chunk), slot 16 dD, slot 17 dbias.
constexpr int kChanSlots = kS + 2;

__global__ __launch_bounds__(256) void bwd_reduce_chan_kernel(const float* __restrict__ dA_part,
                                                              const float* __restrict__ dDb_part,
                                                              float* __restrict__ dA, float* __restrict__ dD,
                                                              float* __restrict__ dbias, int64_t parts, int64_t E,
                                                              int N) {
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= E * kChanSlots) return;
  const int64_t e = gid / kChanSlots;
  const int n = int(gid % kChanSlots);
  float* out = n < kS ? (n < N ? dA + e * N + n : nullptr) : (n == kS ? dD : dbias);
  if (!out) return;
  if (n >= kS) out += e;
  // slot stride and first element of part p: dA [parts][E][16], dD / dbias [parts][E][2]
  const float* base = n < kS ? dA_part + e * kS + n : dDb_part + e * 2 + (n - kS);
  const int64_t stride = n < kS ? E * kS : E * 2;
  constexpr int U = 8;
  float acc[U];
#pragma unroll
  for (int k = 0; k < U; k++) acc[k] = 0.f;
  int64_t p = 0;
  for (; p + U <= parts; p += U) {
#pragma unroll
    for (int k = 0; k < U; k++) acc[k] += base[(p + k) * stride];
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < U; k++) s += acc[k];
  for (; p < parts; p++) s += base[p * stride];
  *out = s;
}

// fill n floats with src (or zero when src is null)
__global__ __launch_bounds__(256) void bwd_fill_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                                       int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.f;
}

hipError_t fill(float* dst, const float* src, int64_t n, hipStream_t s) {
  if (!dst || n <= 0) return hipSuccess;
  return launch_kind(kKindBwdReduce, bwd_fill_kernel, (n + 255) / 256, 256, s, dst, src, n);
}

template <typename T, bool SOFTPLUS, bool HAS_Z, bool HAS_D>
hipError_t run_main(const BwdArgs& a, int n_chunks, int e_blocks, const float* B16, const float* C16,
                    const float* fcarry, int fslots, int fchunks, const float* xin, float* dA_part, float* dDb_part,
                    float* dbc_part) {
  return launch_kind(kKindBwdMain, bwd_main_kernel<T, SOFTPLUS, HAS_Z, HAS_D>, a.b * n_chunks * e_blocks,
                     kBwdWaves * kWave, a.stream, static_cast<const T*>(a.u), static_cast<const T*>(a.delta), a.A, B16,
                     C16, a.D, static_cast<const T*>(a.z), a.bias, static_cast<const T*>(a.dy), a.h0, fcarry, fslots,
                     fchunks, xin, static_cast<T*>(a.du), static_cast<T*>(a.ddelta), static_cast<T*>(a.dz), a.dh0,
                     dA_part, dDb_part, dbc_part, a.L, a.E, int(a.N), n_chunks, e_blocks);
}

// The forward and reverse chunk maps of a call without saved states, in one walk.
template <typename T>
hipError_t run_maps(const BwdArgs& a, int n_chunks, const float* B16, const float* C16, float* fagg, int fslots,
                    float* xagg, float* sums) {
  const int eb = int((a.E + kWave - 1) / kWave);
  const int64_t blocks = a.b * n_chunks * eb;
  const T* u = static_cast<const T*>(a.u);
  const T* dl = static_cast<const T*>(a.delta);
  const T* dyp = static_cast<const T*>(a.dy);
  const T* zp = static_cast<const T*>(a.z);
#define SSM_BWD_MAPS(SP, HZ)                                                                                     \
  return launch_kind(kKindBwdAgg, bwd_chunk_maps_kernel<T, SP, HZ>, blocks, kWave, a.stream, u, dl, dyp, zp, a.A, \
                     B16, C16, a.bias, fagg, fslots, xagg, sums, a.L, a.E, int(a.N), n_chunks, eb)
  if (a.softplus) {
    if (a.z) SSM_BWD_MAPS(true, true);
    SSM_BWD_MAPS(true, false);
  }
  if (a.z) SSM_BWD_MAPS(false, true);
  SSM_BWD_MAPS(false, false);
#undef SSM_BWD_MAPS
}

// rev_done: the reverse chunk maps and sums are already in xagg / xsum (run_maps)
template <typename T>
hipError_t bwd_typed(const BwdArgs& a, int n_chunks, const float* B16, const float* C16, const float* fcarry,
                     int fslots, int fchunks, float* xagg, float* xsum, float* dA_part, float* dDb_part,
                     float* dbc_part, bool rev_done) {
  const int N = int(a.N);
  const int eb_agg = int((a.E + kWave - 1) / kWave);
  hipError_t err = hipSuccess;
  if (n_chunks > 1 && !rev_done) {
    const int64_t blocks = a.b * (n_chunks - 1) * eb_agg;
    const T* dl = static_cast<const T*>(a.delta);
    const T* dyp = static_cast<const T*>(a.dy);
    const T* zp = static_cast<const T*>(a.z);
#define SSM_BWD_AGG(SP, HZ)                                                                                       \
  err = launch_kind(kKindBwdAgg, bwd_chunk_agg_kernel<T, SP, HZ>, blocks, kWave, a.stream, dl, dyp, zp, a.A, C16, \
                    a.bias, xagg, xsum, a.L, a.E, N, n_chunks, eb_agg)
    if (a.softplus) {
      if (a.z) SSM_BWD_AGG(true, true); else SSM_BWD_AGG(true, false);
    } else {
      if (a.z) SSM_BWD_AGG(false, true); else SSM_BWD_AGG(false, false);
    }
#undef SSM_BWD_AGG
    if (err != hipSuccess) return err;
  }
  // slot c <- the gradient entering chunk c from its end, for c = last .. 1 (reverse, exclusive),
  // then slot 0 <- the gradient reaching the start of the sequence
  const ChainArgs chain{xagg, xsum, a.A, a.dlast, nullptr, a.b, a.E, kS, N, n_chunks, n_chunks - 1};
  err = launch_chain<true, true, true>(kKindBwdCarry, chain, a.stream);
  if (err != hipSuccess) return err;
  const int e_blocks = int((a.E + kChPerBlock - 1) / kChPerBlock);
#define SSM_BWD_MAIN(SP, HZ, HD)                                                                              \
  return run_main<T, SP, HZ, HD>(a, n_chunks, e_blocks, B16, C16, fcarry, fslots, fchunks, xagg, dA_part, dDb_part, \
                                 dbc_part)
  const bool hz = a.z != nullptr, hd = a.D != nullptr;
  if (a.softplus) {
    if (hz) { if (hd) SSM_BWD_MAIN(true, true, true); else SSM_BWD_MAIN(true, true, false); }
    if (hd) SSM_BWD_MAIN(true, false, true);
    SSM_BWD_MAIN(true, false, false);
  }
  if (hz) { if (hd) SSM_BWD_MAIN(false, true, true); else SSM_BWD_MAIN(false, true, false); }
  if (hd) SSM_BWD_MAIN(false, false, true);
  SSM_BWD_MAIN(false, false, false);
#undef SSM_BWD_MAIN
}

}  // namespace

int64_t bwd_chunk_steps() { return kBwdChunk; }

hipError_t launch_scan_bwd(const BwdArgs& a) {
  const int64_t b = a.b, L = a.L, E = a.E, N = a.N;
  if (E == 0) {  // no channel: B and C receive nothing
    hipError_t err = fill(a.dB, nullptr, b * L * N, a.stream);
    return err == hipSuccess ? fill(a.dC, nullptr, b * L * N, a.stream) : err;
  }
  if (b == 0 || L == 0) {  // nothing flows through a step: parameter gradients are zero
    hipError_t err = fill(a.dA, nullptr, E * N, a.stream);
    if (err == hipSuccess) err = fill(a.dD, nullptr, a.D ? E : 0, a.stream);
    if (err == hipSuccess) err = fill(a.dbias, nullptr, a.bias ? E : 0, a.stream);
    if (err == hipSuccess) err = fill(a.dh0, a.dlast, b * E * N, a.stream);
    return err;
  }
  const int n_chunks = int((L + kBwdChunk - 1) / kBwdChunk);
  const int e_blocks = int((E + kChPerBlock - 1) / kChPerBlock);
  // states entering the chunks: the forward's saved states ([b, chunk - 1, E, N]) when
  // given (the chunk is the save interval), else recomputed here
  static_assert(kBwdChunk == kSaveEvery, "the saved states are the chunk boundaries");
  const bool saved = a.saved != nullptr;
  const int fslots = saved ? int(N) : chunk_state_slots(N);
  const int fchunks = saved ? n_chunks - 1 : n_chunks;  // chunk slots per batch row
  // workspace (floats): [B16 | C16 | forward carries | (unused) | reverse carries |
  //                      chunk sums | dB/dC partials | dA partials | dD/dbias partials]
  // (without saved states one walk per chunk gives both carries' maps and the sums both chains use)
  const size_t nb = size_t(b), nL = size_t(L), nE = size_t(E), nc = size_t(n_chunks);
  const size_t n_row16 = nb * nL * kS;
  const size_t n_fc = n_chunks > 1 && !saved ? nb * nc * nE * size_t(fslots) : 0;
  const size_t n_fs = 0;
  const size_t n_xa = nb * nc * nE * kS;
  const size_t n_xs = nb * nc * nE;
  const size_t n_bc = nb * nL * size_t(e_blocks) * kRed;
  const size_t n_da = nb * nc * nE * kS;
  const size_t n_dd = nb * nc * nE * 2;
  // every segment starts on a 256-byte boundary (the main kernel reads rows as float4)
  const size_t sizes[9] = {n_row16, n_row16, n_fc, n_fs, n_xa, n_xs, n_bc, n_da, n_dd};
  size_t offs[9], total = 0;
  for (int i = 0; i < 9; i++) {
    offs[i] = total;
    total += (sizes[i] + 63) / 64 * 64;
  }
  void* ws = nullptr;
  hipError_t err = hipMallocAsync(&ws, total * sizeof(float), a.stream);
  if (err != hipSuccess) return err;
  float* f = static_cast<float*>(ws);
  float* B16 = f + offs[0];
  float* C16 = f + offs[1];
  const float* fcarry = saved ? a.saved : f + offs[2];
  float* xagg = f + offs[4];
  float* xsum = f + offs[5];
  float* dbc = f + offs[6];
  float* dA_part = f + offs[7];
  float* dDb_part = f + offs[8];

  const int64_t nr16 = b * L * kS;
  err = a.dtype == 0 ? launch_kind(kKindBwdRows, bwd_rows_kernel<float>, (nr16 + 255) / 256, 256, a.stream,
                                   static_cast<const float*>(a.B), static_cast<const float*>(a.C), B16, C16, b * L,
                                   int(N))
                     : launch_kind(kKindBwdRows, bwd_rows_kernel<bf16_bits>, (nr16 + 255) / 256, 256, a.stream,
                                   static_cast<const bf16_bits*>(a.B), static_cast<const bf16_bits*>(a.C), B16, C16,
                                   b * L, int(N));
  const bool maps = n_chunks > 1 && !saved;
  if (err == hipSuccess && maps) {
    // both chunk maps and the sums, then the forward chain: slot c <- the state leaving chunk c
    err = a.dtype == 0 ? run_maps<float>(a, n_chunks, B16, C16, f + offs[2], fslots, xagg, xsum)
                       : run_maps<bf16_bits>(a, n_chunks, B16, C16, f + offs[2], fslots, xagg, xsum);
    if (err == hipSuccess) {
      const ChainArgs fc{f + offs[2], xsum, a.A, a.h0, nullptr, b, E, fslots, int(N), n_chunks, n_chunks - 1};
      err = launch_chain<false, false, false>(kKindCarry, fc, a.stream);
    }
  }
  if (err == hipSuccess)
    err = a.dtype == 0 ? bwd_typed<float>(a, n_chunks, B16, C16, fcarry, fslots, fchunks, xagg, xsum, dA_part,
                                          dDb_part, dbc, maps)
                       : bwd_typed<bf16_bits>(a, n_chunks, B16, C16, fcarry, fslots, fchunks, xagg, xsum, dA_part,
                                              dDb_part, dbc, maps);
  if (err == hipSuccess) {
    const int64_t n = b * L * kRed;
    err = launch_kind(kKindBwdReduce, bwd_reduce_bc_kernel, (n + 255) / 256, 256, a.stream, (const float*)dbc, a.dB,
                      a.dC, b * L, e_blocks, int(N));
  }
  if (err == hipSuccess) {
    const int64_t n = E * kChanSlots;
    err = launch_kind(kKindBwdReduce, bwd_reduce_chan_kernel, (n + 255) / 256, 256, a.stream, (const float*)dA_part,
                      (const float*)dDb_part, a.dA, a.D ? a.dD : nullptr, a.bias ? a.dbias : nullptr,
                      b * int64_t(n_chunks), E, int(N));
  }
  hipError_t ferr = hipFreeAsync(ws, a.stream);
  return err != hipSuccess ? err : ferr;
}

}  // namespace ssm
