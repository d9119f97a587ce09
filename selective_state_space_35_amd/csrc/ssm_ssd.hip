// ssm_ssd.hip -- the scan with a scalar transition per head (structured
// state-space duality), computed in chunks of matrix products on the MFMA units.
//
// Pages: "Mamba: Linear-Time Sequence Modeling with Selective State Spaces"
// (abhik.ai), "Key takeaways" / "Related reading": restricting the transition
// turns the state update into a structured mixing matrix computed in chunks;
// "mamba-from-scratch" README: Mamba-2 / SSD as a chunked parallel scan.
//
// Definition (the scan of ssm_scan_fwd with A, the step, D and the step bias
// shared by the P = 64 channels of a head and A the same for every state):
//   d_t = softplus(delta[t,h] + bias[h]),  S_t = running sum of d over the sequence
//   y[t, e] = sum_{s<=t} (C_t . B_s) exp(A_h (S_t - S_s)) d_s x[s, e] + D_h x[t, e]
//             (+ the incoming state's contribution), then times silu(z[t, e])
// For a chunk of Q steps starting from state S_in [N, P] of head h
// (cum_t = A_h * (S_t - S_{chunk start})):
//   Y   = diag(exp(cum)) (C S_in)  +  (L o (C B^T)) X,   L[t,s] = exp(cum_t - cum_s) d_s for s <= t
//   S_out = exp(cum_last) S_in + B^T (w o X),            w_s = exp(cum_last - cum_s) d_s
//
// Kernels (bf16 I/O; matrix products take bf16 operands and accumulate in fp32;
// chunk states are handed between kernels in bf16, laid out [p][n]):
//   ssd_state_kernel  per (batch, chunk, head): (w o X)^T B -> chunk state [P, N]
//   ssd_carry_kernel  per (batch, head, p, n): chain of chunk states (fp32 in registers) -> state entering each chunk
//   ssd_scan_kernel   per (batch, chunk, head): Y as above, + D x, gate, store
// MFMA: v_mfma_f32_16x16x32_bf16.  Lane l of a wave holds A-operand row l % 16,
// k = 8 (l / 16) .. +7; B-operand column l % 16, same k; result rows
// 4 (l / 16) .. +3 of column l % 16.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "ssm_device.h"
#include "ssm_internal.h"
#include "ssm_profile.h"

namespace ssm {
namespace {

constexpr int kQ = 64;           // steps per chunk
constexpr int kP = 64;           // channels per head
constexpr int kSsdThreads = 256; // 4 waves
constexpr int kPad = 8;          // bf16 elements added to every LDS row (breaks bank aliasing)

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 8 consecutive bf16 from LDS (16-byte aligned)
__device__ __forceinline__ bf16x8 lds8(const bf16_bits* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16_bits to_bf16(float v) { return __builtin_bit_cast(bf16_bits, static_cast<__bf16>(v)); }
__device__ __forceinline__ float from_bf16(bf16_bits v) { return __uint_as_float(uint32_t(v) << 16); }

// Column index of element k in row r of a transposed tile: 8-element (16-byte)
// blocks are XOR-swizzled by (r / 8) mod 8, so the transposed writes of eight
// rows r, r + 8, ... land in different LDS banks, while every 16-byte block
// (all an MFMA fragment reads) stays contiguous.
__device__ __forceinline__ int swz(int r, int k) { return (((k >> 3) ^ ((r >> 3) & 7)) << 3) | (k & 7); }

// Steps and their running sums inside the chunk: d[s] (0 past the end) and
// cum[s] = A_h * (d_0 + ... + d_s), computed by the first wave.
template <bool SOFTPLUS>
__device__ __forceinline__ void chunk_steps(const bf16_bits* __restrict__ delta, const float* __restrict__ bias,
                                            float Ah, int64_t row0, int H, int h, int n_steps, float* d_s,
                                            float* cum_s) {
  if (threadIdx.x < kWave) {
    const int s = threadIdx.x;
    float d = 0.f;
    if (s < n_steps) {
      d = from_bf16(delta[(row0 + s) * H + h]) + (bias ? bias[h] : 0.f);
      if (SOFTPLUS) d = softplus(d);
    }
    float c = d * Ah;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const float o = __shfl_up(c, off);
      if (s >= off) c += o;
    }
    d_s[s] = d;
    cum_s[s] = c;
  }
}

// [rows x cols] bf16 tile of a row-major global matrix (row stride ld elements,
// 16-byte aligned rows, cols a multiple of 8) into LDS with row stride lds_ld;
// rows >= valid_rows and columns >= valid_cols are zero.
__device__ __forceinline__ void stage_rows(const bf16_bits* __restrict__ src, int64_t ld, int rows, int valid_rows,
                                           int cols, int valid_cols, bf16_bits* dst, int lds_ld) {
  const int per_row = cols / 8;
  for (int i = threadIdx.x; i < rows * per_row; i += kSsdThreads) {
    const int r = i / per_row, c8 = (i % per_row) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < valid_rows && c8 < valid_cols) v = *reinterpret_cast<const uint4*>(src + r * ld + c8);
    *reinterpret_cast<uint4*>(dst + r * lds_ld + c8) = v;
  }
}

// ---------------------------------------------------------------------------
// chunk state, transposed: S_c[p, n] = sum_s (w o X)[s, p] B[s, n]  (bf16 out)
// ---------------------------------------------------------------------------
template <int NK, bool SOFTPLUS>  // NK: the state size padded to a multiple of 32, in units of 32
__global__ __launch_bounds__(kSsdThreads) void ssd_state_kernel(
    const bf16_bits* __restrict__ x, const bf16_bits* __restrict__ delta, const float* __restrict__ A,
    const bf16_bits* __restrict__ B, const float* __restrict__ bias, bf16_bits* __restrict__ states,
    float* __restrict__ cum_last, int64_t L, int H, int N, int n_chunks) {
  constexpr int NP = NK * 32;
  __shared__ float d_s[kQ], cum_s[kQ];
  __shared__ __attribute__((aligned(16))) bf16_bits Bt[NP][kQ + kPad];   // B transposed: [n][s]
  __shared__ __attribute__((aligned(16))) bf16_bits Xw[kP][kQ + kPad];   // (w o X) transposed: [p][s]
  const int h = blockIdx.x % H;
  const int rest = blockIdx.x / H;
  const int c = rest % n_chunks;
  const int64_t bi = rest / n_chunks;
  const int64_t t0 = int64_t(c) * kQ;
  const int n_steps = int(std::min<int64_t>(kQ, L - t0));
  const int64_t row0 = bi * L + t0;
  const int64_t E = int64_t(H) * kP;
  chunk_steps<SOFTPLUS>(delta, bias, A[h], row0, H, h, n_steps, d_s, cum_s);
  // B^T: 16-byte row reads, transposed writes
  for (int i = threadIdx.x; i < kQ * (NP / 8); i += kSsdThreads) {
    const int s = i / (NP / 8), n8 = (i % (NP / 8)) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (s < n_steps && n8 < N) v = *reinterpret_cast<const uint4*>(B + (row0 + s) * N + n8);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; j++) {
      Bt[n8 + 2 * j][swz(n8 + 2 * j, s)] = bf16_bits(u[j] & 0xffff);
      Bt[n8 + 2 * j + 1][swz(n8 + 2 * j + 1, s)] = bf16_bits(u[j] >> 16);
    }
  }
  __syncthreads();
  const float last = cum_s[kQ - 1];
  for (int i = threadIdx.x; i < kQ * (kP / 8); i += kSsdThreads) {
    const int s = i / (kP / 8), p8 = (i % (kP / 8)) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (s < n_steps) v = *reinterpret_cast<const uint4*>(x + (row0 + s) * E + int64_t(h) * kP + p8);
    const float w = exp2_fast((last - cum_s[s]) * kLog2e) * d_s[s];
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; j++) {
      Xw[p8 + 2 * j][swz(p8 + 2 * j, s)] = to_bf16(from_bf16(bf16_bits(u[j] & 0xffff)) * w);
      Xw[p8 + 2 * j + 1][swz(p8 + 2 * j + 1, s)] = to_bf16(from_bf16(bf16_bits(u[j] >> 16)) * w);
    }
  }
  __syncthreads();
  // wave w: rows p in [16 w, 16 w + 16), every 16-column block of n
  const int wv = threadIdx.x / kWave, l = threadIdx.x % kWave;
  const int lr = l % 16, lk = 8 * (l / 16);
  bf16_bits* out = states + ((bi * n_chunks + c) * H + h) * int64_t(kP) * N;  // [p][n]
  bf16x8 xf[kQ / 32];
#pragma unroll
  for (int kk = 0; kk < kQ / 32; kk++) xf[kk] = lds8(&Xw[wv * 16 + lr][swz(wv * 16 + lr, kk * 32 + lk)]);
#pragma unroll
  for (int nb = 0; nb < NP / 16; nb++) {
    if (nb * 16 >= N) break;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kQ / 32; kk++)
      acc = mfma(xf[kk], lds8(&Bt[nb * 16 + lr][swz(nb * 16 + lr, kk * 32 + lk)]), acc);
#pragma unroll
    for (int r = 0; r < 4; r++) out[int64_t(wv * 16 + 4 * (l / 16) + r) * N + nb * 16 + lr] = to_bf16(acc[r]);
  }
  if (threadIdx.x == 0) cum_last[(bi * n_chunks + c) * H + h] = last;
}

// ---------------------------------------------------------------------------
// carry: per (batch, head, p, n), state entering chunk c (bf16, in place of
// S_c; the chain itself is kept in fp32); the state after the last chunk goes
// to last_state [b, E, N] in fp32
// ---------------------------------------------------------------------------
template <int U>
__global__ __launch_bounds__(256) void ssd_carry_kernel(bf16_bits* states, const float* __restrict__ cum_last,
                                                        const float* __restrict__ h0, float* __restrict__ last_state,
                                                        int64_t b, int H, int N, int n_chunks) {
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per_head = int64_t(N) * kP;
  if (gid >= b * H * per_head) return;
  const int64_t within = gid % per_head;  // p * N + n
  const int64_t bh = gid / per_head;
  const int h = int(bh % H);
  const int64_t bi = bh / H;
  const int64_t E = int64_t(H) * kP;
  const int64_t st = (bi * E + int64_t(h) * kP) * N + within;  // [b][e = h P + p][n]
  float S = h0 ? h0[st] : 0.f;
  auto slot = [&](int c) { return ((bi * n_chunks + c) * H + h) * per_head + within; };
  float Ss[U], Ls[U];
  auto load = [&](int c0) {
#pragma unroll
    for (int k = 0; k < U; k++) {
      const int cc = (c0 + k < n_chunks) ? c0 + k : n_chunks - 1;  // past the end: a valid slot, unused
      Ss[k] = from_bf16(states[slot(cc)]);
      Ls[k] = cum_last[(bi * n_chunks + cc) * H + h];
    }
  };
  load(0);
  for (int c0 = 0; c0 < n_chunks; c0 += U) {
    float Sc[U], Lc[U];
#pragma unroll
    for (int k = 0; k < U; k++) { Sc[k] = Ss[k]; Lc[k] = Ls[k]; }
    if (c0 + U < n_chunks) load(c0 + U);
#pragma unroll
    for (int k = 0; k < U; k++) {
      if (c0 + k < n_chunks) {
        states[slot(c0 + k)] = to_bf16(S);
        S = fmaf(exp2_fast(Lc[k] * kLog2e), S, Sc[k]);
      }
    }
  }
  if (last_state) last_state[st] = S;
}

// ---------------------------------------------------------------------------
// outputs of a chunk.  Wave w owns steps t in [16 w, 16 w + 16).  The mixing
// matrix is built transposed (rows s, columns t) so that each lane ends with
// its own step t in registers: those values are the A operand of the next
// product directly, with the contraction index s in the order the transposed
// tiles give it (s = 4 g + r and 16 + 4 g + r for lane group g); X is read in
// the same order.
// ---------------------------------------------------------------------------
template <int NK, bool SOFTPLUS, bool HAS_Z, bool HAS_D>
__global__ __launch_bounds__(kSsdThreads) void ssd_scan_kernel(
    const bf16_bits* __restrict__ x, const bf16_bits* __restrict__ delta, const float* __restrict__ A,
    const bf16_bits* __restrict__ B, const bf16_bits* __restrict__ C, const float* __restrict__ D,
    const bf16_bits* __restrict__ z, const float* __restrict__ bias, const bf16_bits* __restrict__ states,
    bf16_bits* __restrict__ y, int64_t L, int H, int N, int n_chunks) {
  constexpr int NP = NK * 32;
  __shared__ float d_s[kQ], cum_s[kQ];
  __shared__ __attribute__((aligned(16))) bf16_bits Cs[kQ][NP + kPad];    // C rows [t][n]
  __shared__ __attribute__((aligned(16))) bf16_bits Bs[kQ][NP + kPad];    // B rows [s][n]
  __shared__ __attribute__((aligned(16))) bf16_bits Xt[kP][kQ + kPad];    // X transposed [p][s]
  const int h = blockIdx.x % H;
  const int rest = blockIdx.x / H;
  const int c = rest % n_chunks;
  const int64_t bi = rest / n_chunks;
  const int64_t t0 = int64_t(c) * kQ;
  const int n_steps = int(std::min<int64_t>(kQ, L - t0));
  const int64_t row0 = bi * L + t0;
  const int64_t E = int64_t(H) * kP;
  const int wv = threadIdx.x / kWave, l = threadIdx.x % kWave;
  const int lr = l % 16, lg = l / 16, lk = 8 * lg, lq = 4 * lg;
  const int tb = wv;                 // this wave's step block
  const int t_own = tb * 16 + lr;    // the step this lane carries through the mixing product
  // Global reads this lane needs later are issued first, so their latency overlaps
  // the staging and the mixing matrix: the gate of its outputs and the incoming
  // state's fragments ([p][n] bf16).
  float zv[kP / 16][4];
  if (HAS_Z) {
#pragma unroll
    for (int pb = 0; pb < kP / 16; pb++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int t = tb * 16 + lq + r;
        zv[pb][r] = t < n_steps ? from_bf16(z[(row0 + t) * E + int64_t(h) * kP + pb * 16 + lr]) : 0.f;
      }
  }
  const bf16_bits* Sin = states + ((bi * n_chunks + c) * H + h) * int64_t(kP) * N;
  bf16x8 sfr[kP / 16][NK];
#pragma unroll
  for (int pb = 0; pb < kP / 16; pb++)
#pragma unroll
    for (int kk = 0; kk < NK; kk++) {
      if (kk * 32 + lk < N) {
        sfr[pb][kk] = *reinterpret_cast<const bf16x8*>(Sin + int64_t(pb * 16 + lr) * N + kk * 32 + lk);
      } else {
#pragma unroll
        for (int j = 0; j < 8; j++) sfr[pb][kk][j] = static_cast<__bf16>(0.f);
      }
    }
  chunk_steps<SOFTPLUS>(delta, bias, A[h], row0, H, h, n_steps, d_s, cum_s);
  stage_rows(C + row0 * N, N, kQ, n_steps, NP, N, &Cs[0][0], NP + kPad);
  stage_rows(B + row0 * N, N, kQ, n_steps, NP, N, &Bs[0][0], NP + kPad);
  for (int i = threadIdx.x; i < kQ * (kP / 8); i += kSsdThreads) {
    const int s = i / (kP / 8), p8 = (i % (kP / 8)) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (s < n_steps) v = *reinterpret_cast<const uint4*>(x + (row0 + s) * E + int64_t(h) * kP + p8);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; j++) {
      Xt[p8 + 2 * j][s] = bf16_bits(u[j] & 0xffff);
      Xt[p8 + 2 * j + 1][s] = bf16_bits(u[j] >> 16);
    }
  }
  __syncthreads();

  const float cum_t = cum_s[t_own];
  bf16x8 cf[NK];                     // C rows of this wave's steps, as the operand [k = n][column t]
#pragma unroll
  for (int kk = 0; kk < NK; kk++) cf[kk] = lds8(&Cs[tb * 16 + lr][kk * 32 + lk]);

  // mixing matrix, transposed tiles (rows s, column t): m[sb][r] = M[t_own][16 sb + 4 g + r]
  float m[kQ / 16][4];
#pragma unroll
  for (int sb = 0; sb < kQ / 16; sb++) {
#pragma unroll
    for (int r = 0; r < 4; r++) m[sb][r] = 0.f;
    if (sb <= tb) {  // blocks above the diagonal are zero
      f32x4 g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK; kk++) g = mfma(lds8(&Bs[sb * 16 + lr][kk * 32 + lk]), cf[kk], g);
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int s = sb * 16 + lq + r;
        m[sb][r] = (s <= t_own) ? g[r] * exp2_fast((cum_t - cum_s[s]) * kLog2e) * d_s[s] : 0.f;
      }
    }
  }
  // A operands of the in-chunk product: K block kk covers s in [32 kk, 32 kk + 32) in the order
  // (4 g + r, 16 + 4 g + r), r = 0..3
  bf16x8 mf[kQ / 32];
#pragma unroll
  for (int kk = 0; kk < kQ / 32; kk++) {
#pragma unroll
    for (int r = 0; r < 4; r++) {
      mf[kk][r] = static_cast<__bf16>(m[2 * kk][r]);
      mf[kk][4 + r] = static_cast<__bf16>(m[2 * kk + 1][r]);
    }
  }
  const float Dh = HAS_D ? D[h] : 0.f;
  float row_scale[4];  // exp(cum_t) of this lane's output rows
#pragma unroll
  for (int r = 0; r < 4; r++) row_scale[r] = exp2_fast(cum_s[tb * 16 + lq + r] * kLog2e);
#pragma unroll
  for (int pb = 0; pb < kP / 16; pb++) {
    const int p = pb * 16 + lr;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // incoming-state part: [t][n] x [n][p]; rows scaled by exp(cum_t)
#pragma unroll
    for (int kk = 0; kk < NK; kk++)
      acc = mfma(cf[kk], sfr[pb][kk], acc);  // the C fragment serves as the A operand [row t][k = n] here
#pragma unroll
    for (int r = 0; r < 4; r++) acc[r] *= row_scale[r];
    // in-chunk part: M [t][s] x X [s][p], s in the permuted order
#pragma unroll
    for (int kk = 0; kk < kQ / 32; kk++) {
      if (2 * kk > tb) break;  // M is zero there
      bf16x8 xf;
      const uint2 lo = *reinterpret_cast<const uint2*>(&Xt[p][kk * 32 + lq]);
      const uint2 hi = *reinterpret_cast<const uint2*>(&Xt[p][kk * 32 + 16 + lq]);
      xf = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
      acc = mfma(mf[kk], xf, acc);
    }
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int t = tb * 16 + lq + r;
      if (t < n_steps) {
        const int64_t idx = (row0 + t) * E + int64_t(h) * kP + p;
        float v = acc[r];
        if (HAS_D) v = fmaf(Dh, from_bf16(Xt[p][t]), v);
        if (HAS_Z) v *= silu(zv[pb][r]);
        y[idx] = to_bf16(v);
      }
    }
  }
}

// last state of an empty sequence: the incoming one (same [b, E, N] layout), or zeros
__global__ __launch_bounds__(256) void ssd_fill_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                                       int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.f;
}

template <int NK, bool SOFTPLUS>
hipError_t run_ssd(const SsdArgs& a, int n_chunks, bf16_bits* states, float* cum_last) {
  const int H = int(a.H), N = int(a.N);
  const int64_t blocks = a.b * n_chunks * H;
  const bf16_bits* x = static_cast<const bf16_bits*>(a.x);
  const bf16_bits* dl = static_cast<const bf16_bits*>(a.delta);
  const bf16_bits* B = static_cast<const bf16_bits*>(a.B);
  const bf16_bits* C = static_cast<const bf16_bits*>(a.C);
  const bf16_bits* z = static_cast<const bf16_bits*>(a.z);
  hipError_t err = launch_kind(kKindSsdState, ssd_state_kernel<NK, SOFTPLUS>, blocks, kSsdThreads, a.stream, x, dl,
                               a.A, B, a.bias, states, cum_last, a.L, H, N, n_chunks);
  if (err != hipSuccess) return err;
  const int64_t lanes = a.b * H * int64_t(N) * kP;
  err = n_chunks > 33 ? launch_kind(kKindSsdCarry, ssd_carry_kernel<16>, (lanes + 255) / 256, 256, a.stream, states,
                                    (const float*)cum_last, a.h0, a.last_state, a.b, H, N, n_chunks)
                      : launch_kind(kKindSsdCarry, ssd_carry_kernel<4>, (lanes + 255) / 256, 256, a.stream, states,
                                    (const float*)cum_last, a.h0, a.last_state, a.b, H, N, n_chunks);
  if (err != hipSuccess) return err;
  bf16_bits* y = static_cast<bf16_bits*>(a.y);
#define SSM_SSD_SCAN(HZ, HD)                                                                                  \
  return launch_kind(kKindSsdScan, ssd_scan_kernel<NK, SOFTPLUS, HZ, HD>, blocks, kSsdThreads, a.stream, x, dl, \
                     a.A, B, C, a.D, z, a.bias, (const bf16_bits*)states, y, a.L, H, N, n_chunks)
  if (a.z) {
    if (a.D) SSM_SSD_SCAN(true, true);
    SSM_SSD_SCAN(true, false);
  }
  if (a.D) SSM_SSD_SCAN(false, true);
  SSM_SSD_SCAN(false, false);
#undef SSM_SSD_SCAN
}

template <int NK>
hipError_t ssd_sp(const SsdArgs& a, int n_chunks, bf16_bits* states, float* cum_last) {
  return a.softplus ? run_ssd<NK, true>(a, n_chunks, states, cum_last) : run_ssd<NK, false>(a, n_chunks, states, cum_last);
}

}  // namespace

int64_t ssd_chunk_steps() { return kQ; }
int64_t ssd_head_dim() { return kP; }

hipError_t launch_ssd(const SsdArgs& a) {
  if (a.b == 0 || a.H == 0) return hipSuccess;
  if (a.L == 0) {  // no step: the last state is the incoming one
    if (!a.last_state) return hipSuccess;
    const int64_t n = a.b * a.H * kP * a.N;
    return launch_kind(kKindSsdCarry, ssd_fill_kernel, (n + 255) / 256, 256, a.stream, a.last_state, a.h0, n);
  }
  const int n_chunks = int((a.L + kQ - 1) / kQ);
  // workspace: chunk states [b][chunk][h][p][n] in bf16, then the chunks' decay exponents
  const size_t n_states = size_t(a.b) * size_t(n_chunks) * size_t(a.H) * size_t(a.N) * kP;
  const size_t n_cum = size_t(a.b) * size_t(n_chunks) * size_t(a.H);
  const size_t state_bytes = (n_states * sizeof(bf16_bits) + 255) / 256 * 256;
  void* ws = nullptr;
  hipError_t err = hipMallocAsync(&ws, state_bytes + n_cum * sizeof(float), a.stream);
  if (err != hipSuccess) return err;
  bf16_bits* states = static_cast<bf16_bits*>(ws);
  float* cum_last = reinterpret_cast<float*>(static_cast<char*>(ws) + state_bytes);
  const int nk = int((a.N + 31) / 32);
  switch (nk) {
    case 1: err = ssd_sp<1>(a, n_chunks, states, cum_last); break;
    case 2: err = ssd_sp<2>(a, n_chunks, states, cum_last); break;
    case 3: err = ssd_sp<3>(a, n_chunks, states, cum_last); break;
    default: err = ssd_sp<4>(a, n_chunks, states, cum_last); break;
  }
  hipError_t ferr = hipFreeAsync(ws, a.stream);
  return err != hipSuccess ? err : ferr;
}

}  // namespace ssm
