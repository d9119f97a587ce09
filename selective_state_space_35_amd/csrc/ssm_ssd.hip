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

#ifndef SSM_SSD_CHUNK
#define SSM_SSD_CHUNK 128
#endif
constexpr int kQ = SSM_SSD_CHUNK;   // steps per chunk (64 or 128)
constexpr int kP = 64;              // channels per head
constexpr int kSsdThreads = 4 * kQ; // a thread per (pair of steps, 8 channels) of a chunk: kQ / 16 waves
constexpr int kJ = kQ / kWave;      // steps per lane of the first wave in the running sum
static_assert(kQ % kWave == 0 && kQ >= 64 && kQ <= 128, "chunk of 64 or 128 steps");
#ifndef SSM_SSD_CARRY_U
#define SSM_SSD_CARRY_U 16  // chunks whose loads the chain keeps in flight
#endif
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

// Raw steps kJ l .. kJ l + kJ - 1 of lane l of the first wave (delta + bias; 0
// past the end of the sequence), read early so their latency overlaps the other
// loads of the chunk.
struct StepRaw {
  float v[kJ];
};
__device__ __forceinline__ StepRaw step_input(const bf16_bits* __restrict__ delta, const float* __restrict__ bias,
                                              int64_t row0, int H, int h, int n_steps) {
  StepRaw r;
  const float bh = (threadIdx.x < kWave && bias) ? bias[h] : 0.f;
#pragma unroll
  for (int j = 0; j < kJ; j++) {
    const int s = kJ * int(threadIdx.x) + j;
    r.v[j] = (threadIdx.x < kWave && s < n_steps) ? from_bf16(delta[(row0 + s) * H + h]) + bh : 0.f;
  }
  return r;
}

// Steps and their running sums inside the chunk, by the first wave: d[s] (0 past
// the end) and cum[s] = A_h * (d_0 + ... + d_s), written to LDS.  Lane l sums its
// own kJ steps, then the lanes' totals are scanned across the wave.  With w_s,
// also w[s] = exp(cum[e] - cum[s]) d[s], e the last step of the 16-step block of s.
template <bool SOFTPLUS>
__device__ __forceinline__ void chunk_steps(const StepRaw& raw, float Ah, int n_steps, float* d_s, float* cum_s,
                                            float* w_s = nullptr) {
  if (threadIdx.x < kWave) {
    const int l = threadIdx.x;
    float d[kJ], c[kJ], run = 0.f;
#pragma unroll
    for (int j = 0; j < kJ; j++) {
      const int s = kJ * l + j;
      d[j] = s < n_steps ? (SOFTPLUS ? softplus(raw.v[j]) : raw.v[j]) : 0.f;
      run += d[j] * Ah;
      c[j] = run;
    }
    float tot = run;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const float o = __shfl_up(tot, off);
      if (l >= off) tot += o;
    }
    const float before = tot - run;  // the lanes below this one
    float cum[kJ];
#pragma unroll
    for (int j = 0; j < kJ; j++) {
      cum[j] = kJ == 1 ? tot : before + c[j];
      d_s[kJ * l + j] = d[j];
      cum_s[kJ * l + j] = cum[j];
    }
    if (w_s) {
      constexpr int kLanesPerBlock = 16 / kJ;
      const float cum_e = __shfl(cum[kJ - 1], (l & ~(kLanesPerBlock - 1)) | (kLanesPerBlock - 1));
#pragma unroll
      for (int j = 0; j < kJ; j++) w_s[kJ * l + j] = exp2_fast((cum_e - cum[j]) * kLog2e) * d[j];
    }
  }
}

__device__ __forceinline__ uint4 ld16(const bf16_bits* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return uint32_t(to_bf16(lo)) | (uint32_t(to_bf16(hi)) << 16);
}
// the 8 bf16 of v, each times w, rounded back to bf16
__device__ __forceinline__ uint4 scale8(uint4 v, float w) {
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; j++)
    o[j] = pack2(__uint_as_float(u[j] << 16) * w, __uint_as_float(u[j] & 0xffff0000u) * w);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Rows s and s + 1 (s even) of columns c8 .. c8 + 7 (c8 a multiple of 8), given
// as two 16-byte vectors, stored transposed into T (row stride ld): T[c8 + e][s]
// and T[c8 + e][s + 1] go out as one 32-bit word, in the swizzled column blocks
// of swz (the same for all 8 rows, which share r / 8).  The words are assembled
// with byte permutes (low halves of a and b; high halves of a and b).
__device__ __forceinline__ void store_pair_t(bf16_bits* T, int ld, int c8, int s, uint4 a, uint4 b) {
  const uint32_t ua[4] = {a.x, a.y, a.z, a.w}, ub[4] = {b.x, b.y, b.z, b.w};
  bf16_bits* col = T + swz(c8, s);
#pragma unroll
  for (int j = 0; j < 4; j++) {
    *reinterpret_cast<uint32_t*>(col + (c8 + 2 * j) * ld) = __builtin_amdgcn_perm(ub[j], ua[j], 0x05040100u);
    *reinterpret_cast<uint32_t*>(col + (c8 + 2 * j + 1) * ld) = __builtin_amdgcn_perm(ub[j], ua[j], 0x07060302u);
  }
}

// ---------------------------------------------------------------------------
// chunk state, transposed: S_c[p, n] = sum_s (w o X)[s, p] B[s, n]  (bf16 out)
// Every global read of the chunk is issued first (B and x as pairs of rows, so
// the transposed LDS tiles are written one 32-bit word per two steps); the
// result goes back through LDS and out in whole 16-byte row pieces.
// ---------------------------------------------------------------------------
template <int NK, bool SOFTPLUS>  // NK: the state size padded to a multiple of 32, in units of 32
__global__ __launch_bounds__(kSsdThreads) void ssd_state_kernel(
    const bf16_bits* __restrict__ x, const bf16_bits* __restrict__ delta, const float* __restrict__ A,
    const bf16_bits* __restrict__ B, const float* __restrict__ bias, bf16_bits* __restrict__ states,
    float* __restrict__ cum_last, int64_t L, int H, int N, int n_chunks) {
  constexpr int NP = NK * 32;
  constexpr int kBV = kQ / 2 * (NP / 8);  // (row pair, 16-byte column block) items of B
  constexpr int nBV = (kBV + kSsdThreads - 1) / kSsdThreads;
  constexpr int kTileB = NP * (kQ + kPad) + kP * (kQ + kPad);  // Bt then Xw, bf16 elements
  constexpr int kOutB = kP * (NP + kPad);                      // the result [p][n], over them afterwards
  static_assert(kOutB <= kTileB, "result tile fits over the operand tiles");
  __shared__ float d_s[kQ], cum_s[kQ];
  __shared__ __attribute__((aligned(16))) bf16_bits pool[kTileB];
  bf16_bits* Bt = pool;                         // B transposed: [n][s]
  bf16_bits* Xw = pool + NP * (kQ + kPad);      // (w o X) transposed: [p][s]
  bf16_bits* So = pool;                         // result [p][n]
  constexpr int ldt = kQ + kPad, ldo = NP + kPad;
  const int h = blockIdx.x % H;
  const int rest = blockIdx.x / H;
  const int c = rest % n_chunks;
  const int64_t bi = rest / n_chunks;
  const int64_t t0 = int64_t(c) * kQ;
  const int n_steps = int(std::min<int64_t>(kQ, L - t0));
  const int64_t row0 = bi * L + t0;
  const int64_t E = int64_t(H) * kP;
  const uint4 zero = make_uint4(0, 0, 0, 0);
  // this thread's x rows s0, s0 + 1 and channels p8 .. p8 + 7
  const int s0 = 2 * (threadIdx.x >> 3), p8 = (threadIdx.x & 7) * 8;
  const bf16_bits* xr = x + (row0 + s0) * E + int64_t(h) * kP + p8;
  const uint4 x0 = s0 < n_steps ? ld16(xr) : zero;
  const uint4 x1 = s0 + 1 < n_steps ? ld16(xr + E) : zero;
  uint4 b0[nBV], b1[nBV];
#pragma unroll
  for (int k = 0; k < nBV; k++) {
    const int v = threadIdx.x + k * kSsdThreads;
    const int sp = 2 * (v / (NP / 8)), n8 = (v % (NP / 8)) * 8;
    const bool ok = v < kBV && n8 < N;
    b0[k] = ok && sp < n_steps ? ld16(B + (row0 + sp) * N + n8) : zero;
    b1[k] = ok && sp + 1 < n_steps ? ld16(B + (row0 + sp + 1) * N + n8) : zero;
  }
  const StepRaw raw = step_input(delta, bias, row0, H, h, n_steps);
  chunk_steps<SOFTPLUS>(raw, A[h], n_steps, d_s, cum_s);
#pragma unroll
  for (int k = 0; k < nBV; k++) {
    const int v = threadIdx.x + k * kSsdThreads;
    if (v < kBV) store_pair_t(Bt, ldt, (v % (NP / 8)) * 8, 2 * (v / (NP / 8)), b0[k], b1[k]);
  }
  __syncthreads();
  const float last = cum_s[kQ - 1];
  const float w0 = exp2_fast((last - cum_s[s0]) * kLog2e) * d_s[s0];
  const float w1 = exp2_fast((last - cum_s[s0 + 1]) * kLog2e) * d_s[s0 + 1];
  store_pair_t(Xw, ldt, p8, s0, scale8(x0, w0), scale8(x1, w1));
  __syncthreads();
  // wave w: rows p in [16 pb, 16 pb + 16) with pb = w mod 4, and the 16-column
  // blocks of n congruent to w / 4 modulo the number of waves / 4
  constexpr int kWaves = kSsdThreads / kWave, kNBW = (NP / 16) * 4 / kWaves;  // column blocks per wave
  static_assert(kNBW * kWaves == (NP / 16) * 4, "the column blocks divide over the waves");
  const int wv = threadIdx.x / kWave, l = threadIdx.x % kWave;
  const int lr = l % 16, lk = 8 * (l / 16);
  const int pb = wv % 4, nb0 = wv / 4;
  bf16x8 xf[kQ / 32];
#pragma unroll
  for (int kk = 0; kk < kQ / 32; kk++) xf[kk] = lds8(&Xw[(pb * 16 + lr) * ldt + swz(pb * 16 + lr, kk * 32 + lk)]);
  f32x4 acc[kNBW];
#pragma unroll
  for (int i = 0; i < kNBW; i++) {
    const int nb = nb0 + i * (kWaves / 4);
    acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (nb * 16 < N) {
#pragma unroll
      for (int kk = 0; kk < kQ / 32; kk++)
        acc[i] = mfma(xf[kk], lds8(&Bt[(nb * 16 + lr) * ldt + swz(nb * 16 + lr, kk * 32 + lk)]), acc[i]);
    }
  }
  __syncthreads();  // every wave is done with Bt and Xw before the result goes over them
#pragma unroll
  for (int i = 0; i < kNBW; i++)
#pragma unroll
    for (int r = 0; r < 4; r++)
      So[(pb * 16 + 4 * (l / 16) + r) * ldo + (nb0 + i * (kWaves / 4)) * 16 + lr] = to_bf16(acc[i][r]);
  __syncthreads();
  bf16_bits* out = states + ((bi * n_chunks + c) * H + h) * int64_t(kP) * N;  // [p][n]
  for (int v = threadIdx.x; v < kP * (NP / 8); v += kSsdThreads) {
    const int p = v / (NP / 8), n8 = (v % (NP / 8)) * 8;
    if (n8 < N) *reinterpret_cast<uint4*>(out + int64_t(p) * N + n8) = *reinterpret_cast<const uint4*>(&So[p * ldo + n8]);
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
// Every global read of the chunk (x, z, C, B, the incoming state, the steps) is
// issued before anything else.  x, z and y are handled per thread as two rows
// of 8 channels (16-byte accesses); the products' results go through an fp32
// LDS tile laid over the C and B tiles, and D x and the gate are applied with
// the thread's own x and z.
// ---------------------------------------------------------------------------
template <int NK, bool SOFTPLUS, bool HAS_Z, bool HAS_D>
__global__ __launch_bounds__(kSsdThreads) __attribute__((amdgpu_waves_per_eu(6))) void ssd_scan_kernel(
    const bf16_bits* __restrict__ x, const bf16_bits* __restrict__ delta, const float* __restrict__ A,
    const bf16_bits* __restrict__ B, const bf16_bits* __restrict__ C, const float* __restrict__ D,
    const bf16_bits* __restrict__ z, const float* __restrict__ bias, const bf16_bits* __restrict__ states,
    bf16_bits* __restrict__ y, int64_t L, int H, int N, int n_chunks) {
  constexpr int NP = NK * 32;
  constexpr int ldr = NP + kPad;          // B and incoming-state tiles, bf16 elements per row
  constexpr int ldt = kQ + kPad;          // X transposed
  constexpr int ldy = kP + 4;             // fp32 result tile
  constexpr int kBV = kQ * (NP / 8);      // 16-byte pieces of the B tile
  constexpr int kSV = kP * (NP / 8);      // 16-byte pieces of the incoming state
  constexpr int nBV = (kBV + kSsdThreads - 1) / kSsdThreads;
  constexpr int nSV = (kSV + kSsdThreads - 1) / kSsdThreads;
  constexpr int kBbytes = kQ * ldr * 2, kXbytes = kP * ldt * 2, kSbytes = kP * ldr * 2;
  constexpr int kTiles = kBbytes + kXbytes + kSbytes, kYbytes = kQ * ldy * 4;
  __shared__ float d_s[kQ], cum_s[kQ], w_s[kQ];
  // B rows [s][n], X transposed [p][s] and the incoming state [p][n]; once the
  // products are done, the fp32 results [t][p] over all three
  __shared__ __attribute__((aligned(16))) char pool[kTiles > kYbytes ? kTiles : kYbytes];
  bf16_bits* Bs = reinterpret_cast<bf16_bits*>(pool);
  bf16_bits* Xt = reinterpret_cast<bf16_bits*>(pool + kBbytes);
  bf16_bits* Ss = reinterpret_cast<bf16_bits*>(pool + kBbytes + kXbytes);
  float* Ys = reinterpret_cast<float*>(pool);
  const int h = blockIdx.x % H;
  const int rest = blockIdx.x / H;
  const int c = rest % n_chunks;
  const int64_t bi = rest / n_chunks;
  const int64_t t0 = int64_t(c) * kQ;
  const int n_steps = int(std::min<int64_t>(kQ, L - t0));
  const int64_t row0 = bi * L + t0;
  const int64_t E = int64_t(H) * kP;
  const uint4 zero = make_uint4(0, 0, 0, 0);

  // ---- global reads ----
  const int s0 = 2 * (threadIdx.x >> 3), p8 = (threadIdx.x & 7) * 8;  // this thread's rows and channels
  const bool ok0 = s0 < n_steps, ok1 = s0 + 1 < n_steps;
  const int64_t xo = (row0 + s0) * E + int64_t(h) * kP + p8;
  const uint4 x0 = ok0 ? ld16(x + xo) : zero;
  const uint4 x1 = ok1 ? ld16(x + xo + E) : zero;
  uint4 bv[nBV];
#pragma unroll
  for (int k = 0; k < nBV; k++) {
    const int v = threadIdx.x + k * kSsdThreads;
    const int r = v / (NP / 8), n8 = (v % (NP / 8)) * 8;
    bv[k] = v < kBV && r < n_steps && n8 < N ? ld16(B + (row0 + r) * N + n8) : zero;
  }
  const int wv = threadIdx.x / kWave, l = threadIdx.x % kWave;
  const int lr = l % 16, lg = l / 16, lk = 8 * lg, lq = 4 * lg;
  const int tb = wv;                 // this wave's step block
  const int t_own = tb * 16 + lr;    // the step this lane carries through the mixing product
  bf16x8 cf[NK];  // C row of step t_own, n = 32 kk + lk .. + 7: the operand [k = n][column t], straight from memory
#pragma unroll
  for (int kk = 0; kk < NK; kk++) {
    const uint4 v = t_own < n_steps && kk * 32 + lk < N ? ld16(C + (row0 + t_own) * N + kk * 32 + lk) : zero;
    cf[kk] = __builtin_bit_cast(bf16x8, v);
  }
  const bf16_bits* Sin = states + ((bi * n_chunks + c) * H + h) * int64_t(kP) * N;
  uint4 sv[nSV];
#pragma unroll
  for (int k = 0; k < nSV; k++) {
    const int v = threadIdx.x + k * kSsdThreads;
    const int p = v / (NP / 8), n8 = (v % (NP / 8)) * 8;
    sv[k] = v < kSV && n8 < N ? ld16(Sin + int64_t(p) * N + n8) : zero;
  }
  const StepRaw raw = step_input(delta, bias, row0, H, h, n_steps);

  // ---- LDS tiles ----
  chunk_steps<SOFTPLUS>(raw, A[h], n_steps, d_s, cum_s, SOFTPLUS ? w_s : nullptr);
#pragma unroll
  for (int k = 0; k < nBV; k++) {
    const int v = threadIdx.x + k * kSsdThreads;
    if (v < kBV) *reinterpret_cast<uint4*>(Bs + (v / (NP / 8)) * ldr + (v % (NP / 8)) * 8) = bv[k];
  }
#pragma unroll
  for (int k = 0; k < nSV; k++) {
    const int v = threadIdx.x + k * kSsdThreads;
    if (v < kSV) *reinterpret_cast<uint4*>(Ss + (v / (NP / 8)) * ldr + (v % (NP / 8)) * 8) = sv[k];
  }
  store_pair_t(Xt, ldt, p8, s0, x0, x1);
  __syncthreads();

  const float cum_t = cum_s[t_own];

  // Mixing matrix, transposed tiles (rows s, column t): lane (g, t_own) computes
  // M[t_own][16 sb + 4 g + r] and stores it straight into the A operand of the
  // in-chunk product: K block kk covers s in [32 kk, 32 kk + 32) in the order
  // (4 g + r, 16 + 4 g + r), r = 0..3.  Blocks above the diagonal are zero.
  // With softplus steps (d >= 0, so cum moves one way along the chunk), a block
  // below the diagonal takes exp(cum_t - cum_s) as exp(cum_t - cum_e) w_s / d_s,
  // e the block's last step: both factors lie between 1 and the product, and
  // one exponential per lane serves the block's four values.
  bf16x8 mf[kQ / 32];
#pragma unroll
  for (int kk = 0; kk < kQ / 32; kk++) {
#pragma unroll
    for (int half = 0; half < 2; half++) {
      const int sb = 2 * kk + half;
      float mv[4] = {0.f, 0.f, 0.f, 0.f};
      if (sb <= tb) {
        f32x4 g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k2 = 0; k2 < NK; k2++) g = mfma(lds8(&Bs[(sb * 16 + lr) * ldr + k2 * 32 + lk]), cf[k2], g);
        if (SOFTPLUS && sb < tb) {
          const float rf = exp2_fast((cum_t - cum_s[sb * 16 + 15]) * kLog2e);
#pragma unroll
          for (int r = 0; r < 4; r++) mv[r] = g[r] * rf * w_s[sb * 16 + lq + r];
        } else {
#pragma unroll
          for (int r = 0; r < 4; r++) {
            const int s = sb * 16 + lq + r;
            mv[r] = (s <= t_own) ? g[r] * exp2_fast((cum_t - cum_s[s]) * kLog2e) * d_s[s] : 0.f;
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 4; r++) mf[kk][4 * half + r] = static_cast<__bf16>(mv[r]);
    }
  }
  // the gate, needed only at the end: read now, so its latency overlaps the products
  uint4 z0 = zero, z1 = zero;
  if (HAS_Z) {
    if (ok0) z0 = ld16(z + xo);
    if (ok1) z1 = ld16(z + xo + E);
  }
  float row_scale[4];  // exp(cum_t) of this lane's output rows
#pragma unroll
  for (int r = 0; r < 4; r++) row_scale[r] = exp2_fast(cum_s[tb * 16 + lq + r] * kLog2e);
  f32x4 acc[kP / 16];
#pragma unroll
  for (int pb = 0; pb < kP / 16; pb++) {
    const int p = pb * 16 + lr;
    acc[pb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // incoming-state part: [t][n] x [n][p]; rows scaled by exp(cum_t)
#pragma unroll
    for (int kk = 0; kk < NK; kk++)  // the C fragment serves as the A operand [row t][k = n] here
      acc[pb] = mfma(cf[kk], lds8(&Ss[p * ldr + kk * 32 + lk]), acc[pb]);
#pragma unroll
    for (int r = 0; r < 4; r++) acc[pb][r] *= row_scale[r];
    // in-chunk part: M [t][s] x X [s][p], s in the permuted order
#pragma unroll
    for (int kk = 0; kk < kQ / 32; kk++) {
      if (2 * kk > tb) break;  // M is zero there
      const uint2 lo = *reinterpret_cast<const uint2*>(&Xt[p * ldt + swz(p, kk * 32 + lq)]);
      const uint2 hi = *reinterpret_cast<const uint2*>(&Xt[p * ldt + swz(p, kk * 32 + 16 + lq)]);
      acc[pb] = mfma(mf[kk], __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y)), acc[pb]);
    }
  }
  __syncthreads();  // every wave is done with the operand tiles before the results go over them
  // Volatile: hipcc (ROCm 7.2) pairs two of these 16 stores into one ds_write2_b32 with
  // the first offset divided by 4 twice (816 bytes encoded as 51 dwords), so rows
  // t = 3 mod 4 of the first 16 channels were never written.  Single stores avoid it.
  volatile float* Yv = Ys;
#pragma unroll
  for (int pb = 0; pb < kP / 16; pb++)
#pragma unroll
    for (int r = 0; r < 4; r++) Yv[(tb * 16 + lq + r) * ldy + pb * 16 + lr] = acc[pb][r];
  __syncthreads();

  // ---- D x, gate, bf16 rows out ----
  const float Dh = HAS_D ? D[h] : 0.f;
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int s = s0 + j;
    if (j ? ok1 : ok0) {
      const float4 a = *reinterpret_cast<const float4*>(&Ys[s * ldy + p8]);
      const float4 b = *reinterpret_cast<const float4*>(&Ys[s * ldy + p8 + 4]);
      float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      const uint4 xv = j ? x1 : x0, zv = j ? z1 : z0;
      const uint32_t xu[4] = {xv.x, xv.y, xv.z, xv.w}, zu[4] = {zv.x, zv.y, zv.z, zv.w};
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        float lo = v[2 * q], hi = v[2 * q + 1];
        if (HAS_D) {
          lo = fmaf(Dh, __uint_as_float(xu[q] << 16), lo);
          hi = fmaf(Dh, __uint_as_float(xu[q] & 0xffff0000u), hi);
        }
        if (HAS_Z) {
          lo *= silu(__uint_as_float(zu[q] << 16));
          hi *= silu(__uint_as_float(zu[q] & 0xffff0000u));
        }
        o[q] = pack2(lo, hi);
      }
      *reinterpret_cast<uint4*>(y + xo + int64_t(j) * E) = make_uint4(o[0], o[1], o[2], o[3]);
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
  err = n_chunks > 33 ? launch_kind(kKindSsdCarry, ssd_carry_kernel<SSM_SSD_CARRY_U>, (lanes + 255) / 256, 256, a.stream, states,
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
