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
// states laid out [p][n]).  The chunks are grouped in segments of kSeg:
//   ssd_state_kernel  per (batch, segment, head): walks the segment's chunks, (w o X)^T B
//                     per chunk chained in fp32 registers -> each chunk's incoming state
//                     from inside the segment (bf16) and the segment's own state (fp32)
//   chain_kernel      per (batch, head, p, n): chain over segments (fp32, ssm_chain.h) ->
//                     state entering each segment, and the last state
//   ssd_scan_kernel   per (batch, chunk, head): S_in = inside part + decayed segment state,
//                     then Y as above, + D x, gate, store
// MFMA: v_mfma_f32_16x16x32_bf16.  Lane l of a wave holds A-operand row l % 16,
// k = 8 (l / 16) .. +7; B-operand column l % 16, same k; result rows
// 4 (l / 16) .. +3 of column l % 16.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "ssm_chain.h"
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
constexpr int kSeg = 8;             // chunks per segment of the chunk-state walk

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

// Four consecutive rows of one column of a row-major bf16 tile, by the
// transposing LDS read of gfx950 (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane m names 8 bytes and lane i receives element i % 4 of the bytes
// named by lanes i / 4 + 4 j, j = 0..3 (measured on the device).  With lane m of
// the group pointing at T[r0 + m / 4][c0 + 4 (m % 4)], lane i receives
// T[r0 + j][c0 + i], j = 0..3: half of an MFMA operand fragment (column c0 + i,
// four consecutive k) of a tile stored [k][column].  r0 may differ between the
// four lane groups.  Rows of 144 bytes (or any stride that puts the 16 rows read
// at once on distinct multiples of 4 banks) keep the read at two passes.
typedef short v4i16 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_col4(const bf16_bits* T, int ld, int r0, int c0) {
  const int m = threadIdx.x % 16;
  const bf16_bits* p = T + (r0 + m / 4) * ld + c0 + 4 * (m % 4);
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p);
  return __builtin_bit_cast(uint2, v);
}
// an MFMA operand fragment of a [k][column] tile: column c0 + lane % 16, k = r0 .. r0 + 3 and r1 .. r1 + 3
__device__ __forceinline__ bf16x8 lds_frag(const bf16_bits* T, int ld, int r0, int r1, int c0) {
  const uint2 a = lds_col4(T, ld, r0, c0), b = lds_col4(T, ld, r1, c0);
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}

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

// Head of a workgroup: workgroups are dealt to the 8 XCDs in turn, so with H a
// multiple of 8 the XCD k = id mod 8 takes heads k H/8 .. (k+1) H/8 - 1: each XCD
// streams contiguous runs of every row of x, z and y, and a head always runs on
// the same XCD (its segment state stays in one L2).  Measured at ssd_long (H = 80):
// 0.98 ms per call against 1.02 with head = id mod H.
__device__ __forceinline__ int head_of(int id, int H) {
  return H % 8 == 0 ? (id % 8) * (H / 8) + (id / 8) % (H / 8) : id % H;
}

__device__ __forceinline__ uint4 ld16(const bf16_bits* p) { return *reinterpret_cast<const uint4*>(p); }
// 16 bytes at byte offset off of a buffer, or zeros when !ok (the offset is then
// pushed past the descriptor's range, which the hardware answers with zeros)
__device__ __forceinline__ uint4 ld16_or_zero(__amdgpu_buffer_rsrc_t r, bool ok, int off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, ok ? off : 0x7fffffff, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
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

// ---------------------------------------------------------------------------
// chunk states along a segment of kSeg chunks, per (batch, segment, head).
// Chunk c's own state, transposed, S_c[p, n] = sum_s (w o X)[s, p] B[s, n], comes
// from the MFMA units in fp32 and is chained in registers along the segment:
//   R_c = state entering chunk c from the segment's earlier chunks alone
//       = exp(cum_last of chunk c-1) R_{c-1} + S_{c-1},   R = 0 at the segment start.
// Written per chunk: R_c in bf16 [p][n] (not for the segment's first chunk, where
// it is zero) and phi_c = A_h * (steps of the segment before chunk c); per
// segment: R after its last chunk in fp32 [p][n] and the segment's A_h * (sum of
// its steps).  B and the weighted X are staged row-major ([s][n], [s][p], 16-byte
// row writes) and the MFMA operands are read down their columns with the
// transposing LDS read.  Capped at 80 VGPRs so that three 8-wave workgroups share a CU: their
// interleaving hides the reads better than a prefetch of the next chunk, whose
// registers would leave room for two (measured 302 against 333 us at ssd_long).
// Above 64 states the tiles take more than a third of the LDS and two workgroups
// share a CU.
// ---------------------------------------------------------------------------
template <int NK, bool SOFTPLUS>  // NK: the state size padded to a multiple of 32, in units of 32
__global__ __launch_bounds__(kSsdThreads) __attribute__((amdgpu_waves_per_eu(NK <= 2 ? 6 : 4))) void ssd_state_kernel(
    const bf16_bits* __restrict__ x, const bf16_bits* __restrict__ delta, const float* __restrict__ A,
    const bf16_bits* __restrict__ B, const float* __restrict__ bias, bf16_bits* __restrict__ rin,
    float* __restrict__ phi, float* __restrict__ seg_state, float* __restrict__ seg_decay, int64_t L, int H, int N,
    int n_chunks, int n_segs) {
  constexpr int NP = NK * 32;
  constexpr int kBV = kQ / 2 * (NP / 8);  // (row pair, 16-byte column block) items of B
  constexpr int nBV = (kBV + kSsdThreads - 1) / kSsdThreads;
  constexpr int ldb = NP + kPad, ldx = kP + kPad, ldo = NP + kPad;
  constexpr int kWaves = kSsdThreads / kWave, kNBW = (NP / 16) * 4 / kWaves;  // 16-column blocks per wave
  static_assert(kNBW * kWaves == (NP / 16) * 4, "the column blocks divide over the waves");
  __shared__ float d_s[kQ], cum_s[kQ];
  __shared__ __attribute__((aligned(16))) bf16_bits Bs[kQ * ldb];   // B rows [s][n]
  __shared__ __attribute__((aligned(16))) bf16_bits Xw[kQ * ldx];   // (w o X) rows [s][p]
  __shared__ __attribute__((aligned(16))) bf16_bits So[kP * ldo];   // R_c in bf16 [p][n], on its way out
  const int h = head_of(blockIdx.x, H);
  const int rest = blockIdx.x / H;
  const int g = rest % n_segs;
  const int64_t bi = rest / n_segs;
  const int c_begin = g * kSeg, c_end = std::min(c_begin + kSeg, n_chunks);
  const int64_t E = int64_t(H) * kP;
  const float Ah = A[h];
  // this thread's x rows s0, s0 + 1 and channels p8 .. p8 + 7
  const int s0 = 2 * (threadIdx.x >> 3), p8 = (threadIdx.x & 7) * 8;
  // wave w: rows p in [16 pb, 16 pb + 16) with pb = w mod 4, and the 16-column
  // blocks of n congruent to w / 4 modulo the number of waves / 4
  const int wv = threadIdx.x / kWave, l = threadIdx.x % kWave;
  const int lr = l % 16, lk = 8 * (l / 16);
  const int pb = wv % 4, nb0 = wv / 4;

  struct Reads {
    uint4 x0, x1, b0[nBV], b1[nBV];
    StepRaw raw;
  };
  // the chunk's reads through buffer descriptors based at its first row, so a
  // guarded load needs neither a branch nor a select of addresses
  auto read_chunk = [&](int c) {
    Reads r;
    const int64_t t0 = int64_t(c) * kQ;
    const int n_steps = int(std::min<int64_t>(kQ, L - t0));
    const int64_t row0 = bi * L + t0;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + row0 * E + int64_t(h) * kP);
    const int xoff = (s0 * int(E) + p8) * 2;  // kQ rows of E bf16 stay far below 2 GiB
    r.x0 = ld16_or_zero(rx, s0 < n_steps, xoff);
    r.x1 = ld16_or_zero(rx, s0 + 1 < n_steps, xoff + int(E) * 2);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + row0 * N);
#pragma unroll
    for (int k = 0; k < nBV; k++) {
      const int v = threadIdx.x + k * kSsdThreads;
      const int sp = 2 * (v / (NP / 8)), n8 = (v % (NP / 8)) * 8;
      const bool ok = v < kBV && n8 < N;
      r.b0[k] = ld16_or_zero(rb, ok && sp < n_steps, (sp * N + n8) * 2);
      r.b1[k] = ld16_or_zero(rb, ok && sp + 1 < n_steps, ((sp + 1) * N + n8) * 2);
    }
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(delta + row0 * H + h);
    const float bh = bias ? bias[h] : 0.f;
#pragma unroll
    for (int j = 0; j < kJ; j++) {
      const int st = kJ * int(threadIdx.x) + j;
      const bool ok = threadIdx.x < kWave && st < n_steps;
      const float dv = __uint_as_float(
          uint32_t(__builtin_amdgcn_raw_buffer_load_b16(rd, ok ? st * H * 2 : 0x7fffffff, 0, 0)) << 16);
      r.raw.v[j] = ok ? dv + bh : 0.f;
    }
    return r;
  };

  f32x4 R[kNBW];
#pragma unroll
  for (int i = 0; i < kNBW; i++) R[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float lphi = 0.f;  // A_h * (steps of the segment so far); uniform
  for (int c = c_begin; c < c_end; c++) {
    const Reads cur = read_chunk(c);
    const int n_steps = int(std::min<int64_t>(kQ, L - int64_t(c) * kQ));
    __syncthreads();  // the previous chunk is done with d_s, cum_s and the tiles
    chunk_steps<SOFTPLUS>(cur.raw, Ah, n_steps, d_s, cum_s);
#pragma unroll
    for (int k = 0; k < nBV; k++) {
      const int v = threadIdx.x + k * kSsdThreads;
      if (v < kBV) {
        bf16_bits* row = Bs + 2 * (v / (NP / 8)) * ldb + (v % (NP / 8)) * 8;
        *reinterpret_cast<uint4*>(row) = cur.b0[k];
        *reinterpret_cast<uint4*>(row + ldb) = cur.b1[k];
      }
    }
    if (c > c_begin) {
#pragma unroll
      for (int i = 0; i < kNBW; i++)
#pragma unroll
        for (int r = 0; r < 4; r++)
          So[(pb * 16 + 4 * (l / 16) + r) * ldo + (nb0 + i * (kWaves / 4)) * 16 + lr] = to_bf16(R[i][r]);
    }
    __syncthreads();
    const float last = cum_s[kQ - 1];
    const float w0 = exp2_fast((last - cum_s[s0]) * kLog2e) * d_s[s0];
    const float w1 = exp2_fast((last - cum_s[s0 + 1]) * kLog2e) * d_s[s0 + 1];
    *reinterpret_cast<uint4*>(Xw + s0 * ldx + p8) = scale8(cur.x0, w0);
    *reinterpret_cast<uint4*>(Xw + (s0 + 1) * ldx + p8) = scale8(cur.x1, w1);
    if (c > c_begin) {  // R_c out in 16-byte row pieces
      bf16_bits* out = rin + ((bi * n_chunks + c) * H + h) * int64_t(kP) * N;
      for (int v = threadIdx.x; v < kP * (NP / 8); v += kSsdThreads) {
        const int p = v / (NP / 8), n8 = (v % (NP / 8)) * 8;
        if (n8 < N)
          *reinterpret_cast<uint4*>(out + int64_t(p) * N + n8) = *reinterpret_cast<const uint4*>(&So[p * ldo + n8]);
      }
    }
    if (threadIdx.x == 0) phi[(bi * n_chunks + c) * H + h] = lphi;
    __syncthreads();
    bf16x8 xf[kQ / 32];
#pragma unroll
    for (int kk = 0; kk < kQ / 32; kk++)  // A operand: rows p, k = s (read down the columns of [s][p])
      xf[kk] = lds_frag(Xw, ldx, kk * 32 + lk, kk * 32 + lk + 4, pb * 16);
    const float decay = exp2_fast(last * kLog2e);
#pragma unroll
    for (int i = 0; i < kNBW; i++) {
      const int nb = nb0 + i * (kWaves / 4);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (nb * 16 < N) {
#pragma unroll
        for (int kk = 0; kk < kQ / 32; kk++)
          acc = mfma(xf[kk], lds_frag(Bs, ldb, kk * 32 + lk, kk * 32 + lk + 4, nb * 16), acc);
      }
#pragma unroll
      for (int r = 0; r < 4; r++) R[i][r] = fmaf(decay, R[i][r], acc[r]);
    }
    lphi += last;
  }
  // the segment's aggregate: R after its last chunk (fp32 [p][n]) and its log-decay
  float* so = seg_state + ((bi * n_segs + g) * H + h) * int64_t(kP) * N;
#pragma unroll
  for (int i = 0; i < kNBW; i++) {
    const int n = (nb0 + i * (kWaves / 4)) * 16 + lr;
    if (n < N) {
#pragma unroll
      for (int r = 0; r < 4; r++) so[int64_t(pb * 16 + 4 * (l / 16) + r) * N + n] = R[i][r];
    }
  }
  if (threadIdx.x == 0) seg_decay[(bi * n_segs + g) * H + h] = lphi;
}


// ---------------------------------------------------------------------------
// outputs of a chunk.  Wave w owns steps t in [16 w, 16 w + 16).  The mixing
// matrix is built transposed (rows s, columns t) so that each lane ends with
// its own step t in registers: those values are the A operand of the next
// product directly, with the contraction index s in the order the transposed
// tiles give it (s = 4 g + r and 16 + 4 g + r for lane group g); X, staged
// row-major, is read in the same order down its columns (transposing LDS read).
// Every global read of the chunk (x, z, C, B, the incoming state, the steps) is
// issued before anything else.  x, z and y are handled per thread as two rows
// of 8 channels (16-byte accesses); the products' results go through an fp32
// LDS tile laid over the C and B tiles, and D x and the gate are applied with
// the thread's own x and z.  Three workgroups share a CU up to 64 states (46 KB
// of LDS each), two above.
// ---------------------------------------------------------------------------
template <int NK, bool SOFTPLUS, bool HAS_Z, bool HAS_D>
__global__ __launch_bounds__(kSsdThreads) __attribute__((amdgpu_waves_per_eu(NK <= 2 ? 6 : 4))) void ssd_scan_kernel(
    const bf16_bits* __restrict__ x, const bf16_bits* __restrict__ delta, const float* __restrict__ A,
    const bf16_bits* __restrict__ B, const bf16_bits* __restrict__ C, const float* __restrict__ D,
    const bf16_bits* __restrict__ z, const float* __restrict__ bias, const bf16_bits* __restrict__ rin,
    const float* __restrict__ phi, const float* __restrict__ seg_state, bf16_bits* __restrict__ y, int64_t L, int H,
    int N, int n_chunks, int n_segs) {
  constexpr int NP = NK * 32;
  constexpr int ldr = NP + kPad;          // B and incoming-state tiles, bf16 elements per row
  constexpr int ldx = kP + kPad;          // X rows [s][p]
  constexpr int ldy = kP + 4;             // fp32 result tile
  constexpr int kBV = kQ * (NP / 8);      // 16-byte pieces of the B tile
  constexpr int kSV = kP * (NP / 8);      // 16-byte pieces of the incoming state
  constexpr int nBV = (kBV + kSsdThreads - 1) / kSsdThreads;
  constexpr int nSV = (kSV + kSsdThreads - 1) / kSsdThreads;
  constexpr int kBbytes = kQ * ldr * 2, kXbytes = kQ * ldx * 2, kSbytes = kP * ldr * 2;
  constexpr int kTiles = kBbytes + kXbytes + kSbytes, kYbytes = kQ * ldy * 4;
  __shared__ float d_s[kQ], cum_s[kQ], w_s[kQ];
  // B rows [s][n], X rows [s][p] and the incoming state [p][n]; once the
  // products are done, the fp32 results [t][p] over all three
  __shared__ __attribute__((aligned(16))) char pool[kTiles > kYbytes ? kTiles : kYbytes];
  bf16_bits* Bs = reinterpret_cast<bf16_bits*>(pool);
  bf16_bits* Xs = reinterpret_cast<bf16_bits*>(pool + kBbytes);
  bf16_bits* Ss = reinterpret_cast<bf16_bits*>(pool + kBbytes + kXbytes);
  float* Ys = reinterpret_cast<float*>(pool);
  const int h = head_of(blockIdx.x, H);
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
  // incoming state S_in = R_c + exp(phi_c) S_g: the segment-local part (bf16, zero at
  // the segment's first chunk) and the state entering the segment (fp32)
  const bool seg_first = c % kSeg == 0;
  const bf16_bits* Rin = rin + ((bi * n_chunks + c) * H + h) * int64_t(kP) * N;
  const float* Sg = seg_state + ((bi * n_segs + c / kSeg) * H + h) * int64_t(kP) * N;
  uint4 sv[nSV];
  float4 sg0[nSV], sg1[nSV];
#pragma unroll
  for (int k = 0; k < nSV; k++) {
    const int v = threadIdx.x + k * kSsdThreads;
    const int p = v / (NP / 8), n8 = (v % (NP / 8)) * 8;
    const bool ok = v < kSV && n8 < N;
    sv[k] = ok && !seg_first ? ld16(Rin + int64_t(p) * N + n8) : zero;
    sg0[k] = ok ? *reinterpret_cast<const float4*>(Sg + int64_t(p) * N + n8) : make_float4(0.f, 0.f, 0.f, 0.f);
    sg1[k] = ok ? *reinterpret_cast<const float4*>(Sg + int64_t(p) * N + n8 + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const float ephi = exp2_fast(phi[(bi * n_chunks + c) * H + h] * kLog2e);
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
    if (v < kSV) {
      const uint32_t r[4] = {sv[k].x, sv[k].y, sv[k].z, sv[k].w};
      const float sg[8] = {sg0[k].x, sg0[k].y, sg0[k].z, sg0[k].w, sg1[k].x, sg1[k].y, sg1[k].z, sg1[k].w};
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; q++)
        o[q] = pack2(fmaf(ephi, sg[2 * q], __uint_as_float(r[q] << 16)),
                     fmaf(ephi, sg[2 * q + 1], __uint_as_float(r[q] & 0xffff0000u)));
      *reinterpret_cast<uint4*>(Ss + (v / (NP / 8)) * ldr + (v % (NP / 8)) * 8) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  *reinterpret_cast<uint4*>(Xs + s0 * ldx + p8) = x0;
  *reinterpret_cast<uint4*>(Xs + (s0 + 1) * ldx + p8) = x1;
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
      // B operand: column p, k = s in the permuted order, read down the columns of [s][p]
      acc[pb] = mfma(mf[kk], lds_frag(Xs, ldx, kk * 32 + lq, kk * 32 + 16 + lq, pb * 16), acc[pb]);
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

// Workspace of one call: the chunks' segment-local incoming states (bf16), the
// chunks' phi, the segments' states (fp32) and their log-decays.
struct SsdWork {
  bf16_bits* rin;
  float* phi;
  float* seg_state;
  float* seg_decay;
};

template <int NK, bool SOFTPLUS>
hipError_t run_ssd(const SsdArgs& a, int n_chunks, int n_segs, const SsdWork& w) {
  const int H = int(a.H), N = int(a.N);
  const bf16_bits* x = static_cast<const bf16_bits*>(a.x);
  const bf16_bits* dl = static_cast<const bf16_bits*>(a.delta);
  const bf16_bits* B = static_cast<const bf16_bits*>(a.B);
  const bf16_bits* C = static_cast<const bf16_bits*>(a.C);
  const bf16_bits* z = static_cast<const bf16_bits*>(a.z);
  hipError_t err = launch_kind(kKindSsdState, ssd_state_kernel<NK, SOFTPLUS>, a.b * n_segs * H, kSsdThreads, a.stream,
                               x, dl, a.A, B, a.bias, w.rin, w.phi, w.seg_state, w.seg_decay, a.L, H, N, n_chunks,
                               n_segs);
  if (err != hipSuccess) return err;
  // the state entering every segment (forward, exclusive) from the incoming state, the state
  // after the last one to last_state; per (batch, head, p, n), a segment's decay is exp(seg_decay)
  const int per_head = N * kP;
  const ChainArgs chain{w.seg_state, w.seg_decay, nullptr, a.h0, a.last_state, a.b, H, per_head, per_head, n_segs,
                        n_segs};
  err = launch_chain<false, true, false>(kKindSsdCarry, chain, a.stream);
  if (err != hipSuccess) return err;
  bf16_bits* y = static_cast<bf16_bits*>(a.y);
  const int64_t blocks = a.b * n_chunks * H;
#define SSM_SSD_SCAN(HZ, HD)                                                                                  \
  return launch_kind(kKindSsdScan, ssd_scan_kernel<NK, SOFTPLUS, HZ, HD>, blocks, kSsdThreads, a.stream, x, dl, \
                     a.A, B, C, a.D, z, a.bias, (const bf16_bits*)w.rin, (const float*)w.phi,               \
                     (const float*)w.seg_state, y, a.L, H, N, n_chunks, n_segs)
  if (a.z) {
    if (a.D) SSM_SSD_SCAN(true, true);
    SSM_SSD_SCAN(true, false);
  }
  if (a.D) SSM_SSD_SCAN(false, true);
  SSM_SSD_SCAN(false, false);
#undef SSM_SSD_SCAN
}

template <int NK>
hipError_t ssd_sp(const SsdArgs& a, int n_chunks, int n_segs, const SsdWork& w) {
  return a.softplus ? run_ssd<NK, true>(a, n_chunks, n_segs, w) : run_ssd<NK, false>(a, n_chunks, n_segs, w);
}

}  // namespace

int64_t ssd_chunk_steps() { return kQ; }
int64_t ssd_head_dim() { return kP; }
// The chunk-state kernel reads x through a buffer descriptor based at the chunk's first row,
// with 32-bit byte offsets up to (kQ + 1) rows of H * kP bf16 channels.
int64_t ssd_max_channels() { return (int64_t(INT32_MAX) / 2 - kP) / (kQ + 1); }

hipError_t launch_ssd(const SsdArgs& a) {
  if (a.b == 0 || a.H == 0) return hipSuccess;
  if (a.L == 0) {  // no step: the last state is the incoming one
    if (!a.last_state) return hipSuccess;
    const int64_t n = a.b * a.H * kP * a.N;
    return launch_kind(kKindSsdCarry, ssd_fill_kernel, (n + 255) / 256, 256, a.stream, a.last_state, a.h0, n);
  }
  const int n_chunks = int((a.L + kQ - 1) / kQ);
  const int n_segs = (n_chunks + kSeg - 1) / kSeg;
  auto up = [](size_t bytes) { return (bytes + 255) / 256 * 256; };
  const size_t per_state = size_t(a.N) * kP;
  const size_t rin_bytes = up(size_t(a.b) * n_chunks * a.H * per_state * sizeof(bf16_bits));
  const size_t phi_bytes = up(size_t(a.b) * n_chunks * a.H * sizeof(float));
  const size_t seg_bytes = up(size_t(a.b) * n_segs * a.H * per_state * sizeof(float));
  const size_t dec_bytes = up(size_t(a.b) * n_segs * a.H * sizeof(float));
  void* ws = nullptr;
  hipError_t err = hipMallocAsync(&ws, rin_bytes + phi_bytes + seg_bytes + dec_bytes, a.stream);
  if (err != hipSuccess) return err;
  char* p = static_cast<char*>(ws);
  const SsdWork w = {reinterpret_cast<bf16_bits*>(p), reinterpret_cast<float*>(p + rin_bytes),
                     reinterpret_cast<float*>(p + rin_bytes + phi_bytes),
                     reinterpret_cast<float*>(p + rin_bytes + phi_bytes + seg_bytes)};
  const int nk = int((a.N + 31) / 32);
  switch (nk) {
    case 1: err = ssd_sp<1>(a, n_chunks, n_segs, w); break;
    case 2: err = ssd_sp<2>(a, n_chunks, n_segs, w); break;
    case 3: err = ssd_sp<3>(a, n_chunks, n_segs, w); break;
    default: err = ssd_sp<4>(a, n_chunks, n_segs, w); break;
  }
  hipError_t ferr = hipFreeAsync(ws, a.stream);
  return err != hipSuccess ? err : ferr;
}

}  // namespace ssm
