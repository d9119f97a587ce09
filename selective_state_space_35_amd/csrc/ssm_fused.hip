// ssm_fused.hip -- the single-pass selective scan (forward) for gfx950: every
// input is read from HBM once, every retention exp2 is evaluated once, and
// only y and the last state (plus, on request, the saved states) are written.
//
// Pages that define the arithmetic (title, site):
//   [KK] "mamba, from scratch" (khushi keswani)
//   [AB] "Mamba: Linear-Time Sequence Modeling with Selective State Spaces" (abhik.ai)
//
// Per step t, channel e, state n (float32):
//   d   = softplus(delta + bias)            [KK] "from ssm to selective ssm"
//   h_n = exp(d*A_n) * h_n + (d*u) * B_n    [AB] "Original paper, equations and
//                                           runnable CPU code", row 2
//   y   = (sum_n C_n h_n + D*u) * silu(z)   same row 2; [AB] row 5
//
// Work layout
// -----------
// A workgroup owns cg consecutive channels of one batch row for the whole
// sequence.  The grid holds about one workgroup per CU, and the workgroups
// that land on one XCD (dispatch is round-robin over the 8 XCDs) own
// neighbouring channel ranges, so the rows they share stay in that XCD's L2.
//
// Compute waves.  LPC = NS / 4 lanes share a channel, each holding 4 of its
// states in VGPRs.  The sequence is walked in blocks of W chunks of kT = 8
// steps; lane (j, c, q) takes chunk j of every block for channel c, states
// 4q .. 4q+3.  Per block:
//   phase 1  every lane runs its chunk from a zero state and keeps each step's
//            retention a = exp2(d * A * log2 e) and write w = d * u * B in
//            registers; the chunk's affine map is (exp2(A * log2 e * sum d),
//            end state) ([KK] "the scan": (a2, b2) o (a1, b1) = (a2 a1,
//            a2 b1 + b2)).
//   combine  the lanes of chunk 0 chain the block's maps through LDS from the
//            state entering the block: every chunk gets its incoming state,
//            and the state leaving the block stays in their registers for the
//            next block ([AB] "Compose the updates instead of waiting for
//            every state").
//   phase 2  every lane reruns its chunk from its incoming state with the kept
//            a and w (no exponential, no memory read), reads out C . h and
//            sums it over the LPC lanes of the channel (DPP); lane q finishes
//            steps q, q + LPC, ..: + D*u, * silu(z), rounding, into an LDS tile.
//
// Producer waves (the last n_prod).  They move whole 4-byte words between HBM
// and LDS: the inputs of block k + 2 (loaded into registers one block before)
// go into a triple-buffered LDS tile while the compute waves work on block k,
// and the y tile of block k - 1 goes out.  Their loads never wait on the
// compute and the compute never waits on memory.
//
// Nothing is re-read, no exponential is recomputed and no workspace is
// needed.  Nothing here is a dense contraction, so no MFMA is used.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "ssm_device.h"
#include "ssm_internal.h"
#include "ssm_profile.h"

namespace ssm {
namespace {

constexpr int kT = 8;                   // steps per chunk: a lane keeps 2 * 4 * kT floats
constexpr int kMaxThreads = 64 * kFusedMaxWaves;
constexpr int kProd = 2;                // producer waves
constexpr int kPoolBytes = 150 * 1024;  // LDS pool carved by the plan

// The value of group lane r in every lane of the group of LPC lanes (DPP
// quad_perm); r is a constant once the calling loop is unrolled.
template <int LPC>
__device__ __forceinline__ float grp_bcast(float v, int r) {
  if constexpr (LPC == 1) {
    return v;
  } else if constexpr (LPC == 2) {  // pairs (0,1), (2,3): [r, r, r + 2, r + 2]
    const int b = __float_as_int(v);
    if (r == 0) return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0xA0, 0xF, 0xF, false));
    return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0xF5, 0xF, 0xF, false));
  } else {  // quads: [r, r, r, r]
    const int b = __float_as_int(v);
    switch (r) {
      case 0: return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x00, 0xF, 0xF, false));
      case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x55, 0xF, 0xF, false));
      case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0xAA, 0xF, 0xF, false));
      default: return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0xFF, 0xF, 0xF, false));
    }
  }
}

// Sum over the LPC lanes of a group, in every lane of the group.
template <int LPC>
__device__ __forceinline__ float grp_sum(float v) {
  if constexpr (LPC >= 2) v += quad_xor1(v);
  if constexpr (LPC >= 4) v += quad_xor2(v);
  return v;
}

typedef unsigned int v2u __attribute__((ext_vector_type(2)));

// Buffer resource over [base, base + bytes): accesses at or past the end read
// zero / are dropped, which clips the last block of a sequence.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_n(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : int(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

template <typename T, int LPC, bool SOFTPLUS, bool HAS_Z, bool SAVE>
__global__ __launch_bounds__(kMaxThreads) void scan_fused_kernel(
    const T* __restrict__ u, const T* __restrict__ delta, const float* __restrict__ A, const T* __restrict__ B,
    const T* __restrict__ C, const float* __restrict__ D, const T* __restrict__ z, const float* __restrict__ bias,
    T* __restrict__ y, float* __restrict__ last_state, const float* __restrict__ h0, float* __restrict__ saved,
    int64_t L, int64_t E, int N, const FusedPlan p) {
  constexpr int NSP = 4 * LPC;        // states per channel, padded to the lanes
  constexpr int EPL = kT / LPC;       // steps of a chunk a lane finishes
  constexpr int ES = int(sizeof(T));
  constexpr int NIN = HAS_Z ? 3 : 2;  // streamed per-step inputs: u, delta (, z)
  __shared__ __attribute__((aligned(16))) char pool[kPoolBytes];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;

  // workgroup -> (batch row, channel group); the groups on one XCD are neighbours
  const int wg = blockIdx.x;
  const int G = (p.n_wg % 8 == 0) ? (wg % 8) * (p.n_wg / 8) + wg / 8 : wg;
  const int64_t bi = G / p.groups_row;
  const int64_t e0 = int64_t(G % p.groups_row) * p.cg;
  const int cg = p.cg;
  const int ce = int(E - e0 < cg ? E - e0 : cg);  // channels of this group
  const int BT = p.BT;
  const int64_t row0 = bi * L;

  // padded B / C state slots stay zero in all three tiles
  if (NSP > N) {
    float* const bcz = reinterpret_cast<float*>(pool + p.o_bc[0]);
    const int nz = (p.o_bc[2] - p.o_bc[0]) / 4 + p.brows * 2 * NSP;
    for (int i = tid; i < nz; i += p.n_threads) bcz[i] = 0.f;
    __syncthreads();
  }

  if (wave >= p.n_cmp) {
    // =============================== producer waves ===============================
    // Every access moves 8 bytes.  Lane pl takes unit column d of rows r, r + R, ..;
    // lanes past the last whole row of a pass read out of range (zero) and write a junk slot.
    const int pl = (wave - p.n_cmp) * 64 + lane;
    const int xdu = cg * ES / 8, bdu = N * ES / 8;  // units per row
    const int xr = pl / xdu, xd = pl - (pl / xdu) * xdu;
    const int br = pl / bdu, bd = pl - (pl / bdu) * bdu;
    const bool xon = xr < p.xR, bon = br < p.bR;
    constexpr int kOob = 0x7ffffff0;  // past the end of every buffer range
    const int xg0 = xon ? int(int64_t(xr) * E * ES) + 8 * xd : kOob;
    const int xgs = xon ? int(int64_t(p.xR) * E * ES) : 0;
    const int xl0 = xon ? xr * cg * ES + 8 * xd : p.o_junk;
    const int xls = xon ? p.xR * cg * ES : 0;
    const int bg0 = bon ? br * N * ES + 8 * bd : kOob;
    const int bgs = bon ? p.bR * N * ES : 0;
    const int bl0 = bon ? (br * 2 * NSP + bd * (8 / ES)) * 4 : p.o_junk;
    const int bls = bon ? p.bR * 2 * NSP * 4 : 0;
    const int cw8 = ce * ES / 8;  // units of this group's channels in a row
    const bool yon = xon && xd < cw8;
    constexpr int kX = 6, kB = 3;  // most passes per block kept in registers
    uint2 px[NIN][kX], pb[2][kB];
    auto load = [&](int blk) {  // block blk's inputs into registers
      const int64_t t_blk = int64_t(blk) * BT;
      const int64_t xbytes = ((L - t_blk) * E - e0) * ES, bbytes = (L - t_blk) * N * ES;
#pragma unroll
      for (int a = 0; a < NIN; a++) {
        const T* const src = a == 0 ? u : a == 1 ? delta : z;
        const __amdgpu_buffer_rsrc_t r = rsrc_n(src + (row0 + t_blk) * E + e0, xbytes);
#pragma unroll
        for (int m = 0; m < kX; m++)
          if (m < p.xM) {
            const v2u v = __builtin_amdgcn_raw_buffer_load_b64(r, xg0 + m * xgs, 0, 0);
            px[a][m] = make_uint2(v[0], v[1]);
          }
      }
#pragma unroll
      for (int a = 0; a < 2; a++) {
        const __amdgpu_buffer_rsrc_t r = rsrc_n((a ? C : B) + (row0 + t_blk) * N, bbytes);
#pragma unroll
        for (int m = 0; m < kB; m++)
          if (m < p.bM) {
            const v2u v = __builtin_amdgcn_raw_buffer_load_b64(r, bg0 + m * bgs, 0, 0);
            pb[a][m] = make_uint2(v[0], v[1]);
          }
      }
    };
    auto put = [&](int buf) {  // registers into the block's LDS tiles
#pragma unroll
      for (int a = 0; a < NIN; a++) {
        char* const tile = pool + (xon ? p.o_x[buf] + a * p.xrows * cg * ES : 0) + xl0;
#pragma unroll
        for (int m = 0; m < kX; m++)
          if (m < p.xM) *reinterpret_cast<uint2*>(tile + m * xls) = px[a][m];
      }
#pragma unroll
      for (int a = 0; a < 2; a++) {
        char* const tile = pool + (bon ? p.o_bc[buf] + a * NSP * 4 : 0) + bl0;
#pragma unroll
        for (int m = 0; m < kB; m++)
          if (m < p.bM) {
            const uint2 v = pb[a][m];
            if (ES == 2) {
              *reinterpret_cast<float4*>(tile + m * bls) =
                  make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                              __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
            } else {
              *reinterpret_cast<uint2*>(tile + m * bls) = v;
            }
          }
      }
    };
    auto store_y = [&](int buf, int blk) {  // the y tile of block blk to HBM
      const int64_t t_blk = int64_t(blk) * BT;
      const __amdgpu_buffer_rsrc_t r = rsrc_n(y + (row0 + t_blk) * E + e0, ((L - t_blk) * E - e0) * ES);
      const char* const tile = pool + p.o_y[buf] + (yon ? xl0 : 0);
      for (int m = 0; m < p.xM; m++) {
        if (yon && xr + m * p.xR < BT) {
          const uint2 v = *reinterpret_cast<const uint2*>(tile + m * xls);
          const v2u vv = {v.x, v.y};
          __builtin_amdgcn_raw_buffer_store_b64(vv, r, xg0 + m * xgs, 0, 0);
        }
      }
    };

    load(0);
    put(0);
    if (p.nblk > 1) {
      load(1);
      put(1);
    }
    if (p.nblk > 2) load(2);
    __syncthreads();
    for (int k = 0; k < p.nblk; k++) {
      __syncthreads();  // A: the compute waves hold their chunk maps
      __syncthreads();  // B: every chunk has its incoming state
      if (k + 2 < p.nblk) put((k + 2) % 3);  // its tiles were last read in block k - 1
      if (k + 3 < p.nblk) load(k + 3);
      if (k >= 1) store_y((k - 1) & 1, k - 1);
    }
    __syncthreads();
    store_y((p.nblk - 1) & 1, p.nblk - 1);
    return;
  }

  // ================================ compute waves ================================
  const int lpg = LPC * cg;
  const bool lane_ok = tid < p.lanes;
  const int jr = tid / lpg;
  const int j = jr < p.W ? jr : p.W - 1;  // idle lanes shadow the last chunk and write nothing
  const int rq = tid - jr * lpg;
  const int c = rq / LPC, q = rq - c * LPC;
  const bool ch_ok = lane_ok && c < ce;
  const int64_t e = e0 + (c < ce ? c : ce - 1);
  float A2[4];
#pragma unroll
  for (int k = 0; k < 4; k++) A2[k] = (4 * q + k < N) ? A[e * N + 4 * q + k] * kLog2e : 0.f;
  const float bv = bias ? bias[e] : 0.f;
  const float Dv = D ? D[e] : 0.f;
  float4* const aggP = reinterpret_cast<float4*>(pool + p.o_agg);     // [lanes]: decay of each chunk
  float4* const aggH = aggP + p.lanes;                                 // [lanes]: its state from zero
  float4* const hin = reinterpret_cast<float4*>(pool + p.o_hin);  // [lanes]: state entering each chunk

  // the state entering the current block, held by the lanes of chunk 0
  const bool chain_lane = tid < lpg;
  float hb[4];
#pragma unroll
  for (int k = 0; k < 4; k++)
    hb[k] = (chain_lane && h0 && 4 * q + k < N) ? h0[(bi * E + e) * N + 4 * q + k] : 0.f;
  const int64_t n_saved = (L + kSaveEvery - 1) / kSaveEvery - 1;
  const int tl0 = j * kT;  // the chunk's first row in a block's tiles
  __syncthreads();

  for (int k = 0; k < p.nblk; k++) {
    const int buf = k % 3;
    const int64_t t_blk = int64_t(k) * BT;
    const T* const xt = reinterpret_cast<const T*>(pool + p.o_x[buf]);
    const float* const bct = reinterpret_cast<const float*>(pool + p.o_bc[buf]);

    // ---- phase 1: the chunk from a zero state, retentions and writes kept -------------------
    // step d and d * u: lane q of a channel works them out for steps q, q + LPC, .. and the
    // channel's lanes read them by DPP broadcast (with one lane per channel, inline)
    auto step_of = [&](int s, float& d, float& dxo) {
      const int tl = tl0 + s;
      const float raw = load_elem(xt + (p.xrows + tl) * cg + c) + bv;
      d = SOFTPLUS ? softplus(raw) : raw;
      d = (t_blk + tl < L) ? d : 0.f;  // steps past the end are the identity map
      dxo = d * load_elem(xt + tl * cg + c);
    };
    float dd[EPL], dx[EPL];
    float ssum = 0.f;
    if constexpr (LPC > 1) {
#pragma unroll
      for (int i = 0; i < EPL; i++) {
        step_of(i * LPC + q, dd[i], dx[i]);
        ssum += dd[i];
      }
    }
    float a[kT][4], w[kT][4], hl[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kT; s++) {
      float ds, dxs;
      if constexpr (LPC > 1) {
        ds = grp_bcast<LPC>(dd[s / LPC], s % LPC);
        dxs = grp_bcast<LPC>(dx[s / LPC], s % LPC);
      } else {
        step_of(s, ds, dxs);
        ssum += ds;
      }
      const float4 b4 = *reinterpret_cast<const float4*>(bct + (tl0 + s) * 2 * NSP + 4 * q);
      const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
      for (int k2 = 0; k2 < 4; k2++) {
        a[s][k2] = exp2_fast(ds * A2[k2]);
        w[s][k2] = dxs * bb[k2];
        hl[k2] = fmaf(a[s][k2], hl[k2], w[s][k2]);
      }
    }
    ssum = grp_sum<LPC>(ssum);
    if (lane_ok) {
      aggP[tid] = make_float4(exp2_fast(A2[0] * ssum), exp2_fast(A2[1] * ssum), exp2_fast(A2[2] * ssum),
                              exp2_fast(A2[3] * ssum));
      aggH[tid] = make_float4(hl[0], hl[1], hl[2], hl[3]);
    }
    __syncthreads();  // A

    // ---- combine: the lanes of chunk 0 chain the block's maps ------------------------------
    if (chain_lane) {
      auto link = [&](int jj, const float4& P, const float4& H) {
        hin[jj * lpg + tid] = make_float4(hb[0], hb[1], hb[2], hb[3]);
        if (SAVE) {  // the state entering step 64 m, m >= 1 (the backward's chunk boundaries)
          const int64_t ts = t_blk + int64_t(jj) * kT;
          if (ts > 0 && ts < L && ts % kSaveEvery == 0 && c < ce) {
            float* const dst = saved + ((bi * n_saved + ts / kSaveEvery - 1) * E + e) * N + 4 * q;
#pragma unroll
            for (int k2 = 0; k2 < 4; k2++)
              if (4 * q + k2 < N) dst[k2] = hb[k2];
          }
        }
        hb[0] = fmaf(P.x, hb[0], H.x);
        hb[1] = fmaf(P.y, hb[1], H.y);
        hb[2] = fmaf(P.z, hb[2], H.z);
        hb[3] = fmaf(P.w, hb[3], H.w);
      };
      int jj = 0;
      for (; jj + 2 <= p.W; jj += 2) {  // both chunks' maps are read before the first is applied
        const int i0 = jj * lpg + tid, i1 = i0 + lpg;
        const float4 P0 = aggP[i0], H0 = aggH[i0], P1 = aggP[i1], H1 = aggH[i1];
        link(jj, P0, H0);
        link(jj + 1, P1, H1);
      }
      if (jj < p.W) {
        const int i0 = jj * lpg + tid;
        link(jj, aggP[i0], aggH[i0]);
      }
    }
    __syncthreads();  // B

    // ---- phase 2: the chunk from its incoming state with the kept a, w; readout ------------
    const float4 hi = hin[lane_ok ? tid : 0];
    float h[4] = {hi.x, hi.y, hi.z, hi.w};
    T* const yt = reinterpret_cast<T*>(pool + p.o_y[k & 1]);
    // finishes step tl: + D*u, * silu(z), rounded into the y tile
    auto finish = [&](int tl, float yv) {
      float out = fmaf(Dv, load_elem(xt + tl * cg + c), yv);
      if (HAS_Z) out *= silu(load_elem(xt + (2 * p.xrows + tl) * cg + c));
      if (ch_ok) store_elem(yt + tl * cg + c, out);
    };
    float own[EPL];
#pragma unroll
    for (int i = 0; i < EPL; i++) own[i] = 0.f;
#pragma unroll
    for (int s = 0; s < kT; s++) {
      const float4 c4 = *reinterpret_cast<const float4*>(bct + ((tl0 + s) * 2 + 1) * NSP + 4 * q);
      const float cc4[4] = {c4.x, c4.y, c4.z, c4.w};
      float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
      for (int k2 = 0; k2 < 4; k2++) {
        h[k2] = fmaf(a[s][k2], h[k2], w[s][k2]);
        if (k2 % 2 == 0) acc0 = fmaf(cc4[k2], h[k2], acc0);
        else acc1 = fmaf(cc4[k2], h[k2], acc1);
      }
      const float yv = grp_sum<LPC>(acc0 + acc1);
      if constexpr (LPC > 1) own[s / LPC] = (q == s % LPC) ? yv : own[s / LPC];
      else finish(tl0 + s, yv);
    }
    if constexpr (LPC > 1) {
#pragma unroll
      for (int i = 0; i < EPL; i++) finish(tl0 + i * LPC + q, own[i]);
    }
  }
  __syncthreads();
  if (chain_lane && c < ce && last_state) {
#pragma unroll
    for (int k = 0; k < 4; k++)
      if (4 * q + k < N) last_state[(bi * E + e) * N + 4 * q + k] = hb[k];
  }
}

template <typename T, int LPC, bool SOFTPLUS, bool HAS_Z, bool SAVE>
hipError_t fused_launch(const ScanArgs& a, const FusedPlan& p) {
  return launch_kind(kKindFused, scan_fused_kernel<T, LPC, SOFTPLUS, HAS_Z, SAVE>, p.n_wg, p.n_threads, a.stream,
                     static_cast<const T*>(a.u), static_cast<const T*>(a.delta), a.A, static_cast<const T*>(a.B),
                     static_cast<const T*>(a.C), a.D, static_cast<const T*>(a.z), a.bias, static_cast<T*>(a.y),
                     a.last_state, a.h0, a.saved, a.L, a.E, int(a.N), p);
}

template <typename T, int LPC>
hipError_t fused_flags(const ScanArgs& a, const FusedPlan& p) {
  const bool z = a.z != nullptr, sv = a.saved != nullptr;
#define SSM_FUSED(SP, HZ) \
  return sv ? fused_launch<T, LPC, SP, HZ, true>(a, p) : fused_launch<T, LPC, SP, HZ, false>(a, p)
  if (a.softplus) {
    if (z) { SSM_FUSED(true, true); }
    SSM_FUSED(true, false);
  }
  if (z) { SSM_FUSED(false, true); }
  SSM_FUSED(false, false);
#undef SSM_FUSED
}

template <typename T>
hipError_t fused_typed(const ScanArgs& a, const FusedPlan& p) {
  if (p.lpc == 4) return fused_flags<T, 4>(a, p);
  if (p.lpc == 2) return fused_flags<T, 2>(a, p);
  return fused_flags<T, 1>(a, p);
}

}  // namespace

bool plan_fused(const ScanArgs& a, int n_cu, int max_w, FusedPlan* out) {
  FusedPlan p{};
  const int64_t b = a.b, L = a.L, E = a.E, N = a.N;
  const int es = a.dtype == 0 ? 4 : 2;
  const int nin = a.z ? 3 : 2;
  if (b <= 0 || L <= 0 || E <= 0 || N < 1 || N > 16 || n_cu <= 0) return false;
  // the producers move 8-byte units: rows of u, delta, z, y, B and C and the tensors'
  // starts must be whole units
  const void* ptrs[] = {a.u, a.delta, a.z, a.y, a.B, a.C};
  for (const void* q : ptrs)
    if (q && reinterpret_cast<uintptr_t>(q) % 8 != 0) return false;
  if ((E * es) % 8 != 0 || (N * es) % 8 != 0) return false;
  p.lpc = N <= 4 ? 1 : (N <= 8 ? 2 : 4);
  const int nsp = 4 * p.lpc;
  const int unit = 8 / es;  // channels per 8-byte unit
  // about one workgroup per CU; a chunk's lanes leave room for two chunks or more
  const int64_t per_row = std::max<int64_t>(1, (n_cu + b - 1) / b);
  int64_t cg = (E + per_row - 1) / per_row;
  cg = (cg + unit - 1) / unit * unit;
  const int64_t cg_max = 448 / p.lpc / unit * unit;
  if (cg > cg_max) cg = cg_max;
  p.cg = int(cg);
  p.groups_row = int((E + cg - 1) / cg);
  if (b * p.groups_row > INT32_MAX) return false;
  p.n_wg = int(b * p.groups_row);
  const int lpg = p.lpc * p.cg;
  // one producer pass moves plane units: xR rows of the group's channels, bR rows of B / C
  const int plane = 64 * kProd;
  const int xdu = p.cg * es / 8, bdu = int(N) * es / 8;
  p.xR = plane / xdu;
  p.bR = plane / bdu;
  if (p.xR < 1 || p.bR < 1) return false;
  // chunks per block: as many as the compute waves hold, within the producers' registers
  // (6 passes of [u | delta | z], 3 of B / C per block) and the sequence
  int64_t W = (64 * (kFusedMaxWaves - kProd)) / lpg;
  W = std::min<int64_t>(W, kFusedMaxChunks);
  W = std::min<int64_t>(W, 6 * p.xR / kT);
  W = std::min<int64_t>(W, 3 * p.bR / kT);
  W = std::min<int64_t>(W, (L + kT - 1) / kT);
  if (W < 1 || W > max_w) return false;  // the chunk-0 lanes chain W maps per block
  p.W = int(W);
  p.BT = p.W * kT;
  p.lanes = p.W * lpg;
  p.n_cmp = (p.lanes + 63) / 64;
  p.n_prod = kProd;
  p.n_threads = 64 * (p.n_cmp + p.n_prod);
  if (p.n_cmp < 8) return false;  // too few compute waves to keep the SIMDs issuing
  const int64_t nblk = (L + p.BT - 1) / p.BT;
  if (nblk > INT32_MAX) return false;
  p.nblk = int(nblk);
  p.xM = (p.BT + p.xR - 1) / p.xR;
  p.bM = (p.BT + p.bR - 1) / p.bR;
  if (p.xM > 6 || p.bM > 3) return false;  // the producers' registers
  p.xrows = p.xR * p.xM;
  p.brows = p.bR * p.bM;
  p.ux = p.ub = 8;
  // LDS: B / C rows and [u | delta | z] tiles (three blocks in flight), the chunk maps,
  // the incoming states, the y tile (two blocks in flight), a junk slot for idle lanes
  auto al16 = [](int64_t v) { return (v + 15) / 16 * 16; };
  const int64_t bcb = al16(int64_t(p.brows) * 2 * nsp * 4), xb = al16(int64_t(nin) * p.xrows * p.cg * es);
  const int64_t ab = int64_t(p.lanes) * 32, hb = int64_t(p.lanes) * 16, yb = al16(int64_t(p.xrows) * p.cg * es);
  int64_t off = 0;
  for (int i = 0; i < 3; i++) { p.o_bc[i] = int(off); off += bcb; }  // contiguous: zeroed together
  for (int i = 0; i < 3; i++) { p.o_x[i] = int(off); off += xb; }
  p.o_agg = int(off); off += ab;
  p.o_hin = int(off); off += hb;
  for (int i = 0; i < 2; i++) { p.o_y[i] = int(off); off += yb; }
  p.o_junk = int(off); off += 16;
  if (off > kPoolBytes) return false;
  p.lds_bytes = int(off);
  // buffer offsets inside a block's rows are 32-bit
  if (int64_t(p.xrows) * E * es > INT32_MAX / 2) return false;
  *out = p;
  return true;
}

hipError_t launch_fused(const ScanArgs& a, const FusedPlan& p) {
  return a.dtype == 0 ? fused_typed<float>(a, p) : fused_typed<bf16_bits>(a, p);
}

}  // namespace ssm
