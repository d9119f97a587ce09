// The chain of chunk aggregates that joins the chunks of a cut sequence.
//
// A chunk of steps acts on the state it receives as an affine map
// v -> exp2(a2 * s_c) * v + H_c (a2 = A * log2(e) per state coordinate,
// s_c the chunk's summed step; abhik.ai page, "Compose the updates instead of
// waiting for every state").  Per position (a state coordinate of one chain)
// the value entering every chunk follows from chaining those maps from a
// start value.  The forward scan, its backward (in reverse time) and the
// scalar-per-head scan all keep their aggregates in the same layout:
//   agg  [outer][n_chunks][mid][inner]  aggregates in, chained values out (in place)
//   sums [outer][n_chunks][mid]         decay exponent of each chunk (times a2)
// with a position = (outer, mid, inner) index.
//
// With many positions (the long scans: 80k and more) the chain is bound by
// memory bandwidth, one thread per position walking its chain with the next
// U aggregates in flight.  With few positions (a long sequence over few
// channels, as on one GPU of several that split the channels) one thread per
// position leaves most of the chip idle and the walk is bound by load
// latency.  Then each chain is cut into G stretches, one thread each (the G
// threads of a position share a workgroup): every thread reduces its stretch
// from zero (summed exponent and aggregate), the G results go through LDS,
// each thread composes the ones before its own with the start value, then
// walks its stretch again from the value entering it, writing the chained
// values.  The second walk re-reads what the first brought into the caches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ssm_device.h"

namespace ssm {

struct ChainArgs {
  float* agg;
  const float* sums;
  const float* A;     // [mid][N]: a2 = A * log2(e) for inner < N, 0 beyond; null: a2 = log2(e) everywhere
  const float* init;  // start value at [(outer * mid + mid_index) * N + inner] (inner < N); null: zero
  float* final_out;   // value after the last chunk, indexed as init; null: not written
  int64_t outer, mid;
  int inner, N;
  int n_chunks;
  int K;  // chunks in the chain; forward: chunks 0 .. K-1, reverse: chunks n_chunks-1 down to n_chunks-K
};

// REVERSE: walk from the last chunk down.  EXCL: a chunk's slot receives the
// value entering it (else the value leaving it).  SLOT0: after a reverse walk,
// the final value also goes to chunk 0's slot.  A workgroup holds P positions
// x G stretches, P a multiple of 64, so every wave walks one stretch: its
// chunk range, the chunk offsets and the loop branches are wave-uniform
// (scalar), and only the per-lane base addresses are vector values.
template <int G, int U, bool REVERSE, bool EXCL, bool SLOT0>
__global__ __launch_bounds__(64 * G > 256 ? 64 * G : 256) void chain_kernel(ChainArgs c) {
  constexpr int P = 64 * G > 256 ? 64 : 256 / G;  // positions per workgroup
  __shared__ float sh_v[G][P], sh_l[G][P];
  const int j = threadIdx.x % P;
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x / P);
  const int64_t total = c.outer * c.mid * c.inner;
  const int64_t pos = int64_t(blockIdx.x) * P + j;
  const bool valid = pos < total;
  const int64_t pp = valid ? pos : 0;
  const int i = int(pp % c.inner);
  const int64_t m = (pp / c.inner) % c.mid;
  const int64_t o = pp / (int64_t(c.inner) * c.mid);
  const bool real = i < c.N;
  const float a2 = c.A ? (real ? c.A[m * c.N + i] * kLog2e : 0.f) : kLog2e;
  const int64_t state_at = (o * c.mid + m) * c.N + i;
  const int S = (c.K + G - 1) / G;
  const int kb = min(c.K, g * S), ke = min(c.K, kb + S);
  // item k of the chain is chunk k (forward) or n_chunks - 1 - k (reverse): its slot and
  // its exponent sit k uniform strides from item 0's
  const int64_t sa = (REVERSE ? -c.mid : c.mid) * int64_t(c.inner), ss = REVERSE ? -c.mid : c.mid;
  const int64_t c0 = REVERSE ? c.n_chunks - 1 : 0;
  float* const a0 = c.agg + ((o * c.n_chunks + c0) * c.mid + m) * c.inner + i;
  const float* const s0 = c.sums + (o * c.n_chunks + c0) * c.mid + m;

  // one walk over items [kb, ke) from v; with WRITE, the chained values are stored
  auto walk = [&](float v, float& lsum, auto write_tag) {
    constexpr bool WRITE = decltype(write_tag)::value;
    float Hs[U], Ss[U];
    auto load = [&](int k0) {
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int k = min(k0 + u, ke - 1);  // past the end: a valid item, unused
        Hs[u] = a0[k * sa];
        Ss[u] = s0[k * ss];
      }
    };
    if (kb < ke) load(kb);
    for (int k0 = kb; k0 < ke; k0 += U) {
      float Hc[U], Sc[U];
#pragma unroll
      for (int u = 0; u < U; u++) { Hc[u] = Hs[u]; Sc[u] = Ss[u]; }
      if (k0 + U < ke) load(k0 + U);
#pragma unroll
      for (int u = 0; u < U; u++) {
        if (k0 + u < ke) {
          if (WRITE && EXCL) a0[(k0 + u) * sa] = v;
          v = fmaf(exp2_fast(a2 * Sc[u]), v, Hc[u]);
          lsum += Sc[u];
          if (WRITE && !EXCL) a0[(k0 + u) * sa] = v;
        }
      }
    }
    return v;
  };

  float v0 = (valid && real && c.init) ? c.init[state_at] : 0.f;
  if constexpr (G > 1) {
    float agg = 0.f, lsum = 0.f;
    if (valid && g < G - 1) agg = walk(0.f, lsum, std::false_type{});  // the last stretch's is used by no one
    sh_v[g][j] = agg;
    sh_l[g][j] = lsum;
    __syncthreads();
    for (int q = 0; q < g; q++) v0 = fmaf(exp2_fast(a2 * sh_l[q][j]), v0, sh_v[q][j]);
  }
  if (valid) {
    float unused = 0.f;
    const float v = walk(v0, unused, std::true_type{});
    if (g == G - 1) {
      if (SLOT0) c.agg[((o * c.n_chunks) * c.mid + m) * c.inner + i] = v;
      if (c.final_out && real) c.final_out[state_at] = v;
    }
  }
}

// Stretches per chain: 1 with at least 65536 positions (1024 waves: enough
// loads in flight to stream the aggregates at full bandwidth), else doubled
// up to 8 while the threads stay below that count and every stretch keeps at
// least 32 chunks.
inline int chain_stretches(int64_t positions, int K) {
  constexpr int64_t kEnough = int64_t(1) << 16;
  int G = 1;
  while (G < 8 && positions * G < kEnough && K / (2 * G) >= 32) G *= 2;
  return G;
}

template <int G, bool REVERSE, bool EXCL, bool SLOT0>
hipError_t launch_chain_g(int kind, const ChainArgs& c, hipStream_t s, int64_t positions) {
  constexpr int P = 64 * G > 256 ? 64 : 256 / G, T = P * G;  // as in chain_kernel
  const int64_t blocks = (positions + P - 1) / P;
  const int S = (c.K + G - 1) / G;  // chunks per stretch: loads in flight to match
  if (S > 64) return launch_kind(kind, chain_kernel<G, 32, REVERSE, EXCL, SLOT0>, blocks, T, s, c);
  if (S > 16) return launch_kind(kind, chain_kernel<G, 16, REVERSE, EXCL, SLOT0>, blocks, T, s, c);
  return launch_kind(kind, chain_kernel<G, 8, REVERSE, EXCL, SLOT0>, blocks, T, s, c);
}

template <bool REVERSE, bool EXCL, bool SLOT0>
hipError_t launch_chain(int kind, const ChainArgs& c, hipStream_t s) {
  const int64_t positions = c.outer * c.mid * c.inner;
  if (positions <= 0) return hipSuccess;
  switch (chain_stretches(positions, c.K)) {
    case 1: return launch_chain_g<1, REVERSE, EXCL, SLOT0>(kind, c, s, positions);
    case 2: return launch_chain_g<2, REVERSE, EXCL, SLOT0>(kind, c, s, positions);
    case 4: return launch_chain_g<4, REVERSE, EXCL, SLOT0>(kind, c, s, positions);
    default: return launch_chain_g<8, REVERSE, EXCL, SLOT0>(kind, c, s, positions);
  }
}

}  // namespace ssm
