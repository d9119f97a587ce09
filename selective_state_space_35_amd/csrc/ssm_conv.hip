// ssm_conv.hip -- causal depthwise convolution + SiLU that precedes the scan
// in the Mamba block, and its single-token form used while generating.
//
// Page defining the operation: "Mamba: Linear-Time Sequence Modeling with
// Selective State Spaces" (abhik.ai), section "Original paper, equations and
// runnable CPU code":
//   row 4 "Add causal local context before selecting coefficients":
//     x[t,c] = silu(cb[c] + sum_{k=0..K-1} q[c,k] * v[t-K+1+k, c]), left zero padding;
//   row 6 "Carry both buffers to the next token": the convolution state keeps
//     the K most recent samples (the latest included), shifted left by one
//     and appended to before the same sum.
//
// Layout: v, x [b, L, E] (channels fastest, like the scan's inputs);
// q [E, K] float; cb [E] float; convolution state [b, E, K] in the I/O dtype,
// oldest sample first.
//
// conv_fwd_vec_kernel (E a multiple of 8 bf16 / 4 f32 channels, 16-byte aligned
// rows): each lane owns 16 bytes of a row, so a wave moves 1 KiB per load and
// per store; kConvVGroup rows are in flight.  conv_fwd_kernel (any E and
// alignment): one lane per channel.  Both give a wave a chunk of kConvChunk
// steps; the K-1 previous samples live in registers and slide along, and the
// chunk's first window reads the K-1 rows before it (or the incoming state /
// zeros).  Each input and output element crosses HBM once, apart from those
// K-1 rows per chunk: an HBM-bound kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ssm_device.h"
#include "ssm_internal.h"
#include "ssm_profile.h"

namespace ssm {
namespace {

#ifndef SSM_CONV_CHUNK
#define SSM_CONV_CHUNK 32
#endif
#ifndef SSM_CONV_VGROUP
#define SSM_CONV_VGROUP 8
#endif
constexpr int kConvChunk = SSM_CONV_CHUNK;    // steps per wave
constexpr int kConvGroup = 8;                 // loads issued together (one channel per lane)
constexpr int kConvVGroup = SSM_CONV_VGROUP;  // 16-byte rows in flight (vector kernel)

template <typename T, int K>
__global__ __launch_bounds__(kWave) void conv_fwd_kernel(const T* __restrict__ v, const float* __restrict__ q,
                                                         const float* __restrict__ cb,
                                                         const T* __restrict__ state_in, T* __restrict__ x,
                                                         T* __restrict__ state_out, int64_t L, int64_t E,
                                                         int n_chunks, int e_blocks) {
  const int eb = blockIdx.x % e_blocks;
  const int rest = blockIdx.x / e_blocks;
  const int c = rest % n_chunks;
  const int64_t bi = rest / n_chunks;
  const int64_t e = int64_t(eb) * kWave + threadIdx.x;
  const bool active = e < E;
  const int64_t ec = active ? e : E - 1;
  const int64_t t0 = int64_t(c) * kConvChunk;
  const int64_t t1 = (t0 + kConvChunk < L) ? t0 + kConvChunk : L;

  float w[K];
#pragma unroll
  for (int k = 0; k < K; k++) w[k] = q[ec * K + k];
  const float bias = cb ? cb[ec] : 0.f;
  // hist[j] = sample at time t0 - (K-1) + j, j < K-1
  float hist[K > 1 ? K - 1 : 1];
#pragma unroll
  for (int j = 0; j < K - 1; j++) {
    const int64_t s = t0 - (K - 1) + j;
    if (s >= 0) hist[j] = load_elem(v + (bi * L + s) * E + ec);
    else hist[j] = state_in ? load_elem(state_in + (bi * E + ec) * K + (K + s)) : 0.f;
  }

  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + (bi * L + t0) * E + int64_t(eb) * kWave);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + (bi * L + t0) * E + int64_t(eb) * kWave);
  const int voff = int(ec - int64_t(eb) * kWave) * int(sizeof(T));
  const int row_bytes = int(E * int64_t(sizeof(T)));  // kConvChunk * row_bytes < 2^31 is checked by the caller
  const int n_steps = int(t1 - t0);
  float last = 0.f;     // newest sample seen
  float dropped = 0.f;  // sample that last left the window (the oldest of the K most recent)
  for (int g0 = 0; g0 < n_steps; g0 += kConvGroup) {
    float vs[kConvGroup];
#pragma unroll
    for (int k = 0; k < kConvGroup; k++) {
      const int kk = (g0 + k < n_steps) ? g0 + k : n_steps - 1;  // past the end: a valid row, unused
      vs[k] = buf_load(rv, voff, kk * row_bytes, (T*)nullptr);
    }
#pragma unroll
    for (int k = 0; k < kConvGroup; k++) {
      if (g0 + k < n_steps) {
        float acc = bias;
#pragma unroll
        for (int j = 0; j < K - 1; j++) acc = fmaf(w[j], hist[j], acc);
        acc = fmaf(w[K - 1], vs[k], acc);
        if (active) buf_store(rx, voff, (g0 + k) * row_bytes, silu(acc), (T*)nullptr);
        if (K > 1) dropped = hist[0];
#pragma unroll
        for (int j = 0; j + 1 < K - 1; j++) hist[j] = hist[j + 1];
        if (K > 1) hist[K - 2] = vs[k];
        last = vs[k];
      }
    }
  }
  if (state_out && c == n_chunks - 1 && active) {
    T* dst = state_out + (bi * E + e) * K;
    // the K most recent samples, oldest first: the one that just left the window,
    // then the window (whose newest entry is the last sample)
    if (K == 1) {
      store_elem(dst, last);
    } else {
      store_elem(dst, dropped);
#pragma unroll
      for (int j = 0; j < K - 1; j++) store_elem(dst + 1 + j, hist[j]);
    }
  }
}

// 16 bytes of a row: 8 bf16 or 4 f32 channels, widened to f32
template <typename T>
struct Vec16 {
  static constexpr int V = 16 / int(sizeof(T));
  float v[V];
};
__device__ __forceinline__ Vec16<float> unpack16(uint32_t a, uint32_t b, uint32_t c, uint32_t d, float*) {
  Vec16<float> r;
  r.v[0] = __uint_as_float(a); r.v[1] = __uint_as_float(b); r.v[2] = __uint_as_float(c); r.v[3] = __uint_as_float(d);
  return r;
}
__device__ __forceinline__ Vec16<bf16_bits> unpack16(uint32_t a, uint32_t b, uint32_t c, uint32_t d, bf16_bits*) {
  Vec16<bf16_bits> r;
  const uint32_t w[4] = {a, b, c, d};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    r.v[2 * i] = __uint_as_float(w[i] << 16);
    r.v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
  return r;
}
template <typename T>
__device__ __forceinline__ Vec16<T> load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const auto u = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return unpack16(u[0], u[1], u[2], u[3], (T*)nullptr);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(__builtin_bit_cast(bf16_bits, static_cast<__bf16>(lo))) |
         (uint32_t(__builtin_bit_cast(bf16_bits, static_cast<__bf16>(hi))) << 16);
}
template <typename T>
__device__ __forceinline__ void store16(__amdgpu_buffer_rsrc_t r, int voff, int soff, const float (&v)[Vec16<T>::V]) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u4;
  u4 w;
  if constexpr (sizeof(T) == 4) {
    w = u4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
  } else {
    w = u4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
  }
  __builtin_amdgcn_raw_buffer_store_b128(w, r, voff, soff, 0);
}

// Same operation as conv_fwd_kernel with 16-byte accesses: each lane owns V
// consecutive channels (V = 8 for bf16, 4 for f32), so a wave moves 1 KiB of a
// row per load.  Needs E % V == 0 and 16-byte aligned rows (checked by the launcher).
template <typename T, int K>
__global__ __launch_bounds__(kWave) void conv_fwd_vec_kernel(const T* __restrict__ v, const float* __restrict__ q,
                                                             const float* __restrict__ cb,
                                                             const T* __restrict__ state_in, T* __restrict__ x,
                                                             T* __restrict__ state_out, int64_t L, int64_t E,
                                                             int n_chunks, int e_blocks) {
  constexpr int V = Vec16<T>::V;
  const int eb = blockIdx.x % e_blocks;
  const int rest = blockIdx.x / e_blocks;
  const int c = rest % n_chunks;
  const int64_t bi = rest / n_chunks;
  const int64_t e0 = (int64_t(eb) * kWave + threadIdx.x) * V;  // first channel of the lane
  const bool active = e0 < E;
  const int64_t ec0 = active ? e0 : E - V;                      // inactive lanes read a valid vector
  const int64_t t0 = int64_t(c) * kConvChunk;
  const int64_t t1 = (t0 + kConvChunk < L) ? t0 + kConvChunk : L;

  float w[V][K], bias[V];
#pragma unroll
  for (int j = 0; j < V; j++) {
#pragma unroll
    for (int k = 0; k < K; k++) w[j][k] = q[(ec0 + j) * K + k];
    bias[j] = cb ? cb[ec0 + j] : 0.f;
  }
  const int64_t row_base = bi * L * E;
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + row_base + t0 * E);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + row_base + t0 * E);
  const int voff = int(ec0) * int(sizeof(T));
  const int row_bytes = int(E * int64_t(sizeof(T)));  // kConvChunk * row_bytes < 2^31 is checked by the caller

  // hist[i][j] = sample at time t0 - (K-1) + i of channel ec0 + j
  float hist[K > 1 ? K - 1 : 1][V];
#pragma unroll
  for (int i = 0; i < K - 1; i++) {
    const int64_t s = t0 - (K - 1) + i;
    if (s >= 0) {
      const __amdgpu_buffer_rsrc_t rp = make_rsrc(v + row_base + s * E);
      const Vec16<T> r = load16<T>(rp, voff, 0);
#pragma unroll
      for (int j = 0; j < V; j++) hist[i][j] = r.v[j];
    } else {
#pragma unroll
      for (int j = 0; j < V; j++)
        hist[i][j] = state_in ? load_elem(state_in + (bi * E + ec0 + j) * K + (K + s)) : 0.f;
    }
  }

  const int n_steps = int(t1 - t0);
  float dropped[V];
#pragma unroll
  for (int j = 0; j < V; j++) dropped[j] = 0.f;
  float last[V];
#pragma unroll
  for (int j = 0; j < V; j++) last[j] = 0.f;
  constexpr int G = kConvVGroup;
  for (int g0 = 0; g0 < n_steps; g0 += G) {
    Vec16<T> in[G];
#pragma unroll
    for (int k = 0; k < G; k++) {
      const int kk = (g0 + k < n_steps) ? g0 + k : n_steps - 1;  // past the end: a valid row, unused
      in[k] = load16<T>(rv, voff, kk * row_bytes);
    }
#pragma unroll
    for (int k = 0; k < G; k++) {
      if (g0 + k < n_steps) {
        float out[V];
#pragma unroll
        for (int j = 0; j < V; j++) {
          float acc = bias[j];
#pragma unroll
          for (int i = 0; i < K - 1; i++) acc = fmaf(w[j][i], hist[i][j], acc);
          acc = fmaf(w[j][K - 1], in[k].v[j], acc);
          out[j] = silu(acc);
          if (K > 1) dropped[j] = hist[0][j];
#pragma unroll
          for (int i = 0; i + 1 < K - 1; i++) hist[i][j] = hist[i + 1][j];
          if (K > 1) hist[K - 2][j] = in[k].v[j];
          last[j] = in[k].v[j];
        }
        if (active) store16<T>(rx, voff, (g0 + k) * row_bytes, out);
      }
    }
  }
  if (state_out && c == n_chunks - 1 && active) {
#pragma unroll
    for (int j = 0; j < V; j++) {
      T* dst = state_out + (bi * E + e0 + j) * K;
      if (K == 1) {
        store_elem(dst, last[j]);
      } else {
        store_elem(dst, dropped[j]);
#pragma unroll
        for (int i = 0; i < K - 1; i++) store_elem(dst + 1 + i, hist[i][j]);
      }
    }
  }
}

// last convolution state of an empty sequence: the incoming one, or zeros
template <typename T>
__global__ __launch_bounds__(256) void conv_state_copy_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                                              int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) store_elem(dst + i, src ? load_elem(src + i) : 0.f);
}

// Bytes of a channel's K-sample state slice and of its K weights, when each
// can move as one aligned vector access (a power of two, at most 16 bytes).
template <typename T, int K>
struct ConvSlice {
  static constexpr int kStateBytes = K * int(sizeof(T)), kWeightBytes = K * 4;
  static constexpr bool pow2(int n) { return n > 0 && n <= 16 && (n & (n - 1)) == 0; }
  static constexpr bool kVec = pow2(kStateBytes) && pow2(kWeightBytes);
};

// One token for every (b, e): shift the K-sample state left, append v, x = silu(cb + q . state).
// VEC: the state slice and the weights of a channel each move as one vector access
// (K = 4 in bf16: 8 and 16 bytes) instead of K element accesses.
template <typename T, int K, bool VEC>
__global__ __launch_bounds__(256) void conv_update_kernel(T* __restrict__ state, const T* __restrict__ v,
                                                          const float* __restrict__ q, const float* __restrict__ cb,
                                                          T* __restrict__ x, int E, int row_blocks) {
  const int bi = blockIdx.x / row_blocks;  // batch row: uniform per workgroup
  const int e = (blockIdx.x - bi * row_blocks) * 256 + threadIdx.x;
  if (e >= E) return;
  const int64_t cc = int64_t(bi) * E + e;
  T* st = state + cc * K;
  constexpr bool kV = ConvSlice<T, K>::kVec;  // the slice sizes are alignments only when they are powers of two
  struct alignas(kV ? ConvSlice<T, K>::kStateBytes : int(sizeof(T))) SV { T v[K]; };
  struct alignas(kV ? ConvSlice<T, K>::kWeightBytes : 4) QV { float v[K]; };
  static_assert(!VEC || kV, "vector access needs power-of-two slices");
  float s[K], w[K];
  if constexpr (VEC) {
    const SV sv = *reinterpret_cast<const SV*>(st);
    const QV qv = *reinterpret_cast<const QV*>(q + int64_t(e) * K);
#pragma unroll
    for (int k = 0; k < K; k++) {
      s[k] = load_elem(&sv.v[k]);
      w[k] = qv.v[k];
    }
  } else {
#pragma unroll
    for (int k = 0; k < K; k++) {
      s[k] = load_elem(st + k);
      w[k] = q[int64_t(e) * K + k];
    }
  }
  const float vt = load_elem(v + cc);
  float acc = cb ? cb[e] : 0.f;
  float sh[K];
#pragma unroll
  for (int k = 0; k < K; k++) {
    sh[k] = (k + 1 < K) ? s[k + 1] : vt;  // shifted state: oldest dropped, newest appended
    acc = fmaf(w[k], sh[k], acc);
  }
  if constexpr (VEC) {
    SV out;
#pragma unroll
    for (int k = 0; k < K; k++) store_elem(&out.v[k], sh[k]);
    *reinterpret_cast<SV*>(st) = out;
  } else {
#pragma unroll
    for (int k = 0; k < K; k++) store_elem(st + k, sh[k]);
  }
  store_elem(x + cc, silu(acc));
}

template <typename T, int K>
hipError_t conv_fwd_k(const ConvArgs& a) {
  const int n_chunks = int((a.L + kConvChunk - 1) / kConvChunk);
  constexpr int V = Vec16<T>::V;
  const bool vec = a.E % V == 0 && reinterpret_cast<uintptr_t>(a.v) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(a.x) % 16 == 0;
  if (vec) {
    const int e_blocks = int((a.E / V + kWave - 1) / kWave);
    return launch_kind(kKindConv, conv_fwd_vec_kernel<T, K>, a.b * n_chunks * e_blocks, kWave, a.stream,
                       static_cast<const T*>(a.v), a.q, a.cb, static_cast<const T*>(a.state_in), static_cast<T*>(a.x),
                       static_cast<T*>(a.state_out), a.L, a.E, n_chunks, e_blocks);
  }
  const int e_blocks = int((a.E + kWave - 1) / kWave);
  return launch_kind(kKindConv, conv_fwd_kernel<T, K>, a.b * n_chunks * e_blocks, kWave, a.stream,
                     static_cast<const T*>(a.v), a.q, a.cb, static_cast<const T*>(a.state_in), static_cast<T*>(a.x),
                     static_cast<T*>(a.state_out), a.L, a.E, n_chunks, e_blocks);
}

template <typename T, int K>
hipError_t conv_update_k(const ConvArgs& a) {
  const int row_blocks = int((a.E + 255) / 256);
  if constexpr (ConvSlice<T, K>::kVec) {
    const bool vec = reinterpret_cast<uintptr_t>(a.state_out) % ConvSlice<T, K>::kStateBytes == 0 &&
                     reinterpret_cast<uintptr_t>(a.q) % ConvSlice<T, K>::kWeightBytes == 0;
    if (vec)
      return launch_kind(kKindConvUpdate, conv_update_kernel<T, K, true>, a.b * row_blocks, 256, a.stream,
                         static_cast<T*>(a.state_out), static_cast<const T*>(a.v), a.q, a.cb, static_cast<T*>(a.x),
                         int(a.E), row_blocks);
  }
  return launch_kind(kKindConvUpdate, conv_update_kernel<T, K, false>, a.b * row_blocks, 256, a.stream,
                     static_cast<T*>(a.state_out), static_cast<const T*>(a.v), a.q, a.cb, static_cast<T*>(a.x),
                     int(a.E), row_blocks);
}

// Dispatch on the kernel width K (1..kMaxConvK) as a compile-time constant.
template <typename T, template <typename, int> class F>
struct ByK {
  static hipError_t run(const ConvArgs& a) {
    switch (a.K) {
      case 1: return F<T, 1>::run(a);
      case 2: return F<T, 2>::run(a);
      case 3: return F<T, 3>::run(a);
      case 4: return F<T, 4>::run(a);
      case 5: return F<T, 5>::run(a);
      case 6: return F<T, 6>::run(a);
      case 7: return F<T, 7>::run(a);
      default: return F<T, 8>::run(a);
    }
  }
};
template <typename T, int K>
struct FwdK {
  static hipError_t run(const ConvArgs& a) { return conv_fwd_k<T, K>(a); }
};
template <typename T, int K>
struct UpdK {
  static hipError_t run(const ConvArgs& a) { return conv_update_k<T, K>(a); }
};

}  // namespace

int64_t conv_chunk_steps() { return kConvChunk; }

hipError_t launch_conv_fwd(const ConvArgs& a) {
  if (a.b == 0 || a.E == 0) return hipSuccess;
  if (a.L == 0) {
    if (!a.state_out) return hipSuccess;
    const int64_t n = a.b * a.E * a.K;
    return a.dtype == 0
               ? launch_kind(kKindConv, conv_state_copy_kernel<float>, (n + 255) / 256, 256, a.stream,
                             static_cast<const float*>(a.state_in), static_cast<float*>(a.state_out), n)
               : launch_kind(kKindConv, conv_state_copy_kernel<bf16_bits>, (n + 255) / 256, 256, a.stream,
                             static_cast<const bf16_bits*>(a.state_in), static_cast<bf16_bits*>(a.state_out), n);
  }
  return a.dtype == 0 ? ByK<float, FwdK>::run(a) : ByK<bf16_bits, FwdK>::run(a);
}

hipError_t launch_conv_update(const ConvArgs& a) {
  if (a.b == 0 || a.E == 0) return hipSuccess;
  return a.dtype == 0 ? ByK<float, UpdK>::run(a) : ByK<bf16_bits, UpdK>::run(a);
}

}  // namespace ssm
