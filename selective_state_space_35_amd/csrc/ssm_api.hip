// ssm_api.hip -- the extern "C" entry points declared in include/ssm.h:
// argument validation, status codes, and the hand-off to the launchers.
// Every argument check runs before any HIP call, so an invalid call enqueues
// nothing and also works on a host without a GPU.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstring>

#include "ssm.h"
#include "ssm_internal.h"

namespace {

thread_local char g_last_hip_error[256] = "";

int hip_status(hipError_t err) {
  if (err == hipSuccess) return SSM_OK;
  const char* s = hipGetErrorString(err);
  std::strncpy(g_last_hip_error, s ? s : "unknown HIP error", sizeof(g_last_hip_error) - 1);
  g_last_hip_error[sizeof(g_last_hip_error) - 1] = '\0';
  (void)hipGetLastError();  // clear the sticky launch error
  return SSM_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

// Every size is at most 2^48 on its own (any real tensor is far smaller), so the plans' sums and
// rounded divisions cannot overflow even where another size is zero and the products are.
constexpr int64_t kMaxSize = int64_t(1) << 48;
bool size_ok(int64_t v) { return v >= 0 && v <= kMaxSize; }

// Common size / dtype checks.  `elems` receives b*L*E (or b*E).
int check_sizes(int64_t b, int64_t L, int64_t E, int64_t N, int dtype) {
  if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (!size_ok(b) || !size_ok(L) || !size_ok(E) || N < 0) return SSM_ERR_DIM;
  if (N < 1 || N > 16) return SSM_ERR_UNSUPPORTED_N;
  int64_t t = 0;
  if (!mul_ok(b, L, &t) || !mul_ok(t, E, &t) || !mul_ok(t, 4, &t)) return SSM_ERR_DIM;
  if (!mul_ok(b, L, &t) || !mul_ok(t, N, &t) || !mul_ok(t, 4, &t)) return SSM_ERR_DIM;
  if (!mul_ok(b, E, &t) || !mul_ok(t, N, &t) || !mul_ok(t, 16, &t)) return SSM_ERR_DIM;
  return SSM_OK;
}

// states saved by ssm_scan_fwd_save: one [E, N] slice per kSaveEvery steps but the last
int64_t saved_count(int64_t b, int64_t L, int64_t E, int64_t N) {
  if (b <= 0 || L <= ssm::kSaveEvery || E <= 0 || N <= 0) return 0;
  return b * ((L + ssm::kSaveEvery - 1) / ssm::kSaveEvery - 1) * E * N;
}

int prepare_scan(const void* u, const void* delta, const float* A, const void* B, const void* C, const float* D,
                 const void* z, const float* delta_bias, int softplus, const float* initial_state, void* y,
                 float* last_state, float* saved, const ssm_scan_tuning* tuning, int64_t b, int64_t L, int64_t E,
                 int64_t N, int dtype, void* stream, ssm::ScanArgs* a, ssm::ScanPlan* pl);
int scan_fwd_impl(const void* u, const void* delta, const float* A, const void* B, const void* C, const float* D,
                  const void* z, const float* delta_bias, int softplus, const float* initial_state, void* y,
                  float* last_state, float* saved, const ssm_scan_tuning* tuning, int64_t b, int64_t L, int64_t E,
                  int64_t N, int dtype, void* stream);
int scan_bwd_impl(const void* u, const void* delta, const float* A, const void* B, const void* C, const float* D,
                  const void* z, const float* delta_bias, int softplus, const float* initial_state,
                  const float* saved, const void* dy, const float* d_last_state, void* du, void* ddelta, float* dA,
                  float* dB, float* dC, float* dD, void* dz, float* d_delta_bias, float* d_initial_state, int64_t b,
                  int64_t L, int64_t E, int64_t N, int dtype, void* stream);

}  // namespace

extern "C" {

int ssm_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C, const float* D,
                 const void* z, const float* delta_bias, int softplus, void* y, float* last_state, int64_t b,
                 int64_t L, int64_t E, int64_t N, int dtype, void* stream) {
  return ssm_scan_fwd_from(u, delta, A, B, C, D, z, delta_bias, softplus, nullptr, y, last_state, b, L, E, N, dtype,
                           stream);
}

int ssm_scan_fwd_from(const void* u, const void* delta, const float* A, const void* B, const void* C,
                      const float* D, const void* z, const float* delta_bias, int softplus,
                      const float* initial_state, void* y, float* last_state, int64_t b, int64_t L, int64_t E,
                      int64_t N, int dtype, void* stream) {
  return scan_fwd_impl(u, delta, A, B, C, D, z, delta_bias, softplus, initial_state, y, last_state, nullptr, nullptr, b,
                       L, E, N, dtype, stream);
}

int ssm_scan_fwd_save(const void* u, const void* delta, const float* A, const void* B, const void* C,
                      const float* D, const void* z, const float* delta_bias, int softplus,
                      const float* initial_state, void* y, float* last_state, float* saved_states, int64_t b,
                      int64_t L, int64_t E, int64_t N, int dtype, void* stream) {
  int st = check_sizes(b, L, E, N, dtype);
  if (st != SSM_OK) return st;
  if (saved_count(b, L, E, N) > 0 && !saved_states) return SSM_ERR_NULL;
  if (saved_states && !aligned(saved_states, 4)) return SSM_ERR_ALIGN;
  return scan_fwd_impl(u, delta, A, B, C, D, z, delta_bias, softplus, initial_state, y, last_state, saved_states,
                       nullptr, b, L, E, N, dtype, stream);
}

int ssm_scan_fwd_tuned(const void* u, const void* delta, const float* A, const void* B, const void* C,
                       const float* D, const void* z, const float* delta_bias, int softplus,
                       const float* initial_state, void* y, float* last_state, float* saved_states,
                       const ssm_scan_tuning* tuning, int64_t b, int64_t L, int64_t E, int64_t N, int dtype,
                       void* stream) {
  int st = check_sizes(b, L, E, N, dtype);
  if (st != SSM_OK) return st;
  if (saved_states && !aligned(saved_states, 4)) return SSM_ERR_ALIGN;
  return scan_fwd_impl(u, delta, A, B, C, D, z, delta_bias, softplus, initial_state, y, last_state, saved_states,
                       tuning, b, L, E, N, dtype, stream);
}

int ssm_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B, const void* C,
                         const float* D, const void* z, const float* delta_bias, int softplus,
                         const float* initial_state, void* y, float* last_state, int64_t b, int64_t L, int64_t E,
                         int64_t N, int dtype, void* stream) {
  ssm::ScanArgs a{};
  ssm::ScanPlan pl{};
  int st = prepare_scan(u, delta, A, B, C, D, z, delta_bias, softplus, initial_state, y, last_state, nullptr, nullptr,
                        b, L, E, N, dtype, stream, &a, &pl);
  if (st != SSM_OK || b == 0 || E == 0) return st;
  if (L == 0) return hip_status(ssm::launch_scan(a));  // no workspace: the last state only
  int n_cu = 0;
  hipError_t err = ssm::device_cu_count(&n_cu);
  if (err != hipSuccess) return hip_status(err);
  ssm::FusedPlan fp;
  if (ssm::choose_path(a, pl, n_cu, &fp) == ssm::kPathSinglePass) return hip_status(ssm::launch_scan(a));
  const size_t need = ssm::chunked_workspace_bytes(a, pl);
  if (need > ssm::kScratchBytes) return SSM_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    err = ssm::scratch_address(&ws);
    if (err != hipSuccess) return hip_status(err);
  }
  return hip_status(ssm::launch_scan(a, ws, ssm::kScratchBytes));
}

}  // extern "C"

namespace {

// The library's form of ssm_scan_tuning (NULL: every choice from the sizes).
int to_tuning(const ssm_scan_tuning* t, ssm::ScanTuning* out) {
  *out = ssm::ScanTuning{};
  if (!t) return SSM_OK;
  if (t->path != SSM_PATH_AUTO && t->path != SSM_PATH_CHUNKED && t->path != SSM_PATH_SINGLE_PASS) return SSM_ERR_PLAN;
  if (t->min_chunk < 0 || t->target_waves < 0) return SSM_ERR_PLAN;
  out->path = t->path == SSM_PATH_CHUNKED ? ssm::kPathChunked
              : t->path == SSM_PATH_SINGLE_PASS ? ssm::kPathSinglePass : ssm::kPathAuto;
  out->min_chunk = t->min_chunk;
  out->target_waves = t->target_waves;
  return SSM_OK;
}

// Checks the arguments of a forward scan and fills *a and *pl.  Enqueues nothing.
int prepare_scan(const void* u, const void* delta, const float* A, const void* B, const void* C, const float* D,
                 const void* z, const float* delta_bias, int softplus, const float* initial_state, void* y,
                 float* last_state, float* saved, const ssm_scan_tuning* tuning, int64_t b, int64_t L, int64_t E,
                 int64_t N, int dtype, void* stream, ssm::ScanArgs* a, ssm::ScanPlan* pl) {
  int st = check_sizes(b, L, E, N, dtype);
  if (st != SSM_OK) return st;
  ssm::ScanTuning tune;
  st = to_tuning(tuning, &tune);
  if (st != SSM_OK) return st;
  if (b == 0 || E == 0) return SSM_OK;
  if (L > 0 && (!u || !delta || !A || !B || !C || !y)) return SSM_ERR_NULL;
  const size_t es = dtype == SSM_F32 ? 4 : 2;
  const void* streamed[] = {u, delta, B, C, z, y};
  for (const void* p : streamed)
    if (p && !aligned(p, es)) return SSM_ERR_ALIGN;
  const void* fl[] = {A, D, delta_bias, last_state, initial_state};
  for (const void* p : fl)
    if (p && !aligned(p, 4)) return SSM_ERR_ALIGN;
  // the grid of the chunked form is b * ceil(E / 64) * chunks workgroups
  *pl = ssm::plan_scan(b, L, E, int(es), tune);
  int64_t grid = 0;
  if (pl->chunk_len <= 0 || !mul_ok(b * pl->e_blocks, pl->n_chunks, &grid) || grid > INT32_MAX) return SSM_ERR_DIM;
  a->u = u; a->delta = delta; a->A = A; a->B = B; a->C = C; a->D = D; a->z = z; a->bias = delta_bias;
  a->softplus = softplus ? 1 : 0; a->y = y; a->last_state = last_state; a->h0 = initial_state;
  a->saved = saved_count(b, L, E, N) > 0 ? saved : nullptr;
  a->b = b; a->L = L; a->E = E; a->N = N; a->dtype = dtype;
  a->stream = static_cast<hipStream_t>(stream);
  a->tune = tune;
  return SSM_OK;
}

int scan_fwd_impl(const void* u, const void* delta, const float* A, const void* B, const void* C, const float* D,
                  const void* z, const float* delta_bias, int softplus, const float* initial_state, void* y,
                  float* last_state, float* saved, const ssm_scan_tuning* tuning, int64_t b, int64_t L, int64_t E,
                  int64_t N, int dtype, void* stream) {
  ssm::ScanArgs a{};
  ssm::ScanPlan pl{};
  int st = prepare_scan(u, delta, A, B, C, D, z, delta_bias, softplus, initial_state, y, last_state, saved, tuning, b,
                        L, E, N, dtype, stream, &a, &pl);
  if (st != SSM_OK || b == 0 || E == 0) return st;
  if (a.tune.path == ssm::kPathSinglePass && L > 0) {  // asked for explicitly: it has to apply
    int n_cu = 0;
    hipError_t err = ssm::device_cu_count(&n_cu);
    if (err != hipSuccess) return hip_status(err);
    ssm::FusedPlan fp;
    if (ssm::choose_path(a, pl, n_cu, &fp) != ssm::kPathSinglePass) return SSM_ERR_PLAN;
  }
  return hip_status(ssm::launch_scan(a));
}

}  // namespace

extern "C" {

int ssm_state_update(float* state, const void* x, const void* delta, const float* A, const void* B, const void* C,
                     const float* D, const void* z, const float* delta_bias, int softplus, void* y, int64_t b,
                     int64_t E, int64_t N, int dtype, void* stream) {
  int st = check_sizes(b, 1, E, N, dtype);
  if (st != SSM_OK) return st;
  if (b == 0 || E == 0) return SSM_OK;
  if (!state || !x || !delta || !A || !B || !C || !y) return SSM_ERR_NULL;
  const size_t es = dtype == SSM_F32 ? 4 : 2;
  const void* streamed[] = {x, delta, B, C, z, y};
  for (const void* p : streamed)
    if (p && !aligned(p, es)) return SSM_ERR_ALIGN;
  const void* fl[] = {state, A, D, delta_bias};
  for (const void* p : fl)
    if (p && !aligned(p, 4)) return SSM_ERR_ALIGN;
  // one row of workgroups per batch row; channels and lanes use 32-bit indices
  int64_t blocks = 0;
  if (E > (int64_t(1) << 28) || b > INT32_MAX || !mul_ok(b, (E * 4 + 255) / 256, &blocks) || blocks > INT32_MAX)
    return SSM_ERR_DIM;

  ssm::UpdateArgs a;
  a.state = state; a.x = x; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
  a.softplus = softplus ? 1 : 0; a.y = y; a.b = b; a.E = E; a.N = N; a.dtype = dtype;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(ssm::launch_state_update(a));
}

int ssm_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C, const float* D,
                 const void* z, const float* delta_bias, int softplus, const float* initial_state, const void* dy,
                 const float* d_last_state, void* du, void* ddelta, float* dA, float* dB, float* dC, float* dD,
                 void* dz, float* d_delta_bias, float* d_initial_state, int64_t b, int64_t L, int64_t E, int64_t N,
                 int dtype, void* stream) {
  return scan_bwd_impl(u, delta, A, B, C, D, z, delta_bias, softplus, initial_state, nullptr, dy, d_last_state, du,
                       ddelta, dA, dB, dC, dD, dz, d_delta_bias, d_initial_state, b, L, E, N, dtype, stream);
}

int ssm_scan_bwd_saved(const void* u, const void* delta, const float* A, const void* B, const void* C,
                       const float* D, const void* z, const float* delta_bias, int softplus,
                       const float* initial_state, const float* saved_states, const void* dy,
                       const float* d_last_state, void* du, void* ddelta, float* dA, float* dB, float* dC, float* dD,
                       void* dz, float* d_delta_bias, float* d_initial_state, int64_t b, int64_t L, int64_t E,
                       int64_t N, int dtype, void* stream) {
  int st = check_sizes(b, L, E, N, dtype);
  if (st != SSM_OK) return st;
  if (saved_count(b, L, E, N) > 0 && !saved_states) return SSM_ERR_NULL;
  if (saved_states && !aligned(saved_states, 4)) return SSM_ERR_ALIGN;
  return scan_bwd_impl(u, delta, A, B, C, D, z, delta_bias, softplus, initial_state, saved_states, dy, d_last_state,
                       du, ddelta, dA, dB, dC, dD, dz, d_delta_bias, d_initial_state, b, L, E, N, dtype, stream);
}

}  // extern "C"

namespace {

int scan_bwd_impl(const void* u, const void* delta, const float* A, const void* B, const void* C, const float* D,
                  const void* z, const float* delta_bias, int softplus, const float* initial_state,
                  const float* saved, const void* dy, const float* d_last_state, void* du, void* ddelta, float* dA,
                  float* dB, float* dC, float* dD, void* dz, float* d_delta_bias, float* d_initial_state, int64_t b,
                  int64_t L, int64_t E, int64_t N, int dtype, void* stream) {
  int st = check_sizes(b, L, E, N, dtype);
  if (st != SSM_OK) return st;
  int64_t bl = 0, ble = 0;
  if (!mul_ok(b, L, &bl) || !mul_ok(bl, E, &ble)) return SSM_ERR_DIM;
  if (E > 0 && (!A || !dA)) return SSM_ERR_NULL;
  if (bl > 0 && (!dB || !dC)) return SSM_ERR_NULL;
  if (ble > 0 && (!u || !delta || !B || !C || !dy || !du || !ddelta || (z && !dz))) return SSM_ERR_NULL;
  const size_t es = dtype == SSM_F32 ? 4 : 2;
  const void* streamed[] = {u, delta, B, C, z, dy, du, ddelta, dz};
  for (const void* p : streamed)
    if (p && !aligned(p, es)) return SSM_ERR_ALIGN;
  const void* fl[] = {A, D, delta_bias, initial_state, d_last_state, dA, dB, dC, dD, d_delta_bias, d_initial_state};
  for (const void* p : fl)
    if (p && !aligned(p, 4)) return SSM_ERR_ALIGN;
  // a chunk's rows are addressed with 32-bit offsets; grids stay below 2^31 workgroups
  if (E * int64_t(es) * ssm::bwd_chunk_steps() > INT32_MAX) return SSM_ERR_DIM;
  const int64_t chunks = (L + ssm::bwd_chunk_steps() - 1) / ssm::bwd_chunk_steps();
  int64_t grid = 0;
  if (!mul_ok(b, (E + 63) / 64, &grid) || !mul_ok(grid, chunks, &grid) || grid > INT32_MAX) return SSM_ERR_DIM;
  if (b * E * 16 / 256 > INT32_MAX || bl * 32 / 256 > INT32_MAX) return SSM_ERR_DIM;

  ssm::BwdArgs a;
  a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
  a.softplus = softplus ? 1 : 0; a.h0 = initial_state; a.dy = dy; a.dlast = d_last_state;
  a.du = du; a.ddelta = ddelta; a.dA = dA; a.dB = dB; a.dC = dC; a.dD = D ? dD : nullptr; a.dz = z ? dz : nullptr;
  a.dbias = delta_bias ? d_delta_bias : nullptr; a.dh0 = d_initial_state;
  a.saved = saved_count(b, L, E, N) > 0 ? saved : nullptr;
  a.b = b; a.L = L; a.E = E; a.N = N; a.dtype = dtype;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(ssm::launch_scan_bwd(a));
}

}  // namespace

extern "C" {

int ssm_ssd_fwd(const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
                const void* z, const float* delta_bias, int softplus, const float* initial_state, void* y,
                float* last_state, int64_t b, int64_t L, int64_t H, int64_t P, int64_t N, int dtype, void* stream) {
  if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (dtype != SSM_BF16) return SSM_ERR_DTYPE;  // the matrix products take bf16 operands
  if (!size_ok(b) || !size_ok(L) || !size_ok(H) || P != ssm::ssd_head_dim()) return SSM_ERR_DIM;
  if (H > ssm::ssd_max_channels() / P) return SSM_ERR_DIM;
  if (N < 16 || N > 128 || N % 16 != 0) return SSM_ERR_UNSUPPORTED_N;
  int64_t E = 0, t = 0;
  if (!mul_ok(H, P, &E) || !mul_ok(b, L, &t) || !mul_ok(t, E, &t) || !mul_ok(t, 4, &t)) return SSM_ERR_DIM;
  if (!mul_ok(b, E, &t) || !mul_ok(t, N, &t) || !mul_ok(t, 4, &t)) return SSM_ERR_DIM;
  if (b == 0 || H == 0) return SSM_OK;
  if (L > 0 && (!x || !delta || !A || !B || !C || !y)) return SSM_ERR_NULL;
  // rows of x, z, y, B and C are read and written 16 bytes at a time
  const void* vec[] = {x, z, y, B, C};
  for (const void* p : vec)
    if (p && !aligned(p, 16)) return SSM_ERR_ALIGN;
  if (delta && !aligned(delta, 2)) return SSM_ERR_ALIGN;
  const void* fl[] = {A, D, delta_bias, initial_state, last_state};
  for (const void* p : fl)
    if (p && !aligned(p, 4)) return SSM_ERR_ALIGN;
  const int64_t chunks = (L + ssm::ssd_chunk_steps() - 1) / ssm::ssd_chunk_steps();
  int64_t grid = 0;
  if (!mul_ok(b * chunks, H, &grid) || grid > INT32_MAX) return SSM_ERR_DIM;
  if (b * E * N / 256 > INT32_MAX) return SSM_ERR_DIM;
  ssm::SsdArgs a;
  a.x = x; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
  a.softplus = softplus ? 1 : 0; a.h0 = initial_state; a.y = y; a.last_state = last_state;
  a.b = b; a.L = L; a.H = H; a.N = N; a.stream = static_cast<hipStream_t>(stream);
  return hip_status(ssm::launch_ssd(a));
}

int ssm_scan_plan(int64_t b, int64_t L, int64_t E, int64_t N, int dtype, const ssm_scan_tuning* tuning, int* path,
                  int64_t* chunk_len, int64_t* n_chunks) {
  int st = check_sizes(b, L, E, N, dtype);
  if (st != SSM_OK) return st;
  if (!path || !chunk_len || !n_chunks) return SSM_ERR_NULL;
  ssm::ScanTuning tune;
  st = to_tuning(tuning, &tune);
  if (st != SSM_OK) return st;
  const ssm::ScanPlan pl = ssm::plan_scan(b, L, E, dtype == SSM_F32 ? 4 : 2, tune);
  if (pl.chunk_len <= 0) return SSM_ERR_DIM;
  // the single-pass plan depends on the device's CU count (256 on MI355X, taken when no device is visible)
  int n_cu = 0;
  if (ssm::device_cu_count(&n_cu) != hipSuccess || n_cu <= 0) {
    (void)hipGetLastError();
    n_cu = 256;
  }
  ssm::ScanArgs a{};
  a.b = b; a.L = L; a.E = E; a.N = N; a.dtype = dtype; a.tune = tune;
  // the single pass reads 8-byte units: it is planned for 256-byte aligned tensors, as an allocator returns them
  a.u = a.delta = a.B = a.C = a.y = reinterpret_cast<void*>(uintptr_t(256));
  ssm::FusedPlan fp;
  const int form = L > 0 ? ssm::choose_path(a, pl, n_cu, &fp) : ssm::kPathChunked;
  if (form < 0) return SSM_ERR_PLAN;
  if (form == ssm::kPathSinglePass) {
    *path = SSM_PATH_SINGLE_PASS;
    *chunk_len = 8;
    *n_chunks = (L + 7) / 8;
  } else {
    *path = SSM_PATH_CHUNKED;
    *chunk_len = pl.chunk_len;
    *n_chunks = pl.n_chunks;
  }
  return SSM_OK;
}

int ssm_conv_fwd(const void* v, const float* q, const float* conv_bias, const void* state_in, void* x,
                 void* state_out, int64_t b, int64_t L, int64_t E, int64_t K, int dtype, void* stream) {
  if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (!size_ok(b) || !size_ok(L) || !size_ok(E) || K < 1 || K > ssm::kMaxConvK) return SSM_ERR_DIM;
  int64_t t = 0;
  if (!mul_ok(b, L, &t) || !mul_ok(t, E, &t) || !mul_ok(t, 4, &t)) return SSM_ERR_DIM;
  if (!mul_ok(b, E, &t) || !mul_ok(t, K, &t) || !mul_ok(t, 4, &t)) return SSM_ERR_DIM;
  if (b == 0 || E == 0) return SSM_OK;
  if ((L > 0 && (!v || !x)) || !q) return SSM_ERR_NULL;
  const size_t es = dtype == SSM_F32 ? 4 : 2;
  const void* streamed[] = {v, x, state_in, state_out};
  for (const void* p : streamed)
    if (p && !aligned(p, es)) return SSM_ERR_ALIGN;
  if (!aligned(q, 4) || (conv_bias && !aligned(conv_bias, 4))) return SSM_ERR_ALIGN;
  // one wave covers 64 channels of a conv_chunk_steps() row band; offsets inside it are 32-bit
  const int64_t e_blocks = (E + 63) / 64, chunks = (L + ssm::conv_chunk_steps() - 1) / ssm::conv_chunk_steps();
  if (E * int64_t(es) * ssm::conv_chunk_steps() > INT32_MAX) return SSM_ERR_DIM;
  int64_t grid = 0;
  if (!mul_ok(b, e_blocks, &grid) || !mul_ok(grid, chunks, &grid) || grid > INT32_MAX) return SSM_ERR_DIM;
  ssm::ConvArgs a;
  a.v = v; a.q = q; a.cb = conv_bias; a.state_in = state_in; a.x = x; a.state_out = state_out;
  a.b = b; a.L = L; a.E = E; a.K = K; a.dtype = dtype; a.stream = static_cast<hipStream_t>(stream);
  return hip_status(ssm::launch_conv_fwd(a));
}

int ssm_conv_update(void* conv_state, const void* v, const float* q, const float* conv_bias, void* x, int64_t b,
                    int64_t E, int64_t K, int dtype, void* stream) {
  if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (!size_ok(b) || !size_ok(E) || K < 1 || K > ssm::kMaxConvK) return SSM_ERR_DIM;
  int64_t t = 0;
  if (!mul_ok(b, E, &t) || !mul_ok(t, K, &t) || !mul_ok(t, 4, &t)) return SSM_ERR_DIM;
  if (b == 0 || E == 0) return SSM_OK;
  if (!conv_state || !v || !q || !x) return SSM_ERR_NULL;
  const size_t es = dtype == SSM_F32 ? 4 : 2;
  const void* streamed[] = {conv_state, v, x};
  for (const void* p : streamed)
    if (!aligned(p, es)) return SSM_ERR_ALIGN;
  if (!aligned(q, 4) || (conv_bias && !aligned(conv_bias, 4))) return SSM_ERR_ALIGN;
  int64_t blocks = 0;
  if (E > INT32_MAX || b > INT32_MAX || !mul_ok(b, (E + 255) / 256, &blocks) || blocks > INT32_MAX) return SSM_ERR_DIM;
  ssm::ConvArgs a;
  a.v = v; a.q = q; a.cb = conv_bias; a.state_in = nullptr; a.x = x; a.state_out = conv_state;
  a.b = b; a.L = 1; a.E = E; a.K = K; a.dtype = dtype; a.stream = static_cast<hipStream_t>(stream);
  return hip_status(ssm::launch_conv_update(a));
}

const char* ssm_status_string(int status) {
  switch (status) {
    case SSM_OK: return "ok";
    case SSM_ERR_NULL: return "a required pointer is NULL";
    case SSM_ERR_DIM: return "invalid or overflowing size";
    case SSM_ERR_DTYPE: return "unknown dtype";
    case SSM_ERR_UNSUPPORTED_N:
      return "state size N outside the entry point's range (1..16; ssm_ssd_fwd: 16..128 in steps of 16)";
    case SSM_ERR_PLAN: return "the requested scan form or tuning does not apply to this call";
    case SSM_ERR_SCRATCH:
      return "the call needs more workspace than the fixed buffer of ssm_scan_fwd_noalloc holds "
             "(SSM_NOALLOC_SCRATCH_BYTES)";
    case SSM_ERR_ALIGN: return "array not aligned to its element size";
    case SSM_ERR_HIP: return "HIP launch or allocation failed";
    default: return "unknown status";
  }
}

const char* ssm_last_hip_error(void) { return g_last_hip_error; }

int ssm_version(void) { return 10000; }

}  // extern "C"
