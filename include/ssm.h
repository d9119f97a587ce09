/*
 * ssm.h -- C ABI of the MI355X (gfx950) selective-scan library (libssm.so).
 *
 * The Mamba-1 (S6) selective state-space operation and the steps around it,
 * on one GPU:
 *
 *   ssm_scan_fwd, ssm_scan_fwd_from   the selective scan over a whole sequence
 *                                     (from zero, or from a given state)
 *   ssm_state_update                  one recurrent step of the same recurrence (generation)
 *   ssm_scan_bwd                      the gradients of the scan
 *   ssm_scan_fwd_save, ssm_scan_bwd_saved
 *                                     the training form: the forward keeps the state
 *                                     every SSM_SAVE_INTERVAL steps for the backward
 *   ssm_scan_fwd_tuned                the forward with its form and split chosen by the caller
 *   ssm_scan_fwd_noalloc              the forward for callers that cannot allocate device memory
 *   ssm_ssd_fwd                       the scan with a scalar transition per head
 *   ssm_conv_fwd, ssm_conv_update     the causal depthwise convolution + SiLU before
 *                                     the scan, and its token step
 *   ssm_scan_plan, ssm_profile_*, ssm_status_string, ssm_last_hip_error, ssm_version
 *                                     host-side queries
 *
 * Pages that define the operations (title, site):
 *   [KK] "mamba, from scratch" (khushi keswani)
 *   [AB] "Mamba: Linear-Time Sequence Modeling with Selective State Spaces" (abhik.ai)
 *   [NC] "Mamba: Linear-Time Sequence Modeling with Selective State Spaces"
 *        (nadeemcite research-papers summary)
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 * Memory.  Every pointer is a DEVICE pointer on the current HIP device, owned
 * by the caller.  Arrays are dense, row-major (last index fastest).  The
 * library keeps no pointer after a call returns.
 *
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the default
 * stream).  Work is enqueued on it and the call returns without waiting;
 * errors raised while the kernels run surface at the caller's next
 * synchronisation.  A forward scan in the single-pass form, or in one chunk,
 * takes no workspace.  A forward scan cut into chunks (chunked form), the
 * backward and the per-head scan take a temporary workspace from the
 * stream-ordered allocator (hipMallocAsync / hipFreeAsync on `stream`), so
 * concurrent calls on different streams do not share memory.
 * ssm_state_update and ssm_conv_update take none and issue no memset: a
 * caller can capture them in a HIP graph.
 *
 * Data types.  `dtype` (ssm_dtype) is the element type of the streamed
 * tensors u/x, delta, B, C, z and y: SSM_F32 (float) or SSM_BF16 (bfloat16,
 * raw 16-bit storage).  A, D, delta_bias and every state are always float.
 * Arithmetic is float32 throughout; bf16 outputs are rounded to nearest-even.
 *
 * Sizes.  b (batch), L (sequence length), E (expanded channels) and
 * N (state size per channel).  Supported: 1 <= N <= 16 (ssm_ssd_fwd: N a
 * multiple of 16 up to 128); 0 <= b, L, E <= 2^48.  b == 0 or E == 0 is a no-op.
 * L == 0 writes a zero last_state (or the incoming state, where one is given).
 *
 * Alignment.  Every array must be aligned to its element size; float arrays
 * to 4 bytes, bf16 arrays to 2 bytes.  (Tensors from a PyTorch allocator
 * always are.)
 *
 * Aliasing.  Outputs must not overlap inputs.
 *
 * Errors.  Argument errors are detected before anything is enqueued and
 * reported as a negative ssm_status; nothing is written in that case.
 * SSM_ERR_HIP reports a failed HIP launch or allocation (the HIP error is
 * cleared and its text is available from ssm_last_hip_error()).
 */
#ifndef SSM_H_
#define SSM_H_

#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define SSM_API __attribute__((visibility("default")))
#else
#define SSM_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSM_F32 = 0,
  SSM_BF16 = 1
} ssm_dtype;

typedef enum {
  SSM_OK = 0,
  SSM_ERR_NULL = -1,          /* a required pointer is NULL */
  SSM_ERR_DIM = -2,           /* a negative size, a size above 2^48, or a size product that overflows */
  SSM_ERR_DTYPE = -3,         /* dtype is not an ssm_dtype value */
  SSM_ERR_UNSUPPORTED_N = -4, /* N outside the supported range (1..16; ssm_ssd_fwd: 16..128 in steps of 16) */
  SSM_ERR_ALIGN = -5,         /* an array is not aligned to its element size */
  SSM_ERR_HIP = -6,           /* HIP launch / allocation failure */
  SSM_ERR_PLAN = -7,          /* an ssm_scan_tuning value is invalid or does not apply to the call */
  SSM_ERR_SCRATCH = -8        /* ssm_scan_fwd_noalloc: the call needs more than SSM_NOALLOC_SCRATCH_BYTES */
} ssm_status;

/*
 * Selective scan, forward.
 *
 * For every batch row b, channel e and state n, starting from h = 0:
 *   d      = delta[b,t,e] + delta_bias[e], then softplus(d) when softplus != 0
 *            (bias added before the softplus: [NC] "Core Idea"; [KK] "from ssm
 *            to selective ssm")
 *   h[n]   = exp(d * A[e,n]) * h[n] + d * B[b,t,n] * u[b,t,e]
 *            (retention exp(step*A) and write step*B*x: [AB] "Original paper,
 *            equations and runnable CPU code", row 2 "Retain, write and read
 *            each channel's state"; the write is not the exact zero-order-hold
 *            integral)
 *   y[b,t,e] = (sum_n C[b,t,n] * h[n] + D[e] * u[b,t,e]) * silu(z[b,t,e])
 *            (read after the update, direct D*x path: same row 2; silu gate:
 *            [AB] row 5 "Put the selective operator inside the complete mixer")
 *   last_state[b,e,n] = h[n] after step L-1
 * The recurrence is an associative affine composition
 * ([KK] "the scan"; [AB] "Compose the updates instead of waiting for every
 * state"), which is how the library splits long sequences across the GPU.
 *
 * Arguments (all device pointers):
 *   u, delta, z, y   [b, L, E]  dtype       (z nullable: no gate)
 *   A                [E, N]     float       (used as given; the usual
 *                                            parameterisation is A = -exp(A_log))
 *   B, C             [b, L, N]  dtype       (shared by all E channels)
 *   D, delta_bias    [E]        float       (nullable: treated as zero)
 *   softplus         0 or 1
 *   last_state       [b, E, N]  float       (nullable: not written)
 */
SSM_API int ssm_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                 const float* D, const void* z, const float* delta_bias, int softplus,
                 void* y, float* last_state,
                 int64_t b, int64_t L, int64_t E, int64_t N, int dtype, void* stream);

/*
 * Selective scan that continues from a given state: identical to
 * ssm_scan_fwd except that the recurrence starts from initial_state
 * [b, E, N] (float, device; NULL means zero) instead of zero.  An optional
 * incoming state is part of the recurrence's definition ([AB] row 2: the loop
 * continues an earlier prefix), so
 *   scan(L1 + L2) == scan(L2, initial_state = last_state of scan(L1))
 * and a prefill can hand its state to ssm_state_update for decoding.
 * With L == 0, last_state receives a copy of initial_state.
 * initial_state must not overlap last_state (or any other output).
 */
SSM_API int ssm_scan_fwd_from(const void* u, const void* delta, const float* A, const void* B, const void* C,
                              const float* D, const void* z, const float* delta_bias, int softplus,
                              const float* initial_state, void* y, float* last_state,
                              int64_t b, int64_t L, int64_t E, int64_t N, int dtype, void* stream);

/*
 * Interval of the states saved by ssm_scan_fwd_save: the backward's chunk.
 */
#define SSM_SAVE_INTERVAL 64

/*
 * ssm_scan_fwd_from that also saves the state at every SSM_SAVE_INTERVAL-th
 * step, for ssm_scan_bwd_saved.  The backward recomputes the states inside its
 * 64-step chunks from the state entering each chunk; taking those boundary
 * states from the forward spares it a pass over the sequence.  Only the
 * boundaries are kept (1/64 of the [b, L, E, N] states), in line with keeping
 * the expanded state on chip and recomputing intermediates in the backward
 * ("Mamba: Linear-Time Sequence Modeling with Selective State Spaces",
 * abhik.ai, "Compose the updates instead of waiting for every state").
 *
 * saved_states  [b, K, E, N] float (device), K = ceil(L / 64) - 1 (0 when
 *               L <= 64; then it may be NULL): saved_states[bi, k, e, n] is
 *               the state h[n] of (bi, e) after step 64 (k + 1) - 1, i.e. the
 *               state entering step 64 (k + 1).  Written fully; must not
 *               overlap any other argument.
 * Everything else, and the results y and last_state, as ssm_scan_fwd_from.
 * Errors: SSM_ERR_NULL when K > 0 and saved_states is NULL; SSM_ERR_ALIGN
 * when it is not 4-byte aligned; otherwise as ssm_scan_fwd_from.
 */
SSM_API int ssm_scan_fwd_save(const void* u, const void* delta, const float* A, const void* B, const void* C,
                              const float* D, const void* z, const float* delta_bias, int softplus,
                              const float* initial_state, void* y, float* last_state, float* saved_states,
                              int64_t b, int64_t L, int64_t E, int64_t N, int dtype, void* stream);

/*
 * Forms of the forward scan (ssm_scan_tuning.path, ssm_scan_plan).
 *   SSM_PATH_CHUNKED      the sequence is cut into chunks when batch x channels
 *                         alone cannot fill the GPU: a pass computes each
 *                         chunk's map from zero, a chain composes the maps
 *                         ([KK] "the scan"), a main pass rescans every chunk
 *                         from its incoming state; one chunk is a single pass.
 *   SSM_PATH_SINGLE_PASS  a workgroup walks the whole sequence for a slice of
 *                         channels; chunks of 8 steps are run from zero, their
 *                         maps chained through LDS and replayed from registers,
 *                         so every input is read once and every retention
 *                         exponential is evaluated once.
 * SSM_PATH_AUTO takes the single pass where the sequence has to be cut and the
 * chain of chunk maps per workgroup block stays short, else the chunked form.
 */
typedef enum {
  SSM_PATH_AUTO = 0,
  SSM_PATH_CHUNKED = 1,
  SSM_PATH_SINGLE_PASS = 2
} ssm_scan_path;

/*
 * Plan choices of a forward scan.  Zero fields leave the choice to the sizes.
 *   path          an ssm_scan_path value
 *   min_chunk     chunked form: shortest chunk, in steps (> 0 to set it)
 *   target_waves  chunked form: the waves the cut aims for; the sequence is cut
 *                 while b * ceil(E / 64) * 2 is below it (> 0 to set it)
 * The choices change the order of the floating-point operations, not the
 * definition computed.
 */
typedef struct {
  int32_t path;
  int32_t min_chunk;
  int32_t target_waves;
} ssm_scan_tuning;

/*
 * ssm_scan_fwd_save with explicit plan choices.  tuning may be NULL (every
 * choice from the sizes, as ssm_scan_fwd_save); saved_states may be NULL (not
 * saved, as ssm_scan_fwd_from); initial_state may be NULL (zero).
 * Errors: SSM_ERR_PLAN when a tuning field is out of range or path is
 * SSM_PATH_SINGLE_PASS and the single pass does not apply (its tiles need the
 * rows of u, delta, z, y, B and C to be whole 8-byte units and 8-byte aligned
 * tensors, and enough channels per compute unit); otherwise as
 * ssm_scan_fwd_save.
 */
SSM_API int ssm_scan_fwd_tuned(const void* u, const void* delta, const float* A, const void* B, const void* C,
                               const float* D, const void* z, const float* delta_bias, int softplus,
                               const float* initial_state, void* y, float* last_state, float* saved_states,
                               const ssm_scan_tuning* tuning, int64_t b, int64_t L, int64_t E, int64_t N, int dtype,
                               void* stream);

/*
 * Size of the fixed device buffer of ssm_scan_fwd_noalloc (128 MiB).
 */
#define SSM_NOALLOC_SCRATCH_BYTES (128ll << 20)

/*
 * ssm_scan_fwd_from for callers that cannot allocate device memory: code
 * under HIP graph capture, serving loops, harnesses that forbid hipMalloc.
 * It runs the same plan as ssm_scan_fwd_from (same kernels, same results),
 * but a scan in the chunked form cut into several chunks takes its workspace
 * (chunk aggregates, chunk step sums, float copies of bf16 B / C rows) from a
 * buffer of SSM_NOALLOC_SCRATCH_BYTES that the library holds in device memory
 * on every GPU it runs on until the process ends; no call allocates or frees
 * device memory.  The single-pass form and one-chunk scans need no workspace.
 *
 * The buffer is shared by every call on one GPU and keeps the last call's
 * contents (no call reads a part of it before writing that part): calls on one
 * GPU whose executions overlap (different streams, or threads enqueueing
 * concurrently without ordering their streams) race on it and must be
 * serialised by the caller.
 *
 * Arguments, results and errors as ssm_scan_fwd_from, plus SSM_ERR_SCRATCH
 * when the plan's workspace exceeds SSM_NOALLOC_SCRATCH_BYTES (then nothing
 * is enqueued).  At the long-sequence size (b1 L65536 E5120 N16 bf16) the
 * workspace is 98 MB.
 */
SSM_API int ssm_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B, const void* C,
                                 const float* D, const void* z, const float* delta_bias, int softplus,
                                 const float* initial_state, void* y, float* last_state, int64_t b, int64_t L,
                                 int64_t E, int64_t N, int dtype, void* stream);

/*
 * One recurrent step for every (b, e) -- the SSM half of the decode step of
 * [AB] row 6 "Carry both buffers to the next token":
 *   d          = delta[b,e] + delta_bias[e], softplus(d) when softplus != 0
 *   state[b,e,n] = exp(d * A[e,n]) * state[b,e,n] + d * B[b,n] * x[b,e]   (in place)
 *   y[b,e]     = (sum_n C[b,n] * state[b,e,n] + D[e] * x[b,e]) * silu(z[b,e])
 *
 * Arguments (all device pointers):
 *   state            [b, E, N]  float       (read and written in place)
 *   x, delta, z, y   [b, E]     dtype       (z nullable)
 *   A                [E, N]     float
 *   B, C             [b, N]     dtype
 *   D, delta_bias    [E]        float       (nullable)
 * Calling it L times on the token slices of a sequence reproduces
 * ssm_scan_fwd (same recurrence, [AB] "What persists when the next token
 * arrives").
 */
SSM_API int ssm_state_update(float* state, const void* x, const void* delta, const float* A,
                     const void* B, const void* C, const float* D, const void* z,
                     const float* delta_bias, int softplus, void* y,
                     int64_t b, int64_t E, int64_t N, int dtype, void* stream);

/*
 * Backward of the scan: gradients of
 *   loss = sum dy[b,t,e] * y[b,t,e] + sum d_last_state[b,e,n] * last_state[b,e,n]
 * with respect to every input of ssm_scan_fwd_from.  The gradients are the
 * chain rule of the forward definition above; the states are recomputed from
 * per-chunk incoming states instead of being stored ("Mamba: Linear-Time
 * Sequence Modeling with Selective State Spaces", nadeemcite summary, "Core
 * Idea"; abhik.ai page, "Compose the updates instead of waiting for every
 * state").
 *
 * Inputs: the forward's arguments (same layouts and dtypes; initial_state
 * nullable = zero), dy [b, L, E] (dtype), d_last_state [b, E, N] float
 * (nullable = zero).
 * Outputs (device pointers, fully overwritten, never accumulated into):
 *   du, ddelta      [b, L, E]  dtype
 *   dz              [b, L, E]  dtype   (required when z is given, ignored otherwise)
 *   dA              [E, N]     float
 *   dB, dC          [b, L, N]  float   (sums over the channels)
 *   dD              [E]        float   (nullable; written when D is given)
 *   d_delta_bias    [E]        float   (nullable; written when delta_bias is given)
 *   d_initial_state [b, E, N]  float   (nullable; the gradient reaching the
 *                                       initial state, also when it is zero)
 * ddelta is the gradient with respect to the raw step (before bias and softplus).
 * Results are deterministic: every sum over chunks or channel blocks is added
 * in a fixed order.  The call takes a workspace of about
 * 1.3 * b * L * E + 34 * b * L floats from the stream-ordered allocator on
 * `stream`.  Sizes: 64 * E * sizeof(dtype) < 2^31.
 */
SSM_API int ssm_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                         const float* D, const void* z, const float* delta_bias, int softplus,
                         const float* initial_state, const void* dy, const float* d_last_state, void* du,
                         void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz, float* d_delta_bias,
                         float* d_initial_state, int64_t b, int64_t L, int64_t E, int64_t N, int dtype,
                         void* stream);

/*
 * ssm_scan_bwd with the states entering its chunks taken from saved_states
 * (the output of ssm_scan_fwd_save on the same inputs and initial_state:
 * [b, K, E, N] float, K = ceil(L / 64) - 1, read only) instead of being
 * recomputed.  Same outputs as ssm_scan_bwd up to rounding (the forward's
 * states are the same recurrence evaluated over its own chunks); the
 * workspace shrinks by the recomputed states.  Errors: SSM_ERR_NULL when
 * K > 0 and saved_states is NULL; SSM_ERR_ALIGN when it is not 4-byte
 * aligned; otherwise as ssm_scan_bwd.
 */
SSM_API int ssm_scan_bwd_saved(const void* u, const void* delta, const float* A, const void* B, const void* C,
                               const float* D, const void* z, const float* delta_bias, int softplus,
                               const float* initial_state, const float* saved_states, const void* dy,
                               const float* d_last_state, void* du, void* ddelta, float* dA, float* dB, float* dC,
                               float* dD, void* dz, float* d_delta_bias, float* d_initial_state, int64_t b,
                               int64_t L, int64_t E, int64_t N, int dtype, void* stream);

/*
 * The scan with a scalar transition per head -- structured state-space
 * duality -- computed in chunks of matrix products on the MFMA units ("Mamba:
 * Linear-Time Sequence Modeling with Selective State Spaces", abhik.ai, "Key
 * takeaways" / "Related reading": a restricted state update becomes a
 * structured mixing matrix computed in chunks; "mamba-from-scratch" README,
 * Mamba-2 / SSD).  The result is ssm_scan_fwd_from's for E = H * P channels
 * where channel e = h * P + p uses the head's step delta[b,t,h], A[h] (the same
 * for every state), D[h] and delta_bias[h]:
 *   y[t,e] = sum_{s<=t} (C_t . B_s) exp(A_h (S_t - S_s)) d_s x[s,e] + D_h x[t,e]
 *            (+ the initial state's part), times silu(z[t,e]);  S_t = d_0 + ... + d_t
 *
 * Arguments (device pointers):
 *   x, z, y         [b, L, H*P]  bf16   (z nullable; x, z, y 16-byte aligned)
 *   delta           [b, L, H]    bf16
 *   A, D, delta_bias [H]         float  (D, delta_bias nullable)
 *   B, C            [b, L, N]    bf16   (16-byte aligned)
 *   initial_state, last_state [b, H*P, N] float (nullable)
 *   P == 64; N a multiple of 16 in 16..128 (else SSM_ERR_DIM / SSM_ERR_UNSUPPORTED_N);
 *   H * P at most 8,323,520 channels, H <= 130,055 (a chunk's rows are addressed with 32-bit
 *   offsets; larger returns SSM_ERR_DIM);
 *   dtype must be SSM_BF16 (the matrix products take bf16 operands and
 *   accumulate in fp32; SSM_F32 returns SSM_ERR_DTYPE).
 * Takes a workspace from the stream-ordered allocator on `stream`: with
 * C = ceil(L/128) chunks and S = ceil(C/8) segments, b * C * H * 64 * N bf16
 * values (each chunk's state from inside its segment), b * C * H floats, and
 * b * S * H * (64 * N + 1) floats (the segment states and their decays).
 */
SSM_API int ssm_ssd_fwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                        const float* D, const void* z, const float* delta_bias, int softplus,
                        const float* initial_state, void* y, float* last_state, int64_t b, int64_t L, int64_t H,
                        int64_t P, int64_t N, int dtype, void* stream);

/*
 * Causal depthwise convolution + SiLU, the step before the scan in the Mamba
 * block ([AB] row 4 "Add causal local context before selecting coefficients"):
 *   x[b,t,c] = silu(conv_bias[c] + sum_{k=0..K-1} q[c,k] * v[b, t-K+1+k, c])
 * Samples before t = 0 come from state_in (the K most recent earlier samples,
 * oldest first) or are zero when state_in is NULL (left zero padding).
 *
 * Arguments (device pointers):
 *   v, x             [b, L, E]  dtype       (x must not overlap v)
 *   q                [E, K]     float       (a depthwise Conv1d weight [E, 1, K])
 *   conv_bias        [E]        float       (nullable: zero)
 *   state_in         [b, E, K]  dtype       (nullable)
 *   state_out        [b, E, K]  dtype       (nullable): the K most recent samples after the
 *                                            last step, oldest first -- the state
 *                                            ssm_conv_update continues from
 *   1 <= K <= 8.  L == 0 copies state_in (or zeros) to state_out.
 */
SSM_API int ssm_conv_fwd(const void* v, const float* q, const float* conv_bias, const void* state_in, void* x,
                         void* state_out, int64_t b, int64_t L, int64_t E, int64_t K, int dtype, void* stream);

/*
 * One token of the convolution ([AB] row 6 "Carry both buffers to the next
 * token"): conv_state [b, E, K] (dtype, in place) is shifted left by one
 * sample and v [b, E] is appended; then
 *   x[b,c] = silu(conv_bias[c] + sum_k q[c,k] * conv_state[b,c,k]).
 * Calling it L times reproduces ssm_conv_fwd over the L tokens.
 */
SSM_API int ssm_conv_update(void* conv_state, const void* v, const float* q, const float* conv_bias, void* x,
                            int64_t b, int64_t E, int64_t K, int dtype, void* stream);

/*
 * How a forward scan of this size runs (tuning NULL: as ssm_scan_fwd): *path
 * receives SSM_PATH_CHUNKED or SSM_PATH_SINGLE_PASS, *chunk_len and *n_chunks
 * the chunks (single pass: chunks of 8 steps; chunked form: one chunk means a
 * single pass over each channel, more chunks the aggregate, carry and main
 * passes).  The plan assumes 256-byte aligned tensors (as allocators return
 * them) and the current device's CU count (256, MI355X, when no device is
 * visible).  Host-only: enqueues nothing.  Same argument checks as
 * ssm_scan_fwd_tuned.
 */
SSM_API int ssm_scan_plan(int64_t b, int64_t L, int64_t E, int64_t N, int dtype, const ssm_scan_tuning* tuning,
                          int* path, int64_t* chunk_len, int64_t* n_chunks);

/*
 * Kernel timing for benchmarks.  While enabled (on != 0), every kernel the
 * library enqueues is bracketed by two HIP events recorded on the caller's
 * stream.  ssm_profile_read() waits for those events, writes per-kind totals
 * (milliseconds) and launch counts for kinds 0 .. n_kinds-1 and clears the
 * record.  Kinds: 0 chunk_aggregate, 1 chunk_carry, 2 scan_main,
 * 3 fill_state, 4 state_update, 5 conv, 6 conv_update, 7 bwd_rows,
 * 8 bwd_aggregate (the backward's per-chunk maps: with no saved states the
 * forward and the reverse ones from one walk, whose forward chain is timed as
 * chunk_carry), 9 bwd_carry, 10 bwd_main, 11 bwd_reduce, 12 ssd_state,
 * 13 ssd_carry, 14 ssd_scan, 15 scan_fused (the single-pass forward),
 * 16 widen_rows (float copies of the bf16 B / C rows of a cut forward); names
 * from ssm_profile_kind_name().  Off by default; the events add a few
 * microseconds per launch.  Process-wide, thread-safe.
 */
SSM_API int ssm_profile_enable(int on);
SSM_API int ssm_profile_read(double* total_ms, int64_t* launches, int n_kinds);
SSM_API const char* ssm_profile_kind_name(int kind);

/* Static text for an ssm_status value (never NULL). */
SSM_API const char* ssm_status_string(int status);

/* Text of the last HIP error that produced SSM_ERR_HIP in this thread ("" if none). */
SSM_API const char* ssm_last_hip_error(void);

/* Library version as major*10000 + minor*100 + patch. */
SSM_API int ssm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSM_H_ */
