/*
 * ssm_oracle.c -- plain, sequential, double-precision CPU reference of the
 * Mamba-1 (S6) selective scan, its backward (gradients of every input), its
 * single-token recurrent state update, and the causal convolution before it.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness oracle for the GPU
 * library.  Only the test suite, the package's smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, table or helper
 * with the GPU path, and the GPU path never calls it.
 *
 * Pages cited (title, site):
 *   [KK] "mamba, from scratch" (khushi keswani)
 *   [AB] "Mamba: Linear-Time Sequence Modeling with Selective State Spaces" (abhik.ai)
 *   [NC] "Mamba: Linear-Time Sequence Modeling with Selective State Spaces"
 *        (nadeemcite research-papers summary)
 *
 * What is computed, for every batch row b and expanded channel e, with a state
 * vector h[0..N-1] that starts at zero (or at a given h0):
 *
 *   d_t     = delta[b,t,e] + bias[e]                 bias added before the
 *             then softplus(d_t) if requested         softplus ([NC] "Core Idea":
 *                                                     the step is the softplus of a
 *                                                     parameter plus a projection;
 *                                                     [KK] "from ssm to selective ssm")
 *   a_t,n   = exp(d_t * A[e,n])                       retention ([AB] "The input
 *                                                     changes the coefficients";
 *                                                     [KK] "from ssm to selective ssm")
 *   h_t,n   = a_t,n * h_{t-1},n + d_t * B[b,t,n] * u[b,t,e]
 *             (write term is step * B * x, not the exact zero-order-hold
 *             integral: [AB] "Original paper, equations and runnable CPU code",
 *             row 2 "Retain, write and read each channel's state")
 *   y[b,t,e] = sum_n C[b,t,n] * h_t,n + D[e] * u[b,t,e]
 *             (read after the update, then the direct D*x path: same row 2)
 *   y[b,t,e] *= silu(z[b,t,e]) = z / (1 + exp(-z))   when a gate is given
 *             ([AB] row 5 "Put the selective operator inside the complete
 *             mixer": the z branch multiplies the scan result through SiLU)
 *   last_state[b,e,n] = h_{L-1},n
 *
 * The single-token update applies the same body once to a given state
 * ([AB] row 6 "Carry both buffers to the next token", the SSM half of `step`).
 *
 * The causal depthwise convolution that precedes the scan in the block
 * ([AB] row 4 "Add causal local context before selecting coefficients"):
 *   x[b,t,c] = silu(cb[c] + sum_{k=0..K-1} q[c,k] * v[b, t-K+1+k, c])
 * with samples before t = 0 taken from an incoming convolution state
 * (the K most recent earlier samples, oldest first) or zero (left padding).
 * Its single-token form shifts the K-sample state left by one, appends the
 * new sample and evaluates the same sum ([AB] row 6, the convolution half).
 *
 * Arithmetic: every input is widened to double before use; exp/log1p come
 * from the C library; there is no blocking, fusion or reordering of the
 * definition above.  Chains (b,e) are independent, so threads split chains,
 * never time.  Build without -ffast-math and with floating-point contraction
 * off so the arithmetic is the plain definition.
 */
#include <math.h>
#include <pthread.h>

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* softplus(x) = log(1 + e^x), written so neither branch overflows. */
static double oracle_softplus(double x) {
  if (x > 0.0) return x + log1p(exp(-x));
  return log1p(exp(x));
}

/* silu(z) = z * sigmoid(z) = z / (1 + e^{-z}). */
static double oracle_silu(double z) {
  return z / (1.0 + exp(-z));
}

typedef struct {
  const double *u, *delta, *A, *B, *C, *D, *z, *bias, *h0;
  double *y, *last_state, *states;
  int64_t b, L, E, N;
  int softplus;
  int64_t chain_begin, chain_end; /* chains are flattened (b, e) */
} scan_job;

static void scan_chain(const scan_job* j, int64_t bi, int64_t e, double* h) {
  const int64_t L = j->L, E = j->E, N = j->N;
  for (int64_t n = 0; n < N; n++) h[n] = j->h0 ? j->h0[(bi * E + e) * N + n] : 0.0;
  for (int64_t t = 0; t < L; t++) {
    const int64_t xe = (bi * L + t) * E + e; /* index into [b, L, E] */
    const int64_t xn = (bi * L + t) * N;     /* row index into [b, L, N] */
    const double x = j->u[xe];
    double d = j->delta[xe] + (j->bias ? j->bias[e] : 0.0);
    if (j->softplus) d = oracle_softplus(d);
    double acc = 0.0;
    for (int64_t n = 0; n < N; n++) {
      const double a = exp(d * j->A[e * N + n]);
      const double w = d * j->B[xn + n] * x;
      h[n] = a * h[n] + w;
      acc += j->C[xn + n] * h[n];
      if (j->states) j->states[((bi * L + t) * E + e) * N + n] = h[n];
    }
    double yv = acc + (j->D ? j->D[e] * x : 0.0);
    if (j->z) yv *= oracle_silu(j->z[xe]);
    j->y[xe] = yv;
  }
  if (j->last_state)
    for (int64_t n = 0; n < N; n++) j->last_state[(bi * E + e) * N + n] = h[n];
}

static void* scan_worker(void* arg) {
  const scan_job* j = (const scan_job*)arg;
  double* h = (double*)malloc(sizeof(double) * (size_t)(j->N > 0 ? j->N : 1));
  if (!h) return (void*)1;
  for (int64_t c = j->chain_begin; c < j->chain_end; c++) scan_chain(j, c / j->E, c % j->E, h);
  free(h);
  return NULL;
}

/* Returns 0 on success, -1 on bad arguments, -2 on allocation/thread failure. */
int oracle_scan(const double* u, const double* delta, const double* A, const double* B, const double* C,
                const double* D, const double* z, const double* delta_bias, int softplus, const double* h0,
                double* y, double* last_state, double* states, int64_t b, int64_t L, int64_t E, int64_t N,
                int threads) {
  if (b < 0 || L < 0 || E < 0 || N < 0) return -1;
  if ((L > 0 && (!u || !delta || !B || !C || !y)) || (N > 0 && E > 0 && !A)) return -1;
  const int64_t chains = b * E;
  if (chains == 0) return 0;
  if (threads < 1) threads = 1;
  if (threads > chains) threads = (int)chains;
  scan_job base;
  memset(&base, 0, sizeof base);
  base.u = u; base.delta = delta; base.A = A; base.B = B; base.C = C; base.D = D; base.z = z;
  base.bias = delta_bias; base.h0 = h0; base.y = y; base.last_state = last_state; base.states = states;
  base.b = b; base.L = L; base.E = E; base.N = N; base.softplus = softplus;
  scan_job* jobs = (scan_job*)malloc(sizeof(scan_job) * (size_t)threads);
  pthread_t* tid = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)threads);
  if (!jobs || !tid) { free(jobs); free(tid); return -2; }
  int rc = 0, started = 0;
  for (int i = 0; i < threads; i++) {
    jobs[i] = base;
    jobs[i].chain_begin = chains * i / threads;
    jobs[i].chain_end = chains * (i + 1) / threads;
    if (threads == 1) {
      if (scan_worker(&jobs[i])) rc = -2;
    } else if (pthread_create(&tid[i], NULL, scan_worker, &jobs[i]) != 0) {
      rc = -2;
      break;
    } else {
      started++;
    }
  }
  for (int i = 0; i < started; i++) {
    void* ret = NULL;
    pthread_join(tid[i], &ret);
    if (ret) rc = -2;
  }
  free(jobs);
  free(tid);
  return rc;
}

typedef struct {
  double* state;
  const double *x, *delta, *A, *B, *C, *D, *z, *bias;
  double* y;
  int64_t b, E, N;
  int softplus;
  int64_t chain_begin, chain_end;
} update_job;

static void* update_worker(void* arg) {
  const update_job* j = (const update_job*)arg;
  const int64_t E = j->E, N = j->N;
  for (int64_t c = j->chain_begin; c < j->chain_end; c++) {
    const int64_t bi = c / E, e = c % E;
    const double x = j->x[c];
    double d = j->delta[c] + (j->bias ? j->bias[e] : 0.0);
    if (j->softplus) d = oracle_softplus(d);
    double acc = 0.0;
    for (int64_t n = 0; n < N; n++) {
      double* s = &j->state[c * N + n];
      *s = exp(d * j->A[e * N + n]) * *s + d * j->B[bi * N + n] * x;
      acc += j->C[bi * N + n] * *s;
    }
    double yv = acc + (j->D ? j->D[e] * x : 0.0);
    if (j->z) yv *= oracle_silu(j->z[c]);
    j->y[c] = yv;
  }
  return NULL;
}

/* One recurrent step for every (b, e): state [b,E,N] is updated in place,
 * x, delta, z, y are [b,E], B and C are [b,N].  Returns 0, -1 or -2 as above. */
int oracle_state_update(double* state, const double* x, const double* delta, const double* A, const double* B,
                        const double* C, const double* D, const double* z, const double* delta_bias, int softplus,
                        double* y, int64_t b, int64_t E, int64_t N, int threads) {
  if (b < 0 || E < 0 || N < 0) return -1;
  const int64_t chains = b * E;
  if (chains == 0) return 0;
  if (!x || !delta || !y || (N > 0 && (!state || !A || !B || !C))) return -1;
  if (threads < 1) threads = 1;
  if (threads > chains) threads = (int)chains;
  update_job base;
  memset(&base, 0, sizeof base);
  base.state = state; base.x = x; base.delta = delta; base.A = A; base.B = B; base.C = C; base.D = D;
  base.z = z; base.bias = delta_bias; base.y = y; base.b = b; base.E = E; base.N = N;
  base.softplus = softplus;
  update_job* jobs = (update_job*)malloc(sizeof(update_job) * (size_t)threads);
  pthread_t* tid = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)threads);
  if (!jobs || !tid) { free(jobs); free(tid); return -2; }
  int rc = 0, started = 0;
  for (int i = 0; i < threads; i++) {
    jobs[i] = base;
    jobs[i].chain_begin = chains * i / threads;
    jobs[i].chain_end = chains * (i + 1) / threads;
    if (threads == 1) {
      update_worker(&jobs[i]);
    } else if (pthread_create(&tid[i], NULL, update_worker, &jobs[i]) != 0) {
      rc = -2;
      break;
    } else {
      started++;
    }
  }
  for (int i = 0; i < started; i++) pthread_join(tid[i], NULL);
  free(jobs);
  free(tid);
  return rc;
}

/* Causal depthwise convolution + silu over a sequence.
 * v, x [b, L, E]; q [E, K]; cb [E] (nullable: zero); state_in [b, E, K] (nullable: zero history);
 * state_out [b, E, K] (nullable): the K most recent samples after the last step, oldest first. */
int oracle_conv_fwd(const double* v, const double* q, const double* cb, const double* state_in, double* x,
                    double* state_out, int64_t b, int64_t L, int64_t E, int64_t K) {
  if (b < 0 || L < 0 || E < 0 || K < 1) return -1;
  for (int64_t bi = 0; bi < b; bi++) {
    for (int64_t c = 0; c < E; c++) {
      for (int64_t t = 0; t < L; t++) {
        double acc = cb ? cb[c] : 0.0;
        for (int64_t k = 0; k < K; k++) {
          const int64_t s = t - K + 1 + k; /* time index of this tap */
          double sample;
          if (s >= 0) sample = v[(bi * L + s) * E + c];
          else sample = state_in ? state_in[(bi * E + c) * K + (K + s)] : 0.0;
          acc += q[c * K + k] * sample;
        }
        x[(bi * L + t) * E + c] = oracle_silu(acc);
      }
      if (state_out) {
        for (int64_t k = 0; k < K; k++) {
          const int64_t s = L - K + k;
          double sample;
          if (s >= 0) sample = v[(bi * L + s) * E + c];
          else sample = state_in ? state_in[(bi * E + c) * K + (K + s)] : 0.0;
          state_out[(bi * E + c) * K + k] = sample;
        }
      }
    }
  }
  return 0;
}

/* One token: state [b, E, K] shifted left by one with v [b, E] appended (in place), then
 * x [b, E] = silu(cb + sum_k q[c,k] * state[b,c,k]). */
int oracle_conv_update(double* state, const double* v, const double* q, const double* cb, double* x, int64_t b,
                       int64_t E, int64_t K) {
  if (b < 0 || E < 0 || K < 1) return -1;
  for (int64_t bi = 0; bi < b; bi++) {
    for (int64_t c = 0; c < E; c++) {
      double* st = state + (bi * E + c) * K;
      for (int64_t k = 0; k + 1 < K; k++) st[k] = st[k + 1];
      st[K - 1] = v[bi * E + c];
      double acc = cb ? cb[c] : 0.0;
      for (int64_t k = 0; k < K; k++) acc += q[c * K + k] * st[k];
      x[bi * E + c] = oracle_silu(acc);
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------
 * Backward of the scan: the gradient of a scalar loss
 *     loss = sum dy[b,t,e] * y[b,t,e] + sum d_last[b,e,n] * last_state[b,e,n]
 * with respect to every input, by the chain rule applied to the definition
 * above.  The pages train the block end to end and recompute the states in
 * the backward pass instead of storing them ([NC] "Core Idea"; [AB] "Compose
 * the updates instead of waiting for every state"); the oracle simply keeps
 * every state of a chain in memory.
 *
 * Per chain, walking t from L-1 down to 0 with X = dloss/dh_t coming from
 * the future (X = d_last at t = L-1):
 *   g   = silu(z_t) (1 without a gate);  dq = dy_t * g
 *   dz_t = dy_t * q_t * silu'(z_t),  silu'(z) = s(z) * (1 + z * (1 - s(z))),  s the logistic
 *   dD  += dq * u_t;   du_t = dq * D
 *   G_n = X_n + dq * C[t,n]                       (total dloss/dh_t,n)
 *   dC[t,n] += dq * h_t,n ;  dB[t,n] += G_n * d_t * u_t
 *   du_t += G_n * d_t * B[t,n];  dd += G_n * u_t * B[t,n] + G_n * h_{t-1},n * a_t,n * A[n]
 *   dA[n] += G_n * h_{t-1},n * a_t,n * d_t;   X_n = a_t,n * G_n   (dloss/dh_{t-1})
 *   ddelta_t = dd * s(delta_t + bias) with softplus (dd without);  dbias += ddelta_t
 * and dloss/dh0 = X after t = 0.  B and C are shared by every channel of a
 * batch row, A, D and bias by every batch row and step, so their gradients
 * are sums over chains.
 * ------------------------------------------------------------------------ */
typedef struct {
  const double *u, *delta, *A, *B, *C, *D, *z, *bias, *h0, *dy, *dlast;
  double *du, *ddelta, *dz, *dh0;
  double *dA, *dB, *dC, *dD, *dbias; /* this thread's private sums */
  int64_t b, L, E, N;
  int softplus;
  int64_t chain_begin, chain_end;
} bwd_job;

static double oracle_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

static void bwd_chain(const bwd_job* j, int64_t bi, int64_t e, double* hist, double* q, double* X) {
  const int64_t L = j->L, E = j->E, N = j->N;
  /* forward, keeping every state: hist[(t + 1) * N + n] = h_t,n, hist[n] = h_{-1},n */
  for (int64_t n = 0; n < N; n++) hist[n] = j->h0 ? j->h0[(bi * E + e) * N + n] : 0.0;
  for (int64_t t = 0; t < L; t++) {
    const int64_t xe = (bi * L + t) * E + e, xn = (bi * L + t) * N;
    double d = j->delta[xe] + (j->bias ? j->bias[e] : 0.0);
    if (j->softplus) d = oracle_softplus(d);
    double acc = 0.0;
    for (int64_t n = 0; n < N; n++) {
      const double h = exp(d * j->A[e * N + n]) * hist[t * N + n] + d * j->B[xn + n] * j->u[xe];
      hist[(t + 1) * N + n] = h;
      acc += j->C[xn + n] * h;
    }
    q[t] = acc + (j->D ? j->D[e] * j->u[xe] : 0.0);
  }
  /* backward */
  for (int64_t n = 0; n < N; n++) X[n] = j->dlast ? j->dlast[(bi * E + e) * N + n] : 0.0;
  for (int64_t t = L - 1; t >= 0; t--) {
    const int64_t xe = (bi * L + t) * E + e, xn = (bi * L + t) * N;
    const double x = j->u[xe];
    const double raw = j->delta[xe] + (j->bias ? j->bias[e] : 0.0);
    const double d = j->softplus ? oracle_softplus(raw) : raw;
    double dq = j->dy[xe];
    if (j->z) {
      const double zz = j->z[xe], sg = oracle_sigmoid(zz);
      j->dz[xe] = j->dy[xe] * q[t] * sg * (1.0 + zz * (1.0 - sg));
      dq *= oracle_silu(zz);
    }
    double dut = 0.0, dd = 0.0;
    if (j->D) {
      j->dD[e] += dq * x;
      dut = dq * j->D[e];
    }
    for (int64_t n = 0; n < N; n++) {
      const double G = X[n] + dq * j->C[xn + n];
      const double h_t = hist[(t + 1) * N + n], h_prev = hist[t * N + n];
      const double a = exp(d * j->A[e * N + n]);
      j->dC[xn + n] += dq * h_t;
      j->dB[xn + n] += G * d * x;
      dut += G * d * j->B[xn + n];
      const double ha = h_prev * a;
      dd += G * x * j->B[xn + n] + G * ha * j->A[e * N + n];
      j->dA[e * N + n] += G * ha * d;
      X[n] = a * G;
    }
    j->du[xe] = dut;
    const double ddelta = j->softplus ? dd * oracle_sigmoid(raw) : dd;
    j->ddelta[xe] = ddelta;
    if (j->bias) j->dbias[e] += ddelta;
  }
  if (j->dh0)
    for (int64_t n = 0; n < N; n++) j->dh0[(bi * E + e) * N + n] = X[n];
}

static void* bwd_worker(void* arg) {
  const bwd_job* j = (const bwd_job*)arg;
  const int64_t N = j->N > 0 ? j->N : 1;
  double* hist = (double*)malloc(sizeof(double) * (size_t)((j->L + 1) * N));
  double* q = (double*)malloc(sizeof(double) * (size_t)(j->L > 0 ? j->L : 1));
  double* X = (double*)malloc(sizeof(double) * (size_t)N);
  if (!hist || !q || !X) {
    free(hist); free(q); free(X);
    return (void*)1;
  }
  for (int64_t c = j->chain_begin; c < j->chain_end; c++) bwd_chain(j, c / j->E, c % j->E, hist, q, X);
  free(hist); free(q); free(X);
  return NULL;
}

/* Gradients of the scan.  Outputs: du, ddelta [b,L,E]; dz [b,L,E] (when z is given);
 * dA [E,N]; dB, dC [b,L,N]; dD [E] (when D is given); dbias [E] (when a bias is given);
 * dh0 [b,E,N] (nullable).  dlast [b,E,N] is nullable (zero).  Returns 0, -1 on bad
 * arguments, -2 on allocation or thread failure. */
int oracle_scan_bwd(const double* u, const double* delta, const double* A, const double* B, const double* C,
                    const double* D, const double* z, const double* delta_bias, int softplus, const double* h0,
                    const double* dy, const double* dlast, double* du, double* ddelta, double* dA, double* dB,
                    double* dC, double* dD, double* dz, double* dbias, double* dh0, int64_t b, int64_t L, int64_t E,
                    int64_t N, int threads) {
  if (b < 0 || L < 0 || E < 0 || N < 0) return -1;
  if (!A || !dA || !dB || !dC || (L > 0 && (!u || !delta || !B || !C || !dy || !du || !ddelta)) ||
      (z && !dz) || (D && !dD) || (delta_bias && !dbias))
    return -1;
  memset(dA, 0, sizeof(double) * (size_t)(E * N));
  memset(dB, 0, sizeof(double) * (size_t)(b * L * N));
  memset(dC, 0, sizeof(double) * (size_t)(b * L * N));
  if (dD) memset(dD, 0, sizeof(double) * (size_t)E);
  if (dbias) memset(dbias, 0, sizeof(double) * (size_t)E);
  const int64_t chains = b * E;
  if (chains == 0) return 0;
  if (threads < 1) threads = 1;
  if (threads > chains) threads = (int)chains;
  /* private sums per thread: dA [E,N], dB, dC [b,L,N], dD, dbias [E] */
  const int64_t per = E * N + 2 * b * L * N + 2 * E;
  double* priv = (double*)calloc((size_t)(per * threads), sizeof(double));
  bwd_job* jobs = (bwd_job*)malloc(sizeof(bwd_job) * (size_t)threads);
  pthread_t* tid = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)threads);
  if (!priv || !jobs || !tid) { free(priv); free(jobs); free(tid); return -2; }
  int rc = 0, started = 0;
  for (int i = 0; i < threads; i++) {
    bwd_job* jb = &jobs[i];
    memset(jb, 0, sizeof *jb);
    jb->u = u; jb->delta = delta; jb->A = A; jb->B = B; jb->C = C; jb->D = D; jb->z = z; jb->bias = delta_bias;
    jb->h0 = h0; jb->dy = dy; jb->dlast = dlast; jb->du = du; jb->ddelta = ddelta; jb->dz = dz; jb->dh0 = dh0;
    double* base = priv + per * i;
    jb->dA = base; jb->dB = base + E * N; jb->dC = jb->dB + b * L * N; jb->dD = jb->dC + b * L * N;
    jb->dbias = jb->dD + E;
    jb->b = b; jb->L = L; jb->E = E; jb->N = N; jb->softplus = softplus;
    jb->chain_begin = chains * i / threads;
    jb->chain_end = chains * (i + 1) / threads;
    if (threads == 1) {
      if (bwd_worker(jb)) rc = -2;
    } else if (pthread_create(&tid[i], NULL, bwd_worker, jb) != 0) {
      rc = -2;
      break;
    } else {
      started++;
    }
  }
  for (int i = 0; i < started; i++) {
    void* ret = NULL;
    pthread_join(tid[i], &ret);
    if (ret) rc = -2;
  }
  if (rc == 0) {
    /* add the private sums in thread order */
    for (int i = 0; i < threads; i++) {
      const bwd_job* jb = &jobs[i];
      for (int64_t k = 0; k < E * N; k++) dA[k] += jb->dA[k];
      for (int64_t k = 0; k < b * L * N; k++) { dB[k] += jb->dB[k]; dC[k] += jb->dC[k]; }
      if (dD) for (int64_t k = 0; k < E; k++) dD[k] += jb->dD[k];
      if (dbias) for (int64_t k = 0; k < E; k++) dbias[k] += jb->dbias[k];
    }
  }
  free(priv);
  free(jobs);
  free(tid);
  return rc;
}

/* Exposed for the softplus / gate pins: the scalar helpers exactly as used above. */
double oracle_softplus_value(double x) { return oracle_softplus(x); }
double oracle_silu_value(double z) { return oracle_silu(z); }
