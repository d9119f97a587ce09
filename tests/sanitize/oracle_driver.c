/* Exercises every function of the C oracle on small inputs (every optional
 * argument present and absent, several thread counts, edge sizes) so that a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer sees all of its
 * paths.  Exit status 0 when every call returned 0 and produced finite
 * values; the sanitizers abort the process on the first error they find. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_scan(const double* u, const double* delta, const double* A, const double* B, const double* C,
                const double* D, const double* z, const double* delta_bias, int softplus, const double* h0,
                double* y, double* last_state, double* states, int64_t b, int64_t L, int64_t E, int64_t N,
                int threads);
int oracle_state_update(double* state, const double* x, const double* delta, const double* A, const double* B,
                        const double* C, const double* D, const double* z, const double* delta_bias, int softplus,
                        double* y, int64_t b, int64_t E, int64_t N, int threads);
int oracle_conv_fwd(const double* v, const double* q, const double* cb, const double* state_in, double* x,
                    double* state_out, int64_t b, int64_t L, int64_t E, int64_t K);
int oracle_conv_update(double* state, const double* v, const double* q, const double* cb, double* x, int64_t b,
                       int64_t E, int64_t K);
int oracle_scan_bwd(const double* u, const double* delta, const double* A, const double* B, const double* C,
                    const double* D, const double* z, const double* delta_bias, int softplus, const double* h0,
                    const double* dy, const double* dlast, double* du, double* ddelta, double* dA, double* dB,
                    double* dC, double* dD, double* dz, double* dbias, double* dh0, int64_t b, int64_t L, int64_t E,
                    int64_t N, int threads);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static double rnd(void) { /* xorshift64*, uniform in [-1, 1) */
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (double)((g_state * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}

/* exactly n doubles on the heap, so that any access past the end is caught */
static double* arr(int64_t n) {
  double* p = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; i++) p[i] = rnd();
  return p;
}

static int finite_all(const double* p, int64_t n) {
  for (int64_t i = 0; i < n; i++)
    if (!isfinite(p[i])) return 0;
  return 1;
}

static int fails = 0;
#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      fails++;                                                   \
    }                                                            \
  } while (0)

static void scan_case(int64_t b, int64_t L, int64_t E, int64_t N, int opt, int threads) {
  const int64_t x = b * L * E, r = b * L * N, s = b * E * N;
  double *u = arr(x), *dl = arr(x), *A = arr(E * N), *B = arr(r), *C = arr(r), *D = arr(E), *z = arr(x),
         *bias = arr(E), *h0 = arr(s), *y = arr(x), *last = arr(s), *states = arr(x * N), *dy = arr(x),
         *dlast = arr(s), *du = arr(x), *dd = arr(x), *dA = arr(E * N), *dB = arr(r), *dC = arr(r), *dD = arr(E),
         *dz = arr(x), *db = arr(E), *dh0 = arr(s);
  for (int64_t i = 0; i < E * N; i++) A[i] = -1.0 - fabs(A[i]); /* retention below 1 */
  const int with = opt & 1, sp = (opt >> 1) & 1;
  CHECK(oracle_scan(u, dl, A, B, C, with ? D : 0, with ? z : 0, with ? bias : 0, sp, with ? h0 : 0, y, last,
                    (opt & 4) ? states : 0, b, L, E, N, threads) == 0);
  CHECK(finite_all(y, x) && finite_all(last, s));
  CHECK(oracle_scan_bwd(u, dl, A, B, C, with ? D : 0, with ? z : 0, with ? bias : 0, sp, with ? h0 : 0, dy,
                        with ? dlast : 0, du, dd, dA, dB, dC, with ? dD : 0, with ? dz : 0, with ? db : 0, dh0, b,
                        L, E, N, threads) == 0);
  CHECK(finite_all(du, x) && finite_all(dd, x) && finite_all(dA, E * N) && finite_all(dh0, s));
  if (L > 0) {
    double* st = arr(s);
    CHECK(oracle_state_update(st, u, dl, A, B, C, with ? D : 0, with ? z : 0, with ? bias : 0, sp, y, b, E, N,
                              threads) == 0);
    CHECK(finite_all(st, s));
    free(st);
  }
  double* ptrs[] = {u, dl, A, B, C, D, z, bias, h0, y, last, states, dy, dlast, du, dd, dA, dB, dC, dD, dz, db, dh0};
  for (size_t i = 0; i < sizeof(ptrs) / sizeof(ptrs[0]); i++) free(ptrs[i]);
}

static void conv_case(int64_t b, int64_t L, int64_t E, int64_t K, int opt) {
  double *v = arr(b * L * E), *q = arr(E * K), *cb = arr(E), *sin = arr(b * E * K), *x = arr(b * L * E),
         *sout = arr(b * E * K), *tok = arr(b * E), *xt = arr(b * E);
  CHECK(oracle_conv_fwd(v, q, (opt & 1) ? cb : 0, (opt & 2) ? sin : 0, x, (opt & 4) ? sout : 0, b, L, E, K) == 0);
  CHECK(finite_all(x, b * L * E));
  CHECK(oracle_conv_update(sin, tok, q, (opt & 1) ? cb : 0, xt, b, E, K) == 0);
  CHECK(finite_all(xt, b * E));
  double* ptrs[] = {v, q, cb, sin, x, sout, tok, xt};
  for (size_t i = 0; i < sizeof(ptrs) / sizeof(ptrs[0]); i++) free(ptrs[i]);
}

int main(void) {
  const int64_t shapes[][4] = {{1, 1, 1, 1}, {2, 7, 3, 5}, {1, 0, 4, 3}, {3, 33, 9, 16}, {1, 65, 2, 4}, {2, 5, 1, 13}};
  for (size_t k = 0; k < sizeof(shapes) / sizeof(shapes[0]); k++)
    for (int opt = 0; opt < 8; opt++)
      for (int threads = 1; threads <= 5; threads += 2)
        scan_case(shapes[k][0], shapes[k][1], shapes[k][2], shapes[k][3], opt, threads);
  const int64_t conv[][4] = {{1, 1, 1, 1}, {2, 9, 5, 4}, {1, 3, 7, 8}, {3, 0, 2, 3}};
  for (size_t k = 0; k < sizeof(conv) / sizeof(conv[0]); k++)
    for (int opt = 0; opt < 8; opt++) conv_case(conv[k][0], conv[k][1], conv[k][2], conv[k][3], opt);
  /* invalid sizes are refused, not run */
  CHECK(oracle_scan(0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, -1, 1, 1, 1, 1) != 0);
  CHECK(oracle_conv_fwd(0, 0, 0, 0, 0, 0, 1, 1, 1, 0) != 0);
  if (fails) fprintf(stderr, "%d checks failed\n", fails);
  printf("oracle driver: %s\n", fails ? "FAILED" : "ok");
  return fails ? 1 : 0;
}
