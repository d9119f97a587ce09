/* Exercises the host side of libssm.so (argument checks, plans, status and
 * profiling queries) on a host without a GPU, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer on the host code.  Every
 * call here is refused by the checks or stops at the first HIP call (no
 * device), so no kernel runs.  Exit status 0 when every status is the one the
 * header documents; the sanitizers abort the process on the first error. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ssm.h"

static int fails = 0;
#define EXPECT(call, want)                                                          \
  do {                                                                              \
    int got_ = (call);                                                              \
    if (got_ != (want)) {                                                           \
      fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, (want)); \
      fails++;                                                                      \
    }                                                                               \
  } while (0)

/* a fake device address: the checks look at its value only, nothing dereferences it */
#define P ((void*)(uintptr_t)0x10000000)
#define F ((float*)(uintptr_t)0x10000000)
#define P2 ((void*)(uintptr_t)0x10000002)
#define F2 ((float*)(uintptr_t)0x10000002)

int main(void) {
  const int64_t big = (int64_t)1 << 40;
  /* forward scans */
  EXPECT(ssm_scan_fwd(P, P, F, P, P, 0, 0, 0, 1, P, 0, 1, 8, 64, 16, 7, 0), SSM_ERR_DTYPE);
  EXPECT(ssm_scan_fwd(P, P, F, P, P, 0, 0, 0, 1, P, 0, -1, 8, 64, 16, 0, 0), SSM_ERR_DIM);
  EXPECT(ssm_scan_fwd(P, P, F, P, P, 0, 0, 0, 1, P, 0, 1, 8, 64, 0, 0, 0), SSM_ERR_UNSUPPORTED_N);
  EXPECT(ssm_scan_fwd(P, P, F, P, P, 0, 0, 0, 1, P, 0, 1, 8, 64, 17, 0, 0), SSM_ERR_UNSUPPORTED_N);
  EXPECT(ssm_scan_fwd(0, P, F, P, P, 0, 0, 0, 1, P, 0, 1, 8, 64, 16, 0, 0), SSM_ERR_NULL);
  EXPECT(ssm_scan_fwd(P2, P, F, P, P, 0, 0, 0, 1, P, 0, 1, 8, 64, 16, 0, 0), SSM_ERR_ALIGN);
  EXPECT(ssm_scan_fwd(P, P, F, P, P, 0, 0, 0, 1, P, 0, big, big, big, 16, 0, 0), SSM_ERR_DIM);
  EXPECT(ssm_scan_fwd(P, P, F, P, P, 0, 0, 0, 1, P, 0, INT64_MAX, 2, 2, 16, 1, 0), SSM_ERR_DIM);
  EXPECT(ssm_scan_fwd(0, 0, 0, 0, 0, 0, 0, 0, 1, 0, 0, 0, 8, 64, 16, 0, 0), SSM_OK);
  EXPECT(ssm_scan_fwd_from(P, P, F, P, P, 0, 0, 0, 1, F2, P, 0, 1, 8, 64, 16, 0, 0), SSM_ERR_ALIGN);
  EXPECT(ssm_scan_fwd_save(P, P, F, P, P, 0, 0, 0, 1, 0, P, 0, 0, 1, 200, 64, 16, 0, 0), SSM_ERR_NULL);
  ssm_scan_tuning t = {SSM_PATH_CHUNKED, 8, 100000};
  EXPECT(ssm_scan_fwd_tuned(P, P, F, P, P, 0, 0, 0, 1, 0, P, 0, 0, &t, 1, 8, 64, 16, 9, 0), SSM_ERR_DTYPE);
  t.path = 9;
  EXPECT(ssm_scan_fwd_tuned(P, P, F, P, P, 0, 0, 0, 1, 0, P, 0, 0, &t, 1, 8, 64, 16, 0, 0), SSM_ERR_PLAN);
  t.path = SSM_PATH_AUTO;
  t.min_chunk = -3;
  EXPECT(ssm_scan_fwd_tuned(P, P, F, P, P, 0, 0, 0, 1, 0, P, 0, 0, &t, 1, 8, 64, 16, 0, 0), SSM_ERR_PLAN);
  EXPECT(ssm_scan_fwd_noalloc(P, P, F, P, P, 0, 0, 0, 1, 0, 0, 0, 1, 8, 64, 16, 0, 0), SSM_ERR_NULL);
  EXPECT(ssm_scan_fwd_noalloc(P, P, F, P, P, 0, 0, 0, 1, F2, P, 0, 1, 8, 64, 16, 0, 0), SSM_ERR_ALIGN);
  /* valid arguments: the first HIP call fails without a device */
  EXPECT(ssm_scan_fwd(P, P, F, P, P, 0, 0, 0, 1, P, 0, 1, 8, 64, 16, 0, 0), SSM_ERR_HIP);
  EXPECT(ssm_scan_fwd_noalloc(P, P, F, P, P, 0, 0, 0, 1, 0, P, 0, 1, 4096, 5120, 16, 1, 0), SSM_ERR_HIP);
  if (strlen(ssm_last_hip_error()) == 0) {
    fprintf(stderr, "no HIP error text after SSM_ERR_HIP\n");
    fails++;
  }
  /* plans over a range of sizes, including ones whose products overflow */
  const int64_t sizes[] = {0, 1, 7, 64, 65, 1000, 65536, (int64_t)1 << 31, (int64_t)1 << 40, INT64_MAX};
  const int n_sizes = (int)(sizeof(sizes) / sizeof(sizes[0]));
  for (int i = 0; i < n_sizes; i++)
    for (int j = 0; j < n_sizes; j++)
      for (int k = 0; k < n_sizes; k += 3)
        for (int dt = 0; dt < 2; dt++)
          for (int path = 0; path < 3; path++) {
            ssm_scan_tuning tt = {path, (int32_t)(k * 7), (int32_t)(j * 1000)};
            int form = -1;
            int64_t cl = -1, nc = -1;
            const int st = ssm_scan_plan(sizes[i], sizes[j], sizes[k], 16, dt, &tt, &form, &cl, &nc);
            if (st == SSM_OK && (cl < 1 || nc < 1 || (form != SSM_PATH_CHUNKED && form != SSM_PATH_SINGLE_PASS))) {
              fprintf(stderr, "plan b=%lld L=%lld E=%lld: %d %lld %lld\n", (long long)sizes[i],
                      (long long)sizes[j], (long long)sizes[k], form, (long long)cl, (long long)nc);
              fails++;
            }
          }
  /* the other entry points' checks */
  EXPECT(ssm_state_update(F, P, P, F, P, P, 0, 0, 0, 1, P, 1, 64, 16, 3, 0), SSM_ERR_DTYPE);
  EXPECT(ssm_state_update(F2, P, P, F, P, P, 0, 0, 0, 1, P, 1, 64, 16, 0, 0), SSM_ERR_ALIGN);
  EXPECT(ssm_state_update(F, P, P, F, P, P, 0, 0, 0, 1, P, big, big, 16, 0, 0), SSM_ERR_DIM);
  EXPECT(ssm_scan_bwd(P, P, F, P, P, 0, 0, 0, 1, 0, P, 0, P, P, F, F, F, 0, 0, 0, 0, 1, 8, 64, 16, 5, 0),
         SSM_ERR_DTYPE);
  EXPECT(ssm_scan_bwd(P, P, F, P, P, 0, P, 0, 1, 0, P, 0, P, P, F, F, F, 0, 0, 0, 0, 1, 8, 64, 16, 0, 0),
         SSM_ERR_NULL); /* z without dz */
  EXPECT(ssm_scan_bwd(P, P, F, P, P, 0, 0, 0, 1, 0, P, 0, P, P, F, F, F, 0, 0, 0, 0, big, big, 64, 16, 0, 0),
         SSM_ERR_DIM);
  EXPECT(ssm_scan_bwd_saved(P, P, F, P, P, 0, 0, 0, 1, 0, 0, P, 0, P, P, F, F, F, 0, 0, 0, 0, 1, 200, 64, 16, 0, 0),
         SSM_ERR_NULL);
  EXPECT(ssm_ssd_fwd(P, P, F, P, P, 0, 0, 0, 1, 0, P, 0, 1, 128, 2, 64, 16, 0, 0), SSM_ERR_DTYPE);
  EXPECT(ssm_ssd_fwd(P, P, F, P, P, 0, 0, 0, 1, 0, P, 0, 1, 128, 2, 64, 20, 1, 0), SSM_ERR_UNSUPPORTED_N);
  EXPECT(ssm_ssd_fwd(P, P, F, P, P, 0, 0, 0, 1, 0, P, 0, 1, 128, 2, 32, 16, 1, 0), SSM_ERR_DIM);
  EXPECT(ssm_ssd_fwd(P2, P, F, P, P, 0, 0, 0, 1, 0, P, 0, 1, 128, 2, 64, 16, 1, 0), SSM_ERR_ALIGN);
  EXPECT(ssm_conv_fwd(P, F, 0, 0, P, 0, 1, 8, 64, 9, 0, 0), SSM_ERR_DIM);
  EXPECT(ssm_conv_fwd(P, F, 0, 0, P, 0, big, big, 64, 4, 0, 0), SSM_ERR_DIM);
  EXPECT(ssm_conv_update(P, P, F, 0, P, 1, 64, 0, 0, 0), SSM_ERR_DIM);
  EXPECT(ssm_conv_update(P2, P, F, 0, P, 1, 64, 4, 0, 0), SSM_ERR_ALIGN);
  /* queries */
  for (int s = -20; s <= 5; s++)
    if (!ssm_status_string(s)) fails++;
  for (int k = -3; k < 40; k++) (void)ssm_profile_kind_name(k);
  double ms[64];
  int64_t n[64];
  EXPECT(ssm_profile_read(ms, n, 64), SSM_OK);
  EXPECT(ssm_profile_read(ms, n, 0), SSM_OK);
  (void)ssm_profile_read(0, 0, 5);
  (void)ssm_profile_read(ms, n, -1);
  EXPECT(ssm_profile_enable(0), SSM_OK);
  if (ssm_version() < 10000) fails++;
  if (fails) fprintf(stderr, "%d checks failed\n", fails);
  printf("api driver: %s\n", fails ? "FAILED" : "ok");
  return fails ? 1 : 0;
}
