// ssm_profile.hip -- opt-in per-kernel timing: while enabled, every kernel the
// library enqueues is bracketed by two HIP events on its own stream; reading
// the totals waits for those events.  Off by default (no events, no cost).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "ssm.h"
#include "ssm_profile.h"

namespace ssm {
namespace {

struct Pending {
  int kind;
  hipEvent_t ev0, ev1;
};

std::atomic<bool> g_enabled{false};
std::mutex g_mu;
std::vector<Pending> g_pending;

const char* const kNames[kNumKinds] = {"chunk_aggregate", "chunk_carry",   "scan_main",     "fill_state",
                                       "state_update",    "conv",          "conv_update",   "bwd_rows",
                                       "bwd_aggregate",   "bwd_carry",     "bwd_main",      "bwd_reduce",
                                       "ssd_state",       "ssd_carry",     "ssd_scan",      "scan_fused",
                                       "widen_rows"};

}  // namespace

bool profile_begin(hipStream_t s, hipEvent_t* ev0, hipEvent_t* ev1) {
  if (!g_enabled.load(std::memory_order_relaxed)) return false;
  if (hipEventCreate(ev0) != hipSuccess) return false;
  if (hipEventCreate(ev1) != hipSuccess) {
    (void)hipEventDestroy(*ev0);
    return false;
  }
  if (hipEventRecord(*ev0, s) != hipSuccess) {
    (void)hipEventDestroy(*ev0);
    (void)hipEventDestroy(*ev1);
    return false;
  }
  return true;
}

void profile_end(int kind, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  if (hipEventRecord(ev1, s) != hipSuccess) {
    (void)hipEventDestroy(ev0);
    (void)hipEventDestroy(ev1);
    return;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  g_pending.push_back({kind, ev0, ev1});
}

}  // namespace ssm

extern "C" {

int ssm_profile_enable(int on) {
  ssm::g_enabled.store(on != 0);
  return SSM_OK;
}

int ssm_profile_read(double* total_ms, int64_t* launches, int n_kinds) {
  if (!total_ms || !launches || n_kinds < 0) return SSM_ERR_NULL;
  for (int k = 0; k < n_kinds; k++) {
    total_ms[k] = 0.0;
    launches[k] = 0;
  }
  std::vector<ssm::Pending> pend;
  {
    std::lock_guard<std::mutex> lock(ssm::g_mu);
    pend.swap(ssm::g_pending);
  }
  int status = SSM_OK;
  for (const ssm::Pending& p : pend) {
    float ms = 0.f;
    if (hipEventSynchronize(p.ev1) != hipSuccess || hipEventElapsedTime(&ms, p.ev0, p.ev1) != hipSuccess) {
      status = SSM_ERR_HIP;
      (void)hipGetLastError();
    } else if (p.kind >= 0 && p.kind < n_kinds) {
      total_ms[p.kind] += ms;
      launches[p.kind] += 1;
    }
    (void)hipEventDestroy(p.ev0);
    (void)hipEventDestroy(p.ev1);
  }
  return status;
}

const char* ssm_profile_kind_name(int kind) {
  return (kind >= 0 && kind < ssm::kNumKinds) ? ssm::kNames[kind] : "";
}

}  // extern "C"
