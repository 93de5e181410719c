// Event timing of the library's own kernels.  When enabled, every launch the
// library makes goes out through hipExtLaunchKernel with its own pair of HIP
// events, which the dispatch records at the kernel's start and end, so the
// elapsed time between them is that kernel's duration on the device.  Used by
// the benchmark to time the dominant kernel live; off by default.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "common.h"

namespace moe {

namespace {

struct Record {
  int kind;
  hipEvent_t start, stop;
};

struct ProfState {
  std::mutex mu;
  bool on = false;
  size_t cap = 0;
  std::vector<hipEvent_t> pool;
  size_t next = 0;
  std::vector<Record> recs;
};

ProfState& prof() {
  static ProfState p;
  return p;
}

}  // namespace

bool prof_events(int kind, hipEvent_t* start, hipEvent_t* stop) {
  ProfState& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  if (!p.on || p.next + 2 > p.pool.size()) return false;
  Record r{kind, p.pool[p.next], p.pool[p.next + 1]};
  p.next += 2;
  p.recs.push_back(r);
  *start = r.start;
  *stop = r.stop;
  return true;
}

}  // namespace moe

using namespace moe;

extern "C" {

moe_status moe_profile_begin(int max_launches) {
  if (max_launches < 1 || max_launches > (1 << 20))
    return fail(MOE_EINVAL, "moe_profile_begin: max_launches=%d outside 1..2^20", max_launches);
  ProfState& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  if (p.on) return fail(MOE_ESTATE, "moe_profile_begin: profiling already on");
  p.pool.resize(2 * (size_t)max_launches);
  for (auto& e : p.pool) {
    hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) return fail(MOE_EHIP, "hipEventCreate failed: %s", hipGetErrorString(err));
  }
  p.next = 0;
  p.recs.clear();
  p.on = true;
  return MOE_OK;
}

moe_status moe_profile_end(double* total_ms, int* counts, int nkinds) {
  ProfState& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  if (!p.on) return fail(MOE_ESTATE, "moe_profile_end: profiling is off");
  p.on = false;
  for (int i = 0; i < nkinds; ++i) {
    if (total_ms) total_ms[i] = 0.0;
    if (counts) counts[i] = 0;
  }
  moe_status st = MOE_OK;
  for (const Record& r : p.recs) {
    hipError_t err = hipEventSynchronize(r.stop);
    float ms = 0.0f;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, r.start, r.stop);
    if (err != hipSuccess) {
      st = fail(MOE_EHIP, "moe_profile_end: %s", hipGetErrorString(err));
      break;
    }
    if (r.kind >= 0 && r.kind < nkinds) {
      if (total_ms) total_ms[r.kind] += ms;
      if (counts) counts[r.kind] += 1;
    }
  }
  for (auto& e : p.pool) (void)hipEventDestroy(e);
  p.pool.clear();
  p.recs.clear();
  return st;
}

}  // extern "C"
