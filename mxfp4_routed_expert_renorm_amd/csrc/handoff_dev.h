// Cross-workgroup handoff of the single-launch decode steps: 256 workgroups
// ("units"), all resident at once, each publish their part of the SwiGLU
// outputs and then wait until every unit has published.
//
// Sync words (uint32), kept between launches at the end of the workspace:
//   [0, 256)          each unit's launch tag; only that unit writes it, so a
//                     unit reads its tag for this launch as its word plus one
//   [256]             error word (nonzero: a wait gave up; output meaningless)
//   [320 + 32 x]      arrivals of the units u with u % 8 == x, x < 8: one
//                     128-byte line each, so the arrivals of the eight groups
//                     do not queue on one address
//   [576]             groups of 32 complete
// A unit arrives after its data stores have completed (write-through,
// agent-scope stores, then vmcnt 0): it adds one to its group's counter, and
// the unit that completes the group (the counter reaches 32 x tag) adds one
// to the last word.  Every unit then polls that one word until it reads
// 8 x tag.  All counters move by fixed amounts per launch (32 per group, 8
// overall, 1 per tag), so they stay consistent modulo 2^32 with no reset:
// they must start at zero (a zeroed workspace), and launches that share them
// must not overlap.  Compared with polling 256 per-unit flags, each poll is
// one request instead of a kilobyte from every workgroup, which is what kept
// the last flags from being seen quickly.
#pragma once

#include "common.h"

namespace moe {

constexpr int kHandoffUnits = 256;
constexpr int kSyncErr = 256, kSyncGroup = 320, kSyncAll = 576;
constexpr size_t kHandoffSyncBytes = 1024 * 4;

// this launch's tag of unit `unit` (read before the unit arrives)
__device__ __forceinline__ uint32_t handoff_tag(uint32_t* sync, int unit) {
  return __hip_atomic_load(&sync[unit], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
}

// Called by one whole wavefront of unit `unit` once its stores of the data to
// hand over have completed: records the arrival and waits, at most `spin`
// polls, until all 256 units of this launch have arrived.  A wait that gives
// up sets bit 0 of the error word and returns.
__device__ __forceinline__ void handoff_arrive_wait(uint32_t* sync, int unit, uint32_t tag, uint32_t spin) {
  const int lane = threadIdx.x & 63;
  if (lane == 0) {
    __hip_atomic_store(&sync[unit], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t old =
        __hip_atomic_fetch_add(&sync[kSyncGroup + 32 * (unit & 7)], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1u == 32u * tag) __hip_atomic_fetch_add(&sync[kSyncAll], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  uint32_t it = 0;
  for (;;) {
    const uint32_t v = __hip_atomic_load(&sync[kSyncAll], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__builtin_amdgcn_readfirstlane(v) == 8u * tag) break;
    if (++it > spin) {
      if (lane == 0) atomicOr(&sync[kSyncErr], 1u);
      break;
    }
  }
}

}  // namespace moe
