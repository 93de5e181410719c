// Device side of the slot cache's per-call exchange with the host.
//
// "An elephant through a straw", §43 graphs, 43 syncs: each layer call reads
// the router's picks on the host once and hands back the rewritten ids.  The
// picks (ids and weights) leave in one small kernel that writes them into
// mapped pinned host memory, and the rewritten slots, weights and precision
// tags come back in one kernel that reads them from there: two launches per
// call instead of one copy per array.
#include "common.h"

namespace moe {

namespace {

// One workgroup: the picks go out, then (after the workgroup's stores and a
// system-scope fence) the call's sequence number, which the host polls: it
// learns the picks as soon as they are in its memory, without waiting for
// the kernel's completion signal.
__global__ __launch_bounds__(1024) void cache_gather_kernel(const int32_t* __restrict__ ids,
                                                            const float* __restrict__ w, int n,
                                                            int32_t* __restrict__ ids_h, float* __restrict__ w_h,
                                                            uint32_t* __restrict__ flag_h, uint32_t seq) {
  for (int i = threadIdx.x; i < n; i += 1024) {
    ids_h[i] = ids[i];
    w_h[i] = w[i];
  }
  // every wavefront waits for its own stores to reach this CU's L2, then one
  // system-scope release by thread 0 (an L2 write-back) makes them all
  // visible to the host ahead of the sequence number
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(flag_h, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

__global__ __launch_bounds__(256) void cache_scatter_kernel(const int32_t* __restrict__ slots_h,
                                                            const float* __restrict__ w_h,
                                                            const int8_t* __restrict__ prec_h, int n,
                                                            int32_t* __restrict__ ids, float* __restrict__ w,
                                                            int8_t* __restrict__ prec) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    ids[i] = slots_h[i];
    w[i] = w_h[i];
    prec[i] = prec_h[i];
  }
}

}  // namespace

moe_status launch_cache_gather(const int32_t* ids, const float* w, int n, int32_t* ids_h, float* w_h, uint32_t* flag_h,
                               uint32_t seq, hipStream_t s) {
  launch(MOE_PROF_CACHE, cache_gather_kernel, dim3(1), dim3(1024), 0, s, ids, w, n, ids_h, w_h, flag_h, seq);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

moe_status launch_cache_scatter(const int32_t* slots_h, const float* w_h, const int8_t* prec_h, int n, int32_t* ids,
                                float* w, int8_t* prec, hipStream_t s) {
  if (n <= 0) return MOE_OK;
  launch(MOE_PROF_CACHE, cache_scatter_kernel, dim3((n + 255) / 256), dim3(256), 0, s, slots_h, w_h, prec_h, n, ids, w,
         prec);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
