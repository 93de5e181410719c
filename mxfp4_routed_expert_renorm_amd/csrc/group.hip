// Stable grouping of (token, rank) pairs by key (moe_group): one workgroup
// running group_body (group_dev.h).
#include "group_dev.h"

namespace moe {

namespace {

__global__ __launch_bounds__(kGroupThreads) void group_kernel(const int32_t* __restrict__ keys, int n, int nkeys,
                                                               int W, int32_t* __restrict__ counts,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ perm) {
  extern __shared__ int lds[];
  group_body(keys, n, nkeys, W, counts, offsets, perm, lds);
}

}  // namespace

moe_status launch_group(const int32_t* keys, int n, int nkeys, int32_t* counts, int32_t* offsets, int32_t* perm,
                        hipStream_t s) {
  const int W = group_chunks(nkeys);
  const size_t lds = (size_t)(W + 1) * nkeys * sizeof(int);
  launch(MOE_PROF_GROUP, group_kernel, dim3(1), dim3(kGroupThreads), lds, s, keys, n, nkeys, W, counts, offsets,
         perm);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
