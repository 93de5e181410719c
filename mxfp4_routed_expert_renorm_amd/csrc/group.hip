// Stable grouping of (token, rank) pairs by key: counts, exclusive offsets and
// the permutation that lists each key's pairs in ascending pair order.
//
// Grouping lets each selected expert's weights stream from HBM once for all
// the tokens that picked it ("An elephant through a straw", §43 graphs, 43
// syncs: the picks are classified and the grouped expert kernels fired).
//
// One 1024-thread workgroup: LDS atomics build the histogram (counts do not
// depend on the order of the adds), one wavefront scans it, and one
// wavefront places the keys 64 at a time in input order: lanes holding the
// same key find each other with a ballot per key bit, take their rank among
// the lower lanes, and the group's lowest lane advances the key's cursor.
// The placement is therefore stable and identical run to run.
#include "common.h"

namespace moe {

namespace {

constexpr int kGroupThreads = 1024;
constexpr int kMaxKeys = 4096;

__global__ __launch_bounds__(kGroupThreads) void group_kernel(const int32_t* __restrict__ keys, int n,
                                                               int nkeys, int32_t* __restrict__ counts,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ perm) {
  __shared__ int cnt[kMaxKeys];
  __shared__ int cur[kMaxKeys];
  const int tid = threadIdx.x;
  for (int i = tid; i < nkeys; i += kGroupThreads) cnt[i] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kGroupThreads) {
    const int key = keys[i];
    if (key >= 0 && key < nkeys) atomicAdd(&cnt[key], 1);
  }
  __syncthreads();
  const int lane = tid & 63;
  if (tid < 64) {
    // exclusive scan over nkeys in chunks of 64
    int carry = 0;
    for (int base = 0; base < nkeys; base += 64) {
      const int i = base + lane;
      const int c = (i < nkeys) ? cnt[i] : 0;
      int incl = c;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
      }
      if (i < nkeys) {
        cur[i] = carry + incl - c;
        offsets[i] = carry + incl - c;
        counts[i] = c;
      }
      carry += __shfl(incl, 63, 64);
    }
    if (lane == 0) offsets[nkeys] = carry;
  }
  __syncthreads();
  if (tid < 64) {
    int nbits = 1;
    while ((1 << nbits) < nkeys) ++nbits;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = 0; base < n; base += 64) {
      const int i = base + lane;
      int key = (i < n) ? keys[i] : -1;
      const bool valid = key >= 0 && key < nkeys;
      if (!valid) key = -1;
      // lanes with an identical key (invalid lanes match only each other)
      uint64_t peers = __ballot(1);
      for (int b = 0; b < nbits; ++b) {
        const uint64_t ones = __ballot((key >> b) & 1);
        peers &= ((key >> b) & 1) ? ones : ~ones;
      }
      const uint64_t vmask = __ballot(valid);
      peers &= valid ? vmask : ~vmask;
      const int before = __popcll(peers & below);
      int pos = 0;
      if (valid) pos = cur[key] + before;
      __builtin_amdgcn_wave_barrier();
      if (valid && before == 0) cur[key] += __popcll(peers);
      __builtin_amdgcn_wave_barrier();
      if (valid) perm[pos] = i;
    }
  }
}

}  // namespace

moe_status launch_group(const int32_t* keys, int n, int nkeys, int32_t* counts, int32_t* offsets, int32_t* perm,
                        hipStream_t s) {
  launch(MOE_PROF_GROUP, group_kernel, dim3(1), dim3(kGroupThreads), 0, s, keys, n, nkeys, counts, offsets, perm);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
