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

// ------------------------------------------------------------ many workgroups
//
// The same grouping for tens of thousands of keys, spread over the chip in
// three launches instead of one workgroup's 16 wavefronts:
//   1. chunk c (kWideChunk consecutive keys, one wavefront) counts its keys
//      into an LDS histogram and writes it to hist[c][0 .. nkeys);
//   2. one workgroup runs, per key, an exclusive scan over the chunks (each
//      chunk's first position inside the key's run, written back in place)
//      and over the keys' totals (counts and offsets);
//   3. chunk c places its keys in input order from cursors offsets[key] +
//      hist[c][key], with the same ballot-based peer detection as the
//      one-workgroup placement.
// Chunks are in input order and placement within a chunk is in input order,
// so the permutation is the one-workgroup grouping's, bit for bit.

namespace moe {

namespace {

constexpr int kWideChunk = 512;  // keys per chunk: 8 per lane of one wavefront

__global__ __launch_bounds__(64) void group_hist_kernel(const int32_t* __restrict__ keys, int n, int nkeys,
                                                        int32_t* __restrict__ hist) {
  extern __shared__ int h[];  // [nkeys]
  const int c = blockIdx.x, lane = threadIdx.x;
  for (int i = lane; i < nkeys; i += 64) h[i] = 0;
  __syncthreads();
  const int lo = c * kWideChunk, hi = min(n, lo + kWideChunk);  // lo < n: the grid covers n exactly
  int kk[kWideChunk / 64];
#pragma unroll
  for (int j = 0; j < kWideChunk / 64; ++j) kk[j] = keys[min(lo + j * 64 + lane, hi - 1)];  // unconditional
#pragma unroll
  for (int j = 0; j < kWideChunk / 64; ++j) {
    const int key = kk[j];
    if (lo + j * 64 + lane < hi && key >= 0 && key < nkeys) atomicAdd(&h[key], 1);
  }
  __syncthreads();
  for (int i = lane; i < nkeys; i += 64) hist[(size_t)c * nkeys + i] = h[i];
}

// one workgroup of 1024 threads; nkeys <= 1024 (one key per thread)
__global__ __launch_bounds__(1024) void group_scan_kernel(int32_t* __restrict__ hist, int C, int nkeys,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets) {
  __shared__ int wsum[16];
  const int key = threadIdx.x, lane = key & 63, wave = key >> 6;
  int run = 0;
  if (key < nkeys) {
    // the chunks' counts of this key, 8 requested at a time
    for (int c0 = 0; c0 < C; c0 += 8) {
      int v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = hist[(size_t)min(c0 + j, C - 1) * nkeys + key];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (c0 + j < C) {
          hist[(size_t)(c0 + j) * nkeys + key] = run;
          run += v[j];
        }
    }
  }
  // exclusive scan of the totals over the keys: within each wavefront, then over wavefronts
  int incl = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  if (key < nkeys) {
    counts[key] = run;
    offsets[key] = before + incl - run;
  }
  if (key == 1023) offsets[nkeys] = before + incl;  // every key's run: the valid keys
}

__global__ __launch_bounds__(64) void group_place_kernel(const int32_t* __restrict__ keys, int n, int nkeys,
                                                         const int32_t* __restrict__ hist,
                                                         const int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ perm) {
  extern __shared__ int cur[];  // [nkeys]
  const int c = blockIdx.x, lane = threadIdx.x;
  for (int i = lane; i < nkeys; i += 64) cur[i] = offsets[i] + hist[(size_t)c * nkeys + i];
  __syncthreads();
  const int lo = c * kWideChunk, hi = min(n, lo + kWideChunk);
  int nbits = 1;
  while ((1 << nbits) < nkeys) ++nbits;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int kk[kWideChunk / 64];
#pragma unroll
  for (int j = 0; j < kWideChunk / 64; ++j) kk[j] = keys[min(lo + j * 64 + lane, hi - 1)];  // unconditional
#pragma unroll
  for (int j = 0; j < kWideChunk / 64; ++j) {
    const int i = lo + j * 64 + lane;
    int key = kk[j];
    const bool valid = i < hi && key >= 0 && key < nkeys;
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

}  // namespace

// Words of scratch the many-workgroup grouping needs (its per-chunk
// histograms), or 0 when n and nkeys call for the one-workgroup grouping.
size_t group_wide_scratch_ints(int n, int nkeys) {
  if (n <= 4 * kWideChunk || nkeys > 1024) return 0;
  const long C = (n + kWideChunk - 1) / kWideChunk;
  return (size_t)C * (size_t)nkeys;
}

// The grouping with per-chunk histograms in scratch (at least
// group_wide_scratch_ints(n, nkeys) ints, device memory); falls back to the
// one-workgroup grouping when that needs none.
moe_status launch_group_wide(const int32_t* keys, int n, int nkeys, int32_t* counts, int32_t* offsets,
                             int32_t* perm, int32_t* scratch, hipStream_t s) {
  if (group_wide_scratch_ints(n, nkeys) == 0) return launch_group(keys, n, nkeys, counts, offsets, perm, s);
  const int C = (n + kWideChunk - 1) / kWideChunk;
  const size_t lds = (size_t)nkeys * sizeof(int);
  launch(MOE_PROF_GROUP, group_hist_kernel, dim3(C), dim3(64), lds, s, keys, n, nkeys, scratch);
  MOE_LAUNCH_CHECK();
  launch(MOE_PROF_GROUP, group_scan_kernel, dim3(1), dim3(1024), 0, s, scratch, C, nkeys, counts, offsets);
  MOE_LAUNCH_CHECK();
  launch(MOE_PROF_GROUP, group_place_kernel, dim3(C), dim3(64), lds, s, keys, n, nkeys, (const int32_t*)scratch,
         (const int32_t*)offsets, perm);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
