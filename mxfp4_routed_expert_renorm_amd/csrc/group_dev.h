// Stable grouping of (token, rank) pairs by key: counts, exclusive offsets and
// the permutation that lists each key's pairs in ascending pair order.  A
// device function, run by the grouping kernel (moe_group) and by the batched
// decode GEMM's planning kernel.
//
// Grouping lets each selected expert's weights stream from HBM once for all
// the tokens that picked it ("An elephant through a straw", §43 graphs, 43
// syncs: the picks are classified and the grouped expert kernels fired).
//
// One 1024-thread workgroup.  The input is cut into W contiguous chunks, one
// per wavefront (W = 16 for up to ~1000 keys, fewer for more keys so the
// per-chunk histograms fit in LDS):
//   1. each wavefront counts its chunk's keys into its own LDS histogram;
//   2. per key, an exclusive scan over the chunks gives each chunk's first
//      position inside the key's run, and a scan over the keys' totals gives
//      the offsets;
//   3. each wavefront places its chunk 64 keys at a time in input order:
//      lanes holding the same key find each other with one ballot per key
//      bit, take their rank among the lower lanes, and the lowest lane of
//      the group advances the chunk's cursor for that key.
// Chunks are in input order and placement within a chunk is in input order,
// so the permutation is stable and identical run to run.
#pragma once

#include "common.h"

namespace moe {

constexpr int kGroupThreads = 1024;
constexpr int kGroupWaves = kGroupThreads / 64;
constexpr int kGroupLdsInts = 16384;  // 64 KiB of dynamic LDS

__host__ __device__ inline int group_chunks(int nkeys) {
  const int w = kGroupLdsInts / nkeys - 1;  // W histograms + the key totals
  return w < 1 ? 1 : (w > kGroupWaves ? kGroupWaves : w);
}

// The grouping, run by one whole workgroup of kGroupThreads threads with
// (W + 1) * nkeys ints of LDS at lds; every thread of the workgroup calls it.
__device__ __forceinline__ void group_body(const int32_t* __restrict__ keys, int n, int nkeys, int W,
                                           int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                           int32_t* __restrict__ perm, int* lds) {
  int* hist = lds;                // [W][nkeys]: counts, then cursors
  int* tot = lds + W * nkeys;     // [nkeys]: key totals, then key offsets
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = ((n + W - 1) / W + 63) / 64 * 64;
  const int lo = wave * chunk, hi = min(n, lo + chunk);
  for (int i = tid; i < W * nkeys; i += kGroupThreads) hist[i] = 0;
  __syncthreads();
  // 1. per-chunk histograms (16 keys per lane in flight: the loads are
  // unconditional, at clamped positions, and the out-of-range ones unused)
  if (wave < W && lo < hi) {
    int* hw = hist + wave * nkeys;
    for (int base = lo; base < hi; base += 16 * 64) {
      int kk[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) kk[j] = keys[min(base + j * 64 + lane, hi - 1)];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = kk[j];
        if (base + j * 64 + lane < hi && key >= 0 && key < nkeys) atomicAdd(&hw[key], 1);
      }
    }
  }
  __syncthreads();
  // 2. chunk prefix per key, then offsets over the keys
  for (int key = tid; key < nkeys; key += kGroupThreads) {
    int run = 0;
    for (int w = 0; w < W; ++w) {
      const int c = hist[w * nkeys + key];
      hist[w * nkeys + key] = run;
      run += c;
    }
    tot[key] = run;
  }
  __syncthreads();
  if (wave == 0) {
    int carry = 0;
    for (int base = 0; base < nkeys; base += 64) {
      const int i = base + lane;
      const int c = i < nkeys ? tot[i] : 0;
      int incl = c;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
      }
      if (i < nkeys) {
        tot[i] = carry + incl - c;
        offsets[i] = carry + incl - c;
        counts[i] = c;
      }
      carry += __shfl(incl, 63, 64);
    }
    if (lane == 0) offsets[nkeys] = carry;
  }
  __syncthreads();
  for (int i = tid; i < W * nkeys; i += kGroupThreads) hist[i] += tot[i % nkeys];
  __syncthreads();
  // 3. stable placement, one chunk per wavefront (an empty chunk loads nothing)
  if (wave < W && lo < hi) {
    int* cur = hist + wave * nkeys;
    int nbits = 1;
    while ((1 << nbits) < nkeys) ++nbits;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    // keys of the next kPF steps in registers, rotated one step at a time
    // (unconditional loads at clamped positions; positions past hi are invalid)
    constexpr int kPF = 8;
    int kb[kPF];
#pragma unroll
    for (int j = 0; j < kPF; ++j) kb[j] = keys[min(lo + j * 64 + lane, hi - 1)];
    for (int base = lo; base < hi; base += 64) {
      const int i = base + lane;
      int key = kb[0];
#pragma unroll
      for (int j = 0; j + 1 < kPF; ++j) kb[j] = kb[j + 1];
      kb[kPF - 1] = keys[min(base + kPF * 64 + lane, hi - 1)];
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
}

}  // namespace moe
