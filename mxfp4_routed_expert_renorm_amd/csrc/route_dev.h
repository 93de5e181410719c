// Wavefront top-k routing, shared by the router kernel and the batch-1
// decode kernel that routes its own token.
//
// Top-k follows "Running DeepSeek-V4-Flash across four free GPUs", §What the
// expert cache actually does (the router picks top_k experts per token) and
// "An elephant through a straw", §Not all six experts matter equally (weights
// per token, renormalised).  One 64-lane wavefront owns one token: each lane
// holds E/64 logits, and k rounds of a wavefront argmax over a packed 64-bit
// (value, inverted id) key pick the experts in rank order, ties to the lower
// id.  The renormalised softmax over the selected experts equals a softmax
// over their logits alone, so the full-E denominator is never formed.
#pragma once

#include "common.h"

namespace moe {

// Order-preserving unsigned image of a logit: -0 folded onto +0 and NaN onto
// -inf first, so equal images mean equal (canonical) values.  Every real
// logit maps above 0, which therefore means "no candidate".
__device__ __forceinline__ uint32_t sel_key(float v) {
  v = (v == v) ? v + 0.0f : -INFINITY;
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key ^ 0x80000000u) : ~key);
}

// wavefront maximum / minimum of an unsigned value, returned uniformly: DPP
// lane moves (butterflies in quads, mirrors in rows of 16, then row
// broadcasts), lanes without a source contribute the identity
template <bool MAX>
__device__ __forceinline__ uint32_t wave_ext_u32(uint32_t v) {
  constexpr int id = MAX ? 0 : -1;
  auto step = [&](uint32_t w) { return MAX ? (w > v ? w : v) : (w < v ? w : v); };
  v = step((uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, dpp::kQuadXor1, 0xF, 0xF, false));
  v = step((uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, dpp::kQuadXor2, 0xF, 0xF, false));
  v = step((uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, dpp::kRowHalfMirror, 0xF, 0xF, false));
  v = step((uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, dpp::kRowMirror, 0xF, 0xF, false));
  v = step((uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, dpp::kRowBcast15, 0xA, 0xF, false));
  v = step((uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, dpp::kRowBcast31, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Route one token's logits row [E] with the whole wavefront: on return lane
// r < k holds the r-th selected expert and its renormalised weight (other
// lanes: expert 0, weight 0).  Every lane must call it (DPP and readlane).
// Each round takes the wavefront maximum of the 32-bit images; among the
// positions holding it the lowest expert id wins (a ballot settles the
// common single-holder case, a wavefront minimum over ids the rest).
// The two halves of route_wave, for callers that issue other loads between
// the logits loads and the selection: lane l loads experts l + 64 j.
template <int EPL>
__device__ __forceinline__ void route_load(const float* __restrict__ row, int E, float (&v)[EPL]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < EPL; ++j) v[j] = row[min(lane + 64 * j, E - 1)];  // unconditional (clamped)
}

template <int EPL>
__device__ __forceinline__ void route_select(const float (&v)[EPL], int E, int k, int* my_e, float* my_w);

template <int EPL>
__device__ __forceinline__ void route_wave(const float* __restrict__ row, int E, int k, int* my_e, float* my_w) {
  float v[EPL];
  route_load<EPL>(row, E, v);
  route_select<EPL>(v, E, k, my_e, my_w);
}

template <int EPL>
__device__ __forceinline__ void route_select(const float (&lv)[EPL], int E, int k, int* my_e, float* my_w) {
  const int lane = threadIdx.x & 63;
  uint32_t key[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    key[j] = sel_key(lv[j]) & (0u - (uint32_t)(e < E));  // arithmetic mask: no branch around the load
  }
  uint32_t kv = 0;  // lane r keeps the r-th selected image
  int ee = 0;
  for (int r = 0; r < k; ++r) {
    uint32_t best = key[0];
#pragma unroll
    for (int j = 1; j < EPL; ++j) best = key[j] > best ? key[j] : best;
    const uint32_t m = wave_ext_u32<true>(best);
    uint32_t cid = 0xffffffffu;  // this lane's lowest expert id holding m
#pragma unroll
    for (int j = EPL - 1; j >= 0; --j) cid = key[j] == m ? (uint32_t)(lane + 64 * j) : cid;
    const uint64_t holders = __ballot(cid != 0xffffffffu);
    uint32_t win;
    if (__popcll(holders) == 1)
      win = (uint32_t)__builtin_amdgcn_readlane((int)cid, __builtin_ctzll(holders));
    else
      win = wave_ext_u32<false>(cid);
#pragma unroll
    for (int j = 0; j < EPL; ++j) key[j] = (uint32_t)(lane + 64 * j) == win ? 0u : key[j];
    if (lane == r) {
      kv = m;
      ee = (int)win;
    }
  }
  const float v = key_value(kv);
  const float vmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float z = (lane < k) ? expf(v - vmax) : 0.0f;
  const float s = wave_sum(z);
  *my_e = ee;
  *my_w = (lane < k) ? z / s : 0.0f;
}

}  // namespace moe
