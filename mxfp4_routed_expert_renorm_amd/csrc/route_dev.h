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

#include <utility>

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

// wavefront maximum / minimum of an unsigned value, in every lane: DPP lane
// moves within each row of 16 (butterflies in quads, then the mirrors), then
// gfx950's permlane swaps across row pairs and across the two halves.
// Nothing goes through a scalar register, so a selection round has no
// vector-to-scalar round trip.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_ext_u32(uint32_t v) {
  auto step = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, dpp::kQuadXor1, 0xF, 0xF, false));
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, dpp::kQuadXor2, 0xF, 0xF, false));
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, dpp::kRowHalfMirror, 0xF, 0xF, false));
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, dpp::kRowMirror, 0xF, 0xF, false));
  // every lane now holds its row's result; rows 2j and 2j+1 swap (p[0] the
  // even row's, p[1] the odd row's), then the halves (q[0] the low half's)
  const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = step(p[0], p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return step(q[0], q[1]);
}

// Route one token's logits row [E] with the whole wavefront: on return lane
// r < k holds the r-th selected expert and its renormalised weight (other
// lanes: expert 0, weight 0).  Every lane must call it (DPP and readlane).
// Each round takes the wavefront maximum of the 32-bit images, then the
// wavefront minimum of the expert ids holding it (the lowest id wins a tie),
// both left in every lane.
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

// The parts of the selection.  route_keys: the lane's order-preserving images
// (experts past E hold 0, "no candidate").  route_round: one round — the
// wavefront maximum m, the lowest expert id holding it (win, in every lane),
// that candidate removed, and lane r keeping (m, win).  route_finish: the
// softmax over the k selected logits, lane r < k getting rank r's weight.
template <int EPL>
__device__ __forceinline__ void route_keys(const float (&lv)[EPL], int E, uint32_t (&key)[EPL]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    key[j] = sel_key(lv[j]) & (0u - (uint32_t)(e < E));  // arithmetic mask: no branch around the load
  }
}

template <int EPL>
__device__ __forceinline__ uint32_t route_round(uint32_t (&key)[EPL], int r, uint32_t& kv, int& ee) {
  const int lane = threadIdx.x & 63;
  uint32_t best = key[0];
#pragma unroll
  for (int j = 1; j < EPL; ++j) best = key[j] > best ? key[j] : best;
  const uint32_t m = wave_ext_u32<true>(best);
  uint32_t cid = 0xffffffffu;  // this lane's lowest expert id holding m
#pragma unroll
  for (int j = EPL - 1; j >= 0; --j) cid = key[j] == m ? (uint32_t)(lane + 64 * j) : cid;
  const uint32_t win = wave_ext_u32<false>(cid);
#pragma unroll
  for (int j = 0; j < EPL; ++j) key[j] = (uint32_t)(lane + 64 * j) == win ? 0u : key[j];
  if (lane == r) {
    kv = m;
    ee = (int)win;
  }
  return win;
}

__device__ __forceinline__ void route_finish(uint32_t kv, int ee, int k, int* my_e, float* my_w) {
  const int lane = threadIdx.x & 63;
  const float v = key_value(kv);
  const float vmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float z = (lane < k) ? expf(v - vmax) : 0.0f;
  const float s = wave_sum(z);
  *my_e = ee;
  *my_w = (lane < k) ? z / s : 0.0f;
}

template <int EPL>
__device__ __forceinline__ void route_select(const float (&lv)[EPL], int E, int k, int* my_e, float* my_w) {
  uint32_t key[EPL];
  route_keys<EPL>(lv, E, key);
  uint32_t kv = 0;  // lane r keeps the r-th selected image
  int ee = 0;
  for (int r = 0; r < k; ++r) route_round<EPL>(key, r, kv, ee);
  route_finish(kv, ee, k, my_e, my_w);
}

// f(std::integral_constant<int, r>()) for r = rs... in order
template <class F, int... rs>
__device__ __forceinline__ void for_each_index(F&& f, std::integer_sequence<int, rs...>) {
  (f(std::integral_constant<int, rs>()), ...);
}

// route_select with the rounds unrolled to R >= k and a call after each one,
// for a caller that requests each rank's data as soon as its round picks it:
// on_pick(std::integral_constant<int, r>(), e) with e the rank-r expert,
// wavefront-uniform; the rounds past k pass rank k-1's expert again, so the
// caller issues the same number of requests whatever k is.
template <int EPL, int R, class OnPick>
__device__ __forceinline__ void route_select_each(const float (&lv)[EPL], int E, int k, int* my_e, float* my_w,
                                                  OnPick&& on_pick) {
  uint32_t key[EPL];
  route_keys<EPL>(lv, E, key);
  uint32_t kv = 0;
  int ee = 0;
  uint32_t last = 0;
  auto round = [&](auto rc) {
    constexpr int r = decltype(rc)::value;
    if (r < k) last = __builtin_amdgcn_readfirstlane(route_round<EPL>(key, r, kv, ee));
    on_pick(rc, last);
  };
  for_each_index(round, std::make_integer_sequence<int, R>());
  route_finish(kv, ee, k, my_e, my_w);
}

}  // namespace moe
