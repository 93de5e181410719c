// Router: top-k selection with renormalised weights, and the small router
// GEMV of the tiny configuration.
//
// Top-k follows "Running DeepSeek-V4-Flash across four free GPUs", §What the
// expert cache actually does (the router picks top_k experts per token) and
// "An elephant through a straw", §Not all six experts matter equally (weights
// per token, renormalised).  One 64-lane wavefront owns one token: each lane
// holds E/64 logits in registers, and k rounds of a wavefront argmax
// (butterfly over (value, id) pairs, ties to the lower id) pick the experts
// in rank order; the butterflies run on DPP lane moves over a packed 64-bit
// (value, inverted id) key.  The renormalised softmax over the selected experts equals a
// softmax over their logits alone, so the full-E denominator is never formed.
#include "common.h"

namespace moe {

namespace {

constexpr int kMaxE = 1024;
constexpr int kMaxEPL = kMaxE / 64;  // logits per lane

// Selection key of (logit v, expert e): the order-preserving unsigned image
// of v in the high word (-0 folded onto +0, NaN onto -inf) and the inverted
// id in the low word, so the largest key is the largest logit with ties to
// the lower id.  Key 0 means "no candidate".
__device__ __forceinline__ uint64_t sel_key(float v, int e) {
  v = (v == v) ? v + 0.0f : -INFINITY;
  const uint32_t u = __float_as_uint(v);
  const uint32_t hi = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)hi << 32) | (uint32_t)(0xffffffffu - (uint32_t)e);
}

__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t hi = (uint32_t)(key >> 32);
  return __uint_as_float((hi & 0x80000000u) ? (hi ^ 0x80000000u) : ~hi);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void dpp_max_step(uint32_t& hi, uint32_t& lo) {
  const uint32_t h2 = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, CTRL, ROW_MASK, 0xF, false);
  const uint32_t l2 = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, CTRL, ROW_MASK, 0xF, false);
  const bool take = (h2 > hi) || (h2 == hi && l2 > lo);
  hi = take ? h2 : hi;
  lo = take ? l2 : lo;
}

// maximum key over the wavefront, returned uniformly
__device__ __forceinline__ uint64_t wave_max_key(uint64_t key) {
  uint32_t hi = (uint32_t)(key >> 32), lo = (uint32_t)key;
  dpp_max_step<dpp::kQuadXor1, 0xF>(hi, lo);
  dpp_max_step<dpp::kQuadXor2, 0xF>(hi, lo);
  dpp_max_step<dpp::kRowHalfMirror, 0xF>(hi, lo);
  dpp_max_step<dpp::kRowMirror, 0xF>(hi, lo);
  dpp_max_step<dpp::kRowBcast15, 0xA>(hi, lo);
  dpp_max_step<dpp::kRowBcast31, 0xC>(hi, lo);
  const uint32_t h = (uint32_t)__builtin_amdgcn_readlane((int)hi, 63);
  const uint32_t l = (uint32_t)__builtin_amdgcn_readlane((int)lo, 63);
  return ((uint64_t)h << 32) | l;
}

template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                    int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wavefront exits together
  const float* row = logits + (size_t)t * E;
  uint64_t key[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    key[j] = (e < E) ? sel_key(row[e], e) : 0ull;
  }
  float my_v = -INFINITY;  // lane r keeps the r-th selected logit
  int my_e = 0;
  for (int r = 0; r < k; ++r) {
    uint64_t best = 0ull;
#pragma unroll
    for (int j = 0; j < EPL; ++j) best = key[j] > best ? key[j] : best;
    best = wave_max_key(best);
    const int be = (int)(0xffffffffu - (uint32_t)best);
    // the owner retires the winner
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (key[j] == best) key[j] = 0ull;
    if (lane == r) {
      my_v = key_value(best);
      my_e = be;
    }
  }
  const float vmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v), 0));
  const float z = (lane < k) ? expf(my_v - vmax) : 0.0f;
  const float s = wave_sum(z);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_e;
    w[(size_t)t * k + lane] = z / s;
  }
}

// logits[t][e] = x[t] . w_router[e]; one wavefront per (t, e)
template <bool XBF16>
__global__ __launch_bounds__(256) void router_logits_kernel(const void* __restrict__ x,
                                                            const float* __restrict__ wr, int T, int E,
                                                            int H, float* __restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= T * E) return;
  const int t = item / E, e = item % E;
  const float* wrow = wr + (size_t)e * H;
  float acc = 0.0f;
  for (int h = lane; h < H; h += 64) {
    float xv;
    if (XBF16) {
      xv = __uint_as_float((uint32_t)((const uint16_t*)x)[(size_t)t * H + h] << 16);
    } else {
      xv = ((const float*)x)[(size_t)t * H + h];
    }
    acc = fmaf(xv, wrow[h], acc);
  }
  acc = group_sum<64>(acc);
  if (lane == 0) logits[(size_t)t * E + e] = acc;
}

}  // namespace

moe_status launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s) {
  if (T == 0) return MOE_OK;
  const int epl = (E + 63) / 64;
  const dim3 grid((T + 3) / 4), block(256);
  ProfScope prof(MOE_PROF_ROUTE, s);
  if (epl <= 1) {
    hipLaunchKernelGGL(route_kernel<1>, grid, block, 0, s, logits, T, E, k, ids, w);
  } else if (epl <= 2) {
    hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, s, logits, T, E, k, ids, w);
  } else if (epl <= 4) {
    hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, s, logits, T, E, k, ids, w);
  } else if (epl <= 8) {
    hipLaunchKernelGGL(route_kernel<8>, grid, block, 0, s, logits, T, E, k, ids, w);
  } else {
    hipLaunchKernelGGL(route_kernel<kMaxEPL>, grid, block, 0, s, logits, T, E, k, ids, w);
  }
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

moe_status launch_router_logits(const void* x, moe_dtype xt, const float* wr, int T, int E, int H,
                                float* logits, hipStream_t s) {
  if (T == 0) return MOE_OK;
  const long items = (long)T * E;
  const dim3 grid((unsigned)((items + 3) / 4)), block(256);
  ProfScope prof(MOE_PROF_ROUTER_LOGITS, s);
  if (xt == MOE_BF16) {
    hipLaunchKernelGGL(router_logits_kernel<true>, grid, block, 0, s, x, wr, T, E, H, logits);
  } else {
    hipLaunchKernelGGL(router_logits_kernel<false>, grid, block, 0, s, x, wr, T, E, H, logits);
  }
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
