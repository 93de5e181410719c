// Router: top-k selection with renormalised weights, and the small router
// GEMV of the tiny configuration.
//
// Top-k follows "Running DeepSeek-V4-Flash across four free GPUs", §What the
// expert cache actually does (the router picks top_k experts per token) and
// "An elephant through a straw", §Not all six experts matter equally (weights
// per token, renormalised).  One 64-lane wavefront owns one token: each lane
// holds E/64 logits in registers, and k rounds of a wavefront argmax
// (butterfly over (value, id) pairs, ties to the lower id) pick the experts
// in rank order.  The renormalised softmax over the selected experts equals a
// softmax over their logits alone, so the full-E denominator is never formed.
#include "common.h"

namespace moe {

namespace {

constexpr int kMaxE = 1024;
constexpr int kMaxEPL = kMaxE / 64;  // logits per lane

// (v, e) beats (v2, e2) if larger, ties to the lower id.  NaN never wins.
__device__ __forceinline__ bool beats(float v, int e, float v2, int e2) {
  return (v > v2) || (v == v2 && e < e2);
}

template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                    int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wavefront exits together
  const float* row = logits + (size_t)t * E;
  float v[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    float x = (e < E) ? row[e] : -INFINITY;
    v[j] = (x == x) ? x : -INFINITY;  // NaN treated as -inf
  }
  uint32_t taken = 0;  // bit j: v[j] already selected
  float my_v = -INFINITY;  // lane r keeps the r-th selected logit
  int my_e = 0;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      if (e < E && !((taken >> j) & 1u) && beats(v[j], e, bv, be)) {
        bv = v[j];
        be = e;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      if (beats(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    // every lane now holds the winner; its owner marks it taken
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == r) {
      my_v = bv;
      my_e = be;
    }
  }
  const float vmax = __shfl(my_v, 0, 64);
  const float z = (lane < k) ? expf(my_v - vmax) : 0.0f;
  float s = z;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
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
