// Router kernels: top-k selection with renormalised weights (one wavefront
// per token, see route_dev.h), and the small router GEMV of the tiny
// configuration.
#include "route_dev.h"

namespace moe {

namespace {

constexpr int kMaxE = 1024;
constexpr int kMaxEPL = kMaxE / 64;  // logits per lane

template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                    int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wavefront exits together
  int e;
  float wt;
  route_wave<EPL>(logits + (size_t)t * E, E, k, &e, &wt);
  if (lane < k) {
    ids[(size_t)t * k + lane] = e;
    w[(size_t)t * k + lane] = wt;
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
  if (epl <= 1) {
    launch(MOE_PROF_ROUTE, route_kernel<1>, grid, block, 0, s, logits, T, E, k, ids, w);
  } else if (epl <= 2) {
    launch(MOE_PROF_ROUTE, route_kernel<2>, grid, block, 0, s, logits, T, E, k, ids, w);
  } else if (epl <= 4) {
    launch(MOE_PROF_ROUTE, route_kernel<4>, grid, block, 0, s, logits, T, E, k, ids, w);
  } else if (epl <= 8) {
    launch(MOE_PROF_ROUTE, route_kernel<8>, grid, block, 0, s, logits, T, E, k, ids, w);
  } else {
    launch(MOE_PROF_ROUTE, route_kernel<kMaxEPL>, grid, block, 0, s, logits, T, E, k, ids, w);
  }
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

moe_status launch_router_logits(const void* x, moe_dtype xt, const float* wr, int T, int E, int H,
                                float* logits, hipStream_t s) {
  if (T == 0) return MOE_OK;
  const long items = (long)T * E;
  const dim3 grid((unsigned)((items + 3) / 4)), block(256);
  if (xt == MOE_BF16) {
    launch(MOE_PROF_ROUTER_LOGITS, router_logits_kernel<true>, grid, block, 0, s, x, wr, T, E, H, logits);
  } else {
    launch(MOE_PROF_ROUTER_LOGITS, router_logits_kernel<false>, grid, block, 0, s, x, wr, T, E, H, logits);
  }
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
