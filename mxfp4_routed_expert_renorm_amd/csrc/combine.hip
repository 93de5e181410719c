// Weighted combine of the per-rank expert outputs back into the token stream.
//
// "Running DeepSeek-V4-Flash across four free GPUs", §What the expert cache
// actually does: the expert GEMM takes the token weights; "An elephant
// through a straw", §Not all six experts matter equally: dropped ranks leave
// the sum and the survivors' weights are renormalised (done before this
// kernel).  Each thread owns four consecutive outputs of one token and sums
// the ranks in rank order with fp32 FMAs, adds the shared expert with weight
// one, and rounds once to the output type.
#include "common.h"

namespace moe {

namespace {

template <bool OBF16>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, const float* __restrict__ w,
                                                      const int8_t* __restrict__ prec, int T, int k, int H,
                                                      int has_shared, void* __restrict__ out) {
  const int K1 = k + has_shared;
  const int quads = H / 4;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)T * quads) return;
  const int t = (int)(idx / quads), j = (int)(idx % quads) * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const float* yt = y + (size_t)t * K1 * H + j;
  for (int r = 0; r < k; ++r) {
    if (prec && prec[(size_t)t * k + r] < 0) continue;
    const float wr = w[(size_t)t * k + r];
    const float4 v = *(const float4*)(yt + (size_t)r * H);
    acc.x = fmaf(wr, v.x, acc.x);
    acc.y = fmaf(wr, v.y, acc.y);
    acc.z = fmaf(wr, v.z, acc.z);
    acc.w = fmaf(wr, v.w, acc.w);
  }
  if (has_shared) {
    const float4 v = *(const float4*)(yt + (size_t)k * H);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  if (OBF16) {
    uint16_t* o = (uint16_t*)out + (size_t)t * H + j;
    const uint32_t lo = (uint32_t)f32_to_bf16(acc.x) | ((uint32_t)f32_to_bf16(acc.y) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(acc.z) | ((uint32_t)f32_to_bf16(acc.w) << 16);
    *(uint2*)o = make_uint2(lo, hi);
  } else {
    *(float4*)((float*)out + (size_t)t * H + j) = acc;
  }
}

}  // namespace

moe_status launch_combine(const float* y, const float* w, const int8_t* prec, int T, int k, int H, int has_shared,
                          void* out, moe_dtype ot, hipStream_t s) {
  if (T == 0) return MOE_OK;
  const long n = (long)T * (H / 4);
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (ot == MOE_BF16)
    launch(MOE_PROF_COMBINE, combine_kernel<true>, grid, block, 0, s, y, w, prec, T, k, H, has_shared, out);
  else
    launch(MOE_PROF_COMBINE, combine_kernel<false>, grid, block, 0, s, y, w, prec, T, k, H, has_shared, out);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe

