// One tensor-parallel share of MXFP4 expert records, cut along the expert
// intermediate dimension.
//
// "Running DeepSeek-V4-Flash across four free GPUs", §Step 2 (Pick your
// split, then check it divides): the tensor-parallel runtime gives every rank
// its own slice of each expert, and the split must fall on the FP4 32-element
// scale blocks.  Rank g of G keeps rows [g*I/G, (g+1)*I/G) of w1 and w3 (with
// their scale rows) and the same columns of w2 (with the scale blocks along
// I), so each rank's expert MLP gives a partial output and the G partials sum
// to the full one (the all-reduce that completes the layer).
#include <hip/hip_runtime.h>

#include "common.h"

using namespace moe;

extern "C" {

moe_status moe_tp_slice(const uint8_t* src, size_t src_stride, int n, int H, int I, int G, int g, uint8_t* dst,
                        size_t dst_stride, moe_stream_t stream) {
  if (n < 0 || H <= 0 || I <= 0 || H % 32) return fail(MOE_ESHAPE, "moe_tp_slice: n=%d H=%d I=%d", n, H, I);
  if (G < 1 || g < 0 || g >= G) return fail(MOE_EINVAL, "moe_tp_slice: rank g=%d of G=%d", g, G);
  if (I % G || (I / G) % 32)
    return fail(MOE_ESHAPE, "moe_tp_slice: G=%d does not cut I=%d on 32-element scale blocks", G, I);
  if (n == 0) return MOE_OK;
  if (!src || !dst) return fail(MOE_EINVAL, "moe_tp_slice: NULL pointer");
  const int Is = I / G, i0 = g * Is;
  const RecordLayout L = record_layout(H, I, 4), Ls = record_layout(H, Is, 4);
  if (src_stride < L.bytes || dst_stride < Ls.bytes)
    return fail(MOE_EINVAL, "moe_tp_slice: strides %zu / %zu below the record sizes %zu / %zu", src_stride,
                dst_stride, L.bytes, Ls.bytes);
  hipStream_t s = (hipStream_t)stream;
  for (int e = 0; e < n; ++e) {
    const uint8_t* r = src + (size_t)e * src_stride;
    uint8_t* o = dst + (size_t)e * dst_stride;
    // w1, w3 codes and scales: whole rows, contiguous
    MOE_HIP_CHECK(hipMemcpyAsync(o + Ls.w1c, r + L.w1c + (size_t)i0 * (H / 2), (size_t)Is * (H / 2),
                                 hipMemcpyDeviceToDevice, s));
    MOE_HIP_CHECK(hipMemcpyAsync(o + Ls.w3c, r + L.w3c + (size_t)i0 * (H / 2), (size_t)Is * (H / 2),
                                 hipMemcpyDeviceToDevice, s));
    MOE_HIP_CHECK(hipMemcpyAsync(o + Ls.w1s, r + L.w1s + (size_t)i0 * (H / 32), (size_t)Is * (H / 32),
                                 hipMemcpyDeviceToDevice, s));
    MOE_HIP_CHECK(hipMemcpyAsync(o + Ls.w3s, r + L.w3s + (size_t)i0 * (H / 32), (size_t)Is * (H / 32),
                                 hipMemcpyDeviceToDevice, s));
    // w2 codes and scales: a column band of every one of the H rows
    MOE_HIP_CHECK(hipMemcpy2DAsync(o + Ls.w2c, (size_t)Is / 2, r + L.w2c + (size_t)i0 / 2, (size_t)I / 2,
                                   (size_t)Is / 2, (size_t)H, hipMemcpyDeviceToDevice, s));
    MOE_HIP_CHECK(hipMemcpy2DAsync(o + Ls.w2s, (size_t)Is / 32, r + L.w2s + (size_t)i0 / 32, (size_t)I / 32,
                                   (size_t)Is / 32, (size_t)H, hipMemcpyDeviceToDevice, s));
  }
  return MOE_OK;
}

}  // extern "C"
