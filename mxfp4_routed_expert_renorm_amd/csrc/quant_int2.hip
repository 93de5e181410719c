// The 2-bit fallback copy of MXFP4 expert records, made on the GPU.
//
// "An elephant through a straw" (opening section; §Rig, model & methodology)
// keeps a 2-bit copy of every expert next to its MXFP4 original, with one fp8
// E4M3 scale per 32 weights chosen by clip search, made offline.  Per 32-weight
// group: each clip ratio alpha (1.00 down to 0.50 in steps of 0.05) proposes
// the scale s nearest (ties to even) to alpha * amax / 1.5 among the E4M3
// values, every weight takes its nearest level (c - 1.5) s, c in 0..3 (round
// half to even of w / s + 1.5, clamped), and the ratio with the least squared
// error, summed in element order, wins (ties to the larger ratio).  A scale
// that rounds to zero gives every weight the level 0 (code 2).
//
// One thread per group, all arithmetic in float64 one IEEE operation at a
// time (no fused multiply-adds), so the choices are reproducible exactly.
// Off the hot path: run once per record, before records are used.
#include "common.h"

namespace moe {

namespace {

// nearest E4M3 (E4M3FN) code of t >= 0, ties to the even code, saturating at 448
__device__ __forceinline__ uint32_t e4m3_nearest(double t) {
  if (!(t > 0.0)) return 0u;
  if (t >= 448.0) return 0x7Eu;
  if (t < 0.015625) return (uint32_t)rint(ldexp(t, 9));  // subnormals: steps of 2^-9 (8 is 2^-6, code 0x08)
  int e = ilogb(t);                                        // -6 .. 8
  double q = rint((ldexp(t, -e) - 1.0) * 8.0);             // mantissa eighths
  if (q == 8.0) {
    q = 0.0;
    ++e;
  }
  return (uint32_t)(((e + 7) << 3) | (int)q);
}

__device__ __forceinline__ double e4m3_value_d(uint32_t code) {
  const int ef = (int)((code >> 3) & 15u), m = (int)(code & 7u);
  return ef == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), ef - 10);
}

__global__ __launch_bounds__(256) void int2_from_fp4_kernel(const uint8_t* __restrict__ src, size_t src_stride,
                                                            uint8_t* __restrict__ dst, size_t dst_stride, int H, int I,
                                                            long nblk) {
#pragma clang fp contract(off)
  const long b = (long)blockIdx.x * 256 + threadIdx.x;  // group of the record
  if (b >= nblk) return;
  const uint8_t* rec = src + (size_t)blockIdx.y * src_stride;
  uint8_t* out = dst + (size_t)blockIdx.y * dst_stride;
  const RecordLayout L4 = record_layout(H, I, 4), L2 = record_layout(H, I, 2);
  const long per = (long)H * I / 32;  // groups per matrix
  const int mat = (int)(b / per);
  const long g = b - (long)mat * per;  // groups of a matrix follow its row-major element order
  const size_t c4 = (mat == 0 ? L4.w1c : mat == 1 ? L4.w3c : L4.w2c) + (size_t)g * 16;
  const size_t s4 = (mat == 0 ? L4.w1s : mat == 1 ? L4.w3s : L4.w2s) + (size_t)g;
  const size_t c2 = (mat == 0 ? L2.w1c : mat == 1 ? L2.w3c : L2.w2c) + (size_t)g * 8;
  const size_t s2 = (mat == 0 ? L2.w1s : mat == 1 ? L2.w3s : L2.w2s) + (size_t)g;

  // the group's 32 MXFP4 weights, exactly, in float64
  const uint4 q = *(const uint4*)(rec + c4);
  const double sc = ldexp(1.0, (int)rec[s4] - 127);
  const uint32_t d[4] = {q.x, q.y, q.z, q.w};
  double w[32];
  double amax = 0.0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t nib = (d[i / 8] >> (4 * (i % 8))) & 15u;  // element 2j: low nibble of byte j
    const uint32_t mag = nib & 7u;
    const double v = mag < 4u ? 0.5 * (double)mag : (double)(1u << (mag / 2u - 1u)) * (mag & 1u ? 1.5 : 1.0);
    w[i] = (nib & 8u) ? -(v * sc) : v * sc;
    amax = fmax(amax, fabs(w[i]));
  }

  constexpr double kAlpha[11] = {1.00, 0.95, 0.90, 0.85, 0.80, 0.75, 0.70, 0.65, 0.60, 0.55, 0.50};
  double best = INFINITY;
  uint32_t bc0 = 0xAAAAAAAAu, bc1 = 0xAAAAAAAAu, bs = 0u;  // code 2 everywhere, scale 0
  for (int a = 0; a < 11; ++a) {
    const double t = (kAlpha[a] * amax) / 1.5;
    const uint32_t scode = e4m3_nearest(t);
    const double s = e4m3_value_d(scode);
    uint32_t cw0 = 0u, cw1 = 0u;
    double err = 0.0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      int c = 2;
      if (s > 0.0) c = (int)fmin(fmax(rint(w[i] / s + 1.5), 0.0), 3.0);
      const double wh = ((double)c - 1.5) * s;
      const double dd = w[i] - wh;
      err = err + dd * dd;
      if (i < 16)
        cw0 |= (uint32_t)c << (2 * i);  // element 4j+q: bits 2q..2q+1 of byte j
      else
        cw1 |= (uint32_t)c << (2 * (i - 16));
    }
    if (err < best) {
      best = err;
      bc0 = cw0, bc1 = cw1, bs = scode;
    }
  }
  *(uint2*)(out + c2) = make_uint2(bc0, bc1);
  out[s2] = (uint8_t)bs;
}

}  // namespace

}  // namespace moe

using namespace moe;

extern "C" {

moe_status moe_int2_from_fp4(const uint8_t* src, size_t src_stride, int n, int H, int I, uint8_t* dst,
                             size_t dst_stride, moe_stream_t stream) {
  if (n < 0 || n > 65535) return fail(MOE_ESHAPE, "moe_int2_from_fp4: n=%d outside 0..65535", n);
  if (H <= 0 || I <= 0 || H % 32 != 0 || I % 32 != 0)
    return fail(MOE_ESHAPE, "moe_int2_from_fp4: H=%d I=%d must be positive multiples of 32", H, I);
  if (n == 0) return MOE_OK;
  if (!src || !dst) return fail(MOE_EINVAL, "moe_int2_from_fp4: NULL pointer");
  const size_t b4 = record_layout(H, I, 4).bytes, b2 = record_layout(H, I, 2).bytes;
  if ((n > 1 && src_stride < b4) || (n > 1 && dst_stride < b2) || src_stride % 16 != 0 || dst_stride % 8 != 0)
    return fail(MOE_EINVAL, "moe_int2_from_fp4: strides %zu, %zu must be >= %zu, %zu and multiples of 16, 8", src_stride,
                dst_stride, b4, b2);
  if ((uintptr_t)src % 16 != 0 || (uintptr_t)dst % 8 != 0)
    return fail(MOE_EINVAL, "moe_int2_from_fp4: src must be 16-byte and dst 8-byte aligned");
  const long nblk = 3L * H * I / 32;
  launch(MOE_PROF_QUANT, int2_from_fp4_kernel, dim3((unsigned)((nblk + 255) / 256), (unsigned)n), dim3(256), 0,
         (hipStream_t)stream, src, src_stride, dst, dst_stride, H, I, nblk);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // extern "C"
