// Dequantise one matrix of an expert record to fp32 with the decode steps the
// expert kernels use, so the formats can be checked bit for bit against the
// oracle:
//   mode 0: the gfx950 FP4 convert at scale 1.0, times the E8M0 block scale in
//           fp32 (the grouped kernels apply the scale to each 32-element
//           partial sum, so their factors are these two);
//   mode 1: the 2-bit level (code - 1.5) times the E4M3 block scale;
//   mode 2: the scaled FP4 convert to bf16 with the E8M0 block scale as the
//           convert's own scale operand, widened to fp32: the decode of the
//           batch-1, single-launch and batched-decode kernels.
#include <algorithm>

#include "common.h"

namespace moe {

namespace {

// one thread per 4 code bytes (8 FP4 or 16 two-bit elements)
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales, int rows, int cols,
                                                      int bits, int scaled, float* __restrict__ out) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const int per_dw = 32 / bits;  // elements per dword
  const long ndw = (long)rows * cols / per_dw;
  if (idx >= ndw) return;
  const long e0 = idx * per_dw;
  const int r = (int)(e0 / cols), c0 = (int)(e0 % cols);
  const uint32_t dw = ((const uint32_t*)codes)[idx];
  const uint32_t sb = scales[(size_t)r * (cols / 32) + c0 / 32];
  float* o = out + e0;
  if (bits == 4 && scaled) {
    const float s = e8m0_to_f32(sb);
    const uint32_t p0 = fp4x2_to_bf16x2_scaled<0>(dw, s), p1 = fp4x2_to_bf16x2_scaled<1>(dw, s),
                   p2 = fp4x2_to_bf16x2_scaled<2>(dw, s), p3 = fp4x2_to_bf16x2_scaled<3>(dw, s);
    o[0] = bf16_lo(p0); o[1] = bf16_hi(p0); o[2] = bf16_lo(p1); o[3] = bf16_hi(p1);
    o[4] = bf16_lo(p2); o[5] = bf16_hi(p2); o[6] = bf16_lo(p3); o[7] = bf16_hi(p3);
  } else if (bits == 4) {
    const float s = e8m0_to_f32(sb);
    const v2f a0 = fp4x2_to_f32<0>(dw), a1 = fp4x2_to_f32<1>(dw), a2 = fp4x2_to_f32<2>(dw),
              a3 = fp4x2_to_f32<3>(dw);
    o[0] = a0.x * s; o[1] = a0.y * s; o[2] = a1.x * s; o[3] = a1.y * s;
    o[4] = a2.x * s; o[5] = a2.y * s; o[6] = a3.x * s; o[7] = a3.y * s;
  } else {
    const float s = e4m3_to_f32(sb);
    for (int q = 0; q < 16; ++q) o[q] = ((float)((dw >> (2 * q)) & 3u) - 1.5f) * s;
  }
}

}  // namespace

moe_status launch_dequant(const uint8_t* record, int H, int I, int prec, int matrix, float* out, hipStream_t s) {
  const int bits = prec == 1 ? 2 : 4;
  const RecordLayout L = record_layout(H, I, bits);
  const size_t coff[3] = {L.w1c, L.w3c, L.w2c}, soff[3] = {L.w1s, L.w3s, L.w2s};
  const int rows = matrix == 2 ? H : I, cols = matrix == 2 ? I : H;
  const long ndw = (long)rows * cols / (32 / bits);
  launch(MOE_PROF_DEQUANT, dequant_kernel, dim3((unsigned)((ndw + 255) / 256)), dim3(256), 0, s, record + coff[matrix],
                     record + soff[matrix], rows, cols, bits, prec == 2 ? 1 : 0, out);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

namespace {

// grid-stride read of the buffer with non-temporal 16-byte loads; the sum is
// stored only under a condition the data cannot meet, so nothing is written
__global__ __launch_bounds__(256) void stream_read_kernel(const uint8_t* __restrict__ buf, long n16,
                                                          uint32_t* __restrict__ sink) {
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n16; i += (long)gridDim.x * 256)
    acc += __builtin_nontemporal_load((const u32x4_t*)buf + i);
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u && acc.x == 0x7f4a7c15u) sink[0] = acc.y;
}

}  // namespace

moe_status launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s) {
  const long n16 = (long)(bytes / 16);
  const long grid = std::min<long>(std::max<long>((n16 + 255) / 256, 1), 2048);
  launch(MOE_PROF_READ, stream_read_kernel, dim3((unsigned)grid), dim3(256), 0, s, (const uint8_t*)buf, n16, sink);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
