// Device helpers shared by the batch-1 decode kernels (the two-launch step
// and the fused single-launch step): 32-element activation chunks, the FP4
// and 2-bit dot products over them, SwiGLU, and set-bit selection.
#pragma once

#include "common.h"

namespace moe {

__device__ __forceinline__ float silu_mul_b1(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// 32 bf16 activations (16 pairs) of one 32-element chunk
struct B1Chunk {
  uint32_t p[16];
  __device__ __forceinline__ void load_lds(const uint8_t* lds, size_t elem) {
    const uint4* src = (const uint4*)(lds + elem * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = src[i];
      p[4 * i] = v.x, p[4 * i + 1] = v.y, p[4 * i + 2] = v.z, p[4 * i + 3] = v.w;
    }
  }
  __device__ __forceinline__ void load_global(const void* base, size_t elem) {
    const uint4* src = (const uint4*)((const uint16_t*)base + elem);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = src[i];
      p[4 * i] = v.x, p[4 * i + 1] = v.y, p[4 * i + 2] = v.z, p[4 * i + 3] = v.w;
    }
  }
  // 32 FP4 codes (16 bytes, element 2j in the low nibble of byte j) . chunk
  __device__ __forceinline__ float fp4(const uint4 c) const {
    float a0 = 0.0f, a1 = 0.0f;
    const uint32_t d[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a0 = dot2_bf16(fp4x2_to_bf16x2<0>(d[i]), p[4 * i + 0], a0);
      a1 = dot2_bf16(fp4x2_to_bf16x2<1>(d[i]), p[4 * i + 1], a1);
      a0 = dot2_bf16(fp4x2_to_bf16x2<2>(d[i]), p[4 * i + 2], a0);
      a1 = dot2_bf16(fp4x2_to_bf16x2<3>(d[i]), p[4 * i + 3], a1);
    }
    return a0 + a1;
  }
  // acc0/acc1 += 32 FP4 codes . chunk, each code times the block scale
  // inside the convert (exact: bf16 holds every E2M1 value times any power
  // of two in range)
  __device__ __forceinline__ void fp4_acc(const uint4 c, float scale, float& acc0, float& acc1) const {
    const uint32_t d[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc0 = dot2_bf16(fp4x2_to_bf16x2_scaled<0>(d[i], scale), p[4 * i + 0], acc0);
      acc1 = dot2_bf16(fp4x2_to_bf16x2_scaled<1>(d[i], scale), p[4 * i + 1], acc1);
      acc0 = dot2_bf16(fp4x2_to_bf16x2_scaled<2>(d[i], scale), p[4 * i + 2], acc0);
      acc1 = dot2_bf16(fp4x2_to_bf16x2_scaled<3>(d[i], scale), p[4 * i + 3], acc1);
    }
  }
  // 32 2-bit codes (8 bytes, element 4j+q in bits 2q..2q+1 of byte j) . chunk
  __device__ __forceinline__ float int2(const uint2 c) const {
    float a0 = 0.0f, a1 = 0.0f;
    const uint32_t d[2] = {c.x, c.y};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int q = 0; q < 16; q += 2) {
        const uint32_t xp = p[8 * i + q / 2];
        a0 = fmaf((float)((d[i] >> (2 * q)) & 3u) - 1.5f, bf16_lo(xp), a0);
        a1 = fmaf((float)((d[i] >> (2 * q + 2)) & 3u) - 1.5f, bf16_hi(xp), a1);
      }
    }
    return a0 + a1;
  }
};

// position of the n-th set bit of m (n < popcount(m)); wave-uniform
__device__ __forceinline__ int nth_set_bit(uint64_t m, int n) {
  for (int t = 0; t < n; ++t) m &= m - 1;
  return __builtin_ctzll(m);
}

}  // namespace moe
