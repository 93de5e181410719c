// Device helpers shared by the batch-1 decode kernels (the two-launch step
// and the fused single-launch step): 32-element activation chunks, the FP4
// and 2-bit dot products over them, SwiGLU, set-bit selection, and the
// one-row products on the scaled FP4 matrix cores.
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

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// A weight row times x on the matrix cores, for one token, with
// v_mfma_scale_f32_16x16x128_f8f6f4 (A: x as E4M3, B: the FP4 weights and
// their E8M0 block scales exactly as stored, so no weight is converted).
// Operand layout on gfx950: lane l = 16h + c gives B column c as 32 FP4
// values at K [32h, 32h+32) with the scale of that block, and A row c as 32
// E4M3 bytes at K [16h, 16h+16) and [64+16h, 64+16h+16) with the scale of
// A's K block h.  A row's 16-byte chunk of lane l (weights 32l .. 32l+31,
// one scale block) is B column c's K block h, so if A row c holds at every K
// the x element of the weight at that K, tile entry (c, c) sums exactly the
// products of the lanes with l%16 = c, the tile's diagonal sums to the dot
// product over the 64 chunks, and the other entries (mismatched positions)
// are dropped.  x enters as two parts, each E4M3 under a power-of-two scale
// per 32-element block of x: hi under 2^(E-7) (E = floor(log2) of the
// block's largest magnitude, so hi stays below 256 and never saturates), lo
// = the remainder under 2^(E-11).  hi + lo is x exactly for every element
// within 2^13 of its block's largest (an E4M3 value holds 4 significant
// bits, bf16 8); below that the remainder's rounding error stays under
// 2^-21 of the block's largest.  Every product is exact and the tile sums in
// fp32.  t += row chunks (codes c, scale byte sc) . both parts of x.
__device__ __forceinline__ v4f tile_fp4_x(v8i xh, v8i xl, uint32_t sh, uint32_t sl, uint4 c, uint32_t sc, v4f t) {
  const v8i b = {(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
  t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(xh, b, t, 0, 4, 0, (int)sh, 0, (int)sc);
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(xl, b, t, 0, 4, 0, (int)sl, 0, (int)sc);
}

// The lane's share of the dot product held in tile t: the diagonal entry it
// holds, or zero.  The 16x16 result tile sits as entry (4(l/16) + j, l%16)
// in register j of lane l, so entry (m, m) is register m%4 of lane
// 16(m/4) + m.
__device__ __forceinline__ float tile_diag(v4f t, int lane) {
  const int j = lane & 3;
  const float lo = (j & 1) ? t[1] : t[0];
  const float hi = (j & 1) ? t[3] : t[2];
  const float v = (j & 2) ? hi : lo;
  return ((lane >> 4) == ((lane & 15) >> 2)) ? v : 0.0f;
}

// A group's h in LDS: lane l's 64 bytes (elements 32l .. 32l+31) as four
// 16-byte pieces, piece i in slot 4l + ((i + r) & 3) with a per-lane rotation
// r, so that the lanes' i-th 16-byte reads fall in different banks (with
// pieces in order, lanes 64 bytes apart would share banks four ways).  The
// rotation is conflict-free for 32 and for 64 banks of 4 bytes.
__device__ __forceinline__ int h_slot(int l, int i) { return 4 * l + ((i + ((l >> 1) ^ (l >> 3))) & 3); }


// Where elements o .. o+7 (o a multiple of 8) of chunk C (0..63) of a
// 2048-element stretch of x go in the A operand of tile_fp4_x: K =
// 32 (C / 16) + o of row C % 16, i.e. lane 16h + C % 16, bytes j .. j+7,
// with (h, j) = (K / 16, K % 16) below K = 64 and ((K - 64) / 16,
// 16 + K % 16) above.  The chunk's scales belong to lane C.
__device__ __forceinline__ void a_operand_pos(int C, int o, int& ln, int& j) {
  const int K = 32 * (C >> 4) + o;
  const int h = K < 64 ? K >> 4 : (K - 64) >> 4;
  j = K < 64 ? (K & 15) : 16 + (K & 15);
  ln = 16 * h + (C & 15);
}

// The two E4M3 parts (tile_fp4_x) of 8 bf16 activations (w: bf16 pairs,
// element 2i in the low half of w[i]) and the parts' scale exponents.  The
// 32-element block is the 8-element pieces of four neighbouring lanes
// (aligned), so every lane of the wavefront calls this together.
__device__ __forceinline__ void split_e4m3(uint4 w4, uint2& hi, uint2& lo, int& sh, int& sl) {
  const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
  float v[8], m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    m = fmaxf(m, fmaxf(fabsf(v[2 * i]), fabsf(v[2 * i + 1])));
  }
  m = fmaxf(m, __shfl_xor(m, 1, 64));
  m = fmaxf(m, __shfl_xor(m, 2, 64));
  const int E = (int)((__float_as_uint(m) >> 23) & 0xffu) - 127;  // floor(log2 m); zero or subnormal: -127
  sh = min(127, max(-127, E - 7));
  sl = min(127, max(-127, E - 11));
  uint32_t ch[2], cl[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    float vh[4], vl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) vh[i] = __builtin_amdgcn_ldexpf(v[4 * q + i], -sh);
    int c = __builtin_amdgcn_cvt_pk_fp8_f32(vh[0], vh[1], 0, false);
    c = __builtin_amdgcn_cvt_pk_fp8_f32(vh[2], vh[3], c, true);
    ch[q] = (uint32_t)c;
    const v2f d0 = __builtin_amdgcn_cvt_pk_f32_fp8(c, false), d1 = __builtin_amdgcn_cvt_pk_f32_fp8(c, true);
    vl[0] = __builtin_amdgcn_ldexpf(vh[0] - d0[0], sh - sl);  // the remainders are exact
    vl[1] = __builtin_amdgcn_ldexpf(vh[1] - d0[1], sh - sl);
    vl[2] = __builtin_amdgcn_ldexpf(vh[2] - d1[0], sh - sl);
    vl[3] = __builtin_amdgcn_ldexpf(vh[3] - d1[1], sh - sl);
    const int l2 = __builtin_amdgcn_cvt_pk_fp8_f32(vl[0], vl[1], 0, false);
    cl[q] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(vl[2], vl[3], l2, true);
  }
  hi = make_uint2(ch[0], ch[1]);
  lo = make_uint2(cl[0], cl[1]);
}

}  // namespace moe
