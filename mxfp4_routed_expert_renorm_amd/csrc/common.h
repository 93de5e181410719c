// Internal helpers of the gfx950 MoE library: device-side format decoding,
// wavefront reductions, the expert record layout and host error plumbing.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <string>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------------------
// expert record layout (shared by every kernel; the byte order is fixed by
// the public header): w1 codes | w3 codes | w2 codes | w1 scales | w3 scales
// | w2 scales, each matrix [out][in] row-major, one scale per 32 inputs.
struct RecordLayout {
  size_t w1c, w3c, w2c, w1s, w3s, w2s, bytes;
};

__host__ __device__ inline RecordLayout record_layout(int H, int I, int bits) {
  const size_t n = (size_t)H * (size_t)I;
  const size_t cb = n * (size_t)bits / 8;  // code bytes per matrix
  const size_t sb = n / 32;                // scale bytes per matrix
  RecordLayout L;
  L.w1c = 0;
  L.w3c = cb;
  L.w2c = 2 * cb;
  L.w1s = 3 * cb;
  L.w3s = 3 * cb + sb;
  L.w2s = 3 * cb + 2 * sb;
  L.bytes = 3 * cb + 3 * sb;
  return L;
}

// ---------------------------------------------------------------------------
// scalar formats

// E8M0 scale byte -> float 2^(e-127); 0 -> 2^-127 (a float32 subnormal);
// 255 -> NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  uint32_t bits = e << 23;
  bits = (e == 0u) ? 0x00400000u : bits;
  bits = (e == 255u) ? 0x7fc00000u : bits;
  return __uint_as_float(bits);
}

// FP8 E4M3 (OCP E4M3FN: bias 7, no infinities, S.1111.111 = NaN) -> float.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t s = (b >> 7) & 1u, ef = (b >> 3) & 15u, m = b & 7u;
  float v;
  if (ef == 0u) {
    v = (float)m * 0.001953125f;  // m/8 * 2^-6
  } else {
    v = __uint_as_float(((ef + 120u) << 23) | (m << 20));
  }
  if (ef == 15u && m == 7u) v = __uint_as_float(0x7fc00000u);
  return s ? -v : v;
}

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// float -> bfloat16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// streaming loads of expert weights: read once per step, so they are fetched
// non-temporally (no reuse to protect in the caches)

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld_stream16(const uint8_t* p) {
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint2 ld_stream8(const uint8_t* p) {
  const u32x2_t v = __builtin_nontemporal_load((const u32x2_t*)p);
  return make_uint2(v.x, v.y);
}

// ---------------------------------------------------------------------------
// packed conversions (gfx950 scaled FP4 converts, scale 1.0: the block scale
// is applied once per 32 products)

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// element 2j of a byte is its low nibble; sel picks the byte of the dword
template <int SEL>
__device__ __forceinline__ v2f fp4x2_to_f32(uint32_t dw) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(dw, 1.0f, SEL);
}

template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t dw) {
  v2bf r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, 1.0f, SEL);
  return __builtin_bit_cast(uint32_t, r);
}

// the same convert with a block scale applied: bf16(E2M1 value * scale);
// exact for a power-of-two scale (including 2^-127 and NaN, every E8M0 byte)
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2_scaled(uint32_t dw, float scale) {
  v2bf r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, scale, SEL);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, a), __builtin_bit_cast(v2bf, b), c, false);
}

// ---------------------------------------------------------------------------
// wavefront reductions over aligned groups of N lanes (N a power of two <= 64)

template <int N>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = N / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Full-wavefront reductions on DPP lane moves (no LDS crossbar): butterfly
// within quads, mirrors within rows of 16, then row broadcasts fold the four
// rows so that lane 63 ends up with the result over all 64 lanes.
namespace dpp {
constexpr int kQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
constexpr int kRowBcast15 = 0x142;
constexpr int kRowBcast31 = 0x143;
}  // namespace dpp

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

// sum over each aligned group of 8 lanes, in every lane of the group: the
// quads' butterflies, then the mirror within the 8 (lane i and 7 - i hold
// the two quads' sums)
__device__ __forceinline__ float group8_sum_dpp(float v) {
  v += dpp_f32<dpp::kQuadXor1>(v);
  v += dpp_f32<dpp::kQuadXor2>(v);
  v += dpp_f32<dpp::kRowHalfMirror>(v);
  return v;
}

// sum over the 64 lanes, valid in lane 63
__device__ __forceinline__ float wave_sum_to_lane63(float v) {
  v += dpp_f32<dpp::kQuadXor1>(v);
  v += dpp_f32<dpp::kQuadXor2>(v);
  v += dpp_f32<dpp::kRowHalfMirror>(v);
  v += dpp_f32<dpp::kRowMirror>(v);
  v += dpp_f32<dpp::kRowBcast15, 0xA>(v);
  v += dpp_f32<dpp::kRowBcast31, 0xC>(v);
  return v;
}

// sum over the 64 lanes, uniform (every lane gets it)
__device__ __forceinline__ float wave_sum(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_sum_to_lane63(v)), 63));
}

// ---------------------------------------------------------------------------
// host-side error plumbing

void set_error(const char* fmt, ...);
moe_status fail(moe_status st, const char* fmt, ...);

#define MOE_HIP_CHECK(expr)                                                      \
  do {                                                                           \
    hipError_t _e = (expr);                                                      \
    if (_e != hipSuccess)                                                        \
      return ::moe::fail(MOE_EHIP, "%s failed: %s", #expr, hipGetErrorString(_e)); \
  } while (0)

#define MOE_LAUNCH_CHECK()                                                       \
  do {                                                                           \
    hipError_t _e = hipGetLastError();                                           \
    if (_e != hipSuccess)                                                        \
      return ::moe::fail(MOE_EHIP, "kernel launch failed: %s", hipGetErrorString(_e)); \
  } while (0)

// ---------------------------------------------------------------------------
// launches, timed when profiling is on (moe_profile_begin): each launch then
// gets its own event pair, recorded by the dispatch itself at the kernel's
// start and end (hipExtLaunchKernel), so the elapsed time is the kernel's
// duration on the device, not the gap between two stream commands

// a fresh event pair for a launch of `kind`; false when profiling is off
bool prof_events(int kind, hipEvent_t* start, hipEvent_t* stop);

template <typename F, typename... Args>
inline void launch(int kind, F kernel, dim3 grid, dim3 block, size_t shmem, hipStream_t s, Args... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (prof_events(kind, &e0, &e1))
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)shmem, s, e0, e1, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
}

// ---------------------------------------------------------------------------
// internal launchers (each validates nothing: the C entry points do)

struct ExpertArgs;  // defined in expert_decode.hip
moe_status launch_expert_decode(const moe_layer* L, const void* x, moe_dtype xt, int T, int k,
                                const int32_t* slot_ids, const int8_t* prec, float* h, float* y,
                                int32_t* plan, hipStream_t s);
moe_status launch_combine(const float* y, const float* w, const int8_t* prec, int T, int k, int H,
                          int has_shared, void* out, moe_dtype ot, hipStream_t s);
moe_status launch_group(const int32_t* keys, int n, int nkeys, int32_t* counts, int32_t* offsets,
                        int32_t* perm, hipStream_t s);
// slot cache exchange: device picks -> mapped pinned host memory, and back
// (flag_h: a word of the same mapped buffer that receives seq after the picks)
moe_status launch_cache_gather(const int32_t* ids, const float* w, int n, int32_t* ids_h, float* w_h, uint32_t* flag_h,
                               uint32_t seq, hipStream_t s);
moe_status launch_cache_scatter(const int32_t* slots_h, const float* w_h, const int8_t* prec_h, int n, int32_t* ids,
                                float* w, int8_t* prec, hipStream_t s);

}  // namespace moe
