// Batch-1 decode kernels: one token, k routed experts plus the shared expert.
//
// At batch 1 the layer is a pure stream of expert bytes ("Running
// DeepSeek-V4-Flash across four free GPUs", §The arithmetic that explains 20
// tok/s; "An elephant through a straw", §The number: the GPU spends its time
// receiving experts, not multiplying them), so both kernels are organised
// around keeping enough HBM requests in flight:
//
// gateup_b1_kernel: a fixed grid of persistent wavefronts splits the
//   (expert, row) pairs of all selected experts into contiguous runs.  Each
//   wavefront keeps D rows of W1 and W3 in flight in registers (a rotating
//   prefetch pipeline), so the next rows' loads are outstanding while the
//   current row is converted, multiplied and reduced.  A row of K = H
//   elements is split over the 64 lanes in 32-element chunks (one 16-byte
//   FP4 load plus one scale byte per lane and chunk); the token's activations
//   are staged in LDS once per workgroup and read per row, which keeps the
//   register count low enough for several wavefronts per SIMD.  The gate and up sums are reduced
//   with DPP lane moves and lane 63 writes silu(g) * u.
//
// down_combine_b1_kernel: a workgroup owns a tile of output rows for every
//   expert at once, so the weighted combine is fused: each lane accumulates
//   w_r * (its partial W2 row . h_r) over all experts in rank order, and one
//   wavefront reduction per row gives the layer output, rounded once.  The
//   SwiGLU outputs of all experts (a few tens of KiB) are staged in LDS once
//   per workgroup; W2 rows of the next experts are prefetched while the
//   current expert is multiplied.
#include <algorithm>

#include "common.h"

#ifndef MOE_B1_GU_WAVES_PER_CU
#define MOE_B1_GU_WAVES_PER_CU 8
#endif
#ifndef MOE_B1_GU_DEPTH
#define MOE_B1_GU_DEPTH 3
#endif
#ifndef MOE_B1_GU_OCC
#define MOE_B1_GU_OCC 3
#endif
#ifndef MOE_B1_DN_ROWS
#define MOE_B1_DN_ROWS 2
#endif
#ifndef MOE_B1_DN_DEPTH
#define MOE_B1_DN_DEPTH 3
#endif

namespace moe {

namespace {

constexpr int kNumCU = 256;
constexpr int kMaxGroups = 64;

struct B1Args {
  int H, I, k, K1;
  const uint8_t* fp4_base;
  size_t fp4_stride;
  int num_slots;
  const uint8_t* int2_base;
  size_t int2_stride;
  int num_int2;
  const uint8_t* shared;
  const void* x;            // [1][H]
  const int32_t* slot_ids;  // [k]
  const int8_t* prec;       // [k] or null
  const float* w;           // [k]
  void* h;                  // [K1][I], bf16 or fp32
  void* out;                // [1][H]
};

// record and precision of group g (rank g, or the shared expert at g == k)
__device__ __forceinline__ const uint8_t* b1_group(const B1Args& a, int g, int* pr) {
  if (g == a.k) {
    *pr = 0;
    return a.shared;
  }
  const int p = a.prec ? (int)a.prec[g] : 0;
  const int s = a.slot_ids[g];
  if (p == 0 && s >= 0 && s < a.num_slots) {
    *pr = 0;
    return a.fp4_base + (size_t)s * a.fp4_stride;
  }
  if (p == 1 && a.int2_base && s >= 0 && s < a.num_int2) {
    *pr = 1;
    return a.int2_base + (size_t)s * a.int2_stride;
  }
  *pr = -1;
  return nullptr;
}

__device__ __forceinline__ float silu_mul_b1(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// 32 bf16 (16 pairs) or 32 fp32 activations of one chunk
template <bool BF16>
struct Act;
template <>
struct Act<true> {
  uint32_t p[16];
  __device__ __forceinline__ void load_global(const void* base, size_t elem) {
    const uint4* src = (const uint4*)((const uint16_t*)base + elem);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = src[i];
      p[4 * i] = v.x, p[4 * i + 1] = v.y, p[4 * i + 2] = v.z, p[4 * i + 3] = v.w;
    }
  }
  __device__ __forceinline__ void load_lds(const uint8_t* lds, size_t elem) {
    const uint4* src = (const uint4*)(lds + elem * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = src[i];
      p[4 * i] = v.x, p[4 * i + 1] = v.y, p[4 * i + 2] = v.z, p[4 * i + 3] = v.w;
    }
  }
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
template <>
struct Act<false> {
  float f[32];
  __device__ __forceinline__ void load_global(const void* base, size_t elem) {
    const float4* src = (const float4*)((const float*)base + elem);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 v = src[i];
      f[4 * i] = v.x, f[4 * i + 1] = v.y, f[4 * i + 2] = v.z, f[4 * i + 3] = v.w;
    }
  }
  __device__ __forceinline__ void load_lds(const uint8_t* lds, size_t elem) {
    const float4* src = (const float4*)(lds + elem * 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 v = src[i];
      f[4 * i] = v.x, f[4 * i + 1] = v.y, f[4 * i + 2] = v.z, f[4 * i + 3] = v.w;
    }
  }
  __device__ __forceinline__ float fp4(const uint4 c) const {
    float a0 = 0.0f, a1 = 0.0f;
    const uint32_t d[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v2f t = fp4x2_to_f32<0>(d[i]);
      a0 = fmaf(t.x, f[8 * i + 0], a0), a1 = fmaf(t.y, f[8 * i + 1], a1);
      t = fp4x2_to_f32<1>(d[i]);
      a0 = fmaf(t.x, f[8 * i + 2], a0), a1 = fmaf(t.y, f[8 * i + 3], a1);
      t = fp4x2_to_f32<2>(d[i]);
      a0 = fmaf(t.x, f[8 * i + 4], a0), a1 = fmaf(t.y, f[8 * i + 5], a1);
      t = fp4x2_to_f32<3>(d[i]);
      a0 = fmaf(t.x, f[8 * i + 6], a0), a1 = fmaf(t.y, f[8 * i + 7], a1);
    }
    return a0 + a1;
  }
  __device__ __forceinline__ float int2(const uint2 c) const {
    float a0 = 0.0f, a1 = 0.0f;
    const uint32_t d[2] = {c.x, c.y};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int q = 0; q < 16; q += 2) {
        a0 = fmaf((float)((d[i] >> (2 * q)) & 3u) - 1.5f, f[16 * i + q], a0);
        a1 = fmaf((float)((d[i] >> (2 * q + 2)) & 3u) - 1.5f, f[16 * i + q + 1], a1);
      }
    }
    return a0 + a1;
  }
};

template <bool HBF16>
__device__ __forceinline__ void store_h(void* h, size_t i, float v) {
  if (HBF16)
    ((uint16_t*)h)[i] = f32_to_bf16(v);
  else
    ((float*)h)[i] = v;
}

// ------------------------------------------------------------------ gate/up

template <int CPL>
struct GURow {
  uint4 c1[CPL], c3[CPL];
  uint32_t s1[CPL], s3[CPL];
};

template <int CPL, bool XBF16, int D>
__global__ __launch_bounds__(256, MOE_B1_GU_OCC) void gateup_b1_kernel(B1Args a) {
  // the token's activations, staged once per workgroup; each lane reads its
  // chunks from LDS per row instead of holding them in registers
  __shared__ __align__(16) uint8_t xs[CPL * 64 * 32 * (XBF16 ? 2 : 4)];
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nw = gridDim.x * 4;
  const int H = a.H, I = a.I;
  {
    const int nv = H * (XBF16 ? 2 : 4) / 16;
    for (int v = threadIdx.x; v < nv; v += 256) ((uint4*)xs)[v] = ((const uint4*)a.x)[v];
  }
  __syncthreads();
  const int total = a.K1 * I;
  const int per = (total + nw - 1) / nw;
  const int j0 = gw * per, j1 = min(j0 + per, total);
  if (j0 >= j1) return;
  auto xchunk = [&](int q) {
    Act<XBF16> x;
    x.load_lds(xs, (size_t)(q * 64 + lane) * 32);
    return x;
  };

  const size_t rowb4 = (size_t)H / 2, rowb2 = (size_t)H / 4, rows = (size_t)H / 32;
  for (int g = j0 / I; g <= (j1 - 1) / I; ++g) {
    const int r0 = max(j0, g * I) - g * I, r1 = min(j1, (g + 1) * I) - g * I;
    int pr;
    const uint8_t* rec = b1_group(a, g, &pr);
    if (pr < 0) continue;
    if (pr != 0) continue;  // 2-bit groups run in gateup_int2_b1_kernel
    const RecordLayout L = record_layout(H, I, 4);
    {
      const uint8_t* w1 = rec + L.w1c;
      const uint8_t* w3 = rec + L.w3c;
      const uint8_t* s1 = rec + L.w1s;
      const uint8_t* s3 = rec + L.w3s;
      GURow<CPL> sl[D];
      // loads of one row into a slot (callers guarantee row < r1)
      auto issue = [&](int row, GURow<CPL>& s) {
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
          const size_t c = (size_t)(q * 64 + lane);
          s.c1[q] = ld_stream16(w1 + (size_t)row * rowb4 + c * 16);
          s.c3[q] = ld_stream16(w3 + (size_t)row * rowb4 + c * 16);
          s.s1[q] = s1[(size_t)row * rows + c];
          s.s3[q] = s3[(size_t)row * rows + c];
        }
      };
      auto consume = [&](int row, const GURow<CPL>& s) {
        float gs = 0.0f, us = 0.0f;
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
          const Act<XBF16> xq = xchunk(q);
          gs = fmaf(xq.fp4(s.c1[q]), e8m0_to_f32(s.s1[q]), gs);
          us = fmaf(xq.fp4(s.c3[q]), e8m0_to_f32(s.s3[q]), us);
        }
        gs = wave_sum_to_lane63(gs);
        us = wave_sum_to_lane63(us);
        if (lane == 63) store_h<XBF16>(a.h, (size_t)g * I + row, silu_mul_b1(gs, us));
      };
#pragma unroll
      for (int u = 0; u < D; ++u)
        if (r0 + u < r1) issue(r0 + u, sl[u]);
      int row = r0;
      // steady state: every refill is in range, so the loads are
      // unconditional and stay in flight across rows
      for (; row + 2 * D <= r1; row += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
          consume(row + u, sl[u]);
          issue(row + u + D, sl[u]);
        }
      }
      // tail: at most 2D-1 rows left
#pragma unroll
      for (int u = 0; u < D; ++u) {
        if (row + u < r1) {
          consume(row + u, sl[u]);
          if (row + u + D < r1) issue(row + u + D, sl[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < D; ++u)
        if (row + D + u < r1) consume(row + D + u, sl[u]);
    }
  }
}

// 2-bit groups of the batch-1 gate/up (the slot cache's fallback copies):
// a separate kernel so the FP4 streaming kernel keeps its register budget.
// One wavefront per row; the activations come from global memory (L2).
template <int CPL, bool XBF16>
__global__ __launch_bounds__(256) void gateup_int2_b1_kernel(B1Args a) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nw = gridDim.x * 4;
  const int H = a.H, I = a.I;
  const RecordLayout L = record_layout(H, I, 2);
  const size_t rowb2 = (size_t)H / 4, rows = (size_t)H / 32;
  for (int g = 0; g < a.K1; ++g) {
    int pr;
    const uint8_t* rec = b1_group(a, g, &pr);
    if (pr != 1) continue;
    for (int row = gw; row < I; row += nw) {
      float gs = 0.0f, us = 0.0f;
#pragma unroll
      for (int q = 0; q < CPL; ++q) {
        const size_t c = (size_t)(q * 64 + lane);
        const uint2 c1 = ld_stream8(rec + L.w1c + (size_t)row * rowb2 + c * 8);
        const uint2 c3 = ld_stream8(rec + L.w3c + (size_t)row * rowb2 + c * 8);
        Act<XBF16> xq;
        xq.load_global(a.x, c * 32);
        gs = fmaf(xq.int2(c1), e4m3_to_f32(rec[L.w1s + (size_t)row * rows + c]), gs);
        us = fmaf(xq.int2(c3), e4m3_to_f32(rec[L.w3s + (size_t)row * rows + c]), us);
      }
      gs = wave_sum_to_lane63(gs);
      us = wave_sum_to_lane63(us);
      if (lane == 63) store_h<XBF16>(a.h, (size_t)g * I + row, silu_mul_b1(gs, us));
    }
  }
}

// ------------------------------------------------------------- down+combine

template <int CPL, int RW>
struct DNSlot {
  uint4 c[RW][CPL];  // 2-bit rows use .x/.y only
  uint32_t s[RW][CPL];
};

struct ActiveGroup {
  const uint8_t* rec;
  float w;
  int g, prec;
};

template <int CPL, bool HBF16, bool OBF16, int RW, int DG>
__global__ __launch_bounds__(512) void down_combine_b1_kernel(B1Args a) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ ActiveGroup act[kMaxGroups];
  __shared__ int nact_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, I = a.I;
  const size_t hsz = HBF16 ? 2 : 4;

  if (wave == 0) {
    int pr = -1;
    const uint8_t* rec = nullptr;
    if (lane < a.K1) rec = b1_group(a, lane, &pr);
    const bool on = lane < a.K1 && pr >= 0;
    const uint64_t m = __ballot(on);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (on) {
      const int i = __popcll(m & below);
      act[i].rec = rec;
      act[i].w = (lane == a.k) ? 1.0f : a.w[lane];
      act[i].g = lane;
      act[i].prec = pr;
    }
    if (lane == 0) nact_s = __popcll(m);
  }
  __syncthreads();
  const int nact = nact_s;
  const int row0 = (blockIdx.x * 8 + wave) * RW;  // < H: the grid tiles H exactly
  const size_t rowb4 = (size_t)I / 2, rowb2 = (size_t)I / 4, rows = (size_t)I / 32;
  const RecordLayout L4 = record_layout(H, I, 4), L2 = record_layout(H, I, 2);

  // W2 rows of active group i into a slot (callers guarantee i < nact)
  auto issue = [&](int i, DNSlot<CPL, RW>& s) {
    const ActiveGroup& ag = act[i];
    if (ag.prec == 0) {
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
          const size_t c = (size_t)(q * 64 + lane), row = (size_t)(row0 + r);
          s.c[r][q] = ld_stream16(ag.rec + L4.w2c + row * rowb4 + c * 16);
          s.s[r][q] = ag.rec[L4.w2s + row * rows + c];
        }
    } else {
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
          const size_t c = (size_t)(q * 64 + lane), row = (size_t)(row0 + r);
          const uint2 v = ld_stream8(ag.rec + L2.w2c + row * rowb2 + c * 8);
          s.c[r][q] = make_uint4(v.x, v.y, 0u, 0u);
          s.s[r][q] = ag.rec[L2.w2s + row * rows + c];
        }
    }
  };

  // first weight loads go out before the SwiGLU outputs are staged
  DNSlot<CPL, RW> sl[DG];
#pragma unroll
  for (int u = 0; u < DG; ++u)
    if (u < nact) issue(u, sl[u]);

  const size_t row_bytes = (size_t)I * hsz;
  for (int i = 0; i < nact; ++i) {
    const uint4* src = (const uint4*)((const uint8_t*)a.h + (size_t)act[i].g * row_bytes);
    uint4* dst = (uint4*)(lds + (size_t)i * row_bytes);
    for (size_t v = tid; v < row_bytes / 16; v += 512) dst[v] = src[v];
  }
  __syncthreads();

  float acc[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) acc[r] = 0.0f;

  auto consume = [&](int i, const DNSlot<CPL, RW>& s) {
    const float wgt = act[i].w;
    Act<HBF16> hv[CPL];
#pragma unroll
    for (int q = 0; q < CPL; ++q) hv[q].load_lds(lds + (size_t)i * row_bytes, (size_t)(q * 64 + lane) * 32);
    if (act[i].prec == 0) {
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        float part = 0.0f;
#pragma unroll
        for (int q = 0; q < CPL; ++q) part = fmaf(hv[q].fp4(s.c[r][q]), e8m0_to_f32(s.s[r][q]), part);
        acc[r] = fmaf(wgt, part, acc[r]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        float part = 0.0f;
#pragma unroll
        for (int q = 0; q < CPL; ++q)
          part = fmaf(hv[q].int2(make_uint2(s.c[r][q].x, s.c[r][q].y)), e4m3_to_f32(s.s[r][q]), part);
        acc[r] = fmaf(wgt, part, acc[r]);
      }
    }
  };

  int i = 0;
  for (; i + 2 * DG <= nact; i += DG) {
#pragma unroll
    for (int u = 0; u < DG; ++u) {
      consume(i + u, sl[u]);
      issue(i + u + DG, sl[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < DG; ++u) {
    if (i + u < nact) {
      consume(i + u, sl[u]);
      if (i + u + DG < nact) issue(i + u + DG, sl[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < DG; ++u)
    if (i + DG + u < nact) consume(i + DG + u, sl[u]);

#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const float v = wave_sum_to_lane63(acc[r]);
    if (lane == 63) {
      if (OBF16)
        ((uint16_t*)a.out)[row0 + r] = f32_to_bf16(v);
      else
        ((float*)a.out)[row0 + r] = v;
    }
  }
}

template <int CPL>
void launch_gateup_b1(const B1Args& a, bool xbf16, hipStream_t s) {
  const int grid = kNumCU * MOE_B1_GU_WAVES_PER_CU / 4;
  if (xbf16)
    hipLaunchKernelGGL((gateup_b1_kernel<CPL, true, MOE_B1_GU_DEPTH>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((gateup_b1_kernel<CPL, false, MOE_B1_GU_DEPTH>), dim3(grid), dim3(256), 0, s, a);
  if (a.prec) {  // 2-bit copies can only appear when precisions are given
    const int grid2 = std::max(1, std::min(a.I / 4, 1024));
    if (xbf16)
      hipLaunchKernelGGL((gateup_int2_b1_kernel<CPL, true>), dim3(grid2), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((gateup_int2_b1_kernel<CPL, false>), dim3(grid2), dim3(256), 0, s, a);
  }
}

template <int CPL, bool HBF16>
void launch_down_b1(const B1Args& a, bool obf16, size_t lds, hipStream_t s) {
  constexpr int RW = MOE_B1_DN_ROWS;
  const int grid = (a.H + 8 * RW - 1) / (8 * RW);
  if (obf16)
    hipLaunchKernelGGL((down_combine_b1_kernel<CPL, HBF16, true, RW, MOE_B1_DN_DEPTH>), dim3(grid), dim3(512), lds,
                       s, a);
  else
    hipLaunchKernelGGL((down_combine_b1_kernel<CPL, HBF16, false, RW, MOE_B1_DN_DEPTH>), dim3(grid), dim3(512), lds,
                       s, a);
}

}  // namespace

// The batch-1 fused path applies when both reduction lengths split evenly
// over 64 lanes (H, I in {2048, 4096}), the output rows tile exactly,
// and the SwiGLU outputs of every group fit the LDS budget.
bool b1_path_ok(int H, int I, int K1, bool xbf16) {
  const int ch = H / 32, ci = I / 32;
  if (H % 32 || I % 32 || ch % 64 || ci % 64) return false;
  const int cph = ch / 64, cpi = ci / 64;
  if (!(cph == 1 || cph == 2) || !(cpi == 1 || cpi == 2)) return false;
  if (K1 > kMaxGroups) return false;
  if (H % (8 * MOE_B1_DN_ROWS)) return false;
  const size_t lds = (size_t)K1 * I * (xbf16 ? 2 : 4);
  return lds <= 60 * 1024;
}

moe_status launch_b1(const moe_layer* L, const void* x, moe_dtype xt, int k, const int32_t* slot_ids,
                     const int8_t* prec, const float* w, void* h, void* out, moe_dtype ot, hipStream_t s) {
  B1Args a;
  a.H = L->H;
  a.I = L->I;
  a.k = k;
  a.K1 = k + (L->shared ? 1 : 0);
  a.fp4_base = L->fp4_base;
  a.fp4_stride = L->fp4_stride;
  a.num_slots = L->num_slots;
  a.int2_base = L->int2_base;
  a.int2_stride = L->int2_stride;
  a.num_int2 = L->int2_base ? L->num_int2 : 0;
  a.shared = L->shared;
  a.x = x;
  a.slot_ids = slot_ids;
  a.prec = prec;
  a.w = w;
  a.h = h;
  a.out = out;
  const bool xbf16 = xt == MOE_BF16, obf16 = ot == MOE_BF16;
  const int cph = a.H / 2048, cpi = a.I / 2048;
  {
    ProfScope prof(MOE_PROF_GATEUP, s);
    if (cph == 1)
      launch_gateup_b1<1>(a, xbf16, s);
    else
      launch_gateup_b1<2>(a, xbf16, s);
    MOE_LAUNCH_CHECK();
  }
  {
    ProfScope prof(MOE_PROF_DOWN, s);
    const size_t lds = (size_t)a.K1 * a.I * (xbf16 ? 2 : 4);
    switch (cpi * 2 + (xbf16 ? 1 : 0)) {
      case 2: launch_down_b1<1, false>(a, obf16, lds, s); break;
      case 3: launch_down_b1<1, true>(a, obf16, lds, s); break;
      case 4: launch_down_b1<2, false>(a, obf16, lds, s); break;
      default: launch_down_b1<2, true>(a, obf16, lds, s); break;
    }
    MOE_LAUNCH_CHECK();
  }
  return MOE_OK;
}

}  // namespace moe
