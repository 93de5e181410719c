// Batch-1 decode kernels: one token, k routed experts plus the shared expert.
//
// At batch 1 the layer is a pure stream of expert bytes ("Running
// DeepSeek-V4-Flash across four free GPUs", §The arithmetic that explains 20
// tok/s; "An elephant through a straw", §The number: the GPU spends its time
// receiving experts, not multiplying them).  A whole token is only ~120 MB,
// a few tens of KiB per wavefront, so each kernel requests everything it
// will read up front and then consumes it in arrival order:
//
// gateup_b1_kernel: every wavefront owns NR consecutive rows of the
//   flattened (FP4 expert, gate/up row) space.  It issues the activation
//   loads, then (optionally) routes the token itself from the logits row,
//   stages the activation in LDS (once per workgroup), then issues all NR
//   rows of W1 and W3 (codes and E8M0 scales) at once.  Each row's gate and
//   up sums are reduced with DPP lane moves and lane 63 writes
//   silu(g) * u in bf16.  The shared expert comes first in the row order.
//
// down_combine_b1_kernel: a wavefront owns one output row for every active
//   expert at once, so the weighted combine is fused: each lane accumulates
//   w_r * (its partial W2 row . h_r) over the experts in rank order (shared
//   last, weight 1) and one wavefront reduction gives the layer output,
//   rounded once.  The SwiGLU outputs are requested first, then every
//   expert's W2 row, so the staging of h into LDS waits only for h.
//
// Loads are unconditional (indices are clamped instead), which keeps the
// compiler's wait counts exact: a consumer waits for its own row only.
#include <algorithm>

#include "common.h"
#include "route_dev.h"

#ifndef MOE_B1_GU_ROWS
#define MOE_B1_GU_ROWS 6
#endif
#ifndef MOE_B1_GU_OCC
#define MOE_B1_GU_OCC 3
#endif
#ifndef MOE_B1_DN_ORDER
#define MOE_B1_DN_ORDER 1
#endif

namespace moe {

namespace {

constexpr int kMaxGroups = 12;  // k + shared handled by the batch-1 kernels
constexpr int kMaxE = 1024;     // experts routed in-kernel (16 logits per lane)

struct B1Args {
  int H, I, k, K1, E;
  const uint8_t* fp4_base;
  size_t fp4_stride;
  int num_slots;
  const uint8_t* int2_base;
  size_t int2_stride;
  int num_int2;
  const uint8_t* shared;
  const float* logits;  // [E]: the gate/up kernel routes the token; null: slot_ids and w are inputs
  const void* x;        // [1][H] bf16
  int32_t* slot_ids;    // [k]
  const int8_t* prec;   // [k] or null (all FP4)
  float* w;             // [k]
  uint16_t* h;          // [K1][I] bf16
  void* out;            // [1][H] bf16
};

__device__ __forceinline__ float silu_mul_b1(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// 32 bf16 activations (16 pairs) of one 32-element chunk
struct XChunk {
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

// position of the n-th set bit of m (n < popcount(m)); wave-uniform
__device__ __forceinline__ int nth_set_bit(uint64_t m, int n) {
  for (int t = 0; t < n; ++t) m &= m - 1;
  return __builtin_ctzll(m);
}

// ------------------------------------------------------------------ gate/up

template <int CPL>
struct GURow {
  uint4 c1[CPL], c3[CPL];
  uint32_t s1[CPL], s3[CPL];
};

template <int CPL, int NR, int EPL>
__global__ __launch_bounds__(256, MOE_B1_GU_OCC) void gateup_b1_kernel(B1Args a) {
  static_assert(NR >= 1 && NR <= 64, "rows per wavefront");
  constexpr int XBYTES = CPL * 64 * 32 * 2;  // H bf16 activations
  constexpr int XV = XBYTES / 16 / 256;      // 16-byte pieces per thread
  static_assert(XV == 1 || XV == 2, "H is 2048 or 4096");
  __shared__ __align__(16) uint8_t xs[XBYTES];
  __shared__ float stab[256];  // E8M0 byte -> scale
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int I = a.I, k = a.k;

  // activations first in this wavefront's memory queue (named registers, not
  // an array, so they stay in VGPRs)
  const uint4 xv0 = ((const uint4*)a.x)[threadIdx.x];
  const uint4 xv1 = XV == 2 ? ((const uint4*)a.x)[threadIdx.x + 256] : make_uint4(0u, 0u, 0u, 0u);
  stab[threadIdx.x] = e8m0_to_f32(threadIdx.x);

  // lane r < k: slot and precision of rank r (routed here when logits are given)
  int my_slot = -1, my_prec = -1;
  if constexpr (EPL > 0) {
    float my_w;
    route_wave<EPL>(a.logits, a.E, k, &my_slot, &my_w);
    my_prec = 0;
    if (gw == 0 && lane < k) {
      a.slot_ids[lane] = my_slot;
      a.w[lane] = my_w;
    }
  } else {
    if (lane < k) {
      my_slot = a.slot_ids[lane];
      my_prec = a.prec ? (int)a.prec[lane] : 0;
    }
  }
  // FP4 groups in row order: the shared expert, then the FP4 ranks
  const bool fp4 = lane < k && my_prec == 0 && my_slot >= 0 && my_slot < a.num_slots;
  const uint64_t m = __ballot(fp4);
  const int nsh = a.shared ? 1 : 0;
  const int total = (nsh + __popcll(m)) * I;
  const int j0 = gw * NR;
  const bool live = j0 < total;

  // the activation has long arrived (the routing inputs came after it); it
  // goes to LDS before the weight loads, so no wait below covers them, and
  // the barrier comes first too, so loads and their consumers share one block
  ((uint4*)xs)[threadIdx.x] = xv0;
  if (XV == 2) ((uint4*)xs)[threadIdx.x + 256] = xv1;
  __syncthreads();
  if (!live) return;

  // the NR rows span at most two groups: g0 (from row r0) and g0 + 1
  const int g0 = j0 / I, r0 = j0 - g0 * I, last = total - 1;
  auto group = [&](int gi, int* kx) -> const uint8_t* {
    if (gi < nsh) {
      *kx = k;
      return a.shared;
    }
    const int r = nth_set_bit(m, gi - nsh);
    *kx = r;
    return a.fp4_base + (size_t)__builtin_amdgcn_readlane(my_slot, r) * a.fp4_stride;
  };
  int kx0, kx1 = k;
  const uint8_t* rec0 = group(g0, &kx0);
  const uint8_t* rec1 = (j0 + NR - 1 >= (g0 + 1) * I && last >= (g0 + 1) * I) ? group(g0 + 1, &kx1) : rec0;

  const size_t rowb4 = (size_t)a.H / 2, rows = (size_t)a.H / 32;
  const RecordLayout L = record_layout(a.H, I, 4);
  GURow<CPL> sl[NR];
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    const int j = min(j0 + u, last);  // rows past the end repeat the last (not stored)
    const bool second = j - g0 * I >= I;
    const int row = second ? j - g0 * I - I : j - g0 * I;
    const uint8_t* rec = second ? rec1 : rec0;
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const size_t c = (size_t)(q * 64 + lane);
      sl[u].c1[q] = ld_stream16(rec + L.w1c + (size_t)row * rowb4 + c * 16);
      sl[u].c3[q] = ld_stream16(rec + L.w3c + (size_t)row * rowb4 + c * 16);
      sl[u].s1[q] = rec[L.w1s + (size_t)row * rows + c];
      sl[u].s3[q] = rec[L.w3s + (size_t)row * rows + c];
    }
  }

  // every load above is issued before any row is consumed
  __builtin_amdgcn_sched_barrier(0);

  // rows in arrival order; the block scale rides in the convert, so each row
  // is one accumulation chain per matrix (two for instruction overlap)
  float gsum[NR], usum[NR];
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    float g0a = 0.0f, g1a = 0.0f, u0a = 0.0f, u1a = 0.0f;
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      XChunk xq;  // re-read per row: LDS bandwidth is cheaper than 16 registers per chunk
      xq.load_lds(xs, (size_t)(q * 64 + lane) * 32);
      xq.fp4_acc(sl[u].c1[q], stab[sl[u].s1[q]], g0a, g1a);
      xq.fp4_acc(sl[u].c3[q], stab[sl[u].s3[q]], u0a, u1a);
    }
    gsum[u] = wave_sum_to_lane63(g0a + g1a);
    usum[u] = wave_sum_to_lane63(u0a + u1a);
  }
  // SwiGLU of all NR rows at once: lane t < NR takes row t
  float gv = 0.0f, uv = 0.0f;
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    const float gu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gsum[u]), 63));
    const float uu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(usum[u]), 63));
    gv = lane == u ? gu : gv;
    uv = lane == u ? uu : uv;
  }
  const int rl = r0 + lane;
  if (lane < NR && j0 + lane <= last) {
    const bool second = rl >= I;
    const size_t hrow = second ? (size_t)kx1 * I + (rl - I) : (size_t)kx0 * I + rl;
    a.h[hrow] = f32_to_bf16(silu_mul_b1(gv, uv));
  }
}

// 2-bit groups of the batch-1 gate/up (the slot cache's fallback copies):
// a separate kernel so the FP4 streaming kernel keeps its register budget.
// One wavefront per row; the activations come from global memory (L2).
template <int CPL>
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
        XChunk xq;
        xq.load_global(a.x, c * 32);
        gs = fmaf(xq.int2(c1), e4m3_to_f32(rec[L.w1s + (size_t)row * rows + c]), gs);
        us = fmaf(xq.int2(c3), e4m3_to_f32(rec[L.w3s + (size_t)row * rows + c]), us);
      }
      gs = wave_sum_to_lane63(gs);
      us = wave_sum_to_lane63(us);
      if (lane == 63) a.h[(size_t)g * I + row] = f32_to_bf16(silu_mul_b1(gs, us));
    }
  }
}

// ------------------------------------------------------------- down+combine

template <int CPL>
struct DNRow {
  uint4 c[CPL];  // 2-bit rows use .x/.y only
  uint32_t s[CPL];
};

template <int CPL, int NB, bool HAS2>
__global__ __launch_bounds__(256) void down_combine_b1_kernel(B1Args a) {
  extern __shared__ __align__(16) uint8_t lds[];  // [NB][I] bf16 SwiGLU outputs
  __shared__ float stab[256];                      // E8M0 byte -> scale
  const int tid = threadIdx.x, lane = tid & 63;
  stab[tid] = e8m0_to_f32(tid);
  const int orow = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(tid >> 6);  // < H: the grid tiles H exactly
  const int I = a.I;

  // active groups in rank order, shared last (lane g < K1 holds group g);
  // the three small loads go out together
  int pr = -1, slot = 0;
  float wg = 0.0f;
  if (lane < a.k) {
    const int p = a.prec ? (int)a.prec[lane] : 0;
    slot = a.slot_ids[lane];
    wg = a.w[lane];
    pr = (p == 0 && slot >= 0 && slot < a.num_slots) ? 0 : (p == 1 && slot >= 0 && slot < a.num_int2) ? 1 : -1;
  } else if (lane == a.k && a.shared) {
    pr = 0;
    wg = 1.0f;
  }
  const uint64_t m = __ballot(lane < a.K1 && pr >= 0);
  const int nact = __popcll(m);
  if (nact == 0) {  // every expert dropped and no shared expert
    if (lane == 63) ((uint16_t*)a.out)[orow] = 0;
    return;
  }
  int gi[NB], pi[NB];
  const uint8_t* ri[NB];
  float wi[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int g = nth_set_bit(m, min(i, nact - 1));
    gi[i] = g;
    pi[i] = __builtin_amdgcn_readlane(pr, g);
    const size_t sl_g = (size_t)__builtin_amdgcn_readlane(slot, g);
    // pointers rebuilt from the kernel arguments stay in the global address space
    ri[i] = g == a.k ? a.shared : pi[i] == 0 ? a.fp4_base + sl_g * a.fp4_stride : a.int2_base + sl_g * a.int2_stride;
    wi[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wg), g));
  }

  // The SwiGLU outputs of the batch, staged in LDS, and this wavefront's W2
  // row of every active group, all in flight before the first wait.
  const size_t rowb4 = (size_t)I / 2, rowb2 = (size_t)I / 4, rows = (size_t)I / 32;
  const RecordLayout L4 = record_layout(a.H, I, 4), L2 = record_layout(a.H, I, 2);
  DNRow<CPL> sl[NB];
  auto issue_w2 = [&](int i) {
    if (!HAS2 || pi[i] == 0) {
#pragma unroll
      for (int q = 0; q < CPL; ++q) {
        const size_t c = (size_t)(q * 64 + lane);
        sl[i].c[q] = ld_stream16(ri[i] + L4.w2c + (size_t)orow * rowb4 + c * 16);
        sl[i].s[q] = ri[i][L4.w2s + (size_t)orow * rows + c];
      }
    } else {
#pragma unroll
      for (int q = 0; q < CPL; ++q) {
        const size_t c = (size_t)(q * 64 + lane);
        const uint2 v = ld_stream8(ri[i] + L2.w2c + (size_t)orow * rowb2 + c * 8);
        sl[i].c[q] = make_uint4(v.x, v.y, 0u, 0u);
        sl[i].s[q] = ri[i][L2.w2s + (size_t)orow * rows + c];
      }
    }
  };
  auto stage_h = [&]() {  // I * 2 / 16 / 256 = CPL pieces per thread and group
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const uint4* src = (const uint4*)(a.h + (size_t)gi[i] * I);
      uint4* dst = (uint4*)(lds + (size_t)i * I * 2);
      dst[tid] = src[tid];
      if (CPL == 2) dst[tid + 256] = src[tid + 256];
    }
  };
#if MOE_B1_DN_ORDER == 0
  // h first: its loads come back from L2/MALL long before the weights would
  stage_h();
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NB; ++i) issue_w2(i);
#else
  // the first half of the weights, then h (whose wait covers only that
  // half), then the rest
  constexpr int NH = (NB + 1) / 2;
#pragma unroll
  for (int i = 0; i < NH; ++i) issue_w2(i);
  stage_h();
#pragma unroll
  for (int i = NH; i < NB; ++i) issue_w2(i);
  __syncthreads();
#endif

  // 4. consume in rank order.  Straight-line code: a batch slot past the
  // active groups (a repeat of the last one) is computed and then selected
  // away, so no load is sunk into a branch below the barrier.
  int nact_v;  // nact in a vector register: the selects stay selects
  asm volatile("v_mov_b32 %0, %1" : "=v"(nact_v) : "s"(nact));
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    float part = 0.0f, part2 = 0.0f;
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      XChunk hq;
      hq.load_lds(lds + (size_t)i * I * 2, (size_t)(q * 64 + lane) * 32);
      if (!HAS2 || pi[i] == 0)
        hq.fp4_acc(sl[i].c[q], stab[sl[i].s[q]], part, part2);
      else
        part = fmaf(hq.int2(make_uint2(sl[i].c[q].x, sl[i].c[q].y)), e4m3_to_f32(sl[i].s[q]), part);
    }
    const float t = fmaf(wi[i], part + part2, acc);
    acc = (i < nact_v) ? t : acc;
  }
  const float v = wave_sum_to_lane63(acc);
  if (lane == 63) ((uint16_t*)a.out)[orow] = f32_to_bf16(v);
}

// ------------------------------------------------------------------ launch

// batch of the down kernel: every group of the token at once (k = 6 or 8
// plus the shared expert are exact; other counts repeat the last group)
int down_batch(int K1) { return K1 <= 4 ? 4 : K1 <= 7 ? 7 : K1 <= 9 ? 9 : kMaxGroups; }

template <int CPL>
void launch_gateup_b1(const B1Args& a, hipStream_t s) {
  constexpr int NR = MOE_B1_GU_ROWS;
  const int waves = (a.K1 * a.I + NR - 1) / NR;
  const int grid = std::max(1, (waves + 3) / 4);
  if (!a.logits)
    hipLaunchKernelGGL((gateup_b1_kernel<CPL, NR, 0>), dim3(grid), dim3(256), 0, s, a);
  else if (a.E <= 256)
    hipLaunchKernelGGL((gateup_b1_kernel<CPL, NR, 4>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((gateup_b1_kernel<CPL, NR, kMaxE / 64>), dim3(grid), dim3(256), 0, s, a);
  if (a.prec) {  // 2-bit copies can only appear when precisions are given
    const int grid2 = std::max(1, std::min(a.I / 4, 1024));
    hipLaunchKernelGGL((gateup_int2_b1_kernel<CPL>), dim3(grid2), dim3(256), 0, s, a);
  }
}

template <int CPL, bool HAS2>
void launch_down_nb(const B1Args& a, hipStream_t s) {
  const int grid = a.H / 4;
  const int nb = down_batch(a.K1);
  const size_t lds = (size_t)nb * a.I * 2;
  if (nb == 4)
    hipLaunchKernelGGL((down_combine_b1_kernel<CPL, 4, HAS2>), dim3(grid), dim3(256), lds, s, a);
  else if (nb == 7)
    hipLaunchKernelGGL((down_combine_b1_kernel<CPL, 7, HAS2>), dim3(grid), dim3(256), lds, s, a);
  else if (nb == 9)
    hipLaunchKernelGGL((down_combine_b1_kernel<CPL, 9, HAS2>), dim3(grid), dim3(256), lds, s, a);
  else
    hipLaunchKernelGGL((down_combine_b1_kernel<CPL, kMaxGroups, HAS2>), dim3(grid), dim3(256), lds, s, a);
}

template <int CPL>
void launch_down_b1(const B1Args& a, hipStream_t s) {
  if (a.prec)
    launch_down_nb<CPL, true>(a, s);
  else
    launch_down_nb<CPL, false>(a, s);
}

}  // namespace

// The batch-1 path applies to bf16 activations and outputs (the SwiGLU
// outputs between the two kernels are bf16 too, within the bf16 output
// tolerance but not the fp32 one) when both reduction lengths split evenly
// over 64 lanes in 16-byte pieces (H, I in {2048, 4096}) and the groups fit
// the down kernel's batch (its LDS holds the batch's h rows).
bool b1_path_ok(int H, int I, int K1, bool xbf16, bool obf16) {
  if (!xbf16 || !obf16) return false;
  if (!(H == 2048 || H == 4096) || !(I == 2048 || I == 4096)) return false;
  if (K1 < 1 || K1 > kMaxGroups) return false;
  return (size_t)down_batch(K1) * I * 2 <= 64 * 1024;
}

// in-kernel routing: every expert id must be a resident slot
bool b1_route_ok(int E, int num_slots) { return E >= 1 && E <= kMaxE && num_slots >= E; }

// logits != null: the gate/up kernel routes the token (slot = expert id) and
// writes slot_ids / w; otherwise they (and prec) are inputs.
moe_status launch_b1(const moe_layer* L, const float* logits, int E, const void* x, int k, int32_t* slot_ids,
                     const int8_t* prec, float* w, uint16_t* h, void* out, hipStream_t s) {
  B1Args a;
  a.H = L->H;
  a.I = L->I;
  a.k = k;
  a.K1 = k + (L->shared ? 1 : 0);
  a.E = E;
  a.fp4_base = L->fp4_base;
  a.fp4_stride = L->fp4_stride;
  a.num_slots = L->num_slots;
  a.int2_base = L->int2_base;
  a.int2_stride = L->int2_stride;
  a.num_int2 = L->int2_base ? L->num_int2 : 0;
  a.shared = L->shared;
  a.logits = logits;
  a.x = x;
  a.slot_ids = slot_ids;
  a.prec = logits ? nullptr : prec;
  a.w = w;
  a.h = h;
  a.out = out;
  {
    ProfScope prof(MOE_PROF_GATEUP, s);
    if (a.H == 2048)
      launch_gateup_b1<1>(a, s);
    else
      launch_gateup_b1<2>(a, s);
    MOE_LAUNCH_CHECK();
  }
  {
    ProfScope prof(MOE_PROF_DOWN, s);
    if (a.I == 2048)
      launch_down_b1<1>(a, s);
    else
      launch_down_b1<2>(a, s);
    MOE_LAUNCH_CHECK();
  }
  return MOE_OK;
}

}  // namespace moe
