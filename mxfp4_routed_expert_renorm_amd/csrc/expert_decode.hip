// Decode-sized expert MLP on MXFP4 weights (and the 2-bit copies), VALU GEMV.
//
// "An elephant through a straw" (§The evening the numbers lied, §The number)
// and "Running DeepSeek-V4-Flash across four free GPUs" (§The arithmetic that
// explains 20 tok/s) both find decode bound by moving expert bytes, not by
// arithmetic.  At batch 1 an expert is a matrix-vector product, so these
// kernels are built as a coalesced stream of the packed weight bytes:
//
//   * a wavefront splits a row's K dimension over LPR lanes (64 when K has
//     >= 2048 elements); each lane owns 32-element chunks, i.e. exactly one
//     16-byte FP4 load (or one 8-byte 2-bit load) plus its one scale byte, so
//     consecutive lanes read consecutive 16-byte pieces of the row and a
//     wave instruction moves 1 KiB of contiguous codes;
//   * the lane's activations for its chunks sit in registers for the whole
//     item (bf16 pairs for bf16 activations, floats otherwise), loaded once;
//   * FP4 codes are converted two at a time by the gfx950 scaled converts
//     (v_cvt_scalef32_pk_{bf16,f32}_fp4, scale 1.0) and multiplied in: a bf16
//     pair product goes through v_dot2_f32_bf16 (exact products, fp32 sums),
//     an fp32 activation through fp32 FMAs; the block's E8M0 scale is applied
//     once per 32 products;
//   * the LPR partial sums are reduced with lane shuffles, SwiGLU is applied
//     to the gate and up sums in the same kernel.
//
// Work items are (group, row tile).  A group is one expert record with the
// pairs (token, rank) that use it: at batch 1 each rank is its own group
// (implicit mode, no planning kernel); for larger batches the pairs are
// grouped by key (slot, 2-bit staging entry, shared) so each record streams
// once per group and the grid loops over the active groups.
#include <algorithm>

#include "common.h"

namespace moe {

namespace {

struct DecodeArgs {
  int H, I, T, k, K1;  // K1 = k + has_shared pairs per token
  const uint8_t* fp4_base;
  size_t fp4_stride;
  int num_slots;
  const uint8_t* int2_base;
  size_t int2_stride;
  int num_int2;
  const uint8_t* shared;
  const void* x;            // [T][H]
  const int32_t* slot_ids;  // [T][k]
  const int8_t* prec;       // [T][k] or null
  float* h;                 // [T*K1][I]
  float* y;                 // [T*K1][H]
  // grouped mode plan
  const int32_t* offsets;   // [nkeys+1]
  const int32_t* perm;      // pairs sorted by key
  const int32_t* active;    // [0] = number of active keys, then the keys
};

struct Group {
  const uint8_t* rec;  // null: nothing to do
  int prec;            // 0 FP4, 1 2-bit
  int start, count;    // pair list: perm[start .. start+count) (grouped) or the pair `start` (implicit)
};

// key of a pair for grouping: FP4 slot s -> s; 2-bit entry j -> num_slots + j;
// shared -> num_slots + num_int2; dropped or invalid -> -1
__device__ __forceinline__ int pair_key(const DecodeArgs& a, int p) {
  const int t = p / a.K1, r = p % a.K1;
  if (r == a.k) return a.num_slots + a.num_int2;
  const int pr = a.prec ? (int)a.prec[(size_t)t * a.k + r] : 0;
  const int s = a.slot_ids[(size_t)t * a.k + r];
  if (pr == 0) return (s >= 0 && s < a.num_slots) ? s : -1;
  if (pr == 1) return (s >= 0 && s < a.num_int2 && a.int2_base) ? a.num_slots + s : -1;
  return -1;
}

__device__ __forceinline__ Group key_group(const DecodeArgs& a, int key) {
  Group g;
  g.rec = nullptr;
  g.prec = 0;
  if (key < 0) return g;
  if (key < a.num_slots) {
    g.rec = a.fp4_base + (size_t)key * a.fp4_stride;
  } else if (key < a.num_slots + a.num_int2) {
    g.rec = a.int2_base + (size_t)(key - a.num_slots) * a.int2_stride;
    g.prec = 1;
  } else {
    g.rec = a.shared;
  }
  return g;
}

template <bool TABLE>
__device__ __forceinline__ Group resolve_group(const DecodeArgs& a, int gi) {
  if (TABLE) {
    const int key = a.active[1 + gi];
    Group g = key_group(a, key);
    g.start = a.offsets[key];
    g.count = a.offsets[key + 1] - g.start;
    return g;
  } else {
    Group g = key_group(a, pair_key(a, gi));  // batch 1: pair index == group index
    g.start = gi;
    g.count = 1;
    return g;
  }
}

template <bool TABLE>
__device__ __forceinline__ int group_pair(const DecodeArgs& a, const Group& g, int m) {
  return TABLE ? a.perm[g.start + m] : g.start;
}

// ----------------------------------------------------------------- dot kernels

// 32 FP4 codes (one 16-byte chunk) against 32 bf16 activations (16 pairs)
__device__ __forceinline__ float dot_fp4_bf16(const uint4 c, const uint32_t* xp) {
  float a0 = 0.0f, a1 = 0.0f;
  a0 = dot2_bf16(fp4x2_to_bf16x2<0>(c.x), xp[0], a0);
  a1 = dot2_bf16(fp4x2_to_bf16x2<1>(c.x), xp[1], a1);
  a0 = dot2_bf16(fp4x2_to_bf16x2<2>(c.x), xp[2], a0);
  a1 = dot2_bf16(fp4x2_to_bf16x2<3>(c.x), xp[3], a1);
  a0 = dot2_bf16(fp4x2_to_bf16x2<0>(c.y), xp[4], a0);
  a1 = dot2_bf16(fp4x2_to_bf16x2<1>(c.y), xp[5], a1);
  a0 = dot2_bf16(fp4x2_to_bf16x2<2>(c.y), xp[6], a0);
  a1 = dot2_bf16(fp4x2_to_bf16x2<3>(c.y), xp[7], a1);
  a0 = dot2_bf16(fp4x2_to_bf16x2<0>(c.z), xp[8], a0);
  a1 = dot2_bf16(fp4x2_to_bf16x2<1>(c.z), xp[9], a1);
  a0 = dot2_bf16(fp4x2_to_bf16x2<2>(c.z), xp[10], a0);
  a1 = dot2_bf16(fp4x2_to_bf16x2<3>(c.z), xp[11], a1);
  a0 = dot2_bf16(fp4x2_to_bf16x2<0>(c.w), xp[12], a0);
  a1 = dot2_bf16(fp4x2_to_bf16x2<1>(c.w), xp[13], a1);
  a0 = dot2_bf16(fp4x2_to_bf16x2<2>(c.w), xp[14], a0);
  a1 = dot2_bf16(fp4x2_to_bf16x2<3>(c.w), xp[15], a1);
  return a0 + a1;
}

template <int SEL>
__device__ __forceinline__ void fma_fp4x2_f32(uint32_t dw, const float* x2, float& a0, float& a1) {
  const v2f wv = fp4x2_to_f32<SEL>(dw);
  a0 = fmaf(wv.x, x2[0], a0);
  a1 = fmaf(wv.y, x2[1], a1);
}

// 32 FP4 codes against 32 fp32 activations
__device__ __forceinline__ float dot_fp4_f32(const uint4 c, const float* xf) {
  float a0 = 0.0f, a1 = 0.0f;
  const uint32_t d[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    fma_fp4x2_f32<0>(d[i], xf + 8 * i + 0, a0, a1);
    fma_fp4x2_f32<1>(d[i], xf + 8 * i + 2, a0, a1);
    fma_fp4x2_f32<2>(d[i], xf + 8 * i + 4, a0, a1);
    fma_fp4x2_f32<3>(d[i], xf + 8 * i + 6, a0, a1);
  }
  return a0 + a1;
}

// 32 two-bit codes (8 bytes) against 32 fp32 activations: sum (c - 1.5) x
__device__ __forceinline__ float dot_int2_f32(const uint2 c, const float* xf) {
  float a0 = 0.0f, a1 = 0.0f;
  const uint32_t d[2] = {c.x, c.y};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int q = 0; q < 16; q += 2) {
      a0 = fmaf((float)((d[i] >> (2 * q)) & 3u) - 1.5f, xf[16 * i + q], a0);
      a1 = fmaf((float)((d[i] >> (2 * q + 2)) & 3u) - 1.5f, xf[16 * i + q + 1], a1);
    }
  }
  return a0 + a1;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// activations of one 32-element chunk in registers
template <bool XBF16>
struct XChunk;
template <>
struct XChunk<true> {
  uint32_t p[16];
  __device__ __forceinline__ void load(const void* x, size_t elem) {
    const uint4* src = (const uint4*)((const uint16_t*)x + elem);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = src[i];
      p[4 * i + 0] = v.x;
      p[4 * i + 1] = v.y;
      p[4 * i + 2] = v.z;
      p[4 * i + 3] = v.w;
    }
  }
  __device__ __forceinline__ float dot_fp4(const uint4 c) const { return dot_fp4_bf16(c, p); }
  __device__ __forceinline__ float dot_int2(const uint2 c) const {
    float f[32];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      f[2 * i] = bf16_lo(p[i]);
      f[2 * i + 1] = bf16_hi(p[i]);
    }
    return dot_int2_f32(c, f);
  }
};
template <>
struct XChunk<false> {
  float f[32];
  __device__ __forceinline__ void load(const void* x, size_t elem) {
    const float4* src = (const float4*)((const float*)x + elem);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 v = src[i];
      f[4 * i + 0] = v.x;
      f[4 * i + 1] = v.y;
      f[4 * i + 2] = v.z;
      f[4 * i + 3] = v.w;
    }
  }
  __device__ __forceinline__ float dot_fp4(const uint4 c) const { return dot_fp4_f32(c, f); }
  __device__ __forceinline__ float dot_int2(const uint2 c) const { return dot_int2_f32(c, f); }
};

// --------------------------------------------------------------- gate / up

// h[p][row] = silu(W1[row] . x_t) * (W3[row] . x_t) for every pair p of a group
template <int LPR, int CPL, int U, bool XBF16, bool TABLE>
__global__ __launch_bounds__(256) void gateup_kernel(DecodeArgs a) {
  constexpr int RPW = 64 / LPR;
  constexpr int TILE = 4 * RPW * U;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & (LPR - 1), rsub = lane / LPR;
  const int H = a.H, I = a.I;
  const int tiles = I / TILE;
  const int nitems = TABLE ? a.active[0] * tiles : a.K1 * tiles;
  const size_t rowc4 = (size_t)H / 2, rowc2 = (size_t)H / 4, rows = (size_t)H / 32;

  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int gi = item / tiles, tile = item - gi * tiles;
    const Group g = resolve_group<TABLE>(a, gi);
    if (!g.rec) continue;
    const int row0 = tile * TILE + wave * RPW * U + rsub;
    const RecordLayout L = record_layout(H, I, g.prec == 0 ? 4 : 2);
    if (g.prec == 0) {
      uint4 c1[U][CPL], c3[U][CPL];
      uint32_t s1[U][CPL], s3[U][CPL];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t row = (size_t)(row0 + u * RPW);
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
          const int c = q * LPR + sub;
          c1[u][q] = ld_stream16(g.rec + L.w1c + row * rowc4 + (size_t)c * 16);
          c3[u][q] = ld_stream16(g.rec + L.w3c + row * rowc4 + (size_t)c * 16);
          s1[u][q] = g.rec[L.w1s + row * rows + c];
          s3[u][q] = g.rec[L.w3s + row * rows + c];
        }
      }
      for (int m = 0; m < g.count; ++m) {
        const int p = group_pair<TABLE>(a, g, m);
        const int t = p / a.K1;
        XChunk<XBF16> xc[CPL];
#pragma unroll
        for (int q = 0; q < CPL; ++q) xc[q].load(a.x, (size_t)t * H + (size_t)(q * LPR + sub) * 32);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float gs = 0.0f, us = 0.0f;
#pragma unroll
          for (int q = 0; q < CPL; ++q) {
            gs = fmaf(xc[q].dot_fp4(c1[u][q]), e8m0_to_f32(s1[u][q]), gs);
            us = fmaf(xc[q].dot_fp4(c3[u][q]), e8m0_to_f32(s3[u][q]), us);
          }
          gs = group_sum<LPR>(gs);
          us = group_sum<LPR>(us);
          if (sub == 0) a.h[(size_t)p * I + row0 + u * RPW] = silu_mul(gs, us);
        }
      }
    } else {
      uint2 c1[U][CPL], c3[U][CPL];
      uint32_t s1[U][CPL], s3[U][CPL];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t row = (size_t)(row0 + u * RPW);
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
          const int c = q * LPR + sub;
          c1[u][q] = ld_stream8(g.rec + L.w1c + row * rowc2 + (size_t)c * 8);
          c3[u][q] = ld_stream8(g.rec + L.w3c + row * rowc2 + (size_t)c * 8);
          s1[u][q] = g.rec[L.w1s + row * rows + c];
          s3[u][q] = g.rec[L.w3s + row * rows + c];
        }
      }
      for (int m = 0; m < g.count; ++m) {
        const int p = group_pair<TABLE>(a, g, m);
        const int t = p / a.K1;
        XChunk<XBF16> xc[CPL];
#pragma unroll
        for (int q = 0; q < CPL; ++q) xc[q].load(a.x, (size_t)t * H + (size_t)(q * LPR + sub) * 32);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float gs = 0.0f, us = 0.0f;
#pragma unroll
          for (int q = 0; q < CPL; ++q) {
            gs = fmaf(xc[q].dot_int2(c1[u][q]), e4m3_to_f32(s1[u][q]), gs);
            us = fmaf(xc[q].dot_int2(c3[u][q]), e4m3_to_f32(s3[u][q]), us);
          }
          gs = group_sum<LPR>(gs);
          us = group_sum<LPR>(us);
          if (sub == 0) a.h[(size_t)p * I + row0 + u * RPW] = silu_mul(gs, us);
        }
      }
    }
  }
}

// -------------------------------------------------------------------- down

// y[p][row] = W2[row] . h[p] for every pair p of a group (dropped pairs of
// the implicit mode get zeros)
template <int LPR, int CPL, int U, bool TABLE>
__global__ __launch_bounds__(256) void down_kernel(DecodeArgs a) {
  constexpr int RPW = 64 / LPR;
  constexpr int TILE = 4 * RPW * U;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & (LPR - 1), rsub = lane / LPR;
  const int H = a.H, I = a.I;
  const int tiles = H / TILE;
  const int nitems = TABLE ? a.active[0] * tiles : a.K1 * tiles;
  const size_t rowc4 = (size_t)I / 2, rowc2 = (size_t)I / 4, rows = (size_t)I / 32;

  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int gi = item / tiles, tile = item - gi * tiles;
    const Group g = resolve_group<TABLE>(a, gi);
    const int row0 = tile * TILE + wave * RPW * U + rsub;
    if (!g.rec) {
      if (!TABLE && sub == 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) a.y[(size_t)g.start * H + row0 + u * RPW] = 0.0f;
      }
      continue;
    }
    const RecordLayout L = record_layout(H, I, g.prec == 0 ? 4 : 2);
    if (g.prec == 0) {
      uint4 c2[U][CPL];
      uint32_t s2[U][CPL];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t row = (size_t)(row0 + u * RPW);
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
          const int c = q * LPR + sub;
          c2[u][q] = ld_stream16(g.rec + L.w2c + row * rowc4 + (size_t)c * 16);
          s2[u][q] = g.rec[L.w2s + row * rows + c];
        }
      }
      for (int m = 0; m < g.count; ++m) {
        const int p = group_pair<TABLE>(a, g, m);
        XChunk<false> hc[CPL];
#pragma unroll
        for (int q = 0; q < CPL; ++q) hc[q].load(a.h, (size_t)p * I + (size_t)(q * LPR + sub) * 32);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float ys = 0.0f;
#pragma unroll
          for (int q = 0; q < CPL; ++q) ys = fmaf(hc[q].dot_fp4(c2[u][q]), e8m0_to_f32(s2[u][q]), ys);
          ys = group_sum<LPR>(ys);
          if (sub == 0) a.y[(size_t)p * H + row0 + u * RPW] = ys;
        }
      }
    } else {
      uint2 c2[U][CPL];
      uint32_t s2[U][CPL];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t row = (size_t)(row0 + u * RPW);
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
          const int c = q * LPR + sub;
          c2[u][q] = ld_stream8(g.rec + L.w2c + row * rowc2 + (size_t)c * 8);
          s2[u][q] = g.rec[L.w2s + row * rows + c];
        }
      }
      for (int m = 0; m < g.count; ++m) {
        const int p = group_pair<TABLE>(a, g, m);
        XChunk<false> hc[CPL];
#pragma unroll
        for (int q = 0; q < CPL; ++q) hc[q].load(a.h, (size_t)p * I + (size_t)(q * LPR + sub) * 32);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float ys = 0.0f;
#pragma unroll
          for (int q = 0; q < CPL; ++q) ys = fmaf(hc[q].dot_int2(c2[u][q]), e4m3_to_f32(s2[u][q]), ys);
          ys = group_sum<LPR>(ys);
          if (sub == 0) a.y[(size_t)p * H + row0 + u * RPW] = ys;
        }
      }
    }
  }
}

// ------------------------------------------------------------ grouped plan

// keys[p] for every pair; dropped pairs get key -1 and a zeroed output row
__global__ __launch_bounds__(256) void pair_keys_kernel(DecodeArgs a, int32_t* __restrict__ keys) {
  const int p = blockIdx.x;
  const int key = pair_key(a, p);
  if (threadIdx.x == 0) keys[p] = key;
  if (key < 0) {
    for (int j = threadIdx.x; j < a.H; j += 256) a.y[(size_t)p * a.H + j] = 0.0f;
  }
}

// active[0] = number of keys with a non-zero count, active[1..] = those keys ascending
__global__ __launch_bounds__(64) void active_keys_kernel(const int32_t* __restrict__ counts, int nkeys,
                                                         int32_t* __restrict__ active) {
  const int lane = threadIdx.x;
  int n = 0;
  for (int base = 0; base < nkeys; base += 64) {
    const int i = base + lane;
    const bool on = i < nkeys && counts[i] > 0;
    const uint64_t m = __ballot(on);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (on) active[1 + n + __popcll(m & below)] = i;
    n += __popcll(m);
  }
  if (lane == 0) active[0] = n;
}

// ---------------------------------------------------------------- dispatch

// lanes per row and 32-element chunks per lane for a reduction length K
bool lanes_for(int K, int* lpr, int* cpl) {
  const int n = K / 32;
  if (K % 32 != 0 || n < 4) return false;
  if (n <= 64) {
    if (n & (n - 1)) return false;
    *lpr = n;
    *cpl = 1;
    return true;
  }
  if (n % 64 != 0) return false;
  *lpr = 64;
  *cpl = n / 64;
  return *cpl == 2 || *cpl == 4;
}

template <bool TABLE>
struct Launcher {
  template <int LPR, int CPL>
  static void gateup(const DecodeArgs& a, bool xbf16, int grid, hipStream_t s) {
    constexpr int U = (LPR == 64) ? 2 : 1;
    if (xbf16)
      launch(MOE_PROF_GATEUP, (gateup_kernel<LPR, CPL, U, true, TABLE>), dim3(grid), dim3(256), 0, s, a);
    else
      launch(MOE_PROF_GATEUP, (gateup_kernel<LPR, CPL, U, false, TABLE>), dim3(grid), dim3(256), 0, s, a);
  }
  template <int LPR, int CPL>
  static void down(const DecodeArgs& a, int grid, hipStream_t s) {
    constexpr int U = (LPR == 64) ? 2 : 1;
    launch(MOE_PROF_DOWN, (down_kernel<LPR, CPL, U, TABLE>), dim3(grid), dim3(256), 0, s, a);
  }
};

int tile_rows(int lpr) { return 4 * (64 / lpr) * (lpr == 64 ? 2 : 1); }

template <bool TABLE>
bool dispatch_gateup(int lpr, int cpl, const DecodeArgs& a, bool xbf16, int grid, hipStream_t s) {
  using Lc = Launcher<TABLE>;
  switch (lpr * 8 + cpl) {
    case 4 * 8 + 1: Lc::template gateup<4, 1>(a, xbf16, grid, s); return true;
    case 8 * 8 + 1: Lc::template gateup<8, 1>(a, xbf16, grid, s); return true;
    case 16 * 8 + 1: Lc::template gateup<16, 1>(a, xbf16, grid, s); return true;
    case 32 * 8 + 1: Lc::template gateup<32, 1>(a, xbf16, grid, s); return true;
    case 64 * 8 + 1: Lc::template gateup<64, 1>(a, xbf16, grid, s); return true;
    case 64 * 8 + 2: Lc::template gateup<64, 2>(a, xbf16, grid, s); return true;
    case 64 * 8 + 4: Lc::template gateup<64, 4>(a, xbf16, grid, s); return true;
  }
  return false;
}

template <bool TABLE>
bool dispatch_down(int lpr, int cpl, const DecodeArgs& a, int grid, hipStream_t s) {
  using Lc = Launcher<TABLE>;
  switch (lpr * 8 + cpl) {
    case 4 * 8 + 1: Lc::template down<4, 1>(a, grid, s); return true;
    case 8 * 8 + 1: Lc::template down<8, 1>(a, grid, s); return true;
    case 16 * 8 + 1: Lc::template down<16, 1>(a, grid, s); return true;
    case 32 * 8 + 1: Lc::template down<32, 1>(a, grid, s); return true;
    case 64 * 8 + 1: Lc::template down<64, 1>(a, grid, s); return true;
    case 64 * 8 + 2: Lc::template down<64, 2>(a, grid, s); return true;
    case 64 * 8 + 4: Lc::template down<64, 4>(a, grid, s); return true;
  }
  return false;
}

}  // namespace

bool decode_shape_ok(int H, int I) {
  int l, c;
  return lanes_for(H, &l, &c) && lanes_for(I, &l, &c);
}

// plan buffer (grouped mode): keys [P] | counts [kMaxKeys] | offsets [kMaxKeys+1] | perm [P] | active [kMaxKeys+1]
moe_status launch_expert_decode(const moe_layer* L, const void* x, moe_dtype xt, int T, int k,
                                const int32_t* slot_ids, const int8_t* prec, float* h, float* y,
                                int32_t* plan, hipStream_t s) {
  const int K1 = k + (L->shared ? 1 : 0);
  const int P = T * K1;
  DecodeArgs a;
  a.H = L->H;
  a.I = L->I;
  a.T = T;
  a.k = k;
  a.K1 = K1;
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
  a.h = h;
  a.y = y;
  a.offsets = nullptr;
  a.perm = nullptr;
  a.active = nullptr;

  int lpr_gu, cpl_gu, lpr_dn, cpl_dn;
  lanes_for(a.H, &lpr_gu, &cpl_gu);
  lanes_for(a.I, &lpr_dn, &cpl_dn);
  const int tiles_gu = a.I / tile_rows(lpr_gu);
  const int tiles_dn = a.H / tile_rows(lpr_dn);
  const bool xbf16 = xt == MOE_BF16;

  if (T == 1) {
    {
      if (!dispatch_gateup<false>(lpr_gu, cpl_gu, a, xbf16, K1 * tiles_gu, s))
        return fail(MOE_ESHAPE, "H=%d unsupported", a.H);
      MOE_LAUNCH_CHECK();
    }
    {
      if (!dispatch_down<false>(lpr_dn, cpl_dn, a, K1 * tiles_dn, s)) return fail(MOE_ESHAPE, "I=%d unsupported", a.I);
      MOE_LAUNCH_CHECK();
    }
    return MOE_OK;
  }
  const int nkeys = a.num_slots + a.num_int2 + 1;
  int32_t* keys = plan;
  int32_t* counts = keys + P;
  int32_t* offsets = counts + 4096;
  int32_t* perm = offsets + 4097;
  int32_t* active = perm + P;
  {
    launch(MOE_PROF_PLAN, pair_keys_kernel, dim3(P), dim3(256), 0, s, a, keys);
    MOE_LAUNCH_CHECK();
  }
  moe_status st = launch_group(keys, P, nkeys, counts, offsets, perm, s);
  if (st != MOE_OK) return st;
  {
    launch(MOE_PROF_PLAN, active_keys_kernel, dim3(1), dim3(64), 0, s, counts, nkeys, active);
    MOE_LAUNCH_CHECK();
  }
  a.offsets = offsets;
  a.perm = perm;
  a.active = active;
  // persistent grid over (active group, tile) items
  const int max_groups = (P < nkeys ? P : nkeys);
  const int grid_gu = (int)std::min<long>((long)max_groups * tiles_gu, 4096);
  const int grid_dn = (int)std::min<long>((long)max_groups * tiles_dn, 4096);
  {
    if (!dispatch_gateup<true>(lpr_gu, cpl_gu, a, xbf16, grid_gu, s)) return fail(MOE_ESHAPE, "H=%d unsupported", a.H);
    MOE_LAUNCH_CHECK();
  }
  {
    if (!dispatch_down<true>(lpr_dn, cpl_dn, a, grid_dn, s)) return fail(MOE_ESHAPE, "I=%d unsupported", a.I);
    MOE_LAUNCH_CHECK();
  }
  return MOE_OK;
}

size_t decode_plan_ints(int P) { return (size_t)P * 2 + 3 * 4097; }

}  // namespace moe
