// Prefill-sized grouped GEMM on gfx950 scaled MFMA (MXFP8 activations x MXFP4 weights).
//
// With thousands of tokens every expert sees a block of tokens, so the expert
// MLP is a dense contraction and belongs on the matrix cores.  Per layer:
//   1. x is quantised to MXFP8 (E4M3 codes, one E8M0 scale per 32 along H);
//   2. the (token, rank) pairs are grouped by expert (stable counting sort);
//   3. gate/up: for every expert, G = A_e W1^T and U = A_e W3^T over the
//      expert's gathered token rows, SwiGLU in the epilogue, and h requantised
//      to MXFP8 along I, written in grouped row order;
//   4. down: Y = h_e W2^T per expert, written as bf16 per (token, rank);
//   5. combine: out = sum_r w_r y_r (+ shared), one rounding to bf16.
// "Running DeepSeek-V4-Flash across four free GPUs", §What the expert cache
// actually does and §Step 7 (prefill takes a whole-layer path above the
// T*top_k >= num_experts crossover) describe prefill as streaming whole
// expert layers; here the layer is resident and streamed once per expert.
//
// MFMA operand layout (v_mfma_scale_f32_32x32x64_f8f6f4, measured on gfx950):
// lane l = 32*h + c.  B (FP4, one weight row c per lane): 16 bytes holding
// K [32h, 32h+32) of the 64-wide K step, i.e. exactly one scale block of the
// row, whose E8M0 byte is the lane's B scale.  A (FP8, one token row c per
// lane): bytes 0..15 hold K [16h, 16h+16), bytes 16..31 hold K [32+16h, +16);
// the lane's A scale is the row's block h.  Output: acc[i] is row
// 8*(i/4) + 4*h + i%4, column c.
#include <algorithm>

#include "common.h"

namespace moe {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

#ifndef MOE_PF_WAVES
#define MOE_PF_WAVES 8
#endif
constexpr int kWaves = MOE_PF_WAVES;  // wavefronts per GEMM workgroup, one 32-row block each
constexpr int kMT = 32 * kWaves;      // grouped token rows per GEMM item
constexpr int kNT = 64;       // weight rows per GEMM item (2 MFMA column blocks)
constexpr int kMaxKeys = 4096;

// ------------------------------------------------------------------ MXFP8

// nearest E4M3 (OCP E4M3FN) code of a value, ties to even, saturating at 448
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {  // below 2^-6: subnormal steps of 2^-9 (code 8 is the smallest normal)
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;
    const float mant = a * __uint_as_float((uint32_t)(127 - e) << 23);  // in [1, 2)
    uint32_t m3 = (uint32_t)__builtin_rintf((mant - 1.0f) * 8.0f);
    if (m3 == 8u) {
      m3 = 0u;
      e += 1;
    }
    code = ((uint32_t)(e + 7) << 3) | m3;
  }
  return sign | code;
}

// shared exponent of a 32-block with maximum magnitude amax: floor(log2 amax) - 8,
// clamped to the E8M0 range; an all-zero block gets -127 (scale byte 0)
__device__ __forceinline__ int mx_shared_exp(float amax) {
  if (!(amax > 0.0f)) return -127;
  const int e = ilogbf(amax) - 8;
  return max(-127, min(127, e));
}

// one thread per 32-element block of a bf16 row-major [rows][K] matrix
__global__ __launch_bounds__(256) void quant_mxfp8_kernel(const uint16_t* __restrict__ x, long nblk,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const long b = (long)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblk) return;
  const uint4* src = (const uint4*)(x + b * 32);
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 q = src[i];
    const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = bf16_lo(d[j]);
      v[8 * i + 2 * j + 1] = bf16_hi(d[j]);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int sh = mx_shared_exp(amax);
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    out[i] = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) out[i] |= e4m3_encode(ldexpf(v[4 * i + j], -sh)) << (8 * j);
  }
  uint4* dst = (uint4*)(codes + b * 32);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  scales[b] = (uint8_t)(sh + 127);
}

// ------------------------------------------------------------------ planning

struct PrefillArgs {
  int T, H, I, k, K1, E;
  const uint8_t* bank;  // expert e at bank + e*stride
  size_t stride;
  const uint8_t* shared;
  const int32_t* ids;   // [T][k] expert ids
  const uint8_t* xq;    // [T][H] E4M3
  const uint8_t* xs;    // [T][H/32] E8M0
  // plan
  int32_t* keys;        // [P]
  int32_t* counts;      // [nkeys]
  int32_t* offsets;     // [nkeys+1]
  int32_t* perm;        // [P] sorted position -> pair
  int32_t* items;       // [0] = number of M-tiles, then (key, row0) pairs
  // intermediate and output
  uint8_t* hq;          // [P][I] E4M3, grouped order
  uint8_t* hs;          // [P][I/32]
  uint16_t* y;          // [P][H] bf16, pair order
};

__global__ __launch_bounds__(256) void prefill_keys_kernel(PrefillArgs a) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= a.T * a.K1) return;
  const int t = p / a.K1, r = p % a.K1;
  int key;
  if (r == a.k) {
    key = a.E;
  } else {
    const int e = a.ids[(size_t)t * a.k + r];
    key = (e >= 0 && e < a.E) ? e : -1;
  }
  a.keys[p] = key;
  if (key < 0) {  // an out-of-range id contributes nothing: its output row is zero
    uint4* yrow = (uint4*)(a.y + (size_t)p * a.H);
    for (int j = 0; j < a.H / 8; ++j) yrow[j] = make_uint4(0u, 0u, 0u, 0u);
  }
}

// items[0] = number of (key, row0) M-tiles; tiles of kMT rows per non-empty key
__global__ __launch_bounds__(64) void prefill_items_kernel(const int32_t* __restrict__ counts, int nkeys,
                                                           int32_t* __restrict__ items) {
  const int lane = threadIdx.x;
  int n = 0;
  for (int base = 0; base < nkeys; base += 64) {
    const int key = base + lane;
    const int c = key < nkeys ? counts[key] : 0;
    const int tiles = (c + kMT - 1) / kMT;
    int incl = tiles;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    const int first = n + incl - tiles;
    for (int i = 0; i < tiles; ++i) {
      items[1 + 2 * (first + i)] = key;
      items[2 + 2 * (first + i)] = i * kMT;
    }
    n += __shfl(incl, 63, 64);
  }
  if (lane == 0) items[0] = n;
}

__device__ __forceinline__ const uint8_t* key_record(const PrefillArgs& a, int key) {
  return key == a.E ? a.shared : a.bank + (size_t)key * a.stride;
}

// XCD-aware order: workgroup b runs on XCD b % 8; give each XCD a contiguous
// range of virtual ids so neighbouring items (the N tiles of one M tile share
// its activation rows) stay in one L2
__device__ __forceinline__ int virtual_block() {
  const int g = gridDim.x;
  const int per = g / 8;
  return (blockIdx.x % 8) * per + blockIdx.x / 8;
}

__device__ __forceinline__ v16f mfma_fp8_fp4(v8i a, v8i b, v16f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 4, 0, sa, 0, sb);
}

// max over the 32 lanes of each half-wave, returned to every lane of the half
__device__ __forceinline__ float half_wave_max(float v) {
  v = fmaxf(v, dpp_f32<dpp::kQuadXor1>(v));
  v = fmaxf(v, dpp_f32<dpp::kQuadXor2>(v));
  v = fmaxf(v, dpp_f32<dpp::kRowHalfMirror>(v));
  v = fmaxf(v, dpp_f32<dpp::kRowMirror>(v));
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return v;
}

// ------------------------------------------------------------- grouped GEMM
//
// One template for both products.  An item is (M tile = up to 256 grouped rows
// of one expert, N tile = 64 weight rows of each of NMAT matrices).  The
// workgroup's 8 wavefronts own one 32-row block of the M tile each and every
// 32x32 output block of the N tile.  K advances 128 at a time through a
// double-buffered LDS stage: each thread's share of the next stage's
// activation rows, weight rows and their scale bytes is loaded into registers
// while the current stage feeds the MFMAs, then written to the other buffer.
// LDS rows are padded by 16 bytes so the 32 rows a fragment read touches fall
// in different banks.  Items run N tile innermost and each XCD takes a
// contiguous range, so the N tiles of one M tile share its activation rows in
// one L2 while the expert's weights stream from HBM once per M tile.

constexpr int kKS = 128;                 // K per stage
constexpr int kArow = kKS + 16;          // padded bytes per activation row in LDS
constexpr int kBrow = kKS / 2 + 16;      // padded bytes per weight row in LDS

template <int NMAT>
struct GemmSmem {
  uint8_t a[2][kMT * kArow];
  uint8_t b[2][NMAT * kNT * kBrow];
  uint32_t as[2][kMT];                  // 4 scale bytes (this stage's 4 blocks) per row
  uint32_t bs[2][NMAT * kNT];
};

// 16-byte pieces of the weight tile per thread (4 pieces per 64-byte row)
template <int NMAT>
constexpr int pieces_b() { return (NMAT * kNT * 4 + kWaves * 64 - 1) / (kWaves * 64); }

template <int NMAT>
struct StageRegs {
  uint4 a[4];              // 64 activation bytes: half of row tid/2
  uint4 b[pieces_b<NMAT>()];  // weight pieces tid + j*threads
  uint32_t as, bs;         // scale dwords of activation row tid and weight row tid
};

// thread tid loads, for K [k0, k0+kKS): 64 bytes of activation row tid/2, the 4
// scale bytes of activation row tid (tid < kMT), 16-byte pieces p = tid +
// j*threads of the weight tile (row p/4, quarter p%4) and the 4 scale bytes of
// weight row tid (tid < NMAT*kNT)
template <int NMAT>
__device__ __forceinline__ void stage_load(StageRegs<NMAT>& r, const uint8_t* arow, const uint8_t* asrow,
                                           const uint8_t* const* brow, const uint8_t* bsrow, int k0, int tid,
                                           bool arow_live, bool asrow_live) {
  if (arow_live) {  // rows past the group's end feed only discarded outputs: not loaded
    const uint4* ap = (const uint4*)(arow + k0 + 64 * (tid & 1));
#pragma unroll
    for (int i = 0; i < 4; ++i) r.a[i] = ap[i];
  }
  if (tid < kMT && asrow_live) r.as = *(const uint32_t*)(asrow + k0 / 32);
#pragma unroll
  for (int j = 0; j < pieces_b<NMAT>(); ++j) {
    const int p = tid + j * kWaves * 64;
    if (p < NMAT * kNT * 4) r.b[j] = ld_stream16(brow[j] + k0 / 2 + 16 * (p & 3));
  }
  if (tid < NMAT * kNT) r.bs = *(const uint32_t*)(bsrow + k0 / 32);
}

template <int NMAT>
__device__ __forceinline__ void stage_store(GemmSmem<NMAT>& sm, int buf, const StageRegs<NMAT>& r, int tid,
                                            bool arow_live, bool asrow_live) {
  if (arow_live) {
    uint4* ad = (uint4*)(sm.a[buf] + (tid >> 1) * kArow + 64 * (tid & 1));
#pragma unroll
    for (int i = 0; i < 4; ++i) ad[i] = r.a[i];
  }
  if (tid < kMT && asrow_live) sm.as[buf][tid] = r.as;
#pragma unroll
  for (int j = 0; j < pieces_b<NMAT>(); ++j) {
    const int p = tid + j * kWaves * 64;
    if (p < NMAT * kNT * 4) *(uint4*)(sm.b[buf] + (p >> 2) * kBrow + 16 * (p & 3)) = r.b[j];
  }
  if (tid < NMAT * kNT) sm.bs[buf][tid] = r.bs;
}

// NMAT = 2: gate/up (W1, W3 of the expert, K = H), SwiGLU + MXFP8 epilogue into hq/hs.
// NMAT = 1: down (W2, K = I), bf16 epilogue into y at each row's (token, rank) pair.
template <int NMAT>
__global__ __launch_bounds__(kWaves * 64) void gemm_kernel(PrefillArgs a) {
  __shared__ GemmSmem<NMAT> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, h = lane >> 5;
  const int H = a.H, I = a.I;
  const int K = NMAT == 2 ? H : I;        // reduction length
  const int Nall = NMAT == 2 ? I : H;     // weight rows per matrix
  const int ntiles = Nall / kNT;
  const int nitems = a.items[0] * ntiles;
  const RecordLayout L = record_layout(H, I, 4);
  const size_t wrowb = (size_t)K / 2, wrows = (size_t)K / 32;

  for (int item = virtual_block(); item < nitems; item += gridDim.x) {
    const int mi = item / ntiles, nt = item - mi * ntiles;
    const int key = a.items[1 + 2 * mi], row0 = a.items[2 + 2 * mi];
    const int start = a.offsets[key], count = a.offsets[key + 1] - start;
    const uint8_t* rec = key_record(a, key);
    // this thread's load rows: activation row tid/2 (codes) and tid (scales),
    // weight row tid/4 (codes) and tid (scales)
    auto act_rows = [&](int i, const uint8_t** codes, const uint8_t** scales) {
      const int ri = min(row0 + i, count - 1);
      if (NMAT == 2) {
        const int t = a.perm[start + ri] / a.K1;
        *codes = a.xq + (size_t)t * H;
        *scales = a.xs + (size_t)t * (H / 32);
      } else {
        *codes = a.hq + (size_t)(start + ri) * I;
        *scales = a.hs + (size_t)(start + ri) * (I / 32);
      }
    };
    auto weight_rows = [&](int wr, const uint8_t** codes, const uint8_t** scales) {
      wr = min(wr, NMAT * kNT - 1);
      const int mat = wr / kNT;
      const size_t n = (size_t)(nt * kNT + (wr % kNT));
      const size_t code_off = NMAT == 2 ? (mat == 0 ? L.w1c : L.w3c) : L.w2c;
      const size_t scale_off = NMAT == 2 ? (mat == 0 ? L.w1s : L.w3s) : L.w2s;
      *codes = rec + code_off + n * wrowb;
      *scales = rec + scale_off + n * wrows;
    };
    const uint8_t *arow, *asrow, *bsrow, *unused;
    const uint8_t* brow[pieces_b<NMAT>()];
    act_rows(tid >> 1, &arow, &unused);
    act_rows(min(tid, kMT - 1), &unused, &asrow);
#pragma unroll
    for (int j = 0; j < pieces_b<NMAT>(); ++j) weight_rows((tid + j * kWaves * 64) >> 2, &brow[j], &unused);
    weight_rows(tid, &unused, &bsrow);
    const bool live = row0 + wave * 32 < count;
    const bool arow_live = row0 + (tid >> 1) < count;
    const bool asrow_live = row0 + tid < count;

    v16f acc[NMAT][2];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[m][nb][i] = 0.0f;

    StageRegs<NMAT> st;
    stage_load<NMAT>(st, arow, asrow, brow, bsrow, 0, tid, arow_live, asrow_live);
    __syncthreads();  // the previous item's last stage reads are done
    stage_store<NMAT>(sm, 0, st, tid, arow_live, asrow_live);
    __syncthreads();
    const int nstage = K / kKS;
    for (int s = 0; s < nstage; ++s) {
      const int buf = s & 1;
      if (s + 1 < nstage) stage_load<NMAT>(st, arow, asrow, brow, bsrow, (s + 1) * kKS, tid, arow_live, asrow_live);
      if (live) {
#pragma unroll
        for (int kc = 0; kc < kKS / 64; ++kc) {
          const uint8_t* ar = sm.a[buf] + (wave * 32 + c) * kArow + kc * 64;
          const uint4 lo = *(const uint4*)(ar + 16 * h);
          const uint4 hi = *(const uint4*)(ar + 32 + 16 * h);
          v8i av;
          av[0] = (int)lo.x, av[1] = (int)lo.y, av[2] = (int)lo.z, av[3] = (int)lo.w;
          av[4] = (int)hi.x, av[5] = (int)hi.y, av[6] = (int)hi.z, av[7] = (int)hi.w;
          const int sa = (int)((sm.as[buf][wave * 32 + c] >> (8 * (2 * kc + h))) & 0xffu);
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
              const int r = m * kNT + nb * 32 + c;
              const uint4 q = *(const uint4*)(sm.b[buf] + r * kBrow + kc * 32 + 16 * h);
              v8i bv;
              bv[0] = (int)q.x, bv[1] = (int)q.y, bv[2] = (int)q.z, bv[3] = (int)q.w;
              bv[4] = 0, bv[5] = 0, bv[6] = 0, bv[7] = 0;
              const int sb = (int)((sm.bs[buf][r] >> (8 * (2 * kc + h))) & 0xffu);
              acc[m][nb] = mfma_fp8_fp4(av, bv, acc[m][nb], sa, sb);
            }
        }
      }
      if (s + 1 < nstage) stage_store<NMAT>(sm, buf ^ 1, st, tid, arow_live, asrow_live);
      __syncthreads();
    }
    if (!live) continue;
    if (NMAT == 2) {
      // SwiGLU, MXFP8 requantisation along I (a 32-column block is one half-wave row)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int col = nt * kNT + nb * 32 + c;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float g = acc[0][nb][i], u = acc[NMAT - 1][nb][i];
          const float hv = g / (1.0f + expf(-g)) * u;
          const float amax = half_wave_max(fabsf(hv));
          const int sh = mx_shared_exp(amax);
          const int r = row0 + wave * 32 + 8 * (i / 4) + 4 * h + (i % 4);
          if (r < count) {
            const size_t pos = (size_t)(start + r);
            a.hq[pos * I + col] = (uint8_t)e4m3_encode(ldexpf(hv, -sh));
            if (c == 0) a.hs[pos * (I / 32) + col / 32] = (uint8_t)(sh + 127);
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = row0 + wave * 32 + 8 * (i / 4) + 4 * h + (i % 4);
        if (r < count) {
          const size_t pair = (size_t)a.perm[start + r];
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) a.y[pair * H + nt * kNT + nb * 32 + c] = f32_to_bf16(acc[0][nb][i]);
        }
      }
    }
  }
}

// out[t] = sum_{r<k} w[t][r] * y[t][r] (+ y[t][k]), y bf16, rank order, one rounding
__global__ __launch_bounds__(256) void combine_bf16y_kernel(const uint16_t* __restrict__ y, const float* __restrict__ w,
                                                            int T, int k, int K1, int H, uint16_t* __restrict__ out) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const int oct = H / 8;
  if (idx >= (long)T * oct) return;
  const int t = (int)(idx / oct), j = (int)(idx % oct) * 8;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int r = 0; r < K1; ++r) {
    const uint4 v = *(const uint4*)(y + ((size_t)t * K1 + r) * H + j);
    const float wr = r < k ? w[(size_t)t * k + r] : 1.0f;
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] = fmaf(wr, bf16_lo(d[q]), acc[2 * q]);
      acc[2 * q + 1] = fmaf(wr, bf16_hi(d[q]), acc[2 * q + 1]);
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = (uint32_t)f32_to_bf16(acc[2 * q]) | ((uint32_t)f32_to_bf16(acc[2 * q + 1]) << 16);
  *(uint4*)(out + (size_t)t * H + j) = make_uint4(o[0], o[1], o[2], o[3]);
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

struct PrefillWs {
  size_t xq, xs, keys, counts, offsets, perm, items, hq, hs, y, total;
};

PrefillWs prefill_ws_layout(int H, int I, int T, int K1) {
  const size_t P = (size_t)T * K1;
  PrefillWs w;
  size_t o = 0;
  w.xq = o; o += align256((size_t)T * H);
  w.xs = o; o += align256((size_t)T * H / 32);
  w.keys = o; o += align256(P * 4);
  w.counts = o; o += align256((size_t)kMaxKeys * 4);
  w.offsets = o; o += align256((size_t)(kMaxKeys + 1) * 4);
  w.perm = o; o += align256(P * 4);
  w.items = o; o += align256((1 + 2 * (P / kMT + kMaxKeys + 1)) * 4);
  w.hq = o; o += align256(P * I);
  w.hs = o; o += align256(P * I / 32);
  w.y = o; o += align256(P * H * 2);
  w.total = o;
  return w;
}

}  // namespace

size_t prefill_workspace_bytes(int H, int I, int T, int k, int has_shared) {
  return prefill_ws_layout(H, I, T, k + (has_shared ? 1 : 0)).total;
}

moe_status launch_quant_mxfp8(const void* x, long rows, int K, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const long nblk = rows * (K / 32);
  if (nblk == 0) return MOE_OK;
  launch(MOE_PROF_QUANT, quant_mxfp8_kernel, dim3((unsigned)((nblk + 255) / 256)), dim3(256), 0, s, (const uint16_t*)x,
                     nblk, codes, scales);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

moe_status launch_prefill(const moe_layer* Lr, int E, const void* x, int T, int k, const int32_t* ids, const float* w,
                          void* out, void* workspace, hipStream_t s) {
  const int K1 = k + (Lr->shared ? 1 : 0);
  const int H = Lr->H, I = Lr->I;
  const int P = T * K1;
  const PrefillWs lay = prefill_ws_layout(H, I, T, K1);
  char* ws = (char*)workspace;
  PrefillArgs a;
  a.T = T, a.H = H, a.I = I, a.k = k, a.K1 = K1, a.E = E;
  a.bank = Lr->fp4_base;
  a.stride = Lr->fp4_stride;
  a.shared = Lr->shared;
  a.ids = ids;
  a.xq = (uint8_t*)(ws + lay.xq);
  a.xs = (uint8_t*)(ws + lay.xs);
  a.keys = (int32_t*)(ws + lay.keys);
  a.counts = (int32_t*)(ws + lay.counts);
  a.offsets = (int32_t*)(ws + lay.offsets);
  a.perm = (int32_t*)(ws + lay.perm);
  a.items = (int32_t*)(ws + lay.items);
  a.hq = (uint8_t*)(ws + lay.hq);
  a.hs = (uint8_t*)(ws + lay.hs);
  a.y = (uint16_t*)(ws + lay.y);

  moe_status st = launch_quant_mxfp8(x, T, H, (uint8_t*)a.xq, (uint8_t*)a.xs, s);
  if (st != MOE_OK) return st;
  {
    launch(MOE_PROF_PLAN, prefill_keys_kernel, dim3((P + 255) / 256), dim3(256), 0, s, a);
    MOE_LAUNCH_CHECK();
  }
  st = launch_group(a.keys, P, E + 1, a.counts, a.offsets, a.perm, s);
  if (st != MOE_OK) return st;
  {
    launch(MOE_PROF_PLAN, prefill_items_kernel, dim3(1), dim3(64), 0, s, a.counts, E + 1, a.items);
    MOE_LAUNCH_CHECK();
  }
  // persistent grids: as many workgroups as fit per CU (LDS-limited: one of 8
  // wavefronts or two of 4), a multiple of 8 (one share per XCD)
  const long per_cu = kWaves >= 8 ? 1 : 2;
  const int max_items_m = P / kMT + E + 1;
  const int grid_gu = (int)std::min<long>((long)max_items_m * (I / kNT), 256L * per_cu) / 8 * 8;
  const int grid_dn = (int)std::min<long>((long)max_items_m * (H / kNT), 256L * per_cu) / 8 * 8;
  {
    launch(MOE_PROF_GEMM_GATEUP, gemm_kernel<2>, dim3(std::max(grid_gu, 8)), dim3(kWaves * 64), 0, s, a);
    MOE_LAUNCH_CHECK();
  }
  {
    launch(MOE_PROF_GEMM_DOWN, gemm_kernel<1>, dim3(std::max(grid_dn, 8)), dim3(kWaves * 64), 0, s, a);
    MOE_LAUNCH_CHECK();
  }
  {
    const long n = (long)T * (H / 8);
    launch(MOE_PROF_COMBINE, combine_bf16y_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.y, w, T, k, K1,
                       H, (uint16_t*)out);
    MOE_LAUNCH_CHECK();
  }
  return MOE_OK;
}

}  // namespace moe
