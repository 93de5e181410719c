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

constexpr int kMT = 256;      // token rows per GEMM item (8 MFMA row blocks, 2 per wave)
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

__device__ __forceinline__ v8i load_a(const uint8_t* row, int k0, int h) {
  const uint4 lo = *(const uint4*)(row + k0 + 16 * h);
  const uint4 hi = *(const uint4*)(row + k0 + 32 + 16 * h);
  v8i r;
  r[0] = (int)lo.x, r[1] = (int)lo.y, r[2] = (int)lo.z, r[3] = (int)lo.w;
  r[4] = (int)hi.x, r[5] = (int)hi.y, r[6] = (int)hi.z, r[7] = (int)hi.w;
  return r;
}

__device__ __forceinline__ v8i load_b(const uint8_t* wrow, int k0, int h) {
  const uint4 q = ld_stream16(wrow + (k0 + 32 * h) / 2);
  v8i r;
  r[0] = (int)q.x, r[1] = (int)q.y, r[2] = (int)q.z, r[3] = (int)q.w;
  r[4] = 0, r[5] = 0, r[6] = 0, r[7] = 0;
  return r;
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

// ------------------------------------------------------------- gate / up GEMM

// item = (M tile of one expert's grouped rows, 64 intermediate rows); wave w owns
// row blocks w and w+4 of the M tile and both 32-row column blocks, for W1 and W3
__global__ __launch_bounds__(256) void gemm_gateup_kernel(PrefillArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 31, h = lane >> 5;
  const int H = a.H, I = a.I;
  const int ntiles = I / kNT;
  const int nitems = a.items[0] * ntiles;
  const RecordLayout L = record_layout(H, I, 4);
  const size_t rowb = (size_t)H / 2, rows = (size_t)H / 32;

  for (int item = virtual_block(); item < nitems; item += gridDim.x) {
    const int mi = item / ntiles, nt = item - mi * ntiles;
    const int key = a.items[1 + 2 * mi], row0 = a.items[2 + 2 * mi];
    const int start = a.offsets[key], count = a.offsets[key + 1] - start;
    const uint8_t* rec = key_record(a, key);
    // the wave's two row blocks (token rows) and their activation rows
    int nrb = 0;
    const uint8_t* arow[2];
    const uint8_t* srow[2];
    bool live[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = row0 + (wave + 4 * j) * 32;  // first row of the block
      live[j] = r < count;
      nrb += live[j] ? 1 : 0;
      const int pos = min(r + c, count - 1);
      const int t = a.perm[start + pos] / a.K1;
      arow[j] = a.xq + (size_t)t * H;
      srow[j] = a.xs + (size_t)t * (H / 32);
    }
    if (nrb == 0) continue;
    const uint8_t* w1r[2];
    const uint8_t* w3r[2];
    const uint8_t* s1r[2];
    const uint8_t* s3r[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const size_t n = (size_t)(nt * kNT + nb * 32 + c);
      w1r[nb] = rec + L.w1c + n * rowb;
      w3r[nb] = rec + L.w3c + n * rowb;
      s1r[nb] = rec + L.w1s + n * rows;
      s3r[nb] = rec + L.w3s + n * rows;
    }
    v16f acc_g[2][2], acc_u[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc_g[j][nb][i] = 0.0f, acc_u[j][nb][i] = 0.0f;

    for (int k0 = 0; k0 < H; k0 += 64) {
      const int kb = k0 / 32 + h;
      v8i bg[2], bu[2];
      int sg[2], su[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        bg[nb] = load_b(w1r[nb], k0, h);
        bu[nb] = load_b(w3r[nb], k0, h);
        sg[nb] = s1r[nb][kb];
        su[nb] = s3r[nb][kb];
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (!live[j]) continue;
        const v8i av = load_a(arow[j], k0, h);
        const int sa = srow[j][kb];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          acc_g[j][nb] = mfma_fp8_fp4(av, bg[nb], acc_g[j][nb], sa, sg[nb]);
          acc_u[j][nb] = mfma_fp8_fp4(av, bu[nb], acc_u[j][nb], sa, su[nb]);
        }
      }
    }
    // SwiGLU, MXFP8 requantisation along I (a 32-column block is one half-wave row)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (!live[j]) continue;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int col = nt * kNT + nb * 32 + c;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float g = acc_g[j][nb][i], u = acc_u[j][nb][i];
          const float hv = g / (1.0f + expf(-g)) * u;
          const float amax = half_wave_max(fabsf(hv));
          const int sh = mx_shared_exp(amax);
          const int r = row0 + (wave + 4 * j) * 32 + 8 * (i / 4) + 4 * h + (i % 4);
          if (r < count) {
            const size_t pos = (size_t)(start + r);
            a.hq[pos * I + col] = (uint8_t)e4m3_encode(ldexpf(hv, -sh));
            if (c == 0) a.hs[pos * (I / 32) + col / 32] = (uint8_t)(sh + 127);
          }
        }
      }
    }
  }
}

// ----------------------------------------------------------------- down GEMM

// item = (M tile of grouped rows, 64 output columns of H); the grouped h rows are
// contiguous; each result goes to its (token, rank) pair as bf16
__global__ __launch_bounds__(256) void gemm_down_kernel(PrefillArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 31, h = lane >> 5;
  const int H = a.H, I = a.I;
  const int ntiles = H / kNT;
  const int nitems = a.items[0] * ntiles;
  const RecordLayout L = record_layout(H, I, 4);
  const size_t rowb = (size_t)I / 2, rows = (size_t)I / 32;

  for (int item = virtual_block(); item < nitems; item += gridDim.x) {
    const int mi = item / ntiles, nt = item - mi * ntiles;
    const int key = a.items[1 + 2 * mi], row0 = a.items[2 + 2 * mi];
    const int start = a.offsets[key], count = a.offsets[key + 1] - start;
    const uint8_t* rec = key_record(a, key);
    const uint8_t* arow[2];
    const uint8_t* srow[2];
    bool live[2];
    int nrb = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = row0 + (wave + 4 * j) * 32;
      live[j] = r < count;
      nrb += live[j] ? 1 : 0;
      const size_t pos = (size_t)(start + min(r + c, count - 1));
      arow[j] = a.hq + pos * I;
      srow[j] = a.hs + pos * (I / 32);
    }
    if (nrb == 0) continue;
    const uint8_t* wr[2];
    const uint8_t* sr[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const size_t n = (size_t)(nt * kNT + nb * 32 + c);
      wr[nb] = rec + L.w2c + n * rowb;
      sr[nb] = rec + L.w2s + n * rows;
    }
    v16f acc[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][nb][i] = 0.0f;
    for (int k0 = 0; k0 < I; k0 += 64) {
      const int kb = k0 / 32 + h;
      v8i bw[2];
      int sw[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        bw[nb] = load_b(wr[nb], k0, h);
        sw[nb] = sr[nb][kb];
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (!live[j]) continue;
        const v8i av = load_a(arow[j], k0, h);
        const int sa = srow[j][kb];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[j][nb] = mfma_fp8_fp4(av, bw[nb], acc[j][nb], sa, sw[nb]);
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (!live[j]) continue;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = row0 + (wave + 4 * j) * 32 + 8 * (i / 4) + 4 * h + (i % 4);
        if (r < count) {
          const size_t pair = (size_t)a.perm[start + r];
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) a.y[pair * H + nt * kNT + nb * 32 + c] = f32_to_bf16(acc[j][nb][i]);
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
  ProfScope prof(MOE_PROF_QUANT, s);
  hipLaunchKernelGGL(quant_mxfp8_kernel, dim3((unsigned)((nblk + 255) / 256)), dim3(256), 0, s, (const uint16_t*)x,
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
    ProfScope prof(MOE_PROF_PLAN, s);
    hipLaunchKernelGGL(prefill_keys_kernel, dim3((P + 255) / 256), dim3(256), 0, s, a);
    MOE_LAUNCH_CHECK();
  }
  st = launch_group(a.keys, P, E + 1, a.counts, a.offsets, a.perm, s);
  if (st != MOE_OK) return st;
  {
    ProfScope prof(MOE_PROF_PLAN, s);
    hipLaunchKernelGGL(prefill_items_kernel, dim3(1), dim3(64), 0, s, a.counts, E + 1, a.items);
    MOE_LAUNCH_CHECK();
  }
  // persistent grids, a multiple of 8 workgroups (one share per XCD)
  const int max_items_m = P / kMT + E + 1;
  const int grid_gu = (int)std::min<long>((long)max_items_m * (I / kNT), 256L * 8) / 8 * 8;
  const int grid_dn = (int)std::min<long>((long)max_items_m * (H / kNT), 256L * 8) / 8 * 8;
  {
    ProfScope prof(MOE_PROF_GEMM_GATEUP, s);
    hipLaunchKernelGGL(gemm_gateup_kernel, dim3(std::max(grid_gu, 8)), dim3(256), 0, s, a);
    MOE_LAUNCH_CHECK();
  }
  {
    ProfScope prof(MOE_PROF_GEMM_DOWN, s);
    hipLaunchKernelGGL(gemm_down_kernel, dim3(std::max(grid_dn, 8)), dim3(256), 0, s, a);
    MOE_LAUNCH_CHECK();
  }
  {
    ProfScope prof(MOE_PROF_COMBINE, s);
    const long n = (long)T * (H / 8);
    hipLaunchKernelGGL(combine_bf16y_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.y, w, T, k, K1,
                       H, (uint16_t*)out);
    MOE_LAUNCH_CHECK();
  }
  return MOE_OK;
}

}  // namespace moe
