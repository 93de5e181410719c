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
#include <type_traits>

#include "common.h"
#include "group_dev.h"

namespace moe {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

#ifndef MOE_PF_WAVES
#define MOE_PF_WAVES 4
#endif
constexpr int kWaves = MOE_PF_WAVES;  // wavefronts per GEMM workgroup (4: one per SIMD, or 8)
#ifndef MOE_PF_MB
#define MOE_PF_MB 6
#endif
constexpr int kMB = MOE_PF_MB;  // 32-row M blocks per item at most (4 or 6)
constexpr int kMT = 32 * kMB; // grouped rows per item at most
constexpr int kNR = 256;      // weight rows per item (8 MFMA column blocks)
#ifndef MOE_PF_DEPTH
#define MOE_PF_DEPTH 1
#endif
constexpr int kDepth = MOE_PF_DEPTH;  // K stages held in registers ahead of the LDS stage
constexpr int kMaxKeys = 4096;

// ------------------------------------------------------------------ MXFP8

// nearest E4M3 (OCP E4M3FN) code of a value, ties to even, saturating at
// +-448: gfx950's convert rounds to nearest even, and clamping first turns
// its overflow into the saturation the MX rule asks for
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const float c = fminf(fmaxf(v, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, 0.0f, 0, false) & 0xffu;
}

// four codes packed low byte first
__device__ __forceinline__ uint32_t e4m3_encode4(float v0, float v1, float v2, float v3) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(v0, -448.0f), 448.0f), fminf(fmaxf(v1, -448.0f), 448.0f),
                                                 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(v2, -448.0f), 448.0f),
                                                   fminf(fmaxf(v3, -448.0f), 448.0f), lo, true);
}

// shared exponent of a 32-block with maximum magnitude amax: floor(log2 amax) - 8,
// clamped to the E8M0 range; an all-zero block gets -127 (scale byte 0)
__device__ __forceinline__ int mx_shared_exp(float amax) {
  if (!(amax > 0.0f)) return -127;
  const int f = (int)((__float_as_uint(amax) >> 23) & 0xffu);  // subnormal: 0, clamps to -127 below
  const int e = (f == 255 ? 255 : f - 127) - 8;
  return max(-127, min(127, e));
}

// one thread per 32-element block of a bf16 row-major [rows][K] matrix
// four lanes per 32-element block, eight elements each: a wavefront's loads
// cover 1 KiB of contiguous activations; the block's maximum meets over the
// quad by two DPP steps (a maximum does not depend on the order)
__global__ __launch_bounds__(256) void quant_mxfp8_kernel(const uint16_t* __restrict__ x, long nblk,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const long i8 = (long)blockIdx.x * 256 + threadIdx.x;  // this lane's 8 elements
  const long b = i8 >> 2;
  if (b >= nblk) return;  // whole quads only: a quad shares b
  const uint4 q = *(const uint4*)(x + i8 * 8);
  const uint32_t d[4] = {q.x, q.y, q.z, q.w};
  float v[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = bf16_lo(d[j]);
    v[2 * j + 1] = bf16_hi(d[j]);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, dpp_f32<dpp::kQuadXor1>(amax));
  amax = fmaxf(amax, dpp_f32<dpp::kQuadXor2>(amax));
  const int sh = mx_shared_exp(amax);
  const uint32_t o0 = e4m3_encode4(ldexpf(v[0], -sh), ldexpf(v[1], -sh), ldexpf(v[2], -sh), ldexpf(v[3], -sh));
  const uint32_t o1 = e4m3_encode4(ldexpf(v[4], -sh), ldexpf(v[5], -sh), ldexpf(v[6], -sh), ldexpf(v[7], -sh));
  *(uint2*)(codes + i8 * 8) = make_uint2(o0, o1);
  if ((i8 & 3) == 0) scales[b] = (uint8_t)(sh + 127);
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
  int32_t* items;       // [0] = number of M tiles, then (key, start, rows) per tile
  // intermediate and output
  uint8_t* hq;          // [P][I] E4M3, grouped order
  uint8_t* hs;          // [P][I/32]
  uint16_t* y;          // [P][H] bf16, pair order
  // decode batches (bf16 activations on bf16 MFMA)
  const uint16_t* xb;   // [T][H] bf16
  uint16_t* hb;         // [P][I] bf16, grouped order
  float* yf;            // [P][H] fp32, pair order (when non-null, instead of y)
};

// key of pair p = (token p / K1, rank p % K1): the slot id, E for the shared
// expert, -1 for an id out of range (its output row is zeroed: it contributes
// nothing)
__device__ __forceinline__ void pair_key(const PrefillArgs& a, int p) {
  const int t = p / a.K1, r = p % a.K1;
  int key;
  if (r == a.k) {
    key = a.E;
  } else {
    const int e = a.ids[(size_t)t * a.k + r];
    key = (e >= 0 && e < a.E) ? e : -1;
  }
  a.keys[p] = key;
  if (key < 0) {
    uint4* yrow = a.yf ? (uint4*)(a.yf + (size_t)p * a.H) : (uint4*)(a.y + (size_t)p * a.H);
    const int n16 = a.yf ? a.H / 4 : a.H / 8;
    for (int j = 0; j < n16; ++j) yrow[j] = make_uint4(0u, 0u, 0u, 0u);
  }
}

__global__ __launch_bounds__(256) void prefill_keys_kernel(PrefillArgs a) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p < a.T * a.K1) pair_key(a, p);
}

// items[0] = number of M tiles, then (key, start, rows) per tile, start being
// the tile's first position in the grouped order.  A key with c
// rows gets ceil(c / MT) tiles of equal size rounded up to whole 32-row
// blocks (the last one takes the rest), so e.g. 140 rows run as one tile of
// the prefill GEMM (MT 192).
template <int MT>
__device__ __forceinline__ void items_body(const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
                                           int nkeys, int32_t* __restrict__ items) {
  const int lane = threadIdx.x & 63;
  int n = 0;
  // keys in the order nkeys-1, 0, 1, ..., nkeys-2: the shared expert's key
  // (the last, and the largest group) first, so that its tiles, the heaviest
  // items, are not the ones left for the last round of workgroups
  for (int base = 0; base < nkeys; base += 64) {
    const int kk = base + lane;
    const int key = kk == 0 ? nkeys - 1 : kk - 1;
    const int c = kk < nkeys ? counts[key] : 0;
    const int o = kk < nkeys ? offsets[key] : 0;
    const int tiles = (c + MT - 1) / MT;
    int incl = tiles;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    const int first = n + incl - tiles;
    const int sz = tiles ? ((c + tiles - 1) / tiles + 31) / 32 * 32 : 0;
    for (int i = 0; i < tiles; ++i) {
      items[1 + 3 * (first + i)] = key;
      items[2 + 3 * (first + i)] = o + i * sz;
      items[3 + 3 * (first + i)] = min(sz, c - i * sz);
    }
    n += __shfl(incl, 63, 64);
  }
  if (lane == 0) items[0] = n;
}

template <int MT>
__global__ __launch_bounds__(64) void prefill_items_kernel(const int32_t* __restrict__ counts,
                                                           const int32_t* __restrict__ offsets, int nkeys,
                                                           int32_t* __restrict__ items) {
  items_body<MT>(counts, offsets, nkeys, items);
}

// The whole plan of a decode batch's grouped GEMM in one launch of one
// workgroup: the pairs' keys, their stable grouping (counts, offsets, perm),
// then the M tiles.  The barriers order each step's global writes before the
// next step's reads within the workgroup; wavefront 0 writes counts and
// offsets in the grouping and reads them, lane for lane, for the tiles.  (A
// prefill's tens of thousands of pairs group faster with the keys spread over
// many workgroups, so prefill keeps three launches.)
template <int MT>
__global__ __launch_bounds__(kGroupThreads) void plan_kernel(PrefillArgs a, int W) {
  extern __shared__ int lds[];
  const int P = a.T * a.K1, nkeys = a.E + 1;
  for (int p = threadIdx.x; p < P; p += kGroupThreads) pair_key(a, p);
  __syncthreads();
  group_body(a.keys, P, nkeys, W, a.counts, a.offsets, a.perm, lds);
  __syncthreads();
  if (threadIdx.x < 64) items_body<MT>(a.counts, a.offsets, nkeys, a.items);
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
  // rows 2j and 2j+1 of 16 lanes swap: p[0] holds the even row's value, p[1] the odd row's
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// ------------------------------------------------------------- grouped GEMM
//
// One template for both products.  An item is (M tile = up to 192 grouped
// rows of one expert, 256 weight rows): for gate/up, 128 rows of w1 and the
// same 128 rows of w3 (128 columns of h); for down, 256 rows of w2.  The
// workgroup's 4 wavefronts (one per SIMD) split the item's 32x32 output
// blocks: wavefront w takes the M blocks of parity w / 2 (blocks w/2, w/2 + 2,
// w/2 + 4; blocks past the tile's rows are skipped) and the column blocks of
// half w % 2 — for gate/up the gate blocks and the up blocks of the same 64
// columns, so SwiGLU pairs them in registers.
//
// K advances kKS at a time.  Every thread loads its share of a stage (16-byte
// pieces of the activation and weight rows, and the stage's scale bytes of
// one activation row and one weight row) into registers kDepth stages ahead
// and stores it to one of two LDS buffers one stage ahead of the MFMAs.
// Loads are unconditional (row indices are clamped to the tile), so the
// compiler's in-order wait counts make each store wait for its own stage
// only and kDepth stages stay in flight.  LDS rows are padded by 16 bytes so
// the 32 rows a fragment read touches fall in different banks.  Items run N
// tile innermost and each XCD takes a contiguous range of them, so the N
// tiles of one M tile share its activation rows in one L2 while the
// expert's weights stream from HBM once per M tile.

#ifndef MOE_PF_KS
#define MOE_PF_KS 128
#endif
#ifndef MOE_PF_BNT
#define MOE_PF_BNT 0
#endif
constexpr int kKS = MOE_PF_KS;           // K per stage (64 or 128)
#ifndef MOE_PF_PADA
#define MOE_PF_PADA 16
#endif
#ifndef MOE_PF_PADB
#define MOE_PF_PADB 16
#endif
constexpr int kArow = kKS + MOE_PF_PADA;      // padded bytes per activation row in LDS
constexpr int kBrow = kKS / 2 + MOE_PF_PADB;  // padded bytes per weight row in LDS
constexpr int kNB = 16 / kWaves;              // column blocks per wavefront (the M blocks split in 2)
constexpr int kThreads = kWaves * 64;
constexpr int kCA = kKS / 16;            // 16-byte pieces per activation row and stage
constexpr int kCB = kKS / 32;            // 16-byte pieces per weight row and stage
constexpr int kPiecesA = kMT * kCA / kThreads;  // activation pieces per thread and stage
constexpr int kPiecesB = kNR * kCB / kThreads;  // weight pieces per thread and stage
static_assert(kPiecesA * kThreads == kMT * kCA && kPiecesB * kThreads == kNR * kCB,
              "stage pieces must divide evenly over the workgroup");
static_assert(kKS == 64 || kKS == 128, "a stage is one or two MFMA K steps");
static_assert(kThreads >= kMT && kThreads >= kNR, "one scale entry per thread covers every row");
// the stage's scale bytes of one row: one per 32 elements of K
typedef std::conditional<kKS == 64, uint16_t, uint32_t>::type StageScales;

struct alignas(16) GemmSmem {
  uint8_t a[2][kMT * kArow];
  uint8_t b[2][kNR * kBrow];
  StageScales as[2][kThreads];  // entry i: the stage's scale bytes of activation row i (i < kMT used)
  StageScales bs[2][kThreads];  // entry i: the stage's scale bytes of weight row i % kNR
  int32_t pm[kMT];              // down: the (token, rank) pair of each tile row
};

// The epilogue turns a wavefront's 32 x 32 accumulator block around through
// LDS: the MFMA leaves lane (c, h) with rows 8(e/4) + 4h + e%4 of column c;
// afterwards lane l holds 16 consecutive columns (16 (l & 1) ..) of row l / 2,
// so an MX block's maximum is one lane-pair exchange and a row leaves in
// 16-byte stores.  Each wavefront uses its own kTLd-padded tile.
constexpr int kTLd = 36;  // floats per row of the transpose tile
static_assert((size_t)kWaves * 32 * kTLd * 4 <= sizeof(((GemmSmem*)nullptr)->a), "transpose tiles fit the A stages");

__device__ __forceinline__ void acc_transpose(float* tw, const float (&v)[16], int c, int h, int lane, float (&out)[16]) {
#pragma unroll
  for (int e = 0; e < 16; ++e) tw[(8 * (e / 4) + 4 * h + (e % 4)) * kTLd + c] = v[e];
  __builtin_amdgcn_wave_barrier();
  const u32x4_t* src = (const u32x4_t*)(tw + (lane >> 1) * kTLd + 16 * (lane & 1));
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const u32x4_t t = src[k];
    out[4 * k] = __uint_as_float(t.x), out[4 * k + 1] = __uint_as_float(t.y);
    out[4 * k + 2] = __uint_as_float(t.z), out[4 * k + 3] = __uint_as_float(t.w);
  }
  __builtin_amdgcn_wave_barrier();  // the reads are done before the tile is written again
}

// native vectors, not uint4: a struct copy of a register array goes through scratch
struct StageRegs {
  u32x4_t a[kPiecesA];
  u32x4_t b[kPiecesB];
  StageScales as, bs;
};

// this thread's load offsets at K = 0 for one item (32-bit, from wave-uniform bases)
struct LoadOffs {
  uint32_t a[kPiecesA];  // piece p = tid + j*kThreads: activation row p/kCA (clamped), 16 bytes at 16*(p%kCA)
  uint32_t b[kPiecesB];  // piece p = tid + j*kThreads: weight row p/kCB, 16 bytes at 16*(p%kCB)
  uint32_t as;           // scale row of activation row min(tid, rows-1)
  uint32_t bs;           // scale row of weight row tid % kNR
};

__device__ __forceinline__ void stage_load(StageRegs& r, const LoadOffs& o, const uint8_t* abase,
                                           const uint8_t* asbase, const uint8_t* rec, int k0) {
#pragma unroll
  for (int j = 0; j < kPiecesA; ++j) r.a[j] = *(const u32x4_t*)(abase + (o.a[j] + k0));
#pragma unroll
  for (int j = 0; j < kPiecesB; ++j) {
#if MOE_PF_BNT
    r.b[j] = __builtin_nontemporal_load((const u32x4_t*)(rec + (o.b[j] + k0 / 2)));
#else
    r.b[j] = *(const u32x4_t*)(rec + (o.b[j] + k0 / 2));
#endif
  }
  r.as = *(const StageScales*)(asbase + (o.as + k0 / 32));
  r.bs = *(const StageScales*)(rec + (o.bs + k0 / 32));
}

__device__ __forceinline__ void stage_store(GemmSmem& sm, int buf, const StageRegs& r, int tid) {
#pragma unroll
  for (int j = 0; j < kPiecesA; ++j) {
    const int p = tid + j * kThreads;
    *(u32x4_t*)(sm.a[buf] + (p / kCA) * kArow + 16 * (p % kCA)) = r.a[j];
  }
#pragma unroll
  for (int j = 0; j < kPiecesB; ++j) {
    const int p = tid + j * kThreads;
    *(u32x4_t*)(sm.b[buf] + (p / kCB) * kBrow + 16 * (p % kCB)) = r.b[j];
  }
  sm.as[buf][tid] = r.as;
  sm.bs[buf][tid] = r.bs;
}

struct ItemCtx {
  LoadOffs O;
  const uint8_t *abase, *asbase, *rec;
  int tid, c, h, mp, nh, nstage, rows, start, nt;
};

// LDS weight-tile block of column block j (0..kNB-1) of the wavefront's
// column group nh: for gate/up the first kNB/2 are gate blocks and the rest
// the up blocks of the same columns (gate block b pairs with up block 4 + b);
// for down, kNB consecutive blocks
template <int NMAT>
__device__ __forceinline__ int col_block(int nh, int j) {
  constexpr int half = kNB / 2;
  return NMAT == 2 ? (j < half ? half * nh + j : 4 + half * nh + (j - half)) : kNB * nh + j;
}

// One item for a wavefront with NL live M blocks (mp, mp + 2, ...).  Every
// wavefront runs the same loads, stores and barriers whatever its NL; the
// live count only selects how many MFMA rows it computes, so the accumulators
// stay in fixed registers.
template <int NMAT, int NL>
__device__ __forceinline__ void gemm_item(GemmSmem& sm, const PrefillArgs& a, const ItemCtx& x) {
  const int tid = x.tid, c = x.c, h = x.h, nstage = x.nstage;
  v16f acc[NL > 0 ? NL : 1][kNB];
#pragma unroll
  for (int i = 0; i < NL; ++i)
#pragma unroll
    for (int j = 0; j < kNB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // R[j] holds stage j mod kDepth.  nstage is a multiple of kDepth (checked
  // at launch), so the unrolled body needs no guards: at the tail the loads are
  // clamped to the last stage and the last store fills a buffer nobody reads.
  StageRegs R[kDepth];
#pragma unroll
  for (int d = 0; d < kDepth; ++d) stage_load(R[d], x.O, x.abase, x.asbase, x.rec, d * kKS);
  __syncthreads();  // the previous item's last stage reads and epilogue are done
  stage_store(sm, 0, R[0], tid);
  if (NMAT == 1 && tid < kMT) sm.pm[tid] = a.perm[x.start + min(tid, x.rows - 1)];
  stage_load(R[0], x.O, x.abase, x.asbase, x.rec, min(kDepth, nstage - 1) * kKS);
  __syncthreads();

  for (int s0 = 0; s0 < nstage; s0 += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int s = s0 + d;
      const int buf = (kDepth % 2 == 0) ? (d & 1) : (s & 1);
      if (NL > 0) {
#pragma unroll
        for (int kc = 0; kc < kKS / 64; ++kc) {
          v8i bv[kNB];
          int sb[kNB];
#pragma unroll
          for (int j = 0; j < kNB; ++j) {
            const int r = col_block<NMAT>(x.nh, j) * 32 + c;
            const u32x4_t q = *(const u32x4_t*)(sm.b[buf] + r * kBrow + kc * 32 + 16 * h);
            bv[j][0] = (int)q.x, bv[j][1] = (int)q.y, bv[j][2] = (int)q.z, bv[j][3] = (int)q.w;
            bv[j][4] = 0, bv[j][5] = 0, bv[j][6] = 0, bv[j][7] = 0;
            sb[j] = (int)(((uint32_t)sm.bs[buf][r] >> (8 * (2 * kc + h))) & 0xffu);
          }
#pragma unroll
          for (int i = 0; i < NL; ++i) {
            const int r = 32 * (x.mp + 2 * i) + c;
            const uint8_t* ar = sm.a[buf] + r * kArow + kc * 64;
            const u32x4_t lo = *(const u32x4_t*)(ar + 16 * h);
            const u32x4_t hi = *(const u32x4_t*)(ar + 32 + 16 * h);
            v8i av;
            av[0] = (int)lo.x, av[1] = (int)lo.y, av[2] = (int)lo.z, av[3] = (int)lo.w;
            av[4] = (int)hi.x, av[5] = (int)hi.y, av[6] = (int)hi.z, av[7] = (int)hi.w;
            const int sa = (int)(((uint32_t)sm.as[buf][r] >> (8 * (2 * kc + h))) & 0xffu);
#pragma unroll
            for (int j = 0; j < kNB; ++j) acc[i][j] = mfma_fp8_fp4(av, bv[j], acc[i][j], sa, sb[j]);
          }
        }
      }
      stage_store(sm, buf ^ 1, R[(d + 1) % kDepth], tid);
      stage_load(R[(d + 1) % kDepth], x.O, x.abase, x.asbase, x.rec, min(s + 1 + kDepth, nstage - 1) * kKS);
      __syncthreads();
    }
  }

  // the epilogue's lane indices pass through an empty asm so the compiler
  // cannot hoist its address arithmetic into registers held across the loop;
  // the stage buffers are free here (the loop ended at a barrier) and hold the
  // transpose tiles
  int ce = c, he = h;
  asm volatile("" : "+v"(ce), "+v"(he));
  const int lane = 32 * he + ce, half = lane & 1;
  float* tw = (float*)sm.a[0] + (tid >> 6) * (32 * kTLd);
  const int H = a.H, I = a.I;
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int rb = 32 * (x.mp + 2 * i);
    const int r = rb + (lane >> 1);  // the row this lane holds after the transpose
    if (NMAT == 2) {
      // SwiGLU, MXFP8 requantisation along I (a 32-column block is one lane pair's row)
#pragma unroll
      for (int q = 0; q < kNB / 2; ++q) {
        const int col0 = x.nt * (kNR / 2) + 32 * col_block<2>(x.nh, q);
        float hv[16], v[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float g = acc[i][q][e], u = acc[i][kNB / 2 + q][e];
          // silu(g) * u with the hardware exp2 and reciprocal (the result is
          // requantised to 8 bits next)
          hv[e] = g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504f * g)) * u;
        }
        acc_transpose(tw, hv, ce, he, lane, v);
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < 16; ++k) amax = fmaxf(amax, fabsf(v[k]));
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        const int sh = mx_shared_exp(amax);
        if (r < x.rows) {
          const size_t pos = (size_t)(x.start + r);
          uint32_t w[4];
#pragma unroll
          for (int k = 0; k < 4; ++k)
            w[k] = e4m3_encode4(__builtin_amdgcn_ldexpf(v[4 * k], -sh), __builtin_amdgcn_ldexpf(v[4 * k + 1], -sh),
                                __builtin_amdgcn_ldexpf(v[4 * k + 2], -sh), __builtin_amdgcn_ldexpf(v[4 * k + 3], -sh));
          *(u32x4_t*)(a.hq + pos * I + col0 + 16 * half) = u32x4_t{w[0], w[1], w[2], w[3]};
          if (half == 0) a.hs[pos * (I / 32) + col0 / 32] = (uint8_t)(sh + 127);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < kNB; ++j) {
        float yv[16], v[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) yv[e] = acc[i][j][e];
        acc_transpose(tw, yv, ce, he, lane, v);
        if (r < x.rows) {
          const size_t pair = (size_t)sm.pm[r];
          uint32_t w[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) w[k] = (uint32_t)f32_to_bf16(v[2 * k]) | ((uint32_t)f32_to_bf16(v[2 * k + 1]) << 16);
          u32x4_t* dst = (u32x4_t*)(a.y + pair * H + (size_t)x.nt * kNR + col_block<1>(x.nh, j) * 32 + 16 * half);
          dst[0] = u32x4_t{w[0], w[1], w[2], w[3]};
          dst[1] = u32x4_t{w[4], w[5], w[6], w[7]};
        }
      }
    }
  }
}

// NMAT = 2: gate/up (w1, w3 of the expert, K = H), SwiGLU + MXFP8 epilogue into hq/hs.
// NMAT = 1: down (w2, K = I), bf16 epilogue into y at each row's (token, rank) pair.
template <int NMAT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(PrefillArgs a) {
  __shared__ GemmSmem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, h = lane >> 5;
  const int mp = wave / (kWaves / 2), nh = wave % (kWaves / 2);
  const int H = a.H, I = a.I;
  const int K = NMAT == 2 ? H : I;                      // reduction length
  const int ncol = NMAT == 2 ? I / (kNR / 2) : H / kNR; // N tiles per M tile
  const int nitems = a.items[0] * ncol;
  const int nstage = K / kKS;
  const RecordLayout L = record_layout(H, I, 4);
  const uint32_t wrowb = (uint32_t)K / 2, wrows = (uint32_t)K / 32;

  // a workgroup takes `pair` N tiles of one M tile in a row: the second
  // reuses the first's activation offsets (the tile entry and its rows'
  // token ids, two dependent trips); consecutive pairs still go to
  // neighbouring workgroups of one XCD
  const int pair = (ncol % 2 == 0) ? 2 : 1;
  const int nchunks = nitems / pair;
  for (int chunk = virtual_block(); chunk < nchunks; chunk += gridDim.x) {
    const int mi = chunk / (ncol / pair), nt0 = (chunk - mi * (ncol / pair)) * pair;
    const int key = a.items[1 + 3 * mi], start = a.items[2 + 3 * mi], rows = a.items[3 + 3 * mi];  // first grouped position of the tile
    const uint8_t* rec = key_record(a, key);
    // activation rows: x (gathered by token) for gate/up, h (grouped) for down
    const uint8_t* abase = NMAT == 2 ? a.xq : a.hq;
    const uint8_t* asbase = NMAT == 2 ? a.xs : a.hs;
    auto act_row = [&](int r) -> uint32_t {  // row index into abase / asbase
      r = min(r, rows - 1);
      return NMAT == 2 ? (uint32_t)(a.perm[start + r] / a.K1) : (uint32_t)(start + r);
    };
    // weight rows of N tile nt: offsets of codes or scales inside the record
    auto weight_row = [&](int nt, int wr, bool scales) -> uint32_t {
      uint32_t n, off;
      if (NMAT == 2) {
        const int mat = wr / (kNR / 2);
        n = (uint32_t)(nt * (kNR / 2) + wr % (kNR / 2));
        off = (uint32_t)(scales ? (mat == 0 ? L.w1s : L.w3s) : (mat == 0 ? L.w1c : L.w3c));
      } else {
        n = (uint32_t)(nt * kNR + wr);
        off = (uint32_t)(scales ? L.w2s : L.w2c);
      }
      return off + n * (scales ? wrows : wrowb);
    };
    ItemCtx x;
#pragma unroll
    for (int j = 0; j < kPiecesA; ++j) {
      const int p = tid + j * kThreads;
      x.O.a[j] = act_row(p / kCA) * (uint32_t)K + 16u * (p % kCA);
    }
    x.O.as = act_row(tid) * (uint32_t)(K / 32);
    x.abase = abase, x.asbase = asbase, x.rec = rec;
    x.tid = tid, x.c = c, x.h = h, x.mp = mp, x.nh = nh, x.nstage = nstage;
    x.rows = rows, x.start = start;
    // the wavefront's live M blocks: mp, mp + 2, mp + 4 while below the tile's rows
    const int nl = max(0, min(kMB / 2, (rows - 32 * mp + 63) / 64));
    for (int u = 0; u < pair; ++u) {
      const int nt = nt0 + u;
#pragma unroll
      for (int j = 0; j < kPiecesB; ++j) {
        const int p = tid + j * kThreads;
        x.O.b[j] = weight_row(nt, p / kCB, false) + 16u * (p % kCB);
      }
      x.O.bs = weight_row(nt, tid % kNR, true);
      x.nt = nt;
      switch (nl) {
        case 0: gemm_item<NMAT, 0>(sm, a, x); break;
        case 1: gemm_item<NMAT, 1>(sm, a, x); break;
        case 2: gemm_item<NMAT, 2>(sm, a, x); break;
        default: gemm_item<NMAT, 3>(sm, a, x); break;
      }
    }
  }
}

// ------------------------------------------------ decode-batch grouped GEMM
//
// A decode batch of tens of tokens gives each selected expert a handful of
// rows: too few for FP8 activations to pay off, and per-token GEMVs would
// convert the same weights once per token.  Here each 16-byte FP4 piece is
// dequantised once per item to bf16 by the scaled FP4 converts (exact: the
// block scale is a power of two) and multiplied on v_mfma_f32_32x32x16_bf16
// against the bf16 activations, so the products are exact as on the batch-1
// path.  Items are (M tile of up to 64 grouped rows of one record, 256 weight
// rows); their K stages go from HBM straight into a ring of LDS stages (see
// dgemm_item below).  A tile of two M blocks
// gives wavefront w M block w / 2 and column half w % 2 (for gate/up, 64 gate
// and the same 64 up columns); a tile of one M block (most of a decode
// batch's groups) splits the columns four ways instead, so no wavefront idles.  A K step of the MFMA takes, per lane, 8 consecutive elements of
// the 32 its FP4 piece covers; the activation fragment is read at the same K.

constexpr int kDMT = 64;                      // grouped rows per item at most
constexpr int kDKS = 128;                     // K per stage
constexpr int kDThreads = 256;                // 4 wavefronts
constexpr int kDCA = 2 * kDKS / 16;           // 16-byte pieces per activation row and stage
constexpr int kDCB = kDKS / 32;               // 16-byte pieces per weight row and stage
constexpr int kDPiecesA = kDMT * kDCA / kDThreads;
constexpr int kDPiecesB = kNR * kDCB / kDThreads;
static_assert(kDPiecesA * kDThreads == kDMT * kDCA && kDPiecesB * kDThreads == kNR * kDCB,
              "stage pieces must divide evenly over the workgroup");
#ifndef MOE_DG_PER_CU
#define MOE_DG_PER_CU 1  // workgroups per CU (two fit, but measured slower)
#endif

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// global offsets of what this thread loads into stage slot p = tid + j*kDThreads
struct DLoadOffs {
  uint32_t a[kDPiecesA];  // activation row r = p/kDCA (clamped), piece (p % kDCA) ^ (r % 16)
  uint32_t b[kDPiecesB];  // weight row r = p/kDCB, piece (p % kDCB) ^ (r / 4 % 4)
  uint32_t bs;            // scale row of weight row tid
};

// LDS weight-tile block of the wavefront's column block j (0..NBW-1) in its
// column share cs.  NBW = 4 (a tile of two M blocks; cs = column half):
// gate/up: gate blocks 2cs, 2cs+1 then the up blocks 4+2cs, 5+2cs; down:
// blocks 4cs .. 4cs+3.  NBW = 2 (a tile of one M block, the columns split four
// ways; cs = wavefront): gate/up: gate block cs and up block 4+cs; down: 2cs, 2cs+1.
template <int NMAT, int NBW>
__device__ __forceinline__ int dcol_block(int cs, int j) {
  constexpr int half = NBW / 2;
  return NMAT == 2 ? (j < half ? half * cs + j : 4 + half * cs + (j - half)) : NBW * cs + j;
}

struct DItemCtx {
  DLoadOffs O;
  const uint8_t *abase, *rec;
  int tid, c, h, wave, mp, nh, nstage, rows, start, nt;
};

// Each stage's activation, weight and scale pieces go from HBM to LDS by
// global_load_lds (no register staging) into a ring of kDRing stages,
// kDRing - 1 stages ahead of the one being multiplied.  A wavefront waits for
// its own loads of a stage by vmcnt, and one barrier per stage publishes
// everyone's.  Lane l of a direct load writes 16-byte LDS slot base + l, so
// the lane decides which global piece lands in which slot: the pieces are
// XOR-swizzled (activation row r: piece q at slot 16 r + (q ^ (r % 16));
// weight row r: piece q at slot 4 r + (q ^ (r / 4 % 4))) so that the 32 rows
// one MFMA operand reads fall on distinct banks, two lanes per bank.
#ifndef MOE_DG_RING
#define MOE_DG_RING 3  // 2 and 4 measured slower
#endif
constexpr int kDRing = MOE_DG_RING;
constexpr int kDStageA = kDMT * 2 * kDKS;   // bytes of a stage's activation tile
constexpr int kDStageB = kNR * kDKS / 2;    // bytes of a stage's weight tile
static_assert(kDRing >= 2 && kDRing <= 6, "ring of 2..6 stages");

struct alignas(16) DGemmSmem {
  uint8_t a[kDRing][kDStageA];
  uint8_t b[kDRing][kDStageB];
  uint32_t bs[kDRing][kDThreads];  // entry i: the stage's 4 scale bytes of weight row i
  int32_t pm[kDMT];
};

typedef __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// this thread's loads of stage k0 into ring slot buf: pieces j < NA of the
// activation tile (NA = 2: its first 32 rows only) and every piece of the
// weight tile (slot tid + 256 j, offsets swizzled by the caller), and the
// scale word of weight row tid
template <int NA>
__device__ __forceinline__ void dstage_issue_lds(DGemmSmem& sm, int buf, const DLoadOffs& o, const uint8_t* abase,
                                                 const uint8_t* rec, int k0, int wave) {
#pragma unroll
  for (int j = 0; j < NA; ++j)
    __builtin_amdgcn_global_load_lds((gptr_t)(abase + (o.a[j] + 2 * k0)),
                                     (lptr_t)(sm.a[buf] + (j * kDThreads + wave * 64) * 16), 16, 0, 0);
#pragma unroll
  for (int j = 0; j < kDPiecesB; ++j)
    __builtin_amdgcn_global_load_lds((gptr_t)(rec + (o.b[j] + k0 / 2)),
                                     (lptr_t)(sm.b[buf] + (j * kDThreads + wave * 64) * 16), 16, 0, 0);
  __builtin_amdgcn_global_load_lds((gptr_t)(rec + (o.bs + k0 / 32)), (lptr_t)(&sm.bs[buf][wave * 64]), 4, 0, 0);
}

// NBW column blocks per wavefront (4: M block mp of two, 2: the only M block),
// LIVE false: the wavefront's M block is past the tile's rows
template <int NMAT, int NBW, bool LIVE>
__device__ __forceinline__ void dgemm_item(DGemmSmem& sm, const PrefillArgs& a, const DItemCtx& x) {
  const int tid = x.tid, c = x.c, h = x.h, nstage = x.nstage;
  const int mb = NBW == 4 ? x.mp : 0;
  const int cs = NBW == 4 ? x.nh : x.wave;
  // a tile of one M block reads activation rows 0..31 only: half the pieces
  constexpr int NA = NBW == 4 ? kDPiecesA : kDPiecesA / 2;
  constexpr int kLoads = NA + kDPiecesB + 1;  // load instructions per stage and thread
  v16f acc[NBW];
#pragma unroll
  for (int j = 0; j < NBW; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;

  __syncthreads();  // the previous item's last stage reads and epilogue are done
  if (NMAT == 1 && tid < kDMT) sm.pm[tid] = a.perm[x.start + min(tid, x.rows - 1)];
  // stages 0 .. kDRing-2 (past the last stage: the last one again, never read)
#pragma unroll
  for (int d = 0; d < kDRing - 1; ++d) dstage_issue_lds<NA>(sm, d, x.O, x.abase, x.rec, min(d, nstage - 1) * kDKS, x.wave);

  const int arow = 32 * mb + c;
  for (int s = 0; s < nstage; ++s) {
    const int buf = s % kDRing;
    // this wavefront's loads of stage s are done when at most the later
    // kDRing-2 stages' loads are outstanding
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoads * (kDRing - 2)) : "memory");
    // everyone's stage s is in LDS and everyone is done with stage s-1: a bare
    // barrier (a fenced one would wait for every load in flight, the ring's
    // later stages included); the empty asm statements keep the compiler from
    // moving LDS accesses across it
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    dstage_issue_lds<NA>(sm, (s + kDRing - 1) % kDRing, x.O, x.abase, x.rec, min(s + kDRing - 1, nstage - 1) * kDKS,
                         x.wave);
    if (LIVE) {
#pragma unroll
      for (int kc = 0; kc < kDKS / 64; ++kc) {
        u32x4_t q[NBW];
        float sc[NBW];
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
          const int r = dcol_block<NMAT, NBW>(cs, j) * 32 + c;
          const int qq = (2 * kc + h) ^ ((r >> 2) & 3);
          q[j] = *(const u32x4_t*)(sm.b[buf] + (r * 4 + qq) * 16);
          sc[j] = e8m0_to_f32((sm.bs[buf][r] >> (8 * (2 * kc + h))) & 0xffu);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int qa = (kc * 8 + 4 * h + m) ^ (arow & 15);
          const v8bf av = *(const v8bf*)(sm.a[buf] + (arow * 16 + qa) * 16);
#pragma unroll
          for (int j = 0; j < NBW; ++j) {
            u32x4_t wv;
            wv.x = fp4x2_to_bf16x2_scaled<0>(q[j][m], sc[j]);
            wv.y = fp4x2_to_bf16x2_scaled<1>(q[j][m], sc[j]);
            wv.z = fp4x2_to_bf16x2_scaled<2>(q[j][m], sc[j]);
            wv.w = fp4x2_to_bf16x2_scaled<3>(q[j][m], sc[j]);
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(v8bf, wv), acc[j], 0, 0, 0);
          }
        }
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the ring's trailing loads land before the next item reuses it
  if (!LIVE) return;

  int ce = c, he = h;
  asm volatile("" : "+v"(ce), "+v"(he));
  const int H = a.H, I = a.I;
  const int rb = 32 * mb;
  if (NMAT == 2) {
#pragma unroll
    for (int q = 0; q < NBW / 2; ++q) {
      const int col = x.nt * (kNR / 2) + 32 * dcol_block<2, NBW>(cs, q) + ce;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = rb + 8 * (e / 4) + 4 * he + (e % 4);
        if (r < x.rows) {
          const float g = acc[q][e], u = acc[NBW / 2 + q][e];
          a.hb[(size_t)(x.start + r) * I + col] = f32_to_bf16(g / (1.0f + expf(-g)) * u);
        }
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = rb + 8 * (e / 4) + 4 * he + (e % 4);
      if (r < x.rows) {
        const size_t pair = (size_t)sm.pm[r];
#pragma unroll
        for (int j = 0; j < NBW; ++j)
          a.yf[pair * H + (size_t)x.nt * kNR + dcol_block<1, NBW>(cs, j) * 32 + ce] = acc[j][e];
      }
    }
  }
}

// NMAT = 2: gate/up (K = H) with SwiGLU into hb; NMAT = 1: down (K = I) into yf
template <int NMAT>
__global__ __launch_bounds__(kDThreads) void dgemm_kernel(PrefillArgs a) {
  __shared__ DGemmSmem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, h = lane >> 5;
  const int mp = wave >> 1, nh = wave & 1;
  const int H = a.H, I = a.I;
  const int K = NMAT == 2 ? H : I;
  const int ncol = NMAT == 2 ? I / (kNR / 2) : H / kNR;
  const int nitems = a.items[0] * ncol;
  const int nstage = K / kDKS;
  const RecordLayout L = record_layout(H, I, 4);
  const uint32_t wrowb = (uint32_t)K / 2, wrows = (uint32_t)K / 32;

  for (int item = virtual_block(); item < nitems; item += gridDim.x) {
    const int mi = item / ncol, nt = item - mi * ncol;
    const int key = a.items[1 + 3 * mi], start = a.items[2 + 3 * mi], rows = a.items[3 + 3 * mi];
    const uint8_t* rec = key_record(a, key);
    auto act_row = [&](int r) -> uint32_t {
      r = min(r, rows - 1);
      return NMAT == 2 ? (uint32_t)(a.perm[start + r] / a.K1) : (uint32_t)(start + r);
    };
    auto weight_row = [&](int wr, bool scales) -> uint32_t {
      uint32_t n, off;
      if (NMAT == 2) {
        const int mat = wr / (kNR / 2);
        n = (uint32_t)(nt * (kNR / 2) + wr % (kNR / 2));
        off = (uint32_t)(scales ? (mat == 0 ? L.w1s : L.w3s) : (mat == 0 ? L.w1c : L.w3c));
      } else {
        n = (uint32_t)(nt * kNR + wr);
        off = (uint32_t)(scales ? L.w2s : L.w2c);
      }
      return off + n * (scales ? wrows : wrowb);
    };
    DItemCtx x;
#pragma unroll
    for (int j = 0; j < kDPiecesA; ++j) {
      const int p = tid + j * kDThreads;
      const int r = p / kDCA, q = (p % kDCA) ^ (r & 15);  // slot p holds piece q
      x.O.a[j] = act_row(r) * (uint32_t)(2 * K) + 16u * q;
    }
#pragma unroll
    for (int j = 0; j < kDPiecesB; ++j) {
      const int p = tid + j * kDThreads;
      const int r = p / kDCB, q = (p % kDCB) ^ ((r >> 2) & 3);
      x.O.b[j] = weight_row(r, false) + 16u * q;
    }
    x.O.bs = weight_row(tid, true);
    x.abase = NMAT == 2 ? (const uint8_t*)a.xb : (const uint8_t*)a.hb;
    x.rec = rec;
    x.tid = tid, x.c = c, x.h = h, x.wave = wave, x.mp = mp, x.nh = nh, x.nstage = nstage;
    x.rows = rows, x.start = start, x.nt = nt;
    if (rows <= 32)  // one M block: every wavefront takes a quarter of the columns
      dgemm_item<NMAT, 2, true>(sm, a, x);
    else if (32 * mp < rows)
      dgemm_item<NMAT, 4, true>(sm, a, x);
    else
      dgemm_item<NMAT, 4, false>(sm, a, x);
  }
}

// out[t] = sum_{r<k} w[t][r] * y[t][r] (+ y[t][k]), y bf16, rank order, one
// rounding.  NK1 > 0: at most NK1 batch slots, every rank's load issued
// before the first is used (a thread's loads would otherwise go out one
// rank at a time); NK1 = 0: any K1.
template <int NK1>
__global__ __launch_bounds__(256) void combine_bf16y_kernel(const uint16_t* __restrict__ y, const float* __restrict__ w,
                                                            int T, int k, int K1, int H, uint16_t* __restrict__ out) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const int oct = H / 8;
  if (idx >= (long)T * oct) return;
  const int t = (int)(idx / oct), j = (int)(idx % oct) * 8;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  auto add = [&](const uint4 v, float wr) {
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] = fmaf(wr, bf16_lo(d[q]), acc[2 * q]);
      acc[2 * q + 1] = fmaf(wr, bf16_hi(d[q]), acc[2 * q + 1]);
    }
  };
  if constexpr (NK1 > 0) {
    uint4 v[NK1];
    float wr[NK1];
#pragma unroll
    for (int r = 0; r < NK1; ++r) {  // unconditional (clamped) loads: a fixed count in flight
      const int rr = min(r, K1 - 1);
      v[r] = ld_stream16((const uint8_t*)(y + ((size_t)t * K1 + rr) * H + j));
      wr[r] = w[(size_t)t * k + min(r, k - 1)];
    }
#pragma unroll
    for (int r = 0; r < NK1; ++r)
      if (r < K1) add(v[r], r < k ? wr[r] : 1.0f);
  } else {
    for (int r = 0; r < K1; ++r)
      add(*(const uint4*)(y + ((size_t)t * K1 + r) * H + j), r < k ? w[(size_t)t * k + r] : 1.0f);
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
  w.items = o; o += align256((1 + 3 * (P / kMT + kMaxKeys + 1)) * 4);
  w.hq = o; o += align256(P * I);
  w.hs = o; o += align256(P * I / 32);
  w.y = o; o += align256(P * H * 2);
  w.total = o;
  return w;
}

}  // namespace

size_t group_wide_scratch_ints(int n, int nkeys);
moe_status launch_group_wide(const int32_t* keys, int n, int nkeys, int32_t* counts, int32_t* offsets,
                             int32_t* perm, int32_t* scratch, hipStream_t s);

size_t prefill_workspace_bytes(int H, int I, int T, int k, int has_shared) {
  return prefill_ws_layout(H, I, T, k + (has_shared ? 1 : 0)).total;
}

moe_status launch_quant_mxfp8(const void* x, long rows, int K, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const long nblk = rows * (K / 32);
  if (nblk == 0) return MOE_OK;
  launch(MOE_PROF_QUANT, quant_mxfp8_kernel, dim3((unsigned)((4 * nblk + 255) / 256)), dim3(256), 0, s,
         (const uint16_t*)x, nblk, codes, scales);
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
  a.xb = nullptr;
  a.hb = nullptr;
  a.yf = nullptr;

  if ((H / kKS) % kDepth != 0 || (I / kKS) % kDepth != 0)
    return fail(MOE_ESHAPE, "moe_prefill_forward: H=%d and I=%d must be multiples of %d", H, I, kKS * kDepth);
  moe_status st = launch_quant_mxfp8(x, T, H, (uint8_t*)a.xq, (uint8_t*)a.xs, s);
  if (st != MOE_OK) return st;
  {
    launch(MOE_PROF_PLAN, prefill_keys_kernel, dim3((P + 255) / 256), dim3(256), 0, s, a);
    MOE_LAUNCH_CHECK();
  }
  // tens of thousands of pairs group over many workgroups; h's region is free
  // until the gate/up GEMM and holds their per-chunk histograms
  if (group_wide_scratch_ints(P, E + 1) * 4 > lay.hs - lay.hq)
    return fail(MOE_EINVAL, "moe_prefill_forward: grouping scratch exceeds the h region");
  st = launch_group_wide(a.keys, P, E + 1, a.counts, a.offsets, a.perm, (int32_t*)(ws + lay.hq), s);
  if (st != MOE_OK) return st;
  {
    launch(MOE_PROF_PLAN, prefill_items_kernel<kMT>, dim3(1), dim3(64), 0, s, a.counts, a.offsets, E + 1, a.items);
    MOE_LAUNCH_CHECK();
  }
  // persistent grids, one workgroup per CU (each wavefront holds a SIMD's 512
  // registers), a multiple of 8 (one share per XCD)
  const long max_items_m = (long)P / kMT + E + 1;
  const int grid_gu = (int)std::min<long>(max_items_m * (I / (kNR / 2)), 256L) / 8 * 8;
  const int grid_dn = (int)std::min<long>(max_items_m * (H / kNR), 256L) / 8 * 8;
  {
    launch(MOE_PROF_GEMM_GATEUP, gemm_kernel<2>, dim3(std::max(grid_gu, 8)), dim3(kThreads), 0, s, a);
    MOE_LAUNCH_CHECK();
  }
  {
    launch(MOE_PROF_GEMM_DOWN, gemm_kernel<1>, dim3(std::max(grid_dn, 8)), dim3(kThreads), 0, s, a);
    MOE_LAUNCH_CHECK();
  }
  {
    const long n = (long)T * (H / 8);
    const dim3 grid((unsigned)((n + 255) / 256));
    if (K1 <= 5)
      launch(MOE_PROF_COMBINE, combine_bf16y_kernel<5>, grid, dim3(256), 0, s, a.y, w, T, k, K1, H, (uint16_t*)out);
    else if (K1 <= 9)
      launch(MOE_PROF_COMBINE, combine_bf16y_kernel<9>, grid, dim3(256), 0, s, a.y, w, T, k, K1, H, (uint16_t*)out);
    else if (K1 <= 17)
      launch(MOE_PROF_COMBINE, combine_bf16y_kernel<17>, grid, dim3(256), 0, s, a.y, w, T, k, K1, H, (uint16_t*)out);
    else
      launch(MOE_PROF_COMBINE, combine_bf16y_kernel<0>, grid, dim3(256), 0, s, a.y, w, T, k, K1, H, (uint16_t*)out);
    MOE_LAUNCH_CHECK();
  }
  return MOE_OK;
}

bool decode_mfma_ok(int H, int I) {
  return H >= 256 && I >= 128 && H % 256 == 0 && I % 128 == 0 && H % kDKS == 0 && I % kDKS == 0;
}

// Grouped decode of T >= 2 bf16 tokens on bf16 MFMA: plan (keys by slot, the
// shared expert last; stable grouping; M tiles of up to 64 rows), gate/up
// with SwiGLU into h (bf16, grouped order), down into y (fp32, [T][K1][H]),
// then the rank-ordered combine.  plan: keys [P] | counts [4096] |
// offsets [4097] | perm [P] | items.
moe_status launch_decode_mfma(const moe_layer* Lr, const void* x, int T, int k, const int32_t* slot_ids, const float* w,
                              void* out, uint16_t* h, float* y, int32_t* plan, hipStream_t s) {
  const int K1 = k + (Lr->shared ? 1 : 0);
  const int H = Lr->H, I = Lr->I, E = Lr->num_slots;
  const int P = T * K1;
  PrefillArgs a;
  a.T = T, a.H = H, a.I = I, a.k = k, a.K1 = K1, a.E = E;
  a.bank = Lr->fp4_base;
  a.stride = Lr->fp4_stride;
  a.shared = Lr->shared;
  a.ids = slot_ids;
  a.xq = nullptr;
  a.xs = nullptr;
  a.keys = plan;
  a.counts = a.keys + P;
  a.offsets = a.counts + kMaxKeys;
  a.perm = a.offsets + kMaxKeys + 1;
  a.items = a.perm + P;
  a.hq = nullptr;
  a.hs = nullptr;
  a.y = nullptr;
  a.xb = (const uint16_t*)x;
  a.hb = h;
  a.yf = y;
  {
    const int W = group_chunks(E + 1);
    const size_t lds = (size_t)(W + 1) * (E + 1) * sizeof(int);
    launch(MOE_PROF_PLAN, plan_kernel<kDMT>, dim3(1), dim3(kGroupThreads), lds, s, a, W);
    MOE_LAUNCH_CHECK();
  }
  const long max_items_m = (long)P / kDMT + std::min(P, E + 1) + 1;
  const long slots = 256L * MOE_DG_PER_CU;  // workgroups resident at once
  const int grid_gu = (int)std::min<long>(max_items_m * (I / (kNR / 2)), slots) / 8 * 8;
  const int grid_dn = (int)std::min<long>(max_items_m * (H / kNR), slots) / 8 * 8;
  {
    launch(MOE_PROF_GATEUP, dgemm_kernel<2>, dim3(std::max(grid_gu, 8)), dim3(kDThreads), 0, s, a);
    MOE_LAUNCH_CHECK();
  }
  {
    launch(MOE_PROF_DOWN, dgemm_kernel<1>, dim3(std::max(grid_dn, 8)), dim3(kDThreads), 0, s, a);
    MOE_LAUNCH_CHECK();
  }
  return launch_combine(y, w, nullptr, T, k, H, Lr->shared ? 1 : 0, out, MOE_BF16, s);
}

size_t decode_mfma_plan_ints(int P) { return (size_t)P * 2 + kMaxKeys + (kMaxKeys + 1) + 1 + 3 * ((size_t)P / kDMT + kMaxKeys + 2); }

}  // namespace moe
