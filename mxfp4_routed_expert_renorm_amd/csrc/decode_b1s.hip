// Batch-1 decode of a narrow expert: one token through an expert whose
// intermediate size I is 256, 512 or 1024 — the share one GPU keeps of a
// 2048-wide expert under 8-, 4- or 2-way tensor parallelism ("Running
// DeepSeek-V4-Flash across four free GPUs", §Step 2: each rank holds I/G rows
// of w1 and w3 and the same I/G columns of w2).  Two launches, as at full
// width: routing + gate/up + SwiGLU, then down + weighted combine.
//
// With I that small the full-width kernels' one-wavefront-per-row mapping
// leaves most of the chip idle (I = 256 gives 64 workgroups) and their down
// rows are too short for 64 lanes, so the work is cut differently:
//
// gateup_b1s_kernel: SPL wavefronts share one gate/up row, each taking H/SPL
//   of its reduction (EL elements per lane, 8 or 16 FP4 bytes), so the grid
//   has I * SPL / 4 workgroups.  Each wavefront routes the token itself from
//   the logits row, requesting its slice of each selected expert's row right
//   after the round that picks it (at this width the step is a chain of
//   trips, so the rounds overlap the first rows' trips), reduces its partial
//   sums, and the row's first wavefront adds the SPL partials in wavefront
//   order and applies SwiGLU.
//
// down_b1s_kernel: LPR = I / 32 lanes per output row, one 32-element chunk
//   (16 FP4 bytes, one scale) per lane, so a wavefront covers 64 / LPR output
//   rows; the weighted combine over the ranks (rank order, shared expert
//   last with weight 1) happens per lane before the LPR-lane reduction, as on
//   the full-width path.
//
// MXFP4 experts only (no 2-bit copies), bf16 activations and output.
#include <algorithm>

#include "common.h"
#include "route_dev.h"
#include "b1_dev.h"

namespace moe {

namespace {

constexpr int kSMaxGroups = 12;
constexpr int kSMaxE = 1024;

struct B1SArgs {
  int H, I, k, K1, E;
  const uint8_t* fp4_base;
  size_t fp4_stride;
  int num_slots;
  const uint8_t* shared;
  const float* logits;  // [E]: the gate/up kernel routes the token; null: slot_ids and w are inputs
  const void* x;        // [1][H] bf16
  int32_t* slot_ids;    // [k]
  float* w;             // [k]
  uint16_t* h;          // [K1][I] bf16
  void* out;            // [1][H] bf16
};

// EL/2 bytes of FP4 codes (EL elements) . EL bf16 activations (EL/2 pairs),
// the block scale inside the convert
template <int EL>
__device__ __forceinline__ void fp4_dot(const uint32_t (&c)[EL / 8], const uint32_t (&xp)[EL / 2], float scale,
                                        float& a0, float& a1) {
#pragma unroll
  for (int i = 0; i < EL / 8; ++i) {
    a0 = dot2_bf16(fp4x2_to_bf16x2_scaled<0>(c[i], scale), xp[4 * i + 0], a0);
    a1 = dot2_bf16(fp4x2_to_bf16x2_scaled<1>(c[i], scale), xp[4 * i + 1], a1);
    a0 = dot2_bf16(fp4x2_to_bf16x2_scaled<2>(c[i], scale), xp[4 * i + 2], a0);
    a1 = dot2_bf16(fp4x2_to_bf16x2_scaled<3>(c[i], scale), xp[4 * i + 3], a1);
  }
}

template <int EL>
struct GUSlice {
  uint32_t c1[EL / 8], c3[EL / 8];
  uint32_t s1, s3;
};

template <int EL>
__device__ __forceinline__ void load_codes(uint32_t (&c)[EL / 8], const uint8_t* p) {
  if constexpr (EL == 16) {
    const uint2 v = ld_stream8(p);
    c[0] = v.x, c[1] = v.y;
  } else {
    const uint4 v = ld_stream16(p);
    c[0] = v.x, c[1] = v.y, c[2] = v.z, c[3] = v.w;
  }
}

template <int SPL, int EL, int NB, int EPL, bool SH>
__global__ __launch_bounds__(256) void gateup_b1s_kernel(B1SArgs a) {
  static_assert(SPL == 1 || SPL == 2 || SPL == 4, "1, 2 or 4 wavefronts per row");
  static_assert(EL == 16 || EL == 32, "8 or 16 code bytes per lane");
  constexpr int RW = 4 / SPL;  // rows per workgroup
  constexpr int S0 = SH ? 1 : 0;
  __shared__ float red[4][NB][2];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = blockIdx.x * RW + wave / SPL, part = wave % SPL;  // row < I: the grid tiles I
  const int I = a.I, k = a.k;
  const int e0 = part * (64 * EL) + lane * EL;  // the lane's first element of the reduction
  const size_t rowb = (size_t)a.H / 2, rows = (size_t)a.H / 32;
  const RecordLayout L = record_layout(a.H, I, 4);
  const size_t o1c = L.w1c + (size_t)row * rowb + e0 / 2, o3c = L.w3c + (size_t)row * rowb + e0 / 2;
  const size_t o1s = L.w1s + (size_t)row * rows + e0 / 32, o3s = L.w3s + (size_t)row * rows + e0 / 32;
  GUSlice<EL> sl[NB];
  auto issue = [&](GUSlice<EL>& s, const uint8_t* rec) {
    load_codes<EL>(s.c1, rec + o1c);
    load_codes<EL>(s.c3, rec + o3c);
    s.s1 = rec[o1s];
    s.s3 = rec[o3s];
  };

  // 1. the activation slice, the routing inputs, then the shared expert's slice
  uint32_t xp[EL / 2];
  {
    const uint4* src = (const uint4*)((const uint16_t*)a.x + e0);
#pragma unroll
    for (int i = 0; i < EL / 8; ++i) {
      const uint4 v = src[i];
      xp[4 * i] = v.x, xp[4 * i + 1] = v.y, xp[4 * i + 2] = v.z, xp[4 * i + 3] = v.w;
    }
  }
  int my_slot = -1;
  float lv[EPL > 0 ? EPL : 1];
  if constexpr (EPL > 0) {
    route_load<EPL>(a.logits, a.E, lv);
  } else {
    if (lane < k) my_slot = a.slot_ids[lane];
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (SH) issue(sl[0], a.shared);

  // 2. the token's ranks.  Routed here when logits are given: the experts are
  // the slots (every pick is valid), and each rank's slice is requested as
  // soon as its round picks it, so the selection overlaps the first rows'
  // trips; batch slots past the k ranks repeat rank k-1 and are not stored.
  // With given ids the valid ranks are listed first, then requested.
  int kx[NB];
  if constexpr (SH) kx[0] = k;
  int nact;
  if constexpr (EPL > 0) {
    float my_w;
    route_select_each<EPL, NB - S0>(lv, a.E, k, &my_slot, &my_w, [&](auto rc, uint32_t e) {
      constexpr int r = decltype(rc)::value;
      issue(sl[S0 + r], a.fp4_base + (size_t)e * a.fp4_stride);
      __builtin_amdgcn_sched_barrier(0);
    });
    if (blockIdx.x == 0 && wave == 0 && lane < k) {
      a.slot_ids[lane] = my_slot;
      a.w[lane] = my_w;
    }
#pragma unroll
    for (int u = S0; u < NB; ++u) kx[u] = min(u - S0, k - 1);
    nact = S0 + k;
  } else {
    const uint64_t m = __ballot(lane < k && my_slot >= 0 && my_slot < a.num_slots);
    const int nf = __popcll(m);
    nact = S0 + nf;
#pragma unroll
    for (int u = S0; u < NB; ++u) {  // batch slots past the active groups repeat the last one and are not stored
      const int r = nf > 0 ? nth_set_bit(m, min(u - S0, nf - 1)) : -1;
      kx[u] = r;
      const uint8_t* rec =
          r >= 0 ? a.fp4_base + (size_t)__builtin_amdgcn_readlane(my_slot, r) * a.fp4_stride : a.shared;
      if (rec) issue(sl[u], rec);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // every load above is out before the first slice is consumed

  // 3. slices in arrival order: partial gate and up sums of every group
  float gsum[NB], usum[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    float g0 = 0.0f, g1 = 0.0f, u0 = 0.0f, u1 = 0.0f;
    fp4_dot<EL>(sl[u].c1, xp, e8m0_to_f32(sl[u].s1), g0, g1);
    fp4_dot<EL>(sl[u].c3, xp, e8m0_to_f32(sl[u].s3), u0, u1);
    gsum[u] = wave_sum_to_lane63(g0 + g1);
    usum[u] = wave_sum_to_lane63(u0 + u1);
  }
  // lane u takes group u
  float gv = 0.0f, uv = 0.0f;
  int kv = 0;
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const float gu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gsum[u]), 63));
    const float uu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(usum[u]), 63));
    gv = lane == u ? gu : gv;
    uv = lane == u ? uu : uv;
    kv = lane == u ? kx[u] : kv;
  }
  if constexpr (SPL > 1) {
    if (lane < NB) {
      red[wave][lane][0] = gv;
      red[wave][lane][1] = uv;
    }
    __syncthreads();
    if (part != 0) return;
    gv = 0.0f, uv = 0.0f;
    if (lane < NB) {
#pragma unroll
      for (int p = 0; p < SPL; ++p) {  // the row's partials in wavefront order
        gv += red[wave + p][lane][0];
        uv += red[wave + p][lane][1];
      }
    }
  }
  if (lane < nact) a.h[(size_t)kv * I + row] = f32_to_bf16(silu_mul_b1(gv, uv));
}

// sum over each aligned group of N = 8, 16 or 32 lanes, in every lane of the
// group, on DPP lane moves (quad butterflies, the mirrors within 8 and 16
// lanes) and, for 32, the swap of row pairs: no LDS round trips
template <int N>
__device__ __forceinline__ float lanes_sum(float v) {
  static_assert(N == 8 || N == 16 || N == 32, "8, 16 or 32 lanes");
  v += dpp_f32<dpp::kQuadXor1>(v);
  v += dpp_f32<dpp::kQuadXor2>(v);
  v += dpp_f32<dpp::kRowHalfMirror>(v);
  if constexpr (N >= 16) v += dpp_f32<dpp::kRowMirror>(v);
  if constexpr (N == 32) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
  return v;
}

template <int LPR, int NB, bool SH>
__global__ __launch_bounds__(256) void down_b1s_kernel(B1SArgs a) {
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "I is 256, 512 or 1024");
  constexpr int I = 32 * LPR;
  constexpr int RPW = 64 / LPR;  // output rows per wavefront
  constexpr int S0 = SH ? 1 : 0;
  __shared__ __align__(16) uint8_t hl[NB * I * 2];  // the SwiGLU outputs of group g at slot g
  __shared__ float stab[256];                      // E8M0 byte -> scale
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int orow = blockIdx.x * (4 * RPW) + wave * RPW + lane / LPR;  // < H: the grid tiles H exactly
  const int c = lane % LPR;                                            // the lane's chunk of the row
  const int k = a.k;
  const RecordLayout L = record_layout(a.H, I, 4);
  const size_t oc = L.w2c + (size_t)orow * (I / 2) + (size_t)c * 16, os = L.w2s + (size_t)orow * (I / 32) + c;

  // 1. ids and weights, the SwiGLU outputs of every group, the shared row
  int slot = -1;
  float wg = 0.0f;
  if (lane < k) {
    slot = a.slot_ids[lane];
    wg = a.w[lane];
  }
  __builtin_amdgcn_sched_barrier(0);
  constexpr int kHPieces = NB * I * 2 / 16;  // 16-byte pieces of the staged h
  constexpr int kHPer = (kHPieces + 255) / 256;
  uint4 hv[kHPer];
#pragma unroll
  for (int j = 0; j < kHPer; ++j) {
    const int i = min(tid + 256 * j, kHPieces - 1);
    const int g = i / (I / 8), q = i % (I / 8);
    hv[j] = ((const uint4*)(a.h + (size_t)min(g, a.K1 - 1) * I))[q];
  }
  uint4 cw[NB];
  uint32_t sw[NB];
  if constexpr (SH) {
    cw[0] = ld_stream16(a.shared + oc);
    sw[0] = a.shared[os];
  }
  stab[tid] = e8m0_to_f32(tid);
#pragma unroll
  for (int j = 0; j < kHPer; ++j) {
    const int i = tid + 256 * j;
    if (i < kHPieces) ((uint4*)hl)[i] = hv[j];
  }

  // 2. the surviving ranks in rank order and their W2 chunks
  const bool live = lane < k && slot >= 0 && slot < a.num_slots;
  const uint64_t m = __ballot(live);
  const int nr = __popcll(m);
  int gi[NB];
  float wi[NB];
  if constexpr (SH) {
    gi[0] = k;
    wi[0] = 1.0f;
  }
#pragma unroll
  for (int u = S0; u < NB; ++u) {
    const int g = nr > 0 ? nth_set_bit(m, min(u - S0, nr - 1)) : 0;
    gi[u] = g;
    wi[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wg), g));
    const uint8_t* rec = a.fp4_base + (size_t)max(__builtin_amdgcn_readlane(slot, g), 0) * a.fp4_stride;
    if (nr > 0) {
      cw[u] = ld_stream16(rec + oc);
      sw[u] = rec[os];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();

  // 3. the weighted sum in rank order, the shared expert (weight 1) last
  auto part_of = [&](int u) {
    B1Chunk hq;
    hq.load_lds(hl + (size_t)gi[u] * I * 2, (size_t)c * 32);
    float p0 = 0.0f, p1 = 0.0f;
    hq.fp4_acc(cw[u], stab[sw[u]], p0, p1);
    return p0 + p1;
  };
  float acc = 0.0f;
  if (nr > 0) {
#pragma unroll
    for (int u = S0; u < NB; ++u) {
      const float t = fmaf(wi[u], part_of(u), acc);
      acc = (u - S0 < nr) ? t : acc;
    }
  }
  if constexpr (SH) acc += part_of(0);
  const float v = lanes_sum<LPR>(acc);
  if (c == 0) ((uint16_t*)a.out)[orow] = f32_to_bf16(v);
}

int s_batch(int K1) { return K1 <= 4 ? 4 : K1 <= 7 ? 7 : K1 <= 9 ? 9 : kSMaxGroups; }

template <int SPL, int EL, int NB, bool SH>
void launch_gateup_s(const B1SArgs& a, hipStream_t s) {
  const dim3 grid(a.I * SPL / 4);
  if (!a.logits)
    launch(MOE_PROF_GATEUP, (gateup_b1s_kernel<SPL, EL, NB, 0, SH>), grid, dim3(256), 0, s, a);
  else if (a.E <= 256)
    launch(MOE_PROF_GATEUP, (gateup_b1s_kernel<SPL, EL, NB, 4, SH>), grid, dim3(256), 0, s, a);
  else
    launch(MOE_PROF_GATEUP, (gateup_b1s_kernel<SPL, EL, NB, kSMaxE / 64, SH>), grid, dim3(256), 0, s, a);
}

// the reduction split: 16 elements per lane where that still leaves H/SPL a
// whole number of wavefronts of at most 4, else 32; SPL = H / (64 EL)
template <int NB, bool SH>
void launch_gateup_nb_s(const B1SArgs& a, hipStream_t s) {
  const bool narrow = a.I <= 256;  // I = 256: split four ways at H 4096 (256 workgroups)
  if (a.H == 4096) {
    if (narrow)
      launch_gateup_s<4, 16, NB, SH>(a, s);
    else
      launch_gateup_s<2, 32, NB, SH>(a, s);
  } else {  // H == 2048
    if (narrow)
      launch_gateup_s<2, 16, NB, SH>(a, s);
    else
      launch_gateup_s<1, 32, NB, SH>(a, s);
  }
}

template <int LPR, int NB, bool SH>
void launch_down_s(const B1SArgs& a, hipStream_t s) {
  const dim3 grid(a.H / (4 * (64 / LPR)));
  launch(MOE_PROF_DOWN, (down_b1s_kernel<LPR, NB, SH>), grid, dim3(256), 0, s, a);
}

template <int NB, bool SH>
void launch_nb_s(const B1SArgs& a, hipStream_t s, moe_status* st) {
  launch_gateup_nb_s<NB, SH>(a, s);
  if (hipGetLastError() != hipSuccess) {
    *st = MOE_EHIP;
    return;
  }
  if (a.I == 256)
    launch_down_s<8, NB, SH>(a, s);
  else if (a.I == 512)
    launch_down_s<16, NB, SH>(a, s);
  else
    launch_down_s<32, NB, SH>(a, s);
  *st = hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

template <bool SH>
void launch_sh_s(const B1SArgs& a, hipStream_t s, moe_status* st) {
  switch (s_batch(a.K1)) {
    case 4: launch_nb_s<4, SH>(a, s, st); break;
    case 7: launch_nb_s<7, SH>(a, s, st); break;
    case 9: launch_nb_s<9, SH>(a, s, st); break;
    default: launch_nb_s<kSMaxGroups, SH>(a, s, st); break;
  }
}

}  // namespace

// Narrow experts at batch 1: bf16 activations and output, MXFP4 ranks only,
// H in {2048, 4096}, I in {256, 512, 1024}, at most 12 groups.
bool b1s_path_ok(int H, int I, int K1, bool xbf16, bool obf16, bool has_prec) {
  if (!xbf16 || !obf16 || has_prec) return false;
  if (!(H == 2048 || H == 4096) || !(I == 256 || I == 512 || I == 1024)) return false;
  return K1 >= 1 && K1 <= kSMaxGroups;
}

bool b1s_route_ok(int E, int num_slots) { return E >= 1 && E <= kSMaxE && num_slots >= E; }

moe_status launch_b1s(const moe_layer* L, const float* logits, int E, const void* x, int k, int32_t* slot_ids,
                      float* w, uint16_t* h, void* out, hipStream_t s) {
  B1SArgs a;
  a.H = L->H;
  a.I = L->I;
  a.k = k;
  a.K1 = k + (L->shared ? 1 : 0);
  a.E = E;
  a.fp4_base = L->fp4_base;
  a.fp4_stride = L->fp4_stride;
  a.num_slots = L->num_slots;
  a.shared = L->shared;
  a.logits = logits;
  a.x = x;
  a.slot_ids = slot_ids;
  a.w = w;
  a.h = h;
  a.out = out;
  moe_status st = MOE_OK;
  if (a.shared)
    launch_sh_s<true>(a, s, &st);
  else
    launch_sh_s<false>(a, s, &st);
  if (st != MOE_OK) return fail(st, "batch-1 narrow-expert launch failed: %s", hipGetErrorString(hipGetLastError()));
  return MOE_OK;
}

}  // namespace moe
