// Batch-1 decode kernels: one token, k routed experts plus the shared expert.
//
// At batch 1 the layer is a pure stream of expert bytes ("Running
// DeepSeek-V4-Flash across four free GPUs", §The arithmetic that explains 20
// tok/s; "An elephant through a straw", §The number: the GPU spends its time
// receiving experts, not multiplying them).  A whole token is only ~120 MB,
// a few tens of KiB per wavefront, so each kernel requests everything it
// will read up front and then consumes it in arrival order:
//
// gateup_b1_kernel: wavefront i owns gate/up row i of every expert of the
//   token (the shared expert first, then the FP4 ranks).  It requests the
//   activation, then the routing inputs, then the shared expert's row, which
//   needs no routing; routes the token itself from the logits row (or reads
//   ids); stages the activation in LDS (once per workgroup); then requests
//   row i of every routed expert at once.  Each row's gate and up sums are
//   reduced with DPP lane moves, and the SwiGLU of the row for all experts
//   runs in one lane-parallel pass (lane g takes expert g).
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
#include "b1_dev.h"


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

// ------------------------------------------------------------------ gate/up

template <int CPL>
struct GURow {
  uint4 c1[CPL], c3[CPL];
  uint32_t s1[CPL], s3[CPL];
};

template <int CPL, int NB, int EPL, bool SH, bool HAS2>
__global__ __launch_bounds__(256, 2) void gateup_b1_kernel(B1Args a) {
  constexpr int XBYTES = CPL * 64 * 32 * 2;  // H bf16 activations
  static_assert(CPL == 1 || CPL == 2, "H is 2048 or 4096");
  static_assert(NB >= 1 + (SH ? 1 : 0), "batch holds the shared expert and at least one rank");
  __shared__ __align__(16) uint8_t xs[XBYTES];
  __shared__ float stab[256];  // E8M0 byte -> scale
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // < I: the grid tiles I
  const int I = a.I, k = a.k;
  const size_t rowb4 = (size_t)a.H / 2, rows4 = (size_t)a.H / 32;
  const RecordLayout L = record_layout(a.H, I, 4);
  GURow<CPL> sl[NB];
  auto issue = [&](GURow<CPL>& s, const uint8_t* rec) {
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const size_t c = (size_t)(q * 64 + lane);
      s.c1[q] = ld_stream16(rec + L.w1c + (size_t)row * rowb4 + c * 16);
      s.c3[q] = ld_stream16(rec + L.w3c + (size_t)row * rowb4 + c * 16);
      s.s1[q] = rec[L.w1s + (size_t)row * rows4 + c];
      s.s3[q] = rec[L.w3s + (size_t)row * rows4 + c];
    }
  };

  // 1. the activation, then the routing inputs, then the shared expert's
  // row (it needs no routing): the routing inputs return ahead of the
  // weights, and the weight stream starts before the routing is done
  const uint4 xv0 = ((const uint4*)a.x)[threadIdx.x];
  const uint4 xv1 = CPL == 2 ? ((const uint4*)a.x)[threadIdx.x + 256] : make_uint4(0u, 0u, 0u, 0u);
  int my_slot = -1, my_prec = -1;
  float lv[EPL > 0 ? EPL : 1];
  if constexpr (EPL > 0) {
    route_load<EPL>(a.logits, a.E, lv);
  } else {
    if (lane < k) {
      my_slot = a.slot_ids[lane];
      my_prec = a.prec ? (int)a.prec[lane] : 0;
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // the routing inputs stay ahead of the shared row in the queue
  if constexpr (SH) issue(sl[0], a.shared);
  stab[threadIdx.x] = e8m0_to_f32(threadIdx.x);

  // 2. the token's FP4 ranks (routed here when logits are given)
  if constexpr (EPL > 0) {
    float my_w;
    route_select<EPL>(lv, a.E, k, &my_slot, &my_w);
    my_prec = 0;
    if (row == 0 && lane < k) {
      a.slot_ids[lane] = my_slot;
      a.w[lane] = my_w;
    }
  }
  const bool fp4 = lane < k && my_prec == 0 && my_slot >= 0 && my_slot < a.num_slots;
  const uint64_t m = __ballot(fp4);
  // the 2-bit ranks (slot-cache fallback copies): their rows follow the FP4 ones
  const uint64_t m2 = HAS2 ? __ballot(lane < k && my_prec == 1 && my_slot >= 0 && my_slot < a.num_int2) : 0;
  const int nf = __popcll(m);
  constexpr int S0 = SH ? 1 : 0;
  const int nact = S0 + nf;
  ((uint4*)xs)[threadIdx.x] = xv0;
  if (CPL == 2) ((uint4*)xs)[threadIdx.x + 256] = xv1;
  __syncthreads();
  if (nact > 0) {
    // 3. this row of every FP4 rank (batch slots past the active groups repeat
    // the last one and are not stored)
    int kx[NB];
    if constexpr (SH) kx[0] = k;
#pragma unroll
    for (int u = S0; u < NB; ++u) {
      const int r = nf > 0 ? nth_set_bit(m, min(u - S0, nf - 1)) : -1;
      kx[u] = r;
      const uint8_t* rec = r >= 0 ? a.fp4_base + (size_t)__builtin_amdgcn_readlane(my_slot, r) * a.fp4_stride : a.shared;
      issue(sl[u], rec);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load above is out before the first row is consumed

    // 4. rows in arrival order; the block scale rides in the convert, so each
    // row is one accumulation chain per matrix (two for instruction overlap)
    float gsum[NB], usum[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      float g0a = 0.0f, g1a = 0.0f, u0a = 0.0f, u1a = 0.0f;
#pragma unroll
      for (int q = 0; q < CPL; ++q) {
        B1Chunk xq;  // re-read per row: LDS bandwidth is cheaper than 16 registers per chunk
        xq.load_lds(xs, (size_t)(q * 64 + lane) * 32);
        xq.fp4_acc(sl[u].c1[q], stab[sl[u].s1[q]], g0a, g1a);
        xq.fp4_acc(sl[u].c3[q], stab[sl[u].s3[q]], u0a, u1a);
      }
      gsum[u] = wave_sum_to_lane63(g0a + g1a);
      usum[u] = wave_sum_to_lane63(u0a + u1a);
    }
    // 5. SwiGLU of the row for every group at once: lane u takes group u
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
    if (lane < nact) a.h[(size_t)kv * I + row] = f32_to_bf16(silu_mul_b1(gv, uv));
  }

  // 6. the 2-bit ranks' rows, one at a time (rarely more than two; the FP4
  // rows' registers are free again): 32 codes per lane and chunk, the
  // activation from LDS, the E4M3 block scale applied per chunk
  if constexpr (HAS2) {
    const RecordLayout L2 = record_layout(a.H, I, 2);
    const size_t rowb2 = (size_t)a.H / 4;
    for (uint64_t mm = m2; mm; mm &= mm - 1) {
      const int g = __builtin_ctzll(mm);
      const uint8_t* rec = a.int2_base + (size_t)__builtin_amdgcn_readlane(my_slot, g) * a.int2_stride;
      float gs = 0.0f, us = 0.0f;
#pragma unroll
      for (int q = 0; q < CPL; ++q) {
        const size_t c = (size_t)(q * 64 + lane);
        const uint2 c1 = ld_stream8(rec + L2.w1c + (size_t)row * rowb2 + c * 8);
        const uint2 c3 = ld_stream8(rec + L2.w3c + (size_t)row * rowb2 + c * 8);
        B1Chunk xq;
        xq.load_lds(xs, c * 32);
        gs = fmaf(xq.int2(c1), e4m3_to_f32(rec[L2.w1s + (size_t)row * rows4 + c]), gs);
        us = fmaf(xq.int2(c3), e4m3_to_f32(rec[L2.w3s + (size_t)row * rows4 + c]), us);
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

template <int CPL, int NB, bool HAS2, bool SH>
__global__ __launch_bounds__(256) void down_combine_b1_kernel(B1Args a) {
  extern __shared__ __align__(16) uint8_t lds[];  // [NB][I] bf16: the SwiGLU outputs of group g at slot g
  __shared__ float stab[256];                      // E8M0 byte -> scale
  constexpr int S0 = SH ? 1 : 0;
  constexpr int NR = NB - S0;  // rank slots
  const int tid = threadIdx.x, lane = tid & 63;
  const int orow = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(tid >> 6);  // < H: the grid tiles H exactly
  const int I = a.I, k = a.k;
  const size_t rowb4 = (size_t)I / 2, rowb2 = (size_t)I / 4, rows = (size_t)I / 32;
  const RecordLayout L4 = record_layout(a.H, I, 4), L2 = record_layout(a.H, I, 2);
  auto issue4 = [&](DNRow<CPL>& d, const uint8_t* rec) {
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const size_t c = (size_t)(q * 64 + lane);
      d.c[q] = ld_stream16(rec + L4.w2c + (size_t)orow * rowb4 + c * 16);
      d.s[q] = rec[L4.w2s + (size_t)orow * rows + c];
    }
  };

  // 1. the ranks' ids, precisions and weights (the small loads go out
  // together), then the SwiGLU outputs of every group (by group index, so
  // independent of the ids) and the shared expert's W2 row
  int p = 0, slot = -1;
  float wg = 0.0f;
  if (lane < k) {
    if constexpr (HAS2) p = (int)a.prec[lane];  // precisions are given exactly when 2-bit copies may appear
    slot = a.slot_ids[lane];
    wg = a.w[lane];
  }
  __builtin_amdgcn_sched_barrier(0);
  uint4 h0[NB], h1[NB];
#pragma unroll
  for (int g = 0; g < NB; ++g) {
    const uint4* src = (const uint4*)(a.h + (size_t)min(g, a.K1 - 1) * I);
    h0[g] = src[tid];
    if (CPL == 2) h1[g] = src[tid + 256];
  }
  DNRow<CPL> sl[NB];  // slot 0: the shared expert when present, then the ranks
  if constexpr (SH) issue4(sl[0], a.shared);
  stab[tid] = e8m0_to_f32(tid);
#pragma unroll
  for (int g = 0; g < NB; ++g) {  // waits for the ids and h, not for the shared row
    ((uint4*)(lds + (size_t)g * I * 2))[tid] = h0[g];
    if (CPL == 2) ((uint4*)(lds + (size_t)g * I * 2))[tid + 256] = h1[g];
  }

  // 2. the surviving ranks in rank order, and their W2 rows (batch slots
  // past them repeat the last one and are not summed)
  const int pr = lane >= k ? -1
                 : (p == 0 && slot >= 0 && slot < a.num_slots) ? 0
                 : (HAS2 && p == 1 && slot >= 0 && slot < a.num_int2) ? 1 : -1;
  const uint64_t m = __ballot(pr >= 0);
  const int nr = __popcll(m);
  int gi[NB], pi[NB];
  float wi[NB];
  if constexpr (SH) {
    gi[0] = k;
    pi[0] = 0;
    wi[0] = 1.0f;
  }
  auto part_of = [&](int u) {
    float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      B1Chunk hq;
      hq.load_lds(lds + (size_t)gi[u] * I * 2, (size_t)(q * 64 + lane) * 32);
      if (!HAS2 || pi[u] == 0)
        hq.fp4_acc(sl[u].c[q], stab[sl[u].s[q]], p0, p1);
      else
        p0 = fmaf(hq.int2(make_uint2(sl[u].c[q].x, sl[u].c[q].y)), e4m3_to_f32(sl[u].s[q]), p0);
    }
    return p0 + p1;
  };
  if (nr == 0) {  // every rank dropped: the shared expert alone, or nothing
    __syncthreads();
    float acc = 0.0f;
    if constexpr (SH) acc = part_of(0);
    const float v = wave_sum_to_lane63(acc);
    if (lane == 63) ((uint16_t*)a.out)[orow] = f32_to_bf16(v);
    return;
  }
#pragma unroll
  for (int u = S0; u < NB; ++u) {
    const int g = nth_set_bit(m, min(u - S0, nr - 1));
    gi[u] = g;
    pi[u] = __builtin_amdgcn_readlane(pr, g);
    wi[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wg), g));
    const size_t sg = (size_t)__builtin_amdgcn_readlane(slot, g);
    if (HAS2 && pi[u] == 1) {
#pragma unroll
      for (int q = 0; q < CPL; ++q) {
        const size_t c = (size_t)(q * 64 + lane);
        const uint8_t* rec = a.int2_base + sg * a.int2_stride;
        const uint2 v = ld_stream8(rec + L2.w2c + (size_t)orow * rowb2 + c * 8);
        sl[u].c[q] = make_uint4(v.x, v.y, 0u, 0u);
        sl[u].s[q] = rec[L2.w2s + (size_t)orow * rows + c];
      }
    } else {
      issue4(sl[u], a.fp4_base + sg * a.fp4_stride);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // every W2 load is out before the first wait
  __syncthreads();

  // 3. the weighted sum in rank order, then the shared expert (weight 1).
  // Straight-line code: slots past the survivors are computed and selected
  // away, so no load is sunk into a branch.
  int nr_v;  // the survivor count in a vector register: the selects stay selects
  asm volatile("v_mov_b32 %0, %1" : "=v"(nr_v) : "s"(nr));
  float acc = 0.0f;
#pragma unroll
  for (int u = S0; u < NB; ++u) {
    const float t = fmaf(wi[u], part_of(u), acc);
    acc = (u - S0 < nr_v) ? t : acc;
  }
  if constexpr (SH) acc += part_of(0);
  const float v = wave_sum_to_lane63(acc);
  if (lane == 63) ((uint16_t*)a.out)[orow] = f32_to_bf16(v);
}

// ------------------------------------------------------------------ launch

// batch of the down kernel: every group of the token at once (k = 6 or 8
// plus the shared expert are exact; other counts repeat the last group)
int down_batch(int K1) { return K1 <= 4 ? 4 : K1 <= 7 ? 7 : K1 <= 9 ? 9 : kMaxGroups; }

template <int CPL, int NB, bool SH>
void launch_gateup_nb(const B1Args& a, hipStream_t s) {
  const int grid = a.I / 4;  // one wavefront per gate/up row
  if (!a.logits && a.prec)  // 2-bit copies can only appear when precisions are given
    launch(MOE_PROF_GATEUP, (gateup_b1_kernel<CPL, NB, 0, SH, true>), dim3(grid), dim3(256), 0, s, a);
  else if (!a.logits)
    launch(MOE_PROF_GATEUP, (gateup_b1_kernel<CPL, NB, 0, SH, false>), dim3(grid), dim3(256), 0, s, a);
  else if (a.E <= 256)
    launch(MOE_PROF_GATEUP, (gateup_b1_kernel<CPL, NB, 4, SH, false>), dim3(grid), dim3(256), 0, s, a);
  else
    launch(MOE_PROF_GATEUP, (gateup_b1_kernel<CPL, NB, kMaxE / 64, SH, false>), dim3(grid), dim3(256), 0, s, a);
}

template <int CPL, bool SH>
void launch_gateup_sh(const B1Args& a, hipStream_t s) {
  const int nb = down_batch(a.K1);
  if (nb == 4)
    launch_gateup_nb<CPL, 4, SH>(a, s);
  else if (nb == 7)
    launch_gateup_nb<CPL, 7, SH>(a, s);
  else if (nb == 9)
    launch_gateup_nb<CPL, 9, SH>(a, s);
  else if constexpr (CPL == 1)
    launch_gateup_nb<CPL, kMaxGroups, SH>(a, s);
}

template <int CPL>
void launch_gateup_b1(const B1Args& a, hipStream_t s) {
  if (a.shared)
    launch_gateup_sh<CPL, true>(a, s);
  else
    launch_gateup_sh<CPL, false>(a, s);
}

template <int CPL, bool HAS2, bool SH>
void launch_down_nb(const B1Args& a, hipStream_t s) {
  const int grid = a.H / 4;
  const int nb = down_batch(a.K1);
  const size_t lds = (size_t)nb * a.I * 2;
  if (nb == 4)
    launch(MOE_PROF_DOWN, (down_combine_b1_kernel<CPL, 4, HAS2, SH>), dim3(grid), dim3(256), lds, s, a);
  else if (nb == 7)
    launch(MOE_PROF_DOWN, (down_combine_b1_kernel<CPL, 7, HAS2, SH>), dim3(grid), dim3(256), lds, s, a);
  else if (nb == 9)
    launch(MOE_PROF_DOWN, (down_combine_b1_kernel<CPL, 9, HAS2, SH>), dim3(grid), dim3(256), lds, s, a);
  else if constexpr (CPL == 1)
    launch(MOE_PROF_DOWN, (down_combine_b1_kernel<CPL, kMaxGroups, HAS2, SH>), dim3(grid), dim3(256), lds, s, a);
}

template <int CPL>
void launch_down_b1(const B1Args& a, hipStream_t s) {
  if (a.prec) {
    if (a.shared)
      launch_down_nb<CPL, true, true>(a, s);
    else
      launch_down_nb<CPL, true, false>(a, s);
  } else {
    if (a.shared)
      launch_down_nb<CPL, false, true>(a, s);
    else
      launch_down_nb<CPL, false, false>(a, s);
  }
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
  if (K1 < 1 || K1 > (H == 2048 ? kMaxGroups : 9)) return false;  // the gate/up rows of a wavefront fit its registers
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
    if (a.H == 2048)
      launch_gateup_b1<1>(a, s);
    else
      launch_gateup_b1<2>(a, s);
    MOE_LAUNCH_CHECK();
  }
  {
    if (a.I == 2048)
      launch_down_b1<1>(a, s);
    else
      launch_down_b1<2>(a, s);
    MOE_LAUNCH_CHECK();
  }
  return MOE_OK;
}

}  // namespace moe
