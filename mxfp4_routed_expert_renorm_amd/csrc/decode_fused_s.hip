// Single-launch batch-1 decode of an 8-way tensor-parallel share (hidden 4096,
// expert intermediate 2048 / 8 = 256 per share: "Running DeepSeek-V4-Flash
// across four free GPUs", §Step 2), opt-in like the full-width single launch.
//
// At this size each of the two launches of the narrow step is a chain of
// dependent trips (inputs, then weight rows, then the reduction) whatever its
// bytes, so the second launch's chain is the cost to remove.  Here the W2
// rows are requested right after routing, while gate/up is still computing,
// and only the 9 x 256 SwiGLU outputs cross workgroups.
//
// 256 workgroups of four wavefronts, one per CU; unit u = workgroup u.
//   Gate/up: unit u computes gate/up row u of every group (the shared expert
//     first, then the valid ranks in rank order); wavefront w takes
//     H [1024 w, 1024 w + 1024), 16 weights per lane, routes the token from
//     the logits row itself, and requests its slices up front.  The partial
//     sums meet in LDS; wavefront 0 applies SwiGLU and publishes the unit's
//     nine bf16 values of h with write-through (agent-scope) stores, then
//     arrives at the launch's handoff (per-unit tags, two levels of arrival
//     counters, one word polled).
//   Down: unit u computes output rows 16u .. 16u + 15.  Lane l of wavefront w
//     takes row 8 (w % 2) + l / 8 and the 32-weight chunk l % 8 of it, for
//     the groups of half w / 2 (the first ceil(NB / 2) groups of the batch,
//     then the rest); those W2 chunks are
//     requested right after the gate/up slices.  Once every unit has
//     arrived, h (at most 4.5 KiB) is staged into LDS with plain loads, each
//     lane dots its chunks, eight lanes reduce a row, and the row's groups
//     are combined in rank order (shared expert last, weight 1), rounded once.
// The handoff is the full-width single launch's: nothing is reset between
// launches (the sync words must start at zero: a zeroed workspace), launches
// sharing them must not overlap, and every wait is bounded (a wait that gives
// up sets the error word; the output is then meaningless).
#include "common.h"
#include "route_dev.h"
#include "b1_dev.h"
#include "handoff_dev.h"

namespace moe {

namespace {

constexpr int kSH = 4096, kSI = 256;
constexpr int kSUnits = kHandoffUnits;   // gate/up rows = workgroups
constexpr int kSRowsDN = kSH / kSUnits;  // 16 down rows per unit
constexpr int kSMaxG = 9;                // shared expert + 8 ranks
constexpr uint32_t kSSpin = 1u << 21;    // poll rounds before a wait gives up
static_assert(kSI == kSUnits, "a unit per gate/up row");

struct FusedSArgs {
  int k, E;
  const uint8_t* fp4_base;
  size_t fp4_stride;
  int num_slots;
  const uint8_t* shared;
  const float* logits;  // [E]: the kernel routes the token; null: slot_ids and w are inputs
  const void* x;        // [kSH] bf16
  int32_t* slot_ids;    // [k]
  float* w;             // [k]
  uint16_t* h;          // [kSMaxG][kSI] bf16
  void* out;            // [kSH] bf16
  uint32_t* sync;       // the handoff's words, kept between launches
};

template <int NB, int EPL, bool SH>
__global__ __launch_bounds__(256, 1) void fused_b1s_kernel(FusedSArgs a) {
  constexpr int S0 = SH ? 1 : 0;
  static_assert(NB <= kSMaxG && NB > S0, "groups of the batch");
  constexpr int GH = (NB + 1) / 2;  // groups per down half
  __shared__ float red[4][NB][2];
  __shared__ __align__(16) uint8_t hl[kSMaxG * kSI * 2];  // every group's h, bf16
  __shared__ float res[kSMaxG][kSRowsDN];                 // group g's W2 row r . h_g
  __shared__ float gw[kSMaxG];                            // group weights (routed groups)
  __shared__ float stab[256];                             // E8M0 byte -> scale
  __shared__ uint32_t go;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int unit = blockIdx.x;
  const int k = a.k;
  const RecordLayout L = record_layout(kSH, kSI, 4);
  if (tid == 0) go = 0u;
  stab[tid] = e8m0_to_f32(tid);

  const uint32_t tag = handoff_tag(a.sync, unit);

  // 1. the activation slice, the routing inputs, the shared expert's slice
  const int e0 = wave * 1024 + lane * 16;
  uint32_t xp[8];
  {
    const uint4* src = (const uint4*)((const uint16_t*)a.x + e0);
    const uint4 v0 = src[0], v1 = src[1];
    xp[0] = v0.x, xp[1] = v0.y, xp[2] = v0.z, xp[3] = v0.w;
    xp[4] = v1.x, xp[5] = v1.y, xp[6] = v1.z, xp[7] = v1.w;
  }
  int my_slot = -1;
  float my_w = 0.0f;
  float lv[EPL > 0 ? EPL : 1];
  if constexpr (EPL > 0) {
    route_load<EPL>(a.logits, a.E, lv);
  } else {
    const int l = min(lane, k - 1);  // unconditional loads: fixed count in flight
    my_slot = a.slot_ids[l];
    my_w = a.w[l];
  }
  __builtin_amdgcn_sched_barrier(0);
  const size_t o1c = L.w1c + (size_t)unit * (kSH / 2) + e0 / 2, o3c = L.w3c + (size_t)unit * (kSH / 2) + e0 / 2;
  const size_t o1s = L.w1s + (size_t)unit * (kSH / 32) + e0 / 32, o3s = L.w3s + (size_t)unit * (kSH / 32) + e0 / 32;
  uint2 c1[NB], c3[NB];
  uint32_t s1[NB], s3[NB];
  auto issue_gu = [&](int g, const uint8_t* rec) {
    c1[g] = ld_stream8(rec + o1c);
    c3[g] = ld_stream8(rec + o3c);
    s1[g] = rec[o1s];
    s3[g] = rec[o3s];
  };
  const uint8_t* rec0 = SH ? a.shared : a.fp4_base;
  if constexpr (SH) issue_gu(0, a.shared);

  // 2. the token's ranks: every wavefront routes (or reads) them itself.
  // Routed here, each rank's slice is requested as soon as its round picks it
  // (the experts are the slots, every pick valid; slots past the k ranks
  // repeat rank k-1); with given ids the valid ranks are listed, then requested.
  if constexpr (EPL > 0)
    route_select_each<EPL, NB - S0>(lv, a.E, k, &my_slot, &my_w, [&](auto rc, uint32_t e) {
      constexpr int r = decltype(rc)::value;
      issue_gu(S0 + r, a.fp4_base + (size_t)e * a.fp4_stride);
      __builtin_amdgcn_sched_barrier(0);
    });
  const bool valid = lane < k && my_slot >= 0 && my_slot < a.num_slots;
  const uint64_t m = __ballot(valid);
  const int nf = __popcll(m), ng = S0 + nf;
  if (wave == 0) {
    if (EPL > 0 && unit == 0 && lane < k) {  // the routing result, for the caller
      a.slot_ids[lane] = my_slot;
      a.w[lane] = my_w;
    }
    if (valid) gw[S0 + __popcll(m & ((1ull << lane) - 1ull))] = my_w;
  }
  // group g's record (past the active groups: the last one again, its loads
  // issued but never used, so the count in flight is fixed)
  auto grec = [&](int g) -> const uint8_t* {
    if (ng == 0) return rec0;
    g = min(g, ng - 1);
    if (g < S0) return a.shared;
    const int r = nth_set_bit(m, g - S0);
    return a.fp4_base + (size_t)__builtin_amdgcn_readlane(my_slot, r) * a.fp4_stride;
  };
  if constexpr (EPL == 0) {
#pragma unroll
    for (int g = S0; g < NB; ++g) issue_gu(g, grec(g));
  }

  // 3. the W2 chunks of this lane's down rows, for its half of the groups
  const int drow = unit * kSRowsDN + 8 * (wave & 1) + (lane >> 3), dc = lane & 7, half = wave >> 1;
  const size_t w2c = L.w2c + (size_t)drow * (kSI / 2) + (size_t)dc * 16, w2s = L.w2s + (size_t)drow * (kSI / 32) + dc;
  uint4 wc[GH];
  uint32_t ws[GH];
#pragma unroll
  for (int j = 0; j < GH; ++j) {
    const uint8_t* rec = grec(half * GH + j);
    wc[j] = ld_stream16(rec + w2c);
    ws[j] = rec[w2s];
  }
  __builtin_amdgcn_sched_barrier(0);  // every load above is out before the first slice is consumed

  // 4. gate/up partial sums of every group, reduced over the four quarters of H
#pragma unroll
  for (int g = 0; g < NB; ++g) {
    float g0 = 0.0f, g1 = 0.0f, u0 = 0.0f, u1 = 0.0f;
    const uint32_t cg[2] = {c1[g].x, c1[g].y}, cu[2] = {c3[g].x, c3[g].y};
    const float sg = e8m0_to_f32(s1[g]), su = e8m0_to_f32(s3[g]);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      g0 = dot2_bf16(fp4x2_to_bf16x2_scaled<0>(cg[i], sg), xp[4 * i + 0], g0);
      g1 = dot2_bf16(fp4x2_to_bf16x2_scaled<1>(cg[i], sg), xp[4 * i + 1], g1);
      g0 = dot2_bf16(fp4x2_to_bf16x2_scaled<2>(cg[i], sg), xp[4 * i + 2], g0);
      g1 = dot2_bf16(fp4x2_to_bf16x2_scaled<3>(cg[i], sg), xp[4 * i + 3], g1);
      u0 = dot2_bf16(fp4x2_to_bf16x2_scaled<0>(cu[i], su), xp[4 * i + 0], u0);
      u1 = dot2_bf16(fp4x2_to_bf16x2_scaled<1>(cu[i], su), xp[4 * i + 1], u1);
      u0 = dot2_bf16(fp4x2_to_bf16x2_scaled<2>(cu[i], su), xp[4 * i + 2], u0);
      u1 = dot2_bf16(fp4x2_to_bf16x2_scaled<3>(cu[i], su), xp[4 * i + 3], u1);
    }
    const float gs = wave_sum_to_lane63(g0 + g1), us = wave_sum_to_lane63(u0 + u1);
    if (lane == 63) {
      red[wave][g][0] = gs;
      red[wave][g][1] = us;
    }
  }
  __syncthreads();

  // 5. wavefront 0: SwiGLU of the unit's row for every group, published with
  // write-through stores; then the unit arrives and waits for every unit
  if (wave == 0) {
    if (lane < ng) {
      float gv = 0.0f, uv = 0.0f;
#pragma unroll
      for (int p = 0; p < 4; ++p) {  // the quarters in wavefront order
        gv += red[p][lane][0];
        uv += red[p][lane][1];
      }
      __hip_atomic_store(&a.h[(size_t)lane * kSI + unit], f32_to_bf16(silu_mul_b1(gv, uv)), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the h stores have completed
    handoff_arrive_wait(a.sync, unit, tag, kSSpin);
    if (lane == 0) __hip_atomic_store(&go, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  } else {
    uint32_t it = 0;
    while (__hip_atomic_load(&go, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0u) {
      if (++it > 4 * kSSpin) break;  // wavefront 0 gives up first and raises go regardless
      __builtin_amdgcn_s_sleep(1);
    }
  }
  asm volatile("" ::: "memory");

  // 6. the h of the ng active groups into LDS (plain loads: nothing read h in
  // this launch before every unit had arrived), then the down rows
  const int hpieces = ng * (kSI * 2 / 16);  // 32 pieces of 16 bytes per group
#pragma unroll
  for (int j = 0; j < (kSMaxG * kSI * 2 / 16 + 255) / 256; ++j) {
    const int i = tid + 256 * j;
    if (i < hpieces) ((uint4*)hl)[i] = ((const uint4*)a.h)[i];
  }
  __syncthreads();
  // every group's chunk first, then the 8-lane sums together, so the groups
  // overlap instead of running as a chain
  const int row = 8 * (wave & 1) + (lane >> 3);
  float v[GH];
#pragma unroll
  for (int j = 0; j < GH; ++j) {
    const int g = min(half * GH + j, NB - 1);  // past the batch (odd NB): a copy, never stored
    B1Chunk hq;
    hq.load_lds(hl + (size_t)g * kSI * 2, (size_t)dc * 32);
    float p0 = 0.0f, p1 = 0.0f;
    hq.fp4_acc(wc[j], stab[ws[j]], p0, p1);
    v[j] = p0 + p1;
  }
#pragma unroll
  for (int j = 0; j < GH; ++j) v[j] = group8_sum_dpp(v[j]);
  if (dc == 0) {
#pragma unroll
    for (int j = 0; j < GH; ++j)
      if (half * GH + j < ng) res[half * GH + j][row] = v[j];
  }
  __syncthreads();

  // 7. each output row: routed groups in rank order, then the shared expert
  if (tid < kSRowsDN) {
    float acc = 0.0f;
    for (int g = S0; g < ng; ++g) acc = fmaf(gw[g], res[g][tid], acc);
    if (SH && ng > 0) acc += res[0][tid];
    ((uint16_t*)a.out)[unit * kSRowsDN + tid] = f32_to_bf16(acc);
  }
}

int g_s_cu_count = -1;  // CUs of the current device, read once

template <int NB, bool SH>
void launch_fused_s_nb(const FusedSArgs& a, hipStream_t s) {
  if (!a.logits)
    launch(MOE_PROF_FUSED, (fused_b1s_kernel<NB, 0, SH>), dim3(kSUnits), dim3(256), 0, s, a);
  else if (a.E <= 256)
    launch(MOE_PROF_FUSED, (fused_b1s_kernel<NB, 4, SH>), dim3(kSUnits), dim3(256), 0, s, a);
  else
    launch(MOE_PROF_FUSED, (fused_b1s_kernel<NB, 16, SH>), dim3(kSUnits), dim3(256), 0, s, a);
}

}  // namespace

// The single launch of a 1/8 share: bf16 activations and output, all-FP4
// ranks, up to 8 of them plus the shared expert, on a device whose CUs hold
// every workgroup at once; its sync words are the full-width single launch's
// (the same 256 units and protocol).
bool fused_s_path_ok(const moe_layer* L, int K1, bool xbf16, bool obf16, bool has_prec) {
  if (!xbf16 || !obf16 || has_prec || !(L->flags & MOE_LAYER_SINGLE_LAUNCH)) return false;
  if (!L->shared && (L->num_slots < 1 || !L->fp4_base)) return false;  // loads need a record to point at
  if (L->H != kSH || L->I != kSI || K1 < 1 || K1 > kSMaxG) return false;
  if (g_s_cu_count < 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 0;
    g_s_cu_count = cus;
  }
  return g_s_cu_count >= kSUnits;
}

moe_status launch_fused_b1s(const moe_layer* L, const float* logits, int E, const void* x, int k, int32_t* slot_ids,
                            float* w, uint16_t* h, void* out, uint32_t* sync, hipStream_t s) {
  FusedSArgs a;
  a.k = k;
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
  a.sync = sync;
  const int K1 = k + (L->shared ? 1 : 0);
  const int nb = K1 <= 4 ? 4 : K1 <= 7 ? 7 : 9;
  if (L->shared) {
    if (nb == 4) launch_fused_s_nb<4, true>(a, s);
    else if (nb == 7) launch_fused_s_nb<7, true>(a, s);
    else launch_fused_s_nb<9, true>(a, s);
  } else {
    if (nb == 4) launch_fused_s_nb<4, false>(a, s);
    else if (nb == 7) launch_fused_s_nb<7, false>(a, s);
    else launch_fused_s_nb<9, false>(a, s);
  }
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
