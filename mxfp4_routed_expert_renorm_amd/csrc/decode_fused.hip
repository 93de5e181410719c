// Fused batch-1 decode step: routing, gate/up GEMV + SwiGLU, down GEMV and
// the weighted combine of one token in ONE launch, for the model shape of the
// pages (hidden 4096, expert intermediate 2048, up to 8 FP4 ranks plus the
// shared expert: "An elephant through a straw", opening section and §Rig,
// model & methodology).
//
// Why one launch.  At batch 1 a token's experts are a pure stream of bytes
// (same page, §The number).  With two launches (gate/up, then down) the
// stream stops at the kernel boundary and while the down kernel's first
// requests travel.  Here every workgroup requests its share of the down
// weights (W2) while it still works on gate/up, so HBM keeps streaming; only
// the SwiGLU outputs h cross workgroups.
//
// Work split: 256 workgroups of 16 wavefronts, one workgroup per CU.
//   - Gate/up unit u: rows 8u..8u+7 of w1 and w3 for every group (group 0 is
//     the shared expert when there is one, then the valid FP4 ranks in rank
//     order).  Computing wavefront w (0..7) takes row 8u+w over all of H,
//     with a few groups' rows in flight at a time, and leaves each group's
//     SwiGLU output in LDS; wavefront 0 then publishes the unit's h with
//     write-through stores and arrives at the handoff below.
//   - Down unit u: output rows 16u..16u+15 for every group.  Copying
//     wavefront c (8..15) loads W2 rows 16u+2c', 16u+2c'+1 (c' = c - 8) of
//     every group and their scale bytes into registers, then moves each
//     group's pair into LDS as it lands and raises a flag there.  The routed
//     groups' rows are requested only once every computing wavefront has
//     requested its last gate/up row, so they queue behind the gate/up
//     stream and land while the workgroups hand h over.
//   - The computing wavefronts then wait until every gate/up unit is done,
//     load h for the (at most two) groups of their down items, and compute
//     each item (one group's W2 row dotted with its h) once its rows are in
//     LDS, overlapping the tail of the W2 stream.  Vector loads retire in
//     issue order, so a wavefront with W2 rows in flight could not use h
//     loaded after them before every row landed: hence the copying and the
//     computing wavefronts are distinct.
//   - The items' results meet in LDS; 16 threads sum each output row over the
//     groups in rank order (shared expert last, weight 1) and round once.
//
// Cross-workgroup handoff.  h is written with agent-scope stores, which write
// through to the device's coherence point; once they have completed (vmcnt 0,
// and the storing wavefront has no other memory operation in flight) the
// unit arrives: its launch tag, then two levels of arrival counters (eight
// groups of 32 units, then one word), all with agent-scope atomics.  A
// reader polls that one word with agent-scope loads and only then reads h
// with ordinary loads; no workgroup reads h before every unit has arrived,
// and a launch starts with invalidated caches, so no stale copy of h can be
// hit.  A unit's tag is its own tag word plus one, since only that unit
// writes it.  Nothing is reset between launches, so the sync words must start
// at zero (a zeroed workspace) and launches that share them must not overlap.
//
// Every workgroup must be resident at once: the host launches this kernel
// only on a device with at least 256 CUs.  Waits are bounded; a wait that
// gives up sets an error word and the launch finishes (its output is then
// meaningless) instead of hanging.
#include "common.h"
#include "route_dev.h"
#include "b1_dev.h"
#include "handoff_dev.h"

namespace moe {

namespace {

constexpr int kFH = 4096, kFI = 2048;
constexpr int kFUnits = kHandoffUnits;   // gate/up units = down units = workgroups
constexpr int kFRowsGU = kFI / kFUnits;  // 8 gate/up rows per unit
constexpr int kFRowsDN = kFH / kFUnits;  // 16 down rows per unit
constexpr int kFWaves = 16, kFThreads = 64 * kFWaves;
constexpr int kFCompute = 8;             // wavefronts 0..7 compute down items, 8..15 copy W2
constexpr int kFMaxG = 9;                // shared expert + 8 ranks
constexpr int kFCopiers = kFWaves - kFCompute;
constexpr int kW2Row = kFI / 2;                     // code bytes of a W2 row
constexpr int kW2RowS = kFI / 32;                   // scale bytes of a W2 row
constexpr int kW2Scales = kFRowsDN * kW2RowS;       // scale bytes of a unit's 16 W2 rows
constexpr uint32_t kFSpin = 1u << 21;    // poll rounds before a wait gives up
#ifndef MOE_FUSED_WIN
#define MOE_FUSED_WIN 3  // gate/up rows in flight per computing wavefront
#endif

static_assert(kFRowsGU == kFCompute, "a computing wavefront per gate/up row");
static_assert(kFRowsDN == 2 * kFCopiers, "a copying wavefront per pair of W2 rows");
static_assert(kW2Row == 64 * 16 && 2 * kW2RowS == 64 * 2, "a row: 16 bytes per lane; a row pair's scales: 2");

struct FusedArgs {
  int k, E;
  const uint8_t* fp4_base;
  size_t fp4_stride;
  int num_slots;
  const uint8_t* shared;
  const float* logits;  // [E]: the kernel routes the token; null: slot_ids and w are inputs
  const void* x;        // [kFH] bf16
  int32_t* slot_ids;    // [k]
  float* w;             // [k]
  uint32_t* h;          // [kFMaxG][kFI] bf16, group-major, as bf16 pairs
  void* out;            // [kFH] bf16
  uint32_t* sync;       // the handoff's words, kept between launches
  uint32_t* err;        // its error word: bit 0 the handoff gave up, bit 1 a W2 wait did
};

struct alignas(16) FusedSmem {
  uint8_t w2c[kFMaxG][kFRowsDN][kW2Row];  // W2 code rows of the unit, per group
  uint8_t w2s[kFMaxG][kW2Scales];         // their scale bytes
  float hrow[kFMaxG][kFRowsGU];           // SwiGLU outputs of the unit's gate/up rows
  float res[kFMaxG][kFRowsDN];            // down items: group g's W2 row r . h_g
  uint32_t ready[kFMaxG][kFCopiers];      // group g's W2 row pair c is in LDS
  int gslot[kFMaxG];                      // slot of each routed group
  float gw[kFMaxG];                       // weight of each routed group
  int ng;                                 // groups with work
  uint32_t issued;                        // computing wavefronts that issued their last gate/up row
  uint32_t go;                            // every gate/up unit is done
};

// workgroup barrier that orders LDS only: a fenced __syncthreads would also
// wait for every global load in flight
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// the record a batch slot g reads: group g, or past the active groups the
// last one (its loads are issued but never used).  Built from the kernel's
// own global pointers, so the loads stay global (not flat) loads.
__device__ __forceinline__ const uint8_t* group_record(const FusedArgs& a, const FusedSmem& sm, int g, int ng,
                                                       int S0) {
  if (ng == 0) return a.fp4_base;
  g = min(g, ng - 1);
  if (g < S0) return a.shared;
  return a.fp4_base + (size_t)sm.gslot[g] * a.fp4_stride;
}

// one gate/up row of one group: both halves of H, w1 and w3
struct GURow {
  uint4 c1[2], c3[2];
  uint32_t s1[2], s3[2];
};

// one copying wavefront's share of a group's W2: two code rows and their
// 128 scale bytes (two per lane)
struct W2Pair {
  uint4 r0, r1;
  uint32_t s;
};

template <int NB, int EPL, bool SH, int WIN>
__global__ __launch_bounds__(kFThreads, 1) void fused_b1_kernel(FusedArgs a) {
  __shared__ FusedSmem sm;
  constexpr int S0 = SH ? 1 : 0;
  static_assert(NB <= kFMaxG && NB > S0, "groups of the batch");
  static_assert(WIN >= 1 && WIN <= NB, "gate/up rows in flight per wavefront");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int unit = blockIdx.x;
  const RecordLayout L = record_layout(kFH, kFI, 4);
  constexpr size_t kRowB = kFH / 2, kRowS = kFH / 32;  // w1/w3 row: code bytes, scale bytes

  if (tid < kFMaxG * kFCopiers) (&sm.ready[0][0])[tid] = 0u;
  if (tid == 0) {
    sm.issued = 0u;
    sm.go = 0u;
  }

  if (wave < kFCompute) {
    // ------------------------------------------------ computing wavefronts
    const int row = unit * kFRowsGU + wave;  // this wavefront's gate/up row (full H)
    auto issue_gu = [&](GURow& s, const uint8_t* rec) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const size_t c = (size_t)(q * 64 + lane);
        s.c1[q] = ld_stream16(rec + L.w1c + (size_t)row * kRowB + c * 16);
        s.c3[q] = ld_stream16(rec + L.w3c + (size_t)row * kRowB + c * 16);
        s.s1[q] = rec[L.w1s + (size_t)row * kRowS + c];
        s.s3[q] = rec[L.w3s + (size_t)row * kRowS + c];
      }
    };
    // this launch's tag (wavefront 0 arrives and waits with it)
    const uint32_t tag = handoff_tag(a.sync, unit);
    // 1. the activation, the routing inputs (wavefront 0), the shared
    // expert's row: none of it needs the routing
    B1Chunk x0, x1;
    x0.load_global(a.x, (size_t)lane * 32);
    x1.load_global(a.x, (size_t)(64 + lane) * 32);
    float lv[EPL > 0 ? EPL : 1];
    int my_slot = -1;
    float my_w = 0.0f;
    if constexpr (EPL > 0) {
      route_load<EPL>(a.logits, a.E, lv);
    } else {
      const int l = min(lane, a.k - 1);  // unconditional loads: fixed count in flight
      my_slot = a.slot_ids[l];
      my_w = a.w[l];
    }
    __builtin_amdgcn_sched_barrier(0);
    GURow ring[WIN];
    if constexpr (SH) issue_gu(ring[0], a.shared);
    __builtin_amdgcn_sched_barrier(0);

    // 2. wavefront 0 routes the token and lists the groups
    if (wave == 0) {
      if constexpr (EPL > 0) route_select<EPL>(lv, a.E, a.k, &my_slot, &my_w);
      const bool valid = lane < a.k && my_slot >= 0 && my_slot < a.num_slots;
      const uint64_t m = __ballot(valid);
      const int ng = S0 + __popcll(m);
      if (lane == 0) sm.ng = ng;
      // lane r < k: the r-th valid rank's group is S0 + (valid ranks before r)
      const int g = S0 + __popcll(m & ((1ull << lane) - 1ull));
      if (valid) {
        sm.gslot[g] = my_slot;
        sm.gw[g] = my_w;
      }
      if (EPL > 0 && unit == 0 && lane < a.k) {  // the routing result, for the caller
        a.slot_ids[lane] = my_slot;
        a.w[lane] = my_w;
      }
    }
    lds_barrier();  // B0: groups listed
    const int ng = sm.ng;
    auto issue_rec = [&](int g) { return group_record(a, sm, g, ng, S0); };

    // 3. gate/up rows of the groups, WIN in flight; each row's SwiGLU output
    // goes to LDS.  Every batch slot is issued (past the active groups: the
    // last one again, never stored), so the loads in flight are counted
    // exactly by the compiler
#pragma unroll
    for (int g = S0; g < WIN; ++g) issue_gu(ring[g], issue_rec(g));
    if (WIN >= NB && lane == 0) atomicAdd(&sm.issued, 1u);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < NB; ++g) {
      GURow& r = ring[g % WIN];
      float g0 = 0.0f, g1 = 0.0f, u0 = 0.0f, u1 = 0.0f;
      x0.fp4_acc(r.c1[0], e8m0_to_f32(r.s1[0]), g0, g1);
      x1.fp4_acc(r.c1[1], e8m0_to_f32(r.s1[1]), g0, g1);
      x0.fp4_acc(r.c3[0], e8m0_to_f32(r.s3[0]), u0, u1);
      x1.fp4_acc(r.c3[1], e8m0_to_f32(r.s3[1]), u0, u1);
      if (g + WIN < NB) {
        issue_gu(r, issue_rec(g + WIN));
        if (g + WIN == NB - 1 && lane == 0) atomicAdd(&sm.issued, 1u);
      }
      __builtin_amdgcn_sched_barrier(0);
      const float gs = wave_sum_to_lane63(g0 + g1);
      const float us = wave_sum_to_lane63(u0 + u1);
      if (lane == 63 && g < ng) sm.hrow[g][wave] = silu_mul_b1(gs, us);
    }
    lds_barrier();  // B1: the unit's SwiGLU outputs are in LDS

    // 4. wavefront 0 publishes the unit's h (bf16 pairs, write-through),
    // then arrives and waits for every unit
    if (wave == 0) {
      if (lane < 4 * ng) {
        const int g = lane >> 2, p = lane & 3;
        const uint32_t pk = (uint32_t)f32_to_bf16(sm.hrow[g][2 * p]) |
                            ((uint32_t)f32_to_bf16(sm.hrow[g][2 * p + 1]) << 16);
        __hip_atomic_store(&a.h[((size_t)g * kFI + (size_t)unit * kFRowsGU + 2 * p) / 2], pk, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the h stores have completed
      handoff_arrive_wait(a.sync, unit, tag, kFSpin);
      if (lane == 0) __hip_atomic_store(&sm.go, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }

  } else {
    // ------------------------------------------------- copying wavefronts
    const int cw = wave - kFCompute;
    const size_t drow = (size_t)unit * kFRowsDN + 2 * cw;  // first of this wavefront's two W2 rows
    auto issue_w2 = [&](W2Pair& p, const uint8_t* rec) {
      p.r0 = ld_stream16(rec + L.w2c + drow * kW2Row + lane * 16);
      p.r1 = ld_stream16(rec + L.w2c + (drow + 1) * kW2Row + lane * 16);
      p.s = *(const uint16_t*)(rec + L.w2s + drow * kW2RowS + lane * 2);
    };
    auto store_w2 = [&](const W2Pair& p, int g) {
      *(uint4*)(sm.w2c[g][2 * cw] + lane * 16) = p.r0;
      *(uint4*)(sm.w2c[g][2 * cw + 1] + lane * 16) = p.r1;
      *(uint16_t*)(sm.w2s[g] + 2 * cw * kW2RowS + lane * 2) = (uint16_t)p.s;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (lane == 0) __hip_atomic_store(&sm.ready[g][cw], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    W2Pair wp[NB];
    // the shared expert's rows need no routing
    if constexpr (SH) issue_w2(wp[0], a.shared);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();  // B0
    const int ng = sm.ng;
    auto issue_rec = [&](int g) { return group_record(a, sm, g, ng, S0); };
    // the routed groups' rows go out once every computing wavefront has
    // issued its last gate/up row, so they queue behind the gate/up stream
    {
      uint32_t it = 0;
      while (__hip_atomic_load(&sm.issued, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < (uint32_t)kFCompute) {
        if (++it > 4 * kFSpin) break;
        __builtin_amdgcn_s_sleep(1);
      }
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int g = S0; g < NB; ++g) issue_w2(wp[g], issue_rec(g));
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();  // B1
    // each group's rows into LDS as they land
#pragma unroll
    for (int g = 0; g < NB; ++g) store_w2(wp[g], g);
  }

  // 5. every wavefront: once every unit's h is out, ng consecutive down items
  // (group-major (group, row) pairs, at most two groups), each one group's W2
  // row dotted with its h.  The copying wavefronts have moved all their rows
  // into LDS by now, so h is the only load in flight for any wavefront here.
  // The rows of all the wavefront's items are read first and reduced
  // together, so the items overlap instead of running as a chain.
  {
    uint32_t it = 0;
    while (__hip_atomic_load(&sm.go, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0u) {
      if (++it > 4 * kFSpin) break;  // wavefront 0 gives up first and raises go regardless
      __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
    const int ng = sm.ng, n = ng;
    if (n > 0) {
      const int i0 = n * wave;
      const int glo = i0 / kFRowsDN, ghi = (i0 + n - 1) / kFRowsDN;
      B1Chunk hlo, hhi;
      hlo.load_global(a.h, (size_t)glo * kFI + (size_t)lane * 32);
      hhi.load_global(a.h, (size_t)ghi * kFI + (size_t)lane * 32);
      // items of group glo first, then those of ghi: each loop reads one
      // activation chunk (a per-item choice between the two would copy it)
      const int nlo = min(n, (glo + 1) * kFRowsDN - i0);
      float v[kFMaxG];
      auto item_dot = [&](const B1Chunk& hx, int i) {
        const int item = i0 + i, g = item / kFRowsDN, r = item % kFRowsDN;
        if (i % 3 == 0) {  // wait for this batch of three items' rows
#pragma unroll
          for (int j = i; j < i + 3 && j < kFMaxG; ++j) {
            const int jt = i0 + min(j, n - 1), gj = jt / kFRowsDN, rj = jt % kFRowsDN;
            uint32_t it2 = 0;
            while (__hip_atomic_load(&sm.ready[gj][rj / 2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0u) {
              if (++it2 > 4 * kFSpin) {
                if (lane == 0) atomicOr(a.err, 2u);
                break;
              }
              __builtin_amdgcn_s_sleep(1);
            }
          }
          asm volatile("" ::: "memory");
        }
        const uint4 c = *(const uint4*)(sm.w2c[g][r] + lane * 16);
        const float sc = e8m0_to_f32(sm.w2s[g][r * kW2RowS + lane]);
        float p0 = 0.0f, p1 = 0.0f;
        hx.fp4_acc(c, sc, p0, p1);
        return p0 + p1;
      };
#pragma unroll
      for (int i = 0; i < kFMaxG; ++i) v[i] = i < nlo ? item_dot(hlo, i) : 0.0f;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < kFMaxG; ++i)
        if (i >= nlo && i < n) v[i] = item_dot(hhi, i);
#pragma unroll
      for (int i = 0; i < kFMaxG; ++i) v[i] = wave_sum_to_lane63(v[i]);
      if (lane == 63) {
#pragma unroll
        for (int i = 0; i < kFMaxG; ++i) {
          const int item = i0 + i;
          if (i < n) sm.res[item / kFRowsDN][item % kFRowsDN] = v[i];
        }
      }
    }
  }
  lds_barrier();  // B2: every item's result is in LDS

  // 6. each output row: routed groups in rank order, then the shared expert
  if (tid < kFRowsDN) {
    const int ng = sm.ng;
    float acc = 0.0f;
    for (int g = S0; g < ng; ++g) acc = fmaf(sm.gw[g], sm.res[g][tid], acc);
    if (SH && ng > 0) acc += sm.res[0][tid];
    ((uint16_t*)a.out)[unit * kFRowsDN + tid] = f32_to_bf16(acc);
  }
}


int g_cu_count = -1;  // CUs of the current device, read once

template <int NB, bool SH>
void launch_fused_nb(const FusedArgs& a, hipStream_t s) {
  if (!a.logits)
    launch(MOE_PROF_FUSED, (fused_b1_kernel<NB, 0, SH, (NB < MOE_FUSED_WIN ? NB : MOE_FUSED_WIN)>), dim3(kFUnits), dim3(kFThreads), 0, s, a);
  else if (a.E <= 256)
    launch(MOE_PROF_FUSED, (fused_b1_kernel<NB, 4, SH, (NB < MOE_FUSED_WIN ? NB : MOE_FUSED_WIN)>), dim3(kFUnits), dim3(kFThreads), 0, s, a);
  else
    launch(MOE_PROF_FUSED, (fused_b1_kernel<NB, 16, SH, (NB < MOE_FUSED_WIN ? NB : MOE_FUSED_WIN)>), dim3(kFUnits), dim3(kFThreads), 0, s, a);
}

}  // namespace

// workspace bytes the single-launch steps keep between launches (the
// handoff's tags and counters)
size_t fused_sync_bytes() { return kHandoffSyncBytes; }

// The fused step covers the pages' model shape with bf16 activations and
// output, all-FP4 ranks, up to 8 of them plus the shared expert, on a device
// whose CUs hold every workgroup at once.
bool fused_path_ok(const moe_layer* L, int K1, bool xbf16, bool obf16, bool has_prec) {
  const int H = L->H, I = L->I;
  if (!xbf16 || !obf16 || has_prec || !(L->flags & MOE_LAYER_SINGLE_LAUNCH)) return false;
  if (!L->shared && (L->num_slots < 1 || !L->fp4_base)) return false;  // loads need a record to point at
  if (H != kFH || I != kFI || K1 < 1 || K1 > kFMaxG) return false;
  if (g_cu_count < 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 0;
    g_cu_count = cus;
  }
  return g_cu_count >= kFUnits;
}

moe_status launch_fused_b1(const moe_layer* L, const float* logits, int E, const void* x, int k, int32_t* slot_ids,
                           float* w, uint16_t* h, void* out, uint32_t* sync, hipStream_t s) {
  FusedArgs a;
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
  a.h = (uint32_t*)h;
  a.out = out;
  a.sync = sync;
  a.err = sync + kSyncErr;
  const int K1 = k + (L->shared ? 1 : 0);
  const int nb = K1 <= 4 ? 4 : K1 <= 7 ? 7 : 9;
  if (L->shared) {
    if (nb == 4) launch_fused_nb<4, true>(a, s);
    else if (nb == 7) launch_fused_nb<7, true>(a, s);
    else launch_fused_nb<9, true>(a, s);
  } else {
    if (nb == 4) launch_fused_nb<4, false>(a, s);
    else if (nb == 7) launch_fused_nb<7, false>(a, s);
    else launch_fused_nb<9, false>(a, s);
  }
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
