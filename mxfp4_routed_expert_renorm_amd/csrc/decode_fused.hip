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
//     wavefront c (8..15) requests W2 rows 16u+2c', 16u+2c'+1 (c' = c - 8)
//     of every group and their scale bytes into registers.  The routed
//     groups' rows are requested only once every computing wavefront has
//     requested its last gate/up row, so they queue behind the gate/up
//     stream and land while the workgroups hand h over.
//   - Once every unit's h is out, the computing wavefronts copy all of it
//     into LDS (at most 36 KiB, one request per thread and 8 KiB).  The down
//     products then split by group: each copying wavefront dots its two rows
//     of the earlier half of the routed groups and of the shared expert
//     straight from its registers; the computing wavefront of the same
//     index takes the same two rows of the later half, whose W2 chunks the
//     copying wavefronts put in LDS while the units handed h over.  Each
//     sums its groups per lane (weighted, rank order), one reduction per row;
//     the copying wavefront adds the two row sums and the shared expert's
//     (weight 1) and rounds once.  Vector loads retire in issue order, so a
//     wavefront with W2 rows in flight could not use h it requested after
//     them before every row had landed: hence h goes through LDS, loaded by
//     the computing wavefronts, which have nothing in flight by then.
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

constexpr int kFHalf = kFMaxG / 2;       // groups whose down rows the computing wavefronts take

struct alignas(16) FusedSmem {
  uint8_t w2c[kFHalf][kFRowsDN][kW2Row];  // W2 rows of the later groups, for the computing wavefronts
  uint8_t w2s[kFHalf][kFRowsDN][kW2RowS]; // their scale bytes
  uint32_t hb[kFMaxG][kFI / 2];           // every unit's h, bf16 pairs, once the handoff has passed
  float part[kFRowsDN];                   // the computing wavefronts' sums of those groups, per output row
  uint32_t stored;                        // copying wavefronts whose later groups' rows are in LDS
  float hrow[kFMaxG][kFRowsGU];           // SwiGLU outputs of the unit's gate/up rows
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

// A group's h in LDS: lane l's 64 bytes (elements 32l .. 32l+31) as four
// 16-byte pieces, piece i in slot 4l + ((i + r) & 3) with a per-lane rotation
// r, so that the lanes' i-th 16-byte reads fall in different banks (with
// pieces in order, lanes 64 bytes apart would share banks four ways).  The
// rotation is conflict-free for 32 and for 64 banks of 4 bytes.
__device__ __forceinline__ int h_slot(int l, int i) { return 4 * l + ((i + ((l >> 1) ^ (l >> 3))) & 3); }

// one gate/up row of one group: both halves of H, w1 and w3
struct GURow {
  uint4 c1[2], c3[2];
  uint32_t s1[2], s3[2];
};

// one copying wavefront's share of a group's W2: two code rows and, per
// lane, the scale byte of its block in each
struct W2Pair {
  uint4 r0, r1;
  uint32_t s0, s1;
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

  if (tid == 0) {
    sm.issued = 0u;
    sm.go = 0u;
    sm.stored = 0u;
  }
  // groups [S0, GS) and the shared expert: the copying wavefronts, from
  // registers; groups [GS, NB): the computing wavefronts, from LDS
  constexpr int GS = S0 + (NB - S0 + 1) / 2;
  static_assert(NB - GS <= kFHalf, "the later groups' rows fit LDS");
  // one group's W2 chunks of rows 2p, 2p+1 of the unit (codes, lane's block
  // scale) . h of the group, per lane
  auto dot2rows = [&](uint4 c0, uint4 c1, uint32_t s0, uint32_t s1, int g, float& d0, float& d1) {
    B1Chunk hx;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = ((const uint4*)sm.hb[g])[h_slot(lane, i)];
      hx.p[4 * i] = v.x, hx.p[4 * i + 1] = v.y, hx.p[4 * i + 2] = v.z, hx.p[4 * i + 3] = v.w;
    }
    float a0 = 0.0f, a1 = 0.0f, b0 = 0.0f, b1 = 0.0f;
    hx.fp4_acc(c0, e8m0_to_f32(s0), a0, a1);
    hx.fp4_acc(c1, e8m0_to_f32(s1), b0, b1);
    d0 = a0 + a1;
    d1 = b0 + b1;
  };
  // wavefront 0 raises go once every unit's h is out (or its wait gave up)
  auto wait_go = [&]() {
    uint32_t it = 0;
    while (__hip_atomic_load(&sm.go, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0u) {
      if (++it > 4 * kFSpin) break;
      __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
  };

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

    // 5. once every unit's h is out: this workgroup's copy of it, into LDS
    // (36 KiB at most, one request per thread and 8 KiB)
    wait_go();
    {
      // every piece requested before the first is stored: one trip, where a
      // load-store loop waits for each piece in turn.  The index is clamped,
      // not branched on, so the requests stay in flight together; lanes past
      // the end load and store the last piece again (the same bytes)
      constexpr int kStride = 64 * kFCompute, kPer = (NB * (kFI / 8) + kStride - 1) / kStride;
      const int last = ng * (kFI / 8) - 1;
      if (last >= 0) {
        uint4 v[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) v[j] = ((const uint4*)a.h)[min(tid + j * kStride, last)];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const int q = min(tid + j * kStride, last);  // group q / 256, piece q % 256 of it
          ((uint4*)sm.hb)[(q & ~255) + h_slot((q & 255) >> 2, q & 3)] = v[j];
        }
      }
    }
    lds_barrier();  // B2: h is in LDS

    // 6. output rows 2w, 2w+1 of the unit over the later groups [GS, ng),
    // their W2 chunks from LDS, stored by the copying wavefronts while the
    // units handed h over; the two row sums meet the copying wavefronts'
    // in LDS
    {
      uint32_t it = 0;
      while (__hip_atomic_load(&sm.stored, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < (uint32_t)kFCopiers) {
        if (++it > 4 * kFSpin) {
          if (lane == 0) atomicOr(a.err, 2u);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      asm volatile("" ::: "memory");
    }
    float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
    for (int g = GS; g < NB; ++g) {
      if (g < ng) {
        const int q = g - GS, r0 = 2 * wave;
        const uint4 c0 = *(const uint4*)(sm.w2c[q][r0] + lane * 16);
        const uint4 c1 = *(const uint4*)(sm.w2c[q][r0 + 1] + lane * 16);
        float d0, d1;
        dot2rows(c0, c1, sm.w2s[q][r0][lane], sm.w2s[q][r0 + 1][lane], g, d0, d1);
        acc0 = fmaf(sm.gw[g], d0, acc0);
        acc1 = fmaf(sm.gw[g], d1, acc1);
      }
    }
    acc0 = wave_sum_to_lane63(acc0);
    acc1 = wave_sum_to_lane63(acc1);
    if (lane == 63) {
      sm.part[2 * wave] = acc0;
      sm.part[2 * wave + 1] = acc1;
    }
    lds_barrier();  // B3: the later groups' sums are in LDS

  } else {
    // ------------------------------------------------- copying wavefronts
    const int cw = wave - kFCompute;
    const size_t drow = (size_t)unit * kFRowsDN + 2 * cw;  // first of this wavefront's two W2 rows
    auto issue_w2 = [&](W2Pair& p, const uint8_t* rec) {
      p.r0 = ld_stream16(rec + L.w2c + drow * kW2Row + lane * 16);
      p.r1 = ld_stream16(rec + L.w2c + (drow + 1) * kW2Row + lane * 16);
      p.s0 = rec[L.w2s + drow * kW2RowS + lane];
      p.s1 = rec[L.w2s + (drow + 1) * kW2RowS + lane];
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
    // the later groups' rows into LDS for the computing wavefronts (the last
    // requested, so this waits for every row: they land while the units hand
    // h over)
#pragma unroll
    for (int g = GS; g < NB; ++g) {
      const int q = g - GS;
      *(uint4*)(sm.w2c[q][2 * cw] + lane * 16) = wp[g].r0;
      *(uint4*)(sm.w2c[q][2 * cw + 1] + lane * 16) = wp[g].r1;
      sm.w2s[q][2 * cw][lane] = (uint8_t)wp[g].s0;
      sm.w2s[q][2 * cw + 1][lane] = (uint8_t)wp[g].s1;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (lane == 0) atomicAdd(&sm.stored, 1u);

    // 5. once every unit's h is out (step 4 of the computing wavefronts) and
    // in this workgroup's LDS: the wavefront's two output rows over the
    // earlier groups [S0, GS) (weighted, rank order) and the shared expert
    // (weight 1), summed per lane from the W2 registers requested above;
    // then the computing wavefronts' sums of the later groups, one rounding
    wait_go();
    lds_barrier();  // B2: h is in LDS
    float acc0 = 0.0f, acc1 = 0.0f, sh0 = 0.0f, sh1 = 0.0f;
#pragma unroll
    for (int g = S0; g < GS; ++g) {
      if (g < ng) {
        float d0, d1;
        dot2rows(wp[g].r0, wp[g].r1, wp[g].s0, wp[g].s1, g, d0, d1);
        acc0 = fmaf(sm.gw[g], d0, acc0);
        acc1 = fmaf(sm.gw[g], d1, acc1);
      }
    }
    if (SH && ng > 0) dot2rows(wp[0].r0, wp[0].r1, wp[0].s0, wp[0].s1, 0, sh0, sh1);
    acc0 = wave_sum_to_lane63(acc0);
    acc1 = wave_sum_to_lane63(acc1);
    sh0 = wave_sum_to_lane63(sh0);
    sh1 = wave_sum_to_lane63(sh1);
    lds_barrier();  // B3: the later groups' sums are in LDS
    if (lane == 63) {
      ((uint16_t*)a.out)[drow] = f32_to_bf16((acc0 + sm.part[2 * cw]) + sh0);
      ((uint16_t*)a.out)[drow + 1] = f32_to_bf16((acc1 + sm.part[2 * cw + 1]) + sh1);
    }
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
