// Slot cache with the (a,b) precision ladder: host policy and miss copies.
//
// "Running DeepSeek-V4-Flash across four free GPUs", §What the expert cache
// actually does: the expert banks live in pinned host memory; a fixed number
// of expert slots in device memory is shared by every layer (global, not per
// layer); each step the router's expert ids are rewritten to slots in place
// and only the misses are copied across the host link; eviction is LRU.
// "An elephant through a straw", §Not all six experts matter equally: ranks
// 1..a always use FP4 (fetched on a miss), ranks a+1..b use FP4 if resident
// and the 2-bit copy otherwise, lower ranks are used if resident and dropped
// otherwise, and the survivors' weights are renormalised; §43 graphs, 43
// syncs: one host sync per layer reads the router's picks.
//
// "An elephant through a straw", §Rig, model & methodology (best
// configuration): a small device tier for the 2-bit copies beside the FP4
// slots, and LFU eviction with frequency decay seeded from a routing trace.
//
// Policy details the pages leave open (same as the oracle): residency is read
// once per token before its fetches, and only FP4 residency classifies; slots
// used anywhere in the call are protected from eviction for the rest of the
// call (in each tier); fetches go in rank order; a global clock stamps every
// use; the victim is the lowest-index empty slot, else the unprotected slot
// with the oldest stamp (LRU) or whose pair has the lowest use count, ties to
// the oldest stamp (LFU).  LFU counts belong to pairs: each call multiplies
// them all by the decay, each use adds one (double precision, the same
// operations in the same order as the oracle, so victims match exactly).
// Without a 2-bit tier, 2-bit copies are copied per use into a staging area
// at index t*(b-a) + (rank-a-1).
//
// "An elephant through a straw", §Guessing the router two layers ahead:
// speculative copies of predicted experts land in a small staging ring after
// the slots, filled round-robin, so a wrong guess never evicts a resident
// expert.  Readings: a
// ring entry counts as FP4-resident for classification; a call uses it in
// place (slot S + entry, its LFU count grows, it takes no stamp and is not
// moved into the cache); a prefetch skips the entries the last call used and
// those it filled itself, and stops when no entry is free.
//
// "Running DeepSeek-V4-Flash across four free GPUs", §What the expert cache
// actually does and §Step 7: above the crossover T*k >= E prefill streams
// whole expert layers into two expert-layer buffers lent by the cache (so it
// needs 2E slots).  Readings: the buffers are slots [0, E) and [E, 2E), filled
// alternately; expert e lands in slot bE + e, evicting that slot's pair; the
// layer's pairs held elsewhere (a slot or the ring) give that place up; pairs
// already in place are not copied; each streamed slot takes the next clock
// stamp, with no LFU use; the streamed experts stay resident.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "common.h"

struct moe_cache {
  moe_cache_desc d;
  size_t fp4_bytes = 0, int2_bytes = 0;
  std::vector<int32_t> map;      // (layer, expert) -> slot or -1
  std::vector<int32_t> owner;    // slot -> pair or -1
  std::vector<int64_t> stamp;    // 0 = empty
  std::vector<int32_t> map2, owner2;  // the 2-bit tier, as map / owner
  std::vector<int64_t> stamp2;
  std::vector<double> count, seed;    // LFU use counts per pair, and their initial values
  std::vector<int32_t> ring_owner, map_ring;  // staging ring: entry -> pair, pair -> entry
  std::vector<uint8_t> ring_used, ring_now;   // entries the last call used / this call uses
  int cursor = 0;
  bool prefetch_pending = false;
  hipEvent_t ev_prefetch = nullptr;
  int next_buf = 0;                    // the layer buffer the next moe_cache_stream_layer fills
  bool stream_pending[2] = {false, false};
  hipEvent_t ev_stream[2] = {nullptr, nullptr}, ev_compute = nullptr;
  int64_t clock = 0;
  moe_cache_stats st{};
  // per-call scratch
  std::vector<int32_t> ids_h, slots_h;
  std::vector<int8_t> prec_h;
  std::vector<float> w_h, wout_h;
  std::vector<uint8_t> prot, prot2;
  struct Copy {
    int kind;  // 0 FP4, 1 2-bit
    int pair, dest;
  };
  std::vector<Copy> copies;
  // device-side plumbing (created on first ensure)
  void* pin_in = nullptr;   // pinned, mapped: ids [T*k] int32, w [T*k] f32, then the sequence word
  uint32_t seq = 0;         // sequence number of the last call's picks
  long long poll_us = 2000000;  // how long the host polls for them before waiting on the event (0: no poll)
  void* pin_out = nullptr;  // pinned, mapped: slots [T*k] int32, w' [T*k] f32, prec [T*k] int8
  void* pin_in_dev = nullptr;   // their device addresses
  void* pin_out_dev = nullptr;
  hipEvent_t ev_read = nullptr, ev_copy = nullptr;
  bool broken = false;
  // the compute stream of every call since creation or the last reset: the
  // host rewrites pin_out, victim slots and ring entries as soon as its own
  // call's kernels are queued, which is safe only behind the previous call's
  // readers, i.e. on the same stream
  hipStream_t compute = nullptr;
  bool compute_set = false;
};

namespace moe {

namespace {

// every call of a cache uses one compute stream (see moe_cache::compute)
moe_status check_compute(moe_cache* c, hipStream_t cs, const char* who) {
  if (c->compute_set && cs != c->compute)
    return fail(MOE_EINVAL,
                "%s: the cache's calls use one compute stream (the first call's) until moe_cache_reset; got another",
                who);
  c->compute = cs;
  c->compute_set = true;
  return MOE_OK;
}

size_t pin_in_bytes(const moe_cache_desc& d) { return (size_t)d.max_tokens * d.k * 8; }
constexpr size_t kFlagBytes = 256;  // after the picks in the mapped input buffer: the call's sequence number
size_t pin_out_bytes(const moe_cache_desc& d) { return (size_t)d.max_tokens * d.k * 9; }

// the lowest-index empty slot not used by this call, else the unprotected slot
// to evict under the cache's rule; -1 when every slot is protected
int victim(const moe_cache* c, const std::vector<int32_t>& owner, const std::vector<int64_t>& stamp,
           const std::vector<uint8_t>& prot) {
  const int n = (int)owner.size();
  for (int s = 0; s < n; ++s)
    if (owner[s] < 0 && !prot[s]) return s;
  int v = -1;
  for (int s = 0; s < n; ++s) {
    if (prot[s]) continue;
    if (v < 0) {
      v = s;
    } else if (c->d.policy == MOE_CACHE_LFU) {
      const double cs = c->count[owner[s]], cv = c->count[owner[v]];
      if (cs < cv || (cs == cv && stamp[s] < stamp[v])) v = s;
    } else if (stamp[s] < stamp[v]) {
      v = s;
    }
  }
  return v;
}

int64_t use(moe_cache* c, int pair) {
  c->count[pair] += 1.0;
  return ++c->clock;
}

// one call of the policy on host arrays; fills c->slots_h, prec_h, wout_h, copies
moe_status plan(moe_cache* c, int layer, int T, const int32_t* ids, const float* w) {
  const moe_cache_desc& d = c->d;
  const int k = d.k, a = d.ladder_a, b = d.ladder_b, E = d.E, S = d.num_slots;
  c->slots_h.assign((size_t)T * k, -1);
  c->prec_h.assign((size_t)T * k, -1);
  c->wout_h.assign((size_t)T * k, 0.0f);
  c->copies.clear();
  c->prot.assign(S, 0);
  c->prot2.assign(c->owner2.size(), 0);
  c->ring_now.assign(c->ring_owner.size(), 0);
  // validate everything before the state changes
  for (int i = 0; i < T * k; ++i)
    if (ids[i] < 0 || ids[i] >= E)
      return fail(MOE_EINVAL, "moe_cache: expert id %d at position %d outside [0, %d)", ids[i], i, E);
  for (int t = 0; t < T; ++t)
    for (int r = 0; r < k; ++r)
      for (int q = 0; q < r; ++q)
        if (ids[(size_t)t * k + q] == ids[(size_t)t * k + r])
          return fail(MOE_EINVAL, "moe_cache: token %d lists expert %d twice", t, ids[(size_t)t * k + r]);
  if (d.policy == MOE_CACHE_LFU)
    for (double& f : c->count) f *= d.lfu_decay;
  for (int t = 0; t < T; ++t) {
    const int32_t* id = ids + (size_t)t * k;
    int cls[64];
    bool res[64];
    for (int r = 0; r < k; ++r) {
      const int rank = r + 1;
      const size_t pr = (size_t)layer * E + id[r];
      res[r] = c->map[pr] >= 0 || (!c->map_ring.empty() && c->map_ring[pr] >= 0);  // snapshot before fetches
      if (rank <= a)
        cls[r] = 0;
      else if (rank <= b)
        cls[r] = res[r] ? 0 : 1;
      else
        cls[r] = res[r] ? 0 : -1;
    }
    for (int r = 0; r < k; ++r)
      if (cls[r] == 0 && res[r] && c->map[(size_t)layer * E + id[r]] >= 0)
        c->prot[c->map[(size_t)layer * E + id[r]]] = 1;
    for (int r = 0; r < k; ++r) {
      const int pair = layer * E + id[r];
      const size_t o = (size_t)t * k + r;
      if (cls[r] == 0 && res[r] && c->map[pair] < 0) {  // in the staging ring: used in place
        const int q = c->map_ring[pair];
        c->count[pair] += 1.0;
        c->ring_now[q] = 1;
        c->slots_h[o] = S + q;
        c->prec_h[o] = 0;
        c->st.ring_hits++;
      } else if (cls[r] == 0 && res[r]) {
        const int s = c->map[pair];
        c->stamp[s] = use(c, pair);
        c->slots_h[o] = s;
        c->prec_h[o] = 0;
        c->st.hits++;
      } else if (cls[r] == 0) {
        const int v = victim(c, c->owner, c->stamp, c->prot);
        if (v < 0) return fail(MOE_ECACHE_SMALL, "moe_cache: every slot is in use by this call");
        if (c->owner[v] >= 0) {
          c->map[c->owner[v]] = -1;
          c->st.evictions++;
        }
        c->owner[v] = pair;
        c->map[pair] = v;
        c->stamp[v] = use(c, pair);
        c->prot[v] = 1;
        c->slots_h[o] = v;
        c->prec_h[o] = 0;
        c->copies.push_back({0, pair, v});
        c->st.misses++;
      } else if (cls[r] == 1 && d.int2_slots == 0) {
        const int st = t * (b - a) + (r + 1 - a - 1);
        use(c, pair);
        c->slots_h[o] = st;
        c->prec_h[o] = 1;
        c->copies.push_back({1, pair, st});
        c->st.int2_uses++;
      } else if (cls[r] == 1) {
        int v = c->map2[pair];
        if (v >= 0) {
          c->st.int2_hits++;
        } else {
          v = victim(c, c->owner2, c->stamp2, c->prot2);
          if (v < 0) return fail(MOE_ECACHE_SMALL, "moe_cache: every 2-bit slot is in use by this call");
          if (c->owner2[v] >= 0) c->map2[c->owner2[v]] = -1;
          c->owner2[v] = pair;
          c->map2[pair] = v;
          c->copies.push_back({1, pair, v});
        }
        c->stamp2[v] = use(c, pair);
        c->prot2[v] = 1;
        c->slots_h[o] = v;
        c->prec_h[o] = 1;
        c->st.int2_uses++;
      } else {
        c->st.drops++;
      }
    }
    double tot = 0.0;
    for (int r = 0; r < k; ++r)
      if (c->prec_h[(size_t)t * k + r] >= 0) tot += (double)w[(size_t)t * k + r];
    if (tot > 0.0)
      for (int r = 0; r < k; ++r)
        if (c->prec_h[(size_t)t * k + r] >= 0)
          c->wout_h[(size_t)t * k + r] = (float)((double)w[(size_t)t * k + r] / tot);
  }
  c->ring_used.swap(c->ring_now);
  c->st.calls++;
  return MOE_OK;
}

// the staging-ring half of a prefetch: fills c->copies (kind 0, dest = slot)
// the policy half of a layer stream: fills c->copies (kind 0, dest = slot), returns the buffer
int plan_stream(moe_cache* c, int layer) {
  const int E = c->d.E;
  const int b = c->next_buf;
  c->next_buf ^= 1;
  c->copies.clear();
  for (int e = 0; e < E; ++e) {
    const int s = b * E + e, pair = layer * E + e;
    if (c->owner[s] != pair) {
      if (c->owner[s] >= 0) {
        c->map[c->owner[s]] = -1;
        c->st.evictions++;
      }
      const int old = c->map[pair];
      if (old >= 0) {
        c->owner[old] = -1;
        c->stamp[old] = 0;
      }
      if (!c->map_ring.empty() && c->map_ring[pair] >= 0) {
        c->ring_owner[c->map_ring[pair]] = -1;
        c->map_ring[pair] = -1;
      }
      c->owner[s] = pair;
      c->map[pair] = s;
      c->copies.push_back({0, pair, s});
      c->st.streamed++;
    }
    c->stamp[s] = ++c->clock;
  }
  return b;
}

moe_status plan_prefetch(moe_cache* c, int layer, int n, const int32_t* experts) {
  const int E = c->d.E, S = c->d.num_slots, R = c->d.prefetch_slots;
  c->copies.clear();
  for (int i = 0; i < n; ++i)
    if (experts[i] < 0 || experts[i] >= E)
      return fail(MOE_EINVAL, "moe_cache_prefetch: expert id %d at position %d outside [0, %d)", experts[i], i, E);
  std::vector<uint8_t> filled(R, 0);
  for (int i = 0; i < n; ++i) {
    const int pair = layer * E + experts[i];
    if (c->map[pair] >= 0 || c->map_ring[pair] >= 0) continue;
    int q = -1;
    for (int j = 0; j < R; ++j) {
      const int cand = (c->cursor + j) % R;
      if (!c->ring_used[cand] && !filled[cand]) {
        q = cand;
        break;
      }
    }
    if (q < 0) break;
    if (c->ring_owner[q] >= 0) c->map_ring[c->ring_owner[q]] = -1;
    c->ring_owner[q] = pair;
    c->map_ring[pair] = q;
    c->cursor = (q + 1) % R;
    filled[q] = 1;
    c->copies.push_back({0, pair, S + q});
    c->st.prefetches++;
  }
  return MOE_OK;
}

moe_status check_call(const moe_cache* c, int layer, int T) {
  if (!c) return fail(MOE_EINVAL, "moe_cache: handle is NULL");
  if (c->broken) return fail(MOE_ESTATE, "moe_cache: an earlier ensure failed midway; reset the cache");
  if (layer < 0 || layer >= c->d.L) return fail(MOE_EINVAL, "moe_cache: layer %d outside [0, %d)", layer, c->d.L);
  if (T < 1 || T > c->d.max_tokens)
    return fail(MOE_ESHAPE, "moe_cache: T=%d outside [1, max_tokens=%d]", T, c->d.max_tokens);
  return MOE_OK;
}

}  // namespace

}  // namespace moe

using namespace moe;

extern "C" {

moe_status moe_pinned_alloc(size_t bytes, void** out) {
  if (!out || bytes == 0) return fail(MOE_EINVAL, "moe_pinned_alloc: bytes=%zu out=%p", bytes, (void*)out);
  *out = nullptr;
  hipError_t e = hipHostMalloc(out, bytes, hipHostMallocDefault);
  if (e != hipSuccess) {
    *out = nullptr;
    return fail(MOE_ENOMEM, "moe_pinned_alloc: hipHostMalloc(%zu) failed: %s", bytes, hipGetErrorString(e));
  }
  return MOE_OK;
}

moe_status moe_pinned_free(void* p) {
  if (!p) return MOE_OK;
  hipError_t e = hipHostFree(p);
  if (e != hipSuccess) return fail(MOE_EHIP, "moe_pinned_free: %s", hipGetErrorString(e));
  return MOE_OK;
}

moe_status moe_cache_create(const moe_cache_desc* d, moe_cache** out) {
  if (!d || !out) return fail(MOE_EINVAL, "moe_cache_create: NULL argument");
  *out = nullptr;
  if (d->L < 1 || d->E < 1 || d->E > 1024) return fail(MOE_ESHAPE, "moe_cache_create: L=%d E=%d", d->L, d->E);
  if (d->k < 1 || d->k > 64 || d->k > d->E) return fail(MOE_EINVAL, "moe_cache_create: k=%d (E=%d)", d->k, d->E);
  if (d->ladder_a < 0 || d->ladder_a > d->ladder_b || d->ladder_b > d->k)
    return fail(MOE_EINVAL, "moe_cache_create: ladder (a=%d, b=%d) must satisfy 0 <= a <= b <= k=%d", d->ladder_a,
                d->ladder_b, d->k);
  if (d->max_tokens < 1) return fail(MOE_EINVAL, "moe_cache_create: max_tokens=%d", d->max_tokens);
  if (d->num_slots < d->E)
    return fail(MOE_ECACHE_SMALL, "moe_cache_create: num_slots=%d is too small: need at least num_experts=%d",
                d->num_slots, d->E);
  if ((long)d->max_tokens * d->k > d->num_slots)
    return fail(MOE_ECACHE_SMALL, "moe_cache_create: max_tokens*k=%ld exceeds num_slots=%d",
                (long)d->max_tokens * d->k, d->num_slots);
  if (d->H % 32 || d->I % 32 || d->H <= 0 || d->I <= 0) return fail(MOE_ESHAPE, "moe_cache_create: H=%d I=%d", d->H, d->I);
  const bool int2 = d->ladder_b > d->ladder_a;
  if (d->int2_slots < 0) return fail(MOE_EINVAL, "moe_cache_create: int2_slots=%d", d->int2_slots);
  if (int2 && d->int2_slots > 0 && (long)d->max_tokens * (d->ladder_b - d->ladder_a) > d->int2_slots)
    return fail(MOE_ECACHE_SMALL, "moe_cache_create: int2_slots=%d below max_tokens*(b-a)=%ld", d->int2_slots,
                (long)d->max_tokens * (d->ladder_b - d->ladder_a));
  if (d->prefetch_slots < 0) return fail(MOE_EINVAL, "moe_cache_create: prefetch_slots=%d", d->prefetch_slots);
  if (d->policy != MOE_CACHE_LRU && d->policy != MOE_CACHE_LFU)
    return fail(MOE_EINVAL, "moe_cache_create: policy=%d", d->policy);
  if (d->policy == MOE_CACHE_LFU && !(d->lfu_decay > 0.0 && d->lfu_decay <= 1.0))
    return fail(MOE_EINVAL, "moe_cache_create: lfu_decay=%g outside (0, 1]", d->lfu_decay);
  if (d->fp4_host == nullptr && d->fp4_arena != nullptr)
    return fail(MOE_EINVAL, "moe_cache_create: fp4_host is NULL");
  if (int2 && d->fp4_arena && (!d->int2_host || !d->int2_staging))
    return fail(MOE_EINVAL, "moe_cache_create: ladder a < b needs int2_host and int2_staging");
  moe_cache* c = new moe_cache();
  c->d = *d;
  c->poll_us = d->poll_us == 0 ? 2000000 : std::max(0LL, d->poll_us);
  c->fp4_bytes = record_layout(d->H, d->I, 4).bytes;
  c->int2_bytes = record_layout(d->H, d->I, 2).bytes;
  c->map.assign((size_t)d->L * d->E, -1);
  c->owner.assign(d->num_slots, -1);
  c->stamp.assign(d->num_slots, 0);
  c->map2.assign((size_t)d->L * d->E, -1);
  c->owner2.assign(d->int2_slots, -1);
  c->stamp2.assign(d->int2_slots, 0);
  c->seed.assign((size_t)d->L * d->E, 0.0);
  if (d->lfu_seed)
    for (size_t i = 0; i < c->seed.size(); ++i) c->seed[i] = (double)d->lfu_seed[i];
  c->count = c->seed;
  c->d.lfu_seed = nullptr;  // copied: the caller's array need not outlive the call
  c->ring_owner.assign(d->prefetch_slots, -1);
  c->ring_used.assign(d->prefetch_slots, 0);
  if (d->prefetch_slots > 0) c->map_ring.assign((size_t)d->L * d->E, -1);
  *out = c;
  return MOE_OK;
}

moe_status moe_cache_destroy(moe_cache* c) {
  if (!c) return MOE_OK;
  if (c->pin_in) (void)hipHostFree(c->pin_in);
  if (c->pin_out) (void)hipHostFree(c->pin_out);
  if (c->ev_read) (void)hipEventDestroy(c->ev_read);
  if (c->ev_copy) (void)hipEventDestroy(c->ev_copy);
  if (c->ev_prefetch) (void)hipEventDestroy(c->ev_prefetch);
  for (hipEvent_t e : {c->ev_stream[0], c->ev_stream[1], c->ev_compute})
    if (e) (void)hipEventDestroy(e);
  delete c;
  return MOE_OK;
}

moe_status moe_cache_reset(moe_cache* c) {
  if (!c) return fail(MOE_EINVAL, "moe_cache_reset: handle is NULL");
  // speculative and streamed copies nobody has waited for yet would land in
  // slots the emptied cache hands out again
  if (c->prefetch_pending) MOE_HIP_CHECK(hipEventSynchronize(c->ev_prefetch));
  for (int b = 0; b < 2; ++b)
    if (c->stream_pending[b]) MOE_HIP_CHECK(hipEventSynchronize(c->ev_stream[b]));
  // the last call's kernels still read pin_out and the slots: after them, any stream may follow
  if (c->compute_set && c->d.fp4_arena) MOE_HIP_CHECK(hipStreamSynchronize(c->compute));
  c->compute_set = false;
  std::fill(c->map.begin(), c->map.end(), -1);
  std::fill(c->owner.begin(), c->owner.end(), -1);
  std::fill(c->stamp.begin(), c->stamp.end(), 0);
  std::fill(c->map2.begin(), c->map2.end(), -1);
  std::fill(c->owner2.begin(), c->owner2.end(), -1);
  std::fill(c->stamp2.begin(), c->stamp2.end(), 0);
  c->count = c->seed;
  std::fill(c->ring_owner.begin(), c->ring_owner.end(), -1);
  std::fill(c->ring_used.begin(), c->ring_used.end(), 0);
  std::fill(c->map_ring.begin(), c->map_ring.end(), -1);
  c->cursor = 0;
  c->prefetch_pending = false;
  c->next_buf = 0;
  c->stream_pending[0] = c->stream_pending[1] = false;
  c->clock = 0;
  c->st = moe_cache_stats{};
  c->broken = false;
  return MOE_OK;
}

moe_status moe_cache_plan(moe_cache* c, int layer, int T, const int32_t* ids, const float* w, int32_t* slots,
                          int8_t* prec, float* w_out) {
  moe_status s = check_call(c, layer, T);
  if (s != MOE_OK) return s;
  if (!ids || !w || !slots || !prec || !w_out) return fail(MOE_EINVAL, "moe_cache_plan: NULL pointer");
  s = plan(c, layer, T, ids, w);
  if (s != MOE_OK) return s;
  const size_t n = (size_t)T * c->d.k;
  std::memcpy(slots, c->slots_h.data(), n * 4);
  std::memcpy(prec, c->prec_h.data(), n);
  std::memcpy(w_out, c->wout_h.data(), n * 4);
  for (const auto& cp : c->copies) c->st.bytes_h2d += (int64_t)(cp.kind == 0 ? c->fp4_bytes : c->int2_bytes);
  return MOE_OK;
}

moe_status moe_cache_ensure(moe_cache* c, int layer, int T, int32_t* ids_inout, float* w_inout, int8_t* prec_out,
                            moe_stream_t compute, moe_stream_t copy) {
  moe_status s = check_call(c, layer, T);
  if (s != MOE_OK) return s;
  if (!ids_inout || !w_inout || !prec_out) return fail(MOE_EINVAL, "moe_cache_ensure: NULL pointer");
  if (!c->d.fp4_arena) return fail(MOE_EINVAL, "moe_cache_ensure: the cache has no device arena");
  hipStream_t cs = (hipStream_t)compute, ps = copy ? (hipStream_t)copy : cs;
  s = check_compute(c, cs, "moe_cache_ensure");
  if (s != MOE_OK) return s;
  const size_t n = (size_t)T * c->d.k;
  if (!c->pin_in) {
    MOE_HIP_CHECK(hipHostMalloc(&c->pin_in, pin_in_bytes(c->d) + kFlagBytes, hipHostMallocMapped));
    std::memset(c->pin_in, 0, pin_in_bytes(c->d) + kFlagBytes);
    MOE_HIP_CHECK(hipHostMalloc(&c->pin_out, pin_out_bytes(c->d), hipHostMallocMapped));
    MOE_HIP_CHECK(hipHostGetDevicePointer(&c->pin_in_dev, c->pin_in, 0));
    MOE_HIP_CHECK(hipHostGetDevicePointer(&c->pin_out_dev, c->pin_out, 0));
    MOE_HIP_CHECK(hipEventCreateWithFlags(&c->ev_read, hipEventDisableTiming));
    MOE_HIP_CHECK(hipEventCreateWithFlags(&c->ev_copy, hipEventDisableTiming));
  }
  int32_t* ids_h = (int32_t*)c->pin_in;
  float* w_h = (float*)((char*)c->pin_in + (size_t)c->d.max_tokens * c->d.k * 4);
  // the one host sync of the call: read the router's picks.  One small
  // kernel writes them into the mapped pinned buffer, then the call's
  // sequence number; the host polls that word.  A poll that has not seen it
  // within poll_us (2 s unless the descriptor says otherwise; 0: no poll)
  // falls back to waiting for the kernel's completion (which also reports a
  // failed launch).
  {
    int32_t* ids_d = (int32_t*)c->pin_in_dev;
    float* w_d = (float*)((char*)c->pin_in_dev + (size_t)c->d.max_tokens * c->d.k * 4);
    uint32_t* flag_d = (uint32_t*)((char*)c->pin_in_dev + pin_in_bytes(c->d));
    s = launch_cache_gather(ids_inout, w_inout, (int)n, ids_d, w_d, flag_d, ++c->seq, cs);
    if (s != MOE_OK) return s;
  }
  {
    const volatile uint32_t* flag_h = (const volatile uint32_t*)((char*)c->pin_in + pin_in_bytes(c->d));
    bool seen = false;
    const auto t0 = std::chrono::steady_clock::now();
    for (uint64_t it = 0; c->poll_us > 0; ++it) {
      if (*flag_h == c->seq) {
        seen = true;
        break;
      }
#if defined(__x86_64__) || defined(__i386__)
      __builtin_ia32_pause();
#endif
      if ((it & 63) == 63 && std::chrono::steady_clock::now() - t0 > std::chrono::microseconds(c->poll_us)) break;
    }
    if (!seen) {
      MOE_HIP_CHECK(hipEventRecord(c->ev_read, cs));
      MOE_HIP_CHECK(hipEventSynchronize(c->ev_read));
      if (*flag_h != c->seq) return fail(MOE_EHIP, "moe_cache_ensure: the picks did not arrive");
    }
    std::atomic_thread_fence(std::memory_order_acquire);
  }
  s = plan(c, layer, T, ids_h, w_h);
  if (s != MOE_OK) return s;
  // from here on the host state has advanced: a failure leaves the cache inconsistent
  c->broken = true;
  for (int b = 0; b < 2; ++b)  // streamed layer buffers: their copies precede any use or overwrite
    if (c->stream_pending[b]) {
      MOE_HIP_CHECK(hipStreamWaitEvent(cs, c->ev_stream[b], 0));
      if (ps != cs) MOE_HIP_CHECK(hipStreamWaitEvent(ps, c->ev_stream[b], 0));
      c->stream_pending[b] = false;
    }
  for (const auto& cp : c->copies) {
    if (cp.kind == 0) {
      MOE_HIP_CHECK(hipMemcpyAsync(c->d.fp4_arena + (size_t)cp.dest * c->fp4_bytes,
                                   c->d.fp4_host + (size_t)cp.pair * c->fp4_bytes, c->fp4_bytes,
                                   hipMemcpyHostToDevice, ps));
      c->st.bytes_h2d += (int64_t)c->fp4_bytes;
    } else {
      MOE_HIP_CHECK(hipMemcpyAsync(c->d.int2_staging + (size_t)cp.dest * c->int2_bytes,
                                   c->d.int2_host + (size_t)cp.pair * c->int2_bytes, c->int2_bytes,
                                   hipMemcpyHostToDevice, ps));
      c->st.bytes_h2d += (int64_t)c->int2_bytes;
    }
  }
  if (ps != cs && !c->copies.empty()) {
    MOE_HIP_CHECK(hipEventRecord(c->ev_copy, ps));
    MOE_HIP_CHECK(hipStreamWaitEvent(cs, c->ev_copy, 0));
  }
  if (c->prefetch_pending) {  // ring entries this call may use were filled on the prefetch's stream
    MOE_HIP_CHECK(hipStreamWaitEvent(cs, c->ev_prefetch, 0));
    c->prefetch_pending = false;
  }
  int32_t* slots_o = (int32_t*)c->pin_out;
  float* w_o = (float*)((char*)c->pin_out + (size_t)c->d.max_tokens * c->d.k * 4);
  int8_t* prec_o = (int8_t*)((char*)c->pin_out + (size_t)c->d.max_tokens * c->d.k * 8);
  std::memcpy(slots_o, c->slots_h.data(), n * 4);
  std::memcpy(w_o, c->wout_h.data(), n * 4);
  std::memcpy(prec_o, c->prec_h.data(), n);
  // one small kernel reads them back from the mapped buffer; the next call's
  // host writes come after its own sync, which follows this kernel
  {
    const char* base = (const char*)c->pin_out_dev;
    const size_t nk = (size_t)c->d.max_tokens * c->d.k;
    s = launch_cache_scatter((const int32_t*)base, (const float*)(base + nk * 4), (const int8_t*)(base + nk * 8),
                             (int)n, ids_inout, w_inout, prec_out, cs);
    if (s != MOE_OK) return s;
  }
  c->broken = false;
  return MOE_OK;
}

moe_status moe_cache_prefetch(moe_cache* c, int layer, int n, const int32_t* experts, moe_stream_t copy) {
  if (!c) return fail(MOE_EINVAL, "moe_cache_prefetch: handle is NULL");
  if (c->broken) return fail(MOE_ESTATE, "moe_cache: an earlier ensure failed midway; reset the cache");
  if (c->d.prefetch_slots <= 0) return fail(MOE_EINVAL, "moe_cache_prefetch: the cache has no staging ring");
  if (layer < 0 || layer >= c->d.L) return fail(MOE_EINVAL, "moe_cache_prefetch: layer %d outside [0, %d)", layer, c->d.L);
  if (n < 0 || (n > 0 && !experts)) return fail(MOE_EINVAL, "moe_cache_prefetch: n=%d experts=%p", n, (const void*)experts);
  moe_status s = plan_prefetch(c, layer, n, experts);
  if (s != MOE_OK) return s;
  if (!c->d.fp4_arena || c->copies.empty()) return MOE_OK;
  hipStream_t ps = (hipStream_t)copy;
  if (!c->ev_prefetch) MOE_HIP_CHECK(hipEventCreateWithFlags(&c->ev_prefetch, hipEventDisableTiming));
  // several prefetches before one ensure may use different streams: chain them, so the one
  // event the ensure waits on covers every copy
  if (c->prefetch_pending) MOE_HIP_CHECK(hipStreamWaitEvent(ps, c->ev_prefetch, 0));
  for (const auto& cp : c->copies) {
    MOE_HIP_CHECK(hipMemcpyAsync(c->d.fp4_arena + (size_t)cp.dest * c->fp4_bytes,
                                 c->d.fp4_host + (size_t)cp.pair * c->fp4_bytes, c->fp4_bytes,
                                 hipMemcpyHostToDevice, ps));
    c->st.bytes_h2d += (int64_t)c->fp4_bytes;
  }
  MOE_HIP_CHECK(hipEventRecord(c->ev_prefetch, ps));
  c->prefetch_pending = true;
  return MOE_OK;
}

int moe_prefill_streams(int T, int k, int E) { return (int64_t)T * k >= (int64_t)E ? 1 : 0; }

moe_status moe_cache_stream_layer(moe_cache* c, int layer, int* buffer, moe_stream_t compute, moe_stream_t copy) {
  if (!c) return fail(MOE_EINVAL, "moe_cache_stream_layer: handle is NULL");
  if (c->broken) return fail(MOE_ESTATE, "moe_cache: an earlier ensure failed midway; reset the cache");
  if (layer < 0 || layer >= c->d.L)
    return fail(MOE_EINVAL, "moe_cache_stream_layer: layer %d outside [0, %d)", layer, c->d.L);
  const int E = c->d.E;
  if (c->d.num_slots < 2 * E)
    return fail(MOE_ECACHE_SMALL, "moe_cache_stream_layer: num_slots=%d is too small: two expert-layer buffers need %d",
                c->d.num_slots, 2 * E);
  hipStream_t cs = (hipStream_t)compute, ps = copy ? (hipStream_t)copy : cs;
  if (c->d.fp4_arena) {
    const moe_status s = check_compute(c, cs, "moe_cache_stream_layer");
    if (s != MOE_OK) return s;
  }
  const int b = plan_stream(c, layer);
  if (buffer) *buffer = b;
  if (!c->d.fp4_arena) return MOE_OK;
  c->broken = true;
  for (hipEvent_t* e : {&c->ev_stream[0], &c->ev_stream[1], &c->ev_compute})
    if (!*e) MOE_HIP_CHECK(hipEventCreateWithFlags(e, hipEventDisableTiming));
  if (ps != cs) {  // work already on the compute stream may still read the buffer
    MOE_HIP_CHECK(hipEventRecord(c->ev_compute, cs));
    MOE_HIP_CHECK(hipStreamWaitEvent(ps, c->ev_compute, 0));
  }
  if (c->stream_pending[b ^ 1]) MOE_HIP_CHECK(hipStreamWaitEvent(ps, c->ev_stream[b ^ 1], 0));
  // runs of consecutive experts are contiguous in both the bank and the buffer: one copy each
  const auto& cp = c->copies;
  for (size_t i = 0; i < cp.size();) {
    size_t j = i + 1;
    while (j < cp.size() && cp[j].pair == cp[j - 1].pair + 1) ++j;
    const size_t bytes = (j - i) * c->fp4_bytes;
    MOE_HIP_CHECK(hipMemcpyAsync(c->d.fp4_arena + (size_t)cp[i].dest * c->fp4_bytes,
                                 c->d.fp4_host + (size_t)cp[i].pair * c->fp4_bytes, bytes, hipMemcpyHostToDevice, ps));
    c->st.bytes_h2d += (int64_t)bytes;
    i = j;
  }
  MOE_HIP_CHECK(hipEventRecord(c->ev_stream[b], ps));
  c->stream_pending[b] = true;
  c->broken = false;
  return MOE_OK;
}

moe_status moe_cache_layer_buffer(moe_cache* c, int layer, moe_stream_t compute, moe_layer* out) {
  if (!c || !out) return fail(MOE_EINVAL, "moe_cache_layer_buffer: NULL argument");
  if (layer < 0 || layer >= c->d.L)
    return fail(MOE_EINVAL, "moe_cache_layer_buffer: layer %d outside [0, %d)", layer, c->d.L);
  const int E = c->d.E;
  int found = -1;
  for (int b = 0; b < 2 && found < 0 && c->d.num_slots >= 2 * E; ++b) {
    bool whole = true;
    for (int e = 0; e < E && whole; ++e) whole = c->owner[b * E + e] == layer * E + e;
    if (whole) found = b;
  }
  if (found < 0) return fail(MOE_ESTATE, "moe_cache_layer_buffer: layer %d is not whole in a layer buffer", layer);
  if (c->d.fp4_arena) {
    const moe_status s = check_compute(c, (hipStream_t)compute, "moe_cache_layer_buffer");
    if (s != MOE_OK) return s;
  }
  if (c->stream_pending[found]) {
    MOE_HIP_CHECK(hipStreamWaitEvent((hipStream_t)compute, c->ev_stream[found], 0));
    c->stream_pending[found] = false;
  }
  out->H = c->d.H;
  out->I = c->d.I;
  out->fp4_base = c->d.fp4_arena ? c->d.fp4_arena + (size_t)found * E * c->fp4_bytes : nullptr;
  out->fp4_stride = c->fp4_bytes;
  out->num_slots = E;
  out->int2_base = nullptr;
  out->int2_stride = 0;
  out->num_int2 = 0;
  out->shared = nullptr;
  out->flags = 0;
  return MOE_OK;
}

moe_status moe_cache_slot_map(const moe_cache* c, int32_t* map_host) {
  if (!c || !map_host) return fail(MOE_EINVAL, "moe_cache_slot_map: NULL argument");
  std::memcpy(map_host, c->map.data(), c->map.size() * 4);
  return MOE_OK;
}

moe_status moe_cache_get_stats(const moe_cache* c, moe_cache_stats* out) {
  if (!c || !out) return fail(MOE_EINVAL, "moe_cache_get_stats: NULL argument");
  *out = c->st;
  return MOE_OK;
}

moe_status moe_cache_layer(const moe_cache* c, moe_layer* out) {
  if (!c || !out) return fail(MOE_EINVAL, "moe_cache_layer: NULL argument");
  out->H = c->d.H;
  out->I = c->d.I;
  out->fp4_base = c->d.fp4_arena;
  out->fp4_stride = c->fp4_bytes;
  out->num_slots = c->d.num_slots + c->d.prefetch_slots;
  const bool int2 = c->d.ladder_b > c->d.ladder_a;
  out->int2_base = int2 ? c->d.int2_staging : nullptr;
  out->int2_stride = c->int2_bytes;
  out->num_int2 = !int2 ? 0 : c->d.int2_slots > 0 ? c->d.int2_slots : c->d.max_tokens * (c->d.ladder_b - c->d.ladder_a);
  out->shared = nullptr;
  out->flags = 0;
  return MOE_OK;
}

}  // extern "C"
