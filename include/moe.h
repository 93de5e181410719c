/*
 * moe.h -- C ABI of the MI355X (gfx950) routed MXFP4 mixture-of-experts layer.
 *
 * The layer follows two pages:
 *   [P1] "Running DeepSeek-V4-Flash across four free GPUs",
 *        §What the expert cache actually does: the router picks top_k experts
 *        per token, the cache rewrites expert ids to slots of a fixed-size
 *        slot cache in place, only misses are copied from pinned host banks,
 *        and the expert GEMM indexes the slot buffers with the token weights.
 *   [P2] "An elephant through a straw",
 *        §Not all six experts matter equally: the (a,b) precision ladder and
 *        the renormalisation of the surviving weights;
 *        §43 graphs, 43 syncs: one host sync per layer reads the router's
 *        picks, classifies them, then fires the grouped expert kernels.
 *
 * Conventions (every entry point):
 *   - Pointers are DEVICE memory unless the parameter says "host".  The caller
 *     owns every buffer and stream; the library never frees caller memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     GPU work is enqueued asynchronously on it; no entry point synchronises
 *     except moe_cache_ensure (one host sync per call, as in [P2] §43 graphs).
 *   - Arrays are dense row-major.  Sizes are int.
 *   - On error an entry point returns a non-zero moe_status, launches nothing
 *     (validation happens before any launch), and moe_last_error() returns a
 *     message for the calling thread.  Nothing is thrown across the ABI.
 *
 * Expert record (one expert's weights, contiguous bytes):
 *     w1 codes | w3 codes | w2 codes | w1 scales | w3 scales | w2 scales
 *   w1 = gate [I][H], w3 = up [I][H], w2 = down [H][I]  ([P1] §What you
 *   actually get: three matrices w1, w2, w3 per expert), each [out][in]
 *   row-major with one scale per 32 consecutive inputs ([P1] §Step 2, Check
 *   it divides: FP4 32-element scale blocks).
 *   MXFP4 record: FP4 E2M1 codes, two per byte, element 2j in the low nibble;
 *     E8M0 scale bytes (value 2^(e-127)).  ([P1] §The model: FP4 packed in I8
 *     tensors with F8_E8M0 scales; [P2] opening section: 13,369,344 bytes per
 *     expert at H=4096, I=2048.)  Size: moe_fp4_expert_bytes(H, I).
 *   2-bit record: codes four per byte, element 4j+q in bits 2q..2q+1, value
 *     (code - 1.5) * scale; FP8 E4M3 scale bytes.  ([P2] opening section and
 *     §Rig, model & methodology: 2-bit codes, one fp8 e4m3 scale per 32,
 *     2.25 bits per weight.)  Size: moe_int2_expert_bytes(H, I).
 *
 * Supported shapes: H and I multiples of 32 with H/32 and I/32 either a power
 * of two <= 64 or a multiple of 64 up to 256 (H, I <= 8192); 1 <= k <= E <= 1024,
 * k <= 64.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,        /* NULL pointer, bad enum, k > E, a > b, ... */
  MOE_ESHAPE = 2,        /* unsupported H, I, E, T or k */
  MOE_ECACHE_SMALL = 3,  /* slot cache below its floor */
  MOE_ENOMEM = 4,        /* workspace or host allocation too small / failed */
  MOE_EHIP = 5,          /* a HIP runtime call or kernel launch failed */
  MOE_ESTATE = 6         /* call out of order (e.g. cache used after an error) */
} moe_status;

/* Element types of activations and outputs.  A plain integer rather than an
 * enum type, so that any value a caller passes is a valid argument (and is
 * rejected with MOE_EINVAL unless it is one of these). */
typedef int32_t moe_dtype;
enum { MOE_F32 = 0, MOE_BF16 = 1 };

typedef void* moe_stream_t; /* hipStream_t */

/* Message describing the calling thread's last non-OK return ("" if none).
 * The pointer stays valid until the thread's next failing call. */
const char* moe_last_error(void);

/* Library version string. */
const char* moe_version(void);

/* Bytes of one MXFP4 / 2-bit expert record (host arithmetic, no GPU). */
size_t moe_fp4_expert_bytes(int H, int I);
size_t moe_int2_expert_bytes(int H, int I);

/* Where a layer's expert records live.
 *   fp4_base + s * fp4_stride       : MXFP4 record of slot s, 0 <= s < num_slots
 *                                     (for a fully resident layer, slot = expert id)
 *   int2_base + j * int2_stride     : 2-bit record of staging entry j, 0 <= j < num_int2
 *                                     (NULL / 0 when no 2-bit copies are used)
 *   shared                          : MXFP4 record of the always-on shared expert
 *                                     ([P2] §Rig, model & methodology: 256 routed experts
 *                                     plus 1 shared per layer), weight 1.0, outside the
 *                                     renormalisation; NULL = no shared expert.
 * Strides must be >= the record size and multiples of 16 bytes; records 16-byte aligned.
 * flags: MOE_LAYER_* bits (0 = defaults). */
typedef struct {
  int H, I;
  const uint8_t* fp4_base;
  size_t fp4_stride;
  int num_slots;
  const uint8_t* int2_base;
  size_t int2_stride;
  int num_int2;
  const uint8_t* shared;
  int flags;  /* MOE_LAYER_* bits, 0 for the defaults */
} moe_layer;

/* moe_layer.flags: batch-1 decode at the single-launch shape (see
 * moe_layer_decode) runs the whole step as one kernel instead of two. */
#define MOE_LAYER_SINGLE_LAUNCH 1

/* ---------------------------------------------------------------- routing */

/* Router scores of the tiny configuration: logits[t][e] = sum_h x[t][h] * w_router[e][h],
 * fp32 accumulation.  x [T][H] in xt (MOE_F32 or MOE_BF16), w_router [E][H] fp32,
 * logits [T][E] fp32 out. */
moe_status moe_router_logits(const void* x, moe_dtype xt, const float* w_router, int T, int E, int H,
                             float* logits, moe_stream_t stream);

/* Top-k routing with renormalised weights ([P1] §What the expert cache actually does:
 * the router picks its top_k experts per token; [P2] §Not all six experts matter
 * equally: six weights per token, renormalised).  Softmax scoring; the k largest
 * logits win, ties to the lower expert id; outputs in rank order (weight
 * descending).  The weights equal softmax over the selected logits (the full
 * softmax denominator cancels in the renormalisation).
 *   logits [T][E] fp32 (finite), ids [T][k] int32 out, w [T][k] fp32 out.
 * T may be 0 (no launch). */
moe_status moe_route(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                     moe_stream_t stream);

/* Stable grouping of n keys in [0, nkeys): counts [nkeys], offsets [nkeys+1]
 * (exclusive prefix of counts), perm [n] = indices of the keys sorted by key,
 * ascending index within a key.  Used to group the (token, rank) pairs by
 * expert so each expert's weights stream once ([P2] §43 graphs, 43 syncs:
 * grouped expert kernels).  keys int32 [n] (out-of-range keys are not counted
 * and not placed).  n <= 1<<20, nkeys <= 4096. */
moe_status moe_group(const int32_t* keys, int n, int nkeys, int32_t* counts, int32_t* offsets,
                     int32_t* perm, moe_stream_t stream);

/* moe_group spread over many workgroups, for tens of thousands of keys: each
 * 512-key chunk is counted into its own histogram, one workgroup scans the
 * histograms per key, then each chunk places its keys in input order.  Same
 * result as moe_group, bit for bit.  scratch: device, 4-byte aligned, at
 * least moe_group_scratch_bytes(n, nkeys) bytes (the chunks' histograms;
 * caller-owned, rewritten by every call).  When that is 0 (n <= 2048 or
 * nkeys > 1024) moe_group's one-workgroup grouping runs and scratch may be
 * NULL.  Limits and errors as moe_group. */
size_t moe_group_scratch_bytes(int n, int nkeys);
moe_status moe_group_wide(const int32_t* keys, int n, int nkeys, int32_t* counts, int32_t* offsets,
                          int32_t* perm, void* scratch, moe_stream_t stream);

/* ------------------------------------------------------------ expert MLP */

/* Workspace bytes moe_expert_forward and moe_layer_decode need for T tokens,
 * top-k, with or without the shared expert.
 * The last part of the workspace, from moe_expert_workspace_sync_offset(...)
 * on, holds words that the single-launch batch-1 steps keep from one call to
 * the next (a call tag per workgroup, an error word, arrival counters).  Zero
 * the whole workspace once after allocating it; after that the library keeps
 * those words consistent itself.  Calls that may run at the same
 * time (on different streams) must use different workspaces.  The error word
 * (the uint32 at sync offset + 1024) becomes nonzero only if a call's
 * cross-workgroup wait gave up, which happens only when the device could not
 * hold every workgroup of the call at once; that call's output is then
 * invalid. */
size_t moe_expert_workspace_bytes(int H, int I, int T, int k, int has_shared);
size_t moe_expert_workspace_sync_offset(int H, int I, int T, int k, int has_shared);

/* SwiGLU expert MLP for every selected (token, rank) and the shared expert:
 *     y = W2 (silu(W1 x) * (W3 x)), dequantised in registers, fp32 accumulation.
 * ([P1] §What the expert cache actually does: _expert_gemm over the slot
 * buffers; [P2] §43 graphs, 43 syncs: grouped expert kernels.)
 *   x        [T][H] activations in xt
 *   slot_ids [T][k] int32: record index (FP4 slot, or 2-bit staging entry)
 *   prec     [T][k] int8 or NULL (= all FP4): 0 MXFP4, 1 2-bit copy, -1 dropped
 *   w        [T][k] fp32 renormalised weights, or NULL
 *   out      if w != NULL: [T][H] in ot = sum over non-dropped ranks, in rank order,
 *                          of w * y (+ the shared expert's y), one final rounding
 *            if w == NULL: [T][k + has_shared][H] fp32 per-rank outputs (rank k =
 *                          shared); dropped ranks are zero
 *   workspace: device, >= moe_expert_workspace_bytes(...), 256-byte aligned.
 * Slot ids outside [0, num_slots) (or [0, num_int2) for 2-bit) are treated as dropped. */
moe_status moe_expert_forward(const moe_layer* layer, const void* x, moe_dtype xt, int T, int k,
                              const int32_t* slot_ids, const int8_t* prec, const float* w,
                              void* out, moe_dtype ot, void* workspace, size_t workspace_bytes,
                              moe_stream_t stream);

/* One decode token through a fully resident layer: routing (as moe_route) and
 * the expert MLP with the weighted combine (as moe_expert_forward with w), in
 * one call ([P1] §What the expert cache actually does: router picks, then the
 * expert GEMM over the slot buffers; [P2] §The number: at batch 1 the layer is
 * a stream of expert bytes).  For bf16 activations and output with H, I in
 * {2048, 4096} and k + has_shared <= 12, the routing runs inside the gate/up
 * kernel and the layer is two launches; the same holds for the narrow experts
 * of a tensor-parallel share (H in {2048, 4096}, I in {256, 512, 1024}, k +
 * has_shared <= 12); otherwise moe_route then moe_expert_forward run.  With MOE_LAYER_SINGLE_LAUNCH in layer->flags, at
 * H = 4096 with I = 2048 (the full expert) or I = 256 (a 1/8 tensor-parallel
 * share), k + has_shared <= 9, on a device of at least 256 CUs,
 * the whole step (routing, gate/up, down and combine) is ONE launch whose
 * workgroups hand the SwiGLU outputs to each other through the workspace;
 * moe_expert_forward at T = 1 with prec NULL takes the same single launch
 * from given ids and weights.  Both give the same results within rounding.
 *   layer: expert e in slot e (num_slots >= E), shared optional, no 2-bit copies
 *   logits [E] fp32, x [1][H] in xt
 *   ids [k] int32 out, w [k] fp32 out (rank order, as moe_route)
 *   out [1][H] in ot
 *   workspace: >= moe_expert_workspace_bytes(H, I, 1, k, has_shared), 256-byte aligned.
 * Errors: MOE_ECACHE_SMALL when num_slots < E. */
moe_status moe_layer_decode(const moe_layer* layer, const float* logits, int E, const void* x, moe_dtype xt,
                            int k, int32_t* ids, float* w, void* out, moe_dtype ot, void* workspace,
                            size_t workspace_bytes, moe_stream_t stream);

/* moe_layer_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * workspace is a static array inside the library, one per device, kept until
 * the process ends (4 MiB: the first 4 KiB hold the words the single launch
 * keeps between calls, the rest, moe_noalloc_scratch_bytes(), the per-call
 * workspace).  Arguments, results and errors are those of moe_layer_decode;
 * in addition:
 *   - MOE_ENOMEM when moe_expert_workspace_sync_offset(H, I, 1, k, has_shared)
 *     exceeds moe_noalloc_scratch_bytes();
 *   - the first call on a device clears its array with a kernel on `stream`,
 *     so that call must not be made under stream capture (MOE_EINVAL if it is);
 *     later calls may be captured;
 *   - every call on a device shares that device's array: calls that may
 *     overlap on one device (different streams, no ordering between them) race
 *     and give wrong results.  Nothing is allocated or freed by any call. */
moe_status moe_layer_decode_noalloc(const moe_layer* layer, const float* logits, int E, const void* x, moe_dtype xt,
                                    int k, int32_t* ids, float* w, void* out, moe_dtype ot, moe_stream_t stream);
size_t moe_noalloc_scratch_bytes(void);

/* Weighted combine ([P1] §What the expert cache actually does: the expert GEMM
 * takes topk_weights; [P2] §Not all six experts matter equally: survivors
 * renormalised):  out[t] = sum_{r < k, prec[t][r] >= 0} w[t][r] * y[t][r]
 * (+ y[t][k] if has_shared), summed in rank order, one rounding to ot.
 *   y [T][k + has_shared][H] fp32, w [T][k] fp32, prec [T][k] int8 or NULL,
 *   out [T][H] in ot. */
moe_status moe_combine(const float* y, const float* w, const int8_t* prec, int T, int k, int H,
                       int has_shared, void* out, moe_dtype ot, moe_stream_t stream);

/* Dequantise one matrix of a record to fp32 [rows][cols] with a decode path
 * of the expert kernels (bit-exact check of the formats).
 *   record: device record; matrix 0 = w1, 1 = w3, 2 = w2;
 *   prec (mode) 0 = MXFP4: the FP4 convert at scale 1.0 times the E8M0 scale
 *     in fp32 (the grouped decode kernels' two factors: they apply the scale
 *     to each 32-element partial sum);
 *   1 = 2-bit: (code - 1.5) times the E4M3 scale;
 *   2 = MXFP4 through the scaled FP4-to-bf16 convert with the E8M0 scale as
 *     its scale operand, widened to fp32: exactly the decode of the batch-1,
 *     single-launch and batched-decode (bf16 MFMA) kernels. */
moe_status moe_debug_dequant(const uint8_t* record, int H, int I, int prec, int matrix, float* out,
                             moe_stream_t stream);

/* Streaming-read reference for measurements: reads `bytes` bytes of `buf`
 * (device, 16-byte aligned, bytes a multiple of 16) once with non-temporal
 * 16-byte loads and writes nothing (`sink`, one device uint32, is stored only
 * under a condition the data cannot meet).  Its duration gives the measured
 * HBM read peak that the kernels' achieved bandwidth is compared with, beside
 * the 8 TB/s datasheet figure. */
moe_status moe_debug_stream_read(const void* buf, size_t bytes, uint32_t* sink, moe_stream_t stream);

/* ------------------------------------------------------------ tensor-parallel share */

/* Rank g's share of n MXFP4 records for G-way tensor parallelism ([P1] §Step 2, Check it
 * divides: every rank keeps its own slice of each expert, cut on the FP4 32-element scale
 * blocks).  Record e of src (H, I) at src + e*src_stride becomes record e of dst (H, I/G)
 * at dst + e*dst_stride: rows [g*I/G, (g+1)*I/G) of w1 and w3 with their scale rows, and
 * the same columns of w2 with its scale blocks along I.  The expert MLP of the share gives
 * a partial output; the G partials sum to the full output.  Device to device copies on
 * `stream`; dst_stride >= moe_fp4_expert_bytes(H, I/G).  Errors: MOE_ESHAPE when G does
 * not divide I into multiples of 32. */
moe_status moe_tp_slice(const uint8_t* src, size_t src_stride, int n, int H, int I, int G, int g, uint8_t* dst,
                        size_t dst_stride, moe_stream_t stream);

/* ------------------------------------------------------------ prefill */

/* MXFP8 quantisation of a bf16 matrix along its rows: one E8M0 scale per 32
 * consecutive elements, shared exponent floor(log2 amax) - 8 clamped to the E8M0
 * range, elements rounded to the nearest FP8 E4M3 (ties to even) with saturation
 * at +-448, an all-zero block gets scale byte 0 (the OCP Microscaling rule, cited
 * by [P2] References).  x [rows][K] bf16, codes [rows][K] uint8, scales
 * [rows][K/32] uint8; K a multiple of 32. */
moe_status moe_quant_mxfp8(const void* x, int rows, int K, uint8_t* codes, uint8_t* scales, moe_stream_t stream);

/* The 2-bit fallback copies of n MXFP4 expert records ("An elephant through a
 * straw", opening section and §Rig, model & methodology: 2-bit codes with one
 * fp8 E4M3 scale per 32 weights, the scale chosen by clip search, made
 * offline).  Per 32-weight group of the dequantised weights, each clip ratio
 * alpha in 1.00, 0.95, ..., 0.50 proposes the E4M3 scale s nearest to
 * alpha * amax / 1.5 (ties to even); each weight takes the nearest level
 * (c - 1.5) s, c = clamp(round half to even(w / s + 1.5), 0, 3); the ratio
 * with the least squared error (summed in element order) wins, ties to the
 * larger ratio; a zero scale gives code 2 throughout.  float64 throughout.
 *   src: device, n FP4 records (moe_fp4_expert_bytes(H, I)) src_stride apart,
 *        16-byte aligned; dst: device, n 2-bit records
 *        (moe_int2_expert_bytes(H, I)) dst_stride apart, 8-byte aligned.
 * Strides matter only for n > 1; src_stride a multiple of 16, dst_stride of 8.
 * H, I positive multiples of 32; 0 <= n <= 65535.  E8M0 scale byte 255 (NaN)
 * is outside the input domain. */
moe_status moe_int2_from_fp4(const uint8_t* src, size_t src_stride, int n, int H, int I, uint8_t* dst,
                             size_t dst_stride, moe_stream_t stream);

/* Workspace bytes of moe_prefill_forward. */
size_t moe_prefill_workspace_bytes(int H, int I, int T, int k, int has_shared);

/* Prefill-sized MoE layer on the matrix cores: x [T][H] bf16 quantised to MXFP8,
 * (token, rank) pairs grouped by expert (moe_group's order), per expert the
 * gate/up products on scaled FP8 x FP4 MFMA with SwiGLU and MXFP8 requantisation
 * of h in the epilogue, the down products likewise, and the rank-ordered combine
 * with the shared expert to out [T][H] bf16.  Every expert of the resident layer
 * is streamed once per tile of up to 192 rows of its group.
 *   layer: fp4_base/fp4_stride/num_slots = the E resident experts (slot = expert id),
 *          shared optional, no 2-bit copies; H a multiple of 256, I a multiple of 128.
 *   ids [T][k] int32 expert ids (moe_route's output), w [T][k] fp32 weights.
 * T*(k+has_shared) <= 1<<20, T*H and T*(k+has_shared)*I < 2^31, E <= 4095. */
moe_status moe_prefill_forward(const moe_layer* layer, const void* x, int T, int k, const int32_t* ids,
                               const float* w, void* out, void* workspace, size_t workspace_bytes,
                               moe_stream_t stream);

/* ------------------------------------------------------------ slot cache */

/* Pinned host memory of exactly `bytes` bytes (hipHostMalloc), for the expert
 * banks.  Exact size matters at this scale: a power-of-two rounding allocator
 * would turn a 27.4 GB bank into 34.4 GB ([P3] §Exact-size Engram pinning
 * describes the same loss with torch's pinned allocator).  Free with
 * moe_pinned_free. */
moe_status moe_pinned_alloc(size_t bytes, void** out);
moe_status moe_pinned_free(void* p);

/* Fixed-size slot cache over (layer, expert) pairs with LRU eviction and the
 * (a,b) precision ladder ([P1] §What the expert cache actually does; [P2]
 * §Not all six experts matter equally).  Opaque; created and destroyed on the
 * host.  A handle is not thread-safe: calls on one handle must not overlap. */
typedef struct moe_cache moe_cache;

typedef struct {
  int L, E, H, I;        /* layers, experts per layer, hidden, expert intermediate */
  int num_slots;         /* FP4 slots in device memory, shared by all layers; >= E */
  int k;                 /* ranks per token */
  int ladder_a, ladder_b;/* 0 <= a <= b <= k */
  int max_tokens;        /* most tokens per ensure call; max_tokens * k <= num_slots */
  const uint8_t* fp4_host;   /* host pinned: L*E FP4 records, pair l*E+e at (l*E+e)*moe_fp4_expert_bytes */
  const uint8_t* int2_host;  /* host pinned: L*E 2-bit records (NULL if a == b) */
  uint8_t* fp4_arena;        /* device: num_slots (+ prefetch_slots) FP4 records (NULL: host-only planning) */
  uint8_t* int2_staging;     /* device: 2-bit records (NULL if a == b): max_tokens*(b-a) staging entries when
                                int2_slots == 0, else the int2_slots slots of the 2-bit tier */
  /* Optional tiers and eviction rule ([P2] §Rig, model & methodology, best configuration: a
   * small device tier of 2-bit copies beside the FP4 slots, LFU with frequency decay seeded
   * from a routing trace).  All zero = the plain LRU cache with 2-bit copies staged per use. */
  int int2_slots;            /* > 0: 2-bit copies cached in this many device slots (>= max_tokens*(b-a)) */
  int policy;                /* MOE_CACHE_LRU or MOE_CACHE_LFU: eviction rule of both tiers */
  double lfu_decay;          /* LFU: every pair's use count is multiplied by this at each call, 0 < d <= 1 */
  const float* lfu_seed;     /* LFU: host [L*E] initial use counts (e.g. a routing trace's), NULL = zeros */
  int prefetch_slots;        /* R > 0: a staging ring of R more FP4 records at fp4_arena slots num_slots ..
                                num_slots+R-1 (the arena then holds num_slots+R records) for moe_cache_prefetch */
  long long poll_us;         /* how long moe_cache_ensure polls for the router's picks before it waits for the
                                kernel that publishes them, in microseconds: 0 = 2 s; < 0 = never poll */
} moe_cache_desc;

enum { MOE_CACHE_LRU = 0, MOE_CACHE_LFU = 1 };

typedef struct {
  int64_t calls, hits, misses, int2_uses, drops, bytes_h2d, evictions;
  int64_t int2_hits;         /* 2-bit uses served from the 2-bit tier without a copy */
  int64_t prefetches;        /* records copied into the staging ring */
  int64_t ring_hits;         /* FP4 uses served from the staging ring */
  int64_t streamed;          /* records copied by whole-layer streaming */
} moe_cache_stats;

/* Validates the descriptor (slot floor num_slots >= E: [P1] §Step 7 fails early when the
 * cache has fewer slots than experts), allocates host bookkeeping only; the cache starts
 * cold.  The caller keeps every buffer alive until moe_cache_destroy.
 * Eviction: the lowest-index empty slot, else among the slots this call has not used, LRU:
 * the oldest use; LFU: the pair with the lowest use count (ties: the oldest use).  LFU counts
 * belong to (layer, expert) pairs and survive eviction; each call first multiplies every
 * count by lfu_decay, and every use of a pair (hit or fetch, either tier) adds one. */
moe_status moe_cache_create(const moe_cache_desc* desc, moe_cache** out);
moe_status moe_cache_destroy(moe_cache* c);
/* Back to the cold state (empty slots and ring, clock 0, zero stats, LFU counts at their
 * seed).  Waits for prefetch and layer-stream copies that no call has waited for yet, and
 * for the compute stream the cache's calls have used, which a later call may then change. */
moe_status moe_cache_reset(moe_cache* c);

/* One call of the policy on host arrays, no GPU work: for T tokens of `layer`,
 * ids [T][k] expert ids and w [T][k] weights in rank order (host) ->
 * slots [T][k] (FP4 slot, 2-bit staging entry, or -1), prec [T][k] (0 FP4,
 * 1 2-bit, -1 dropped), w_out [T][k] renormalised over the survivors (host).
 * Advances the cache state exactly as moe_cache_ensure does. */
moe_status moe_cache_plan(moe_cache* c, int layer, int T, const int32_t* ids, const float* w, int32_t* slots,
                          int8_t* prec, float* w_out);

/* The per-layer call of the decode loop ([P1] §What the expert cache actually does:
 * ensure_experts + copy_missing; [P2] §43 graphs, 43 syncs: one host sync per layer).
 *   ids_inout [T][k] int32 device: expert ids in, slot / staging indices out (in place)
 *   w_inout   [T][k] fp32 device: router weights in, renormalised survivors out
 *   prec_out  [T][k] int8 device: 0 FP4, 1 2-bit, -1 dropped
 * Enqueues a device->host read of ids and w on `compute` and waits for it (the one
 * host sync: the host polls a sequence word that the read's kernel writes after the
 * picks; after MOE_CACHE_POLL_US microseconds, read from the environment when the
 * cache is created, default 2000000, 0 = no polling, it waits for the kernel's
 * completion instead), runs the policy, enqueues the FP4 miss copies and 2-bit copies from the
 * pinned banks on `copy` (NULL = compute), makes `compute` wait for them, and
 * enqueues the small host->device writes of the results on `compute`.  Everything the
 * caller enqueues on `compute` afterwards sees the copied experts.  Not capturable in
 * a graph (it synchronises).  Use moe_cache_layer's descriptor with
 * moe_expert_forward. */
moe_status moe_cache_ensure(moe_cache* c, int layer, int T, int32_t* ids_inout, float* w_inout, int8_t* prec_out,
                            moe_stream_t compute, moe_stream_t copy);

/* Speculative prefetch into the staging ring ([P2] §Guessing the router two layers ahead:
 * predicted experts land in a small round-robin ring appended to the slot buffers, so a wrong
 * guess never evicts a resident expert and is overwritten by a later prediction).  experts:
 * host [n] predicted expert ids of `layer`, most likely first.  Each one neither in the cache
 * nor in the ring is copied from the pinned bank to the ring entry at the cursor (which
 * advances), skipping the entries the last moe_cache_ensure call used (its expert kernels may
 * still read them; those of any earlier call have finished, since that ensure waited for its
 * router's picks) and those this call has filled; once every free entry is filled the rest of
 * the list is ignored.  The copies go on `copy`, and the next moe_cache_ensure makes its
 * compute stream wait for them.  A later call finds a ring entry resident and uses it in place
 * (slot num_slots + entry): no copy, no move into the cache.  Without a device arena only the
 * policy runs.  Needs prefetch_slots > 0. */
moe_status moe_cache_prefetch(moe_cache* c, int layer, int n, const int32_t* experts, moe_stream_t copy);

/* The prefill crossover ([P1] §What the expert cache actually does, §Step 7): 1 when a
 * chunk of T tokens with top-k over E experts should stream whole expert layers
 * (T*k >= E: the chunk touches most of the layer anyway), 0 when it should fetch
 * slots on demand through moe_cache_ensure. */
int moe_prefill_streams(int T, int k, int E);

/* Whole-layer streaming for prefill ([P1] §What the expert cache actually does: above
 * the crossover prefill streams whole expert layers; §Step 7: with prefill overlapping
 * the copies the cache lends two full expert-layer buffers, hence at least 2E slots).
 * The buffers are slots [0, E) and [E, 2E), filled alternately starting with the first
 * (*buffer gets 0 or 1, may be NULL).  Expert e of `layer` goes to slot bE + e: the
 * slot's previous pair is evicted, the layer's pairs held elsewhere (a slot or the
 * staging ring) give that place up, pairs already in place are not copied, and every
 * streamed slot is stamped as just used (no LFU use).  The streamed experts stay
 * resident.  Copies go on `copy` (one per run of consecutive experts) after the work
 * already on `compute` (which may still read the buffer) and after the other buffer's
 * pending copies; moe_cache_layer_buffer or the next moe_cache_ensure makes `compute`
 * wait for them.  Without a device arena only the policy runs.
 * Errors: MOE_ECACHE_SMALL when num_slots < 2E. */
moe_status moe_cache_stream_layer(moe_cache* c, int layer, int* buffer, moe_stream_t compute, moe_stream_t copy);

/* moe_layer descriptor (expert e in slot e, E slots, no 2-bit copies, no shared expert)
 * of the layer buffer that holds every expert of `layer`, for moe_prefill_forward or
 * moe_expert_forward with the router's expert ids; makes `compute` wait for that
 * buffer's pending copies.  Errors: MOE_ESTATE when no buffer holds the whole layer
 * (never streamed, or since overwritten). */
moe_status moe_cache_layer_buffer(moe_cache* c, int layer, moe_stream_t compute, moe_layer* out);

/* Host copy of the (layer, expert) -> slot map, [L*E] int32 (-1 = not resident). */
moe_status moe_cache_slot_map(const moe_cache* c, int32_t* map_host);
moe_status moe_cache_get_stats(const moe_cache* c, moe_cache_stats* out);
/* moe_layer descriptor of the cache's device arena (num_slots + prefetch_slots records) and
 * 2-bit staging or tier (no shared expert). */
moe_status moe_cache_layer(const moe_cache* c, moe_layer* out);

/* ------------------------------------------------------------ timing */

/* Kernel kinds reported by moe_profile_end. */
typedef enum {
  MOE_PROF_ROUTE = 0,
  MOE_PROF_ROUTER_LOGITS = 1,
  MOE_PROF_GATEUP = 2,      /* decode gate/up GEMV + SwiGLU */
  MOE_PROF_DOWN = 3,        /* decode down GEMV */
  MOE_PROF_COMBINE = 4,
  MOE_PROF_GROUP = 5,
  MOE_PROF_PLAN = 6,        /* pair keys / active-group list */
  MOE_PROF_QUANT = 7,       /* MXFP8 activation quantisation */
  MOE_PROF_GEMM_GATEUP = 8, /* prefill grouped GEMM, gate/up */
  MOE_PROF_GEMM_DOWN = 9,   /* prefill grouped GEMM, down */
  MOE_PROF_DEQUANT = 10,
  MOE_PROF_READ = 11,       /* streaming-read reference */
  MOE_PROF_CACHE = 12,      /* slot cache: picks to the host, rewritten ids back */
  MOE_PROF_FUSED = 13,      /* fused batch-1 step: routing, gate/up, down and combine in one launch */
  MOE_PROF_SCRATCH = 14,    /* one-time clear of the static scratch (moe_layer_decode_noalloc) */
  MOE_PROF_KINDS = 16
} moe_prof_kind;

/* Start timing the library's kernels: every launch made after this call is
 * bracketed by two HIP events recorded on its own stream (up to max_launches
 * launches; later ones are not timed).  Host-side bookkeeping only. */
moe_status moe_profile_begin(int max_launches);

/* Stop timing, wait for the recorded events and report, per moe_prof_kind,
 * the summed kernel time in milliseconds (total_ms[nkinds], host) and the
 * number of timed launches (counts[nkinds], host).  Either may be NULL. */
moe_status moe_profile_end(double* total_ms, int* counts, int nkinds);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
