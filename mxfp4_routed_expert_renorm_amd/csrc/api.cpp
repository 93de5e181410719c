// C entry points of the MoE library: validate every argument, then enqueue.
//
// Validation happens before any launch and fails with a targeted message
// rather than producing wrong math, the behaviour "Running DeepSeek-V4-Flash
// across four free GPUs" (§Step 2, Check it divides; §Step 7, the slot-count
// floor) asks of a serving runtime.
#include <algorithm>
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "common.h"

namespace moe {

static thread_local std::string g_last_error;

void set_error(const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

moe_status launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s);
moe_status launch_router_logits(const void* x, moe_dtype xt, const float* wr, int T, int E, int H, float* logits,
                                hipStream_t s);
moe_status launch_dequant(const uint8_t* record, int H, int I, int prec, int matrix, float* out, hipStream_t s);
moe_status launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s);
bool decode_shape_ok(int H, int I);
size_t prefill_workspace_bytes(int H, int I, int T, int k, int has_shared);
moe_status launch_quant_mxfp8(const void* x, long rows, int K, uint8_t* codes, uint8_t* scales, hipStream_t s);
size_t group_wide_scratch_ints(int n, int nkeys);
moe_status launch_group_wide(const int32_t* keys, int n, int nkeys, int32_t* counts, int32_t* offsets,
                             int32_t* perm, int32_t* scratch, hipStream_t s);
moe_status launch_prefill(const moe_layer* Lr, int E, const void* x, int T, int k, const int32_t* ids, const float* w,
                          void* out, void* workspace, hipStream_t s);
bool b1_path_ok(int H, int I, int K1, bool xbf16, bool obf16);
bool b1_route_ok(int E, int num_slots);
bool b1s_path_ok(int H, int I, int K1, bool xbf16, bool obf16, bool has_prec);
bool b1s_route_ok(int E, int num_slots);
moe_status launch_b1s(const moe_layer* L, const float* logits, int E, const void* x, int k, int32_t* slot_ids,
                      float* w, uint16_t* h, void* out, hipStream_t s);
moe_status launch_b1(const moe_layer* L, const float* logits, int E, const void* x, int k, int32_t* slot_ids,
                     const int8_t* prec, float* w, uint16_t* h, void* out, hipStream_t s);
size_t decode_plan_ints(int P);
bool decode_mfma_ok(int H, int I);
size_t decode_mfma_plan_ints(int P);
size_t fused_sync_bytes();
bool fused_path_ok(const moe_layer* L, int K1, bool xbf16, bool obf16, bool has_prec);
moe_status launch_fused_b1(const moe_layer* L, const float* logits, int E, const void* x, int k, int32_t* slot_ids,
                           float* w, uint16_t* h, void* out, uint32_t* sync, hipStream_t s);
bool fused_s_path_ok(const moe_layer* L, int K1, bool xbf16, bool obf16, bool has_prec);
moe_status launch_fused_b1s(const moe_layer* L, const float* logits, int E, const void* x, int k, int32_t* slot_ids,
                            float* w, uint16_t* h, void* out, uint32_t* sync, hipStream_t s);
moe_status launch_decode_mfma(const moe_layer* Lr, const void* x, int T, int k, const int32_t* slot_ids, const float* w,
                              void* out, uint16_t* h, float* y, int32_t* plan, hipStream_t s);

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

}  // namespace moe

using namespace moe;

#define REQUIRE(cond, st, ...)          \
  do {                                  \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

extern "C" {

const char* moe_last_error(void) { return g_last_error.c_str(); }

const char* moe_version(void) { return "moe-mi355x 0.1 (gfx950)"; }

size_t moe_fp4_expert_bytes(int H, int I) {
  if (H <= 0 || I <= 0) return 0;
  return record_layout(H, I, 4).bytes;
}

size_t moe_int2_expert_bytes(int H, int I) {
  if (H <= 0 || I <= 0) return 0;
  return record_layout(H, I, 2).bytes;
}

moe_status moe_router_logits(const void* x, moe_dtype xt, const float* w_router, int T, int E, int H, float* logits,
                             moe_stream_t stream) {
  REQUIRE(T >= 0 && E >= 1 && H >= 1, MOE_ESHAPE, "moe_router_logits: bad sizes T=%d E=%d H=%d", T, E, H);
  REQUIRE(xt == MOE_F32 || xt == MOE_BF16, MOE_EINVAL, "moe_router_logits: bad dtype %d", (int)xt);
  REQUIRE(T == 0 || (x && w_router && logits), MOE_EINVAL, "moe_router_logits: NULL pointer");
  return launch_router_logits(x, xt, w_router, T, E, H, logits, (hipStream_t)stream);
}

moe_status moe_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, moe_stream_t stream) {
  REQUIRE(T >= 0, MOE_ESHAPE, "moe_route: T=%d < 0", T);
  REQUIRE(E >= 1 && E <= 1024, MOE_ESHAPE, "moe_route: E=%d outside 1..1024", E);
  REQUIRE(k >= 1 && k <= E && k <= 64, MOE_EINVAL, "moe_route: k=%d must satisfy 1 <= k <= min(E=%d, 64)", k, E);
  REQUIRE(T == 0 || (logits && ids && w), MOE_EINVAL, "moe_route: NULL pointer");
  return launch_route(logits, T, E, k, ids, w, (hipStream_t)stream);
}

moe_status moe_group(const int32_t* keys, int n, int nkeys, int32_t* counts, int32_t* offsets, int32_t* perm,
                     moe_stream_t stream) {
  REQUIRE(n >= 0 && n <= (1 << 20), MOE_ESHAPE, "moe_group: n=%d outside 0..2^20", n);
  REQUIRE(nkeys >= 1 && nkeys <= 4096, MOE_ESHAPE, "moe_group: nkeys=%d outside 1..4096", nkeys);
  REQUIRE(counts && offsets && (n == 0 || (keys && perm)), MOE_EINVAL, "moe_group: NULL pointer");
  return launch_group(keys, n, nkeys, counts, offsets, perm, (hipStream_t)stream);
}

size_t moe_group_scratch_bytes(int n, int nkeys) {
  if (n < 0 || n > (1 << 20) || nkeys < 1 || nkeys > 4096) return 0;
  return group_wide_scratch_ints(n, nkeys) * sizeof(int32_t);
}

moe_status moe_group_wide(const int32_t* keys, int n, int nkeys, int32_t* counts, int32_t* offsets, int32_t* perm,
                          void* scratch, moe_stream_t stream) {
  REQUIRE(n >= 0 && n <= (1 << 20), MOE_ESHAPE, "moe_group_wide: n=%d outside 0..2^20", n);
  REQUIRE(nkeys >= 1 && nkeys <= 4096, MOE_ESHAPE, "moe_group_wide: nkeys=%d outside 1..4096", nkeys);
  REQUIRE(counts && offsets && (n == 0 || (keys && perm)), MOE_EINVAL, "moe_group_wide: NULL pointer");
  REQUIRE(group_wide_scratch_ints(n, nkeys) == 0 || (scratch && aligned(scratch, 4)), MOE_EINVAL,
          "moe_group_wide: scratch is NULL or not 4-byte aligned (%zu bytes needed)",
          group_wide_scratch_ints(n, nkeys) * sizeof(int32_t));
  return launch_group_wide(keys, n, nkeys, counts, offsets, perm, (int32_t*)scratch, (hipStream_t)stream);
}

size_t moe_expert_workspace_sync_offset(int H, int I, int T, int k, int has_shared) {
  if (H <= 0 || I <= 0 || T < 0 || k <= 0) return 0;
  const size_t P = (size_t)T * (size_t)(k + (has_shared ? 1 : 0));
  return align256(P * I * 4) + align256(P * H * 4) +
         align256(std::max(decode_plan_ints((int)P), decode_mfma_plan_ints((int)P)) * 4);
}

size_t moe_expert_workspace_bytes(int H, int I, int T, int k, int has_shared) {
  if (H <= 0 || I <= 0 || T < 0 || k <= 0) return 0;
  return moe_expert_workspace_sync_offset(H, I, T, k, has_shared) + align256(fused_sync_bytes());
}

static moe_status check_layer(const moe_layer* L, const char* who) {
  REQUIRE(L, MOE_EINVAL, "%s: layer is NULL", who);
  REQUIRE(decode_shape_ok(L->H, L->I), MOE_ESHAPE,
          "%s: H=%d I=%d unsupported (need multiples of 32 with H/32, I/32 a power of two in 4..64 or 128/256)", who,
          L->H, L->I);
  const size_t fb = record_layout(L->H, L->I, 4).bytes, ib = record_layout(L->H, L->I, 2).bytes;
  REQUIRE(L->fp4_base || L->num_slots == 0, MOE_EINVAL, "%s: fp4_base is NULL with num_slots=%d", who, L->num_slots);
  REQUIRE(L->num_slots >= 0 && L->num_int2 >= 0, MOE_EINVAL, "%s: negative slot counts", who);
  REQUIRE(L->num_slots == 0 || (L->fp4_stride >= fb && L->fp4_stride % 16 == 0), MOE_EINVAL,
          "%s: fp4_stride=%zu must be >= %zu and a multiple of 16", who, L->fp4_stride, fb);
  REQUIRE(!L->int2_base || L->num_int2 == 0 || (L->int2_stride >= ib && L->int2_stride % 16 == 0), MOE_EINVAL,
          "%s: int2_stride=%zu must be >= %zu and a multiple of 16", who, L->int2_stride, ib);
  REQUIRE(aligned(L->fp4_base, 16) && aligned(L->int2_base, 16) && aligned(L->shared, 16), MOE_EINVAL,
          "%s: expert records must be 16-byte aligned", who);
  return MOE_OK;
}

}  // extern "C"

namespace moe {

// The expert MLP of moe_expert_forward.  sync: the words the single launch
// keeps between calls; NULL puts them at the end of the workspace (the public
// entry point's layout), and then the workspace must cover them too.
moe_status expert_forward_impl(const moe_layer* layer, const void* x, moe_dtype xt, int T, int k,
                               const int32_t* slot_ids, const int8_t* prec, const float* w, void* out, moe_dtype ot,
                               void* workspace, size_t workspace_bytes, uint32_t* sync, hipStream_t s) {
  moe_status st = check_layer(layer, "moe_expert_forward");
  if (st != MOE_OK) return st;
  REQUIRE(T >= 0 && T <= 65536, MOE_ESHAPE, "moe_expert_forward: T=%d outside 0..65536", T);
  REQUIRE(k >= 1 && k <= 64, MOE_EINVAL, "moe_expert_forward: k=%d outside 1..64", k);
  REQUIRE(xt == MOE_F32 || xt == MOE_BF16, MOE_EINVAL, "moe_expert_forward: bad activation dtype %d", (int)xt);
  REQUIRE(w || ot == MOE_F32, MOE_EINVAL, "moe_expert_forward: per-rank outputs (w == NULL) are fp32");
  REQUIRE(ot == MOE_F32 || ot == MOE_BF16, MOE_EINVAL, "moe_expert_forward: bad output dtype %d", (int)ot);
  if (T == 0) return MOE_OK;
  REQUIRE(x && slot_ids && out && workspace, MOE_EINVAL, "moe_expert_forward: NULL pointer");
  REQUIRE(aligned(x, 16) && aligned(out, 16) && aligned(workspace, 256), MOE_EINVAL,
          "moe_expert_forward: x/out must be 16-byte and workspace 256-byte aligned");
  const int has_shared = layer->shared ? 1 : 0;
  const size_t need = sync ? moe_expert_workspace_sync_offset(layer->H, layer->I, T, k, has_shared)
                           : moe_expert_workspace_bytes(layer->H, layer->I, T, k, has_shared);
  REQUIRE(workspace_bytes >= need, MOE_ENOMEM, "moe_expert_forward: workspace %zu bytes < %zu needed",
          workspace_bytes, need);
  const int nkeys = layer->num_slots + (layer->int2_base ? layer->num_int2 : 0) + 1;
  REQUIRE(T == 1 || nkeys <= 4096, MOE_ESHAPE,
          "moe_expert_forward: batched grouping supports at most 4095 slots + 2-bit entries (got %d)", nkeys - 1);
  const int K1 = k + has_shared;
  const size_t P = (size_t)T * K1;
  char* ws = (char*)workspace;
  float* h = (float*)ws;
  float* y = (float*)(ws + align256(P * layer->I * 4));
  int32_t* plan = (int32_t*)(ws + align256(P * layer->I * 4) + align256(P * layer->H * 4));
  float* yout = w ? y : (float*)out;
  if (!sync) sync = (uint32_t*)(ws + moe_expert_workspace_sync_offset(layer->H, layer->I, T, k, has_shared));
  if (T == 1 && w && fused_path_ok(layer, K1, xt == MOE_BF16, ot == MOE_BF16, prec != nullptr))
    return launch_fused_b1(layer, nullptr, 0, x, k, const_cast<int32_t*>(slot_ids), const_cast<float*>(w),
                           (uint16_t*)h, out, sync, s);
  if (T == 1 && w && b1_path_ok(layer->H, layer->I, K1, xt == MOE_BF16, ot == MOE_BF16))  // reads slot_ids and w only
    return launch_b1(layer, nullptr, 0, x, k, const_cast<int32_t*>(slot_ids), prec, const_cast<float*>(w),
                     (uint16_t*)h, out, s);
  if (T == 1 && w && fused_s_path_ok(layer, K1, xt == MOE_BF16, ot == MOE_BF16, prec != nullptr))
    return launch_fused_b1s(layer, nullptr, 0, x, k, const_cast<int32_t*>(slot_ids), const_cast<float*>(w),
                            (uint16_t*)h, out, sync, s);
  if (T == 1 && w && b1s_path_ok(layer->H, layer->I, K1, xt == MOE_BF16, ot == MOE_BF16, prec != nullptr))
    return launch_b1s(layer, nullptr, 0, x, k, const_cast<int32_t*>(slot_ids), const_cast<float*>(w), (uint16_t*)h,
                      out, s);
  // batches of bf16 tokens, all FP4, weighted output: bf16 MFMA on weights dequantised in registers
  if (T >= 2 && w && !prec && xt == MOE_BF16 && ot == MOE_BF16 && decode_mfma_ok(layer->H, layer->I) &&
      P * (size_t)layer->I * 2 < ((size_t)1 << 31) && (size_t)T * layer->H * 2 < ((size_t)1 << 31))
    return launch_decode_mfma(layer, x, T, k, slot_ids, w, out, (uint16_t*)h, y, plan, s);
  st = launch_expert_decode(layer, x, xt, T, k, slot_ids, prec, h, yout, plan, s);
  if (st != MOE_OK) return st;
  if (w) return launch_combine(y, w, prec, T, k, layer->H, has_shared, out, ot, s);
  return MOE_OK;
}

// moe_layer_decode with the same sync convention as expert_forward_impl.
moe_status layer_decode_impl(const moe_layer* layer, const float* logits, int E, const void* x, moe_dtype xt, int k,
                             int32_t* ids, float* w, void* out, moe_dtype ot, void* workspace, size_t workspace_bytes,
                             uint32_t* sync, hipStream_t s) {
  moe_status st = check_layer(layer, "moe_layer_decode");
  if (st != MOE_OK) return st;
  REQUIRE(E >= 1 && E <= 1024, MOE_ESHAPE, "moe_layer_decode: E=%d outside 1..1024", E);
  REQUIRE(k >= 1 && k <= E && k <= 64, MOE_EINVAL, "moe_layer_decode: k=%d must satisfy 1 <= k <= min(E=%d, 64)", k,
          E);
  REQUIRE(layer->num_slots >= E, MOE_ECACHE_SMALL,
          "moe_layer_decode: the layer must hold every expert (num_slots=%d < E=%d); use the slot cache instead",
          layer->num_slots, E);
  REQUIRE(xt == MOE_F32 || xt == MOE_BF16, MOE_EINVAL, "moe_layer_decode: bad activation dtype %d", (int)xt);
  REQUIRE(ot == MOE_F32 || ot == MOE_BF16, MOE_EINVAL, "moe_layer_decode: bad output dtype %d", (int)ot);
  REQUIRE(logits && x && ids && w && out && workspace, MOE_EINVAL, "moe_layer_decode: NULL pointer");
  REQUIRE(aligned(x, 16) && aligned(out, 16) && aligned(workspace, 256), MOE_EINVAL,
          "moe_layer_decode: x/out must be 16-byte and workspace 256-byte aligned");
  const int has_shared = layer->shared ? 1 : 0;
  const size_t need = sync ? moe_expert_workspace_sync_offset(layer->H, layer->I, 1, k, has_shared)
                           : moe_expert_workspace_bytes(layer->H, layer->I, 1, k, has_shared);
  REQUIRE(workspace_bytes >= need, MOE_ENOMEM, "moe_layer_decode: workspace %zu bytes < %zu needed", workspace_bytes,
          need);
  if (!sync)
    sync = (uint32_t*)((char*)workspace + moe_expert_workspace_sync_offset(layer->H, layer->I, 1, k, has_shared));
  if (fused_path_ok(layer, k + has_shared, xt == MOE_BF16, ot == MOE_BF16, false) &&
      b1_route_ok(E, layer->num_slots))
    return launch_fused_b1(layer, logits, E, x, k, ids, w, (uint16_t*)workspace, out, sync, s);
  if (b1_path_ok(layer->H, layer->I, k + has_shared, xt == MOE_BF16, ot == MOE_BF16) && b1_route_ok(E, layer->num_slots))
    return launch_b1(layer, logits, E, x, k, ids, nullptr, w, (uint16_t*)workspace, out, s);
  if (fused_s_path_ok(layer, k + has_shared, xt == MOE_BF16, ot == MOE_BF16, false) &&
      b1s_route_ok(E, layer->num_slots))
    return launch_fused_b1s(layer, logits, E, x, k, ids, w, (uint16_t*)workspace, out, sync, s);
  if (b1s_path_ok(layer->H, layer->I, k + has_shared, xt == MOE_BF16, ot == MOE_BF16, false) &&
      b1s_route_ok(E, layer->num_slots))
    return launch_b1s(layer, logits, E, x, k, ids, w, (uint16_t*)workspace, out, s);
  st = launch_route(logits, 1, E, k, ids, w, s);
  if (st != MOE_OK) return st;
  return expert_forward_impl(layer, x, xt, 1, k, ids, nullptr, w, out, ot, workspace, workspace_bytes, sync, s);
}

}  // namespace moe

extern "C" {

moe_status moe_expert_forward(const moe_layer* layer, const void* x, moe_dtype xt, int T, int k,
                              const int32_t* slot_ids, const int8_t* prec, const float* w, void* out, moe_dtype ot,
                              void* workspace, size_t workspace_bytes, moe_stream_t stream) {
  return expert_forward_impl(layer, x, xt, T, k, slot_ids, prec, w, out, ot, workspace, workspace_bytes, nullptr,
                             (hipStream_t)stream);
}

moe_status moe_layer_decode(const moe_layer* layer, const float* logits, int E, const void* x, moe_dtype xt, int k,
                            int32_t* ids, float* w, void* out, moe_dtype ot, void* workspace, size_t workspace_bytes,
                            moe_stream_t stream) {
  return layer_decode_impl(layer, logits, E, x, xt, k, ids, w, out, ot, workspace, workspace_bytes, nullptr,
                           (hipStream_t)stream);
}

moe_status moe_combine(const float* y, const float* w, const int8_t* prec, int T, int k, int H, int has_shared,
                       void* out, moe_dtype ot, moe_stream_t stream) {
  REQUIRE(T >= 0 && k >= 1 && H >= 4 && H % 4 == 0, MOE_ESHAPE, "moe_combine: bad sizes T=%d k=%d H=%d", T, k, H);
  REQUIRE(ot == MOE_F32 || ot == MOE_BF16, MOE_EINVAL, "moe_combine: bad output dtype %d", (int)ot);
  if (T == 0) return MOE_OK;
  REQUIRE(y && w && out, MOE_EINVAL, "moe_combine: NULL pointer");
  REQUIRE(aligned(y, 16) && aligned(out, 8), MOE_EINVAL, "moe_combine: y must be 16-byte, out 8-byte aligned");
  return launch_combine(y, w, prec, T, k, H, has_shared ? 1 : 0, out, ot, (hipStream_t)stream);
}

moe_status moe_quant_mxfp8(const void* x, int rows, int K, uint8_t* codes, uint8_t* scales, moe_stream_t stream) {
  REQUIRE(rows >= 0 && K >= 32 && K % 32 == 0, MOE_ESHAPE, "moe_quant_mxfp8: rows=%d K=%d (K a multiple of 32)", rows,
          K);
  if (rows == 0) return MOE_OK;
  REQUIRE(x && codes && scales, MOE_EINVAL, "moe_quant_mxfp8: NULL pointer");
  REQUIRE(aligned(x, 16) && aligned(codes, 16), MOE_EINVAL, "moe_quant_mxfp8: x and codes must be 16-byte aligned");
  return launch_quant_mxfp8(x, rows, K, codes, scales, (hipStream_t)stream);
}

size_t moe_prefill_workspace_bytes(int H, int I, int T, int k, int has_shared) {
  if (H <= 0 || I <= 0 || T < 0 || k <= 0) return 0;
  return prefill_workspace_bytes(H, I, T, k, has_shared);
}

moe_status moe_prefill_forward(const moe_layer* layer, const void* x, int T, int k, const int32_t* ids, const float* w,
                               void* out, void* workspace, size_t workspace_bytes, moe_stream_t stream) {
  REQUIRE(layer, MOE_EINVAL, "moe_prefill_forward: layer is NULL");
  const int H = layer->H, I = layer->I, E = layer->num_slots;
  REQUIRE(H >= 256 && I >= 128 && H % 256 == 0 && I % 128 == 0, MOE_ESHAPE,
          "moe_prefill_forward: H=%d must be a multiple of 256 and I=%d a multiple of 128", H, I);
  REQUIRE(E >= 1 && E <= 4095, MOE_ESHAPE, "moe_prefill_forward: num_slots (experts) = %d outside 1..4095", E);
  REQUIRE(k >= 1 && k <= E && k <= 64, MOE_EINVAL, "moe_prefill_forward: k=%d (E=%d)", k, E);
  const int K1 = k + (layer->shared ? 1 : 0);
  REQUIRE(T >= 0 && (long)T * K1 <= (1L << 20), MOE_ESHAPE, "moe_prefill_forward: T=%d too large", T);
  REQUIRE((long)T * K1 * I < (1L << 31) && (long)T * H < (1L << 31), MOE_ESHAPE,
          "moe_prefill_forward: T=%d: activations beyond 2 GiB per matrix", T);
  if (T == 0) return MOE_OK;
  REQUIRE(layer->fp4_base && x && ids && w && out && workspace, MOE_EINVAL, "moe_prefill_forward: NULL pointer");
  const size_t fb = record_layout(H, I, 4).bytes;
  REQUIRE(layer->fp4_stride >= fb && layer->fp4_stride % 16 == 0, MOE_EINVAL,
          "moe_prefill_forward: fp4_stride=%zu must be >= %zu and a multiple of 16", layer->fp4_stride, fb);
  REQUIRE(aligned(layer->fp4_base, 16) && aligned(layer->shared, 16) && aligned(x, 16) && aligned(out, 16) &&
              aligned(workspace, 256),
          MOE_EINVAL, "moe_prefill_forward: records, x, out 16-byte and workspace 256-byte aligned");
  const size_t need = prefill_workspace_bytes(H, I, T, k, layer->shared ? 1 : 0);
  REQUIRE(workspace_bytes >= need, MOE_ENOMEM, "moe_prefill_forward: workspace %zu bytes < %zu needed",
          workspace_bytes, need);
  return launch_prefill(layer, E, x, T, k, ids, w, out, workspace, (hipStream_t)stream);
}

moe_status moe_debug_dequant(const uint8_t* record, int H, int I, int prec, int matrix, float* out,
                             moe_stream_t stream) {
  REQUIRE(H > 0 && I > 0 && H % 32 == 0 && I % 32 == 0, MOE_ESHAPE, "moe_debug_dequant: H=%d I=%d", H, I);
  REQUIRE(prec >= 0 && prec <= 2, MOE_EINVAL, "moe_debug_dequant: mode=%d (0 FP4, 1 2-bit, 2 FP4 scaled convert)",
          prec);
  REQUIRE(matrix >= 0 && matrix <= 2, MOE_EINVAL, "moe_debug_dequant: matrix=%d", matrix);
  REQUIRE(record && out, MOE_EINVAL, "moe_debug_dequant: NULL pointer");
  REQUIRE(aligned(record, 4), MOE_EINVAL, "moe_debug_dequant: record must be 4-byte aligned");
  return launch_dequant(record, H, I, prec, matrix, out, (hipStream_t)stream);
}

moe_status moe_debug_stream_read(const void* buf, size_t bytes, uint32_t* sink, moe_stream_t stream) {
  REQUIRE(buf && sink, MOE_EINVAL, "moe_debug_stream_read: NULL pointer");
  REQUIRE(aligned(buf, 16) && bytes % 16 == 0, MOE_EINVAL,
          "moe_debug_stream_read: buf must be 16-byte aligned and bytes a multiple of 16");
  if (bytes == 0) return MOE_OK;
  return launch_stream_read(buf, bytes, sink, (hipStream_t)stream);
}

}  // extern "C"
