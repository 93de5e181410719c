// Batch-1 decode that allocates nothing: moe_layer_decode with its workspace
// in a file-scope device array instead of a caller's buffer.
//
// Layout of the array (one copy per device, held until the process ends):
//   [0, kSyncBytes)            the words the single-launch step keeps between
//                              calls (a launch tag per workgroup, the error
//                              word at +1024, the arrival counters), at a
//                              fixed place so that calls of different shapes
//                              find them where the last call left them;
//   [kSyncBytes, kScratchBytes) the per-call workspace (SwiGLU outputs, rank
//                              outputs, plans), rewritten by every call.
// The host learns each device's address of the array once, with that device
// current, and passes that address to the kernels; the array's own name is a
// host-side stand-in and never reaches a kernel.
#include <mutex>

#include "common.h"
#include "handoff_dev.h"

namespace moe {

moe_status layer_decode_impl(const moe_layer* layer, const float* logits, int E, const void* x, moe_dtype xt, int k,
                             int32_t* ids, float* w, void* out, moe_dtype ot, void* workspace, size_t workspace_bytes,
                             uint32_t* sync, hipStream_t s);

namespace {

constexpr size_t kSyncBytes = 4096;
static_assert(kSyncBytes >= kHandoffSyncBytes, "the single-launch steps' words fit");
constexpr size_t kScratchBytes = size_t(4) << 20;  // 4 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ __launch_bounds__(256) void zero_kernel(uint4* __restrict__ p, long n16) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n16; i += (long)gridDim.x * 256) p[i] = make_uint4(0, 0, 0, 0);
}

std::mutex g_mu;
uint8_t* g_ptr[kMaxDevices];  // device address of `scratch` per device, once known

// The device address of this device's array; on the first call for a device,
// also clears the array on `s` (ordered before the caller's kernels on s).
moe_status scratch_of_current_device(hipStream_t s, uint8_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(MOE_EHIP, "moe_layer_decode_noalloc: no usable current device (%d)", dev);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
      return fail(MOE_EINVAL,
                  "moe_layer_decode_noalloc: the first call on device %d must run outside stream capture "
                  "(it clears the static scratch once)",
                  dev);
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_EHIP, "moe_layer_decode_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    const long n16 = (long)(kScratchBytes / 16);
    launch(MOE_PROF_SCRATCH, zero_kernel, dim3(1024), dim3(256), 0, s, (uint4*)p, n16);
    MOE_LAUNCH_CHECK();
    g_ptr[dev] = (uint8_t*)p;
  }
  *out = g_ptr[dev];
  return MOE_OK;
}

}  // namespace

}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_noalloc_scratch_bytes(void) { return kScratchBytes - kSyncBytes; }

moe_status moe_layer_decode_noalloc(const moe_layer* layer, const float* logits, int E, const void* x, moe_dtype xt,
                                    int k, int32_t* ids, float* w, void* out, moe_dtype ot, moe_stream_t stream) {
  if (!layer) return fail(MOE_EINVAL, "moe_layer_decode_noalloc: layer is NULL");
  if (k < 1 || k > 64) return fail(MOE_EINVAL, "moe_layer_decode_noalloc: k=%d outside 1..64", k);
  const int has_shared = layer->shared ? 1 : 0;
  const size_t need = moe_expert_workspace_sync_offset(layer->H, layer->I, 1, k, has_shared);
  if (need == 0 || need > kScratchBytes - kSyncBytes)
    return fail(MOE_ENOMEM,
                "moe_layer_decode_noalloc: H=%d I=%d k=%d needs %zu bytes of scratch; the static scratch holds %zu",
                layer->H, layer->I, k, need, kScratchBytes - kSyncBytes);
  hipStream_t s = (hipStream_t)stream;
  uint8_t* base = nullptr;
  const moe_status st = scratch_of_current_device(s, &base);
  if (st != MOE_OK) return st;
  return layer_decode_impl(layer, logits, E, x, xt, k, ids, w, out, ot, base + kSyncBytes, kScratchBytes - kSyncBytes,
                           (uint32_t*)base, s);
}

}  // extern "C"
