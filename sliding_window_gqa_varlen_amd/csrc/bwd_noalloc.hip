// varlen_attn_bwd for callers that cannot allocate: the same kernels, with the per-row delta
// workspace in a library-owned device array instead of a caller buffer.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "swattn.h"

namespace swa {
int32_t abi_fail(int32_t code, const char* detail);
}

namespace {

// delta [T, Hq] f32 of one call: 2^22 floats (16 MiB) per device, held until the process ends.
constexpr int64_t kScratchFloats = int64_t(1) << 22;
static __device__ __align__(256) float scratch[kScratchFloats];

// Per device, the device address of its copy of `scratch` (the array's name is only a host
// stand-in: every host use goes through this address).
constexpr int kMaxDevices = 64;
float* g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

int32_t scratch_for_current_device(float** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return swa::abi_fail(SWA_ERR_LAUNCH, "varlen_attn_bwd_noalloc: cannot query the current device");
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch[dev] == nullptr) {  // once per device, with that device current
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return swa::abi_fail(SWA_ERR_LAUNCH, "varlen_attn_bwd_noalloc: cannot resolve the workspace address");
    g_scratch[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch[dev];
  return SWA_OK;
}

}  // namespace

extern "C" int32_t varlen_attn_bwd_noalloc(const swa_tensor* q, const swa_tensor* k, const swa_tensor* v,
                                           const swa_tensor* out, const swa_tensor* dout, const float* lse,
                                           const int32_t* cu_seqlens, int32_t n_docs, int32_t window, float scale,
                                           const float* sinks, swa_tensor* dq, swa_tensor* dk, swa_tensor* dv,
                                           float* dsinks, void* stream) {
  if (q != nullptr && q->ndim == 3 && q->shape[0] >= 0 && q->shape[1] >= 0 &&
      q->shape[0] * q->shape[1] > kScratchFloats)
    return swa::abi_fail(SWA_ERR_UNSUPPORTED,
                         "varlen_attn_bwd_noalloc: T * Hq exceeds the 4,194,304-row workspace (use varlen_attn_bwd "
                         "with a caller workspace)");
  float* delta = nullptr;
  const int32_t st = scratch_for_current_device(&delta);
  if (st != SWA_OK) return st;
  return varlen_attn_bwd(q, k, v, out, dout, lse, cu_seqlens, n_docs, window, scale, sinks, dq, dk, dv, dsinks,
                         delta, stream);
}
