// Allocation-free decode step: kk_decode_attn with its split partials in a
// static device array instead of a caller-provided workspace.
//
// The array lives in this translation unit's code object, which holds no
// kernels, so only processes that call kk_decode_attn_noalloc map it on a
// device.  Host code never passes the array's name to a kernel or a copy: on
// the host that name is a stand-in, not a device address.  The device address
// is looked up once per device with hipGetSymbolAddress (with that device
// current) and kept here.
#include <hip/hip_runtime.h>

#include <atomic>

#include "kk.h"

static __device__ __align__(256) float scratch[KK_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];   // device address of `scratch` per device

// Device address of `scratch` on device `dev` (looked up on first use).
kk_status scratch_on(int dev, void** addr) {
  if (dev < 0 || dev >= kMaxDevices) return KK_ERR_UNSUPPORTED;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return KK_ERR_DEVICE;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return KK_ERR_DEVICE;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return KK_ERR_DEVICE;
    if (e != hipSuccess || !p) return KK_ERR_DEVICE;
    // concurrent first calls store the same address
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *addr = p;
  return KK_OK;
}

}  // namespace

extern "C" kk_status kk_decode_attn_noalloc(const kk_model_cfg* cfg, const kk_cache* caches, int32_t batch,
                                            int32_t t_cap, const int32_t* seq_lens, int32_t max_seq_len,
                                            const void* q_lat, const void* q_rope, kk_dtype q_dtype, float* out,
                                            int32_t split_tokens, hipStream_t stream) {
  int dev = 0;
  if ((stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev)) != hipSuccess) return KK_ERR_DEVICE;
  void* ws = nullptr;
  const kk_status st = scratch_on(dev, &ws);
  if (st != KK_OK) return st;
  // Every check of kk_decode_attn applies; a step whose split partials need
  // more than the array holds is refused with KK_ERR_WORKSPACE_TOO_SMALL
  // before anything is enqueued.  Each work item writes its whole partial
  // slot before the merge reads it, so nothing in the array must start at
  // zero and what an earlier call left there is never read.
  return kk_decode_attn(cfg, caches, batch, t_cap, seq_lens, max_seq_len, q_lat, q_rope, q_dtype, out, split_tokens,
                        ws, KK_NOALLOC_SCRATCH_BYTES, stream);
}
