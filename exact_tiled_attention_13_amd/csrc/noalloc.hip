// Decode without a caller-supplied workspace: the split partials live in a
// fixed device array of this file, so the entry point allocates nothing
// (for callers that cannot allocate device memory: code under graph
// capture, tight serving loops).  The operation is attn_decode's.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/miattn.h"
#include "launch.h"

namespace {

constexpr size_t kScratchBytes = (size_t)96 << 20;

// One copy per device, held until the process ends.  In host code this
// name is only a stand-in: kernels are given the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_init_mu;

// Device address of the current device's scratch; looked up once per device
// (with that device current) and kept.
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return miattn::record_hip_error(e);
  if (dev < 0 || dev >= kMaxDevices) return MIATTN_ERR_UNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lk(g_init_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr) return miattn::record_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MIATTN_OK;
}

}  // namespace

extern "C" {

size_t attn_decode_noalloc_max_bytes(void) { return kScratchBytes; }

int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int B, int Hq,
                        int Hkv, int S_max, int D, float scale, const int32_t* kv_lens, int dtype, void* stream) {
  // every check runs before any HIP call, the size limit included
  const int chk = miattn::decode_check(q, k_cache, v_cache, o, lse, B, Hq, Hkv, S_max, D, scale, kv_lens, dtype);
  if (chk != MIATTN_OK) return chk;
  // the float32 path uses no workspace at all
  if (dtype == MIATTN_F32)
    return attn_decode(q, k_cache, v_cache, o, lse, B, Hq, Hkv, S_max, D, scale, kv_lens, nullptr, 0, dtype,
                       stream);
  if (attn_decode_workspace_size(B, Hq, Hkv, S_max, D) > kScratchBytes) return MIATTN_ERR_SCRATCH;
  void* ws = nullptr;
  const int r = scratch_address(&ws);
  if (r != MIATTN_OK) return r;
  return attn_decode(q, k_cache, v_cache, o, lse, B, Hq, Hkv, S_max, D, scale, kv_lens, ws, kScratchBytes, dtype,
                     stream);
}

}  // extern "C"
