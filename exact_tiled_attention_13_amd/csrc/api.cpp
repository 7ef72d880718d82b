// C ABI of the attention library: argument checks, kernel selection and
// error reporting.  Every check runs before any HIP call.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdio>

#include "../../include/miattn.h"
#include "launch.h"

namespace {

thread_local char g_hip_msg[256] = "no HIP error recorded";

int hip_fail(hipError_t e) {
  std::snprintf(g_hip_msg, sizeof(g_hip_msg), "HIP error %d: %s", (int)e, hipGetErrorString(e));
  return MIATTN_ERR_HIP;
}

bool supported_d(int D) { return D == 64 || D == 128; }

// Alignment rules of include/miattn.h (NULL passes: its own check comes first).
bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool a4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }

// The scores are scale * (q_scale q).(k_scale k): the product must be finite.
bool fp8_scales_ok(float scale, float q_scale, float k_scale, float v_scale) {
  if (!std::isfinite(q_scale) || !std::isfinite(k_scale) || !std::isfinite(v_scale)) return false;
  const double qk = (double)scale * q_scale * k_scale * 1.4426950408889634;
  return std::isfinite((float)qk);
}

}  // namespace

namespace miattn {

int record_hip_error(hipError_t e) { return hip_fail(e); }

int device_cu_count() {
  // Per-device cache.  Threads that race on a device's first call all store
  // the same value; relaxed atomics make that race well defined.
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace miattn

extern "C" {

int attn_abi_version(void) { return 5; }

const char* attn_strerror(int code) {
  switch (code) {
    case MIATTN_OK: return "ok";
    case MIATTN_ERR_NULL: return "a required pointer is NULL";
    case MIATTN_ERR_SHAPE: return "bad shape or scale (sizes must be > 0, Hq % Hkv == 0, scale finite)";
    case MIATTN_ERR_UNSUPPORTED: return "unsupported argument (D must be 64 or 128, dtype 0/1, causal 0/1)";
    case MIATTN_ERR_WORKSPACE: return "workspace missing or smaller than the size the matching *_workspace_size() gives";
    case MIATTN_ERR_HIP: return g_hip_msg;
    case MIATTN_ERR_ALIGN:
      return "misaligned pointer (tensors and workspaces need 16-byte alignment; lse, kv_lens and block_table 4)";
    case MIATTN_ERR_SCRATCH:
      return "the call needs more scratch than attn_decode_noalloc holds (attn_decode_noalloc_max_bytes)";
    default: return "unknown error code";
  }
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Tq,
             int Tk, int D, float scale, int causal, const int32_t* kv_lens, int dtype, void* stream) {
  if (!q || !k || !v || !o) return MIATTN_ERR_NULL;
  if (!a16(q) || !a16(k) || !a16(v) || !a16(o) || !a4(lse) || !a4(kv_lens)) return MIATTN_ERR_ALIGN;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Tq <= 0 || Tk <= 0 || D <= 0 || Hq % Hkv != 0 || !std::isfinite(scale))
    return MIATTN_ERR_SHAPE;
  if (!supported_d(D) || (dtype != MIATTN_F32 && dtype != MIATTN_BF16) || (causal != 0 && causal != 1))
    return MIATTN_ERR_UNSUPPORTED;
  // one workgroup per 128 query rows per (batch, head) must fit a 1-D grid
  if ((long long)((Tq + 127) / 128) * B * Hq > 0x7fffffffLL) return MIATTN_ERR_SHAPE;
  miattn::FwdArgs a{q, k, v, o, lse, kv_lens, B, Hq, Hkv, Tq, Tk, D, scale, causal};
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = dtype == MIATTN_BF16 ? miattn::launch_fwd_bf16(a, st) : miattn::launch_fwd_f32(a, st);
  return e == hipSuccess ? MIATTN_OK : hip_fail(e);
}

int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Tq,
                 int Tk, int D, float scale, float q_scale, float k_scale, float v_scale, int causal,
                 const int32_t* kv_lens, void* stream) {
  if (!q || !k || !v || !o) return MIATTN_ERR_NULL;
  if (!a16(q) || !a16(k) || !a16(v) || !a16(o) || !a4(lse) || !a4(kv_lens)) return MIATTN_ERR_ALIGN;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Tq <= 0 || Tk <= 0 || D <= 0 || Hq % Hkv != 0 || !std::isfinite(scale) ||
      !fp8_scales_ok(scale, q_scale, k_scale, v_scale))
    return MIATTN_ERR_SHAPE;
  if (!supported_d(D) || (causal != 0 && causal != 1)) return MIATTN_ERR_UNSUPPORTED;
  if ((long long)((Tq + 127) / 128) * B * Hq > 0x7fffffffLL) return MIATTN_ERR_SHAPE;
  miattn::FwdArgs a{q, k, v, o, lse, kv_lens, B, Hq, Hkv, Tq, Tk, D, scale, causal, q_scale, k_scale, v_scale};
  hipError_t e = miattn::launch_fwd_fp8(a, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MIATTN_OK : hip_fail(e);
}

size_t attn_decode_workspace_size(int B, int Hq, int Hkv, int S_max, int D) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S_max <= 0 || D <= 0) return 0;
  return miattn::decode_ws_floats(B, Hq, S_max, D) * sizeof(float);
}

namespace {

// Grid limits of the split-K decode.
int decode_limits(int B, int Hq, int Hkv, int S_max) {
  const long long gy = (long long)Hkv * ((Hq / Hkv + 15) / 16);
  if (gy > 65535 || B > 65535) return MIATTN_ERR_SHAPE;
  // work items (sequence, head block, split) are counted in int32
  if ((long long)B * gy * miattn::decode_num_splits(S_max) > 0x7fffffffLL) return MIATTN_ERR_SHAPE;
  return MIATTN_OK;
}

// Checks and launches shared by the four decode entry points.  Contiguous
// caches pass block_table = NULL; E4M3 caches pass fp8 = 1 and their scales.
int decode_common(const void* q, const void* k, const void* v, const int32_t* block_table, void* o, float* lse,
                  int B, int Hq, int Hkv, int S_max, int D, float scale, const int32_t* kv_lens, void* workspace,
                  size_t workspace_bytes, int page_shift, int num_pages, int max_blocks, int fp8, float q_scale,
                  float k_scale, float v_scale, void* stream) {
  const size_t need = attn_decode_workspace_size(B, Hq, Hkv, S_max, D);
  if (!workspace || workspace_bytes < need) return MIATTN_ERR_WORKSPACE;
  if (!a16(workspace)) return MIATTN_ERR_ALIGN;
  const int lim = decode_limits(B, Hq, Hkv, S_max);
  if (lim != MIATTN_OK) return lim;
  float* ws = static_cast<float*>(workspace);
  const size_t nsp = (size_t)B * Hq * miattn::decode_num_splits(S_max);
  int32_t* idx = reinterpret_cast<int32_t*>(ws + nsp * (D + 2));
  miattn::DecodeArgs a{q,           k,          v,         o,          lse,   kv_lens, B,       Hq,
                       Hkv,         S_max,      D,         scale,      ws,    ws + nsp * D, idx,
                       block_table, page_shift, num_pages, max_blocks, fp8,   q_scale, k_scale, v_scale};
  hipError_t e = miattn::launch_decode(a, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MIATTN_OK : hip_fail(e);
}

// Page-size and pool checks of the paged entry points; sets shift and S_max.
int paged_geometry(int num_pages, int page_size, int max_blocks, int Hkv, int* shift, int* S_max) {
  if (page_size < 8 || page_size > 65536 || (page_size & (page_size - 1)) != 0) return MIATTN_ERR_UNSUPPORTED;
  int sh = 0;
  while ((1 << sh) < page_size) ++sh;
  // logical capacity of a sequence, and rows addressed in the pool
  const long long cap = (long long)max_blocks * page_size;
  if (cap > 0x7fffffffLL || (long long)num_pages * Hkv * page_size > (1LL << 40)) return MIATTN_ERR_SHAPE;
  *shift = sh;
  *S_max = (int)cap;
  return MIATTN_OK;
}

}  // namespace

}  // extern "C"

namespace miattn {

// Every check of attn_decode except the workspace's (no HIP call).
int decode_check(const void* q, const void* k_cache, const void* v_cache, const void* o, const float* lse, int B,
                 int Hq, int Hkv, int S_max, int D, float scale, const int32_t* kv_lens, int dtype) {
  if (!q || !k_cache || !v_cache || !o || !kv_lens) return MIATTN_ERR_NULL;
  if (!a16(q) || !a16(k_cache) || !a16(v_cache) || !a16(o) || !a4(lse) || !a4(kv_lens)) return MIATTN_ERR_ALIGN;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S_max <= 0 || D <= 0 || Hq % Hkv != 0 || !std::isfinite(scale))
    return MIATTN_ERR_SHAPE;
  if (!supported_d(D) || (dtype != MIATTN_F32 && dtype != MIATTN_BF16)) return MIATTN_ERR_UNSUPPORTED;
  if (dtype == MIATTN_F32) return (long long)B * Hq > 0x7fffffffLL ? MIATTN_ERR_SHAPE : MIATTN_OK;
  return decode_limits(B, Hq, Hkv, S_max);
}

}  // namespace miattn

extern "C" {

int attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int B, int Hq,
                int Hkv, int S_max, int D, float scale, const int32_t* kv_lens, void* workspace,
                size_t workspace_bytes, int dtype, void* stream) {
  const int chk = miattn::decode_check(q, k_cache, v_cache, o, lse, B, Hq, Hkv, S_max, D, scale, kv_lens, dtype);
  if (chk != MIATTN_OK) return chk;
  if (dtype == MIATTN_F32) {
    // one query row against the cache, bottom-right causal: exactly the decode step
    miattn::FwdArgs a{q, k_cache, v_cache, o, lse, kv_lens, B, Hq, Hkv, 1, S_max, D, scale, 1};
    hipError_t e = miattn::launch_fwd_f32(a, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? MIATTN_OK : hip_fail(e);
  }
  return decode_common(q, k_cache, v_cache, nullptr, o, lse, B, Hq, Hkv, S_max, D, scale, kv_lens, workspace,
                       workspace_bytes, 0, 0, 0, 0, 1.f, 1.f, 1.f, stream);
}

int attn_decode_fp8(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int B, int Hq,
                    int Hkv, int S_max, int D, float scale, float q_scale, float k_scale, float v_scale,
                    const int32_t* kv_lens, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k_cache || !v_cache || !o || !kv_lens) return MIATTN_ERR_NULL;
  if (!a16(q) || !a16(k_cache) || !a16(v_cache) || !a16(o) || !a4(lse) || !a4(kv_lens)) return MIATTN_ERR_ALIGN;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S_max <= 0 || D <= 0 || Hq % Hkv != 0 || !std::isfinite(scale) ||
      !fp8_scales_ok(scale, q_scale, k_scale, v_scale))
    return MIATTN_ERR_SHAPE;
  if (!supported_d(D)) return MIATTN_ERR_UNSUPPORTED;
  return decode_common(q, k_cache, v_cache, nullptr, o, lse, B, Hq, Hkv, S_max, D, scale, kv_lens, workspace,
                       workspace_bytes, 0, 0, 0, 1, q_scale, k_scale, v_scale, stream);
}

int attn_decode_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table, void* o,
                      float* lse, int B, int Hq, int Hkv, int num_pages, int page_size, int max_blocks, int D,
                      float scale, const int32_t* kv_lens, void* workspace, size_t workspace_bytes, int dtype,
                      void* stream) {
  if (!q || !k_pages || !v_pages || !block_table || !o || !kv_lens) return MIATTN_ERR_NULL;
  if (!a16(q) || !a16(k_pages) || !a16(v_pages) || !a16(o) || !a4(lse) || !a4(kv_lens) || !a4(block_table))
    return MIATTN_ERR_ALIGN;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || num_pages <= 0 || max_blocks <= 0 || D <= 0 || Hq % Hkv != 0 ||
      !std::isfinite(scale))
    return MIATTN_ERR_SHAPE;
  if (!supported_d(D) || dtype != MIATTN_BF16) return MIATTN_ERR_UNSUPPORTED;
  int shift = 0, S_max = 0;
  const int g = paged_geometry(num_pages, page_size, max_blocks, Hkv, &shift, &S_max);
  if (g != MIATTN_OK) return g;
  return decode_common(q, k_pages, v_pages, block_table, o, lse, B, Hq, Hkv, S_max, D, scale, kv_lens, workspace,
                       workspace_bytes, shift, num_pages, max_blocks, 0, 1.f, 1.f, 1.f, stream);
}

int attn_decode_paged_fp8(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                          void* o, float* lse, int B, int Hq, int Hkv, int num_pages, int page_size, int max_blocks,
                          int D, float scale, float q_scale, float k_scale, float v_scale, const int32_t* kv_lens,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k_pages || !v_pages || !block_table || !o || !kv_lens) return MIATTN_ERR_NULL;
  if (!a16(q) || !a16(k_pages) || !a16(v_pages) || !a16(o) || !a4(lse) || !a4(kv_lens) || !a4(block_table))
    return MIATTN_ERR_ALIGN;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || num_pages <= 0 || max_blocks <= 0 || D <= 0 || Hq % Hkv != 0 ||
      !std::isfinite(scale) || !fp8_scales_ok(scale, q_scale, k_scale, v_scale))
    return MIATTN_ERR_SHAPE;
  if (!supported_d(D)) return MIATTN_ERR_UNSUPPORTED;
  int shift = 0, S_max = 0;
  const int g = paged_geometry(num_pages, page_size, max_blocks, Hkv, &shift, &S_max);
  if (g != MIATTN_OK) return g;
  return decode_common(q, k_pages, v_pages, block_table, o, lse, B, Hq, Hkv, S_max, D, scale, kv_lens, workspace,
                       workspace_bytes, shift, num_pages, max_blocks, 1, q_scale, k_scale, v_scale, stream);
}

size_t attn_bwd_workspace_size(int B, int Hq, int Tq) {
  if (B <= 0 || Hq <= 0 || Tq <= 0) return 0;
  return miattn::bwd_ws_floats(B, Hq, Tq) * sizeof(float);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
             void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Tq, int Tk, int D, float scale, int causal,
             const int32_t* kv_lens, void* workspace, size_t workspace_bytes, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return MIATTN_ERR_NULL;
  if (!a16(q) || !a16(k) || !a16(v) || !a16(o) || !a4(lse) || !a16(dout) || !a16(dq) || !a16(dk) || !a16(dv) ||
      !a4(kv_lens))
    return MIATTN_ERR_ALIGN;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Tq <= 0 || Tk <= 0 || D <= 0 || Hq % Hkv != 0 || !std::isfinite(scale))
    return MIATTN_ERR_SHAPE;
  if (!supported_d(D) || dtype != MIATTN_BF16 || (causal != 0 && causal != 1)) return MIATTN_ERR_UNSUPPORTED;
  // 128 query rows (dQ) and 128 keys (dK, dV) per workgroup: each grid must fit a 1-D launch
  if ((long long)((Tq + 127) / 128) * B * Hq > 0x7fffffffLL || (long long)((Tk + 127) / 128) * B * Hkv > 0x7fffffffLL)
    return MIATTN_ERR_SHAPE;
  const size_t need = attn_bwd_workspace_size(B, Hq, Tq);
  if (!workspace || workspace_bytes < need) return MIATTN_ERR_WORKSPACE;
  if (!a16(workspace)) return MIATTN_ERR_ALIGN;
  miattn::BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv, kv_lens, B, Hq, Hkv, Tq, Tk, D, scale, causal,
                    static_cast<float*>(workspace)};
  hipError_t e = miattn::launch_bwd_bf16(a, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MIATTN_OK : hip_fail(e);
}

}  // extern "C"
