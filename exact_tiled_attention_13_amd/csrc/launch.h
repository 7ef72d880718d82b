// Internal launchers behind the C ABI (include/miattn.h).  Arguments are
// validated by the ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace miattn {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;              // may be null
  const int32_t* kv_lens;  // device int32[B] or null
  int B, Hq, Hkv, Tq, Tk, D;
  float scale;
  int causal;
  // E4M3 inputs (launch_fwd_fp8): q, k, v hold codes standing for codes
  // times these scales; o stays bf16
  float q_scale = 1.f, k_scale = 1.f, v_scale = 1.f;
};

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  void* o;
  float* lse;              // may be null
  const int32_t* kv_lens;  // device int32[B], required
  int B, Hq, Hkv, S_max, D;
  float scale;
  float* ws_o;             // split partial outputs
  float* ws_ml;            // split partial (max, sum)
  int32_t* ws_idx;         // [0]: work items; [1 + b]: splits before sequence b
  // paged cache (block_table non-null): k_cache / v_cache are pools of
  // [num_pages, Hkv, 2^page_shift, D]; logical key j of sequence b is row
  // j & (page - 1) of page block_table[b * max_blocks + (j >> page_shift)].
  // S_max is then max_blocks << page_shift.
  const int32_t* block_table;
  int page_shift, num_pages, max_blocks;
  // E4M3 cache (fp8 non-zero): q, k_cache, v_cache hold E4M3 codes, each
  // tensor standing for its codes times its scale; o stays bf16.  The
  // bf16 path uses scales of 1.
  int fp8;
  float q_scale, k_scale, v_scale;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  const int32_t* kv_lens;  // device int32[B] or null
  int B, Hq, Hkv, Tq, Tk, D;
  float scale;
  int causal;
  float* ws;               // 2 * B * Hq * Tq floats: per-row dO.O, then LSE * log2(e)
};

inline size_t bwd_ws_floats(int B, int Hq, int Tq) { return 2 * (size_t)B * Hq * Tq; }

// Keys handled by one decode split (one wave).
#ifndef DEC_SPLIT_KEYS
#define DEC_SPLIT_KEYS 512
#endif
constexpr int kDecodeSplitKeys = DEC_SPLIT_KEYS;

inline int decode_num_splits(int S_max) { return (S_max + kDecodeSplitKeys - 1) / kDecodeSplitKeys; }
// partial outputs and (max, sum) per (sequence, query head, split), then
// B + 1 int32 of work-item bookkeeping
inline size_t decode_ws_floats(int B, int Hq, int S_max, int D) {
  return (size_t)B * Hq * decode_num_splits(S_max) * (size_t)(D + 2) + (size_t)B + 1;
}

// Compute units of the current device (cached per device; 256 if unknown).
int device_cu_count();

// Records a HIP error for attn_strerror and returns MIATTN_ERR_HIP (api.cpp).
int record_hip_error(hipError_t e);

// Every check of attn_decode except the workspace's; no HIP call (api.cpp).
int decode_check(const void* q, const void* k_cache, const void* v_cache, const void* o, const float* lse, int B,
                 int Hq, int Hkv, int S_max, int D, float scale, const int32_t* kv_lens, int dtype);

// Launch choices (tiles.cpp).  Prefill: shape 0 = 256-row workgroups with
// one key group, 1 = 128-row workgroups with two key groups; zig 0/1, or -1
// for the built-in rule.  T = Tk (keys per sequence),
// wg256 = ceil(Tq / 256) * B * Hq.
struct FwdChoice {
  int shape, zig;
};
constexpr long long kFwdSplitBelow = 512;
FwdChoice choose_fwd(int dtype, int D, int causal, long long T, long long wg256);
// Decode: split-kernel workgroups per CU, keyed by S_max and the work-item
// count items = B * NS * Hkv * ceil(G / 16).
int choose_decode_wgs_per_cu(int dtype, int D, long long S_max, long long items);

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t st);
hipError_t launch_fwd_fp8(const FwdArgs& a, hipStream_t st);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t st);

}  // namespace miattn
