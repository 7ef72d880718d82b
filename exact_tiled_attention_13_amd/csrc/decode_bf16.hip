// KV-cache decode with grouped-query attention, bf16 cache, fp32 softmax.
//
// "Implementing attention from scratch", KV caching and Cost model: a decode
// step attends one new query per head over all cached positions of its
// sequence, and is bound by reading the cache.  kv_lens[b] counts the valid
// cached keys including the newest token, so the query sees keys
// 0 .. kv_lens[b]-1.  Query heads h*G .. h*G+G-1 share KV head h.
//
// Split-K: the cache of one (sequence, KV head) is cut into splits of
// kDecodeSplitKeys keys; each split is one wave that runs the online softmax
// over its keys for all query heads of the group at once and writes an
// un-normalised partial output with its running max and sum.  A second
// kernel merges the splits of each (sequence, query head) with the same
// rescale by exp(m_s - m) that the online softmax applies between tiles.
//
// Per 32-key tile a wave runs
//   S^T (keys x heads) = K Q^T    v_mfma_f32_16x16x32_bf16, A = K rows loaded
//                                 straight from HBM (16 B per lane), B = the
//                                 group's queries (columns >= G are zero)
//   O^T (d x heads)   += V^T P^T  A = V^T by transposing reads of the V tile,
//                                 which the wave stages in its own LDS slab.
// The MFMA work is tiny next to the bytes moved; the matrix cores are used
// because they need no bf16->fp32 unpacking and no cross-lane dot products.
#include "device_common.h"
#include "launch.h"

namespace miattn {
namespace {

constexpr int kNW = 4;       // waves (= splits) per workgroup
constexpr int kBN = 32;      // keys per tile

template <int D>
__global__ __launch_bounds__(64 * kNW) void decode_split_kernel(
    const u16* __restrict__ Qd, const u16* __restrict__ Kc, const u16* __restrict__ Vc,
    const int32_t* __restrict__ kv_lens, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    int Hq, int Hkv, int S_max, int NS, int NHB, float c, int negq) {
  constexpr int VST = D + 16;          // LDS row stride (bf16) for conflict-free transposing reads
  constexpr int KSTEPS = D / 32;       // k-steps of K Q^T
  constexpr int DB = D / 16;           // 16-wide blocks of the head dim
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int VLOADS = kBN * CPR / 64;
  __shared__ __attribute__((aligned(16))) u16 Vs[kNW][kBN * VST];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, j = lane & 15;
  const int b = blockIdx.z;
  const int hkv = blockIdx.y / NHB, hb = blockIdx.y - hkv * NHB;
  const int split = blockIdx.x * kNW + w;
  const int G = Hq / Hkv;

  const int L = clampi(kv_lens[b], 0, S_max);
  const int k0 = split * kDecodeSplitKeys;
  const int k1 = min(k0 + kDecodeSplitKeys, L);
  if (k0 >= k1) return;  // whole wave: no keys in this split (no barriers below)

  const int head = hb * 16 + j;        // this lane's query column within the group
  const bool hv = head < G;
  const int hq = hkv * G + (hv ? head : 0);

  bf16x8 qf[KSTEPS];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(Qd + ((size_t)b * Hq + hq) * D + 8 * g);
    const uint32_t flip = negq ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4 x = hv ? src[4 * ks] : u32x4{0u, 0u, 0u, 0u};
      x ^= flip;
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  const size_t slab = ((size_t)b * Hkv + hkv) * (size_t)S_max * D;
  const u16* Kp = Kc + slab;
  const u16* Vp = Vc + slab;
  u16* vs = Vs[w];

  f32x4 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x4{};
  float m = kNegInf, lsum = 0.f;

  const int tr_row = 4 * g + (j >> 2);
  const int tr_col = 4 * (j & 3);

  for (int kt = k0; kt < k1; kt += kBN) {
    // K fragments: A (16 keys x 32 d), lane holds key kt+16*kb+j, d 32*ks+8*g..+7
    u32x4 kf[2][KSTEPS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = kt + 16 * kb + j;
      const bool ok = key < k1;
      const u32x4* src = reinterpret_cast<const u32x4*>(Kp + (size_t)(ok ? key : 0) * D + 8 * g);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) kf[kb][ks] = ok ? src[4 * ks] : u32x4{0u, 0u, 0u, 0u};
    }
    // V tile rows -> this wave's LDS slab; rows past the length are zero
    u32x4 vr[VLOADS];
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int idx = lane + 64 * i;
      const int row = idx / CPR, ch = idx % CPR;
      const int key = kt + row;
      const bool ok = key < k1;
      vr[i] = ok ? *reinterpret_cast<const u32x4*>(Vp + (size_t)(ok ? key : 0) * D + ch * 8)
                 : u32x4{0u, 0u, 0u, 0u};
    }

    f32x4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[kb][ks]), qf[ks],
                                                        s[kb], 0, 0, 0);
    }
    const bool need_mask = kt + kBN > k1;
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kt + 16 * kb + 4 * g + r;
          s[kb][r] = key < k1 ? s[kb][r] : kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = xhalf_max(mx);
    const float mt = (mx == kNegInf) ? kNegInf : mx * c;
    const float mnew = fmaxf(m, mt);
    const float muse = (mnew == kNegInf) ? 0.f : mnew;
    const float alpha = fast_exp2(m - muse);
    m = mnew;
    const float nm = -muse;
    bf16x8 pf;
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float p = fast_exp2(__builtin_fmaf(s[kb][r], c, nm));
        if (need_mask) p = (s[kb][r] == kNegInf) ? 0.f : p;
        ps += p;
        pf[4 * kb + r] = static_cast<__bf16>(p);
      }
    lsum = lsum * alpha + ps;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= alpha;

#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int idx = lane + 64 * i;
      const int row = idx / CPR, ch = idx % CPR;
      *reinterpret_cast<u32x4*>(&vs[row * VST + ch * 8]) = vr[i];
    }
    // LDS operations of one wave complete in issue order; the fence keeps the
    // compiler from moving the reads above the writes.
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    // P^T element e of this lane is key 16*(e/4) + 4*g + e%4; the matching
    // V^T fragment is rows 4*g.. and 16+4*g.. of column 16*db + j.
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const u16* vp = &vs[tr_row * VST + 16 * db + tr_col];
      const u32x2 lo = lds_read_tr16(vp);
      const u32x2 hi = lds_read_tr16(vp + 16 * VST);
      const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf, oacc[db], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }

  // sum over the four lane groups that share a query column
  float lt = lsum + __shfl_xor(lsum, 16);
  lt = xhalf_sum(lt);
  if (hv) {
    const size_t base = ((size_t)b * Hq + hq) * NS + split;
    float* dst = ws_o + base * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(dst + 16 * db + 4 * g) = oacc[db];
    if (g == 0) {
      ws_ml[2 * base] = m;
      ws_ml[2 * base + 1] = lt;
    }
  }
}

// One wave per (query head, sequence): LSE-merge of the split partials.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_ml, const int32_t* __restrict__ kv_lens,
    u16* __restrict__ O, float* __restrict__ LSE, int Hq, int S_max, int NS) {
  constexpr int PER = D / 64;
  const int hq = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int L = clampi(kv_lens[b], 0, S_max);
  const int ns = (L + kDecodeSplitKeys - 1) / kDecodeSplitKeys;
  const size_t base = ((size_t)b * Hq + hq) * NS;
  float M = kNegInf;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, ws_ml[2 * (base + s)]);
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float tot = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float wgt = fast_exp2(ws_ml[2 * (base + s)] - M);
    tot += wgt * ws_ml[2 * (base + s) + 1];
    const float* src = ws_o + (base + s) * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] += wgt * src[lane + 64 * i];
  }
  const bool has = tot > 0.f;
  const float inv = has ? 1.f / tot : 0.f;
  u16* dst = O + ((size_t)b * Hq + hq) * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) dst[lane + 64 * i] = f2bf(acc[i] * inv);
  if (LSE != nullptr && lane == 0) LSE[(size_t)b * Hq + hq] = has ? (M + __log2f(tot)) * kLn2 : kNegInf;
}

template <int D>
hipError_t launch(const DecodeArgs& a, hipStream_t st) {
  const int NS = decode_num_splits(a.S_max);
  const int G = a.Hq / a.Hkv;
  const int NHB = (G + 15) / 16;
  const float c = fabsf(a.scale) * 1.4426950408889634f;
  const int negq = a.scale < 0.f ? 1 : 0;
  const dim3 grid1((unsigned)((NS + kNW - 1) / kNW), (unsigned)(a.Hkv * NHB), (unsigned)a.B);
  hipLaunchKernelGGL((decode_split_kernel<D>), grid1, dim3(64 * kNW), 0, st, (const u16*)a.q,
                     (const u16*)a.k_cache, (const u16*)a.v_cache, a.kv_lens, a.ws_o, a.ws_ml, a.Hq, a.Hkv,
                     a.S_max, NS, NHB, c, negq);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)a.Hq, (unsigned)a.B), dim3(64), 0, st, a.ws_o,
                     a.ws_ml, a.kv_lens, (u16*)a.o, a.lse, a.Hq, a.S_max, NS);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t st) {
  return a.D == 64 ? launch<64>(a, st) : launch<128>(a, st);
}

}  // namespace miattn
