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
// over its keys for all query heads of the group (up to 16 per wave) and
// writes an un-normalised partial output with its running max and sum.  A
// second kernel merges the splits of each (sequence, query head) with the
// same rescale by exp(m_s - m) that the online softmax applies between tiles.
//
// Per 32-key tile a wave runs
//   S^T (keys x heads) = K Q^T    v_mfma_f32_16x16x32_bf16; A = K rows loaded
//                                 from HBM into registers (16 B per lane),
//                                 B = the group's queries (columns >= G zero)
//   O^T (d x heads)   += V^T P^T  A = V^T by transposing reads of the V tile,
//                                 which is copied HBM -> LDS by
//                                 global_load_lds_dwordx4 into the wave's own
//                                 two-stage ring.
// The next tile's K registers and V copies are issued before the current
// tile's math, so every wave keeps ~32 KiB of loads in flight.  The V copies
// (whole 1 KiB runs per instruction) are non-temporal: each cache byte is
// read once, and on gfx950 nt reads stream faster.  The K fragment loads
// touch each 128-byte line in two 64-byte halves from different
// instructions, so they keep the default policy and let L2 serve the
// second half.  The MFMA work
// is tiny next to the bytes moved; the matrix cores are used because they
// need no bf16 unpacking and no cross-lane dot products.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace miattn {
namespace {

constexpr int kNW = 4;       // waves (= splits) per workgroup
constexpr int kBN = 32;      // keys per tile
// cache policy of the cache reads: non-temporal ("nt"), each byte is read once
constexpr int kNonTemporal = 2;

typedef __attribute__((address_space(1))) const void gptr_t;
typedef __attribute__((address_space(3))) void lptr_t;
typedef __attribute__((address_space(3))) const u16 lds_u16;

// V tile chunk permutation: a transposing read (32 lanes) covers 8 rows x two
// adjacent 16-byte chunks; the XOR spreads them over 16 distinct 16-byte
// slots modulo 256 bytes (gfx950: 64 banks of 4 bytes).
template <int D>
__device__ __forceinline__ int swz_v(int r) { return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); }

__device__ __forceinline__ lds_u16* lds_base(lds_u16* p) {
  asm volatile("" : "+v"(p));
  return p;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// One unit of decode work: split s of sequence b for one block of up to 16
// query heads of KV head hkv.  Keys [k0, k1).
struct DecItem {
  int b, hkv, hb, s, k0, k1, ntiles;
};

// Work items are enumerated sequence by sequence, split by split, head block
// by head block: t = (prefix_splits(b) + s) * HBK + hbk.  Every wave computes
// the prefix sums of the per-sequence split counts with a wave scan over 64
// sequences at a time; lens0 caches this lane's length of the first 64.
// Returns false once t is past the last item.  Results are wave-uniform.
__device__ __forceinline__ bool find_item(int t, const int32_t* __restrict__ kv_lens, int lens0, int B, int S_max,
                                          int HBK, int NHB, int lane, DecItem& it) {
  const int u = t / HBK, hbk = t - u * HBK;
  int base = 0;
  for (int c0 = 0; c0 < B; c0 += 64) {
    const int bb = c0 + lane;
    const int L = c0 == 0 ? lens0 : (bb < B ? clampi(kv_lens[bb], 0, S_max) : 0);
    const int ns = (L + kDecodeSplitKeys - 1) / kDecodeSplitKeys;
    int incl = ns;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const int total = __shfl(incl, 63);
    if (u < base + total) {
      const unsigned long long hit = __ballot(base + incl > u);
      const int first = __ffsll((long long)hit) - 1;
      const int pre = base + __shfl(incl - ns, first);
      const int Lb = __shfl(L, first);
      it.b = __builtin_amdgcn_readfirstlane(c0 + first);
      it.s = __builtin_amdgcn_readfirstlane(u - pre);
      it.k0 = it.s * kDecodeSplitKeys;
      it.k1 = __builtin_amdgcn_readfirstlane(min(it.k0 + kDecodeSplitKeys, Lb));
      it.ntiles = (it.k1 - it.k0 + kBN - 1) / kBN;
      it.hkv = hbk / NHB;
      it.hb = hbk - it.hkv * NHB;
      return true;
    }
    base += total;
  }
  return false;
}

// Persistent split kernel: the grid is sized to the chip (two workgroups per
// CU) and wave W takes items W, W + #waves, ...; the next tile, including
// the first tile of the wave's next item, is always in flight.
//
// Paged cache (PAGED): the rows of a sequence live in fixed-size pages of a
// shared pool, found through its block table.  A work item covers 512
// consecutive keys, i.e. at most 64 pages of >= 8 rows, so the wave loads
// the item's page numbers once (one per lane) and every row address takes
// its page from that vector with a lane shuffle.
template <int D, bool PAGED>
__global__ __launch_bounds__(64 * kNW) void decode_split_kernel(
    const u16* __restrict__ Qd, const u16* __restrict__ Kc, const u16* __restrict__ Vc,
    const int32_t* __restrict__ kv_lens, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    int B, int Hq, int Hkv, int S_max, int NS, int NHB, float c, int negq,
    const int32_t* __restrict__ block_table, int lgP, int num_pages, int max_blocks) {
  constexpr int KSTEPS = D / 32;             // k-steps of K Q^T
  constexpr int DB = D / 16;                 // 16-wide blocks of the head dim
  constexpr int TILE = kBN * D;              // elements per V tile
  constexpr int VLOADS = TILE * 2 / 1024;    // 1 KiB copies per V tile
  constexpr int VM_PER_TILE = 2 * KSTEPS + VLOADS;   // vector-memory ops per tile per lane
  __shared__ __attribute__((aligned(1024))) u16 Vs[kNW][2][TILE];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, j = lane & 15;
  const int G = Hq / Hkv;
  const int HBK = Hkv * NHB;
  const int NWAV = gridDim.x * kNW;
  int t = blockIdx.x * kNW + w;

  const int lens0 = lane < B ? clampi(kv_lens[lane], 0, S_max) : 0;
  DecItem cur;
  if (!find_item(t, kv_lens, lens0, B, S_max, HBK, NHB, lane, cur)) return;

  // per-item query fragments (B operand of S^T: column = head, d 32 ks + 8 g)
  bf16x8 qf[KSTEPS];
  int hq = 0;
  bool hv = false;
  auto load_q = [&](const DecItem& it) {
    const int head = it.hb * 16 + j;
    hv = head < G;
    hq = it.hkv * G + (hv ? head : 0);
    const u32x4* src = reinterpret_cast<const u32x4*>(Qd + ((size_t)it.b * Hq + hq) * D + 8 * g);
    const uint32_t flip = negq ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4 x = hv ? src[4 * ks] : u32x4{0u, 0u, 0u, 0u};
      x ^= flip;
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  };
  load_q(cur);

  // Issue tile `tile` of item `it`: K fragments into registers (A of S^T:
  // key 16 kb + j, d 32 ks + 8 g .. +7) and the V rows into LDS stage BUF.
  // Keys at or past k1 are replaced by key k1-1 (finite data; masked below).
  u32x4 kf[2][2][KSTEPS];
  // page numbers of the item being issued (lane i: its i-th page), paged only
  int pvec = 0;
  // element offset of logical key `key` of item `it` in the K and V arrays
  auto row_off = [&](const DecItem& it, int key) -> size_t {
    if constexpr (PAGED) {
      const int page = __shfl(pvec, (key >> lgP) - (it.k0 >> lgP));
      return ((((size_t)page * Hkv + it.hkv) << lgP) + (key & ((1 << lgP) - 1))) * D;
    } else {
      return (((size_t)it.b * Hkv + it.hkv) * (size_t)S_max + key) * D;
    }
  };
  auto issue = [&](auto BUF, const DecItem& it, int tile) {
    constexpr int buf = decltype(BUF)::value;
    if constexpr (PAGED) {
      if (tile == 0) {
        // the item's pages; out-of-range numbers are clamped into the pool
        // (a wrong table gives wrong results, never a stray access)
        const int blk = (it.k0 >> lgP) + lane;
        const int p = blk < max_blocks ? block_table[(size_t)it.b * max_blocks + blk] : 0;
        pvec = clampi(p, 0, num_pages - 1);
      }
    }
    const int kt = it.k0 + tile * kBN;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = min(kt + 16 * kb + j, it.k1 - 1);
      const u32x4* src = reinterpret_cast<const u32x4*>(Kc + row_off(it, key) + 8 * g);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) kf[buf][kb][ks] = src[4 * ks];
    }
#pragma unroll
    for (int li = 0; li < VLOADS; ++li) {
      const int e = li * 512 + lane * 8;
      const int r = e / D, slot = (e % D) / 8;
      const int ch = slot ^ swz_v<D>(r);
      const int key = min(kt + r, it.k1 - 1);
      __builtin_amdgcn_global_load_lds((gptr_t*)(Vc + row_off(it, key) + ch * 8),
                                       (lptr_t*)&Vs[w][buf][li * 512], 16, 0, kNonTemporal);
    }
  };

  // transposing-read offsets: group g covers rows 4 g + 0..3 (+16 for the
  // upper half) and logical columns 16 db + 0..15
  const int vr = 4 * g + (j >> 2);
  int voff[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
    voff[db] = vr * D + 8 * ((2 * db + ((j & 3) >> 1)) ^ swz_v<D>(vr)) + 4 * (j & 1);

  f32x4 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x4{};
  float m = kNegInf, lsum = 0.f;
  int tile = 0;

  // One step: tile `tile` of `cur` sits in buffer BUF.  The next (item,
  // tile) is issued into the other buffer first (that buffer's LDS reads
  // were consumed by the previous step's MFMAs), then the wave waits for the
  // current tile only.  Returns false after the wave's last tile.
  auto step = [&](auto BUF) -> bool {
    constexpr int buf = decltype(BUF)::value;
    DecItem nx = cur;
    int ntile = tile + 1;
    bool more = true;
    if (ntile >= cur.ntiles) {
      t += NWAV;
      more = find_item(t, kv_lens, lens0, B, S_max, HBK, NHB, lane, nx);
      ntile = 0;
    }
    if (more) {
      issue(std::integral_constant<int, buf ^ 1>{}, nx, ntile);
      wait_vmcnt<VM_PER_TILE>();
    } else {
      wait_vmcnt<0>();
    }

    const int kt = cur.k0 + tile * kBN;
    f32x4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[buf][kb][ks]), qf[ks],
                                                        s[kb], 0, 0, 0);
    }
    const bool need_mask = kt + kBN > cur.k1;
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kt + 16 * kb + 4 * g + r;
          s[kb][r] = key < cur.k1 ? s[kb][r] : kNegInf;
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

    // P^T element e of this lane is key 16 (e/4) + 4 g + e%4; the matching
    // V^T fragment is rows 4 g.. and 16 + 4 g.. of column 16 db + j.
    lds_u16* vs = (lds_u16*)&Vs[w][buf][0];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      lds_u16* vp = lds_base(vs + voff[db]);
      const u32x2 lo = lds_read_tr16(vp);
      const u32x2 hi = lds_read_tr16(vp + 16 * D);
      const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf, oacc[db], 0, 0, 0);
    }

    if (tile == cur.ntiles - 1) {
      // item done: write the partial (sum over the four lane groups that
      // share a query column), reset, fetch the next item's queries
      float lt = lsum + __shfl_xor(lsum, 16);
      lt = xhalf_sum(lt);
      if (hv) {
        const size_t base = ((size_t)cur.b * Hq + hq) * NS + cur.s;
        float* dst = ws_o + base * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(dst + 16 * db + 4 * g) = oacc[db];
        if (g == 0) {
          ws_ml[2 * base] = m;
          ws_ml[2 * base + 1] = lt;
        }
      }
#pragma unroll
      for (int i = 0; i < DB; ++i) oacc[i] = f32x4{};
      m = kNegInf;
      lsum = 0.f;
      if (more) load_q(nx);
    }
    cur = nx;
    tile = ntile;
    return more;
  };

  issue(std::integral_constant<int, 0>{}, cur, 0);
  while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{})) {
  }
}

// One workgroup (4 waves) per (query head, sequence): LSE-merge of the split
// partials.  Wave w takes splits w, w+4, ...; lane handles D/64 columns.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_ml, const int32_t* __restrict__ kv_lens,
    u16* __restrict__ O, float* __restrict__ LSE, int Hq, int S_max, int NS) {
  constexpr int PER = D / 64;
  __shared__ float red[4];
  __shared__ float part[4][D + 1];
  const int hq = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int L = clampi(kv_lens[b], 0, S_max);
  const int ns = (L + kDecodeSplitKeys - 1) / kDecodeSplitKeys;
  const size_t base = ((size_t)b * Hq + hq) * NS;

  // global max of the split maxima
  float M = kNegInf;
  for (int s = threadIdx.x; s < ns; s += 256) M = fmaxf(M, ws_ml[2 * (base + s)]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if (lane == 0) red[w] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float tot = 0.f;
#pragma unroll 4
  for (int s = w; s < ns; s += 4) {
    const float wgt = fast_exp2(ws_ml[2 * (base + s)] - M);
    tot += wgt * ws_ml[2 * (base + s) + 1];
    const float* src = ws_o + (base + s) * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] += wgt * src[lane + 64 * i];
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) part[w][lane + 64 * i] = acc[i];
  if (lane == 0) part[w][D] = tot;
  __syncthreads();
  if (w == 0) {
    const float T = part[0][D] + part[1][D] + part[2][D] + part[3][D];
    const bool has = T > 0.f;
    const float inv = has ? 1.f / T : 0.f;
    u16* dst = O + ((size_t)b * Hq + hq) * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int d = lane + 64 * i;
      dst[d] = f2bf((part[0][d] + part[1][d] + part[2][d] + part[3][d]) * inv);
    }
    if (LSE != nullptr && lane == 0) LSE[(size_t)b * Hq + hq] = has ? (M + __log2f(T)) * kLn2 : kNegInf;
  }
}

template <int D, bool PAGED>
hipError_t launch(const DecodeArgs& a, hipStream_t st) {
  const int NS = decode_num_splits(a.S_max);
  const int G = a.Hq / a.Hkv;
  const int NHB = (G + 15) / 16;
  const float c = fabsf(a.scale) * 1.4426950408889634f;
  const int negq = a.scale < 0.f ? 1 : 0;
  // two workgroups (8 waves) per CU, never more waves than work items
  const long long items = (long long)a.B * NS * a.Hkv * NHB;
  const long long wgs = std::min<long long>(2LL * device_cu_count(), (items + kNW - 1) / kNW);
  hipLaunchKernelGGL((decode_split_kernel<D, PAGED>), dim3((unsigned)wgs), dim3(64 * kNW), 0, st, (const u16*)a.q,
                     (const u16*)a.k_cache, (const u16*)a.v_cache, a.kv_lens, a.ws_o, a.ws_ml, a.B, a.Hq, a.Hkv,
                     a.S_max, NS, NHB, c, negq, a.block_table, a.page_shift, a.num_pages, a.max_blocks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)a.Hq, (unsigned)a.B), dim3(256), 0, st, a.ws_o,
                     a.ws_ml, a.kv_lens, (u16*)a.o, a.lse, a.Hq, a.S_max, NS);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t st) {
  if (a.block_table != nullptr) return a.D == 64 ? launch<64, true>(a, st) : launch<128, true>(a, st);
  return a.D == 64 ? launch<64, false>(a, st) : launch<128, false>(a, st);
}

}  // namespace miattn
