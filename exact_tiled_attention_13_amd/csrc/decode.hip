// KV-cache decode with grouped-query attention: bf16 or E4M3 cache, fp32 softmax.
//
// "Implementing attention from scratch", KV caching and Cost model: a decode
// step attends one new query per head over all cached positions of its
// sequence, and is bound by reading the cache.  kv_lens[b] counts the valid
// cached keys including the newest token, so the query sees keys
// 0 .. kv_lens[b]-1.  Query heads h*G .. h*G+G-1 share KV head h.
//
// Split-K: the cache of one (sequence, KV head) is cut into splits of
// kDecodeSplitKeys keys, the work items, for all query heads of the group
// (up to 16 per wave).  A wave runs the online softmax over the splits it is
// given and writes an un-normalised partial output with its running max and
// sum.  A second kernel merges the partials of each (sequence, query head)
// with the same rescale by exp(m_s - m) that the online softmax applies
// between tiles.
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
//
// E4M3 caches (FP8): q, K and V hold 8-bit E4M3 codes with one scale per
// tensor (the FP8 inputs that the self-attention interview question lists,
// in its follow-up questions, among FlashAttention-3's additions).  Half the
// bytes of bf16 move per key, so a tile holds 64 keys (the same 16 KiB of
// K and V in flight per wave).  S^T = K Q^T runs on
// v_mfma_f32_16x16x32_fp8_fp8 straight from the codes (exact products, fp32
// sums); q_scale * k_scale is folded into the softmax constant.  The V tile
// is copied into LDS as codes, read back with byte-transposing reads and
// converted to bf16 (exact), so P stays bf16 as in the bf16 path; v_scale
// multiplies the merged output.
#include <algorithm>
#include <type_traits>

#include "../../include/miattn.h"
#include "device_common.h"
#include "launch.h"

namespace miattn {
namespace {

// lazy-rescale threshold of the running maximum, in log2 units
constexpr float kDecThresh = 8.0f;

constexpr int kNW = 4;       // waves (= splits) per workgroup
// keys per tile: bf16, E4M3 (16 KiB of K and V per tile either way)
template <bool FP8>
constexpr int kBN = FP8 ? 64 : 32;
// cache policy of the cache reads: non-temporal ("nt"), each byte is read once
constexpr int kNonTemporal = 2;

typedef __attribute__((address_space(1))) const void gptr_t;
typedef __attribute__((address_space(3))) void lptr_t;
typedef __attribute__((address_space(3))) const u16 lds_u16;
typedef __attribute__((address_space(3))) const uint8_t lds_u8;

// V tile chunk permutation: a transposing read (32 lanes) covers 8 rows x two
// adjacent 16-byte chunks; the XOR spreads them over 16 distinct 16-byte
// slots modulo 256 bytes (gfx950: 64 banks of 4 bytes).
template <int D>
__device__ __forceinline__ int swz_v(int r) { return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); }

// E4M3 V tile: the 16-byte chunk of logical column block c of row r sits at
// chunk c ^ swz_v8(r).  A byte-transposing read of one column block (32
// lanes) covers 16 rows (4 g + 0..3 and 16 + 4 g + 0..3 for two lane groups
// g, plus a multiple of 32); the XOR places those 16 chunks in 16 distinct
// 16-byte slots modulo 256 bytes.
template <int D>
__device__ __forceinline__ int swz_v8(int r) {
  return D == 128 ? (((r >> 1) & 3) | (((r >> 4) & 1) << 2)) : (((r >> 2) & 1) | (((r >> 4) & 1) << 1));
}

template <typename P>
__device__ __forceinline__ P* lds_base(P* p) {
  asm volatile("" : "+v"(p));
  return p;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// One unit of decode work: split s of sequence b for one block of up to 16
// query heads of KV head hkv.  Keys [k0, k1); ns and L are the sequence's
// split count and length.
struct DecItem {
  int b, hkv, hb, s, k0, k1, ntiles, ns, L;
};

template <int BN>
__device__ __forceinline__ void set_split(DecItem& it) {
  it.k0 = it.s * kDecodeSplitKeys;
  it.k1 = min(it.k0 + kDecodeSplitKeys, it.L);
  it.ntiles = (it.k1 - it.k0 + BN - 1) / BN;
}

// Inclusive wave scan of x over the 64 lanes.
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Work items are enumerated sequence by sequence, then head block by head
// block (hbk = hkv * NHB + hb), then split: item t = P(b) * HBK + hbk * ns_b
// + s with P(b) the splits of the sequences before b, so the splits of one
// (sequence, head block) are adjacent.  The sequence of item t is found with
// a wave scan of the split counts over 64 sequences at a time; lens0 caches
// this lane's length of the first 64.  Returns false once t is past the last
// item.  Results are wave-uniform.
template <int BN>
__device__ __forceinline__ bool find_item(int t, const int32_t* __restrict__ kv_lens, int lens0, int B, int S_max,
                                          int HBK, int NHB, int lane, DecItem& it) {
  int base = 0;   // items before sequence c0
  for (int c0 = 0; c0 < B; c0 += 64) {
    const int bb = c0 + lane;
    const int L = c0 == 0 ? lens0 : (bb < B ? clampi(kv_lens[bb], 0, S_max) : 0);
    const int ns = (L + kDecodeSplitKeys - 1) / kDecodeSplitKeys;
    const int incl = wave_incl_scan(ns, lane) * HBK;
    const int total = __shfl(incl, 63);
    if (t < base + total) {
      const unsigned long long hit = __ballot(base + incl > t);
      const int first = __ffsll((long long)hit) - 1;
      const int r = t - base - __shfl(incl - ns * HBK, first);
      it.ns = __builtin_amdgcn_readfirstlane(__shfl(ns, first));
      it.L = __builtin_amdgcn_readfirstlane(__shfl(L, first));
      it.b = __builtin_amdgcn_readfirstlane(c0 + first);
      const int hbk = __builtin_amdgcn_readfirstlane(r / it.ns);
      it.s = __builtin_amdgcn_readfirstlane(r - hbk * it.ns);
      it.hkv = hbk / NHB;
      it.hb = hbk - it.hkv * NHB;
      set_split<BN>(it);
      return true;
    }
    base += total;
  }
  return false;
}

// Persistent split kernel: the grid is sized to the chip (two workgroups per
// CU) and each wave takes one contiguous range of items, so it mostly walks
// consecutive splits of one (sequence, head block).  Those it accumulates
// into one running softmax (a "run") and writes one partial per run instead
// of one per split: a partial's stores share the vector-memory counter with
// the loads, and a wait for the tile in flight would otherwise also wait for
// the stores after every split.  The next tile, including the first tile of
// the wave's next item, is always in flight.
//
// Paged cache (PAGED): the rows of a sequence live in fixed-size pages of a
// shared pool, found through its block table.  A work item covers 512
// consecutive keys, i.e. at most 64 pages of >= 8 rows, so the wave loads
// the item's page numbers once (one per lane) and every row address takes
// its page from that vector with a lane shuffle.
template <int D, bool PAGED, bool FP8>
__global__ __launch_bounds__(64 * kNW) __attribute__((amdgpu_waves_per_eu(2))) void decode_split_kernel(
    const void* __restrict__ Qp, const void* __restrict__ Kp, const void* __restrict__ Vp,
    const int32_t* __restrict__ kv_lens, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    int32_t* __restrict__ ws_idx, int B, int Hq, int Hkv, int S_max, int NS, int NHB, float c, int negq,
    const int32_t* __restrict__ block_table, int lgP, int num_pages, int max_blocks) {
  using E = std::conditional_t<FP8, uint8_t, u16>;   // element of q and the caches
  const E* __restrict__ Qd = static_cast<const E*>(Qp);
  const E* __restrict__ Kc = static_cast<const E*>(Kp);
  const E* __restrict__ Vc = static_cast<const E*>(Vp);
  constexpr int BN = kBN<FP8>;               // keys per tile
  constexpr int KB = BN / 16;                // 16-key blocks per tile
  constexpr int KSTEPS = D / 32;             // k-steps of K Q^T
  constexpr int DB = D / 16;                 // 16-wide blocks of the head dim
  constexpr int TILE_BYTES = BN * D * (int)sizeof(E);
  constexpr int VLOADS = TILE_BYTES / 1024;  // 1 KiB copies per V tile
  constexpr int KLOADS = FP8 ? D / 64 : KSTEPS;      // 16-byte K loads per lane per 16 keys
  constexpr int VM_PER_TILE = KB * KLOADS + VLOADS;  // vector-memory ops per tile per lane
  __shared__ __attribute__((aligned(1024))) uint8_t Vs[kNW][2][TILE_BYTES];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, j = lane & 15;
  const int G = Hq / Hkv;
  const int HBK = Hkv * NHB;
  const int NWAV = gridDim.x * kNW;
  int t = blockIdx.x * kNW + w;

  // Total items U; wave W takes the contiguous items [W C, W C + C) with
  // C = ceil(U / #waves).  The first wave also records P(b) and U for the
  // merge, which finds the runs from them.
  const int lens0 = lane < B ? clampi(kv_lens[lane], 0, S_max) : 0;
  int U = 0;
  for (int c0 = 0; c0 < B; c0 += 64) {
    const int bb = c0 + lane;
    const int L = c0 == 0 ? lens0 : (bb < B ? clampi(kv_lens[bb], 0, S_max) : 0);
    const int ns = (L + kDecodeSplitKeys - 1) / kDecodeSplitKeys;
    const int incl = wave_incl_scan(ns, lane);
    if (blockIdx.x == 0 && w == 0 && bb < B) ws_idx[1 + bb] = U + incl - ns;
    U += __shfl(incl, 63);
  }
  U *= HBK;
  if (blockIdx.x == 0 && w == 0 && lane == 0) ws_idx[0] = U;
  const int C = (U + NWAV - 1) / NWAV;
  const int tend = min(t * C + C, U);
  t *= C;
  if (t >= tend) return;
  DecItem cur;
  find_item<BN>(t, kv_lens, lens0, B, S_max, HBK, NHB, lane, cur);
  int s0 = cur.s;   // first split of the run being accumulated

  // per-item query fragments (B operand of S^T, column = head).  bf16:
  // qf[ks] = d 32 ks + 8 g .. +7.  E4M3: qf8[2 h + e] = d 64 h + 16 g + 8 e
  // .. +7 (one 16-byte load per h); the K fragments use the same order of
  // d, so every d is paired once.  negq flips the sign bits.
  bf16x8 qf[FP8 ? 1 : KSTEPS];
  int64_t qf8[FP8 ? KSTEPS : 1];
  int hq = 0;
  bool hv = false;
  auto load_q = [&](const DecItem& it) {
    const int head = it.hb * 16 + j;
    hv = head < G;
    hq = it.hkv * G + (hv ? head : 0);
    if constexpr (FP8) {
      const u32x4* src = reinterpret_cast<const u32x4*>(Qd + ((size_t)it.b * Hq + hq) * D + 16 * g);
      const uint32_t flip = negq ? 0x80808080u : 0u;
#pragma unroll
      for (int h = 0; h < KLOADS; ++h) {
        u32x4 x = hv ? src[4 * h] : u32x4{0u, 0u, 0u, 0u};
        x ^= flip;
        qf8[2 * h] = __builtin_bit_cast(int64_t, u32x2{x[0], x[1]});
        qf8[2 * h + 1] = __builtin_bit_cast(int64_t, u32x2{x[2], x[3]});
      }
    } else {
      const u32x4* src = reinterpret_cast<const u32x4*>(Qd + ((size_t)it.b * Hq + hq) * D + 8 * g);
      const uint32_t flip = negq ? 0x80008000u : 0u;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        u32x4 x = hv ? src[4 * ks] : u32x4{0u, 0u, 0u, 0u};
        x ^= flip;
        qf[ks] = __builtin_bit_cast(bf16x8, x);
      }
    }
  };
  load_q(cur);

  // Issue tile `tile` of item `it`: K fragments into registers (A of S^T:
  // key 16 kb + j, d as in the query fragments) and the V rows into LDS
  // stage BUF.  Keys at or past k1 are replaced by key k1-1 (finite data;
  // masked below).
  u32x4 kf[2][KB][KLOADS];
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
    const int kt = it.k0 + tile * BN;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int key = min(kt + 16 * kb + j, it.k1 - 1);
      const u32x4* src = reinterpret_cast<const u32x4*>(Kc + row_off(it, key) + (FP8 ? 16 : 8) * g);
#pragma unroll
      for (int i = 0; i < KLOADS; ++i) kf[buf][kb][i] = src[4 * i];
    }
#pragma unroll
    for (int li = 0; li < VLOADS; ++li) {
      // lane's 16-byte chunk of the tile: row r, stored chunk slot, which
      // holds logical chunk ch of that row
      constexpr int CPR = D * (int)sizeof(E) / 16;   // 16-byte chunks per row
      const int p = li * 64 + lane;
      const int r = p / CPR, slot = p % CPR;
      const int ch = slot ^ (FP8 ? swz_v8<D>(r) : swz_v<D>(r));
      const int key = min(kt + r, it.k1 - 1);
      __builtin_amdgcn_global_load_lds((gptr_t*)(Vc + row_off(it, key) + ch * (16 / (int)sizeof(E))),
                                       (lptr_t*)&Vs[w][buf][li * 1024], 16, 0, kNonTemporal);
    }
  };

  // transposing-read offsets: group g covers rows 4 g + 0..3 (+16 for the
  // upper half) and logical columns 16 db + 0..15.  bf16: elements, rows
  // 4 g + j / 4 (the upper half is a second read 16 rows on).  E4M3: bytes;
  // lane j points at half j & 1 of the column block in row
  // 16 (t / 4) + 4 g + t % 4, t = j / 2, so one read gives lane j column
  // 16 db + j of the 8 rows that pair with its P^T elements (keys 32..63 of
  // the tile: a second read 32 rows on).
  int voff[DB];
  if constexpr (FP8) {
    const int tr = j >> 1;
    const int vr = 16 * (tr >> 2) + 4 * g + (tr & 3);
#pragma unroll
    for (int db = 0; db < DB; ++db) voff[db] = vr * D + 16 * (db ^ swz_v8<D>(vr)) + 8 * (j & 1);
  } else {
    const int vr = 4 * g + (j >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db)
      voff[db] = vr * D + 8 * ((2 * db + ((j & 3) >> 1)) ^ swz_v<D>(vr)) + 4 * (j & 1);
  }

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
    bool more = true, cont = false;
    if (ntile >= cur.ntiles) {
      // next item: the next split of the same (sequence, head block)
      // continues the run; anything else starts a new one
      ++t;
      ntile = 0;
      if (t >= tend) {
        more = false;
      } else if (cur.s + 1 < cur.ns) {
        nx.s = cur.s + 1;
        set_split<BN>(nx);
        cont = true;
      } else {
        find_item<BN>(t, kv_lens, lens0, B, S_max, HBK, NHB, lane, nx);
      }
    }
    if (more) {
      issue(std::integral_constant<int, buf ^ 1>{}, nx, ntile);
      wait_vmcnt<VM_PER_TILE>();
    } else {
      wait_vmcnt<0>();
    }

    const int kt = cur.k0 + tile * BN;
    f32x4 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[kb] = f32x4{};
      if constexpr (FP8) {
#pragma unroll
        for (int h = 0; h < KLOADS; ++h) {
          const u32x4 x = kf[buf][kb][h];
          s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(__builtin_bit_cast(int64_t, u32x2{x[0], x[1]}),
                                                             qf8[2 * h], s[kb], 0, 0, 0);
          s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(__builtin_bit_cast(int64_t, u32x2{x[2], x[3]}),
                                                             qf8[2 * h + 1], s[kb], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
          s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[buf][kb][ks]), qf[ks],
                                                          s[kb], 0, 0, 0);
      }
    }
    const bool need_mask = kt + BN > cur.k1;
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kt + 16 * kb + 4 * g + r;
          s[kb][r] = key < cur.k1 ? s[kb][r] : kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = xhalf_max(mx);
    // the reference m moves only when a column's maximum passes it by more
    // than kDecThresh (log2 units; a wave-uniform test), so P <= 2^8 and the
    // accumulators are rescaled on few tiles; any reference gives the same
    // result, and the partial is written with the one it was summed against
    const float mt = (mx == kNegInf) ? kNegInf : mx * c;
    if (__builtin_amdgcn_ballot_w64(mt > m + kDecThresh) != 0) {
      const float mnew = fmaxf(m, mt);
      const float alpha = fast_exp2(m - ((mnew == kNegInf) ? 0.f : mnew));
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    }
    const float nm = (m == kNegInf) ? 0.f : -m;
    // P^T operands, one per 32 keys: element e of pf[hf] is key
    // 32 hf + 16 (e/4) + 4 g + e%4
    bf16x8 pf[KB / 2];
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float p = fast_exp2(__builtin_fmaf(s[kb][r], c, nm));
        if (need_mask) p = (s[kb][r] == kNegInf) ? 0.f : p;
        ps += p;
        pf[kb >> 1][4 * (kb & 1) + r] = static_cast<__bf16>(p);
      }
    lsum += ps;

    // the matching V^T fragment: rows 4 g.. and 16 + 4 g.. (of each 32-key
    // half) of column 16 db + j
    if constexpr (FP8) {
      lds_u8* vs = (lds_u8*)&Vs[w][buf][0];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        lds_u8* vp = lds_base(vs + voff[db]);
#pragma unroll
        for (int hf = 0; hf < KB / 2; ++hf) {
          const bf16x8 a = e4m3x8_to_bf16(lds_read_tr8(vp + 32 * D * hf));
          oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[hf], oacc[db], 0, 0, 0);
        }
      }
    } else {
      lds_u16* vs = (lds_u16*)&Vs[w][buf][0];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        lds_u16* vp = lds_base(vs + voff[db]);
        const u32x2 lo = lds_read_tr16(vp);
        const u32x2 hi = lds_read_tr16(vp + 16 * D);
        const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[0], oacc[db], 0, 0, 0);
      }
    }

    if (tile == cur.ntiles - 1 && !cont) {
      // run done: write the partial into the slot of its first split (sum
      // over the four lane groups that share a query column), reset, fetch
      // the next run's queries
      float lt = lsum + __shfl_xor(lsum, 16);
      lt = xhalf_sum(lt);
      if (hv) {
        const size_t base = ((size_t)cur.b * Hq + hq) * NS + s0;
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
      s0 = nx.s;
    }
    cur = nx;
    tile = ntile;
    return more;
  };

  issue(std::integral_constant<int, 0>{}, cur, 0);
  while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{})) {
  }
}

// One workgroup (4 waves) per (query head, sequence): LSE-merge of the run
// partials.  A (sequence, head block) with items [base, base + ns) was cut
// into runs at split 0 and wherever a wave's range starts, i.e. where
// base + s is a multiple of C; each run's partial sits in the slot of its
// first split.  Wave w takes runs w, w+4, ...; lane handles D/64 columns.
// oscale multiplies the output (the V scale of an E4M3 cache, else 1).
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_ml, const int32_t* __restrict__ ws_idx,
    const int32_t* __restrict__ kv_lens, u16* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int S_max,
    int NS, int NHB, int NWAV, float oscale) {
  constexpr int PER = D / 64;
  __shared__ float red[4];
  __shared__ float part[4][D + 1];
  const int hq = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int L = clampi(kv_lens[b], 0, S_max);
  const int ns = (L + kDecodeSplitKeys - 1) / kDecodeSplitKeys;
  const int G = Hq / Hkv;
  const int hkv = hq / G, hb = (hq - hkv * G) / 16;
  const int HBK = Hkv * NHB;
  const int U = ws_idx[0];
  const int C = (U + NWAV - 1) / NWAV;
  const int base = ws_idx[1 + b] * HBK + (hkv * NHB + hb) * ns;
  // run k starts at split 0 (k = 0) or s1 + (k - 1) C
  const int rem = C > 0 ? base % C : 0;
  const int s1 = rem == 0 ? C : C - rem;
  const int nruns = ns == 0 ? 0 : 1 + (s1 < ns ? (ns - 1 - s1) / C + 1 : 0);
  auto run_start = [&](int k) { return k == 0 ? 0 : s1 + (k - 1) * C; };
  const size_t row = ((size_t)b * Hq + hq) * NS;

  // global max of the run maxima
  float M = kNegInf;
  for (int k = threadIdx.x; k < nruns; k += 256) M = fmaxf(M, ws_ml[2 * (row + run_start(k))]);
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
  for (int k = w; k < nruns; k += 4) {
    const size_t slot = row + run_start(k);
    const float wgt = fast_exp2(ws_ml[2 * slot] - M);
    tot += wgt * ws_ml[2 * slot + 1];
    const float* src = ws_o + slot * D;
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
    const float inv = has ? oscale / T : 0.f;
    u16* dst = O + ((size_t)b * Hq + hq) * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int d = lane + 64 * i;
      dst[d] = f2bf((part[0][d] + part[1][d] + part[2][d] + part[3][d]) * inv);
    }
    if (LSE != nullptr && lane == 0) LSE[(size_t)b * Hq + hq] = has ? (M + __log2f(T)) * kLn2 : kNegInf;
  }
}

template <int D, bool PAGED, bool FP8>
hipError_t launch(const DecodeArgs& a, hipStream_t st) {
  const int NS = decode_num_splits(a.S_max);
  const int G = a.Hq / a.Hkv;
  const int NHB = (G + 15) / 16;
  // scores are scale * (q_scale q).(k_scale k); the kernel works in base 2
  const double qk = FP8 ? (double)a.scale * a.q_scale * a.k_scale : (double)a.scale;
  const float c = (float)(fabs(qk) * 1.4426950408889634);
  const int negq = qk < 0.0 ? 1 : 0;
  // workgroups per CU from the launch table (built-in: two, i.e. 8 waves),
  // never more waves than work items
  const long long items = (long long)a.B * NS * a.Hkv * NHB;
  const long long per_cu = choose_decode_wgs_per_cu(FP8 ? MIATTN_E4M3 : MIATTN_BF16, D, a.S_max, items);
  const long long wgs = std::min<long long>(per_cu * device_cu_count(), (items + kNW - 1) / kNW);
  const int nwav = (int)wgs * kNW;
  hipLaunchKernelGGL((decode_split_kernel<D, PAGED, FP8>), dim3((unsigned)wgs), dim3(64 * kNW), 0, st, a.q,
                     a.k_cache, a.v_cache, a.kv_lens, a.ws_o, a.ws_ml, a.ws_idx, a.B, a.Hq, a.Hkv, a.S_max, NS, NHB,
                     c, negq, a.block_table, a.page_shift, a.num_pages, a.max_blocks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)a.Hq, (unsigned)a.B), dim3(256), 0, st, a.ws_o,
                     a.ws_ml, a.ws_idx, a.kv_lens, (u16*)a.o, a.lse, a.Hq, a.Hkv, a.S_max, NS, NHB, nwav,
                     FP8 ? a.v_scale : 1.f);
  return hipGetLastError();
}

template <bool FP8>
hipError_t launch_dtype(const DecodeArgs& a, hipStream_t st) {
  if (a.block_table != nullptr) return a.D == 64 ? launch<64, true, FP8>(a, st) : launch<128, true, FP8>(a, st);
  return a.D == 64 ? launch<64, false, FP8>(a, st) : launch<128, false, FP8>(a, st);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  return a.fp8 ? launch_dtype<true>(a, st) : launch_dtype<false>(a, st);
}

}  // namespace miattn
