// Gradients of exact attention, bf16 inputs, fp32 softmax and accumulation.
//
// What is computed (the NumPy tiled-attention build guide, Extending It; the
// self-attention interview question, Task 2 and Hint 2): dQ, dK and dV of
// L = sum(dO * O) for O = softmax(scale * Q K^T + mask) V, recomputing the
// weights tile by tile from Q, K and the forward's per-row log-sum-exp
// instead of storing them.  With P the weights and Drow_i = sum_d dO_id O_id:
//
//   dV = P^T dO,   dP = dO V^T,   dS = P * (dP - Drow),
//   dQ = scale dS K,   dK = scale dS^T Q     (GQA: dK, dV summed over the group)
//
// Three kernels:
//   bwd_prep   per row: Drow = sum(dO * O) and Lc = LSE * log2(e) (+inf for
//              rows that get no gradient: padding rows, rows without keys),
//              so that every later weight is one exp2(c s - Lc).
//   bwd_dq     one workgroup per (batch, query head, 32*NW query rows), the
//              forward's transposed frame (a lane owns a query row): key and
//              value tiles stream through LDS; S^T = K Q^T and dP^T = V dO^T
//              (Q and dO fragments in registers), dS^T elementwise, then
//              dQ^T += K^T dS^T with K^T from transposing LDS reads.
//   bwd_dkdv   one workgroup per (batch, KV head, 32*NW keys), a lane owns a
//              key: the query heads of the group and their query tiles
//              stream through LDS; S = Q K^T and dP = dO V^T (K and V
//              fragments in registers), then dV^T += dO^T P and
//              dK^T += Q^T dS with dO^T, Q^T from transposing LDS reads.
// dQ, dK and dV are each complete inside one workgroup, so nothing is
// accumulated through memory.
//
// LDS tiles are row-major and unpadded with the 16-byte chunks of row r
// XOR-ed by swz(r), chosen so that both read patterns on the same tile are
// free of bank conflicts: 16-byte reads of 16 consecutive rows (one chunk
// each) and transposing 8-byte reads of 4 rows x 4 chunks per 32 lanes.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace miattn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// bijective on every 16 consecutive rows (16-byte row reads) and, for every
// aligned 4 rows, different in the chunk bits the transposing reads span
template <int D>
__device__ __forceinline__ int swz(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70);
}
template <int PER, int R>
__device__ __forceinline__ void wait_tile(int rem) {
  if constexpr (R == 0) {
    wait_vm_lds<0>();
  } else {
    if (rem >= R) wait_vm_lds<PER * R>();
    else wait_tile<PER, R - 1>(rem);
  }
}

typedef __attribute__((address_space(1))) const void gptr_t;
typedef __attribute__((address_space(3))) void lptr_t;
typedef __attribute__((address_space(3))) const u16 lds_u16;
typedef __attribute__((address_space(3))) const float lds_f32;

__device__ __forceinline__ lds_u16* lds_base(lds_u16* p) {
  asm volatile("" : "+v"(p));
  return p;
}

// HBM -> LDS copy of rows [row0, row0 + ROWS) of a [rows x D] bf16 matrix
// into a swizzled tile; each of the NWV waves issues PER 1 KiB wave-loads.
// Rows at or past `last` are replaced by the last 16 bytes of row `last`
// (finite data; masked).  The tile's first row is wave-uniform, so each
// copy is addressed as that row's address plus the lane's byte offset
// (fixed per slot), clamped by one unsigned min.
template <int D, int ROWS, int NWV>
__device__ __forceinline__ void copy_tile(const u16* src, int row0, int last, u16* dst, int w, int lane) {
  constexpr int LOADS = ROWS * D * 2 / 1024;
  constexpr int PER = (LOADS + NWV - 1) / NWV;
  const int rb = min(row0, last);
  const uint32_t lim = (uint32_t)((min(last - rb + 1, ROWS) * D - 8) * 2);
  const uint8_t* base = reinterpret_cast<const uint8_t*>(src + (size_t)rb * D);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int li = (w + NWV * i) % LOADS;
    const int e = li * 512 + lane * 8;
    const int r = e / D, slot = (e % D) / 8;
    const int ch = slot ^ swz<D>(r);
    const uint32_t off = (uint32_t)((r * D + ch * 8) * 2);
    __builtin_amdgcn_global_load_lds((gptr_t*)(base + min(off, lim)), (lptr_t*)(dst + li * 512), 16, 0, 0);
  }
}

// MFMA B-operand fragment of row `row` of a [rows x D] bf16 matrix:
// columns 16 ks + 8 h .. + 7 for every k-step
template <int KS>
__device__ __forceinline__ void row_fragments(bf16x8 (&f)[KS], const u16* src, int row, bool ok, int h, uint32_t flip) {
  const u32x4* p = reinterpret_cast<const u32x4*>(src + (size_t)(ok ? row : 0) * (16 * KS) + 8 * h);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 x = ok ? p[2 * ks] : u32x4{0u, 0u, 0u, 0u};
    x ^= flip;
    f[ks] = __builtin_bit_cast(bf16x8, x);
  }
}

// Per-lane LDS offsets (elements) into a swizzled [32 x D] tile:
//  row reads (A operand of a product over D): row r32, chunk 2 ks + h
//  transposing reads (A operand of a product over the tile's rows): 16-lane
//  group g covers rows vr..vr+3 (+16 sh), and vr+8.. for the upper half,
//  logical columns 32 db + 16 (g & 1) + 0..15
template <int D>
struct TileOffsets {
  static constexpr int KS = D / 16, DB = D / 32;
  int row[KS];
  int tr_lo[DB], tr_hi[DB];
  __device__ __forceinline__ TileOffsets(int lane) {
    const int h = lane >> 5, r32 = lane & 31;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) row[ks] = r32 * D + 8 * ((2 * ks + h) ^ swz<D>(r32));
    const int tg = lane >> 4, tj = lane & 15;
    const int vr = 4 * (tg >> 1) + (tj >> 2);
    const int vc0 = 2 * (tg & 1) + ((tj & 3) >> 1);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      tr_lo[db] = vr * D + 8 * ((4 * db + vc0) ^ swz<D>(vr)) + 4 * (tj & 1);
      tr_hi[db] = (vr + 8) * D + 8 * ((4 * db + vc0) ^ swz<D>(vr + 8)) + 4 * (tj & 1);
    }
  }
};

// A operand (32 d x 16 tile rows) for rows 16 sh .. 16 sh + 15 of a tile
template <int D>
__device__ __forceinline__ bf16x8 tr_fragment(lds_u16* tile, const TileOffsets<D>& to, int db, int sh) {
  const u32x2 lo = lds_read_tr16(tile + to.tr_lo[db] + 16 * sh * D);
  const u32x2 hi = lds_read_tr16(tile + to.tr_hi[db] + 16 * sh * D);
  return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

__device__ __forceinline__ void valid_lengths(const int32_t* kv_lens, int b, int Tq, int Tk, int& Lq, int& Lk) {
  Lk = Tk;
  Lq = Tq;
  if (kv_lens != nullptr) {
    Lk = clampi(kv_lens[b], 0, Tk);
    if (Tq == Tk) Lq = Lk;
  }
}

// ---------------------------------------------------------------- bwd_prep
// Drow = sum_d dO * O and Lc = LSE * log2(e) per query row; 8 lanes per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const u16* __restrict__ O, const u16* __restrict__ dO,
                                                       const float* __restrict__ LSE,
                                                       const int32_t* __restrict__ kv_lens, float* __restrict__ Drow,
                                                       float* __restrict__ Lc, int Hq, int Tq, int Tk, long long rows) {
  const long long row = (long long)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int j = threadIdx.x & 7;
  float acc = 0.f;
  if (row < rows) {
    constexpr int PER = D / 8 / 8;   // 16-byte loads per lane
    const u32x4* po = reinterpret_cast<const u32x4*>(O + row * D) + j * PER;
    const u32x4* pd = reinterpret_cast<const u32x4*>(dO + row * D) + j * PER;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const u32x4 a = po[i], g = pd[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = __builtin_fmaf(__uint_as_float(a[e] << 16), __uint_as_float(g[e] << 16), acc);
        acc = __builtin_fmaf(__uint_as_float(a[e] & 0xffff0000u), __uint_as_float(g[e] & 0xffff0000u), acc);
      }
    }
  }
  acc += __shfl_xor(acc, 1, 8);
  acc += __shfl_xor(acc, 2, 8);
  acc += __shfl_xor(acc, 4, 8);
  if (row < rows && j == 0) {
    const long long bh = row / Tq;
    const int i = (int)(row - bh * Tq);
    const int b = (int)(bh / Hq);
    int Lq, Lk;
    valid_lengths(kv_lens, b, Tq, Tk, Lq, Lk);
    const float l = LSE[row];
    const bool has = i < Lq && l != kNegInf;
    Drow[row] = has ? acc : 0.f;
    Lc[row] = has ? l * kLog2e : __builtin_huge_valf();
  }
}

// ---------------------------------------------------------------- bwd_dq
// (at most 256 registers: two waves per SIMD; left alone the compiler spends
// AccVGPRs and runs one)
template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ V, const u16* __restrict__ dO,
    const float* __restrict__ Drow, const float* __restrict__ Lc, const int32_t* __restrict__ kv_lens,
    u16* __restrict__ dQ, int B, int Hq, int Hkv, int Tq, int Tk, int nqt, float c, float scale, int negk,
    int uorder) {
  constexpr int BN = 32, NS = 3, KS = D / 16, DB = D / 32, BM = 32 * NW;
  constexpr int TILE = BN * D;
  constexpr int LOADS = TILE * 2 / 1024, PER = (LOADS + NW - 1) / NW, VM_PER_TILE = 2 * PER;
  __shared__ __attribute__((aligned(1024))) u16 smem[NS * 2 * TILE];   // [stage][K, V][tile]

  const int tid = threadIdx.x;
  const int lane = tid & 63, h = lane >> 5, r32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // workgroup -> (query tile, batch, head): heaviest tiles first; for grids
  // of several rounds with a multiple of 8 (batch, KV head) units (uorder)
  // each XCD takes whole units, so its resident workgroups stream one
  // head's K/V through L2 together
  const int G = Hq / Hkv;
  const int id = blockIdx.x;
  int tq_slot, b, hq;
  if (uorder) {
    const int k = id >> 3, ul = k / (G * nqt), r = k - ul * (G * nqt);
    tq_slot = r / G;
    const int u = (id & 7) + 8 * ul;
    b = u / Hkv;
    hq = (u - b * Hkv) * G + (r - tq_slot * G);
  } else {
    const int BH = B * Hq;
    tq_slot = id / BH;
    const int bh = id - tq_slot * BH;
    b = bh / Hq;
    hq = bh - b * Hq;
  }
  const int qt = nqt - 1 - tq_slot;
  const int hk = hq / G;
  int Lq, Lk;
  valid_lengths(kv_lens, b, Tq, Tk, Lq, Lk);
  const int off = Lk - Lq;
  const int q0 = qt * BM;

  const size_t qbase = ((size_t)b * Hq + hq) * (size_t)Tq;
  const u16* Kp = K + ((size_t)b * Hkv + hk) * (size_t)Tk * D;
  const u16* Vp = V + ((size_t)b * Hkv + hk) * (size_t)Tk * D;

  int kend = 0;
  const int rows_end = min(q0 + BM, Lq);
  if (rows_end > q0) kend = CAUSAL ? min(Lk, rows_end + off) : Lk;
  if (kend < 0) kend = 0;
  const int ntiles = (kend + BN - 1) / BN;

  const int wrow0 = q0 + 32 * w;
  const int qrow = wrow0 + r32;
  int kmax = -1;
  if (wrow0 < Lq) kmax = CAUSAL ? min(Lk - 1, min(wrow0 + 31, Lq - 1) + off) : Lk - 1;
  const int kfull = CAUSAL ? min(Lk - 1, wrow0 + off) : Lk - 1;
  const int lim = CAUSAL ? min(Lk - 1, qrow + off) : Lk - 1;

  // Q and dO fragments of this lane's row (B operands); the score sign for a
  // negative scale goes into Q (K is used unsigned by dQ = scale dS K)
  // (rows at or past Lq are padding: their dO may hold anything and their
  // fragments are zero, so dP and dS stay finite and zero there)
  bf16x8 qf[KS], gf[KS];
  const bool rok = qrow < Tq;
  row_fragments<KS>(qf, Q + qbase * D, qrow, qrow < Lq, h, negk ? 0x80008000u : 0u);
  row_fragments<KS>(gf, dO + qbase * D, qrow, qrow < Lq, h, 0u);
  const float lc = rok ? Lc[qbase + qrow] : __builtin_huge_valf();
  const float dr = rok ? Drow[qbase + qrow] : 0.f;

  const TileOffsets<D> to(lane);
  f32x16 dq[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dq[i] = f32x16{};

  auto issue = [&](int t, int st) {
    copy_tile<D, BN, NW>(Kp, t * BN, Lk - 1, smem + (st * 2 + 0) * TILE, w, lane);
    copy_tile<D, BN, NW>(Vp, t * BN, Lk - 1, smem + (st * 2 + 1) * TILE, w, lane);
  };
#pragma unroll
  for (int p = 0; p < NS - 1; ++p)
    if (p < ntiles) issue(p, p);
  for (int t = 0; t < ntiles; ++t) {
    const int st = t % NS;
    wait_tile<VM_PER_TILE, NS - 2>(ntiles - 1 - t);
    __builtin_amdgcn_s_barrier();
    if (t + NS - 1 < ntiles) issue(t + NS - 1, (t + NS - 1) % NS);
    const int kbase = t * BN;
    if (kbase > kmax) continue;   // wave-uniform
    lds_u16* Ks = (lds_u16*)&smem[(st * 2 + 0) * TILE];
    lds_u16* Vs = (lds_u16*)&smem[(st * 2 + 1) * TILE];
    // S^T = K Q^T and dP^T = V dO^T (32 keys x 32 queries)
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 ka = *(const __attribute__((address_space(3))) bf16x8*)(lds_base(Ks + to.row[ks]));
      const bf16x8 va = *(const __attribute__((address_space(3))) bf16x8*)(lds_base(Vs + to.row[ks]));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, gf[ks], dp, 0, 0, 0);
    }
    if (kbase + BN - 1 > kfull) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kbase + 8 * (r >> 2) + 4 * h + (r & 3);
        s[r] = key <= lim ? s[r] : kNegInf;
      }
    }
    // dS^T = P^T (dP^T - Drow), P^T = exp2(c s - Lc); bf16 pairs for the
    // B operand of dQ^T += K^T dS^T
    bf16x8 dsf[2];
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
      uint32_t pk[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(s[8 * sh + e], c, -lc));
        const float p1 = fast_exp2(__builtin_fmaf(s[8 * sh + e + 1], c, -lc));
        pk[e >> 1] = pack2_bf16(p0 * (dp[8 * sh + e] - dr), p1 * (dp[8 * sh + e + 1] - dr));
      }
      dsf[sh] = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int sh = 0; sh < 2; ++sh)
        dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_fragment<D>(Ks, to, db, sh), dsf[sh], dq[db], 0, 0, 0);
  }
  wait_vm_lds<0>();

  if (rok) {
    u16* orow = dQ + (qbase + qrow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        u32x2 pk;
        pk[0] = pack2_bf16(dq[db][4 * g4 + 0] * scale, dq[db][4 * g4 + 1] * scale);
        pk[1] = pack2_bf16(dq[db][4 * g4 + 2] * scale, dq[db][4 * g4 + 3] * scale);
        *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * g4 + 4 * h) = pk;
      }
  }
}

// ---------------------------------------------------------------- bwd_dkdv
// At D=128 one pass would hold the K and V fragments and the dK and dV
// accumulators (192 registers per lane) plus the step's scores and
// addresses: past 256 VGPRs, where the compiler parks the accumulators in
// AccVGPRs and copies all 128 of them both ways on every step.  So D=128
// runs two passes over the query tiles: first S, P and dV, then S, dP, dS
// and dK (S is computed twice, 25% more matrix work), each pass holding 64
// accumulators, which fits two waves per SIMD.  D=64 runs both in one pass.
template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dkdv_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ V, const u16* __restrict__ dO,
    const float* __restrict__ Drow, const float* __restrict__ Lc, const int32_t* __restrict__ kv_lens,
    u16* __restrict__ dK, u16* __restrict__ dV, int B, int Hq, int Hkv, int Tq, int Tk, int nkt, float c, float scale,
    int negk, int uorder) {
  constexpr int BMQ = 32, NS = 3, KS = D / 16, DB = D / 32, BNK = 32 * NW;
  constexpr int TILE = BMQ * D;
  constexpr int LOADS = TILE * 2 / 1024, PER = (LOADS + NW - 1) / NW;
  constexpr int VM_PER_STEP = 2 * PER + 2;   // Q, dO tiles + Lc, Drow rows
  constexpr int STAGE = 2 * TILE + 2 * 64 * 2;   // u16 elements: Q, dO, then 64 Lc + 64 Drow floats
  constexpr bool SPLIT = D == 128;
  __shared__ __attribute__((aligned(1024))) u16 smem[NS * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, h = lane >> 5, r32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // workgroup -> (key tile, batch, KV head); as for dQ, with uorder each
  // XCD takes whole units, so its resident workgroups stream one unit's Q
  // and dO through L2 together
  const int NU = B * Hkv;
  const int id = blockIdx.x;
  int kt, b, hk;
  if (uorder) {
    const int k = id >> 3, ul = k / nkt;
    kt = k - ul * nkt;
    const int u = (id & 7) + 8 * ul;
    b = u / Hkv;
    hk = u - b * Hkv;
  } else {
    kt = id / NU;
    const int bh = id - kt * NU;
    b = bh / Hkv;
    hk = bh - b * Hkv;
  }
  const int G = Hq / Hkv;
  int Lq, Lk;
  valid_lengths(kv_lens, b, Tq, Tk, Lq, Lk);
  const int off = Lk - Lq;
  const int k0 = kt * BNK;
  const int wkey0 = k0 + 32 * w;   // this wave's keys [wkey0, wkey0 + 32)
  const int key = wkey0 + r32;     // this lane's key

  const u16* Kp = K + ((size_t)b * Hkv + hk) * (size_t)Tk * D;
  const u16* Vp = V + ((size_t)b * Hkv + hk) * (size_t)Tk * D;

  // query rows that see any key of the workgroup / of this wave
  int qfirst = 0, qend = 0;
  if (k0 < Lk) {
    qfirst = CAUSAL ? max(0, k0 - off) : 0;
    qend = Lq;
  }
  const int nsteps_h = qend > qfirst ? (qend - qfirst + BMQ - 1) / BMQ : 0;
  const int nsteps = G * nsteps_h;
  const int qwave_first = CAUSAL ? wkey0 - off : 0;   // first row that sees this wave's first key

  // K fragments of this lane's key (B operand of S = Q K^T)
  bf16x8 kf[KS];
  const bool kok = key < Lk;
  row_fragments<KS>(kf, Kp, key, kok, h, negk ? 0x80008000u : 0u);
  const TileOffsets<D> to(lane);
  const size_t krow = ((size_t)b * Hkv + hk) * (size_t)Tk + key;

  auto step_rows = [&](int sidx, int& hq, int& q0) {
    const int g = sidx / nsteps_h;
    hq = hk * G + g;
    q0 = qfirst + (sidx - g * nsteps_h) * BMQ;
  };
  auto issue = [&](int sidx, int st) {
    int hq, q0;
    step_rows(sidx, hq, q0);
    const size_t qbase = ((size_t)b * Hq + hq) * (size_t)Tq;
    u16* base = smem + st * STAGE;
    // rows at or past Lq (padding; may hold anything) are replaced by data
    // of row Lq - 1, and the mask below gives them no weight
    copy_tile<D, BMQ, NW>(Q + qbase * D, q0, Lq - 1, base, w, lane);
    copy_tile<D, BMQ, NW>(dO + qbase * D, q0, Lq - 1, base + TILE, w, lane);
    const int row = min(q0 + r32, Lq - 1);
    __builtin_amdgcn_global_load_lds((gptr_t*)(Lc + qbase + row), (lptr_t*)(base + 2 * TILE), 4, 0, 0);
    __builtin_amdgcn_global_load_lds((gptr_t*)(Drow + qbase + row), (lptr_t*)(base + 2 * TILE + 128), 4, 0, 0);
  };

  // One pass over the query tiles.  PASS 0: dV only; 1: dK only; 2: both.
  auto run = [&](auto PASSC) {
    constexpr int PASS = decltype(PASSC)::value;
    constexpr bool DO_V = PASS != 1, DO_K = PASS != 0;
    // V fragments of this lane's key (B operand of dP = dO V^T)
    bf16x8 vf[DO_K ? KS : 1];
    if constexpr (DO_K) row_fragments<KS>(vf, Vp, key, kok, h, 0u);
    f32x16 dk[DO_K ? DB : 1], dv[DO_V ? DB : 1];
#pragma unroll
    for (int i = 0; i < DB; ++i) {
      if constexpr (DO_K) dk[i] = f32x16{};
      if constexpr (DO_V) dv[i] = f32x16{};
    }

#pragma unroll
    for (int p = 0; p < NS - 1; ++p)
      if (p < nsteps) issue(p, p);
    for (int sidx = 0; sidx < nsteps; ++sidx) {
      const int st = sidx % NS;
      wait_tile<VM_PER_STEP, NS - 2>(nsteps - 1 - sidx);
      __builtin_amdgcn_s_barrier();
      if (sidx + NS - 1 < nsteps) issue(sidx + NS - 1, (sidx + NS - 1) % NS);
      int hq, q0;
      step_rows(sidx, hq, q0);
      // wave-uniform: no row of this step sees a key of this wave
      if (wkey0 >= Lk || q0 + BMQ - 1 < qwave_first) continue;
      lds_u16* Qs = (lds_u16*)&smem[st * STAGE];
      lds_u16* Gs = Qs + TILE;
      lds_f32* Ls = (lds_f32*)(Qs + 2 * TILE);
      lds_f32* Ds = Ls + 64;
      // S = Q K^T (and dP = dO V^T) (32 queries x 32 keys; a lane owns a key)
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 qa = *(const __attribute__((address_space(3))) bf16x8*)(lds_base(Qs + to.row[ks]));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], s, 0, 0, 0);
        if constexpr (DO_K) {
          const bf16x8 ga = *(const __attribute__((address_space(3))) bf16x8*)(lds_base(Gs + to.row[ks]));
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vf[ks], dp, 0, 0, 0);
        }
      }
      // register r holds query row q0 + 8 (r >> 2) + 4 h + (r & 3)
      const bool need_mask = (q0 + BMQ > Lq) || (wkey0 + 31 >= Lk) || (CAUSAL && wkey0 + 31 > q0 + off);
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = q0 + 8 * (r >> 2) + 4 * h + (r & 3);
          const bool ok = i < Lq && key < Lk && (!CAUSAL || key <= i + off);
          s[r] = ok ? s[r] : kNegInf;
          if constexpr (DO_K) dp[r] = ok ? dp[r] : 0.f;
        }
      }
      bf16x8 pf[2], dsf[2];
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
        const f32x4 l0 = *(const __attribute__((address_space(3))) f32x4*)(Ls + 16 * sh + 4 * h);
        const f32x4 l1 = *(const __attribute__((address_space(3))) f32x4*)(Ls + 16 * sh + 8 + 4 * h);
        f32x4 d0{}, d1{};
        if constexpr (DO_K) {
          d0 = *(const __attribute__((address_space(3))) f32x4*)(Ds + 16 * sh + 4 * h);
          d1 = *(const __attribute__((address_space(3))) f32x4*)(Ds + 16 * sh + 8 + 4 * h);
        }
        uint32_t pp[4], pd[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          // registers 8 sh + e, e + 1 are rows 16 sh + 8 (e >> 2) + 4 h + (e & 3), +1
          const float la = e < 4 ? l0[e] : l1[e - 4], lb = e < 4 ? l0[e + 1] : l1[e - 3];
          const float p0 = fast_exp2(__builtin_fmaf(s[8 * sh + e], c, -la));
          const float p1 = fast_exp2(__builtin_fmaf(s[8 * sh + e + 1], c, -lb));
          if constexpr (DO_V) pp[e >> 1] = pack2_bf16(p0, p1);
          if constexpr (DO_K) {
            const float da = e < 4 ? d0[e] : d1[e - 4], dbv = e < 4 ? d0[e + 1] : d1[e - 3];
            pd[e >> 1] = pack2_bf16(p0 * (dp[8 * sh + e] - da), p1 * (dp[8 * sh + e + 1] - dbv));
          }
        }
        if constexpr (DO_V) pf[sh] = __builtin_bit_cast(bf16x8, u32x4{pp[0], pp[1], pp[2], pp[3]});
        if constexpr (DO_K) dsf[sh] = __builtin_bit_cast(bf16x8, u32x4{pd[0], pd[1], pd[2], pd[3]});
      }
      // dV^T += dO^T P and dK^T += Q^T dS (D x 32 keys)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
          if constexpr (DO_V)
            dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_fragment<D>(Gs, to, db, sh), pf[sh], dv[db], 0, 0, 0);
          if constexpr (DO_K)
            dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_fragment<D>(Qs, to, db, sh), dsf[sh], dk[db], 0, 0, 0);
        }
    }
    // every copy has landed and every LDS read is done; after the barrier
    // the next pass may refill the stages
    wait_vm_lds<0>();
    __builtin_amdgcn_s_barrier();

    if (key < Tk) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = 32 * db + 8 * g4 + 4 * h;
          if constexpr (DO_K) {
            u32x2 a;
            a[0] = pack2_bf16(dk[db][4 * g4 + 0] * scale, dk[db][4 * g4 + 1] * scale);
            a[1] = pack2_bf16(dk[db][4 * g4 + 2] * scale, dk[db][4 * g4 + 3] * scale);
            *reinterpret_cast<u32x2*>(dK + krow * D + d0) = a;
          }
          if constexpr (DO_V) {
            u32x2 v2;
            v2[0] = pack2_bf16(dv[db][4 * g4 + 0], dv[db][4 * g4 + 1]);
            v2[1] = pack2_bf16(dv[db][4 * g4 + 2], dv[db][4 * g4 + 3]);
            *reinterpret_cast<u32x2*>(dV + krow * D + d0) = v2;
          }
        }
    }
  };
  if constexpr (SPLIT) {
    run(std::integral_constant<int, 0>{});
    run(std::integral_constant<int, 1>{});
  } else {
    run(std::integral_constant<int, 2>{});
  }
}

constexpr int kDqWaves = 4;
constexpr int kDkdvWaves = 4;

template <int D, bool CAUSAL>
hipError_t launch_d(const BwdArgs& a, hipStream_t st) {
  const long long rows = (long long)a.B * a.Hq * a.Tq;
  float* Drow = a.ws;
  float* Lc = a.ws + rows;
  const float c = fmaxf(fabsf(a.scale) * kLog2e, 1e-30f);
  const int negk = a.scale < 0.f ? 1 : 0;
  // per-XCD unit order of the dQ and dK/dV workgroups once a grid takes
  // several rounds (smaller grids keep the heavy-first order across heads)
  auto uorder = [&](long long grid) {
    return ((a.B * a.Hkv) % 8 == 0 && grid >= 4LL * device_cu_count()) ? 1 : 0;
  };
  {
    const long long grid = (rows + 31) / 32;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)grid), dim3(256), 0, st, (const u16*)a.o,
                       (const u16*)a.dout, a.lse, a.kv_lens, Drow, Lc, a.Hq, a.Tq, a.Tk, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int nqt = (a.Tq + 32 * kDqWaves - 1) / (32 * kDqWaves);
    const long long grid = (long long)nqt * a.B * a.Hq;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_dq_kernel<D, kDqWaves, CAUSAL>), dim3((unsigned)grid), dim3(64 * kDqWaves), 0, st,
                       (const u16*)a.q, (const u16*)a.k, (const u16*)a.v, (const u16*)a.dout, Drow, Lc, a.kv_lens,
                       (u16*)a.dq, a.B, a.Hq, a.Hkv, a.Tq, a.Tk, nqt, c, a.scale, negk, uorder(grid));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int nkt = (a.Tk + 32 * kDkdvWaves - 1) / (32 * kDkdvWaves);
    const long long grid = (long long)nkt * a.B * a.Hkv;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, kDkdvWaves, CAUSAL>), dim3((unsigned)grid), dim3(64 * kDkdvWaves), 0, st,
                       (const u16*)a.q, (const u16*)a.k, (const u16*)a.v, (const u16*)a.dout, Drow, Lc, a.kv_lens,
                       (u16*)a.dk, (u16*)a.dv, a.B, a.Hq, a.Hkv, a.Tq, a.Tk, nkt, c, a.scale, negk, uorder(grid));
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t st) {
  if (a.D == 64) return a.causal ? launch_d<64, true>(a, st) : launch_d<64, false>(a, st);
  return a.causal ? launch_d<128, true>(a, st) : launch_d<128, false>(a, st);
}

}  // namespace miattn
