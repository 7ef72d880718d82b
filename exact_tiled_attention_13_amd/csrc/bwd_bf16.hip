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
// Two kernels:
//   bwd_dq     one workgroup per (batch, query head, 32*NW query rows), the
//              forward's transposed frame (a lane owns a query row): key and
//              value tiles stream through LDS; S^T = K Q^T and dP^T = V dO^T
//              (Q and dO fragments in registers), dS^T elementwise, then
//              dQ^T += K^T dS^T with K^T from transposing LDS reads.  It
//              also computes per row Drow = sum(dO * O) and Lc = LSE * log2(e)
//              (+inf for rows that get no gradient: padding rows, rows
//              without keys), so that every weight is one exp2(c s - Lc),
//              and writes them to the workspace for bwd_dkdv_pair.
//   bwd_dkdv_pair  one workgroup per (batch, KV head, 128 keys), a lane
//              owns a key: the query heads of the group and their query
//              tiles stream through LDS.  Each block of 32 keys is owned by
//              a pair of waves: one computes S = Q K^T, P and
//              dV^T += dO^T P, the other, one step behind, dP = dO V^T,
//              dS and dK^T += Q^T dS with its partner's P (handed over
//              through LDS); K and V fragments in registers, dO^T and Q^T
//              from transposing LDS reads.
// dQ, dK and dV are each complete inside one workgroup, so nothing is
// accumulated through memory.  HBM -> LDS copies are inline-asm LDS DMA
// (dma_lds), and the fragment reads of each product are issued ahead of
// its MFMAs.
//
// LDS tiles are row-major and unpadded with the 16-byte chunks of row r
// XOR-ed by swz(r), chosen so that both read patterns on the same tile are
// free of bank conflicts: 16-byte reads of 16 consecutive rows (one chunk
// each) and transposing 8-byte reads of 4 rows x 4 chunks per 32 lanes.
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

typedef __attribute__((address_space(3))) void lptr_t;
typedef __attribute__((address_space(3))) const u16 lds_u16;
typedef __attribute__((address_space(3))) const float lds_f32;

__device__ __forceinline__ lds_u16* lds_base(lds_u16* p) {
  asm volatile("" : "+v"(p));
  return p;
}

// HBM -> LDS copy of BYTES (16 or 4) per lane by global_load_lds from a
// wave-uniform base plus a per-lane byte offset to the wave-uniform LDS
// address `lds` (lane l lands at lds + BYTES l), written as inline asm (M0 =
// the LDS address, then the load).  With an LDS DMA of the compiler builtin
// in flight, the compiler waits for every outstanding LDS read
// (lgkmcnt(0)) before each use of a fragment, where a count suffices; the
// asm copies are ordered against the LDS reads by the loop's explicit vmcnt
// waits and barriers instead.  An SALU write of M0 needs one wait state
// before an LDS DMA reads it (not interlocked, and the hazard pass does not
// look inside asm), hence the s_nop; M0 is declared clobbered.
template <int BYTES>
__device__ __forceinline__ void dma_lds(const void* gbase, uint32_t voff, const void* lds) {
  static_assert(BYTES == 16 || BYTES == 4, "LDS DMA width");
  // readfirstlane returns a signed int: each half is narrowed back to 32
  // unsigned bits before widening, or a low half with bit 31 set would
  // sign-extend into the high one
  const uint64_t g = (uint64_t)(size_t)gbase;
  const uint32_t ghi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(g >> 32));
  const uint32_t glo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)g);
  const uint8_t* gb = reinterpret_cast<const uint8_t*>(((uint64_t)ghi << 32) | (uint64_t)glo);
  const uint32_t la = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(size_t)(lptr_t*)lds);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  if constexpr (BYTES == 16)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(la), "v"(voff), "s"(gb)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(la), "v"(voff), "s"(gb)
                 : "memory", "m0");
#pragma clang diagnostic pop
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
    dma_lds<16>(base, min(off, lim), dst + li * 512);
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

// ---------------------------------------------------------------- bwd_dq
// (at most 256 registers: two waves per SIMD; left alone the compiler spends
// AccVGPRs and runs one)
template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ V, const u16* __restrict__ dO,
    const u16* __restrict__ O, const float* __restrict__ LSE, float* __restrict__ Drow, float* __restrict__ Lc,
    const int32_t* __restrict__ kv_lens, u16* __restrict__ dQ, int B, int Hq, int Hkv, int Tq, int Tk, int nqt,
    float c, float scale, int negk, int uorder) {
  constexpr int BN = 32, NS = 4, KS = D / 16, DB = D / 32, BM = 32 * NW;
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
  // Drow = sum_d dO O and Lc = LSE log2(e) of this lane's row (each lane of
  // the pair l, l ^ 32 holds half of the row's columns), kept for this
  // kernel and written for bwd_dkdv, which runs after it: 0 and +inf for
  // rows that get no gradient (padding rows, rows without keys)
  float dr, lc;
  {
    bf16x8 of[KS];
    row_fragments<KS>(of, O + qbase * D, qrow, qrow < Lq, h, 0u);
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 a = __builtin_bit_cast(u32x4, of[ks]), g = __builtin_bit_cast(u32x4, gf[ks]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        part = __builtin_fmaf(__uint_as_float(a[e] << 16), __uint_as_float(g[e] << 16), part);
        part = __builtin_fmaf(__uint_as_float(a[e] & 0xffff0000u), __uint_as_float(g[e] & 0xffff0000u), part);
      }
    }
    const float dsum = xhalf_sum(part);
    const float l = rok ? LSE[qbase + qrow] : kNegInf;
    const bool has = qrow < Lq && l != kNegInf;
    dr = has ? dsum : 0.f;
    lc = has ? l * kLog2e : __builtin_huge_valf();
    if (rok && h == 0) {
      Drow[qbase + qrow] = dr;
      Lc[qbase + qrow] = lc;
    }
  }

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
  // the fragment, Lc and Drow loads land here with the prologue copies, so
  // that no wait of the compiler's own for them (which cannot count the
  // asm copies) lands inside the loop
  wait_vm_lds<0>();
  for (int t = 0; t < ntiles; ++t) {
    const int st = t % NS;
    wait_tile<VM_PER_TILE, NS - 2>(ntiles - 1 - t);
    __builtin_amdgcn_s_barrier();
    if (t + NS - 1 < ntiles) issue(t + NS - 1, (t + NS - 1) % NS);
    const int kbase = t * BN;
    if (kbase > kmax) continue;   // wave-uniform
    lds_u16* Ks = (lds_u16*)&smem[(st * 2 + 0) * TILE];
    lds_u16* Vs = (lds_u16*)&smem[(st * 2 + 1) * TILE];
    // S^T = K Q^T and dP^T = V dO^T (32 keys x 32 queries).  The K fragment
    // reads are issued before the score MFMAs and each V fragment read right
    // after the MFMA that frees a K fragment's registers (pinned with
    // scheduling barriers: left alone, the scheduler reads each fragment
    // into the same registers just before its MFMA, which then waits out a
    // whole LDS latency); the K^T reads of dQ are issued before the mask and
    // the softmax arithmetic, which hide their latency.
    bf16x8 x[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) x[ks] = *(const __attribute__((address_space(3))) bf16x8*)(lds_base(Ks + to.row[ks]));
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[ks], qf[ks], s, 0, 0, 0);
      x[ks] = *(const __attribute__((address_space(3))) bf16x8*)(lds_base(Vs + to.row[ks]));
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // the MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // then the read
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[ks], gf[ks], dp, 0, 0, 0);
    bf16x8 kt[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) kt[db][sh] = tr_fragment<D>(Ks, to, db, sh);
    __builtin_amdgcn_sched_barrier(0);
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
        dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[db][sh], dsf[sh], dq[db], 0, 0, 0);
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

// ---------------------------------------------------------------- bwd_dkdv_pair
// dK and dV without holding K, V, dK and dV in one wave (at D = 128 that is
// past the registers of two waves per SIMD; at D = 64 the split halves each
// wave's chain of products per step and fits 128 VGPRs, two workgroups per
// CU).  The workgroup's 128 keys are four blocks of 32, each owned by a pair
// of waves on one SIMD (waves p and p + 4).  The first wave of a pair holds
// the K fragments and dV: in iteration u it computes S = Q K^T and P of
// query step u, hands P (fp32) to its partner through LDS and adds
// dV^T += dO^T P.  The second holds the V fragments and dK and finishes step
// u in iteration u + 1: dS = P (dP - Drow) with the partner's P and
// dK^T += Q^T dS, with dP = dO V^T of step u computed in iteration u beside
// the previous step's arithmetic (D = 128) or in iteration u + 1 (D = 64).
// Every product is computed once (S, dP, dV, dK) and each Q / dO tile is
// copied once per 128 keys.  The stage of step u is read in iterations u
// and u + 1, so copies run NS - 2 steps ahead.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(D == 64 ? 4 : 2))) void bwd_dkdv_pair_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ V, const u16* __restrict__ dO,
    const float* __restrict__ Drow, const float* __restrict__ Lc, const int32_t* __restrict__ kv_lens,
    u16* __restrict__ dK, u16* __restrict__ dV, int B, int Hq, int Hkv, int Tq, int Tk, int nkt, float c, float scale,
    int negk, int uorder) {
  constexpr int NW = 8, NPAIR = 4;
  constexpr int BMQ = 32, NS = 4, PD = NS - 2, KS = D / 16, DB = D / 32, BNK = 32 * NPAIR;
  constexpr int TILE = BMQ * D;
  // the Q and dO tiles are 2 LOADS wave-loads of 1 KiB, PER per wave (at
  // D = 64 waves 0-3 copy Q and waves 4-7 dO)
  constexpr int LOADS = TILE * 2 / 1024, PER = 2 * LOADS / NW;
  constexpr int VM_PER_STEP = PER + 2;   // Q, dO tiles + Lc, Drow rows
  constexpr int STAGE = 2 * TILE + 2 * 64 * 2;   // u16 elements: Q, dO, then 64 Lc + 64 Drow floats
  constexpr int PSLOT = 16 * 64;                 // floats: P of one pair, [register quad][lane][4]
  static_assert(D == 64 || D == 128, "head dimension");
  static_assert(PER * NW == 2 * LOADS, "every wave issues the same number of copies");
  __shared__ __attribute__((aligned(1024))) u16 smem[NS * STAGE];
  __shared__ __attribute__((aligned(16))) float pbuf[2 * NPAIR * PSLOT];

  const int tid = threadIdx.x;
  const int lane = tid & 63, h = lane >> 5, r32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pr = w & (NPAIR - 1);
  const bool first = w < NPAIR;   // wave-uniform: S, P, dV (else dP, dS, dK)
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
  const int wkey0 = k0 + 32 * pr;
  const int key = wkey0 + r32;

  const u16* Kp = K + ((size_t)b * Hkv + hk) * (size_t)Tk * D;
  const u16* Vp = V + ((size_t)b * Hkv + hk) * (size_t)Tk * D;

  int qfirst = 0, qend = 0;
  if (k0 < Lk) {
    qfirst = CAUSAL ? max(0, k0 - off) : 0;
    qend = Lq;
  }
  const int nsteps_h = qend > qfirst ? (qend - qfirst + BMQ - 1) / BMQ : 0;
  const int nsteps = G * nsteps_h;
  const int qwave_first = CAUSAL ? wkey0 - off : 0;

  const bool kok = key < Lk;
  const TileOffsets<D> to(lane);
  bf16x8 f[KS];   // K fragments (first waves) or V fragments (second), loaded below
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
    if constexpr (D == 128) {
      copy_tile<D, BMQ, NW>(Q + qbase * D, q0, Lq - 1, base, w, lane);
      copy_tile<D, BMQ, NW>(dO + qbase * D, q0, Lq - 1, base + TILE, w, lane);
    } else {
      const bool q_half = w < NW / 2;   // wave-uniform
      copy_tile<D, BMQ, NW / 2>((q_half ? Q : dO) + qbase * D, q0, Lq - 1, base + (q_half ? 0 : TILE),
                                      w & (NW / 2 - 1), lane);
    }
    const uint32_t roff = (uint32_t)min(q0 + r32, Lq - 1) * 4u;
    dma_lds<4>(Lc + qbase, roff, base + 2 * TILE);
    dma_lds<4>(Drow + qbase, roff, base + 2 * TILE + 128);
  };

  // At D = 128 every step is computed by every pair, also one where no row
  // sees a key of the pair (the mask makes its P zero, so it adds exact
  // zeros): the pairs run in lockstep between barriers and one workgroup
  // fills a CU, so skipping would save no time, and straight-line steps
  // schedule better.
  // register r holds query row q0 + 8 (r >> 2) + 4 h + (r & 3)
  auto q0_of = [&](int u) {
    int hq, q0;
    step_rows(u, hq, q0);
    return q0;
  };
  // (D = 64: a step where no row sees a key of the pair is skipped by both
  // of its waves, which frees their SIMD for the CU's other workgroup)
  auto skips = [&](int q0) { return wkey0 >= Lk || q0 + BMQ - 1 < qwave_first; };
  auto needs_mask = [&](int q0) {
    return (q0 + BMQ > Lq) || (wkey0 + 31 >= Lk) || (CAUSAL && wkey0 + 31 > q0 + off);
  };
  auto keep = [&](int q0, int r) {
    const int i = q0 + 8 * (r >> 2) + 4 * h + (r & 3);
    return (i < Lq) & (key < Lk) & (!CAUSAL | (key <= i + off));
  };
  auto stage_of = [&](int u) { return (lds_u16*)&smem[(u % NS) * STAGE]; };
  auto pslot_of = [&](int u) { return pbuf + ((u & 1) * NPAIR + pr) * PSLOT + 4 * lane; };
  // The fragment reads of each product are all issued before its MFMAs
  // (sched_barrier): left alone, the scheduler reads every fragment into
  // the same registers, and each MFMA then waits out a whole LDS latency.
  // product over D of one [32 x D] tile (row reads) with this wave's fragments
  auto rows_times_frags = [&](lds_u16* tile) {
    bf16x8 x[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      x[ks] = *(const __attribute__((address_space(3))) bf16x8*)(lds_base(tile + to.row[ks]));
    __builtin_amdgcn_sched_barrier(0);
    f32x16 r = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) r = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[ks], f[ks], r, 0, 0, 0);
    return r;
  };
  // acc^T += tile^T (D x 32, transposing reads) x frag (the step's 32 rows)
  auto accumulate = [&](f32x16 (&acc)[DB], lds_u16* tile, const bf16x8 (&frag)[2]) {
    bf16x8 x[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) x[db][sh] = tr_fragment<D>(tile, to, db, sh);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int sh = 0; sh < 2; ++sh)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[db][sh], frag[sh], acc[db], 0, 0, 0);
  };
  auto store = [&](const f32x16 (&acc)[DB], u16* dst, float m) {
    if (key >= Tk) return;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * db + 8 * g4 + 4 * h;
        u32x2 a;
        a[0] = pack2_bf16(acc[db][4 * g4 + 0] * m, acc[db][4 * g4 + 1] * m);
        a[1] = pack2_bf16(acc[db][4 * g4 + 2] * m, acc[db][4 * g4 + 3] * m);
        *reinterpret_cast<u32x2*>(dst + krow * D + d0) = a;
      }
  };
  // iteration t: this wave's copies of step t have landed and its P stores
  // of step t - 1 are done (the wait includes lgkmcnt(0)); after the barrier
  // the whole tile and the partner's P are visible, and the stage of step
  // t - 2 (read by the second waves in t - 1) is free
  auto sync = [&](int t) {
    if (t < nsteps) wait_tile<VM_PER_STEP, PD - 1>(nsteps - 1 - t);
    else wait_vm_lds<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (t + PD < nsteps) issue(t + PD, (t + PD) % NS);
  };
#pragma unroll
  for (int p = 0; p < PD; ++p)
    if (p < nsteps) issue(p, p);
  // K fragments (first waves, with the score sign) or V fragments (second),
  // loaded after the prologue copies and waited for here with them, so that
  // no wait of the compiler's own for these loads lands inside the loops
  // (it cannot see the copies, and its count would wait for the prefetches)
  row_fragments<KS>(f, first ? Kp : Vp, key, kok, h, (first && negk) ? 0x80008000u : 0u);
  wait_vm_lds<0>();

  f32x16 acc[DB];   // dV (first waves) or dK (second)
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};

  // The two roles run separate loops with the same waits and barriers
  // (nsteps + 1 of them).
  if (first) {
    // iteration t: S = Q K^T, P = exp2(c S - Lc) to the partner, dV^T += dO^T P
    for (int t = 0; t < nsteps; ++t) {
      sync(t);
      const int q0 = q0_of(t);
      if constexpr (D == 64)
        if (skips(q0)) continue;
      lds_u16* Qs = stage_of(t);
      lds_f32* Ls = (lds_f32*)(Qs + 2 * TILE);
      float* pslot = pslot_of(t);
      f32x16 s = rows_times_frags(Qs);
      if (needs_mask(q0)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = keep(q0, r) ? s[r] : kNegInf;
      }
      bf16x8 pf[2];
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
        const f32x4 l0 = *(const __attribute__((address_space(3))) f32x4*)(Ls + 16 * sh + 4 * h);
        const f32x4 l1 = *(const __attribute__((address_space(3))) f32x4*)(Ls + 16 * sh + 8 + 4 * h);
        f32x4 p4[2];
        uint32_t pp[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float la = e < 4 ? l0[e] : l1[e - 4], lb = e < 4 ? l0[e + 1] : l1[e - 3];
          const float p0 = fast_exp2(__builtin_fmaf(s[8 * sh + e], c, -la));
          const float p1 = fast_exp2(__builtin_fmaf(s[8 * sh + e + 1], c, -lb));
          p4[e >> 2][e & 3] = p0;
          p4[e >> 2][(e & 3) + 1] = p1;
          pp[e >> 1] = pack2_bf16(p0, p1);
        }
        *reinterpret_cast<f32x4*>(pslot + (2 * sh + 0) * 256) = p4[0];
        *reinterpret_cast<f32x4*>(pslot + (2 * sh + 1) * 256) = p4[1];
        pf[sh] = __builtin_bit_cast(bf16x8, u32x4{pp[0], pp[1], pp[2], pp[3]});
      }
      accumulate(acc, Qs + TILE, pf);
    }
    sync(nsteps);
    store(acc, dV, 1.f);
  } else {
    // iteration t: dP = dO V^T of step t (masked, kept for the next
    // iteration) and, with the partner's P of step t - 1, dS = P (dP - Drow)
    // and dK^T += Q^T dS; the dP products of step t run beside the dS
    // arithmetic of step t - 1
    auto mask_dp = [&](int u, f32x16& dp) {
      const int q0 = q0_of(u);
      if (needs_mask(q0)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = keep(q0, r) ? dp[r] : 0.f;
      }
    };
    auto ds_dk = [&](int u, const f32x16& dp) {
      lds_u16* Qs = stage_of(u);
      lds_f32* Ds = (lds_f32*)(Qs + 2 * TILE) + 64;
      const float* pslot = pslot_of(u);
      bf16x8 dsf[2];
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
        const f32x4 d0 = *(const __attribute__((address_space(3))) f32x4*)(Ds + 16 * sh + 4 * h);
        const f32x4 d1 = *(const __attribute__((address_space(3))) f32x4*)(Ds + 16 * sh + 8 + 4 * h);
        const f32x4 pa = *reinterpret_cast<const f32x4*>(pslot + (2 * sh + 0) * 256);
        const f32x4 pb = *reinterpret_cast<const f32x4*>(pslot + (2 * sh + 1) * 256);
        uint32_t pd[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = e < 4 ? pa[e] : pb[e - 4], p1 = e < 4 ? pa[e + 1] : pb[e - 3];
          const float da = e < 4 ? d0[e] : d1[e - 4], dbv = e < 4 ? d0[e + 1] : d1[e - 3];
          pd[e >> 1] = pack2_bf16(p0 * (dp[8 * sh + e] - da), p1 * (dp[8 * sh + e + 1] - dbv));
        }
        dsf[sh] = __builtin_bit_cast(bf16x8, u32x4{pd[0], pd[1], pd[2], pd[3]});
      }
      accumulate(acc, Qs, dsf);
    };
    if constexpr (D == 128) {
      sync(0);
      f32x16 dpp = f32x16{};   // dP of step t - 1
      if (nsteps > 0) {
        dpp = rows_times_frags(stage_of(0) + TILE);
        mask_dp(0, dpp);
      }
      for (int t = 1; t < nsteps; ++t) {
        sync(t);
        f32x16 dpn = rows_times_frags(stage_of(t) + TILE);
        ds_dk(t - 1, dpp);
        mask_dp(t, dpn);
        dpp = dpn;
      }
      if (nsteps > 0) {
        sync(nsteps);
        ds_dk(nsteps - 1, dpp);
      }
    } else {
      // (D = 64: the chains are short and two dP tiles in flight would not
      // fit 128 registers, so iteration t computes dP, dS and dK of step t - 1)
      sync(0);
      for (int t = 1; t <= nsteps; ++t) {
        sync(t);
        if (skips(q0_of(t - 1))) continue;
        f32x16 dp = rows_times_frags(stage_of(t - 1) + TILE);
        mask_dp(t - 1, dp);
        ds_dk(t - 1, dp);
      }
    }
    store(acc, dK, scale);
  }
}

constexpr int kDqWaves = 4;

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
    const int nqt = (a.Tq + 32 * kDqWaves - 1) / (32 * kDqWaves);
    const long long grid = (long long)nqt * a.B * a.Hq;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_dq_kernel<D, kDqWaves, CAUSAL>), dim3((unsigned)grid), dim3(64 * kDqWaves), 0, st,
                       (const u16*)a.q, (const u16*)a.k, (const u16*)a.v, (const u16*)a.dout, (const u16*)a.o, a.lse,
                       Drow, Lc, a.kv_lens, (u16*)a.dq, a.B, a.Hq, a.Hkv, a.Tq, a.Tk, nqt, c, a.scale, negk,
                       uorder(grid));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int nkt = (a.Tk + 127) / 128;
    const long long grid = (long long)nkt * a.B * a.Hkv;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_dkdv_pair_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(512), 0, st, (const u16*)a.q,
                       (const u16*)a.k, (const u16*)a.v, (const u16*)a.dout, Drow, Lc, a.kv_lens, (u16*)a.dk,
                       (u16*)a.dv, a.B, a.Hq, a.Hkv, a.Tq, a.Tk, nkt, c, a.scale, negk, uorder(grid));
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t st) {
  if (a.D == 64) return a.causal ? launch_d<64, true>(a, st) : launch_d<64, false>(a, st);
  return a.causal ? launch_d<128, true>(a, st) : launch_d<128, false>(a, st);
}

}  // namespace miattn
