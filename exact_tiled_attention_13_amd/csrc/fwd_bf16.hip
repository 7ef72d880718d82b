// Exact tiled attention, prefill, bf16 inputs, fp32 softmax and accumulation.
//
// What is computed ("Implementing attention from scratch", Stable softmax,
// Masks and KV caching; Transformers in Action section 9.4.1, Figure 9.8):
// O = softmax(scale * Q K^T + mask) V, one query tile at a time, streaming
// key/value tiles through on-chip memory with the online softmax: a running
// row maximum m and denominator l, and the partial output rescaled by
// exp(m_old - m_new) when the maximum grows.  Scores never leave registers.
//
// gfx950 mapping.  A workgroup owns BM = 32*NWG query rows of one (batch,
// query head).  Its waves form KSPLIT key groups of NWG waves: every group
// covers all BM rows (32 per wave) over its own share of the key tiles
// (every KSPLIT-th tile), and the groups' partial (m, l, O) are merged
// through LDS at the end with the same rescale rule.  KSPLIT > 1 shortens the chain of key tiles a
// workgroup walks through, for grids too small to fill the chip.  Each wave
// works in the transposed frame, where every lane owns one query row:
//
//   S^T (keys x queries) = K Q^T     v_mfma_f32_32x32x16_bf16; A = K from LDS,
//                                    B = Q fragments held in registers
//   O^T (d x queries)   += V^T P^T   A = V^T from transposing LDS reads of the
//                                    row-major V tile; B = P taken straight
//                                    from the S^T accumulators
//
// so the row maximum is a per-lane max plus one exchange between the wave
// halves, the row sum stays per lane until the epilogue, and rescaling the
// output needs no data movement.  Softmax runs in base 2 with
// scale*log2(e) folded into one FMA; the row sum adds the fp32 P before
// they are rounded to bf16 for the P V product (summing the rounded values
// instead would move the log-sum-exp of rows with few keys by up to ~2e-3).
//
// Rescale threshold: the reference maximum m used in exp2(s - m) is only
// moved when a row's true maximum exceeds it by more than 2^kThresh.  Any
// reference value gives the same result (the final O = acc / l and
// LSE = m + log2 l use the same m); the threshold only bounds P <= 2^8 and
// lets the wave skip the rescale of its accumulators (a wave-uniform branch)
// on almost every tile.
//
// K and V tiles (BN keys) are copied HBM -> LDS by global_load_lds_dwordx4
// (no staging registers) into an NS-stage ring per key group: the copies
// of the next tiles are in flight while a tile is computed, and each wave
// waits (vmcnt) only for the copies of the tiles it is about to read.  Rows are
// stored unpadded, with the 16-byte chunks of each row XOR-permuted (swz_k,
// swz_v below) so that the 16-byte K reads and the transposing V reads are
// free of bank conflicts.
#include "../../include/miattn.h"
#include "device_common.h"
#include "launch.h"


namespace miattn {
namespace {

template <int D, int NWG, int KSPLIT, bool FP8>
struct FwdCfg {
  static constexpr int NW = NWG * KSPLIT;           // waves per workgroup
  // keys per tile and LDS stages per key group (tiles in flight + 1; E4M3
  // keeps one more stage, whose V tile is being widened).  One key group:
  // 64-key tiles, 3-4 stages (64-128 KiB).  Two key groups: two stages
  // each within 64-80 KiB in all, so that two workgroups share a CU.
  static constexpr int BN = (KSPLIT > 1 && D == 128) ? 32 : 64;
  // one key group, D=128: the loop is software-pipelined (the scores of
  // tile j+1 are computed next to the softmax of tile j), so the K half of
  // a tile is read one iteration earlier and the ring keeps 4 stages (bf16
  // 4 x 32 KiB; E4M3 4 x 16 KiB plus the two widened V tiles)
  static constexpr bool PIPE = KSPLIT == 1 && D == 128;
  // unpipelined D = 128 bf16 (two key groups, one workgroup per CU): the
  // fragment reads of each product are issued ahead of its MFMAs, the V^T
  // reads before the softmax of the tile (registers to spare)
  static constexpr bool AHEAD = !PIPE && D == 128 && !FP8;
  static constexpr int NS = PIPE ? 4 : ((KSPLIT > 1) ? 2 : (D == 64 ? 4 : 3)) + (FP8 ? 1 : 0);
  static constexpr int KB = BN / 32;                // 32-key blocks per tile
  static constexpr int BM = 32 * NWG;               // query rows per workgroup
  static constexpr int NT = 64 * NW;                // threads per workgroup
  static constexpr int KS = D / 16;                 // k-steps of Q K^T (bf16)
  static constexpr int KK = D / 64;                 // k-steps of Q K^T (E4M3)
  static constexpr int DB = D / 32;                 // 32-wide blocks of the head dim
  static constexpr int ESZ = FP8 ? 1 : 2;           // bytes per input element
  static constexpr int TILE = BN * D;               // elements per K or V tile
  static constexpr int TB = TILE * ESZ;             // bytes per K or V tile in a stage
  static constexpr int LOADS = TB / 1024;           // 1 KiB wave-loads per tensor per tile
  // every wave of a group issues the same number of copies (vmcnt
  // accounting is per wave); when NWG does not divide 2 LOADS some waves
  // repeat another wave's copy, which writes the same bytes to the same place
  static constexpr int VMEM_PER_TILE = (2 * LOADS + NWG - 1) / NWG;
  static constexpr int VW_BYTES = FP8 ? 2 * TILE * 2 : 0;   // widened V tiles (bf16, two buffers)
  static constexpr int RING_BYTES = NS * 2 * TB + VW_BYTES;
  static constexpr int RING = RING_BYTES / 2;       // u16 elements per key group
  static constexpr int SMEM = KSPLIT * RING;
  static constexpr int WE = TILE / (64 * NWG);      // V elements each thread widens per tile (E4M3)
  // merge through the (then idle) rings: the partial (m, l) of groups 1..,
  // then their accumulators, DBR blocks of 32 columns per round
  static constexpr int ML_FLOATS = (KSPLIT - 1) * NWG * 64 * 2;
  static constexpr int BLK_FLOATS = (KSPLIT - 1) * NWG * 64 * 16;
  static constexpr int AVAIL = SMEM / 2 - ML_FLOATS;
  static constexpr int DBR = (DB * BLK_FLOATS <= AVAIL) ? DB : (DB % 2 == 0 && DB / 2 * BLK_FLOATS <= AVAIL) ? DB / 2 : 1;
  static_assert(KSPLIT == 1 || BLK_FLOATS <= AVAIL, "merge buffer must fit in the rings");
  static_assert(SMEM * 2 <= 160 * 1024, "LDS");
  static_assert(!FP8 || WE == 8 || WE == 16, "widening granule");
};

constexpr float kThresh = 8.0f;

// LDS chunk permutations.  gfx950 LDS has 64 banks of 4 bytes; a 16-byte
// read is serviced 16 lanes at a time and a transposing 8-byte read 32 lanes
// at a time, so every such lane group must touch distinct 16-byte slots
// modulo 256 bytes.  The 16-byte chunks of tile row r are stored XOR-ed:
//   K (read as 16 consecutive rows x one chunk):  D=128: r & 15;  D=64: (r >> 1) & 7
//   V (read as 4 rows x 4 chunks per 32 lanes):   D=128: 4 (r & 3); D=64: 4 ((r >> 1) & 1)
template <int D>
__device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
// E4M3 K rows are D bytes (8 or 4 chunks); 16 consecutive rows x one chunk:
//   D=128: (r >> 1) & 7;  D=64: (r >> 2) & 3
template <int D>
__device__ __forceinline__ int swz_k8(int r) { return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
template <int D>
__device__ __forceinline__ int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// s_waitcnt lgkmcnt(0) only (vmcnt 63, expcnt 7)
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt in bits 3:0 and 15:14)
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70);
}
// wait until this wave's copies of the current tile have landed, given that
// `rem` later tiles (PER copies each) may still be in flight
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
typedef __attribute__((address_space(3))) const uint8_t lds_u8;
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Hide a per-lane LDS base from loop-invariant code motion (an empty asm
// that emits nothing), so that each group of fragment reads is one add plus
// reads whose constant row offsets fold into the DS immediate.
template <typename P>
__device__ __forceinline__ P* lds_base(P* p) {
  asm volatile("" : "+v"(p));
  return p;
}

// Orders of the tiles over the workgroup ids (one tile per workgroup; the
// hardware dispatches ids in increasing order as CUs free up).
enum : int { ORDER_ID_NATURAL = 0, ORDER_ID_UNITS = 1, ORDER_ID_ZIG = 2, ORDER_ID_LIST = 3 };
// ragged grids are ordered by work for up to this many sequences (one per lane)
constexpr int kOrderMaxB = 64;

// Tiles of a sequence with work (key tiles) greater than w, given its valid
// keys Lk, query tiles with a valid row nq and causal offset off = Lk - Lq.
// Work is nondecreasing in the tile index, so these are the last ones.
template <int BM, int BN, bool CAUSAL>
__device__ __forceinline__ int tiles_above(int Lk, int nq, int off, int w) {
  if (nq == 0 || (long long)Lk <= (long long)w * BN) return 0;
  if (!CAUSAL) return nq;
  // the tile's last row plus off must pass w*BN: (qt+1) BM + off > w BN
  const long long x = (long long)w * BN - off;
  const long long qmin = x < 0 ? 0 : x / BM;
  return (int)max(0LL, (long long)nq - qmin);
}

// sum over lanes 0..n-1 of a per-lane value, on the scalar unit
__device__ __forceinline__ int lanes_sum(int v, int n) {
  int s = 0;
  for (int l = 0; l < n; ++l) s += __builtin_amdgcn_readlane(v, l);
  return s;
}

// Tile list of a ragged grid (lengths in kv_lens, B <= kOrderMaxB):
// position p -> (b, hq, hk, qt), computed alike by every wave.  Tiles by
// work (key tiles), most first; ties by sequence, then tile from the last,
// then query head with the KV head fastest; then the tiles with no work at
// all (padding rows, rows that see no key), which only write zeros.  Lane l
// holds sequence l; the sums over sequences run on the scalar unit.
// Workgroups dispatched in this order fill the chip longest-first, and the
// short zero-writing ones fill in the tail.
template <int BM, int BN, bool CAUSAL>
__device__ __forceinline__ void tile_at(int p, const int32_t* __restrict__ kv_lens, int B, int Hq, int Hkv, int Tq,
                                        int Tk, int nqt, int& b, int& hq, int& hk, int& qt) {
  const int G = Hq / Hkv;
  const int lane = threadIdx.x & 63;
  int Lk = 0, nq = 0, off = 0;
  if (lane < B) {
    Lk = clampi(kv_lens[lane], 0, Tk);
    const int Lq = (Tq == Tk) ? Lk : Tq;
    nq = (Lq + BM - 1) / BM;
    off = Lk - Lq;
  }
  const int wmax = (Tk + BN - 1) / BN;
  const int above0 = tiles_above<BM, BN, CAUSAL>(Lk, nq, off, 0);
  const int F0 = Hq * lanes_sum(above0, B);
  int cnt_hi, cnt_lo;   // this lane's tiles with work > w* and > w* - 1
  int r;                // rank inside the group of work w*
  const bool zero = p >= F0;
  if (zero) {
    r = p - F0;
    cnt_hi = above0;
    cnt_lo = 0;
  } else {
    // smallest w >= 1 with (tiles of work > w) <= p: the work of p
    int lo = 1, hi = wmax;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (Hq * lanes_sum(tiles_above<BM, BN, CAUSAL>(Lk, nq, off, mid), B) <= p) hi = mid;
      else lo = mid + 1;
    }
    cnt_hi = tiles_above<BM, BN, CAUSAL>(Lk, nq, off, lo);
    cnt_lo = tiles_above<BM, BN, CAUSAL>(Lk, nq, off, lo - 1);
    r = p - Hq * lanes_sum(cnt_hi, B);
  }
  // tiles of the group per sequence; the sequence whose range holds r
  const int mine = zero ? (lane < B ? nqt - cnt_hi : 0) : (cnt_lo - cnt_hi);
  int l = 0, pre = 0;
  for (; l < B; ++l) {
    const int ml = __builtin_amdgcn_readlane(mine, l);
    if (r < Hq * (pre + ml)) break;
    pre += ml;
  }
  if (l == B) {   // not reached (every position lies in one sequence's range); computes nothing
    b = 0;
    hq = 0;
    hk = 0;
    qt = nqt;
    return;
  }
  b = l;
  const int jj = r - Hq * pre;
  const int t = jj / Hq, hr = jj - t * Hq;
  const int g = hr / Hkv;
  hk = hr - g * Hkv;
  hq = hk * G + g;
  const int nq_l = __builtin_amdgcn_readlane(nq, l), hi_l = __builtin_amdgcn_readlane(cnt_hi, l);
  if (zero) {
    const int zlo = nq_l - hi_l;   // tiles [0, zlo) and [nq, nqt) have no work
    qt = t < zlo ? t : nq_l + (t - zlo);
  } else {
    qt = nq_l - hi_l - 1 - t;      // the group's tiles, last first
  }
}

template <int D, int NWG, int KSPLIT, bool CAUSAL, bool FP8>
__device__ __forceinline__ void fwd_tile(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    u16* __restrict__ O, float* __restrict__ LSE, const int32_t* __restrict__ kv_lens,
    int B, int Hq, int Hkv, int Tq, int Tk, float c, int negq, float oscale, u16* smem, int b, int hq, int hk,
    int qt) {
  using C = FwdCfg<D, NWG, KSPLIT, FP8>;
  const int tid = threadIdx.x;
  const int lane = tid & 63, h = lane >> 5, r32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = w / NWG;          // key group
  const int wg = w - kg * NWG;     // wave within the group = its 32-row block

  int Lk = Tk, Lq = Tq;
  if (kv_lens != nullptr) {
    Lk = clampi(kv_lens[b], 0, Tk);
    if (Tq == Tk) Lq = Lk;
  }
  const int off = Lk - Lq;  // bottom-right causal alignment
  const int q0 = qt * C::BM;

  // byte addresses of this head's rows
  const uint8_t* Qp = Q + ((size_t)b * Hq + hq) * (size_t)Tq * D * C::ESZ;
  const uint8_t* Kp = K + ((size_t)b * Hkv + hk) * (size_t)Tk * D * C::ESZ;
  const uint8_t* Vp = V + ((size_t)b * Hkv + hk) * (size_t)Tk * D * C::ESZ;
  u16* Op = O + ((size_t)b * Hq + hq) * (size_t)Tq * D;

  // keys the workgroup needs: [0, kend) = ntiles_all tiles; key group g
  // takes tiles g, g + KSPLIT, g + 2 KSPLIT, ... (its tile lt is key tile
  // tile_of(lt)).  Interleaved shares keep the workgroups of one head on
  // the same key tiles at the same time, so a grid that starts all at once
  // fetches each tile from HBM once and the rest from L2, and the causal
  // diagonal tiles fall to both groups.
  int kend = 0;
  const int rows_end = min(q0 + C::BM, Lq);
  if (rows_end > q0) kend = CAUSAL ? min(Lk, rows_end + off) : Lk;
  if (kend < 0) kend = 0;
  const int ntiles_all = (kend + C::BN - 1) / C::BN;
  if (ntiles_all == 0) {
    // no row of the tile sees a key (padding rows, or rows before the first
    // key under the causal alignment): O = 0 and LSE = -inf for its rows,
    // written as one contiguous block, without touching Q, K, V or LDS
    const int rows = max(0, min(C::BM, Tq - q0));
    u32x4* o4 = reinterpret_cast<u32x4*>(Op + (size_t)q0 * D);
    for (int i = tid; i < rows * D / 8; i += C::NT) o4[i] = u32x4{0u, 0u, 0u, 0u};
    if (LSE != nullptr)
      for (int i = tid; i < rows; i += C::NT) LSE[((size_t)b * Hq + hq) * Tq + q0 + i] = kNegInf;
    return;
  }
  const int per = (ntiles_all + KSPLIT - 1) / KSPLIT;
  const int ntiles = ntiles_all > kg ? (ntiles_all - kg + KSPLIT - 1) / KSPLIT : 0;
  auto tile_of = [&](int lt) { return lt * KSPLIT + kg; };

  // this wave's rows [wrow0, wrow0 + 32): last key any valid row may see
  // (kmax) and last key every row sees (kfull; past it a tile needs the mask)
  const int wrow0 = q0 + 32 * wg;
  const int qrow = wrow0 + r32;
  int kmax = -1;
  if (wrow0 < Lq) kmax = CAUSAL ? min(Lk - 1, min(wrow0 + 31, Lq - 1) + off) : Lk - 1;
  const int kfull = CAUSAL ? min(Lk - 1, wrow0 + off) : Lk - 1;

  // Q fragments (B operand of S^T = K Q^T), row qrow.  bf16: columns
  // 16 ks + 8 h .. +7.  E4M3: bytes 64 kk + 32 h .. +31; the K fragments
  // use the same bytes of their rows, so every column is paired once.
  // Lanes past Tq read row Tq-1 (their results are never stored), so the
  // loads are unconditional and issue back to back.  They are issued after
  // the first K/V copies (load_q below) and waited for once, in a wait the
  // compiler sees, so that no wait for Q (which would also wait for every
  // copy in flight) is placed inside the loop.  A negative score factor
  // flips the sign bits of Q (flip_q).
  bf16x8 qf[FP8 ? 1 : C::KS];
  i32x8 qf8[FP8 ? C::KK : 1];
  auto load_q = [&]() {
    const int qsrc = min(qrow, Tq - 1);
    if constexpr (FP8) {
      const u32x4* src = reinterpret_cast<const u32x4*>(Qp + (size_t)qsrc * D + 32 * h);
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk) {
        const u32x4 x0 = src[4 * kk];
        const u32x4 x1 = src[4 * kk + 1];
        qf8[kk] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                        (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
      }
    } else {
      const u32x4* src = reinterpret_cast<const u32x4*>(Qp + ((size_t)qsrc * D + 8 * h) * 2);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, src[2 * ks]);
    }
  };
  auto flip_q = [&]() {
    if constexpr (FP8) {
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk) qf8[kk] ^= (int)0x80808080u;
    } else {
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        u32x4 x = __builtin_bit_cast(u32x4, qf[ks]);
        x ^= 0x80008000u;
        qf[ks] = __builtin_bit_cast(bf16x8, x);
      }
    }
  };

  u16* ring = smem + kg * C::RING;
  uint8_t* ring8 = reinterpret_cast<uint8_t*>(ring);
  // E4M3: the widened bf16 V tiles follow the stages
  u16* vwide = ring + C::NS * C::TB;

  // HBM -> LDS copy of the group's tile lt (key tile tile_of(lt)) into
  // stage st.  The tile's 2 LOADS wave-loads (K, then V) are dealt out to
  // the group's waves.  Each 1 KiB wave-load covers 1024 / (D ESZ) rows;
  // lane l lands at byte 16 l of it, i.e. at (row, slot), and fetches the
  // chunk that the swizzle stores in that slot (the E4M3 V tile is stored
  // as is: it is only read back row by row for widening).  Each lane's
  // byte offset from the tile's first row is fixed per copy slot; the
  // tile's base address is wave-uniform, so a copy is one unsigned min of
  // that offset against the last chunk of row Lk-1 (rows at or past Lk
  // read finite data, and those keys are masked) plus the load, addressed
  // as scalar base + 32-bit lane offset.
  //
  // The copy is written as inline asm (M0 = the LDS destination, then
  // global_load_lds_dwordx4) rather than with the compiler builtin: with an
  // LDS write in flight that it can see, the compiler's wait insertion
  // waits for every outstanding LDS read (lgkmcnt(0)) before each use of a
  // fragment, where a count (lgkmcnt(N)) suffices; measured 2-6% faster.
  // The copies are ordered against the reads by the loop's explicit vmcnt
  // waits and barriers, as before.  An SALU write of M0 needs one wait state
  // before an LDS DMA reads it (the hardware does not interlock it, and the
  // compiler's hazard pass does not look inside inline asm), hence the
  // s_nop.  No other instruction of these kernels uses M0 (checked in the
  // generated code), so clobbering it is safe.
  constexpr int RB = D * C::ESZ;   // bytes per row
  constexpr int CPR = RB / 16;     // 16-byte chunks per row
  uint32_t dma_off[C::VMEM_PER_TILE];
#pragma unroll
  for (int i = 0; i < C::VMEM_PER_TILE; ++i) {
    const int ci = (wg + NWG * i) % (2 * C::LOADS);
    const int t = ci / C::LOADS, li = ci - t * C::LOADS;
    const int p = li * 64 + lane;
    const int r = p / CPR, slot = p % CPR;
    int ch;
    if constexpr (FP8)
      ch = t ? slot : slot ^ swz_k8<D>(r);
    else
      ch = slot ^ (t ? swz_v<D>(r) : swz_k<D>(r));
    dma_off[i] = (uint32_t)(r * RB + ch * 16);
  }
  auto issue = [&](int lt, int st) {
    // tiles issued past the group's keys (prologue) start at row Lk-1
    const int kb = min(tile_of(lt) * C::BN, Lk - 1);
    const uint32_t lim = (uint32_t)(min(Lk - kb, C::BN) * RB - 16);
#pragma unroll
    for (int i = 0; i < C::VMEM_PER_TILE; ++i) {
      const int ci = (wg + NWG * i) % (2 * C::LOADS);
      const int t = ci / C::LOADS, li = ci - t * C::LOADS;
      const uint8_t* gb = (t ? Vp : Kp) + (size_t)kb * RB;
      const uint32_t la = __builtin_amdgcn_readfirstlane(
          (uint32_t)(size_t)(lptr_t*)(ring8 + (st * 2 + t) * C::TB + li * 1024));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // M0 on the clobber list: see above
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :: "s"(la), "v"(min(dma_off[i], lim)), "s"(gb) : "memory", "m0");
#pragma clang diagnostic pop
    }
  };

  // per-lane LDS offsets of the fragments
  //  K (A of S^T): row 32 kb + r32.  bf16 (elements): logical chunk
  //  2 ks + h.  E4M3 (bytes): logical chunks 4 kk + 2 h and 4 kk + 2 h + 1.
  int koff[FP8 ? 1 : C::KS];
  int koff8[FP8 ? C::KK : 1][2];
  if constexpr (FP8) {
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk)
#pragma unroll
      for (int e = 0; e < 2; ++e) koff8[kk][e] = r32 * D + 16 * ((4 * kk + 2 * h + e) ^ swz_k8<D>(r32));
  } else {
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) koff[ks] = r32 * D + 8 * ((2 * ks + h) ^ swz_k<D>(r32));
  }
  //  V^T (A of O^T): transposing reads; 16-lane group g covers rows
  //  vr..vr+3 (+16 sh + 32 kb, +8 for the upper half) and logical columns
  //  32 db + 16 (g & 1) + 0..15
  const int tg = lane >> 4, tj = lane & 15;
  const int vr = 4 * (tg >> 1) + (tj >> 2);
  const int vc0 = 2 * (tg & 1) + ((tj & 3) >> 1);
  int voff[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) voff[db] = vr * D + 8 * ((4 * db + vc0) ^ swz_v<D>(vr)) + 4 * (tj & 1);

  f32x16 oacc[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) oacc[i] = f32x16{};
  float m = kNegInf;   // reference maximum of scale*log2(e)*s for this lane's row
  float lsum = 0.f;    // running sum over this lane's half of the keys

  f32x16 s[C::PIPE ? 2 : 1][C::KB];
  bf16x8 pf[C::KB][2];

  // ---- S^T = K Q^T for the tile in stage st
  auto do_scores = [&](int st, f32x16* sd) {
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) sd[kb] = f32x16{};
    if constexpr (FP8) {
      // v_mfma_f32_32x32x64_f8f6f4 on E4M3 A and B (format 0 for both), no
      // block scale: exact products of the codes, fp32 sums
      lds_u8* Ks8 = (lds_u8*)(ring8 + (st * 2 + 0) * C::TB);
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk) {
        lds_u8* k0 = lds_base(Ks8 + koff8[kk][0]);
        lds_u8* k1 = lds_base(Ks8 + koff8[kk][1]);
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
          const u32x4 x0 = *(const __attribute__((address_space(3))) u32x4*)(k0 + 32 * kb * D);
          const u32x4 x1 = *(const __attribute__((address_space(3))) u32x4*)(k1 + 32 * kb * D);
          const i32x8 a = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                                (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
          sd[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf8[kk], sd[kb], 0, 0, 0, 0, 0, 0);
        }
      }
      return;
    }
    lds_u16* Ks = (lds_u16*)&ring[(st * 2 + 0) * C::TILE];
    if constexpr (C::AHEAD) {
      // every fragment read issued before the MFMAs (left alone, the
      // scheduler reads each into the same registers just before its MFMA)
      bf16x8 a[C::KS][C::KB];
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        lds_u16* kp = lds_base(Ks + koff[ks]);
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) a[ks][kb] = *(const __attribute__((address_space(3))) bf16x8*)(kp + 32 * kb * D);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) sd[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks][kb], qf[ks], sd[kb], 0, 0, 0);
      return;
    }
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      // one per-lane base per k-step; the key-block offset folds into the
      // instruction's immediate
      lds_u16* kp = lds_base(Ks + koff[ks]);
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        const bf16x8 a = *(const __attribute__((address_space(3))) bf16x8*)(kp + 32 * kb * D);
        sd[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sd[kb], 0, 0, 0);
      }
    }
  };

  // ---- mask and online-softmax maximum for the tile starting at key kbase
  auto do_max = [&](f32x16* sd, int kbase) {
    const bool need_mask = kbase + C::BN - 1 > kfull;
    if (need_mask) {
      // key kbase + 4 h + (32 kb + 8 (r >> 2) + (r & 3)) is allowed up to
      // lim: compare the constant part against a per-lane bound
      const int lim = CAUSAL ? min(Lk - 1, qrow + off) : Lk - 1;
      const int rel = lim - kbase - 4 * h;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sd[kb][r] = (32 * kb + 8 * (r >> 2) + (r & 3)) <= rel ? sd[kb][r] : kNegInf;
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, sd[kb][r]), sd[kb][r + 1]);
    mx = xhalf_max(mx);
    const float mt = (mx == kNegInf) ? kNegInf : mx * c;
    const bool grow = mt > m + kThresh;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float mnew = fmaxf(m, mt);
      const float alpha = fast_exp2(m - ((mnew == kNegInf) ? 0.f : mnew));
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;
    }
  };

  // ---- P = exp2(c s - m) and its row sums
  auto do_exp = [&](f32x16* sd) {
    const float nm = (m == kNegInf) ? 0.f : -m;
    float ls = lsum;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
        // masked scores are -inf and c > 0, so exp2 gives exactly 0
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = fast_exp2(__builtin_fmaf(sd[kb][8 * sh + e], c, nm));
          const float p1 = fast_exp2(__builtin_fmaf(sd[kb][8 * sh + e + 1], c, nm));
          ls += p0;
          ls += p1;
          pk[e >> 1] = pack2_bf16(p0, p1);
        }
        pf[kb][sh] = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
      }
    lsum = ls;
  };

  // ---- pieces of the pipelined bf16 loop.  exp_tile: P = exp2(c s - m)
  // of a tile, written back over its scores (kept for the row sum) and
  // packed to bf16 MFMA operands in pf; sum_tile: the row sums of those P,
  // added in the order do_exp adds them; raw_max: the per-lane maximum of
  // raw scores; mask_tile: the boundary-tile mask of do_max; finish_max: the
  // row maximum across the wave halves and the lazy rescale of do_max.
  auto exp_tile = [&](f32x16* sd) {
    const float nm = (m == kNegInf) ? 0.f : -m;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = fast_exp2(__builtin_fmaf(sd[kb][8 * sh + e], c, nm));
          const float p1 = fast_exp2(__builtin_fmaf(sd[kb][8 * sh + e + 1], c, nm));
          sd[kb][8 * sh + e] = p0;
          sd[kb][8 * sh + e + 1] = p1;
          pk[e >> 1] = pack2_bf16(p0, p1);
        }
        pf[kb][sh] = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
      }
  };
  auto sum_tile = [&](const f32x16* sd) {
    float ls = lsum;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) ls += sd[kb][r];
    lsum = ls;
  };
  auto raw_max = [&](const f32x16* sd) {
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, sd[kb][r]), sd[kb][r + 1]);
    return mx;
  };
  auto mask_tile = [&](f32x16* sd, int kbase) {
    const int lim = CAUSAL ? min(Lk - 1, qrow + off) : Lk - 1;
    const int rel = lim - kbase - 4 * h;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sd[kb][r] = (32 * kb + 8 * (r >> 2) + (r & 3)) <= rel ? sd[kb][r] : kNegInf;
  };
  auto finish_max = [&](float mx) {
    mx = xhalf_max(mx);
    const float mt = (mx == kNegInf) ? kNegInf : mx * c;
    const bool grow = mt > m + kThresh;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float mnew = fmaxf(m, mt);
      const float alpha = fast_exp2(m - ((mnew == kNegInf) ? 0.f : mnew));
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;
    }
  };

  // ---- E4M3: widen the V tile of stage stv into bf16 buffer vw (the layout
  // of a bf16 V stage).  Each thread of the key group takes WE consecutive
  // elements of one row.
  auto widen = [&](int stv, int vw) {
    const int e0 = (wg * 64 + lane) * C::WE;
    const int r = e0 / D, c0 = e0 % D;
    lds_u8* src = (lds_u8*)(ring8 + (stv * 2 + 1) * C::TB) + r * D + c0;
    u16* dst = vwide + vw * C::TILE + r * D;
    if constexpr (C::WE == 16) {
      const u32x4 x = *(const __attribute__((address_space(3))) u32x4*)src;
      *reinterpret_cast<bf16x8*>(dst + 8 * ((c0 / 8) ^ swz_v<D>(r))) = e4m3x8_to_bf16(u32x2{x[0], x[1]});
      *reinterpret_cast<bf16x8*>(dst + 8 * ((c0 / 8 + 1) ^ swz_v<D>(r))) = e4m3x8_to_bf16(u32x2{x[2], x[3]});
    } else {
      const u32x2 x = *(const __attribute__((address_space(3))) u32x2*)src;
      *reinterpret_cast<bf16x8*>(dst + 8 * ((c0 / 8) ^ swz_v<D>(r))) = e4m3x8_to_bf16(x);
    }
  };

  // ---- V^T fragments of the bf16 V tile at vbase, and O^T += V^T P^T with
  // them (AHEAD: the reads are issued before the tile's softmax)
  auto read_v = [&](u16* vbase, bf16x8 (&vfr)[C::DB][C::KB][2]) {
    lds_u16* Vs = (lds_u16*)vbase;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      lds_u16* vrow = lds_base(Vs + voff[db]);
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
          lds_u16* vp = vrow + (32 * kb + 16 * sh) * D;
          const u32x2 lo = lds_read_tr16(vp);
          const u32x2 hi = lds_read_tr16(vp + 8 * D);
          vfr[db][kb][sh] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
        }
    }
  };
  auto pv_from = [&](const bf16x8 (&vfr)[C::DB][C::KB][2]) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[db][kb][sh], pf[kb][sh], oacc[db], 0, 0, 0);
  };

  // ---- O^T += V^T P^T with the bf16 V tile at vbase
  auto do_pv = [&](u16* vbase) {
    lds_u16* Vs = (lds_u16*)vbase;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      lds_u16* vrow = lds_base(Vs + voff[db]);
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
          lds_u16* vp = vrow + (32 * kb + 16 * sh) * D;
          const u32x2 lo = lds_read_tr16(vp);
          const u32x2 hi = lds_read_tr16(vp + 8 * D);
          const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kb][sh], oacc[db], 0, 0, 0);
        }
    }
  };

  // ---- main loop.  Every key group runs `per` iterations, so that all
  // waves meet the same barriers; a group with a shorter share idles
  // through its last iteration.  The first NS-1 stages are always filled
  // (past the group's keys with data of row Lk-1, never read), so that
  // the number of copies in flight here is fixed and the wait for the Q
  // loads above does not also wait for them.
  // (A workgroup with no keys at all, e.g. query rows past a sequence's
  // length, skips straight to the epilogue.)
  if (ntiles_all > 0) {
#pragma unroll
  for (int p = 0; p < C::NS - 1; ++p) issue(p, p);
  load_q();
  wait_vm_lds<0>();
  if (negq) flip_q();
  if constexpr (C::PIPE) {
    // Iteration lt computes P of tile lt, the scores of tile lt+1 and
    // O += V P of tile lt in one stretch of code with no branch, so that
    // the exponentials (VALU) can issue between the score MFMAs, then masks
    // tile lt+1 and updates the row maximum.  A wave whose last tile is lt
    // still computes (and drops) scores from stage (lt+1) % NS: that stage
    // is not being copied into, so this only costs time.
    // E4M3: iteration lt also widens the V tile of tile lt+1 (into the
    // buffer P V of tile lt-1 read before this iteration's barrier).
    auto kb_of = [&](int lt) { return tile_of(lt) * C::BN; };
    wait_vm_lds<C::VMEM_PER_TILE * (C::NS - 2)>();   // tile 0
    __builtin_amdgcn_s_barrier();
    if constexpr (FP8)
      if (ntiles > 0) widen(0, 0);
    if (ntiles > 0 && kb_of(0) <= kmax) {
      do_scores(0, s[0]);
      do_max(s[0], kb_of(0));
    }
    auto step = [&](int lt, f32x16* sc, f32x16* sn) {
      // this wave's copies of tile lt+1 have landed and its LDS reads of
      // iteration lt-1 are done; after the barrier the same holds for every
      // wave, so stage (lt-1) % NS can be refilled with tile lt+NS-1
      if (lt + 1 < ntiles)
        wait_tile<C::VMEM_PER_TILE, C::NS - 3>(ntiles - 2 - lt);
      else
        wait_lds();
      __builtin_amdgcn_s_barrier();
      if (lt + C::NS - 1 < ntiles) issue(lt + C::NS - 1, (lt + C::NS - 1) % C::NS);
      if constexpr (FP8)
        if (lt + 1 < ntiles) widen((lt + 1) % C::NS, (lt + 1) & 1);
      if (lt >= ntiles || kb_of(lt) > kmax) return;   // wave-uniform
      if constexpr (FP8) {
        do_exp(sc);
        do_scores((lt + 1) % C::NS, sn);
        do_pv(vwide + (lt & 1) * C::TILE);
        if (lt + 1 < ntiles && kb_of(lt + 1) <= kmax) do_max(sn, kb_of(lt + 1));
      } else {
        // bf16: P of tile lt with the scores of tile lt+1, then O += V P of
        // tile lt, then the row sums of tile lt and the raw row maximum of
        // tile lt+1 (their VALU work overlaps the P V products); the mask
        // (boundary tiles only) and the lazy rescale follow
        exp_tile(sc);
        do_scores((lt + 1) % C::NS, sn);
        do_pv(ring + ((lt % C::NS) * 2 + 1) * C::TILE);
        sum_tile(sc);
        float mx = raw_max(sn);
        if (lt + 1 < ntiles && kb_of(lt + 1) <= kmax) {
          const int kb1 = kb_of(lt + 1);
          if (kb1 + C::BN - 1 > kfull) {
            mask_tile(sn, kb1);
            mx = raw_max(sn);
          }
          finish_max(mx);
        }
      }
    };
    for (int lt = 0; lt < per; lt += 2) {
      step(lt, s[0], s[1]);
      if (lt + 1 < per) step(lt + 1, s[1], s[0]);
    }
  } else {
    if constexpr (FP8) {
      // widen tile 0 once every wave's copies of it have landed
      wait_vm_lds<C::VMEM_PER_TILE * (C::NS - 2)>();
      __builtin_amdgcn_s_barrier();
      if (ntiles > 0) widen(0, 0);
    }
    for (int lt = 0; lt < per; ++lt) {
      const int st = lt % C::NS;
      // bf16: this wave's copies of tile lt have landed and its LDS reads of
      // tile lt-1 are done; after the barrier the same holds for every wave,
      // so stage (lt-1) % NS can be refilled with tile lt+NS-1.  E4M3: the
      // same one tile ahead (tile lt+1 is widened in this iteration; tile lt
      // was widened in the previous one, its writes done before the barrier).
      if constexpr (FP8) {
        if (lt + 1 < ntiles)
          wait_tile<C::VMEM_PER_TILE, C::NS - 3>(ntiles - 2 - lt);
        else
          wait_lds();
      } else {
        if (lt < ntiles) wait_tile<C::VMEM_PER_TILE, C::NS - 2>(ntiles - 1 - lt);
      }
      __builtin_amdgcn_s_barrier();
      if (lt + C::NS - 1 < ntiles) issue(lt + C::NS - 1, (lt + C::NS - 1) % C::NS);
      if constexpr (FP8)
        if (lt + 1 < ntiles) widen((lt + 1) % C::NS, (lt + 1) & 1);
      const int kbase = tile_of(lt) * C::BN;
      if (lt >= ntiles || kbase > kmax) continue;   // wave-uniform: nothing of this tile for the wave
      do_scores(st, s[0]);
      if constexpr (C::AHEAD) {
        bf16x8 vfr[C::DB][C::KB][2];
        read_v(ring + (st * 2 + 1) * C::TILE, vfr);
        __builtin_amdgcn_sched_barrier(0);
        do_max(s[0], kbase);
        do_exp(s[0]);
        pv_from(vfr);
        continue;
      }
      do_max(s[0], kbase);
      do_exp(s[0]);
      if constexpr (FP8)
        do_pv(vwide + (lt & 1) * C::TILE);
      else
        do_pv(ring + (st * 2 + 1) * C::TILE);
    }
  }
  }

  // ---- merge of the key groups' partials into group 0: with the combined
  // reference M = max_g m_g, O = sum_g 2^(m_g - M) acc_g and l likewise.
  // The rings are idle once every wave has passed the barrier below (each
  // wave has waited for all of its copies and all of its LDS reads).
  if constexpr (KSPLIT > 1) {
    wait_vm_lds<0>();
    __syncthreads();
    float* part = reinterpret_cast<float*>(smem);
    float* pblk = part + C::ML_FLOATS;
    const int slot = (kg - 1) * NWG + wg;    // groups 1.. : this wave's slot
    if (kg > 0) {
      part[(2 * slot + 0) * 64 + lane] = m;
      part[(2 * slot + 1) * 64 + lane] = lsum;
    }
    float alpha[KSPLIT];
#pragma unroll
    for (int db0 = 0; db0 < C::DB; db0 += C::DBR) {
      if (kg > 0) {
#pragma unroll
        for (int j = 0; j < C::DBR; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            pblk[((slot * C::DBR + j) * 16 + r) * 64 + lane] = oacc[db0 + j][r];
      }
      __syncthreads();
      if (kg == 0) {
        if (db0 == 0) {
          // combined reference and the weight of every group's partial
          float mg[KSPLIT];
          mg[0] = m;
          float mn = m;
#pragma unroll
          for (int g = 1; g < KSPLIT; ++g) {
            mg[g] = part[(2 * ((g - 1) * NWG + wg) + 0) * 64 + lane];
            mn = fmaxf(mn, mg[g]);
          }
          const float ref = (mn == kNegInf) ? 0.f : mn;
          float ltot = 0.f;
#pragma unroll
          for (int g = 0; g < KSPLIT; ++g) {
            alpha[g] = fast_exp2(mg[g] - ref);
            const float lg = g == 0 ? lsum : part[(2 * ((g - 1) * NWG + wg) + 1) * 64 + lane];
            ltot += lg * alpha[g];
          }
          m = mn;
          lsum = ltot;
        }
#pragma unroll
        for (int j = 0; j < C::DBR; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float acc = oacc[db0 + j][r] * alpha[0];
#pragma unroll
            for (int g = 1; g < KSPLIT; ++g)
              acc += pblk[((((g - 1) * NWG + wg) * C::DBR + j) * 16 + r) * 64 + lane] * alpha[g];
            oacc[db0 + j][r] = acc;
          }
      }
      if (db0 + C::DBR < C::DB) __syncthreads();   // group 0 has read this round
    }
    if (kg > 0) return;
  }

  // ---- epilogue: O = acc / l, LSE = ln(2) (m + log2 l); empty rows -> 0, -inf
  // (selected, not multiplied by 0: a padding row's Q may hold NaN)
  const float ltot = xhalf_sum(lsum);
  const bool has = (qrow < Lq) && (ltot > 0.f);
  const float inv = has ? oscale / ltot : 0.f;
  auto outv = [&](float x) { return has ? x * inv : 0.f; };
  if (qrow < Tq) {
    u16* orow = Op + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * db + 8 * g4 + 4 * h;
        u32x2 pk;
        pk[0] = pack2_bf16(outv(oacc[db][4 * g4 + 0]), outv(oacc[db][4 * g4 + 1]));
        pk[1] = pack2_bf16(outv(oacc[db][4 * g4 + 2]), outv(oacc[db][4 * g4 + 3]));
        *reinterpret_cast<u32x2*>(orow + d0) = pk;
      }
    if (LSE != nullptr && h == 0)
      LSE[((size_t)b * Hq + hq) * Tq + qrow] = has ? (m + __log2f(ltot)) * kLn2 : kNegInf;
  }
}

// Workgroup id -> (query tile, batch, head).  ORDER_ID_LIST (ragged grids):
// the id is the position in tile_at's list, longest work first.  Otherwise
// query tiles run from the last tile down, so under a causal mask the
// longest tiles start first.  ORDER_ID_UNITS (grids of several rounds whose (batch, KV head)
// unit count is a multiple of 8): each XCD gets whole units (ids i, i+8,
// i+16, ... run on one XCD), one unit's query heads and tiles after
// another, so that the workgroups resident on an XCD at once share one
// head's K/V in L2.  Otherwise the query-tile index is the slow one and ids
// sharing a (batch, head) are B*Hq apart.  ORDER_ID_ZIG (the whole grid
// resident at once): workgroups id and id + grid/2 share a CU, so the
// second half of the ids runs from the first tile up: each CU then holds a
// long and a short causal tile, equal work in all.
// The E4M3 D=128 two-key-group shape fits two workgroups per CU in LDS; it
// is held to 128 registers per lane (four waves per SIMD) so that two are
// resident (the D=64 shapes stay below that by themselves).
template <int D, int NWG, int KSPLIT, bool CAUSAL, bool FP8>
__global__ __launch_bounds__(64 * NWG * KSPLIT)
__attribute__((amdgpu_waves_per_eu((D == 128 && FP8 && KSPLIT > 1) ? 4 : 1))) void fwd_bf16_kernel(
    const void* __restrict__ Qv, const void* __restrict__ Kv, const void* __restrict__ Vv,
    u16* __restrict__ O, float* __restrict__ LSE, const int32_t* __restrict__ kv_lens,
    int B, int Hq, int Hkv, int Tq, int Tk, int nqt, float c, int negq, int order, float oscale) {
  using C = FwdCfg<D, NWG, KSPLIT, FP8>;
  __shared__ __attribute__((aligned(1024))) u16 smem[C::SMEM];   // [key group][stage][K, V][tile]
  const int id = blockIdx.x;
  const int G = Hq / Hkv;
  if (order == ORDER_ID_LIST) {
    int b, hq, hk, qt;
    tile_at<C::BM, C::BN, CAUSAL>(id, kv_lens, B, Hq, Hkv, Tq, Tk, nqt, b, hq, hk, qt);
    fwd_tile<D, NWG, KSPLIT, CAUSAL, FP8>(static_cast<const uint8_t*>(Qv), static_cast<const uint8_t*>(Kv),
                                          static_cast<const uint8_t*>(Vv), O, LSE, kv_lens, B, Hq, Hkv, Tq, Tk, c,
                                          negq, oscale, smem, b, hq, hk, qt);
    return;
  }
  int tq_slot, b, hq;
  if (order == ORDER_ID_UNITS) {
    const int xcd = id & 7, k = id >> 3;
    const int ul = k / (G * nqt), r = k - ul * (G * nqt);
    tq_slot = r / G;
    const int u = xcd + 8 * ul;
    b = u / Hkv;
    hq = (u - b * Hkv) * G + (r - tq_slot * G);
  } else {
    const int BH = B * Hq;
    tq_slot = id / BH;
    const int bh = id - tq_slot * BH;
    b = bh / Hq;
    hq = bh - b * Hq;
  }
  const int half = (nqt + 1) / 2;
  const int qt = (order == ORDER_ID_ZIG && tq_slot >= half) ? tq_slot - half : nqt - 1 - tq_slot;
  fwd_tile<D, NWG, KSPLIT, CAUSAL, FP8>(static_cast<const uint8_t*>(Qv), static_cast<const uint8_t*>(Kv),
                                        static_cast<const uint8_t*>(Vv), O, LSE, kv_lens, B, Hq, Hkv, Tq, Tk, c,
                                        negq, oscale, smem, b, hq, hq / G, qt);
}

template <int D, int NWG, int KSPLIT, bool CAUSAL, bool FP8>
hipError_t launch(const FwdArgs& a, hipStream_t st, int zig_choice) {
  using C = FwdCfg<D, NWG, KSPLIT, FP8>;
  const int nqt = (a.Tq + C::BM - 1) / C::BM;
  const long long grid = (long long)nqt * a.B * a.Hq;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // scores are scale * (q_scale q).(k_scale k) for E4M3 inputs.  c must be
  // > 0 so that exp2(-inf * c) = 0 for masked keys.  For a zero factor the
  // floor 1e-30 is exact in fp32: every |s| * 1e-30 rounds away against the
  // row maximum, so all allowed keys get weight exactly 1.
  const double qk = FP8 ? (double)a.scale * a.q_scale * a.k_scale : (double)a.scale;
  const float c = fmaxf((float)(fabs(qk) * 1.4426950408889634), 1e-30f);
  const int negq = qk < 0.0 ? 1 : 0;
  // Order of the tiles (see the kernel).  Zig-zag by the built-in rule: at
  // D=64 both shapes fit two workgroups per CU (64 KiB of LDS, at most 128
  // registers per lane), so a causal grid of at most two per CU is resident
  // at once and pairs long and short tiles on each CU; at D=128 one per CU
  // is, and heavy-first order is kept.  The launch table may force zig-zag
  // either way.  Ragged grids of up to kOrderMaxB sequences otherwise run
  // in list order (most work first, tiles with none last); other grids of
  // several rounds take whole (batch, KV head) units per XCD when their
  // count is a multiple of 8.
  int order;
  if (zig_choice == 1 || (zig_choice < 0 && CAUSAL && D == 64 && grid <= 2LL * device_cu_count()))
    order = ORDER_ID_ZIG;
  else if (a.kv_lens != nullptr && a.B <= kOrderMaxB)
    order = ORDER_ID_LIST;
  else
    order = ((a.B * a.Hkv) % 8 == 0 && grid >= 4LL * device_cu_count()) ? ORDER_ID_UNITS : ORDER_ID_NATURAL;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NWG, KSPLIT, CAUSAL, FP8>), dim3((unsigned)grid), dim3(C::NT), 0, st, a.q,
                     a.k, a.v, (u16*)a.o, a.lse, a.kv_lens, a.B, a.Hq, a.Hkv, a.Tq, a.Tk, nqt, c, negq, order,
                     FP8 ? a.v_scale : 1.f);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool FP8>
hipError_t launch_d(const FwdArgs& a, hipStream_t st) {
  // 256-row workgroups with one key group fill the chip once there are two
  // per CU; smaller problems take 128-row workgroups whose two key groups
  // split the key range, which halves the longest chain of tiles and
  // doubles the number of workgroups.  That is the built-in rule; the
  // launch table may choose otherwise per size bucket.
  const long long wg256 = (long long)((a.Tq + 255) / 256) * a.B * a.Hq;
  const FwdChoice ch = choose_fwd(FP8 ? MIATTN_E4M3 : MIATTN_BF16, D, CAUSAL ? 1 : 0, a.Tk, wg256);
  if (ch.shape == 0) return launch<D, 8, 1, CAUSAL, FP8>(a, st, ch.zig);
  return launch<D, 4, 2, CAUSAL, FP8>(a, st, ch.zig);
}

template <bool FP8>
hipError_t launch_all(const FwdArgs& a, hipStream_t st) {
  if (a.D == 64) return a.causal ? launch_d<64, true, FP8>(a, st) : launch_d<64, false, FP8>(a, st);
  return a.causal ? launch_d<128, true, FP8>(a, st) : launch_d<128, false, FP8>(a, st);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t st) { return launch_all<false>(a, st); }
hipError_t launch_fwd_fp8(const FwdArgs& a, hipStream_t st) { return launch_all<true>(a, st); }

}  // namespace miattn
