// Exact tiled attention, prefill, bf16 inputs, fp32 softmax and accumulation.
//
// What is computed ("Implementing attention from scratch", Stable softmax,
// Masks and KV caching; Transformers in Action section 9.4.1, Figure 9.8):
// O = softmax(scale * Q K^T + mask) V, one query tile at a time, streaming
// key/value tiles through on-chip memory with the online softmax: a running
// row maximum m and denominator l, and the earlier partial output rescaled by
// exp(m_old - m_new) whenever the maximum grows.  The score matrix never
// leaves registers.
//
// gfx950 mapping.  One workgroup = NW wave64s = 32*NW query rows of one
// (batch, query head).  Each wave owns 32 query rows and works in the
// transposed frame, so that every lane owns exactly one query row:
//
//   S^T (keys x queries) = K * Q^T     v_mfma_f32_32x32x16_bf16, A = K from LDS,
//                                      B = Q fragments held in registers
//   O^T (d x queries)   += V^T * P^T   A = V^T via transposing LDS reads of the
//                                      row-major V tile, B = P straight from
//                                      the S^T accumulators (no shuffles)
//
// In both results lane l holds query row l%32, so the row maximum is a
// per-lane max plus one exchange between the wave halves, the row sum stays
// per lane until the epilogue, and the rescale by alpha needs no data
// movement.  Softmax runs in base 2 with scale*log2(e) folded into one FMA.
// K and V tiles of BN keys are staged through LDS (padded rows, no bank
// conflicts for the 16-byte K reads and the transposing V reads); the next
// tile's global loads are issued into registers before the current tile's
// math, so HBM latency overlaps the MFMA work.
#include "device_common.h"
#include "launch.h"

namespace miattn {
namespace {

template <int D, int NW>
struct FwdCfg {
  static constexpr int BN = 64;               // keys per tile
  static constexpr int BM = 32 * NW;          // query rows per workgroup
  static constexpr int NT = 64 * NW;          // threads per workgroup
  static constexpr int KST = D + 8;           // K row stride in LDS (bf16)
  static constexpr int VST = D + 16;          // V row stride in LDS (bf16)
  static constexpr int KS = D / 16;           // k-steps of Q K^T
  static constexpr int DB = D / 32;           // 32-wide blocks of the head dim
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int LOADS = BN * CPR / NT; // 16-byte loads per thread per tensor per tile
  static_assert(BN * CPR % NT == 0, "tile must split evenly over the workgroup");
};

template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(64 * NW) void fwd_bf16_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ V,
    u16* __restrict__ O, float* __restrict__ LSE, const int32_t* __restrict__ kv_lens,
    int B, int Hq, int Hkv, int Tq, int Tk, int nqt, float c, int negq) {
  using C = FwdCfg<D, NW>;
  __shared__ __attribute__((aligned(16))) u16 Ks[C::BN * C::KST];
  __shared__ __attribute__((aligned(16))) u16 Vs[C::BN * C::VST];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, r32 = lane & 31;

  // Workgroup -> (query tile, batch, head).  The query-tile index is the slow
  // one and runs from the last tile down, so under a causal mask the longest
  // tiles start first; consecutive ids cover all (batch, head) pairs of one
  // tile, and ids that share a (batch, head) are B*Hq apart.
  const int BH = B * Hq;
  const int id = blockIdx.x;
  const int tq_slot = id / BH;
  const int qt = nqt - 1 - tq_slot;
  const int bh = id - tq_slot * BH;
  const int b = bh / Hq, hq = bh - b * Hq;
  const int hk = hq / (Hq / Hkv);

  int Lk = Tk, Lq = Tq;
  if (kv_lens != nullptr) {
    Lk = clampi(kv_lens[b], 0, Tk);
    if (Tq == Tk) Lq = Lk;
  }
  const int off = Lk - Lq;  // bottom-right causal alignment
  const int q0 = qt * C::BM;

  const u16* Qp = Q + ((size_t)b * Hq + hq) * (size_t)Tq * D;
  const u16* Kp = K + ((size_t)b * Hkv + hk) * (size_t)Tk * D;
  const u16* Vp = V + ((size_t)b * Hkv + hk) * (size_t)Tk * D;
  u16* Op = O + ((size_t)b * Hq + hq) * (size_t)Tq * D;

  // Keys this workgroup needs: [0, kend).
  int kend = 0;
  const int rows_end = min(q0 + C::BM, Lq);
  if (rows_end > q0) kend = CAUSAL ? min(Lk, rows_end + off) : Lk;
  if (kend < 0) kend = 0;
  const int ntiles = (kend + C::BN - 1) / C::BN;

  // Per-wave extent: rows [wrow0, wrow0+32); last key any valid row of the
  // wave may see (wave_kmax) and last key every row of the wave may see.
  const int wrow0 = q0 + w * 32;
  const int qrow = wrow0 + r32;
  int wave_kmax = -1;
  if (wrow0 < Lq) wave_kmax = CAUSAL ? min(Lk - 1, min(wrow0 + 31, Lq - 1) + off) : Lk - 1;
  const int wave_kfull = CAUSAL ? min(Lk - 1, wrow0 + off) : Lk - 1;

  // Q fragments (B operand of S^T = K Q^T): lane holds row qrow, columns
  // 16*ks + 8*h .. +7.
  bf16x8 qf[C::KS];
  {
    const bool ok = qrow < Tq;
    const u32x4* src = reinterpret_cast<const u32x4*>(Qp + (size_t)(ok ? qrow : 0) * D + 8 * h);
    const uint32_t flip = negq ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 x = ok ? src[2 * ks] : u32x4{0u, 0u, 0u, 0u};
      x ^= flip;
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x16 oacc[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) oacc[i] = f32x16{};
  float m = kNegInf;   // running max of scale*log2(e)*s for this lane's row
  float lsum = 0.f;    // running sum over this lane's half of the keys

  u32x4 kreg[C::LOADS], vreg[C::LOADS];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int idx = tid + i * C::NT;
      const int row = idx / C::CPR, ch = idx % C::CPR;
      const int key = kt * C::BN + row;
      const bool ok = key < Lk;
      const size_t g = (size_t)(ok ? key : 0) * D + ch * 8;
      kreg[i] = ok ? *reinterpret_cast<const u32x4*>(Kp + g) : u32x4{0u, 0u, 0u, 0u};
      vreg[i] = ok ? *reinterpret_cast<const u32x4*>(Vp + g) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int idx = tid + i * C::NT;
      const int row = idx / C::CPR, ch = idx % C::CPR;
      *reinterpret_cast<u32x4*>(&Ks[row * C::KST + ch * 8]) = kreg[i];
      *reinterpret_cast<u32x4*>(&Vs[row * C::VST + ch * 8]) = vreg[i];
    }
  };

  // transposing-read coordinates (see device_common.h)
  const int tg = lane >> 4, tj = lane & 15;
  const int tr_row = 4 * (tg >> 1) + (tj >> 2);        // + 32*kb + 16*sh (+8)
  const int tr_col = 16 * (tg & 1) + 4 * (tj & 3);     // + 32*db

  if (ntiles > 0) gload(0);
  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();
    sstore();
    __syncthreads();
    if (kt + 1 < ntiles) gload(kt + 1);
    const int kbase = kt * C::BN;
    if (kbase > wave_kmax) continue;  // wave-uniform: tile fully masked for this wave

    // ---- S^T = K Q^T for the 64 keys of the tile (two 32-key blocks)
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const u16* kr = &Ks[(32 * kb + r32) * C::KST + 8 * h];
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kr + 16 * ks);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
      }
    }

    // ---- mask (only tiles that cross the padding or the diagonal)
    const bool need_mask = kbase + C::BN - 1 > wave_kfull;
    if (need_mask) {
      const int lim = CAUSAL ? min(Lk - 1, qrow + off) : Lk - 1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kbase + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
          s[kb][r] = key <= lim ? s[kb][r] : kNegInf;
        }
    }

    // ---- online softmax update (base 2)
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = xhalf_max(mx);
    const float mt = (mx == kNegInf) ? kNegInf : mx * c;
    const float mnew = fmaxf(m, mt);
    const float muse = (mnew == kNegInf) ? 0.f : mnew;
    const float alpha = fast_exp2(m - muse);
    m = mnew;
    const float nm = -muse;

    bf16x8 pf[2][2];
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(__builtin_fmaf(s[kb][r], c, nm));
        if (need_mask) p = (s[kb][r] == kNegInf) ? 0.f : p;
        ps += p;
        pf[kb][r >> 3][r & 7] = static_cast<__bf16>(p);
      }
    lsum = lsum * alpha + ps;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;

    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
          const u16* vp = &Vs[(32 * kb + 16 * sh + tr_row) * C::VST + 32 * db + tr_col];
          const u32x2 lo = lds_read_tr16(vp);
          const u32x2 hi = lds_read_tr16(vp + 8 * C::VST);
          const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kb][sh], oacc[db], 0, 0, 0);
        }
  }

  // ---- epilogue: O = acc / l, LSE = ln(2) * (m + log2 l); empty rows -> 0, -inf
  const float ltot = xhalf_sum(lsum);
  const bool has = (qrow < Lq) && (ltot > 0.f);
  const float inv = has ? 1.f / ltot : 0.f;
  if (qrow < Tq) {
    u16* orow = Op + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * db + 8 * g4 + 4 * h;
        u32x2 pk;
        pk[0] = pack_bf16x2(oacc[db][4 * g4 + 0] * inv, oacc[db][4 * g4 + 1] * inv);
        pk[1] = pack_bf16x2(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d0) = pk;
      }
    if (LSE != nullptr && h == 0)
      LSE[((size_t)b * Hq + hq) * Tq + qrow] = has ? (m + __log2f(ltot)) * kLn2 : kNegInf;
  }
}

template <int D, int NW, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t st) {
  using C = FwdCfg<D, NW>;
  const int nqt = (a.Tq + C::BM - 1) / C::BM;
  const long long grid = (long long)nqt * a.B * a.Hq;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const float c = fabsf(a.scale) * 1.4426950408889634f;
  const int negq = a.scale < 0.f ? 1 : 0;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, CAUSAL>), dim3((unsigned)grid), dim3(C::NT), 0, st,
                     (const u16*)a.q, (const u16*)a.k, (const u16*)a.v, (u16*)a.o, a.lse, a.kv_lens,
                     a.B, a.Hq, a.Hkv, a.Tq, a.Tk, nqt, c, negq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t st) {
  if (a.D == 64) return a.causal ? launch<64, 4, true>(a, st) : launch<64, 4, false>(a, st);
  return a.causal ? launch<128, 4, true>(a, st) : launch<128, 4, false>(a, st);
}

}  // namespace miattn
