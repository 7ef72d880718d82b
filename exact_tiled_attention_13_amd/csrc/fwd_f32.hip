// Exact tiled attention, prefill, fp32 inputs and outputs, no reduced
// precision anywhere (the NumPy build guide's Step 1 workload is float32).
//
// Same algorithm and the same transposed frame as the bf16 kernel (every
// lane owns one query row), built on v_mfma_f32_32x32x2_f32:
//   S^T = K Q^T   A = K from LDS (row stride D+1 floats: the 32 rows a wave
//                 reads at one column fall in 32 different banks),
//                 B = Q values in registers;
//   O^T += V^T P^T  A = V from LDS (32 consecutive floats of one row per
//                 half-wave), B = P straight from the S^T accumulators.
// Key tiles are 32 wide; the workgroup is 4 waves = 128 query rows.
#include "device_common.h"
#include "launch.h"

namespace miattn {
namespace {

template <int D>
struct F32Cfg {
  static constexpr int BN = 32;
  static constexpr int NW = 4;
  static constexpr int BM = 32 * NW;
  static constexpr int NT = 64 * NW;
  static constexpr int KST = D + 1;
  static constexpr int VST = D + 4;
  static constexpr int CPR = D / 4;           // float4 chunks per row
  static constexpr int LOADS = BN * CPR / NT;
  static constexpr int DB = D / 32;
  static_assert(BN * CPR % NT == 0, "tile must split evenly over the workgroup");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, const int32_t* __restrict__ kv_lens,
    int B, int Hq, int Hkv, int Tq, int Tk, int nqt, float c, int negq) {
  using C = F32Cfg<D>;
  __shared__ float Ks[C::BN * C::KST];
  __shared__ __attribute__((aligned(16))) float Vs[C::BN * C::VST];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, r32 = lane & 31;

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
  const int off = Lk - Lq;
  const int q0 = qt * C::BM;

  const float* Qp = Q + ((size_t)b * Hq + hq) * (size_t)Tq * D;
  const float* Kp = K + ((size_t)b * Hkv + hk) * (size_t)Tk * D;
  const float* Vp = V + ((size_t)b * Hkv + hk) * (size_t)Tk * D;
  float* Op = O + ((size_t)b * Hq + hq) * (size_t)Tq * D;

  int kend = 0;
  const int rows_end = min(q0 + C::BM, Lq);
  if (rows_end > q0) kend = CAUSAL ? min(Lk, rows_end + off) : Lk;
  if (kend < 0) kend = 0;
  const int ntiles = (kend + C::BN - 1) / C::BN;

  const int wrow0 = q0 + w * 32;
  const int qrow = wrow0 + r32;
  int wave_kmax = -1;
  if (wrow0 < Lq) wave_kmax = CAUSAL ? min(Lk - 1, min(wrow0 + 31, Lq - 1) + off) : Lk - 1;
  const int wave_kfull = CAUSAL ? min(Lk - 1, wrow0 + off) : Lk - 1;

  // Q values (B operand): lane holds Q[qrow][2*ks + h].
  float qf[D / 2];
  {
    const bool ok = qrow < Tq;
    const float* src = Qp + (size_t)(ok ? qrow : 0) * D + h;
    const float sg = negq ? -1.f : 1.f;
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks) qf[ks] = ok ? sg * src[2 * ks] : 0.f;
  }

  f32x16 oacc[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) oacc[i] = f32x16{};
  float m = kNegInf, lsum = 0.f;

  f32x4 kreg[C::LOADS], vreg[C::LOADS];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int idx = tid + i * C::NT;
      const int row = idx / C::CPR, ch = idx % C::CPR;
      const int key = kt * C::BN + row;
      const bool ok = key < Lk;
      const size_t g = (size_t)(ok ? key : 0) * D + ch * 4;
      kreg[i] = ok ? *reinterpret_cast<const f32x4*>(Kp + g) : f32x4{0.f, 0.f, 0.f, 0.f};
      vreg[i] = ok ? *reinterpret_cast<const f32x4*>(Vp + g) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int idx = tid + i * C::NT;
      const int row = idx / C::CPR, ch = idx % C::CPR;
#pragma unroll
      for (int e = 0; e < 4; ++e) Ks[row * C::KST + ch * 4 + e] = kreg[i][e];
      *reinterpret_cast<f32x4*>(&Vs[row * C::VST + ch * 4]) = vreg[i];
    }
  };

  if (ntiles > 0) gload(0);
  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();
    sstore();
    __syncthreads();
    if (kt + 1 < ntiles) gload(kt + 1);
    const int kbase = kt * C::BN;
    if (kbase > wave_kmax) continue;

    f32x16 s = f32x16{};
    const float* kr = &Ks[r32 * C::KST + h];
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(kr[2 * ks], qf[ks], s, 0, 0, 0);

    const bool need_mask = kbase + C::BN - 1 > wave_kfull;
    if (need_mask) {
      const int lim = CAUSAL ? min(Lk - 1, qrow + off) : Lk - 1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kbase + 8 * (r >> 2) + 4 * h + (r & 3);
        s[r] = key <= lim ? s[r] : kNegInf;
      }
    }

    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = xhalf_max(mx);
    const float mt = (mx == kNegInf) ? kNegInf : mx * c;
    const float mnew = fmaxf(m, mt);
    const float muse = (mnew == kNegInf) ? 0.f : mnew;
    const float alpha = fast_exp2(m - muse);
    m = mnew;
    const float nm = -muse;

    float p[16];
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = fast_exp2(__builtin_fmaf(s[r], c, nm));
      if (need_mask) x = (s[r] == kNegInf) ? 0.f : x;
      p[r] = x;
      ps += x;
    }
    lsum = lsum * alpha + ps;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;

    // k-step t pairs lane half h with key 8*(t/4) + 4*h + t%4 (this lane's S^T register t)
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const float* vr = &Vs[(8 * (t >> 2) + 4 * h + (t & 3)) * C::VST + r32];
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vr[32 * db], p[t], oacc[db], 0, 0, 0);
    }
  }

  const float ltot = xhalf_sum(lsum);
  const bool has = (qrow < Lq) && (ltot > 0.f);
  const float inv = has ? 1.f / ltot : 0.f;
  // selected, not multiplied by 0: a padding row's Q may hold NaN
  auto outv = [&](float x) { return has ? x * inv : 0.f; };
  if (qrow < Tq) {
    float* orow = Op + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 v4 = {outv(oacc[db][4 * g4]), outv(oacc[db][4 * g4 + 1]), outv(oacc[db][4 * g4 + 2]),
                    outv(oacc[db][4 * g4 + 3])};
        *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * g4 + 4 * h) = v4;
      }
    if (LSE != nullptr && h == 0)
      LSE[((size_t)b * Hq + hq) * Tq + qrow] = has ? (m + log2f(ltot)) * kLn2 : kNegInf;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t st) {
  using C = F32Cfg<D>;
  const int nqt = (a.Tq + C::BM - 1) / C::BM;
  const long long grid = (long long)nqt * a.B * a.Hq;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const float c = fabsf(a.scale) * 1.4426950408889634f;
  const int negq = a.scale < 0.f ? 1 : 0;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(C::NT), 0, st,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse,
                     a.kv_lens, a.B, a.Hq, a.Hkv, a.Tq, a.Tk, nqt, c, negq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t st) {
  if (a.D == 64) return a.causal ? launch<64, true>(a, st) : launch<64, false>(a, st);
  return a.causal ? launch<128, true>(a, st) : launch<128, false>(a, st);
}

}  // namespace miattn
