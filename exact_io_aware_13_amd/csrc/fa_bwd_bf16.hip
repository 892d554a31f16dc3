// Exact attention backward, bf16 inputs, fp32 accumulation, gfx950.
//
// The backward recomputes the probabilities tile by tile from the saved
// per-row log-sum-exp instead of reading a stored P, and uses the row
// statistic D_i = sum_c dO_ic O_ic ("How Flash Attention Improves Transformer
// Memory Efficiency ...", section "Backward Pass Efficiency"; glossary page
// "Flash Attention", section "How it works").  The gradient formulas are the
// chain rule through the forward: dV = P^T dO, dP = dO V^T,
// dS = P * (dP - D), dK = scale dS^T Q, dQ = scale dS K.
//
// Three kernels:
//  1. pre:     D_i = rowsum(dO * O) and zero the fp32 dQ accumulator.
//  2. main:    one workgroup = 4 waves = 128 keys of one slice (32 per
//              wave); K and V rows stay in registers, dK and dV accumulate in
//              registers over all query tiles (64 rows each) that can see
//              the keys.  Per query tile the workgroup stages Q and dO in LDS
//              both row-major and transposed, recomputes S and P, forms dS,
//              and adds its dQ share into the fp32 accumulator with atomics.
//  3. convert: dQ = bf16(scale * accumulator).
//
// Matrix-core orientation in the main kernel: S = Q K^T and dP = dO V^T are
// computed with queries as rows, so each lane owns one key (column) and 16
// queries; those registers are directly the B operands of dV^T = dO^T P and
// dK^T = Q^T dS (contraction over queries in the order the accumulator holds
// them), with dO^T and Q^T read from the transposed LDS copies.  dQ needs dS
// with queries as lanes, so dS goes through LDS once per query tile.

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

// ---------------------------------------------------------------------------
// 1. D statistic and accumulator reset
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_bf16_kernel(
    const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO, float* __restrict__ Dvec,
    float* __restrict__ dQacc, int64_t rows) {
  constexpr int LPR = D / 8;        // lanes per row, 8 elements each
  constexpr int RPB = 256 / LPR;    // rows per workgroup
  const int64_t row = (int64_t)wg_id() * RPB + wi_id() / LPR;
  const int c = wi_id() % LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 o = *reinterpret_cast<const u32x4*>(O + row * D + c * 8);
    const u32x4 g = *reinterpret_cast<const u32x4*>(dO + row * D + c * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += bf16_lo(o[i]) * bf16_lo(g[i]) + bf16_hi(o[i]) * bf16_hi(g[i]);
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(dQacc + row * D + c * 8) = z;
    *reinterpret_cast<f32x4*>(dQacc + row * D + c * 8 + 4) = z;
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && c == 0) Dvec[row] = acc;
}

// ---------------------------------------------------------------------------
// 2. main kernel
// ---------------------------------------------------------------------------
template <int D>
struct BwdTile {
  static constexpr int BK = 128;       // keys per workgroup (32 per wave)
  static constexpr int BQ = 64;        // query rows per step
  static constexpr int KS = D / 16;    // 16-deep steps over the head dimension
  static constexpr int DB = D / 32;    // 32-wide head-dim blocks
  static constexpr int DBW = DB / 2;   // head-dim blocks of dQ per wave
  static constexpr int RLD = D + 8;    // pitch of row-major Q / dO tiles (bf16)
  static constexpr int TLD = BQ + 4;   // pitch of transposed Q^T / dO^T tiles
  static constexpr int SLD = BK + 8;   // pitch of the dS tile (rows = queries)
  static constexpr int KTLD = BK + 8;  // pitch of K^T (rows = head dim)
  static constexpr int KCH = D / 8;    // 16-byte chunks per row
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Dvec, float* __restrict__ dQacc,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int BH, int Lq, int Lk,
    float scale_log2, float scale) {
  using T = BwdTile<D>;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[T::BQ * T::RLD];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[T::BQ * T::RLD];
  __shared__ __attribute__((aligned(16))) uint16_t Qt[D * T::TLD];
  __shared__ __attribute__((aligned(16))) uint16_t dOt[D * T::TLD];
  __shared__ __attribute__((aligned(16))) uint16_t dSs[T::BQ * T::SLD];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[D * T::KTLD];
  __shared__ __attribute__((aligned(16))) float lse_s[T::BQ];
  __shared__ __attribute__((aligned(16))) float dd_s[T::BQ];

  const int tid = wi_id();
  // The wave index is the same on every lane; readfirstlane tells the
  // compiler so, which keeps everything derived from it in scalar registers.
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, n = lane & 31, h = lane >> 5;
  const int bh = wg_id() % BH;
  const int k0 = (wg_id() / BH) * T::BK;
  const int kw0 = k0 + 32 * w;
  const int key = kw0 + n;

  const size_t qoff = (size_t)bh * Lq * D, koff = (size_t)bh * Lk * D;
  const auto rq = make_rsrc(Q + qoff, (uint32_t)Lq * D * 2);
  const auto rdo = make_rsrc(dO + qoff, (uint32_t)Lq * D * 2);
  const auto rk = make_rsrc(K + koff, (uint32_t)Lk * D * 2);
  const auto rv = make_rsrc(V + koff, (uint32_t)Lk * D * 2);
  const auto rlse = make_rsrc(LSE + (size_t)bh * Lq, (uint32_t)Lq * 4);
  const auto rdd = make_rsrc(Dvec + (size_t)bh * Lq, (uint32_t)Lq * 4);

  // This lane's key row of K and V: B operands of S = Q K^T and dP = dO V^T.
  bf16x8 kf[T::KS], vf[T::KS];
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks) {
    kf[ks] = as_bf16x8(load16(rk, (uint32_t)(key * D + ks * 16 + h * 8) * 2));
    vf[ks] = as_bf16x8(load16(rv, (uint32_t)(key * D + ks * 16 + h * 8) * 2));
  }
  // K^T of the workgroup's 128 keys (B operand of dQ = dS K).
  for (int it = tid; it < 32 * T::KCH; it += 256) {
    const int kg = it % 32, ch = it / 32;
    u32x4 r4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) r4[r] = load16(rk, (uint32_t)((k0 + 4 * kg + r) * D + ch * 8) * 2);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      u32x2 ev, od;
      ev.x = (r4[0][a] & 0xffffu) | (r4[1][a] << 16);
      ev.y = (r4[2][a] & 0xffffu) | (r4[3][a] << 16);
      od.x = (r4[0][a] >> 16) | (r4[1][a] & 0xffff0000u);
      od.y = (r4[2][a] >> 16) | (r4[3][a] & 0xffff0000u);
      *reinterpret_cast<u32x2*>(&Kt[(ch * 8 + 2 * a) * T::KTLD + 4 * kg]) = ev;
      *reinterpret_cast<u32x2*>(&Kt[(ch * 8 + 2 * a + 1) * T::KTLD + 4 * kg]) = od;
    }
  }

  f32x16 dvacc[T::DB], dkacc[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dvacc[db][r] = 0.f;
      dkacc[db][r] = 0.f;
    }

  const int n_qt = (Lq + T::BQ - 1) / T::BQ;
  const int qt0 = CAUSAL ? min(k0 / T::BQ, n_qt) : 0;
  for (int qt = qt0; qt < n_qt; ++qt) {
    const int q0 = qt * T::BQ;
    __syncthreads();  // previous step's LDS reads are finished
    for (int it = tid; it < 16 * T::KCH; it += 256) {
      const int rg = it % 16, ch = it / 16;
      u32x4 qv[4], gv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        qv[r] = load16(rq, (uint32_t)((q0 + 4 * rg + r) * D + ch * 8) * 2);
        gv[r] = load16(rdo, (uint32_t)((q0 + 4 * rg + r) * D + ch * 8) * 2);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        *reinterpret_cast<u32x4*>(&Qs[(4 * rg + r) * T::RLD + ch * 8]) = qv[r];
        *reinterpret_cast<u32x4*>(&dOs[(4 * rg + r) * T::RLD + ch * 8]) = gv[r];
      }
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        u32x2 ev, od;
        ev.x = (qv[0][a] & 0xffffu) | (qv[1][a] << 16);
        ev.y = (qv[2][a] & 0xffffu) | (qv[3][a] << 16);
        od.x = (qv[0][a] >> 16) | (qv[1][a] & 0xffff0000u);
        od.y = (qv[2][a] >> 16) | (qv[3][a] & 0xffff0000u);
        *reinterpret_cast<u32x2*>(&Qt[(ch * 8 + 2 * a) * T::TLD + 4 * rg]) = ev;
        *reinterpret_cast<u32x2*>(&Qt[(ch * 8 + 2 * a + 1) * T::TLD + 4 * rg]) = od;
        ev.x = (gv[0][a] & 0xffffu) | (gv[1][a] << 16);
        ev.y = (gv[2][a] & 0xffffu) | (gv[3][a] << 16);
        od.x = (gv[0][a] >> 16) | (gv[1][a] & 0xffff0000u);
        od.y = (gv[2][a] >> 16) | (gv[3][a] & 0xffff0000u);
        *reinterpret_cast<u32x2*>(&dOt[(ch * 8 + 2 * a) * T::TLD + 4 * rg]) = ev;
        *reinterpret_cast<u32x2*>(&dOt[(ch * 8 + 2 * a + 1) * T::TLD + 4 * rg]) = od;
      }
    }
    if (tid < T::BQ) {
      lse_s[tid] = load4f(rlse, (uint32_t)(q0 + tid) * 4) * kLog2e;
      dd_s[tid] = load4f(rdd, (uint32_t)(q0 + tid) * 4);
    }
    __syncthreads();

    // S and dP for 2 blocks of 32 queries: lane owns key `key`, register r of
    // block qb holds query q0 + qb*32 + 8*(r/4) + 4*h + r%4.
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[qb][r] = 0.f;
        dp[qb][r] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&Qs[(qb * 32 + n) * T::RLD + ks * 16 + h * 8]);
        s[qb] = mma(as_bf16x8(a), kf[ks], s[qb]);
        const u32x4 g = *reinterpret_cast<const u32x4*>(&dOs[(qb * 32 + n) * T::RLD + ks * 16 + h * 8]);
        dp[qb] = mma(as_bf16x8(g), vf[ks], dp[qb]);
      }
    }

    // P = exp(S - lse) (masked), dS = P * (dP - D); both rounded to bf16.
    const bool need_mask = (q0 + T::BQ > Lq) || (CAUSAL && q0 < kw0 + 31);
    unsigned pp[2][8], pd[2][8];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 L4 = *reinterpret_cast<const f32x4*>(&lse_s[qb * 32 + 8 * g + 4 * h]);
        const f32x4 D4 = *reinterpret_cast<const f32x4*>(&dd_s[qb * 32 + 8 * g + 4 * h]);
        float p[4], ds[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * g + i;
          float pv = fast_exp2(s[qb][r] * scale_log2 - L4[i]);
          if (need_mask) {
            const int qi = q0 + qb * 32 + 8 * g + 4 * h + i;
            if (qi >= Lq || (CAUSAL && qi < key)) pv = 0.f;
          }
          p[i] = pv;
          ds[i] = pv * (dp[qb][r] - D4[i]);
        }
        pp[qb][2 * g] = pack_bf16x2(p[0], p[1]);
        pp[qb][2 * g + 1] = pack_bf16x2(p[2], p[3]);
        pd[qb][2 * g] = pack_bf16x2(ds[0], ds[1]);
        pd[qb][2 * g + 1] = pack_bf16x2(ds[2], ds[3]);
      }

    // dV^T += dO^T P and dK^T += Q^T dS in 4 steps of 16 queries.
#pragma unroll
    for (int ks2 = 0; ks2 < T::BQ / 16; ++ks2) {
      const int qb = ks2 >> 1, hf = ks2 & 1;
      u32x4 bP, bS;
      bP.x = pp[qb][hf * 4 + 0];
      bP.y = pp[qb][hf * 4 + 1];
      bP.z = pp[qb][hf * 4 + 2];
      bP.w = pp[qb][hf * 4 + 3];
      bS.x = pd[qb][hf * 4 + 0];
      bS.y = pd[qb][hf * 4 + 1];
      bS.z = pd[qb][hf * 4 + 2];
      bS.w = pd[qb][hf * 4 + 3];
#pragma unroll
      for (int db = 0; db < T::DB; ++db) {
        const int dd = db * 32 + n;
        const u32x2 glo = *reinterpret_cast<const u32x2*>(&dOt[dd * T::TLD + ks2 * 16 + 4 * h]);
        const u32x2 ghi = *reinterpret_cast<const u32x2*>(&dOt[dd * T::TLD + ks2 * 16 + 8 + 4 * h]);
        u32x4 ag;
        ag.x = glo.x;
        ag.y = glo.y;
        ag.z = ghi.x;
        ag.w = ghi.y;
        dvacc[db] = mma(as_bf16x8(ag), as_bf16x8(bP), dvacc[db]);
        const u32x2 qlo = *reinterpret_cast<const u32x2*>(&Qt[dd * T::TLD + ks2 * 16 + 4 * h]);
        const u32x2 qhi = *reinterpret_cast<const u32x2*>(&Qt[dd * T::TLD + ks2 * 16 + 8 + 4 * h]);
        u32x4 aq;
        aq.x = qlo.x;
        aq.y = qlo.y;
        aq.z = qhi.x;
        aq.w = qhi.y;
        dkacc[db] = mma(as_bf16x8(aq), as_bf16x8(bS), dkacc[db]);
      }
    }

    // dS -> LDS with queries as rows, then dQ (64 x D) = dS (64 x 128) K.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 2 * j;
        const int ql = qb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        dSs[ql * T::SLD + 32 * w + n] = (uint16_t)(pd[qb][j] & 0xffffu);
        dSs[(ql + 1) * T::SLD + 32 * w + n] = (uint16_t)(pd[qb][j] >> 16);
      }
    __syncthreads();
    {
      const int qb = w >> 1;
      f32x16 dq[T::DBW];
#pragma unroll
      for (int j = 0; j < T::DBW; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) dq[j][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < T::BK / 16; ++ks) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&dSs[(qb * 32 + n) * T::SLD + ks * 16 + 8 * h]);
#pragma unroll
        for (int j = 0; j < T::DBW; ++j) {
          const int db = (w & 1) * T::DBW + j;
          const u32x4 b = *reinterpret_cast<const u32x4*>(&Kt[(db * 32 + n) * T::KTLD + ks * 16 + 8 * h]);
          dq[j] = mma(as_bf16x8(a), as_bf16x8(b), dq[j]);
        }
      }
      float* dst = dQacc + qoff;
#pragma unroll
      for (int j = 0; j < T::DBW; ++j) {
        const int dcol = ((w & 1) * T::DBW + j) * 32 + n;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = q0 + qb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (qi < Lq) atomicAdd(dst + (size_t)qi * D + dcol, dq[j][r]);
        }
      }
    }
  }

  // dK = scale * dK^T accumulator, dV = dV^T accumulator, one key row per lane.
  const auto rdk = make_rsrc(dK + koff, (uint32_t)Lk * D * 2);
  const auto rdv = make_rsrc(dV + koff, (uint32_t)Lk * D * 2);
#pragma unroll
  for (int db = 0; db < T::DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t off = (uint32_t)(key * D + db * 32 + 8 * g + 4 * h) * 2;
      u32x2 vk, vv;
      vk.x = pack_bf16x2(scale * dkacc[db][4 * g + 0], scale * dkacc[db][4 * g + 1]);
      vk.y = pack_bf16x2(scale * dkacc[db][4 * g + 2], scale * dkacc[db][4 * g + 3]);
      vv.x = pack_bf16x2(dvacc[db][4 * g + 0], dvacc[db][4 * g + 1]);
      vv.y = pack_bf16x2(dvacc[db][4 * g + 2], dvacc[db][4 * g + 3]);
      store8(rdk, off, vk);
      store8(rdv, off, vv);
    }
}

// ---------------------------------------------------------------------------
// 3. dQ = bf16(scale * accumulator)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dq_convert_kernel(const float* __restrict__ acc,
                                                         uint16_t* __restrict__ dQ, float scale,
                                                         int64_t n8) {
  const int64_t i = (int64_t)wg_id() * 256 + wi_id();
  if (i >= n8) return;
  const f32x4 a = *reinterpret_cast<const f32x4*>(acc + 8 * i);
  const f32x4 b = *reinterpret_cast<const f32x4*>(acc + 8 * i + 4);
  u32x4 o;
  o.x = pack_bf16x2(scale * a.x, scale * a.y);
  o.y = pack_bf16x2(scale * a.z, scale * a.w);
  o.z = pack_bf16x2(scale * b.x, scale * b.y);
  o.w = pack_bf16x2(scale * b.z, scale * b.w);
  *reinterpret_cast<u32x4*>(dQ + 8 * i) = o;
}

template <int D>
hipError_t launch_d(const BwdArgs& a, hipStream_t stream) {
  using T = BwdTile<D>;
  const int64_t rows = (int64_t)a.BH * a.Lq;
  if (rows > 0) {
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL((bwd_pre_bf16_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256),
                       0, stream, static_cast<const uint16_t*>(a.O),
                       static_cast<const uint16_t*>(a.dO), a.Dvec, a.dQacc, rows);
  }
  const int n_kt = (a.Lk + T::BK - 1) / T::BK;
  const dim3 grid((unsigned)(n_kt * a.BH));
  if (a.causal)
    hipLaunchKernelGGL((bwd_bf16_kernel<D, true>), grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                       static_cast<const uint16_t*>(a.V), static_cast<const uint16_t*>(a.dO), a.lse,
                       a.Dvec, a.dQacc, static_cast<uint16_t*>(a.dK), static_cast<uint16_t*>(a.dV),
                       a.BH, a.Lq, a.Lk, a.scale * kLog2e, a.scale);
  else
    hipLaunchKernelGGL((bwd_bf16_kernel<D, false>), grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                       static_cast<const uint16_t*>(a.V), static_cast<const uint16_t*>(a.dO), a.lse,
                       a.Dvec, a.dQacc, static_cast<uint16_t*>(a.dK), static_cast<uint16_t*>(a.dV),
                       a.BH, a.Lq, a.Lk, a.scale * kLog2e, a.scale);
  if (rows > 0) {
    const int64_t n8 = rows * D / 8;
    hipLaunchKernelGGL(dq_convert_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream,
                       a.dQacc, static_cast<uint16_t*>(a.dQ), a.scale, n8);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  static_assert(BwdTile<128>::BK == kBwdBf16KeysPerBlock, "tile table out of sync");
  if (a.d == 64) return launch_d<64>(a, stream);
  return launch_d<128>(a, stream);
}

}  // namespace fa
