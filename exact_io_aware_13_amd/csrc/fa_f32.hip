// Exact attention in fp32 (forward and backward), gfx950.
//
// The fp32 path serves fp32 callers and small problems where the answer
// must match the definition to ~1e-6 relative; it uses plain fp32 FMA, not
// matrix cores.  Each thread owns one row; tiles of the other operand are
// staged in LDS and read as broadcasts.  The forward uses the same online
// softmax as the bf16 kernels (running max, running sum, rescaled
// unnormalised accumulator; "How Flash Attention Improves Transformer Memory
// Efficiency ...", section "The Three Running Statistics").  The backward
// recomputes P from the saved lse (section "Backward Pass Efficiency") and
// is split so that no atomics are needed: one kernel owns key rows (dK, dV),
// one owns query rows (dQ).  Per-thread accumulators that would not fit in
// registers live in thread-private LDS columns.

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kRows = kF32RowsPerBlock;  // rows (threads) per workgroup
constexpr int kTile = 32;                // rows of the streamed operand per LDS tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kRows) void fwd_f32_kernel(const float* __restrict__ Q,
                                                        const float* __restrict__ K,
                                                        const float* __restrict__ V,
                                                        float* __restrict__ O,
                                                        float* __restrict__ LSE, int BH, int Lq,
                                                        int Lk, int n_qt, float scale_log2) {
  __shared__ float Kl[kTile][D];
  __shared__ float Vl[kTile][D];
  const int tid = wi_id();
  const int bh = wg_id() % BH;
  const int qt = wg_id() / BH;
  const int qi = qt * kRows + tid;
  const bool valid = qi < Lq;
  const float* q = Q + ((size_t)bh * Lq + (valid ? qi : 0)) * D;
  const float* Kb = K + (size_t)bh * Lk * D;
  const float* Vb = V + (size_t)bh * Lk * D;

  float qr[D], acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qr[c] = q[c];
    acc[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  int kend = Lk;
  if (CAUSAL) kend = min(Lk, qt * kRows + kRows);  // last key any row of this block sees, +1
  for (int k0 = 0; k0 < kend; k0 += kTile) {
    __syncthreads();
    for (int e = tid; e < kTile * D; e += kRows) {
      const int r = e / D, c = e % D;
      const bool in = k0 + r < Lk;
      Kl[r][c] = in ? Kb[(size_t)(k0 + r) * D + c] : 0.f;
      Vl[r][c] = in ? Vb[(size_t)(k0 + r) * D + c] : 0.f;
    }
    __syncthreads();
    float t[kTile];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) dot = fmaf(qr[c], Kl[j][c], dot);
      const int kj = k0 + j;
      t[j] = (kj < Lk && !(CAUSAL && kj > qi)) ? dot * scale_log2 : -INFINITY;
      mx = fmaxf(mx, t[j]);
    }
    const float m_new = fmaxf(m, mx);
    const float base = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m - base);
    m = m_new;
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      t[j] = exp2f(t[j] - base);
      rs += t[j];
    }
    l = alpha * l + rs;
#pragma unroll
    for (int c = 0; c < D; ++c) {
      float a = acc[c] * alpha;
#pragma unroll
      for (int j = 0; j < kTile; ++j) a = fmaf(t[j], Vl[j][c], a);
      acc[c] = a;
    }
  }
  if (valid) {
    float* o = O + ((size_t)bh * Lq + qi) * D;
    const float inv = 1.f / l;
#pragma unroll
    for (int c = 0; c < D; ++c) o[c] = acc[c] * inv;
    LSE[(size_t)bh * Lq + qi] = (m + log2f(l)) * kLn2;
  }
}

// D_i = sum_c dO_ic O_ic and lse in base 2, one thread per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_f32_kernel(const float* __restrict__ O,
                                                          const float* __restrict__ dO,
                                                          const float* __restrict__ lse,
                                                          float* __restrict__ Dvec,
                                                          float* __restrict__ lse2, int64_t rows) {
  const int64_t r = (int64_t)wg_id() * 256 + wi_id();
  if (r >= rows) return;
  float acc = 0.f;
  for (int c = 0; c < D; ++c) acc = fmaf(O[r * D + c], dO[r * D + c], acc);
  Dvec[r] = acc;
  lse2[r] = lse[r] * kLog2e;
}

// dK and dV: one thread per key row j, looping over the queries that see it.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kRows) void bwd_dkdv_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE2, const float* __restrict__ Dvec,
    float* __restrict__ dK, float* __restrict__ dV, int BH, int Lq, int Lk, float scale_log2,
    float scale) {
  __shared__ float Ql[kTile][D];
  __shared__ float Gl[kTile][D];
  __shared__ float Ll[kTile], Dl[kTile];
  __shared__ float accK[D][kRows];
  __shared__ float accV[D][kRows];
  const int tid = wi_id();
  const int bh = wg_id() % BH;
  const int kblk = wg_id() / BH;
  const int kj = kblk * kRows + tid;
  const bool valid = kj < Lk;
  const float* kp = K + ((size_t)bh * Lk + (valid ? kj : 0)) * D;
  const float* vp = V + ((size_t)bh * Lk + (valid ? kj : 0)) * D;
  float kr[D], vr[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    kr[c] = kp[c];
    vr[c] = vp[c];
    accK[c][tid] = 0.f;
    accV[c][tid] = 0.f;
  }
  const float* Qb = Q + (size_t)bh * Lq * D;
  const float* Gb = dO + (size_t)bh * Lq * D;
  const int qstart = CAUSAL ? (kblk * kRows) / kTile * kTile : 0;
  for (int q0 = qstart; q0 < Lq; q0 += kTile) {
    __syncthreads();
    for (int e = tid; e < kTile * D; e += kRows) {
      const int r = e / D, c = e % D;
      const bool in = q0 + r < Lq;
      Ql[r][c] = in ? Qb[(size_t)(q0 + r) * D + c] : 0.f;
      Gl[r][c] = in ? Gb[(size_t)(q0 + r) * D + c] : 0.f;
    }
    if (tid < kTile) {
      const bool in = q0 + tid < Lq;
      Ll[tid] = in ? LSE2[(size_t)bh * Lq + q0 + tid] : 0.f;
      Dl[tid] = in ? Dvec[(size_t)bh * Lq + q0 + tid] : 0.f;
    }
    __syncthreads();
    for (int i = 0; i < kTile; ++i) {
      const int qi = q0 + i;
      if (qi >= Lq) break;
      if (CAUSAL && qi < kj) continue;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) {
        s = fmaf(Ql[i][c], kr[c], s);
        dp = fmaf(Gl[i][c], vr[c], dp);
      }
      const float p = exp2f(s * scale_log2 - Ll[i]);
      const float ds = p * (dp - Dl[i]);
#pragma unroll
      for (int c = 0; c < D; ++c) {
        accV[c][tid] = fmaf(p, Gl[i][c], accV[c][tid]);
        accK[c][tid] = fmaf(ds, Ql[i][c], accK[c][tid]);
      }
    }
  }
  if (valid) {
    float* dk = dK + ((size_t)bh * Lk + kj) * D;
    float* dv = dV + ((size_t)bh * Lk + kj) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) {
      dk[c] = scale * accK[c][tid];
      dv[c] = accV[c][tid];
    }
  }
}

// dQ: one thread per query row i, looping over the keys it sees.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kRows) void bwd_dq_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE2, const float* __restrict__ Dvec,
    float* __restrict__ dQ, int BH, int Lq, int Lk, float scale_log2, float scale) {
  __shared__ float Kl[kTile][D];
  __shared__ float Vl[kTile][D];
  __shared__ float accQ[D][kRows];
  const int tid = wi_id();
  const int bh = wg_id() % BH;
  const int qt = wg_id() / BH;
  const int qi = qt * kRows + tid;
  const bool valid = qi < Lq;
  const size_t row = (size_t)bh * Lq + (valid ? qi : 0);
  float qr[D], gr[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qr[c] = Q[row * D + c];
    gr[c] = dO[row * D + c];
    accQ[c][tid] = 0.f;
  }
  const float lse2 = LSE2[row];
  const float Di = Dvec[row];
  const float* Kb = K + (size_t)bh * Lk * D;
  const float* Vb = V + (size_t)bh * Lk * D;
  int kend = Lk;
  if (CAUSAL) kend = min(Lk, qt * kRows + kRows);
  for (int k0 = 0; k0 < kend; k0 += kTile) {
    __syncthreads();
    for (int e = tid; e < kTile * D; e += kRows) {
      const int r = e / D, c = e % D;
      const bool in = k0 + r < Lk;
      Kl[r][c] = in ? Kb[(size_t)(k0 + r) * D + c] : 0.f;
      Vl[r][c] = in ? Vb[(size_t)(k0 + r) * D + c] : 0.f;
    }
    __syncthreads();
    for (int j = 0; j < kTile; ++j) {
      const int kj = k0 + j;
      if (kj >= Lk || (CAUSAL && kj > qi)) break;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) {
        s = fmaf(qr[c], Kl[j][c], s);
        dp = fmaf(gr[c], Vl[j][c], dp);
      }
      const float ds = exp2f(s * scale_log2 - lse2) * (dp - Di);
#pragma unroll
      for (int c = 0; c < D; ++c) accQ[c][tid] = fmaf(ds, Kl[j][c], accQ[c][tid]);
    }
  }
  if (valid) {
#pragma unroll
    for (int c = 0; c < D; ++c) dQ[row * D + c] = scale * accQ[c][tid];
  }
}

template <int D, bool CAUSAL>
hipError_t fwd_launch(const FwdArgs& a, hipStream_t stream) {
  const int n_qt = (a.Lq + kRows - 1) / kRows;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)(n_qt * a.BH)), dim3(kRows), 0,
                     stream, static_cast<const float*>(a.Q), static_cast<const float*>(a.K),
                     static_cast<const float*>(a.V), static_cast<float*>(a.O), a.lse, a.BH, a.Lq,
                     a.Lk, n_qt, a.scale * kLog2e);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t bwd_launch(const BwdArgs& a, unsigned stages, hipStream_t stream) {
  const int64_t rows = (int64_t)a.BH * a.Lq;
  const auto* Q = static_cast<const float*>(a.Q);
  const auto* K = static_cast<const float*>(a.K);
  const auto* V = static_cast<const float*>(a.V);
  const auto* G = static_cast<const float*>(a.dO);
  if ((stages & kBwdPrepare) && rows > 0)
    hipLaunchKernelGGL((bwd_pre_f32_kernel<D>), dim3((unsigned)((rows + 255) / 256)), dim3(256), 0,
                       stream, static_cast<const float*>(a.O), G, a.lse, a.Dvec, a.lse2, rows);
  const int n_kt = (a.Lk + kRows - 1) / kRows;
  if ((stages & kBwdDkDv) && n_kt > 0)
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D, CAUSAL>), dim3((unsigned)(n_kt * a.BH)), dim3(kRows),
                       0, stream, Q, K, V, G, a.lse2, a.Dvec, static_cast<float*>(a.dK),
                       static_cast<float*>(a.dV), a.BH, a.Lq, a.Lk, a.scale * kLog2e, a.scale);
  const int n_qt = (a.Lq + kRows - 1) / kRows;
  if ((stages & kBwdDq) && n_qt > 0)
    hipLaunchKernelGGL((bwd_dq_f32_kernel<D, CAUSAL>), dim3((unsigned)(n_qt * a.BH)), dim3(kRows),
                       0, stream, Q, K, V, G, a.lse2, a.Dvec, static_cast<float*>(a.dQ), a.BH,
                       a.Lq, a.Lk, a.scale * kLog2e, a.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 64) return a.causal ? fwd_launch<64, true>(a, stream) : fwd_launch<64, false>(a, stream);
  return a.causal ? fwd_launch<128, true>(a, stream) : fwd_launch<128, false>(a, stream);
}

hipError_t launch_bwd_f32(const BwdArgs& a, unsigned stages, hipStream_t stream) {
  if (a.d == 64)
    return a.causal ? bwd_launch<64, true>(a, stages, stream) : bwd_launch<64, false>(a, stages, stream);
  return a.causal ? bwd_launch<128, true>(a, stages, stream) : bwd_launch<128, false>(a, stages, stream);
}

}  // namespace fa
