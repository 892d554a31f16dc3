// Exact attention forward, bf16 inputs, fp32 accumulation, gfx950.
//
// One workgroup = 4 waves = 128 query rows of one (batch, head) slice.  The
// Q rows stay in registers for the whole key loop; K and V stream through
// LDS one 64-key tile at a time (the next tile is fetched into registers
// while the current one is multiplied), and an online softmax keeps a
// running max m, a running sum l and an unnormalised output per row,
// rescaling both by exp(m_old - m_new) when the max grows ("How Flash
// Attention Improves Transformer Memory Efficiency ...", sections "Block-Wise
// Processing Algorithm" and "The Three Running Statistics"; "What Is
// FlashAttention?", section "What FlashAttention does instead").  Scores
// and probabilities live only in registers.
//
// Matrix-core orientation.  Each wave computes S^T = K Q^T for its 32 rows,
// so in the 32x32 accumulator every lane owns ONE query row (column n = lane
// % 32) and 16 of the tile's keys; the other 16 keys of that row sit in lane
// ^ 32.  Row max and row sum are therefore in-lane plus one exchange between
// the two wave halves.  The same register layout is then exactly the
// B operand of O^T = V^T P^T: contraction order over keys is free, so the
// keys are taken in the order the accumulator already holds them, and V^T is
// read from a transposed copy of the V tile kept in LDS.  O^T's accumulator
// again gives each lane one query row, so the rescale by exp(m_old - m_new)
// is a per-lane scalar multiply.
//
// Softmax arithmetic runs in base 2: scores are multiplied by
// scale*log2(e), exponentials use the hardware exp2, and the stored lse is
// converted back to natural log.  The running sum l adds the fp32
// probabilities; the P.V product takes them rounded to bf16.  Summing the
// unrounded values keeps lse within ~1e-6 of the exact log-normaliser even
// for rows that see only a few keys (bf16 rounding of those few terms would
// move ln l by up to ~2e-3).

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

template <int D>
struct FwdTile {
  static constexpr int BR = 128;      // query rows per workgroup (32 per wave)
  static constexpr int BC = 64;       // keys per tile
  static constexpr int KS = D / 16;   // 16-deep steps over the head dimension
  static constexpr int DB = D / 32;   // 32-wide blocks of the head dimension
  static constexpr int KLD = D + 8;   // LDS pitch of K rows (bf16); +16 B keeps b128 reads conflict-free
  static constexpr int VLD = BC + 4;  // LDS pitch of V^T rows (bf16); +8 B keeps b64 reads conflict-free
  static constexpr int KCH = D / 8;   // 16-byte chunks per K/V row
  static constexpr int K_ITEMS = BC * KCH / 256;  // K chunks fetched per thread
  static constexpr int V_ITEMS = 16 * KCH;        // (4-key group, chunk) items of the V tile
};

template <int D, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, void* __restrict__ O, float* __restrict__ LSE,
    int BH, int Lq, int Lk, int n_qt, float scale_log2) {
  using T = FwdTile<D>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[T::BC * T::KLD];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * T::VLD];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, n = lane & 31, h = lane >> 5;

  // Consecutive workgroups take the same query tile of different slices; for
  // causal masks the tiles with the most visible keys are dispatched first.
  const int bh = blockIdx.x % BH;
  int qt = blockIdx.x / BH;
  if (CAUSAL) qt = n_qt - 1 - qt;
  const int q0 = qt * T::BR;

  const size_t qoff = (size_t)bh * Lq * D;
  const size_t koff = (size_t)bh * Lk * D;
  const auto rq = make_rsrc(Q + qoff, (uint32_t)Lq * D * 2);
  const auto rk = make_rsrc(K + koff, (uint32_t)Lk * D * 2);
  const auto rv = make_rsrc(V + koff, (uint32_t)Lk * D * 2);

  // This lane's query row; its Q values are the B operand of S^T = K Q^T.
  const int qg = q0 + w * 32 + n;
  bf16x8 qf[T::KS];
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks)
    qf[ks] = as_bf16x8(load16(rq, (uint32_t)(qg * D + ks * 16 + h * 8) * 2));

  f32x16 oacc[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m = -INFINITY, l = 0.f;

  int nkt = (Lk + T::BC - 1) / T::BC;
  if (CAUSAL) nkt = min(nkt, (q0 + T::BR - 1) / T::BC + 1);

  u32x4 kreg[T::K_ITEMS];
  u32x4 vreg[4];
  auto fetch = [&](int kt) {
#pragma unroll
    for (int i = 0; i < T::K_ITEMS; ++i) {
      const int it = tid + 256 * i, row = it / T::KCH, ch = it % T::KCH;
      kreg[i] = load16(rk, (uint32_t)((kt * T::BC + row) * D + ch * 8) * 2);
    }
    if (tid < T::V_ITEMS) {
      const int kg = tid % 16, ch = tid / 16;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vreg[r] = load16(rv, (uint32_t)((kt * T::BC + 4 * kg + r) * D + ch * 8) * 2);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < T::K_ITEMS; ++i) {
      const int it = tid + 256 * i, row = it / T::KCH, ch = it % T::KCH;
      *reinterpret_cast<u32x4*>(&Ks[row * T::KLD + ch * 8]) = kreg[i];
    }
    if (tid < T::V_ITEMS) {
      // Four keys x eight head-dim values -> eight rows of V^T, four keys each.
      const int kg = tid % 16, ch = tid / 16;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        u32x2 ev, od;
        ev.x = (vreg[0][a] & 0xffffu) | (vreg[1][a] << 16);
        ev.y = (vreg[2][a] & 0xffffu) | (vreg[3][a] << 16);
        od.x = (vreg[0][a] >> 16) | (vreg[1][a] & 0xffff0000u);
        od.y = (vreg[2][a] >> 16) | (vreg[3][a] & 0xffff0000u);
        *reinterpret_cast<u32x2*>(&Vt[(ch * 8 + 2 * a) * T::VLD + 4 * kg]) = ev;
        *reinterpret_cast<u32x2*>(&Vt[(ch * 8 + 2 * a + 1) * T::VLD + 4 * kg]) = od;
      }
    }
  };

  fetch(0);
  for (int kt = 0; kt < nkt; ++kt) {
    __syncthreads();  // all waves are done reading the previous tile
    stage();
    __syncthreads();
    if (kt + 1 < nkt) fetch(kt + 1);

    // S^T for 2 blocks of 32 keys: lane owns query qg, register r of block kb
    // holds key kt*64 + kb*32 + 8*(r/4) + 4*h + r%4.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&Ks[(kb * 32 + n) * T::KLD + ks * 16 + h * 8]);
        s[kb] = mma(as_bf16x8(a), qf[ks], s[kb]);
      }
    }

    const int key0 = kt * T::BC;
    const bool need_mask = (key0 + T::BC > Lk) || (CAUSAL && key0 + T::BC - 1 > q0 + w * 32);
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float t = s[kb][r] * scale_log2;
        if (need_mask) {
          const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key >= Lk || (CAUSAL && key > qg)) t = -INFINITY;
        }
        s[kb][r] = t;
        mx = fmaxf(mx, t);
      }
    mx = fmaxf(mx, swap_halves(mx));
    const float m_new = fmaxf(m, mx);
    // A row whose keys so far are all masked keeps m = -inf; exponentiate
    // against 0 then, so masked entries give exactly 0 and nothing is NaN.
    const float base = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m - base);
    m = m_new;

    unsigned pk[2][8];
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p0 = fast_exp2(s[kb][2 * j] - base), p1 = fast_exp2(s[kb][2 * j + 1] - base);
        pk[kb][j] = pack_bf16x2(p0, p1);
        rs += p0 + p1;
      }
    l = alpha * l + rs;
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

    // O^T += V^T P^T in 4 steps of 16 keys.  Step ks2 uses registers
    // 8*(ks2%2) .. +7 of score block ks2/2; slot i of half h is key
    // ks2*16 + 8*(i/4) + 4*h + i%4, which V^T supplies as two 4-key runs.
#pragma unroll
    for (int ks2 = 0; ks2 < T::BC / 16; ++ks2) {
      const int kb = ks2 >> 1, hf = ks2 & 1;
      u32x4 bp;
      bp.x = pk[kb][hf * 4 + 0];
      bp.y = pk[kb][hf * 4 + 1];
      bp.z = pk[kb][hf * 4 + 2];
      bp.w = pk[kb][hf * 4 + 3];
#pragma unroll
      for (int db = 0; db < T::DB; ++db) {
        const int dd = db * 32 + n;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(&Vt[dd * T::VLD + ks2 * 16 + 4 * h]);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(&Vt[dd * T::VLD + ks2 * 16 + 8 + 4 * h]);
        u32x4 av;
        av.x = lo.x;
        av.y = lo.y;
        av.z = hi.x;
        av.w = hi.y;
        oacc[db] = mma(as_bf16x8(av), as_bf16x8(bp), oacc[db]);
      }
    }
  }

  // Epilogue: O = accumulator / l, lse = (m + log2 l) * ln 2.
  const float lt = l + swap_halves(l);
  const float inv = 1.f / lt;
  if (OUT_F32) {
    const auto ro = make_rsrc(static_cast<float*>(O) + qoff, (uint32_t)Lq * D * 4);
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x4 v;
        v.x = __builtin_bit_cast(unsigned, oacc[db][4 * g + 0] * inv);
        v.y = __builtin_bit_cast(unsigned, oacc[db][4 * g + 1] * inv);
        v.z = __builtin_bit_cast(unsigned, oacc[db][4 * g + 2] * inv);
        v.w = __builtin_bit_cast(unsigned, oacc[db][4 * g + 3] * inv);
        store16(ro, (uint32_t)(qg * D + db * 32 + 8 * g + 4 * h) * 4, v);
      }
  } else {
    const auto ro = make_rsrc(static_cast<uint16_t*>(O) + qoff, (uint32_t)Lq * D * 2);
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 v;
        v.x = pack_bf16x2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv);
        v.y = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        store8(ro, (uint32_t)(qg * D + db * 32 + 8 * g + 4 * h) * 2, v);
      }
  }
  if (h == 0 && qg < Lq) LSE[(size_t)bh * Lq + qg] = (m + __log2f(lt)) * kLn2;
}

template <int D, bool CAUSAL, bool OUT_F32>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const int n_qt = (a.Lq + FwdTile<D>::BR - 1) / FwdTile<D>::BR;
  const dim3 grid((unsigned)(n_qt * a.BH));
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, OUT_F32>), grid, dim3(256), 0, stream,
                     static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                     static_cast<const uint16_t*>(a.V), a.O, a.lse, a.BH, a.Lq, a.Lk, n_qt,
                     a.scale * kLog2e);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
  if (a.causal) return a.out_f32 ? launch<D, true, true>(a, stream) : launch<D, true, false>(a, stream);
  return a.out_f32 ? launch<D, false, true>(a, stream) : launch<D, false, false>(a, stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  static_assert(FwdTile<128>::BR == kFwdBf16RowsPerBlock, "tile table out of sync");
  if (a.d == 64) return launch_d<64>(a, stream);
  return launch_d<128>(a, stream);
}

}  // namespace fa
