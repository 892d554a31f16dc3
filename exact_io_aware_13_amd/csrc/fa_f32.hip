// Exact attention in fp32 (forward and backward), gfx950.
//
// The fp32 path serves fp32 callers and small problems where the answer
// must match the definition to ~1e-6 relative; it uses plain fp32 FMA, not
// matrix cores.  The forward uses the same online softmax as the bf16
// kernels (running max, running sum, rescaled unnormalised accumulator; "How
// Flash Attention Improves Transformer Memory Efficiency ...", section "The
// Three Running Statistics"); the backward recomputes P from the saved lse
// (section "Backward Pass Efficiency") and is split so that no atomics are
// needed: one kernel owns key rows (dK, dV), one owns query rows (dQ).
//
// Layout.  A row of the stationary operand (a query row in the forward and
// the dQ kernel, a key row in the dK/dV kernel) is spread over LPR = D/16
// consecutive lanes, each holding 16 of its columns in registers, so a
// wave covers 64/LPR rows and no per-thread array grows with D.  A dot
// product is 16 FMAs per lane and a reduction over the LPR lanes.  The four
// waves of a workgroup share the same rows and split the streamed range
// (keys, or queries for dK/dV) into four contiguous parts; each wave keeps
// its own running statistics or partial sums, and the parts are combined in
// LDS in a fixed order (the softmax merge of the running statistics for the
// forward, plain sums for the gradients), so results are bitwise
// reproducible.  Short sequences thus run on four times as many waves, which
// is what bounds the latency of the smallest workloads (the forward at
// d = 64 takes eight waves when its grid is smaller than the chip).

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr int kWaves = 4;        // waves per workgroup (they split the streamed range)
constexpr int kCols = 16;        // columns of a row per lane
constexpr int kGroup = 4;        // streamed rows per inner step

template <int D, int COLS = kCols>
struct F32Tile {
  static constexpr int LPR = D / COLS;         // lanes per row
  static constexpr int RPW = 64 / LPR;         // rows per wave (= per workgroup)
  static_assert(COLS * LPR == D && COLS % 4 == 0, "head dimension split");
};

// Sum over the LPR consecutive lanes that hold one row.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int o = 1; o < LPR; o <<= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <int N>
__device__ __forceinline__ void load_cols(const float* p, float (&v)[N]) {
  const f32x4* q = reinterpret_cast<const f32x4*>(p);
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    const f32x4 x = q[i];
    v[4 * i] = x[0];
    v[4 * i + 1] = x[1];
    v[4 * i + 2] = x[2];
    v[4 * i + 3] = x[3];
  }
}

template <int N>
__device__ __forceinline__ void store_cols(float* p, const float (&v)[N], float s) {
  f32x4* q = reinterpret_cast<f32x4*>(p);
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    f32x4 x;
    x[0] = v[4 * i] * s;
    x[1] = v[4 * i + 1] * s;
    x[2] = v[4 * i + 2] * s;
    x[3] = v[4 * i + 3] * s;
    q[i] = x;
  }
}

// The contiguous part [lo, hi) of [0, n) that wave w of NWV takes.
template <int NWV = kWaves>
__device__ __forceinline__ void wave_part(int n, int w, int& lo, int& hi) {
  const int chunk = (n + NWV - 1) / NWV;
  lo = min(n, w * chunk);
  hi = min(n, lo + chunk);
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
// Each wave streams its key part through a private ring of kRing LDS slots,
// filled by direct-to-LDS buffer loads kRing-1 chunks ahead of use: a wave
// reads only what it loaded itself, so its own s_waitcnt suffices (no
// barrier), and a short part costs one memory latency instead of one per
// group of keys.
constexpr int kRing = 4;

template <int D>
struct F32Ring {
  static constexpr int CH = kGroup;          // keys per chunk
  static constexpr int ROWB = D * 4;         // bytes per key row
  static constexpr int RPI = 1024 / ROWB;    // rows per 1-KiB load instruction
  static constexpr int LPC = CH / RPI;       // load instructions per tensor per chunk
  static constexpr int CHB = CH * ROWB;      // bytes per chunk of one tensor
  static constexpr int SLOTB = 2 * CHB;      // K then V
  static_assert(LPC >= 1 && LPC * RPI == CH, "chunk split");
};

// NWV waves per workgroup: kWaves, or twice that at d = 64 for launches of
// fewer workgroups than compute units, where each wave's chain of key
// chunks sets the latency (half the keys per wave, half the chain).
template <int D, bool CAUSAL, int NWV, int COLS>
__global__ __launch_bounds__(64 * NWV) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int BH, int Lq, int Lk, float c) {
  using T = F32Tile<D, COLS>;
  using RG = F32Ring<D>;
  // One array per ring slot (every wave's part of it), selected at compile
  // time, so the compiler relates each LDS read only to its own slot's loads.
  __shared__ __attribute__((aligned(1024))) char R0[NWV * RG::SLOTB];
  __shared__ __attribute__((aligned(1024))) char R1[NWV * RG::SLOTB];
  __shared__ __attribute__((aligned(1024))) char R2[NWV * RG::SLOTB];
  __shared__ __attribute__((aligned(1024))) char R3[NWV * RG::SLOTB];
  auto rslot = [&](auto I) __attribute__((always_inline)) -> char* {
    constexpr int v = decltype(I)::value;
    if constexpr (v == 0) return R0;
    else if constexpr (v == 1) return R1;
    else if constexpr (v == 2) return R2;
    else return R3;
  };
  static_assert(kRing == 4, "four slot arrays");
  __shared__ float sm[NWV][T::RPW], sl[NWV][T::RPW];
  __shared__ float sacc[NWV][64][COLS + 1];
  const int tid = wi_id();
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, r = lane / T::LPR, cc = lane % T::LPR;
  const int bh = wg_id() % BH;
  const int r0 = (wg_id() / BH) * T::RPW;
  const int qi = r0 + r;
  const bool valid = qi < Lq;
  const size_t qrow = (size_t)bh * Lq + (valid ? qi : 0);
  const auto rk = make_rsrc(K + (size_t)bh * Lk * D, (uint32_t)Lk * RG::ROWB);
  const auto rv = make_rsrc(V + (size_t)bh * Lk * D, (uint32_t)Lk * RG::ROWB);

  float q[COLS], acc[COLS];
  load_cols(Q + qrow * D + cc * COLS, q);
#pragma unroll
  for (int i = 0; i < COLS; ++i) acc[i] = 0.f;
  // Keys any row of the workgroup sees, split over the waves.
  const int kend = CAUSAL ? min(Lk, r0 + T::RPW) : Lk;
  int k_lo, k_hi;
  wave_part<NWV>(kend, w, k_lo, k_hi);
  const int nch = (k_hi - k_lo + RG::CH - 1) / RG::CH;

  // Chunk ch of the part into its slot: lane l of load i moves the 16 bytes
  // of row i*RPI + l/(D/4), column block l%(D/4), to slot byte 1024 i + 16 l
  // (rows in order, D floats each).  Chunks past the last re-fetch the last
  // one (rows past the part repeat its last row), which keeps the loads in
  // flight the same every iteration.
  const int lrow = lane / (D / 4), lcol = (lane % (D / 4)) * 16;
  auto fetch = [&](auto Sc, int ch) __attribute__((always_inline)) {
    // The resources go to the builtin through local references: passing the
    // by-reference captures themselves makes the host pass drop this
    // kernel's launch stub, with no diagnostic.
    const __amdgpu_buffer_rsrc_t& rkr = rk;
    const __amdgpu_buffer_rsrc_t& rvr = rv;
    const int c0 = k_lo + min(ch, nch - 1) * RG::CH;
    char* slot = rslot(Sc) + w * RG::SLOTB;
    static_for<0, RG::LPC>([&](auto Ic) __attribute__((always_inline)) {
      constexpr int i = decltype(Ic)::value;
      const int row = min(c0 + i * RG::RPI + lrow, k_hi - 1);
      const uint32_t off = (uint32_t)row * RG::ROWB + lcol;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rkr, (lds_void*)(slot + i * 1024), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rvr, (lds_void*)(slot + RG::CHB + i * 1024), 16, off,
                                               0, 0, 0);
    });
  };

  float m = -INFINITY, l = 0.f;
  auto step = [&](auto Sc, int ch) __attribute__((always_inline)) {
    constexpr int S = decltype(Sc)::value;
    fetch(IC<(S + kRing - 1) % kRing>{}, ch + kRing - 1);
    wait_vm<(kRing - 1) * 2 * RG::LPC>();  // chunk ch landed
    asm volatile("" ::: "memory");
    const float* kb = reinterpret_cast<const float*>(rslot(Sc) + w * RG::SLOTB);
    const float* vb = kb + RG::CHB / 4;
    const int j0 = k_lo + ch * RG::CH;
    float kv[kGroup][COLS], vv[kGroup][COLS], t[kGroup];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      load_cols(kb + g * D + cc * COLS, kv[g]);
      load_cols(vb + g * D + cc * COLS, vv[g]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < COLS; ++i) dot = fmaf(q[i], kv[g][i], dot);
      dot = row_sum<T::LPR>(dot);
      const int j = j0 + g;
      t[g] = (j < k_hi && !(CAUSAL && j > qi)) ? dot * c : -INFINITY;
      mx = fmaxf(mx, t[g]);
    }
    const float m_new = fmaxf(m, mx);
    // A row that has seen no visible key yet keeps m = -inf; its
    // probabilities are exp2(-inf) = 0 against a reference of 0.
    const float base = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m - base);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int i = 0; i < COLS; ++i) acc[i] *= alpha;
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const float p = exp2f(t[g] - base);
      l += p;
#pragma unroll
      for (int i = 0; i < COLS; ++i) acc[i] = fmaf(p, vv[g][i], acc[i]);
    }
  };
  if (nch > 0) {
    fetch(IC<0>{}, 0);
    fetch(IC<1>{}, 1);
    fetch(IC<2>{}, 2);
    for (int ch = 0; ch < nch; ch += kRing) {
      step(IC<0>{}, ch);
      if (ch + 1 >= nch) break;
      step(IC<1>{}, ch + 1);
      if (ch + 2 >= nch) break;
      step(IC<2>{}, ch + 2);
      if (ch + 3 >= nch) break;
      step(IC<3>{}, ch + 3);
    }
    wait_vm<0>();  // no load into the ring outlives the kernel's use of LDS
  }
  // Merge the four parts: M = max_w m_w, l = sum_w l_w 2^(m_w - M),
  // acc = sum_w acc_w 2^(m_w - M), in wave order.
  if (cc == 0) {
    sm[w][r] = m;
    sl[w][r] = l;
  }
#pragma unroll
  for (int i = 0; i < COLS; ++i) sacc[w][lane][i] = acc[i];
  __syncthreads();
  if (w == 0) {
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NWV; ++ww) M = fmaxf(M, sm[ww][r]);
    float lt = 0.f, o[COLS];
#pragma unroll
    for (int i = 0; i < COLS; ++i) o[i] = 0.f;
#pragma unroll
    for (int ww = 0; ww < NWV; ++ww) {
      const float mw = sm[ww][r];
      const float f = mw == -INFINITY ? 0.f : exp2f(mw - M);
      lt = fmaf(sl[ww][r], f, lt);
#pragma unroll
      for (int i = 0; i < COLS; ++i) o[i] = fmaf(sacc[ww][lane][i], f, o[i]);
    }
    if (valid) {
      store_cols(O + qrow * D + cc * COLS, o, 1.f / lt);
      if (cc == 0) LSE[qrow] = (M + log2f(lt)) * kLn2;
    }
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

// ---------------------------------------------------------------------------
// dK and dV: a workgroup owns RPW key rows; its waves split the queries that
// can see them, and the four partial sums are added in wave order.  Each
// wave streams its query rows (Q, dO, and the rows' base-2 lse and D)
// through a private LDS ring as the forward streams keys.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, int COLS>
__global__ __launch_bounds__(64 * kWaves) void bwd_dkdv_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE2, const float* __restrict__ Dvec,
    float* __restrict__ dK, float* __restrict__ dV, int BH, int Lq, int Lk, float c,
    float scale) {
  using T = F32Tile<D, COLS>;
  using RG = F32Ring<D>;
  constexpr int SB = RG::SLOTB + 32;  // Q rows, dO rows, 4 lse2, 4 D
  __shared__ __attribute__((aligned(1024))) char R0[kWaves * SB];
  __shared__ __attribute__((aligned(1024))) char R1[kWaves * SB];
  __shared__ __attribute__((aligned(1024))) char R2[kWaves * SB];
  __shared__ __attribute__((aligned(1024))) char R3[kWaves * SB];
  auto rslot = [&](auto I) __attribute__((always_inline)) -> char* {
    constexpr int v = decltype(I)::value;
    if constexpr (v == 0) return R0;
    else if constexpr (v == 1) return R1;
    else if constexpr (v == 2) return R2;
    else return R3;
  };
  __shared__ float sk[kWaves][64][COLS + 1], sv[kWaves][64][COLS + 1];
  const int tid = wi_id();
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, r = lane / T::LPR, cc = lane % T::LPR;
  const int bh = wg_id() % BH;
  const int k0 = (wg_id() / BH) * T::RPW;
  const int kj = k0 + r;
  const bool valid = kj < Lk;
  const size_t krow = (size_t)bh * Lk + (valid ? kj : 0);
  float kr[COLS], vr[COLS], ak[COLS], av[COLS];
  load_cols(K + krow * D + cc * COLS, kr);
  load_cols(V + krow * D + cc * COLS, vr);
#pragma unroll
  for (int i = 0; i < COLS; ++i) {
    ak[i] = 0.f;
    av[i] = 0.f;
  }
  const auto rq = make_rsrc(Q + (size_t)bh * Lq * D, (uint32_t)Lq * RG::ROWB);
  const auto rg = make_rsrc(dO + (size_t)bh * Lq * D, (uint32_t)Lq * RG::ROWB);
  const auto rl = make_rsrc(LSE2 + (size_t)bh * Lq, (uint32_t)Lq * 4);
  const auto rd = make_rsrc(Dvec + (size_t)bh * Lq, (uint32_t)Lq * 4);
  // Queries that can see a key of this workgroup, split over the waves.
  const int qstart = CAUSAL ? min(Lq, k0) : 0;
  int q_lo, q_hi;
  wave_part(Lq - qstart, w, q_lo, q_hi);
  q_lo += qstart;
  q_hi += qstart;
  const int nch = (q_hi - q_lo + RG::CH - 1) / RG::CH;

  // Chunk ch of the part into its slot (the forward's layout for the rows;
  // lanes 0-3 then move the chunk's four lse2 and four D values, rows past
  // Lq reading as zero).  The resources go to the builtin through local
  // references (see the forward).
  const int lrow = lane / (D / 4), lcol = (lane % (D / 4)) * 16;
  auto fetch = [&](auto Sc, int ch) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t& rqr = rq;
    const __amdgpu_buffer_rsrc_t& rgr = rg;
    const __amdgpu_buffer_rsrc_t& rlr = rl;
    const __amdgpu_buffer_rsrc_t& rdr = rd;
    const int c0 = q_lo + min(ch, nch - 1) * RG::CH;
    char* slot = rslot(Sc) + w * SB;
    static_for<0, RG::LPC>([&](auto Ic) __attribute__((always_inline)) {
      constexpr int i = decltype(Ic)::value;
      const int row = min(c0 + i * RG::RPI + lrow, q_hi - 1);
      const uint32_t off = (uint32_t)row * RG::ROWB + lcol;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rqr, (lds_void*)(slot + i * 1024), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rgr, (lds_void*)(slot + RG::CHB + i * 1024), 16, off,
                                               0, 0, 0);
    });
    if (lane < RG::CH) {
      const uint32_t off = (uint32_t)(c0 + lane) * 4;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rlr, (lds_void*)(slot + RG::SLOTB), 4, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rdr, (lds_void*)(slot + RG::SLOTB + 16), 4, off, 0, 0, 0);
    }
  };
  auto step = [&](auto Sc, int ch) __attribute__((always_inline)) {
    constexpr int S = decltype(Sc)::value;
    fetch(IC<(S + kRing - 1) % kRing>{}, ch + kRing - 1);
    wait_vm<(kRing - 1) * (2 * RG::LPC + 2)>();  // chunk ch landed
    asm volatile("" ::: "memory");
    const char* slot = rslot(Sc) + w * SB;
    const float* qb = reinterpret_cast<const float*>(slot);
    const float* gb = qb + RG::CHB / 4;
    const float* st = reinterpret_cast<const float*>(slot + RG::SLOTB);
    const int i0 = q_lo + ch * RG::CH;
    float qv[kGroup][COLS], gv[kGroup][COLS];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      load_cols(qb + g * D + cc * COLS, qv[g]);
      load_cols(gb + g * D + cc * COLS, gv[g]);
    }
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int x = 0; x < COLS; ++x) {
        s = fmaf(qv[g][x], kr[x], s);
        dp = fmaf(gv[g][x], vr[x], dp);
      }
      s = row_sum<T::LPR>(s);
      dp = row_sum<T::LPR>(dp);
      const int i = i0 + g;
      const bool vis = i < q_hi && !(CAUSAL && i < kj);
      const float p = vis ? exp2f(s * c - st[g]) : 0.f;
      const float ds = p * (dp - st[4 + g]);
#pragma unroll
      for (int x = 0; x < COLS; ++x) {
        av[x] = fmaf(p, gv[g][x], av[x]);
        ak[x] = fmaf(ds, qv[g][x], ak[x]);
      }
    }
  };
  static_assert(RG::CH == 4 && kGroup == 4, "four rows of lse2 and D per chunk");
  if (nch > 0) {
    fetch(IC<0>{}, 0);
    fetch(IC<1>{}, 1);
    fetch(IC<2>{}, 2);
    for (int ch = 0; ch < nch; ch += kRing) {
      step(IC<0>{}, ch);
      if (ch + 1 >= nch) break;
      step(IC<1>{}, ch + 1);
      if (ch + 2 >= nch) break;
      step(IC<2>{}, ch + 2);
      if (ch + 3 >= nch) break;
      step(IC<3>{}, ch + 3);
    }
    wait_vm<0>();
  }
#pragma unroll
  for (int x = 0; x < COLS; ++x) {
    sk[w][lane][x] = ak[x];
    sv[w][lane][x] = av[x];
  }
  __syncthreads();
  if (w == 0 && valid) {
    float tk[COLS], tv[COLS];
#pragma unroll
    for (int x = 0; x < COLS; ++x) {
      tk[x] = sk[0][lane][x];
      tv[x] = sv[0][lane][x];
    }
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww)
#pragma unroll
      for (int x = 0; x < COLS; ++x) {
        tk[x] += sk[ww][lane][x];
        tv[x] += sv[ww][lane][x];
      }
    store_cols(dK + krow * D + cc * COLS, tk, scale);
    store_cols(dV + krow * D + cc * COLS, tv, 1.f);
  }
}

// ---------------------------------------------------------------------------
// dQ: a workgroup owns RPW query rows; its waves split the keys they see, and
// the four partial sums are added in wave order.  Keys stream through a
// private LDS ring per wave, as in the forward.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, int COLS>
__global__ __launch_bounds__(64 * kWaves) void bwd_dq_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE2, const float* __restrict__ Dvec,
    float* __restrict__ dQ, int BH, int Lq, int Lk, float c, float scale) {
  using T = F32Tile<D, COLS>;
  using RG = F32Ring<D>;
  __shared__ __attribute__((aligned(1024))) char R0[kWaves * RG::SLOTB];
  __shared__ __attribute__((aligned(1024))) char R1[kWaves * RG::SLOTB];
  __shared__ __attribute__((aligned(1024))) char R2[kWaves * RG::SLOTB];
  __shared__ __attribute__((aligned(1024))) char R3[kWaves * RG::SLOTB];
  auto rslot = [&](auto I) __attribute__((always_inline)) -> char* {
    constexpr int v = decltype(I)::value;
    if constexpr (v == 0) return R0;
    else if constexpr (v == 1) return R1;
    else if constexpr (v == 2) return R2;
    else return R3;
  };
  __shared__ float sq[kWaves][64][COLS + 1];
  const int tid = wi_id();
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, r = lane / T::LPR, cc = lane % T::LPR;
  const int bh = wg_id() % BH;
  const int r0 = (wg_id() / BH) * T::RPW;
  const int qi = r0 + r;
  const bool valid = qi < Lq;
  const size_t qrow = (size_t)bh * Lq + (valid ? qi : 0);
  float qr[COLS], gr[COLS], aq[COLS];
  load_cols(Q + qrow * D + cc * COLS, qr);
  load_cols(dO + qrow * D + cc * COLS, gr);
#pragma unroll
  for (int i = 0; i < COLS; ++i) aq[i] = 0.f;
  const float lse2 = LSE2[qrow];
  const float Di = Dvec[qrow];
  const auto rk = make_rsrc(K + (size_t)bh * Lk * D, (uint32_t)Lk * RG::ROWB);
  const auto rv = make_rsrc(V + (size_t)bh * Lk * D, (uint32_t)Lk * RG::ROWB);
  const int kend = CAUSAL ? min(Lk, r0 + T::RPW) : Lk;
  int k_lo, k_hi;
  wave_part(kend, w, k_lo, k_hi);
  const int nch = (k_hi - k_lo + RG::CH - 1) / RG::CH;
  const int lrow = lane / (D / 4), lcol = (lane % (D / 4)) * 16;
  auto fetch = [&](auto Sc, int ch) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t& rkr = rk;
    const __amdgpu_buffer_rsrc_t& rvr = rv;
    const int c0 = k_lo + min(ch, nch - 1) * RG::CH;
    char* slot = rslot(Sc) + w * RG::SLOTB;
    static_for<0, RG::LPC>([&](auto Ic) __attribute__((always_inline)) {
      constexpr int i = decltype(Ic)::value;
      const int row = min(c0 + i * RG::RPI + lrow, k_hi - 1);
      const uint32_t off = (uint32_t)row * RG::ROWB + lcol;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rkr, (lds_void*)(slot + i * 1024), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rvr, (lds_void*)(slot + RG::CHB + i * 1024), 16, off,
                                               0, 0, 0);
    });
  };
  auto step = [&](auto Sc, int ch) __attribute__((always_inline)) {
    constexpr int S = decltype(Sc)::value;
    fetch(IC<(S + kRing - 1) % kRing>{}, ch + kRing - 1);
    wait_vm<(kRing - 1) * 2 * RG::LPC>();  // chunk ch landed
    asm volatile("" ::: "memory");
    const float* kb = reinterpret_cast<const float*>(rslot(Sc) + w * RG::SLOTB);
    const float* vb = kb + RG::CHB / 4;
    const int j0 = k_lo + ch * RG::CH;
    float kv[kGroup][COLS], vv[kGroup][COLS];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      load_cols(kb + g * D + cc * COLS, kv[g]);
      load_cols(vb + g * D + cc * COLS, vv[g]);
    }
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int x = 0; x < COLS; ++x) {
        s = fmaf(qr[x], kv[g][x], s);
        dp = fmaf(gr[x], vv[g][x], dp);
      }
      s = row_sum<T::LPR>(s);
      dp = row_sum<T::LPR>(dp);
      const int j = j0 + g;
      const bool vis = j < k_hi && !(CAUSAL && j > qi);
      const float ds = vis ? exp2f(s * c - lse2) * (dp - Di) : 0.f;
#pragma unroll
      for (int x = 0; x < COLS; ++x) aq[x] = fmaf(ds, kv[g][x], aq[x]);
    }
  };
  if (nch > 0) {
    fetch(IC<0>{}, 0);
    fetch(IC<1>{}, 1);
    fetch(IC<2>{}, 2);
    for (int ch = 0; ch < nch; ch += kRing) {
      step(IC<0>{}, ch);
      if (ch + 1 >= nch) break;
      step(IC<1>{}, ch + 1);
      if (ch + 2 >= nch) break;
      step(IC<2>{}, ch + 2);
      if (ch + 3 >= nch) break;
      step(IC<3>{}, ch + 3);
    }
    wait_vm<0>();
  }
#pragma unroll
  for (int x = 0; x < COLS; ++x) sq[w][lane][x] = aq[x];
  __syncthreads();
  if (w == 0 && valid) {
    float t[COLS];
#pragma unroll
    for (int x = 0; x < COLS; ++x) t[x] = sq[0][lane][x];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww)
#pragma unroll
      for (int x = 0; x < COLS; ++x) t[x] += sq[ww][lane][x];
    store_cols(dQ + qrow * D + cc * COLS, t, scale);
  }
}

template <int D, bool CAUSAL>
hipError_t fwd_launch(const FwdArgs& a, hipStream_t stream) {
  auto go = [&](auto NWc, auto COLSc) {
    constexpr int NWV = decltype(NWc)::value, COLS = decltype(COLSc)::value;
    using T = F32Tile<D, COLS>;
    const int64_t wgs = (int64_t)((a.Lq + T::RPW - 1) / T::RPW) * a.BH;
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, NWV, COLS>), dim3((unsigned)wgs), dim3(64 * NWV),
                       0, stream, static_cast<const float*>(a.Q), static_cast<const float*>(a.K),
                       static_cast<const float*>(a.V), static_cast<float*>(a.O), a.lse, a.BH, a.Lq,
                       a.Lk, a.scale * kLog2e);
  };
  // At d = 64 a grid smaller than the chip takes eight waves per workgroup
  // (their rings and merge buffers fit a compute unit's LDS; at d = 128
  // they would not) and spreads each row over more lanes -- 4 or 8 columns
  // each instead of 16, the fewest columns whose grid still fits the chip
  // in one round -- so the same work runs on 2-4x the compute units
  // (B1 H1 L128 d64: 7.8 -> 5.5 us; B1 H4 L512 d64: 18.8 -> 14.3 us).
  if constexpr (D == 64) {
    auto wgs = [&](auto COLSc) {
      using T = F32Tile<D, decltype(COLSc)::value>;
      return (int64_t)((a.Lq + T::RPW - 1) / T::RPW) * a.BH;
    };
    if (wgs(IC<kCols>{}) < kComputeUnits) {
      if (wgs(IC<4>{}) <= kComputeUnits) go(IC<2 * kWaves>{}, IC<4>{});
      else if (wgs(IC<8>{}) <= kComputeUnits) go(IC<2 * kWaves>{}, IC<8>{});
      else go(IC<2 * kWaves>{}, IC<kCols>{});
      return hipGetLastError();
    }
  }
  // At d = 128 the same narrower rows with four waves per workgroup
  // (B1 H1 L128 d128: 10.1 -> 7.5 us).
  if constexpr (D == 128) {
    auto wgs = [&](auto COLSc) {
      using T = F32Tile<D, decltype(COLSc)::value>;
      return (int64_t)((a.Lq + T::RPW - 1) / T::RPW) * a.BH;
    };
    if (wgs(IC<kCols>{}) < kComputeUnits) {
      if (wgs(IC<4>{}) <= kComputeUnits) go(IC<kWaves>{}, IC<4>{});
      else if (wgs(IC<8>{}) <= kComputeUnits) go(IC<kWaves>{}, IC<8>{});
      else go(IC<kWaves>{}, IC<kCols>{});
      return hipGetLastError();
    }
  }
  go(IC<kWaves>{}, IC<kCols>{});
  return hipGetLastError();
}

template <int D, bool CAUSAL, int COLS>
void bwd_launch_cols(const BwdArgs& a, unsigned stages, hipStream_t stream) {
  using T = F32Tile<D, COLS>;
  const auto* Q = static_cast<const float*>(a.Q);
  const auto* K = static_cast<const float*>(a.K);
  const auto* V = static_cast<const float*>(a.V);
  const auto* G = static_cast<const float*>(a.dO);
  const int n_kt = (a.Lk + T::RPW - 1) / T::RPW;
  if ((stages & kBwdDkDv) && n_kt > 0)
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D, CAUSAL, COLS>), dim3((unsigned)(n_kt * a.BH)),
                       dim3(64 * kWaves), 0, stream, Q, K, V, G, a.lse2, a.Dvec,
                       static_cast<float*>(a.dK), static_cast<float*>(a.dV), a.BH, a.Lq, a.Lk,
                       a.scale * kLog2e, a.scale);
  const int n_qt = (a.Lq + T::RPW - 1) / T::RPW;
  if ((stages & kBwdDq) && n_qt > 0)
    hipLaunchKernelGGL((bwd_dq_f32_kernel<D, CAUSAL, COLS>), dim3((unsigned)(n_qt * a.BH)),
                       dim3(64 * kWaves), 0, stream, Q, K, V, G, a.lse2, a.Dvec,
                       static_cast<float*>(a.dQ), a.BH, a.Lq, a.Lk, a.scale * kLog2e, a.scale);
}

template <int D, bool CAUSAL>
hipError_t bwd_launch(const BwdArgs& a, unsigned stages, hipStream_t stream) {
  const int64_t rows = (int64_t)a.BH * a.Lq;
  const auto* G = static_cast<const float*>(a.dO);
  if ((stages & kBwdPrepare) && rows > 0)
    hipLaunchKernelGGL((bwd_pre_f32_kernel<D>), dim3((unsigned)((rows + 255) / 256)), dim3(256), 0,
                       stream, static_cast<const float*>(a.O), G, a.lse, a.Dvec, a.lse2, rows);
  // Grids smaller than the chip spread each row over more lanes, as the
  // forward does: the fewest columns per lane (4 or 8) whose larger grid of
  // the two kernels still fits the chip in one round.
  const int64_t lmax = a.Lq > a.Lk ? a.Lq : a.Lk;
  auto wgs = [&](auto COLSc) {
    using T = F32Tile<D, decltype(COLSc)::value>;
    return (lmax + T::RPW - 1) / T::RPW * a.BH;
  };
  if (wgs(IC<kCols>{}) < kComputeUnits && wgs(IC<4>{}) <= kComputeUnits)
    bwd_launch_cols<D, CAUSAL, 4>(a, stages, stream);
  else if (wgs(IC<kCols>{}) < kComputeUnits && wgs(IC<8>{}) <= kComputeUnits)
    bwd_launch_cols<D, CAUSAL, 8>(a, stages, stream);
  else
    bwd_launch_cols<D, CAUSAL, kCols>(a, stages, stream);
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
