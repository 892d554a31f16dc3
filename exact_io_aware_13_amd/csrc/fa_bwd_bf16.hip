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
//  1. pre:     D_i = rowsum(dO * O), lse in base 2, and a zeroed fp32 dQ
//              accumulator.
//  2. main:    one workgroup = 4 waves = 128 keys of one slice (32 per
//              wave).  K and V rows stay in registers as matrix-product
//              operands, dK and dV accumulate in registers over every
//              64-row query tile that can see the keys.  Per query tile the
//              workgroup recomputes S and P, forms dS, and adds its share of
//              dQ into the fp32 accumulator with buffer atomics.
//  3. convert: dQ = bf16(scale * accumulator).
//
// Matrix-core orientation in the main kernel.  S = Q K^T and dP = dO V^T are
// computed with queries as rows, so each lane owns one key (column) and 16
// queries of a 32-row block.  Those registers are directly the B operands of
// dV^T = dO^T P and dK^T = Q^T dS (the contraction over queries runs in the
// order the accumulator holds them); dO^T and Q^T come from the row-major
// LDS tiles through the transposing read (ds_read_b64_tr_b16).  dQ = dS K
// needs dS with queries as lanes, so each wave writes its dS block to LDS
// (keys as rows) and dQ reads it back transposed; the K^T operand of that
// product is read once per workgroup and stays in registers.
//
// Data movement.  Q, dO and the per-row statistics go from HBM/L2 straight
// into LDS with bounds-checked buffer loads (rows past the end read as zero),
// double-buffered one query tile ahead.  Each 16-byte chunk c of a Q/dO/K row
// r sits at chunk c ^ swz(r) (the same layout as the forward's K/V tiles);
// the dS tile swizzles 8-byte chunks the same way.  All reads and writes of
// these tiles are free of bank conflicts.
//
// Pipeline.  The dQ product of query tile t-1 runs during tile t (dS of
// tile t-1 is in LDS by then), so one workgroup barrier per tile suffices;
// its atomics go out in the middle of tile t, well before the barrier that
// waits for them.  Each tile's 80 (d=128) matrix products are issued in a fixed
// order with every LDS fragment read two products ahead and the vector work
// (probabilities, dS, statistics loads, dS stores, atomics) placed between
// them, so the vector ALUs run while the matrix cores are busy.
//
// Zero-filled rows make ragged tails need no masks: a query row past Lq has
// Q = dO = 0 and lse = D = 0, so P = 1 but dP = 0 and dS = 0, and its dO row
// adds nothing to dV; a key row past Lk has K = V = 0, so its dQ share is 0
// and its dK/dV rows are dropped by the store range check.  Only the causal
// diagonal needs a mask, in the first two query tiles of each workgroup.

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {
namespace {

// ---------------------------------------------------------------------------
// 1. D statistic, base-2 lse, accumulator reset
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_bf16_kernel(
    const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
    const float* __restrict__ lse, float* __restrict__ Dvec, float* __restrict__ lse2,
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
  if (row < rows && c == 0) {
    Dvec[row] = acc;
    lse2[row] = lse[row] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// 2. main kernel
// ---------------------------------------------------------------------------
template <int D>
struct BwdTile {
  static constexpr int NW = 4;                       // waves per workgroup
  static constexpr int BK = 32 * NW;                 // keys per workgroup
  static constexpr int BQ = 64;                      // query rows per tile
  static constexpr int KS = D / 16;                  // 16-deep steps over the head dimension
  static constexpr int DB = D / 32;                  // 32-wide head-dim blocks
  static constexpr int DBW = DB / 2;                 // dQ head-dim blocks per wave
  static constexpr int KSK = BK / 16;                // 16-deep steps over the workgroup's keys
  static constexpr int ROWB = D * 2;                 // bytes per Q / dO / K row
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int RPK = 1024 / ROWB;            // rows per 1-KiB load instruction
  static constexpr int QTB = BQ * ROWB;              // bytes per Q (or dO) tile
  static constexpr int QLOADS = QTB / 1024 / NW;     // load instructions per wave per tile
  static constexpr int KTB = BK * ROWB;              // bytes of the K tile (prologue only)
  static constexpr int KLOADS = KTB / 1024 / NW;
  static constexpr int DSB = BK * BQ * 2;            // bytes per dS tile (keys x queries)
  static constexpr int DSROWB = BQ * 2;              // bytes per dS row
  // Matrix products per tile, in issue order: S and dP of query block 0
  // (interleaved), dQ of the previous tile, S and dP of block 1, then dV and
  // dK of block 0 and of block 1 (interleaved).
  static constexpr int NA = 2 * KS;
  static constexpr int NB = KSK * DBW;
  static constexpr int NC = 2 * KS;
  static constexpr int ND = 4 * DB;
  static_assert(KTB <= 2 * DSB, "K staging reuses the two dS tiles");
  static_assert(QLOADS >= 1 && KLOADS >= 1, "tile split");
};

enum { OP_S, OP_DP, OP_DQ, OP_DV, OP_DK };
struct BwdOp {
  int kind, qb, ks, j, hf, db;
};

// Matrix product number i of a tile (see BwdTile for the order).
template <int D, bool HAS_DQ>
constexpr BwdOp bwd_op(int i) {
  using T = BwdTile<D>;
  const int nb = HAS_DQ ? T::NB : 0;
  BwdOp o{0, 0, 0, 0, 0, 0};
  if (i < T::NA) {
    o.kind = (i & 1) ? OP_DP : OP_S;
    o.ks = i >> 1;
  } else if (i < T::NA + nb) {
    const int x = i - T::NA;
    o.kind = OP_DQ;
    o.ks = x / T::DBW;
    o.j = x % T::DBW;
  } else if (i < T::NA + nb + T::NC) {
    const int x = i - T::NA - nb;
    o.kind = (x & 1) ? OP_DP : OP_S;
    o.qb = 1;
    o.ks = x >> 1;
  } else {
    int x = i - T::NA - nb - T::NC;
    o.qb = x / T::ND;
    x %= T::ND;
    o.hf = x / (2 * T::DB);
    x %= 2 * T::DB;
    o.db = x >> 1;
    o.kind = (x & 1) ? OP_DK : OP_DV;
  }
  return o;
}

// Slot of unit u of n units spread evenly over slots [b, b + ns).
constexpr int spread(int u, int n, int b, int ns) { return b + (u * ns) / n; }

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE2, const float* __restrict__ Dvec, float* __restrict__ dQacc,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int BH, int Lq, int Lk, float c,
    float scale) {
  using T = BwdTile<D>;
  // Double-buffered query-side tiles (one LDS array per buffer, so the
  // compiler waits only for the loads a read depends on), and two dS tiles,
  // which also stage the K tile in the prologue.
  __shared__ __attribute__((aligned(1024))) char Q0[T::QTB];
  __shared__ __attribute__((aligned(1024))) char Q1[T::QTB];
  __shared__ __attribute__((aligned(1024))) char G0[T::QTB];
  __shared__ __attribute__((aligned(1024))) char G1[T::QTB];
  __shared__ __attribute__((aligned(1024))) char DS[2 * T::DSB];
  __shared__ __attribute__((aligned(256))) float L0[T::BQ];
  __shared__ __attribute__((aligned(256))) float L1[T::BQ];
  __shared__ __attribute__((aligned(256))) float E0[T::BQ];
  __shared__ __attribute__((aligned(256))) float E1[T::BQ];
  auto qbuf = [&](auto I) __attribute__((always_inline)) -> char* {
    if constexpr (decltype(I)::value == 0) return Q0; else return Q1;
  };
  auto gbuf = [&](auto I) __attribute__((always_inline)) -> char* {
    if constexpr (decltype(I)::value == 0) return G0; else return G1;
  };
  auto lbuf = [&](auto I) __attribute__((always_inline)) -> float* {
    if constexpr (decltype(I)::value == 0) return L0; else return L1;
  };
  auto ebuf = [&](auto I) __attribute__((always_inline)) -> float* {
    if constexpr (decltype(I)::value == 0) return E0; else return E1;
  };

  const int tid = wi_id();
  // The wave index is the same on every lane; readfirstlane tells the
  // compiler so, which keeps everything derived from it in scalar registers.
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, n = lane & 31, h = lane >> 5;
  // Consecutive workgroups take the same key tile of different slices; key
  // tiles with the most visible query tiles are dispatched first.
  const int bh = wg_id() % BH;
  const int k0 = (wg_id() / BH) * T::BK;
  const int kw0 = k0 + 32 * w;
  const int key = kw0 + n;

  const size_t qoff = (size_t)bh * Lq * D, koff = (size_t)bh * Lk * D;
  const auto rq = make_rsrc(Q + qoff, (uint32_t)Lq * D * 2);
  const auto rdo = make_rsrc(dO + qoff, (uint32_t)Lq * D * 2);
  const auto rk = make_rsrc(K + koff, (uint32_t)Lk * D * 2);
  const auto rv = make_rsrc(V + koff, (uint32_t)Lk * D * 2);
  const auto rl = make_rsrc(LSE2 + (size_t)bh * Lq, (uint32_t)Lq * 4);
  const auto re = make_rsrc(Dvec + (size_t)bh * Lq, (uint32_t)Lq * 4);
  const auto racc = make_rsrc(dQacc + qoff, (uint32_t)Lq * D * 4);

  const int n_qt = (Lq + T::BQ - 1) / T::BQ;
  const int qt0 = CAUSAL ? min(k0 / T::BQ, n_qt) : 0;
  const int nsteps = n_qt - qt0;
  // At least two tiles run when any is visible: a tile past the end of the
  // queries reads as zeros and adds exactly nothing (dS = 0, dO = 0, and its
  // dQ atomics fall outside the range check), and one code path for every
  // workgroup keeps the accumulators in registers.
  const int nrun = nsteps > 0 ? max(nsteps, 2) : 0;

  // ---- tile fetch (Q, dO, lse2, D of query tile t into buffer set B) --------
  int fetch_off[T::QLOADS];
#pragma unroll
  for (int i = 0; i < T::QLOADS; ++i) {
    const int row = (w * T::QLOADS + i) * T::RPK + lane / T::CPR;
    const int chunk = (lane % T::CPR) ^ swz<D>(row);
    fetch_off[i] = (row * D + chunk * 8) * 2;
  }
  auto fetch = [&](auto Bc, int t) __attribute__((always_inline)) {
    const int q0 = (qt0 + t) * T::BQ;
#pragma unroll
    for (int i = 0; i < T::QLOADS; ++i) {
      const uint32_t off = (uint32_t)(q0 * T::ROWB + fetch_off[i]);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rq, (lds_void*)(qbuf(Bc) + (w * T::QLOADS + i) * 1024), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rdo, (lds_void*)(gbuf(Bc) + (w * T::QLOADS + i) * 1024), 16, off, 0, 0, 0);
    }
    if (w == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_void*)lbuf(Bc), 4,
                                               (uint32_t)(q0 + lane) * 4, 0, 0, 0);
    if (w == 1)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(re, (lds_void*)ebuf(Bc), 4,
                                               (uint32_t)(q0 + lane) * 4, 0, 0, 0);
  };

  // ---- per-lane LDS offsets ---------------------------------------------------
  // Q / dO fragment (A operand of S, dP): row 32 qb + n, chunk 2 ks + h.
  const int rsw = swz<D>(n);
  int koffs[T::KS];
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks) koffs[ks] = n * T::ROWB + (((2 * ks + h) ^ rsw) << 4);
  // Transposed fragment of a row-major [rows][D] tile: head-dim column
  // 32 db + n, rows 16 step + 8 half + 4 h + j (j = 0..3 from the 4 rows the
  // read gathers).  Used for dO^T, Q^T (rows = queries) and K^T (rows = keys).
  const int g4 = lane >> 4, u = lane & 15, j4 = u >> 2, t4 = u & 3;
  int toffs[2][T::DB];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int row = 8 * half + 4 * h + j4;
    const int sw = swz<D>(row);
#pragma unroll
    for (int db = 0; db < T::DB; ++db) {
      const int chunk = 4 * db + 2 * (g4 & 1) + (t4 >> 1);
      toffs[half][db] = row * T::ROWB + ((chunk ^ sw) << 4) + 8 * (t4 & 1);
    }
  }
  auto tread = [&](const char* base, int step, int db) __attribute__((always_inline)) {
    const u32x2 lo = lds_read_tr(base, step * 16 * T::ROWB + toffs[0][db]);
    const u32x2 hi = lds_read_tr(base, step * 16 * T::ROWB + toffs[1][db]);
    u32x4 a;
    a.x = lo.x;
    a.y = lo.y;
    a.z = hi.x;
    a.w = hi.y;
    return a;
  };
  // dS tile: row = key (0..127), 8-byte chunk q/4 stored at (q/4) ^ dsw(row).
  auto dsw = [](int r) { return ((r & 3) << 2) | ((r >> 2) & 3); };
  // Write of this lane's 4 queries 8g + 4h .. +3 of block qb: row 32 w + n.
  const int ds_wrow = (32 * w + n) * T::DSROWB;
  const int ds_wx = h ^ dsw(n);
  // Transposed read for dQ (A operand dS, queries as lanes): query
  // 32 (w >> 1) + n, keys 16 ks + 8 half + 4 h + j.
  int dsoffs[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int row = 8 * half + 4 * h + j4;
    const int chunk = 8 * (w >> 1) + 4 * (g4 & 1) + t4;
    dsoffs[half] = row * T::DSROWB + ((chunk ^ dsw(row)) << 3);
  }
  auto dsread = [&](const char* base, int ks) __attribute__((always_inline)) {
    const u32x2 lo = lds_read_tr(base, ks * 16 * T::DSROWB + dsoffs[0]);
    const u32x2 hi = lds_read_tr(base, ks * 16 * T::DSROWB + dsoffs[1]);
    u32x4 a;
    a.x = lo.x;
    a.y = lo.y;
    a.z = hi.x;
    a.w = hi.y;
    return a;
  };

  // ---- prologue ---------------------------------------------------------------
  // This lane's key row of K and V: B operands of S = Q K^T and dP = dO V^T.
  bf16x8 kf[T::KS], vf[T::KS];
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks) {
    kf[ks] = as_bf16x8(load16(rk, (uint32_t)(key * D + ks * 16 + h * 8) * 2));
    vf[ks] = as_bf16x8(load16(rv, (uint32_t)(key * D + ks * 16 + h * 8) * 2));
  }
  // K tile of the workgroup into the dS area, then this wave's K^T fragments
  // (B operands of dQ = dS K: head-dim blocks (w & 1) DBW + j).
#pragma unroll
  for (int i = 0; i < T::KLOADS; ++i) {
    const int row = (w * T::KLOADS + i) * T::RPK + lane / T::CPR;
    const int chunk = (lane % T::CPR) ^ swz<D>(row);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(DS + (w * T::KLOADS + i) * 1024), 16,
                                             (uint32_t)((k0 + row) * D + chunk * 8) * 2, 0, 0, 0);
  }
  if (nrun > 0) fetch(IC<0>{}, 0);
  wait_vm<0>();
  block_barrier();
  bf16x8 ktf[T::DBW][T::KSK];
#pragma unroll
  for (int j = 0; j < T::DBW; ++j)
#pragma unroll
    for (int ks = 0; ks < T::KSK; ++ks) ktf[j][ks] = as_bf16x8(tread(DS, ks, (w & 1) * T::DBW + j));
  block_barrier();  // K^T is in registers everywhere; the dS tiles are free

  f32x16 dvacc[T::DB], dkacc[T::DB], dq[T::DBW];
#pragma unroll
  for (int db = 0; db < T::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dvacc[db][r] = 0.f;
      dkacc[db][r] = 0.f;
    }
#pragma unroll
  for (int j = 0; j < T::DBW; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[j][r] = 0.f;

  // dQ rows of this wave: 32 (w >> 1) + 8 (r / 4) + 4 h + r % 4 of a tile,
  // columns 32 ((w & 1) DBW + j) + n.
  // The whole offset goes in the per-lane operand: the range check that drops
  // rows past Lq covers that operand and the immediate, not the scalar one.
  const int at_lane = ((32 * (w >> 1) + 4 * h) * D + (w & 1) * T::DBW * 32 + n) * 4;
  auto atomics = [&](auto Uc, int tq) __attribute__((always_inline)) {
    constexpr int uu = decltype(Uc)::value, j = uu / 16, r = uu % 16;
    const int off = at_lane + (qt0 + tq) * T::BQ * D * 4 + (8 * (r >> 2) * D) * 4 +
                    ((r & 3) * D + j * 32) * 4;
    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(dq[j][r], racc, off, 0, 0);
  };
  // dQ of a finished tile from the dS tile at `dsb` (whole product; epilogue).
  auto dq_tile = [&](const char* dsb) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < T::KSK; ++ks) {
      const bf16x8 a = as_bf16x8(dsread(dsb, ks));
#pragma unroll
      for (int j = 0; j < T::DBW; ++j) {
        if (ks == 0) {
          f32x16 z;
#pragma unroll
          for (int r = 0; r < 16; ++r) z[r] = 0.f;
          dq[j] = mma(a, ktf[j][ks], z);
        } else {
          dq[j] = mma(a, ktf[j][ks], dq[j]);
        }
      }
    }
  };

  // ---- one query tile -----------------------------------------------------------
  // PH 0: first tile (no dQ yet), 1: second, 2: steady state; every tile
  // after the first also computes and adds dQ of the previous tile.
  auto step = [&](auto Bc, auto PHc, int t) __attribute__((always_inline)) {
    constexpr int BUF = decltype(Bc)::value, PH = decltype(PHc)::value;
    constexpr bool HAS_DQ = PH >= 1, MASK = CAUSAL && PH <= 1;
    constexpr int NB = HAS_DQ ? T::NB : 0;
    constexpr int GB = T::NA, GC = GB + NB, GD = GC + T::NC, GE = GD + T::ND, NALL = GE + T::ND;
    constexpr int SM0 = HAS_DQ ? GB : GC, SM0N = HAS_DQ ? NB : T::NC;  // softmax of block 0
    const char* qb_ = qbuf(IC<BUF>{});
    const char* gb_ = gbuf(IC<BUF>{});
    const float* lb_ = lbuf(IC<BUF>{});
    const float* eb_ = ebuf(IC<BUF>{});
    char* dsw_b = DS + BUF * T::DSB;                // dS of this tile
    const char* dsr_b = DS + (BUF ^ 1) * T::DSB;    // dS of the previous tile
    const int q0 = (qt0 + t) * T::BQ;

    if (t + 1 < nrun) fetch(IC<BUF ^ 1>{}, t + 1);

    u32x4 afr[NALL];
    f32x16 s[2], dp[2];
    unsigned pp[2][8], pd[2][8];
    f32x4 lr[2][4], er[2][4];
    float xs[2][4][4], ps[2][4][4];
    // Causal: element (qb, g, i) of this lane is visible iff
    // q0 + 32 qb + 8 g + 4 h + i >= key.
    const int lim = q0 + 4 * h - key;

    auto read_frag = [&](auto Ic) __attribute__((always_inline)) {
      constexpr int i = decltype(Ic)::value;
      constexpr BwdOp o = bwd_op<D, HAS_DQ>(i);
      if constexpr (o.kind == OP_S) {
        afr[i] = lds_read16(qb_, o.qb * 32 * T::ROWB + koffs[o.ks]);
      } else if constexpr (o.kind == OP_DP) {
        afr[i] = lds_read16(gb_, o.qb * 32 * T::ROWB + koffs[o.ks]);
      } else if constexpr (o.kind == OP_DQ) {
        if constexpr (o.j == 0) afr[i] = dsread(dsr_b, o.ks);
      } else if constexpr (o.kind == OP_DV) {
        afr[i] = tread(gb_, 2 * o.qb + o.hf, o.db);
      } else {
        afr[i] = tread(qb_, 2 * o.qb + o.hf, o.db);
      }
    };
    auto product = [&](auto Ic) __attribute__((always_inline)) {
      constexpr int i = decltype(Ic)::value;
      constexpr BwdOp o = bwd_op<D, HAS_DQ>(i);
      f32x16 z;
#pragma unroll
      for (int r = 0; r < 16; ++r) z[r] = 0.f;
      if constexpr (o.kind == OP_S) {
        s[o.qb] = mma(as_bf16x8(afr[i]), kf[o.ks], o.ks == 0 ? z : s[o.qb]);
      } else if constexpr (o.kind == OP_DP) {
        dp[o.qb] = mma(as_bf16x8(afr[i]), vf[o.ks], o.ks == 0 ? z : dp[o.qb]);
      } else if constexpr (o.kind == OP_DQ) {
        dq[o.j] = mma(as_bf16x8(afr[i - o.j]), ktf[o.j][o.ks], o.ks == 0 ? z : dq[o.j]);
      } else if constexpr (o.kind == OP_DV) {
        u32x4 b;
        b.x = pp[o.qb][o.hf * 4 + 0];
        b.y = pp[o.qb][o.hf * 4 + 1];
        b.z = pp[o.qb][o.hf * 4 + 2];
        b.w = pp[o.qb][o.hf * 4 + 3];
        dvacc[o.db] = mma(as_bf16x8(afr[i]), as_bf16x8(b), dvacc[o.db]);
      } else {
        u32x4 b;
        b.x = pd[o.qb][o.hf * 4 + 0];
        b.y = pd[o.qb][o.hf * 4 + 1];
        b.z = pd[o.qb][o.hf * 4 + 2];
        b.w = pd[o.qb][o.hf * 4 + 3];
        dkacc[o.db] = mma(as_bf16x8(afr[i]), as_bf16x8(b), dkacc[o.db]);
      }
    };
    // Softmax unit u (of 12) of query block qb: 4-element group g = u / 3
    // through stage u % 3 (FMA with lse; exp2 and mask; dS and packing).
    auto softmax_unit = [&](auto QBc, auto Uc) __attribute__((always_inline)) {
      constexpr int qb = decltype(QBc)::value, uu = decltype(Uc)::value, g = uu / 3, st = uu % 3;
      if constexpr (st == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xs[qb][g][i] = __builtin_fmaf(s[qb][4 * g + i], c, -lr[qb][g][i]);
          pin(xs[qb][g][i]);
        }
      } else if constexpr (st == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float p = fast_exp2(xs[qb][g][i]);
          if constexpr (MASK) {
            const unsigned hide = (unsigned)((lim + 32 * qb + 8 * g + i) >> 31);
            p = __builtin_bit_cast(float, __builtin_bit_cast(unsigned, p) & ~hide);
          }
          ps[qb][g][i] = p;
          pin(ps[qb][g][i]);
        }
      } else {
        float d4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) d4[i] = ps[qb][g][i] * (dp[qb][4 * g + i] - er[qb][g][i]);
        pp[qb][2 * g] = pack_bf16x2(ps[qb][g][0], ps[qb][g][1]);
        pp[qb][2 * g + 1] = pack_bf16x2(ps[qb][g][2], ps[qb][g][3]);
        pd[qb][2 * g] = pack_bf16x2(d4[0], d4[1]);
        pd[qb][2 * g + 1] = pack_bf16x2(d4[2], d4[3]);
        pin(pp[qb][2 * g]);
        pin(pp[qb][2 * g + 1]);
        pin(pd[qb][2 * g]);
        pin(pd[qb][2 * g + 1]);
      }
    };
    // Vector / memory work issued after matrix product SL.
    auto slot = [&](auto SLc) __attribute__((always_inline)) {
      constexpr int sl = decltype(SLc)::value;
      if constexpr (sl + 2 < NALL) read_frag(IC<sl + 2>{});
      // dQ atomics of tile t-1 (16 DBW per lane) once its products are done.
      if constexpr (HAS_DQ) {
        static_for<0, 16 * T::DBW>([&](auto Uc) __attribute__((always_inline)) {
          if constexpr (spread(decltype(Uc)::value, 16 * T::DBW, GC + 2, T::NC - 2) == sl)
            atomics(Uc, t - 1);
        });
      }
      // Row statistics of group g, two slots before the softmax unit that
      // first needs them (the first groups' during the preceding block).
      static_for<0, 4>([&](auto Gc) __attribute__((always_inline)) {
        constexpr int g = decltype(Gc)::value;
        constexpr int l0 = spread(3 * g, 12, SM0, SM0N) - 2, e0 = spread(3 * g + 2, 12, SM0, SM0N) - 2;
        constexpr int l1 = spread(3 * g, 12, GD, T::ND) - 2, e1 = spread(3 * g + 2, 12, GD, T::ND) - 2;
        if constexpr (l0 == sl) lr[0][g] = *reinterpret_cast<const f32x4*>(lb_ + 8 * g + 4 * h);
        if constexpr (e0 == sl) er[0][g] = *reinterpret_cast<const f32x4*>(eb_ + 8 * g + 4 * h);
        if constexpr (l1 == sl) lr[1][g] = *reinterpret_cast<const f32x4*>(lb_ + 32 + 8 * g + 4 * h);
        if constexpr (e1 == sl) er[1][g] = *reinterpret_cast<const f32x4*>(eb_ + 32 + 8 * g + 4 * h);
      });
      static_for<0, 12>([&](auto Uc) __attribute__((always_inline)) {
        constexpr int uu = decltype(Uc)::value;
        if constexpr (spread(uu, 12, SM0, SM0N) == sl) softmax_unit(IC<0>{}, Uc);
        if constexpr (spread(uu, 12, GD, T::ND) == sl) softmax_unit(IC<1>{}, Uc);
      });
      // dS stores: block 0 early in D, block 1 in the second half of E.
      static_for<0, 8>([&](auto Kc) __attribute__((always_inline)) {
        constexpr int k = decltype(Kc)::value, qb = k >> 2, g = k & 3;
        constexpr int at = qb == 0 ? GD + g : GE + T::ND / 2 + g;
        if constexpr (at == sl) {
          u32x2 v;
          v.x = pd[qb][2 * g];
          v.y = pd[qb][2 * g + 1];
          const int off = ds_wrow + (((qb * 8 + 2 * g) ^ ds_wx) << 3);
          *reinterpret_cast<u32x2*>(dsw_b + off) = v;
        }
      });
    };

    read_frag(IC<0>{});
    read_frag(IC<1>{});
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, NALL>([&](auto Ic) __attribute__((always_inline)) {
      product(Ic);
      slot(Ic);
      __builtin_amdgcn_sched_barrier(0);
    });

    wait_vm<0>();  // next tile landed, atomics issued in this tile done
    block_barrier();
  };

  if (nrun > 0) {
    step(IC<0>{}, IC<0>{}, 0);
    step(IC<1>{}, IC<1>{}, 1);
    for (int t = 2; t < nrun; t += 2) {
      step(IC<0>{}, IC<2>{}, t);
      if (t + 1 >= nrun) break;
      step(IC<1>{}, IC<2>{}, t + 1);
    }
    // dQ of the last tile.
    dq_tile(DS + ((nrun - 1) & 1) * T::DSB);
    static_for<0, 16 * T::DBW>([&](auto Uc) __attribute__((always_inline)) { atomics(Uc, nrun - 1); });
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
                       static_cast<const uint16_t*>(a.dO), a.lse, a.Dvec, a.lse2, a.dQacc, rows);
  }
  const int n_kt = (a.Lk + T::BK - 1) / T::BK;
  const dim3 grid((unsigned)(n_kt * a.BH));
  const float c = a.scale * kLog2e;
  if (a.causal)
    hipLaunchKernelGGL((bwd_bf16_kernel<D, true>), grid, dim3(64 * T::NW), 0, stream,
                       static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                       static_cast<const uint16_t*>(a.V), static_cast<const uint16_t*>(a.dO), a.lse2,
                       a.Dvec, a.dQacc, static_cast<uint16_t*>(a.dK), static_cast<uint16_t*>(a.dV),
                       a.BH, a.Lq, a.Lk, c, a.scale);
  else
    hipLaunchKernelGGL((bwd_bf16_kernel<D, false>), grid, dim3(64 * T::NW), 0, stream,
                       static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                       static_cast<const uint16_t*>(a.V), static_cast<const uint16_t*>(a.dO), a.lse2,
                       a.Dvec, a.dQacc, static_cast<uint16_t*>(a.dK), static_cast<uint16_t*>(a.dV),
                       a.BH, a.Lq, a.Lk, c, a.scale);
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
