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
// Three stages, no atomics, every output written once by one workgroup in
// a fixed summation order (so the backward is bitwise deterministic):
//  1. pre:   -D_i = -rowsum(dO * O) and lse in base 2, per query row (the
//            negated D starts the dP accumulations).  When a call runs it
//            together with dQ (fa_bwd does) and O is bf16, the dQ kernel
//            does this work for its own rows and runs first, so the
//            separate kernel and its second read of dO drop out.
//  2. dK/dV: key-stationary.  One workgroup = 4 waves = 128 keys of one
//            slice (32 per wave); K and V rows stay in registers as
//            matrix-product operands, dK and dV accumulate in registers
//            over every 64-row query tile that can see the keys.
//  3. dQ:    query-stationary, laid out like the forward.  One workgroup =
//            256 query rows, 8 waves x 32 rows; K and V stream through
//            LDS, and per key tile the wave
//            recomputes S^T and dP^T, forms dS^T, and accumulates
//            dQ^T = K^T dS^T in registers.
// Splitting dQ off costs two extra matrix products per (key, query) tile
// pair (S and dP are computed by both kernels), but a fused kernel has to
// add every dQ partial into memory with fp32 atomics, 64 x d of them per
// workgroup per query tile, and L2 executes those far slower than the
// matrix cores run the two extra products.
//
// dK/dV kernel.  S = Q K^T and dP = dO V^T are computed with queries as
// rows, so each lane owns one key (column) and 16 queries of a 32-row block.
// Those registers are directly the B operands of dV^T = dO^T P and
// dK^T = Q^T dS (the contraction over queries runs in the order the
// accumulator holds them); dO^T and Q^T come from the row-major LDS tiles
// through the transposing read (ds_read_b64_tr_b16).  Q, dO and the per-row
// statistics go from HBM/L2 straight into LDS with bounds-checked buffer
// loads, double-buffered one query tile ahead, one workgroup barrier per
// tile.  Each tile's 64 (d=128) matrix products are issued in a fixed order
// with every LDS fragment read two products ahead and the vector work
// (probabilities, dS, statistics loads) placed between them.
//
// dQ kernel.  S^T = K Q^T and dP^T = V dO^T with keys as rows give each lane
// one query row (so lse and D are one register per lane) and 16 keys; the
// packed dS^T registers are the B operand of dQ^T = K^T dS^T, whose A
// operand comes from the K tile through the transposing read.  Iteration j
// runs S^T and dP^T of key tile j and then dQ^T of tile j-1; P of tile j is
// formed while the dP^T products run and dS of tile j while the dQ^T
// products of tile j-1 run.  K and V tiles come into 4-slot LDS rings two
// tiles ahead; the wave's Q and dO rows (B operands of S^T and dP^T) stay in
// registers.
//
// Every 16-byte chunk c of a Q/dO/K/V row r sits at chunk c ^ swz(r) in LDS
// (the forward's layout); all fragment reads are free of bank conflicts.
//
// Zero-filled rows make ragged tails need no masks: a query row past Lq has
// Q = dO = 0 and lse = D = 0, so P = 1 but dP = 0 and dS = 0, and its dO row
// adds nothing to dV; a key row past Lk has K = V = 0, so dP = 0, and its dQ
// share dS K is 0 while its dK/dV rows are dropped by the store range check.
// Only the causal diagonal needs a mask.

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_tile.h"

#include <type_traits>

namespace fa {
namespace {

// ---------------------------------------------------------------------------
// 1. D statistic (stored negated) and base-2 lse
// ---------------------------------------------------------------------------
// O_F32: O is the fp32 output of the forward's fp32-output variant (dO stays
// bf16); D is summed in fp32 either way.  A row takes D/8 lanes, 8 elements
// each.  NT (large bf16 tensors): each thread takes two rows, issuing all
// their loads first, and the O and dO loads carry the non-temporal hint --
// they are read once here (B1 H32 L4096 d128: 11.8 -> 10.2 us); tensors small
// enough to stay in the last-level cache between calls measured slower with
// the hint, and the second row alone gained nothing.
template <int D, bool NT>
constexpr int pre_rows_per_block() { return (NT ? 2 : 1) * 256 / (D / 8); }

// Sum over one 8-element chunk of O[r] * dO[r], one FMA chain in element
// order.  D is the pairwise sum of a row's chunk sums: chunks c and c ^ s
// are added for s = D/16, D/32, ..., 1, i.e. the butterfly over the row's
// lanes below, and the dQ kernel's fused variant adds them in the same
// order, so both give the same bits.
__device__ __forceinline__ float chunk_dot8(const float (&o)[8], u32x4 g) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = __builtin_fmaf(o[2 * i], bf16_lo(g[i]), acc);
    acc = __builtin_fmaf(o[2 * i + 1], bf16_hi(g[i]), acc);
  }
  return acc;
}

template <int D, bool O_F32, bool NT>
__global__ __launch_bounds__(256) void bwd_pre_bf16_kernel(
    const void* __restrict__ O, const uint16_t* __restrict__ dO,
    const float* __restrict__ lse, float* __restrict__ Dvec, float* __restrict__ lse2,
    int64_t rows) {
  constexpr int LPR = D / 8;          // lanes per row, 8 elements each
  constexpr int RPP = 256 / LPR;      // rows per pass of the workgroup
  constexpr int NR = NT ? 2 : 1;      // rows per thread
  const int c = wi_id() % LPR;
  auto ld = [](const auto* p) __attribute__((always_inline)) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
  };
  u32x4 g[NR];
  float o8[NR][8];
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    const int64_t row = ((int64_t)wg_id() * NR + u) * RPP + wi_id() / LPR;
    const int64_t r = row < rows ? row : rows - 1;  // past the end: a repeated row, not stored
    g[u] = ld(reinterpret_cast<const u32x4*>(dO + r * D + c * 8));
    if constexpr (O_F32) {
      const f32x4* op = reinterpret_cast<const f32x4*>(static_cast<const float*>(O) + r * D + c * 8);
      const f32x4 a = ld(op), b = ld(op + 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o8[u][i] = a[i];
        o8[u][4 + i] = b[i];
      }
    } else {
      const u32x4 o = ld(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(O) + r * D + c * 8));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o8[u][2 * i] = bf16_lo(o[i]);
        o8[u][2 * i + 1] = bf16_hi(o[i]);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    const int64_t row = ((int64_t)wg_id() * NR + u) * RPP + wi_id() / LPR;
    float acc = chunk_dot8(o8[u], g[u]);
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (row < rows && c == 0) {
      Dvec[row] = -acc;
      lse2[row] = lse[row] * kLog2e;
    }
  }
}

// Slot of unit u of n units spread evenly over slots [b, b + ns).
constexpr int spread(int u, int n, int b, int ns) { return b + (u * ns) / n; }

// ---------------------------------------------------------------------------
// 2. dK / dV kernel
// ---------------------------------------------------------------------------
template <int D>
struct KvTile {
  static constexpr int NW = 4;                       // waves per workgroup
  static constexpr int BK = 32 * NW;                 // keys per workgroup
  static constexpr int BQ = 64;                      // query rows per tile
  static constexpr int KS = D / 16;                  // 16-deep steps over the head dimension
  static constexpr int DB = D / 32;                  // 32-wide head-dim blocks
  static constexpr int ROWB = D * 2;                 // bytes per Q / dO row
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int RPK = 1024 / ROWB;            // rows per 1-KiB load instruction
  static constexpr int QTB = BQ * ROWB;              // bytes per Q (or dO) tile
  static constexpr int QLOADS = QTB / 1024 / NW;     // load instructions per wave per tile
  static constexpr int NFETCH = 2 * QLOADS + 1;      // Q, dO, row statistics
  static_assert(QLOADS <= 4, "immediate offsets reach 3 KiB");
  // Matrix products per tile, in issue order: S and dP of query block 0
  // (interleaved over the head dimension), the same for block 1, then dV
  // and dK of block 0 and of block 1 (interleaved).
  static constexpr int NA = 2 * KS;
  static constexpr int ND = 4 * DB;
  static constexpr int GC = NA, GD = 2 * NA, GE = GD + ND, NALL = GE + ND;
  static_assert(QLOADS >= 1, "tile split");
};

enum { OP_S, OP_DP, OP_DV, OP_DK };
struct KvOp {
  int kind, qb, ks, hf, db;
};

// Matrix product number i of a dK/dV tile (see KvTile for the order).
template <int D>
constexpr KvOp kv_op(int i) {
  using T = KvTile<D>;
  KvOp o{0, 0, 0, 0, 0};
  if (i < T::GD) {
    o.qb = i / T::NA;
    const int x = i % T::NA;
    o.kind = (x & 1) ? OP_DP : OP_S;
    o.ks = x >> 1;
  } else {
    int x = i - T::GD;
    o.qb = x / T::ND;
    x %= T::ND;
    o.hf = x / (2 * T::DB);
    x %= 2 * T::DB;
    o.db = x >> 1;
    o.kind = (x & 1) ? OP_DK : OP_DV;
  }
  return o;
}

// SPARSE: block-sparse backward -- the workgroup's 128 keys are one key
// block of the mask, and it visits only the 128-row query blocks whose mask
// entry for that key block is set (a compacted list, read through register
// windows as in the forward).
template <int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE2, const float* __restrict__ Dvec,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int BH, int Lq, int Lk, float c,
    float scale, const uint8_t* __restrict__ BM, int bm_stride, int nqb, int nkb) {
  using T = KvTile<D>;
  // Double-buffered query-side tiles, one LDS array per buffer, so the
  // compiler waits only for the loads a read depends on.
  __shared__ __attribute__((aligned(1024))) char Q0[T::QTB];
  __shared__ __attribute__((aligned(1024))) char Q1[T::QTB];
  __shared__ __attribute__((aligned(1024))) char G0[T::QTB];
  __shared__ __attribute__((aligned(1024))) char G1[T::QTB];
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
  const int key = k0 + 32 * w + n;

  const size_t qoff = (size_t)bh * Lq * D, koff = (size_t)bh * Lk * D;
  const auto rq = make_rsrc(Q + qoff, (uint32_t)Lq * D * 2);
  const auto rdo = make_rsrc(dO + qoff, (uint32_t)Lq * D * 2);
  const auto rk = make_rsrc(K + koff, (uint32_t)Lk * D * 2);
  const auto rv = make_rsrc(V + koff, (uint32_t)Lk * D * 2);
  const auto rl = make_rsrc(LSE2 + (size_t)bh * Lq, (uint32_t)Lq * 4);
  const auto re = make_rsrc(Dvec + (size_t)bh * Lq, (uint32_t)Lq * 4);

  const int n_qt = (Lq + T::BQ - 1) / T::BQ;
  const int qt0 = CAUSAL ? min(k0 / T::BQ, n_qt) : 0;
  int nsteps = n_qt - qt0;

  // ---- block-sparse: the query blocks that see this key block --------------
  constexpr int QPB = kSparseBlock / T::BQ;  // query tiles per mask block
  __shared__ uint16_t qlist[SPARSE ? kSparseMaxKeyBlocks : 1];
  __shared__ int wtot[SPARSE ? T::NW : 1];
  int nlist = 0, wbase = 0;
  unsigned win0 = 0, win1 = 0;
  if constexpr (SPARSE) {
    static_assert(T::BK == kSparseBlock, "one mask key block per workgroup");
    const int kb = k0 / kSparseBlock;
    const uint8_t* col = BM + (size_t)bh * bm_stride + kb;
    const int qb_lo = CAUSAL ? kb : 0;
    for (int base = qb_lo; base < nqb; base += 64 * T::NW) {
      const int qb = base + tid;
      const bool keep = qb < nqb && col[(size_t)qb * nkb] != 0;
      const uint64_t bal = __ballot(keep);
      const int below = __popcll(bal & ((uint64_t(1) << lane) - 1));
      if (lane == 0) wtot[w] = __popcll(bal);
      __syncthreads();
      int off = nlist, tot = 0;
      for (int ww = 0; ww < T::NW; ++ww) {
        if (ww < w) off += wtot[ww];
        tot += wtot[ww];
      }
      if (keep) qlist[off + below] = (uint16_t)qb;
      nlist += tot;
      __syncthreads();
    }
    nsteps = nlist * QPB;
    win0 = lane < nlist ? qlist[lane] : 0u;
    win1 = 64 + lane < nlist ? qlist[64 + lane] : 0u;
  }
  // Query tile of step t (past the last step: the first tile past the
  // queries, which reads as zeros).
  auto qtile = [&](int t) __attribute__((always_inline)) -> int {
    if constexpr (SPARSE) {
      if (t >= nsteps) return n_qt;
      const int e = t / QPB - wbase;
      const unsigned src = e < 64 ? win0 : win1;
      return __builtin_amdgcn_readlane((int)src, e & 63) * QPB + t % QPB;
    } else {
      return qt0 + t;
    }
  };
  auto window_for = [&](int tmax) __attribute__((always_inline)) {
    if constexpr (SPARSE) {
      if (min(tmax, nsteps - 1) / QPB - wbase >= 128) {
        wbase += 64;
        win0 = win1;
        const int e = wbase + 64 + lane;
        win1 = e < nlist ? qlist[e] : 0u;
      }
    }
  };
  // At least two tiles run when any is visible: a tile past the end of the
  // queries reads as zeros and adds exactly nothing, and one code path for
  // every workgroup keeps the accumulators in registers.
  const int nrun = nsteps > 0 ? max(nsteps, 2) : 0;

  // ---- tile fetch (Q, dO, lse2, D of query tile t into buffer set B) --------
  int fetch_off[T::QLOADS];
#pragma unroll
  for (int i = 0; i < T::QLOADS; ++i) {
    const int row = (w * T::QLOADS + i) * T::RPK + lane / T::CPR;
    const int chunk = (lane % T::CPR) ^ swz<D>(row);
    fetch_off[i] = (row * D + chunk * 8) * 2;
  }
  // The tile's fetch as NFETCH load instructions per wave, issued one at a
  // time between matrix products (unit u): the wave's Q rows, its dO rows,
  // then one row-statistics vector (lse2 from even waves, D from odd ones;
  // two waves write the same bytes with the same data).  Load i of a wave
  // goes 1 KiB after load i-1 in LDS and in memory (up to the swizzled
  // chunk, which sits in the per-lane offset), so the loads of one tensor
  // share one LDS base and differ in the immediate offset.
  auto fetch_unit = [&](auto Bc, int t, auto Uc) __attribute__((always_inline)) {
    constexpr int u = decltype(Uc)::value;
    const int q0 = qtile(t) * T::BQ;
    if constexpr (u < T::QLOADS) {
      constexpr int i = u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rq, (lds_void*)(qbuf(Bc) + w * T::QLOADS * 1024), 16,
          (uint32_t)(q0 * T::ROWB + fetch_off[i] - i * 1024), 0, i * 1024, 0);
    } else if constexpr (u < 2 * T::QLOADS) {
      constexpr int i = u - T::QLOADS;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rdo, (lds_void*)(gbuf(Bc) + w * T::QLOADS * 1024), 16,
          (uint32_t)(q0 * T::ROWB + fetch_off[i] - i * 1024), 0, i * 1024, 0);
    } else {
      const uint32_t off = (uint32_t)(q0 + lane) * 4;
      if (w & 1)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(re, (lds_void*)ebuf(Bc), 4, off, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_void*)lbuf(Bc), 4, off, 0, 0, 0);
    }
  };
  auto fetch = [&](auto Bc, int t) __attribute__((always_inline)) {
    static_for<0, T::NFETCH>([&](auto Uc) __attribute__((always_inline)) { fetch_unit(Bc, t, Uc); });
  };

  // ---- per-lane LDS offsets ---------------------------------------------------
  // Q / dO fragment (A operand of S, dP): row 32 qb + n, chunk 2 ks + h.
  const int rsw = swz<D>(n);
  int koffs[T::KS];
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks) koffs[ks] = n * T::ROWB + (((2 * ks + h) ^ rsw) << 4);
  // Transposed fragment (dO^T, Q^T): head-dim column 32 db + n, query rows
  // 16 step + 8 half + 4 h + j (j = 0..3 from the 4 rows the read gathers).
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

  // ---- prologue ---------------------------------------------------------------
  // This lane's key row of K and V: B operands of S = Q K^T and dP = dO V^T.
  bf16x8 kf[T::KS], vf[T::KS];
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks) {
    kf[ks] = as_bf16x8(load16(rk, (uint32_t)(key * D + ks * 16 + h * 8) * 2));
    vf[ks] = as_bf16x8(load16(rv, (uint32_t)(key * D + ks * 16 + h * 8) * 2));
  }
  if (nrun > 0) fetch(IC<0>{}, 0);
  wait_vm<0>();
  block_barrier();

  f32x16 dvacc[T::DB], dkacc[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dvacc[db][r] = 0.f;
      dkacc[db][r] = 0.f;
    }

  // ---- one query tile -----------------------------------------------------------
  // The first two tiles of a causal workgroup cross the diagonal and mask.
  auto step = [&](auto Bc, auto MASKc, int t) __attribute__((always_inline)) {
    constexpr int BUF = decltype(Bc)::value;
    constexpr bool MASK = decltype(MASKc)::value;
    const char* qb_ = qbuf(IC<BUF>{});
    const char* gb_ = gbuf(IC<BUF>{});
    const float* lb_ = lbuf(IC<BUF>{});
    const float* eb_ = ebuf(IC<BUF>{});

    u32x4 afr[T::NALL];
    f32x16 s[2], dp[2];
    unsigned pp[2][8], pd[2][8];
    f32x4 lr[2][4];
    // -D of the tile's rows as the dP chains' initial accumulator: the
    // products then leave dP - D in place.
    f32x16 nd[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 e = *reinterpret_cast<const f32x4*>(eb_ + 32 * qb + 8 * g + 4 * h);
#pragma unroll
        for (int i = 0; i < 4; ++i) nd[qb][4 * g + i] = e[i];
      }
    float xs[2][4][4], ps[2][4][4];
    // Causal: element (qb, g, i) of this lane is visible iff
    // q0 + 32 qb + 8 g + 4 h + i >= key.
    const int lim = qtile(t) * T::BQ + 4 * h - key;

    auto read_frag = [&](auto Ic) __attribute__((always_inline)) {
      constexpr int i = decltype(Ic)::value;
      constexpr KvOp o = kv_op<D>(i);
      if constexpr (o.kind == OP_S) afr[i] = lds_read16(qb_, o.qb * 32 * T::ROWB + koffs[o.ks]);
      else if constexpr (o.kind == OP_DP) afr[i] = lds_read16(gb_, o.qb * 32 * T::ROWB + koffs[o.ks]);
      else if constexpr (o.kind == OP_DV) afr[i] = tread(gb_, 2 * o.qb + o.hf, o.db);
      else afr[i] = tread(qb_, 2 * o.qb + o.hf, o.db);
    };
    auto product = [&](auto Ic) __attribute__((always_inline)) {
      constexpr int i = decltype(Ic)::value;
      constexpr KvOp o = kv_op<D>(i);
      f32x16 z;
#pragma unroll
      for (int r = 0; r < 16; ++r) z[r] = 0.f;
      if constexpr (o.kind == OP_S) {
        s[o.qb] = mma(as_bf16x8(afr[i]), kf[o.ks], o.ks == 0 ? z : s[o.qb]);
      } else if constexpr (o.kind == OP_DP) {
        dp[o.qb] = mma(as_bf16x8(afr[i]), vf[o.ks], o.ks == 0 ? nd[o.qb] : dp[o.qb]);
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
        for (int i = 0; i < 4; ++i) d4[i] = ps[qb][g][i] * dp[qb][4 * g + i];
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
    // Vector / memory work issued after matrix product SL.  Block 0's
    // probabilities run under block 1's S/dP products, block 1's under
    // block 0's dV/dK products.
    auto slot = [&](auto SLc) __attribute__((always_inline)) {
      constexpr int sl = decltype(SLc)::value;
      if constexpr (sl + 2 < T::NALL) read_frag(IC<sl + 2>{});
      // Next tile's loads, one every other product early in the tile (so
      // their issue overlaps the matrix cores).  The tile after the last one
      // is fetched too: it reads as zeros and nothing uses it.
      if constexpr (sl >= 2 && sl % 2 == 0 && (sl - 2) / 2 < T::NFETCH)
        fetch_unit(IC<BUF ^ 1>{}, t + 1, IC<(sl - 2) / 2>{});
      // Row statistics of group g, two slots before the unit that needs them.
      static_for<0, 4>([&](auto Gc) __attribute__((always_inline)) {
        constexpr int g = decltype(Gc)::value;
        constexpr int l0 = spread(3 * g, 12, T::GC, T::NA) - 2;
        constexpr int l1 = spread(3 * g, 12, T::GD, T::ND) - 2;
        if constexpr (l0 == sl) lr[0][g] = *reinterpret_cast<const f32x4*>(lb_ + 8 * g + 4 * h);
        if constexpr (l1 == sl) lr[1][g] = *reinterpret_cast<const f32x4*>(lb_ + 32 + 8 * g + 4 * h);
      });
      static_for<0, 12>([&](auto Uc) __attribute__((always_inline)) {
        constexpr int uu = decltype(Uc)::value;
        if constexpr (spread(uu, 12, T::GC, T::NA) == sl) softmax_unit(IC<0>{}, Uc);
        if constexpr (spread(uu, 12, T::GD, T::ND) == sl) softmax_unit(IC<1>{}, Uc);
      });
    };

    read_frag(IC<0>{});
    read_frag(IC<1>{});
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, T::NALL>([&](auto Ic) __attribute__((always_inline)) {
      product(Ic);
      slot(Ic);
      __builtin_amdgcn_sched_barrier(0);
    });

    wait_vm<0>();  // next tile landed
    block_barrier();
  };

  if (nrun > 0) {
    step(IC<0>{}, std::integral_constant<bool, CAUSAL>{}, 0);
    step(IC<1>{}, std::integral_constant<bool, CAUSAL>{}, 1);
    // Pairs of tiles with no exit between them (an exit after the first
    // body makes the register allocator give the two bodies different
    // accumulator registers and copy them every tile), then an odd last one.
    int t = 2;
    for (; t + 1 < nrun; t += 2) {
      window_for(t + 2);  // this pair fetches up to step t + 2
      step(IC<0>{}, std::false_type{}, t);
      step(IC<1>{}, std::false_type{}, t + 1);
    }
    window_for(t + 1);
    if (t < nrun) step(IC<0>{}, std::false_type{}, t);
  }

  // dK = scale * dK^T accumulator, dV = dV^T accumulator, staged for
  // whole-row stores in the query-tile buffers (no wave reads them after the
  // last step's barrier): waves 0 and 1 use Q0 and G0, waves 2 and 3 Q1 and G1.
  static_assert(2 * 32 * T::ROWB == T::QTB, "two waves' rows per query-tile buffer");
  u32x2 pk[T::DB][4], pv[T::DB][4];
#pragma unroll
  for (int db = 0; db < T::DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      pk[db][g].x = pack_bf16x2(scale * dkacc[db][4 * g + 0], scale * dkacc[db][4 * g + 1]);
      pk[db][g].y = pack_bf16x2(scale * dkacc[db][4 * g + 2], scale * dkacc[db][4 * g + 3]);
      pv[db][g].x = pack_bf16x2(dvacc[db][4 * g + 0], dvacc[db][4 * g + 1]);
      pv[db][g].y = pack_bf16x2(dvacc[db][4 * g + 2], dvacc[db][4 * g + 3]);
    }
  const int sto = (w & 1) * 32 * T::ROWB;
  store_rows_staged<D>((w < 2 ? Q0 : Q1) + sto, lane, pk, make_rsrc(dK + koff, (uint32_t)Lk * D * 2),
                       k0 + 32 * w);
  store_rows_staged<D>((w < 2 ? G0 : G1) + sto, lane, pv, make_rsrc(dV + koff, (uint32_t)Lk * D * 2),
                       k0 + 32 * w);
}

// ---------------------------------------------------------------------------
// 3. dQ kernel
// ---------------------------------------------------------------------------
template <int D, bool HALF>
struct DqTile {
  // 8 waves of one 32-row block (two waves per SIMD, each within 256
  // registers).  HALF: 4 waves, 128 rows, two workgroups per compute unit --
  // for launches that would otherwise give fewer than two workgroups per
  // compute unit, and for the block-sparse backward (one mask row block per
  // workgroup).
  static constexpr int NW = HALF ? 4 : 8;         // waves per workgroup
  static constexpr int RB = 1;                    // 32-row blocks per wave
  static constexpr int BR = 32 * RB * NW;         // query rows per workgroup
  static constexpr int BC = D == 128 ? 32 : 64;   // keys per tile
  static constexpr int NKB = BC / 32;             // 32-key blocks per tile
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int ROWB = D * 2;
  static constexpr int CPR = D / 8;
  static constexpr int TILEB = BC * ROWB;         // bytes per K (or V) tile
  static constexpr int RPK = 1024 / ROWB;
  static constexpr int LOADS = TILEB / 1024 / NW; // load instructions per wave per tile
  static_assert(LOADS <= 4, "immediate load offsets reach 3 KiB");
  static constexpr int NFRAG = NKB * KS;          // K (= V) fragments per tile
  static constexpr int NT = (BC / 16) * DB;       // K^T fragments per tile
  // Products per iteration: S^T of tile j, dP^T of tile j, dQ^T of tile j-1.
  static constexpr int NS = RB * NFRAG, NP = RB * NFRAG, NQ = RB * NT;
  static constexpr int NDS = RB * NKB * 4;        // 4-element groups per tile
  static_assert(LOADS >= 1, "tile split");
};

// MODE: 0 dense, 256 rows per workgroup; 1 dense, 128 rows; 2 block-sparse,
// 128 rows -- one row block of the mask, visiting the key blocks that row
// block sees (a compacted list read through register windows, as in the
// forward).
// PREP: the kernel also does the prepare kernel's work for its rows -- it
// reads the bf16 O rows and lse, forms -D and lse2 itself and writes them
// to Dvec / LSE2 for the dK/dV kernel launched after it (else it reads
// them there).
template <int D, bool CAUSAL, int MODE, bool PREP>
__global__ __launch_bounds__((64 * DqTile<D, MODE != 0>::NW), (MODE != 0 ? 2 : 1)) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const uint16_t* __restrict__ O, const float* __restrict__ LSE,
    float* __restrict__ LSE2, float* __restrict__ Dvec, uint16_t* __restrict__ dQ,
    int BH, int Lq, int Lk, int n_qt, float c, float scale,
    const uint8_t* __restrict__ BM, int bm_stride, int nqb, int nkb) {
  using T = DqTile<D, MODE != 0>;
  constexpr bool SPARSE = MODE == 2;
  // 4-slot rings for K and V, one LDS array per slot.
  __shared__ __attribute__((aligned(1024))) char K0[T::TILEB];
  __shared__ __attribute__((aligned(1024))) char K1[T::TILEB];
  __shared__ __attribute__((aligned(1024))) char K2[T::TILEB];
  __shared__ __attribute__((aligned(1024))) char K3[T::TILEB];
  __shared__ __attribute__((aligned(1024))) char V0[T::TILEB];
  __shared__ __attribute__((aligned(1024))) char V1[T::TILEB];
  __shared__ __attribute__((aligned(1024))) char V2[T::TILEB];
  __shared__ __attribute__((aligned(1024))) char V3[T::TILEB];
  auto kslot = [&](auto I) __attribute__((always_inline)) -> char* {
    constexpr int v = decltype(I)::value;
    if constexpr (v == 0) return K0;
    else if constexpr (v == 1) return K1;
    else if constexpr (v == 2) return K2;
    else return K3;
  };
  auto vslot = [&](auto I) __attribute__((always_inline)) -> char* {
    constexpr int v = decltype(I)::value;
    if constexpr (v == 0) return V0;
    else if constexpr (v == 1) return V1;
    else if constexpr (v == 2) return V2;
    else return V3;
  };

  const int tid = wi_id();
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, n = lane & 31, h = lane >> 5;
  // Same tile order as the forward: consecutive workgroups take the same
  // query tile of different slices, the most expensive causal tiles first.
  // With 128-row causal tiles all resident at once, workgroups g and
  // g + grid/2 share a compute unit, and the second half runs lightest-first
  // (the forward's rule).
  const int bh = wg_id() % BH;
  int qt = wg_id() / BH;
  if (CAUSAL) {
    if (MODE == 1 && (n_qt & 1) == 0 && n_qt * BH <= 2 * kComputeUnits && qt >= n_qt / 2)
      qt -= n_qt / 2;
    else
      qt = n_qt - 1 - qt;
  }
  const int q0 = qt * T::BR;
  const int qw0 = q0 + 32 * T::RB * w;

  const size_t qoff = (size_t)bh * Lq * D, koff = (size_t)bh * Lk * D;
  const auto rq = make_rsrc(Q + qoff, (uint32_t)Lq * D * 2);
  const auto rdo = make_rsrc(dO + qoff, (uint32_t)Lq * D * 2);
  const auto rk = make_rsrc(K + koff, (uint32_t)Lk * D * 2);
  const auto rv = make_rsrc(V + koff, (uint32_t)Lk * D * 2);
  const auto rl = make_rsrc(LSE2 + (size_t)bh * Lq, (uint32_t)Lq * 4);
  const auto re = make_rsrc(Dvec + (size_t)bh * Lq, (uint32_t)Lq * 4);

  int nkt = (Lk + T::BC - 1) / T::BC;
  if (CAUSAL) nkt = min(nkt, (q0 + T::BR - 1) / T::BC + 1);

  // ---- block-sparse: the key blocks this row block sees ----------------------
  // Entry: key block in bits 0..13; bit 14 set (the workgroup's one row
  // block sees it -- every listed block, kept in the format the tile masks
  // read).
  constexpr int TPB = kSparseBlock / T::BC;  // key tiles per mask block
  __shared__ uint16_t klist[SPARSE ? kSparseMaxKeyBlocks : 1];
  __shared__ int wtot[SPARSE ? T::NW : 1];
  const int wq = (32 * T::RB * w) / kSparseBlock;  // this wave's row block (0)
  int nlist = 0, wbase = 0;
  unsigned win0 = 0, win1 = 0;
  if constexpr (SPARSE) {
    static_assert(T::BR == kSparseBlock, "one mask row block per workgroup");
    const int qb0 = q0 / kSparseBlock;
    const uint8_t* row0 = BM + (size_t)bh * bm_stride + (size_t)qb0 * nkb;
    const int kb_lim = CAUSAL ? min(nkb, (q0 + T::BR - 1) / kSparseBlock + 1) : nkb;
    for (int base = 0; base < kb_lim; base += 64 * T::NW) {
      const int kb = base + tid;
      const bool f0 = kb < kb_lim && row0[kb] != 0;
      const uint64_t bal = __ballot(f0);
      const int below = __popcll(bal & ((uint64_t(1) << lane) - 1));
      if (lane == 0) wtot[w] = __popcll(bal);
      __syncthreads();
      int off = nlist, tot = 0;
      for (int ww = 0; ww < T::NW; ++ww) {
        if (ww < w) off += wtot[ww];
        tot += wtot[ww];
      }
      if (f0) klist[off + below] = (uint16_t)(kb | (1 << 14));
      nlist += tot;
      __syncthreads();
    }
    nkt = nlist * TPB;
    win0 = lane < nlist ? klist[lane] : 0u;
    win1 = 64 + lane < nlist ? klist[64 + lane] : 0u;
  }
  // This wave's own trip count (the forward's rule): under a causal mask
  // its rows see no key past tile (qw0 + 32 RB - 1) / BC, and rows all past
  // Lq compute nothing that is kept.  Past it the wave only issues its share
  // of the loads and joins the barriers; block-sparse workgroups run their
  // list with every wave.
  int nkt_w = nkt;
  if constexpr (!SPARSE) {
    if (CAUSAL) nkt_w = min(nkt, (qw0 + 32 * T::RB - 1) / T::BC + 1);
    if (qw0 >= Lq) nkt_w = 1;
  }
  auto entry_at = [&](int j) __attribute__((always_inline)) -> unsigned {
    const int e = j / TPB - wbase;
    const unsigned src = e < 64 ? win0 : win1;
    return (unsigned)__builtin_amdgcn_readlane((int)src, e & 63);
  };
  // Key tile of loop position j, and whether this wave's row block sees it.
  auto tile_at = [&](int j) __attribute__((always_inline)) -> int {
    if constexpr (SPARSE) return (int)(entry_at(j) & 0x3fffu) * TPB + j % TPB;
    else return j;
  };
  auto own_sees = [&](int j) __attribute__((always_inline)) -> bool {
    if constexpr (SPARSE) return (entry_at(j) >> (14 + wq)) & 1u;
    else return true;
  };
  auto window_for = [&](int jmax) __attribute__((always_inline)) {
    if constexpr (SPARSE) {
      if (min(jmax, nkt - 1) / TPB - wbase >= 128) {
        wbase += 64;
        win0 = win1;
        const int e = wbase + 64 + lane;
        win1 = e < nlist ? klist[e] : 0u;
      }
    }
  };

  // ---- K / V tile fetch into ring slots -----------------------------------------
  int fetch_off[T::LOADS];
#pragma unroll
  for (int i = 0; i < T::LOADS; ++i) {
    const int row = (w * T::LOADS + i) * T::RPK + lane / T::CPR;
    const int chunk = (lane % T::CPR) ^ swz<D>(row);
    fetch_off[i] = (row * D + chunk * 8) * 2;
  }
  auto fetch = [&](int tile, auto SLc) __attribute__((always_inline)) {
    // Tiles past the last one re-fetch the last tile into a free slot, which
    // keeps the number of loads in flight the same every iteration.
    // One LDS base per tensor; load i adds i KiB through the immediate offset.
    const int t = tile_at(min(tile, nkt - 1));
    lds_void* kd = (lds_void*)(kslot(SLc) + w * T::LOADS * 1024);
    lds_void* vd = (lds_void*)(vslot(SLc) + w * T::LOADS * 1024);
    static_for<0, T::LOADS>([&](auto Ic) __attribute__((always_inline)) {
      constexpr int i = decltype(Ic)::value;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, kd, 16, (uint32_t)(t * T::TILEB + fetch_off[i] - i * 1024), 0, i * 1024, 0);
    });
    static_for<0, T::LOADS>([&](auto Ic) __attribute__((always_inline)) {
      constexpr int i = decltype(Ic)::value;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, vd, 16, (uint32_t)(t * T::TILEB + fetch_off[i] - i * 1024), 0, i * 1024, 0);
    });
  };

  // ---- per-lane LDS offsets ---------------------------------------------------
  // K / V fragment (A operand of S^T, dP^T): key row 32 kb + n, chunk 2 ks + h.
  const int rsw = swz<D>(n);
  int koffs[T::KS];
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks) koffs[ks] = n * T::ROWB + (((2 * ks + h) ^ rsw) << 4);
  auto fread = [&](const char* base, int f) __attribute__((always_inline)) {
    return lds_read16(base, (f % T::NKB) * 32 * T::ROWB + koffs[f / T::NKB]);
  };
  // K^T fragment (A operand of dQ^T): head-dim column 32 db + n, keys
  // 16 step + 8 half + 4 h + j -- the key order the S^T accumulator holds.
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
  auto tread = [&](const char* base, int f) __attribute__((always_inline)) {
    const int step = f / T::DB, db = f % T::DB;
    const u32x2 lo = lds_read_tr(base, step * 16 * T::ROWB + toffs[0][db]);
    const u32x2 hi = lds_read_tr(base, step * 16 * T::ROWB + toffs[1][db]);
    u32x4 a;
    a.x = lo.x;
    a.y = lo.y;
    a.z = hi.x;
    a.w = hi.y;
    return a;
  };

  // ---- per-row operands: Q and dO rows (B operands of S^T and dP^T), lse2
  // and D; all stay in registers for the whole kernel -----------------------
  bf16x8 qf[T::RB][T::KS];
  u32x4 gf[T::RB][T::KS];
  float lse2[T::RB], dd[T::RB];
#pragma unroll
  for (int rb = 0; rb < T::RB; ++rb) {
    const int qrow = qw0 + 32 * rb + n;
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      qf[rb][ks] = as_bf16x8(load16(rq, (uint32_t)(qrow * D + ks * 16 + h * 8) * 2));
      gf[rb][ks] = load16(rdo, (uint32_t)(qrow * D + ks * 16 + h * 8) * 2);
    }
    if constexpr (PREP) {
      // The lane holds chunks c = 2 ks + h of its row (8 elements each) of
      // dO, and reads the same chunks of O: the chunk sums are combined in
      // the prepare kernel's pairwise order (c with c ^ 2s, s = KS/2 .. 1,
      // within the lane; then c with c ^ 1, the other half of the wave).
      // Rows past Lq read zeros and are not stored.
      const auto ro = make_rsrc(O + qoff, (uint32_t)Lq * D * 2);
      const auto rlse = make_rsrc(LSE + (size_t)bh * Lq, (uint32_t)Lq * 4);
      u32x4 of[T::KS];
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) of[ks] = load16(ro, (uint32_t)(qrow * D + ks * 16 + h * 8) * 2);
      const float lraw = load4f(rlse, (uint32_t)qrow * 4);
      float part[T::KS];
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) {
        float o8[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o8[2 * i] = bf16_lo(of[ks][i]);
          o8[2 * i + 1] = bf16_hi(of[ks][i]);
        }
        part[ks] = chunk_dot8(o8, gf[rb][ks]);
      }
#pragma unroll
      for (int st = T::KS / 2; st >= 1; st >>= 1)
#pragma unroll
        for (int ks = 0; ks < st; ++ks) part[ks] = part[ks] + part[ks + st];
      const float dsum = part[0] + __shfl_xor(part[0], 32, 64);
      lse2[rb] = lraw * kLog2e;
      dd[rb] = -dsum;
      if (h == 0 && qrow < Lq) {
        Dvec[(size_t)bh * Lq + qrow] = dd[rb];
        LSE2[(size_t)bh * Lq + qrow] = lse2[rb];
      }
    } else {
      lse2[rb] = load4f(rl, (uint32_t)qrow * 4);
      dd[rb] = load4f(re, (uint32_t)qrow * 4);
    }
  }
  // -D of the lane's row in every element: the initial accumulator of each
  // dP^T chain, so the products leave dP - D in place.
  f32x16 ndv[T::RB];
#pragma unroll
  for (int rb = 0; rb < T::RB; ++rb)
#pragma unroll
    for (int r = 0; r < 16; ++r) ndv[rb][r] = dd[rb];
  f32x16 dq[T::RB][T::DB];
#pragma unroll
  for (int rb = 0; rb < T::RB; ++rb)
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[rb][db][r] = 0.f;

  // Packed dS^T of two consecutive tiles (roles alternate by iteration
  // parity): one is read by the dQ^T products of tile j-1 while iteration j
  // writes the other.
  unsigned dskA[T::RB][T::NKB][8], dskB[T::RB][T::NKB][8];
#pragma unroll
  for (int rb = 0; rb < T::RB; ++rb)
#pragma unroll
    for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        dskA[rb][kb][i] = 0u;
        dskB[rb][kb][i] = 0u;
      }

  // dQ^T product f (K^T fragment a) of row block rb with packed dS^T `ds`.
  auto dq_product = [&](const u32x4& a, const unsigned (&ds)[T::RB][T::NKB][8], auto Fc, auto RBc)
                        __attribute__((always_inline)) {
    constexpr int f = decltype(Fc)::value, rb = decltype(RBc)::value;
    constexpr int step = f / T::DB, db = f % T::DB, kb = step >> 1, hf = step & 1;
    u32x4 b;
    b.x = ds[rb][kb][hf * 4 + 0];
    b.y = ds[rb][kb][hf * 4 + 1];
    b.z = ds[rb][kb][hf * 4 + 2];
    b.w = ds[rb][kb][hf * 4 + 3];
    dq[rb][db] = mma(as_bf16x8(a), as_bf16x8(b), dq[rb][db]);
  };

  // One iteration j.  R = j mod 4 picks the ring slots; FIRST (j = 0) has no
  // previous tile.  Products in issue order: S^T of tile j (P^T of tile j is
  // formed under the dP^T products), dP^T of tile j, then -- after the
  // causal mask, where the tile needs one -- dQ^T of tile j-1 from ds_prev,
  // under which dS^T of tile j is formed into ds_cur.
  auto iter = [&](auto Rc, auto FIRSTc, int j, const unsigned (&ds_prev)[T::RB][T::NKB][8],
                  unsigned (&ds_cur)[T::RB][T::NKB][8]) __attribute__((always_inline)) {
    constexpr int R = decltype(Rc)::value;
    constexpr bool FIRST = decltype(FIRSTc)::value;
    constexpr int N1 = T::NS + T::NP;                // products of phase 1
    constexpr int NALL = N1 + (FIRST ? 0 : T::NQ);
    const char* kb_ = kslot(IC<R>{});
    const char* vb_ = vslot(IC<R>{});
    const char* kp_ = kslot(IC<(R + 3) % 4>{});  // previous tile's K

    fetch(j + 2, IC<(R + 2) % 4>{});

    f32x16 s[T::RB][T::NKB], dpv[T::RB][T::NKB];
    float pv[T::RB][T::NKB][16];
    u32x4 afr[NALL], bfr[T::NP];
    // One K / V / K^T fragment feeds both row blocks; dP^T also takes its
    // dO fragment from registers.
    auto read_frag = [&](auto Ic) __attribute__((always_inline)) {
      constexpr int i = decltype(Ic)::value;
      if constexpr (i >= T::NS && i < N1) {
        constexpr int x = i - T::NS, f = x / T::RB;
        bfr[x] = gf[x % T::RB][f / T::NKB];
      }
      if constexpr (i % T::RB == 0) {
        if constexpr (i < T::NS) afr[i] = fread(kb_, i / T::RB);
        else if constexpr (i < N1) afr[i] = fread(vb_, (i - T::NS) / T::RB);
        else afr[i] = tread(kp_, (i - N1) / T::RB);
      }
    };
    auto product = [&](auto Ic) __attribute__((always_inline)) {
      constexpr int i = decltype(Ic)::value, rb = i % T::RB, i0 = i - rb;
      f32x16 z;
#pragma unroll
      for (int r = 0; r < 16; ++r) z[r] = 0.f;
      if constexpr (i < T::NS) {
        constexpr int f = i / T::RB, kb = f % T::NKB, ks = f / T::NKB;
        s[rb][kb] = mma(as_bf16x8(afr[i0]), qf[rb][ks], ks == 0 ? z : s[rb][kb]);
      } else if constexpr (i < N1) {
        constexpr int f = (i - T::NS) / T::RB, kb = f % T::NKB, ks = f / T::NKB;
        dpv[rb][kb] = mma(as_bf16x8(afr[i0]), as_bf16x8(bfr[i - T::NS]), ks == 0 ? ndv[rb] : dpv[rb][kb]);
      } else {
        dq_product(afr[i0], ds_prev, IC<(i - N1) / T::RB>{}, IC<rb>{});
      }
    };
    // P^T group e (4 elements): FMA with lse, exp2.
    auto p_group = [&](auto Ec) __attribute__((always_inline)) {
      constexpr int e = decltype(Ec)::value, rb = e % T::RB, x = e / T::RB, kb = x / 4, g = x % 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[rb][kb][4 * g + i] = fast_exp2(__builtin_fmaf(s[rb][kb][4 * g + i], c, -lse2[rb]));
        pin(pv[rb][kb][4 * g + i]);
      }
    };
    // dS^T group e: P (dP - D), packed into ds_cur.
    auto ds_group = [&](auto Ec) __attribute__((always_inline)) {
      constexpr int e = decltype(Ec)::value, rb = e % T::RB, x = e / T::RB, kb = x / 4, g = x % 4;
      float d4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) d4[i] = pv[rb][kb][4 * g + i] * dpv[rb][kb][4 * g + i];
      ds_cur[rb][kb][2 * g] = pack_bf16x2(d4[0], d4[1]);
      ds_cur[rb][kb][2 * g + 1] = pack_bf16x2(d4[2], d4[3]);
      pin(ds_cur[rb][kb][2 * g]);
      pin(ds_cur[rb][kb][2 * g + 1]);
    };
    auto slot = [&](auto SLc) __attribute__((always_inline)) {
      constexpr int sl = decltype(SLc)::value;
      if constexpr (sl + 2 < NALL) read_frag(IC<sl + 2>{});
      static_for<0, T::NDS>([&](auto Ec) __attribute__((always_inline)) {
        constexpr int e = decltype(Ec)::value;
        if constexpr (spread(e, T::NDS, T::NS, T::NP) == sl) p_group(Ec);
        if constexpr (!FIRST && spread(e, T::NDS, N1, T::NQ) == sl) ds_group(Ec);
      });
    };
    auto run = [&](auto Ic) __attribute__((always_inline)) {
      constexpr int i = decltype(Ic)::value;
      // Issue priority falls 3, 2, 1, 0 over the quarters of the
      // iteration's products, so the wave of a SIMD pair that runs ahead
      // yields contested matrix-core slots to the one behind (as in the
      // forward).
      if constexpr (!(MODE == 1 && CAUSAL) && (4 * i) % NALL == 0)
        __builtin_amdgcn_s_setprio(3 - (4 * i) / NALL);
      product(Ic);
      slot(Ic);
      __builtin_amdgcn_sched_barrier(0);
    };

    read_frag(IC<0>{});
    read_frag(IC<1>{});
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, N1>(run);

    // Causal: zero P^T where the key is past the row (key > query);
    // block-sparse: the whole tile when this wave's row block does not see it.
    const int key0 = tile_at(j) * T::BC;
    const bool sees = own_sees(j);
    if ((CAUSAL && key0 + T::BC - 1 > qw0) || !sees) {
      static_for<0, T::RB>([&](auto RBc) __attribute__((always_inline)) {
        constexpr int rb = decltype(RBc)::value;
        const int lim = sees ? qw0 + 32 * rb + n - key0 - 4 * h : -(1 << 30);
        static_for<0, 16 * T::NKB>([&](auto Ec) __attribute__((always_inline)) {
          constexpr int e = decltype(Ec)::value, kb = e >> 4, r = e & 15;
          constexpr int off = kb * 32 + 8 * (r >> 2) + (r & 3);
          const unsigned hide = (unsigned)((lim - off) >> 31);
          const float pe = pv[rb][kb][r];
          pv[rb][kb][r] = __builtin_bit_cast(float, __builtin_bit_cast(unsigned, pe) & ~hide);
        });
      });
    }
    __builtin_amdgcn_sched_barrier(0);

    if constexpr (FIRST) {
      static_for<0, T::NDS>([&](auto Ec) __attribute__((always_inline)) { ds_group(Ec); });
    } else {
      static_for<N1, NALL>(run);
    }

    wait_vm<2 * T::LOADS>();  // tile j+1 landed; tile j+2 may still be in flight
    block_barrier();
  };

  // A block-sparse workgroup whose rows see no key writes dQ = 0.
  if (!SPARSE || nkt > 0) {
  // ---- prologue: tile 0 landed, tile 1 in flight ---------------------------------
  fetch(0, IC<0>{});
  __builtin_amdgcn_sched_barrier(0);  // tile 0's loads are issued first
  fetch(1, IC<1>{});
  wait_vm<2 * T::LOADS>();
  block_barrier();

  // dS^T of even tiles goes to dskA, of odd tiles to dskB.
  iter(IC<0>{}, std::true_type{}, 0, dskB, dskA);
  // Whole rounds of four with no exit inside (an exit between bodies makes
  // the register allocator move the accumulators around every round), then
  // up to three more.
  int j = 1;
  for (; j + 3 < nkt_w; j += 4) {
    window_for(j + 5);  // this round fetches up to tile j + 5
    iter(IC<1>{}, std::false_type{}, j, dskA, dskB);
    iter(IC<2>{}, std::false_type{}, j + 1, dskB, dskA);
    iter(IC<3>{}, std::false_type{}, j + 2, dskA, dskB);
    iter(IC<0>{}, std::false_type{}, j + 3, dskB, dskA);
  }
  window_for(j + 4);
  if (j < nkt_w) {
    iter(IC<1>{}, std::false_type{}, j, dskA, dskB);
    if (j + 1 < nkt_w) {
      iter(IC<2>{}, std::false_type{}, j + 1, dskB, dskA);
      if (j + 2 < nkt_w) iter(IC<3>{}, std::false_type{}, j + 2, dskA, dskB);
    }
  }

  // ---- dQ^T of the wave's last tile ------------------------------------------------
  // K[nkt_w-1] was read by this wave's own last iteration; its slot is
  // refilled only in iteration nkt_w+1, after the next barrier.
  if (nkt_w == nkt) wait_vm<0>();
  auto last_dq = [&](const char* kb_, const unsigned (&ds)[T::RB][T::NKB][8])
                     __attribute__((always_inline)) {
    static_for<0, T::NT>([&](auto Fc) __attribute__((always_inline)) {
      const u32x4 a = tread(kb_, decltype(Fc)::value);
      static_for<0, T::RB>([&](auto RBc) __attribute__((always_inline)) { dq_product(a, ds, Fc, RBc); });
    });
  };
  switch ((nkt_w - 1) & 3) {
    case 0: last_dq(K0, dskA); break;
    case 1: last_dq(K1, dskB); break;
    case 2: last_dq(K2, dskA); break;
    default: last_dq(K3, dskB); break;
  }
  // Iterations nkt_w..nkt-1 without products: the same loads into the same
  // slots, the same waits and barriers as the waves that still compute.
  for (int jd = nkt_w; jd < nkt; ++jd) {
    const int t = tile_at(min(jd + 2, nkt - 1));
    const int sl = (jd + 2) & 3;
    char* kd = sl == 0 ? K0 : sl == 1 ? K1 : sl == 2 ? K2 : K3;
    char* vd = sl == 0 ? V0 : sl == 1 ? V1 : sl == 2 ? V2 : V3;
    static_for<0, T::LOADS>([&](auto Ic) __attribute__((always_inline)) {
      constexpr int i = decltype(Ic)::value;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, (lds_void*)(kd + w * T::LOADS * 1024), 16,
          (uint32_t)(t * T::TILEB + fetch_off[i] - i * 1024), 0, i * 1024, 0);
    });
    static_for<0, T::LOADS>([&](auto Ic) __attribute__((always_inline)) {
      constexpr int i = decltype(Ic)::value;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, (lds_void*)(vd + w * T::LOADS * 1024), 16,
          (uint32_t)(t * T::TILEB + fetch_off[i] - i * 1024), 0, i * 1024, 0);
    });
    wait_vm<2 * T::LOADS>();
    block_barrier();
  }
  }  // !SPARSE || nkt > 0
  wait_vm<0>();  // the loads of the tiles past the last one
  // Waves that computed to the last tile read its K slot after the final
  // barrier; the ring is reused below.
  block_barrier();

  // ---- dQ = scale * accumulator, staged for whole-row stores ----------------------
  // Wave w's 32 rows go through ring slot K_w (waves 0-3) or V_(w-4).
  static_assert(T::RB == 1 && 32 * 2 * D <= T::TILEB, "one wave's rows per ring slot");
  u32x2 pq[T::DB][4];
#pragma unroll
  for (int db = 0; db < T::DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      pq[db][g].x = pack_bf16x2(scale * dq[0][db][4 * g + 0], scale * dq[0][db][4 * g + 1]);
      pq[db][g].y = pack_bf16x2(scale * dq[0][db][4 * g + 2], scale * dq[0][db][4 * g + 3]);
    }
  char* const st = w == 0 ? K0 : w == 1 ? K1 : w == 2 ? K2 : w == 3 ? K3
                 : w == 4 ? V0 : w == 5 ? V1 : w == 6 ? V2 : V3;
  store_rows_staged<D>(st, lane, pq, make_rsrc(dQ + qoff, (uint32_t)Lq * D * 2), qw0);
}

// Whether the dQ kernel takes over the prepare kernel's work (a call that
// runs both stages, with bf16 O): it then runs first and writes the
// statistics that the dK/dV kernel, if requested, reads after it.
inline bool fused_prepare(const BwdArgs& a, unsigned stages) {
  constexpr unsigned both = kBwdPrepare | kBwdDq;
  return (stages & both) == both && !a.o_f32 && a.BH > 0 && a.Lq > 0 && a.Lk > 0;
}

template <int D, bool CAUSAL, int QMODE>
void launch_main(const BwdArgs& a, unsigned stages, hipStream_t stream) {
  constexpr bool SPARSE = QMODE == 2;
  using TK = KvTile<D>;
  using TQ = DqTile<D, QMODE != 0>;
  const float c = a.scale * kLog2e;
  const uint16_t* Q = static_cast<const uint16_t*>(a.Q);
  const uint16_t* K = static_cast<const uint16_t*>(a.K);
  const uint16_t* V = static_cast<const uint16_t*>(a.V);
  const uint16_t* dO = static_cast<const uint16_t*>(a.dO);
  const uint16_t* O = static_cast<const uint16_t*>(a.O);
  const int n_kt = (a.Lk + TK::BK - 1) / TK::BK;
  const int n_qt = (a.Lq + TQ::BR - 1) / TQ::BR;
  const bool fused = fused_prepare(a, stages);
  auto dq = [&](auto PREPc) {
    constexpr bool PREP = decltype(PREPc)::value;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, QMODE, PREP>), dim3((unsigned)(n_qt * a.BH)),
                       dim3(64 * TQ::NW), 0, stream, Q, K, V, dO, O, a.lse, a.lse2, a.Dvec,
                       static_cast<uint16_t*>(a.dQ), a.BH, a.Lq, a.Lk, n_qt, c, a.scale,
                       a.block_mask, a.bm_stride, a.nqb, a.nkb);
  };
  if (fused) dq(std::true_type{});
  if ((stages & kBwdDkDv) && n_kt > 0)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, SPARSE>), dim3((unsigned)(n_kt * a.BH)),
                       dim3(64 * TK::NW), 0, stream, Q, K, V, dO, a.lse2, a.Dvec,
                       static_cast<uint16_t*>(a.dK), static_cast<uint16_t*>(a.dV), a.BH, a.Lq, a.Lk,
                       c, a.scale, a.block_mask, a.bm_stride, a.nqb, a.nkb);
  if (!fused && (stages & kBwdDq) && n_qt > 0 && a.Lk > 0) dq(std::false_type{});
}

template <int D>
hipError_t launch_d(const BwdArgs& a, unsigned stages, hipStream_t stream) {
  const int64_t rows = (int64_t)a.BH * a.Lq;
  if ((stages & kBwdPrepare) && rows > 0 && !fused_prepare(a, stages)) {
    // The NT variant once bf16 O and dO together reach 64 MiB (with fp32 O
    // it measured no faster).
    const bool nt = !a.o_f32 && rows * D * 4 >= (int64_t(64) << 20);
    const auto* G = static_cast<const uint16_t*>(a.dO);
    auto grid = [&](int rpb) { return dim3((unsigned)((rows + rpb - 1) / rpb)); };
    if (a.o_f32)
      hipLaunchKernelGGL((bwd_pre_bf16_kernel<D, true, false>), grid(pre_rows_per_block<D, false>()),
                         dim3(256), 0, stream, a.O, G, a.lse, a.Dvec, a.lse2, rows);
    else if (nt)
      hipLaunchKernelGGL((bwd_pre_bf16_kernel<D, false, true>), grid(pre_rows_per_block<D, true>()),
                         dim3(256), 0, stream, a.O, G, a.lse, a.Dvec, a.lse2, rows);
    else
      hipLaunchKernelGGL((bwd_pre_bf16_kernel<D, false, false>), grid(pre_rows_per_block<D, false>()),
                         dim3(256), 0, stream, a.O, G, a.lse, a.Dvec, a.lse2, rows);
  }
  // dQ: 256-row workgroups unless that gives fewer than two per compute
  // unit; then 128-row ones (as the forward).
  const int64_t wgs256 = (int64_t)((a.Lq + 255) / 256) * a.BH;
  if (a.block_mask) {
    if (a.causal) launch_main<D, true, 2>(a, stages, stream);
    else launch_main<D, false, 2>(a, stages, stream);
  } else if (wgs256 < 2 * kComputeUnits) {
    if (a.causal) launch_main<D, true, 1>(a, stages, stream);
    else launch_main<D, false, 1>(a, stages, stream);
  } else {
    if (a.causal) launch_main<D, true, 0>(a, stages, stream);
    else launch_main<D, false, 0>(a, stages, stream);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, unsigned stages, hipStream_t stream) {
  static_assert(KvTile<128>::BK == kBwdBf16KeysPerBlock, "tile table out of sync");
  if (a.d == 64) return launch_d<64>(a, stages, stream);
  return launch_d<128>(a, stages, stream);
}

}  // namespace fa
