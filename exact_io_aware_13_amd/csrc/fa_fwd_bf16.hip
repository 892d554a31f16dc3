// Exact attention forward, bf16 inputs, fp32 accumulation, gfx950.
//
// One workgroup = 256 query rows of one (batch, head) slice, 8 waves of one
// 32-row block each (two waves per SIMD); launches that would give fewer
// than two such workgroups per compute unit use 128-row workgroups of 4
// waves instead (two per compute unit).  The Q rows stay in registers for
// the whole key loop; K and V stream through LDS in tiles of 32 (d=128) or
// 64 (d=64) keys, and an online softmax keeps a running max m, a running
// sum l and an unnormalised output per row, rescaling both by
// exp(m_old - m_new) when the max moves
// ("How Flash Attention Improves Transformer Memory Efficiency ...",
// sections "Block-Wise Processing Algorithm" and "The Three Running
// Statistics"; "What Is FlashAttention?", section "What FlashAttention does
// instead").  Scores and probabilities live only in registers.
//
// Matrix-core orientation.  Each wave computes S^T = K Q^T for its rows, so
// in the 32x32 accumulator every lane owns ONE query row (column n = lane %
// 32) and 16 of a 32-key block; the other 16 keys of that row sit in lane ^
// 32.  Row max and row sum are in-lane plus one exchange between the two
// wave halves.  The same registers are the B operand of O^T = V^T P^T: the
// contraction over keys is taken in the order the accumulator holds them,
// and the A operand V^T comes from the row-major V tile through the
// transposing LDS read (ds_read_b64_tr_b16: in each 16-lane group, lanes
// 4j..4j+3 fetch four consecutive values of row j and lane u receives
// element u of rows 0..3, i.e. four consecutive keys of one head-dim column).
// O^T's accumulator again gives each lane one query row, so the rescale is a
// per-lane scalar multiply.  Every K or V fragment read from LDS feeds the
// products of all the wave's row blocks.
//
// Data movement.  K and V tiles go from HBM/L2 straight into LDS with
// bounds-checked buffer loads (rows past the end of the slice read as zero),
// no VGPR staging.  Each 16-byte chunk c of row r is stored at chunk
// c ^ swz(r), so both the K reads (16 rows, one chunk each) and the
// transposed V reads (4 rows x 32 bytes per 16 lanes) hit distinct banks.
// K and V each use a 4-slot ring (one LDS array per slot, so the compiler
// waits only for the load a read depends on); tile t's K and V are fetched
// three iterations before the products that need them, from inside the
// product sequence, and each iteration ends with one wait and one barrier.
//
// Software pipeline.  Iteration j runs the score product of tile j+1 and the
// value product of tile j-1 on the matrix cores while the vector ALUs run
// the softmax of tile j.  The iteration body is scheduled by hand: 16 steps
// of 4 matrix products, each LDS fragment read issued two steps ahead, the
// softmax work items placed between the products.
//
// Softmax arithmetic runs in base 2: p = exp2(s * c - m) with c =
// |scale| * log2(e) folded into one FMA (a negative scale is applied by
// negating Q, which is exact in bf16).  Any reference m gives the same
// O = acc / l and lse = m + log2 l exactly, so m is not a running max: a
// tile's probabilities are formed against the current m, and only when a
// lane's sum of them exceeds 2^12 (or m is still the initial -3e38, which
// makes them infinite) does a uniform branch take the row max of the tile
// (raw dot products, one cross-half exchange), move m to it, rescale l and
// the output accumulator and form the tile's probabilities again.  In
// practice that happens on a row's first tile and rarely after, which
// takes the per-tile max reduction out of the vector work; probabilities
// stay <= 2^12, far from overflow.  l sums the fp32 probabilities; the
// value product takes them rounded to bf16.
// Tiles that are fully masked for some rows (causal diagonal band) are still
// multiplied; their probabilities are exactly 0.
//
// Block-sparse instantiation (SPARSE).  A mask over 128x128 (query, key)
// blocks removes whole blocks from the attention pattern, a generalisation
// of the causal tile skip (the glossary page, FAQ on block-sparse
// extensions, sets such patterns apart from the dense core).  A workgroup
// then holds 128 rows (half the waves), exactly one row block of the mask:
// it first compacts the key blocks its row block sees into an LDS list
// (ballot + prefix count per wave) and then runs the same pipeline over the
// listed key tiles only.  A workgroup whose list is empty writes O = 0 and
// lse = -inf; the softmax also tolerates a row that has seen no key yet (the
// running max is then -inf and the reference is taken as 0, so every
// probability is exactly 0).

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {
namespace {

// Softmax reference before a row has seen a key: finite (so a masked score,
// -inf, still gives exp2(-inf - m) = 0 and never -inf - -inf), and far
// below any score, so the first visible key makes the tile's sum infinite
// and moves the reference.
constexpr float kInitialRef = -3.0e38f;
// A lane's probability sum over one tile above which the reference moves.
constexpr float kRescaleSum = 4096.f;

template <int D, bool HALF>
struct FwdTile {
  // 256 rows: 8 waves of one 32-row block, two waves per SIMD (each fits
  // in 256 registers), so one wave's softmax runs while the other's matrix
  // products do.  HALF: 128 rows, 4 waves, two workgroups per compute unit
  // -- for launches that would otherwise give fewer than two workgroups per
  // compute unit, and for the block-sparse forward (one mask row block per
  // workgroup).
  static constexpr int NW = HALF ? 4 : 8;  // waves per workgroup
  static constexpr int RB = 1;             // 32-row blocks per wave
  static constexpr int BR = 32 * RB * NW;         // query rows per workgroup
  // Keys per tile: at d=128 a 32-key tile keeps the softmax working set
  // (two score sets, two probability sets) inside the 256 VGPRs the vector
  // ALUs address; d=64 has room for 64.
  static constexpr int BC = D == 128 ? 32 : 64;
  static constexpr int NKB = BC / 32;             // 32-key blocks per tile
  static constexpr int KS = D / 16;               // 16-deep steps over the head dimension
  static constexpr int DB = D / 32;               // 32-wide head-dim blocks
  static constexpr int ROWB = D * 2;              // bytes per K/V row
  static constexpr int CPR = D / 8;               // 16-byte chunks per row
  static constexpr int TILEB = BC * ROWB;         // bytes per K (or V) tile
  static constexpr int RPK = 1024 / ROWB;         // rows per 1-KiB load instruction
  static constexpr int LOADS = TILEB / 1024 / NW; // load instructions per wave per tile
  static_assert(LOADS <= 4, "immediate load offsets reach 3 KiB");
  static constexpr int NFRAG = NKB * KS;          // K fragments per tile (= V fragments)
  static_assert(NFRAG == (BC / 16) * DB, "one K and one V fragment per step");
  // Softmax slot program (all row blocks): 4-probability groups in three
  // stages, then the tile's probability sums.
  static constexpr int NGROUP = RB * 4 * NKB;     // 4-probability groups per iteration
  static constexpr int SL_GROUPS = 0;
  static constexpr int SL_SUMS = SL_GROUPS + 3 * NGROUP;
  static constexpr int NPROG = SL_SUMS + RB;      // program slots
  static constexpr int NPHYS = 2 * RB * NFRAG;    // matrix-product slots per iteration
  // Program slots run after physical slot p: [prog_begin(p), prog_begin(p+1)),
  // an even spread of the program over the products.
  static constexpr int prog_begin(int p) { return (p * NPROG + NPHYS - 1) / NPHYS; }
};

// MODE: 0 dense, 256 rows per workgroup; 1 dense, 128 rows; 2 block-sparse,
// 128 rows.
template <int D, bool CAUSAL, bool OUT_F32, int MODE>
__global__ __launch_bounds__((64 * FwdTile<D, MODE != 0>::NW * (MODE == 3 ? 2 : 1)),
                             ((MODE == 1 || MODE == 2) ? 2 : 1)) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, void* __restrict__ O, float* __restrict__ LSE,
    int BH, int Lq, int Lk, int n_qt, float c, unsigned qsign,
    const uint8_t* __restrict__ BM, int bm_stride, int nqb, int nkb) {
  using T = FwdTile<D, MODE != 0>;
  constexpr bool SPARSE = MODE == 2;
  // MODE 3: 128 query rows and two groups of four waves; group g takes the
  // g-th half of the workgroup's key tiles for the same rows (its own half of
  // every ring slot), and the halves' (reference, sum, accumulator) are
  // merged in LDS at the end.  This halves the longest chain of key tiles,
  // which bounds short causal launches.
  constexpr bool SPLIT = MODE == 3;
  constexpr int NG = SPLIT ? 2 : 1;
  // Quarter priorities within each iteration (see the product loop): for
  // 256-row workgroups, and for 128-row ones without the causal mask, where
  // they measured faster; causal 128-row launches measured slower.
  constexpr bool PRIO = MODE == 0 || MODE == 3 || (MODE == 1 && !CAUSAL);
  __shared__ __attribute__((aligned(1024))) char K0[T::TILEB * NG];
  __shared__ __attribute__((aligned(1024))) char K1[T::TILEB * NG];
  __shared__ __attribute__((aligned(1024))) char K2[T::TILEB * NG];
  __shared__ __attribute__((aligned(1024))) char K3[T::TILEB * NG];
  __shared__ __attribute__((aligned(1024))) char V0[T::TILEB * NG];
  __shared__ __attribute__((aligned(1024))) char V1[T::TILEB * NG];
  __shared__ __attribute__((aligned(1024))) char V2[T::TILEB * NG];
  __shared__ __attribute__((aligned(1024))) char V3[T::TILEB * NG];
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
  // The wave index is the same on every lane; readfirstlane tells the
  // compiler so, which keeps everything derived from it in scalar registers.
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, n = lane & 31, h = lane >> 5;
  // Key-half group and the wave's index within it (its row block).
  const int grp = SPLIT ? w / T::NW : 0;
  const int wr = SPLIT ? w % T::NW : w;
  const int gofs = grp * T::TILEB;  // the group's half of every ring slot

  // Consecutive workgroups take the same query tile of different slices; for
  // causal masks the tiles with the most visible keys are dispatched first.
  const int bh = wg_id() % BH;
  int qt = wg_id() / BH;
  if (CAUSAL) {
    // When every workgroup of a 128-row causal launch is resident at once
    // (two per compute unit), workgroups g and g + grid/2 share a compute
    // unit: the second half runs lightest-first so that each pair holds
    // about the same number of key tiles.  Otherwise heaviest first.
    if (MODE == 1 && (n_qt & 1) == 0 && n_qt * BH <= 2 * kComputeUnits && qt >= n_qt / 2)
      qt -= n_qt / 2;
    else
      qt = n_qt - 1 - qt;
  }
  const int q0 = qt * T::BR;
  const int qw0 = q0 + 32 * T::RB * wr;  // this wave's first row

  const size_t qoff = (size_t)bh * Lq * D;
  const size_t koff = (size_t)bh * Lk * D;
  const auto rq = make_rsrc(Q + qoff, (uint32_t)Lq * D * 2);
  const auto rk = make_rsrc(K + koff, (uint32_t)Lk * D * 2);
  const auto rv = make_rsrc(V + koff, (uint32_t)Lk * D * 2);

  int nkt = (Lk + T::BC - 1) / T::BC;
  if (CAUSAL) nkt = min(nkt, (q0 + T::BR - 1) / T::BC + 1);

  // ---- block-sparse: compacted list of the key blocks this workgroup sees --
  // The workgroup's 128 rows are one row block of the mask; its nonzero
  // entries (up to the causal limit) are compacted in order into LDS, then
  // held 128 at a time in two registers (entry e of the window in lane e % 64
  // of win0 or win1) and read with v_readlane, so the loop never waits on
  // LDS for a tile index.
  constexpr int TPB = kSparseBlock / T::BC;  // key tiles per mask block
  __shared__ uint16_t tlist[SPARSE ? kSparseMaxKeyBlocks : 1];
  __shared__ int wtot[SPARSE ? T::NW : 1];
  int nlist = 0, wbase = 0;
  unsigned win0 = 0, win1 = 0;
  if constexpr (SPARSE) {
    static_assert(T::BR == kSparseBlock, "one mask row block per workgroup");
    const int qb = q0 / kSparseBlock;
    const uint8_t* row = BM + (size_t)bh * bm_stride + (size_t)qb * nkb;
    const int kb_lim = CAUSAL ? min(nkb, qb + 1) : nkb;
    for (int base = 0; base < kb_lim; base += 64 * T::NW) {
      const int kb = base + tid;
      const bool keep = kb < kb_lim && row[kb] != 0;
      const uint64_t bal = __ballot(keep);
      const int below = __popcll(bal & ((uint64_t(1) << lane) - 1));
      if (lane == 0) wtot[w] = __popcll(bal);
      __syncthreads();
      int off = nlist, tot = 0;
      for (int ww = 0; ww < T::NW; ++ww) {
        if (ww < w) off += wtot[ww];
        tot += wtot[ww];
      }
      if (keep) tlist[off + below] = (uint16_t)kb;
      nlist += tot;
      __syncthreads();
    }
    nkt = nlist * TPB;
    win0 = lane < nlist ? tlist[lane] : 0u;
    win1 = 64 + lane < nlist ? tlist[64 + lane] : 0u;
  }
  // This wave's own trip count (after the block-sparse list has set nkt):
  // under a causal mask its rows see no key past tile (qw0 + 32 RB - 1) /
  // BC, and a wave whose rows all lie past Lq has nothing to compute (its
  // stores are dropped).  Tiles past it are not multiplied; the wave still
  // issues its share of every tile's loads and joins every barrier (see the
  // drain after the main loop).  The block-sparse workgroup runs its list
  // with every wave.
  // SPLIT: the group's tiles are tbase .. tbase + nreal - 1, and every wave
  // of the workgroup iterates over the larger half's count (the same
  // barriers).  A wave whose rows see no key of its half computes one fully
  // masked tile (probabilities exactly 0); a half with no tile at all is
  // left out of the merge.
  const int nkt_all = nkt;
  int tbase = 0, nreal = nkt;
  if constexpr (SPLIT) {
    const int half = (nkt + 1) / 2;
    tbase = grp ? half : 0;
    nreal = grp ? nkt - half : half;
    nkt = half;
  }
  int nkt_w = nkt;
  if constexpr (!SPARSE) {
    if (CAUSAL) nkt_w = min(nkt, (qw0 + 32 * T::RB - 1) / T::BC + 1 - tbase);
    if constexpr (SPLIT) nkt_w = min(nkt_w, nreal);
    if (qw0 >= Lq || nkt_w < 1) nkt_w = 1;
  }
  // Key tile of loop position j (the window must hold entry j / TPB).
  auto tile_at = [&](int j) __attribute__((always_inline)) -> int {
    if constexpr (SPARSE) {
      // Pick the window register per lane first (one select, no branch),
      // then read the entry's lane.
      const int e = j / TPB - wbase;
      const unsigned src = e < 64 ? win0 : win1;
      const int kb = __builtin_amdgcn_readlane((int)src, e & 63);
      return kb * TPB + j % TPB;
    } else if constexpr (SPLIT) {
      return tbase + min(j, nreal - 1);
    } else {
      return j;
    }
  };
  // Slide the window by 64 entries when position jmax would leave it.
  auto window_for = [&](int jmax) __attribute__((always_inline)) {
    if constexpr (SPARSE) {
      if (jmax / TPB - wbase >= 128) {
        wbase += 64;
        win0 = win1;
        const int e = wbase + 64 + lane;
        win1 = e < nlist ? tlist[e] : 0u;
      }
    }
  };

  // ---- tile fetch: each wave moves LOADS KiB of the K (or V) tile ----------
  // Lane l of load i writes LDS bytes [16 l, 16 l + 16) of KiB (w*LOADS + i)
  // of the slot; it fetches the logical chunk that the swizzle puts there.
  int fetch_off[T::LOADS];
#pragma unroll
  for (int i = 0; i < T::LOADS; ++i) {
    const int row = (wr * T::LOADS + i) * T::RPK + lane / T::CPR;
    const int chunk = (lane % T::CPR) ^ swz<D>(row);
    fetch_off[i] = (row * D + chunk * 8) * 2;
  }
  auto fetch = [&](const __amdgpu_buffer_rsrc_t& r, int tile, char* slot)
                   __attribute__((always_inline)) {
    // Tiles past the last one re-fetch the last tile into a free slot, which
    // keeps the number of loads in flight the same every iteration.
    // Load i lands 1 KiB after load i-1 in LDS and in memory (up to the
    // swizzled chunk, carried by the per-lane offset): one LDS base for the
    // wave's loads, the rest in the immediate offset.
    const int t = tile_at(min(tile, nkt - 1));
    lds_void* dst = (lds_void*)(slot + gofs + wr * T::LOADS * 1024);
    static_for<0, T::LOADS>([&](auto Ic) __attribute__((always_inline)) {
      constexpr int i = decltype(Ic)::value;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, dst, 16, (uint32_t)(t * T::TILEB + fetch_off[i] - i * 1024), 0, i * 1024, 0);
    });
  };

  // ---- per-lane LDS read offsets (slot-relative) -----------------------------
  // K fragment f (key block f%NKB, step f/NKB): row (f%NKB)*32 + n, chunk
  // 2(f/NKB) + h.
  const int ksw = swz<D>(n);
  int koffs[T::KS];
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks) koffs[ks] = n * T::ROWB + (((2 * ks + h) ^ ksw) << 4);
  // V^T fragment f (key step f/DB, head-dim block f%DB): two transposed reads
  // of rows 16*step + 4h + j (+8), columns 32db + 16(g%2) + 4t .. +3.
  const int g = lane >> 4, u = lane & 15, j4 = u >> 2, t4 = u & 3;
  int voffs[2][T::DB];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int row = 8 * half + 4 * h + j4;
    const int sw = swz<D>(row);
#pragma unroll
    for (int db = 0; db < T::DB; ++db) {
      const int chunk = 4 * db + 2 * (g & 1) + (t4 >> 1);
      voffs[half][db] = row * T::ROWB + ((chunk ^ sw) << 4) + 8 * (t4 & 1);
    }
  }
  auto kread = [&](const char* kb, int f) __attribute__((always_inline)) {
    return lds_read16(kb, (f % T::NKB) * 32 * T::ROWB + koffs[f / T::NKB]);
  };
  auto vread = [&](const char* vb, int f) __attribute__((always_inline)) {
    const int step = f / T::DB, db = f % T::DB;
    const u32x2 lo = lds_read_tr(vb, step * 16 * T::ROWB + voffs[0][db]);
    const u32x2 hi = lds_read_tr(vb, step * 16 * T::ROWB + voffs[1][db]);
    u32x4 a;
    a.x = lo.x;
    a.y = lo.y;
    a.z = hi.x;
    a.w = hi.y;
    return a;
  };

  // ---- Q fragments (B operands of S^T = K Q^T), one set per row block ------
  bf16x8 qf[T::RB][T::KS];
#pragma unroll
  for (int rb = 0; rb < T::RB; ++rb)
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      u32x4 v = load16(rq, (uint32_t)((qw0 + 32 * rb + n) * D + ks * 16 + h * 8) * 2);
      v ^= qsign;  // negative scale: negate Q (sign flip of every bf16)
      qf[rb][ks] = as_bf16x8(v);
    }

  f32x16 oacc[T::RB][T::DB];
#pragma unroll
  for (int rb = 0; rb < T::RB; ++rb)
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[rb][db][r] = 0.f;
  float m[T::RB], l[T::RB];
#pragma unroll
  for (int rb = 0; rb < T::RB; ++rb) {
    m[rb] = kInitialRef;
    l[rb] = 0.f;
  }

  // Pipeline registers: raw scores of the current and next tile, packed bf16
  // probabilities of the previous and current tile.  Defined up front: the
  // first and last iterations leave some of them unwritten.
  f32x16 sA[T::RB][T::NKB], sB[T::RB][T::NKB];
  unsigned pA[T::RB][T::NKB][8], pB[T::RB][T::NKB][8];
#pragma unroll
  for (int rb = 0; rb < T::RB; ++rb)
#pragma unroll
    for (int kb = 0; kb < T::NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sA[rb][kb][r] = 0.f;
        sB[rb][kb][r] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pA[rb][kb][i] = 0u;
        pB[rb][kb][i] = 0u;
      }
    }

  // Whole-tile score product (prologue only; iterations interleave it).
  auto score_tile = [&](const char* kb, f32x16 (&s)[T::RB][T::NKB]) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < T::NFRAG; ++f) {
      const bf16x8 a = as_bf16x8(kread(kb, f));
#pragma unroll
      for (int rb = 0; rb < T::RB; ++rb) {
        if (f < T::NKB) {
          f32x16 z;
#pragma unroll
          for (int r = 0; r < 16; ++r) z[r] = 0.f;
          s[rb][f % T::NKB] = mma(a, qf[rb][f / T::NKB], z);
        } else {
          s[rb][f % T::NKB] = mma(a, qf[rb][f / T::NKB], s[rb][f % T::NKB]);
        }
      }
    }
  };
  // Whole-tile value product (epilogue only).
  auto value_tile = [&](const char* vb, const unsigned (&pk)[T::RB][T::NKB][8])
                        __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < T::NFRAG; ++f) {
      const bf16x8 a = as_bf16x8(vread(vb, f));
      const int step = f / T::DB, db = f % T::DB, kb = step >> 1, hf = step & 1;
#pragma unroll
      for (int rb = 0; rb < T::RB; ++rb) {
        u32x4 bp;
        bp.x = pk[rb][kb][hf * 4 + 0];
        bp.y = pk[rb][kb][hf * 4 + 1];
        bp.z = pk[rb][kb][hf * 4 + 2];
        bp.w = pk[rb][kb][hf * 4 + 3];
        oacc[rb][db] = mma(a, as_bf16x8(bp), oacc[rb][db]);
      }
    }
  };

  // One pipelined iteration j.  R = j mod 4 fixes the ring slots and which
  // register set is current; FIRST (j = 0) has no previous value product.
  auto iter = [&](auto Rc, auto FIRSTc, int j, f32x16 (&s_cur)[T::RB][T::NKB],
                  f32x16 (&s_next)[T::RB][T::NKB], const unsigned (&pk_prev)[T::RB][T::NKB][8],
                  unsigned (&pk_cur)[T::RB][T::NKB][8], u32x4 (&pre)[4]) __attribute__((always_inline)) {
    constexpr int R = decltype(Rc)::value;
    constexpr bool FIRST = decltype(FIRSTc)::value;
    const char* kb = kslot(IC<(R + 1) % 4>{}) + gofs;  // K[j+1]
    const char* vb = vslot(IC<(R + 3) % 4>{}) + gofs;  // V[j-1]

    // K[j+1] and V[j-1] were fetched three iterations ahead and waited for
    // at the end of iteration j-2.  This iteration refills the slots of K[j]
    // and V[j-2], whose last readers ran in iteration j-1 (closed by its
    // barrier), with K[j+4] and V[j+2], from inside the product sequence.

    // Mask tile j where it crosses the causal diagonal or the end of the keys.
    const int key0 = tile_at(j) * T::BC;
    if ((key0 + T::BC > Lk) || (CAUSAL && key0 + T::BC - 1 > qw0)) {
      // Register r of key block kb2 holds key key0 + 4h + (kb2*32 + 8(r/4) + r%4);
      // it is visible iff that constant offset is <= lim.  The sign of
      // (lim - offset) selects -inf without compares.
      static_for<0, T::RB>([&](auto RBc) __attribute__((always_inline)) {
        constexpr int rb = decltype(RBc)::value;
        const int qrow = qw0 + 32 * rb + n;
        const int last = CAUSAL ? min(Lk - 1, qrow) : Lk - 1;
        const int lim = last - key0 - 4 * h;
        static_for<0, 16 * T::NKB>([&](auto Ec) __attribute__((always_inline)) {
          constexpr int e = decltype(Ec)::value, kb2 = e >> 4, r = e & 15;
          constexpr int off = kb2 * 32 + 8 * (r >> 2) + (r & 3);
          const unsigned hide = (unsigned)((lim - off) >> 31);
          // Copy the element first: bit_cast of a vector-element lvalue reads
          // element 0 regardless of the index.
          const float sv = s_cur[rb][kb2][r];
          const unsigned bits = __builtin_bit_cast(unsigned, sv);
          s_cur[rb][kb2][r] = __builtin_bit_cast(float, (hide & 0xff800000u) | (~hide & bits));
        });
      });
    }

    float rs[T::RB][4], tsum[T::RB];
    float xg[T::NGROUP][4];  // probability groups in flight between stages
    // Vector-ALU work placed after the matrix-product slots: groups of 4
    // probabilities, each moving through three stages on consecutive slots
    // (FMA, exp2, pack and sum), so no instruction waits right behind its
    // producer; then the tile's sums.
    auto slot_work = [&](auto SLc) __attribute__((always_inline)) {
      constexpr int sl = decltype(SLc)::value;
      if constexpr (sl < T::SL_SUMS) {
        constexpr int t = sl - T::SL_GROUPS, g = t / 3, stage = t % 3;
        constexpr int rb = g % T::RB, eg = g / T::RB, kb2 = eg >> 2, r0 = (eg & 3) * 4;
        if constexpr (stage == 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xg[g][e] = __builtin_fmaf(s_cur[rb][kb2][r0 + e], c, -m[rb]);
            pin(xg[g][e]);
          }
        } else if constexpr (stage == 1) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xg[g][e] = fast_exp2(xg[g][e]);
            pin(xg[g][e]);
          }
        } else {
          pk_cur[rb][kb2][r0 / 2] = pack_bf16x2(xg[g][0], xg[g][1]);
          pk_cur[rb][kb2][r0 / 2 + 1] = pack_bf16x2(xg[g][2], xg[g][3]);
          // The first group of each partial sum assigns it (an fp add of 0
          // is not folded away and would cost an instruction).
          const float gs = (xg[g][0] + xg[g][1]) + (xg[g][2] + xg[g][3]);
          if constexpr (eg < 4) rs[rb][eg & 3] = gs;
          else rs[rb][eg & 3] += gs;
          pin(pk_cur[rb][kb2][r0 / 2]);
          pin(pk_cur[rb][kb2][r0 / 2 + 1]);
          pin(rs[rb][eg & 3]);
        }
      } else if constexpr (sl < T::SL_SUMS + T::RB) {
        constexpr int rb = sl - T::SL_SUMS;
        tsum[rb] = (rs[rb][0] + rs[rb][1]) + (rs[rb][2] + rs[rb][3]);
        pin(tsum[rb]);
      }
    };

    // All program slots mapped to physical slot P.
    auto run_slot = [&](auto Pc) __attribute__((always_inline)) {
      constexpr int p = decltype(Pc)::value;
      if constexpr (p == 1) fetch(rk, j + 4, kslot(IC<R>{}));
      if constexpr (p == 3) fetch(rv, j + 2, vslot(IC<(R + 2) % 4>{}));
      static_for<T::prog_begin(p), T::prog_begin(p + 1)>(
          [&](auto SLc) __attribute__((always_inline)) { slot_work(SLc); });
    };

    // NFRAG steps: score products of K fragment i (every row block), value
    // products of V fragment i (every row block), slot work after each.
    u32x4 ka[T::NFRAG], va[T::NFRAG];
    if constexpr (FIRST) {
      ka[0] = kread(kb, 0);
      ka[1] = kread(kb, 1);
    } else {
      // Read during iteration j-1 (see the end of the product sequence).
      ka[0] = pre[0];
      ka[1] = pre[1];
      va[0] = pre[2];
      va[1] = pre[3];
    }
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, T::NFRAG>([&](auto Ic) __attribute__((always_inline)) {
      constexpr int i = decltype(Ic)::value;
      // Issue priority falls 3, 2, 1, 0 over the four quarters of the
      // products.  The two waves of a SIMD run the same sequence; with equal
      // priorities the older one wins every contested matrix-core slot and
      // runs ahead while the younger one finishes the iteration alone.  A
      // wave that is a quarter ahead now yields to the one behind.
      if constexpr (PRIO && (8 * i) % (2 * T::NFRAG) == 0)
        __builtin_amdgcn_s_setprio(3 - (8 * i) / (2 * T::NFRAG));
      if constexpr (i + 2 < T::NFRAG) {
        ka[i + 2] = kread(kb, i + 2);
        if constexpr (!FIRST) va[i + 2] = vread(vb, i + 2);
      } else {
        // The next iteration's first K and V fragments: K[j+2] and V[j]
        // were waited for at the end of iteration j-1 and made visible by
        // its barrier, so they are read now and the next iteration starts
        // its products right after its barrier.
        constexpr int f = i + 2 - T::NFRAG;
        pre[f] = kread(kslot(IC<(R + 2) % 4>{}) + gofs, f);
        pre[2 + f] = vread(vslot(IC<R>{}) + gofs, f);
      }
      static_for<0, T::RB>([&](auto RBc) __attribute__((always_inline)) {
        constexpr int rb = decltype(RBc)::value;
        constexpr int kb2 = i % T::NKB, ks = i / T::NKB;
        if constexpr (i < T::NKB) {
          f32x16 z;
#pragma unroll
          for (int r = 0; r < 16; ++r) z[r] = 0.f;
          s_next[rb][kb2] = mma(as_bf16x8(ka[i]), qf[rb][ks], z);
        } else {
          s_next[rb][kb2] = mma(as_bf16x8(ka[i]), qf[rb][ks], s_next[rb][kb2]);
        }
        run_slot(IC<2 * T::RB * i + rb>{});
        __builtin_amdgcn_sched_barrier(0);
      });
      static_for<0, T::RB>([&](auto RBc) __attribute__((always_inline)) {
        constexpr int rb = decltype(RBc)::value;
        if constexpr (!FIRST) {
          constexpr int step = i / T::DB, db = i % T::DB, kb2 = step >> 1, hf = step & 1;
          u32x4 bp;
          bp.x = pk_prev[rb][kb2][hf * 4 + 0];
          bp.y = pk_prev[rb][kb2][hf * 4 + 1];
          bp.z = pk_prev[rb][kb2][hf * 4 + 2];
          bp.w = pk_prev[rb][kb2][hf * 4 + 3];
          oacc[rb][db] = mma(as_bf16x8(va[i]), as_bf16x8(bp), oacc[rb][db]);
        }
        run_slot(IC<2 * T::RB * i + T::RB + rb>{});
        __builtin_amdgcn_sched_barrier(0);
      });
    });
    // Tile j's probabilities grew past the bound on some lane (or a row's
    // reference is still the initial one): move the reference to the row
    // max, rescale l and the output accumulator (which holds tiles up to
    // j-1 at this point) and form tile j's probabilities again.  Every lane
    // of the wave takes the branch; for a row whose max does not exceed its
    // reference nothing changes (alpha = 1, the same probabilities).
    bool big = false;
#pragma unroll
    for (int rb = 0; rb < T::RB; ++rb) big |= tsum[rb] > kRescaleSum;
    if (__any(big)) {
#pragma unroll
      for (int rb = 0; rb < T::RB; ++rb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb2 = 0; kb2 < T::NKB; ++kb2)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s_cur[rb][kb2][r]);
        // A row that sees no key of the tile keeps its reference (mx * c =
        // -inf); the initial reference is finite, so no -inf - -inf arises.
        const float m_new = fmaxf(m[rb], halves_max(mx) * c);
        const float alpha = fast_exp2(m[rb] - m_new);
        m[rb] = m_new;
        l[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[rb][db][r] *= alpha;
        float sum[4];
#pragma unroll
        for (int kb2 = 0; kb2 < T::NKB; ++kb2)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              x[e] = fast_exp2(__builtin_fmaf(s_cur[rb][kb2][4 * q4 + e], c, -m_new));
            pk_cur[rb][kb2][2 * q4] = pack_bf16x2(x[0], x[1]);
            pk_cur[rb][kb2][2 * q4 + 1] = pack_bf16x2(x[2], x[3]);
            const float gs = (x[0] + x[1]) + (x[2] + x[3]);
            sum[q4] = kb2 == 0 ? gs : sum[q4] + gs;
          }
        tsum[rb] = (sum[0] + sum[1]) + (sum[2] + sum[3]);
      }
    }
#pragma unroll
    for (int rb = 0; rb < T::RB; ++rb) l[rb] += tsum[rb];
    // Loads of iteration j-1 and older landed (K[j+3], V[j+1], which the
    // end of iteration j+1 reads).
    wait_vm<2 * T::LOADS>();
    block_barrier();
  };

  // A block-sparse workgroup whose rows see no key skips the pipeline: its
  // outputs are 0 and its lse -inf (the epilogue handles l = 0).
  if (!SPARSE || nkt > 0) {
  // ---- prologue ---------------------------------------------------------------
  // Issue order K0, K1, K2, V0, K3, V1 (each pair of the last four stands
  // for an iteration that fetches K[j+4] and V[j+2], so the end-of-iteration
  // wait covers them); iteration j then fetches K[j+4] and V[j+2].
  fetch(rk, 0, K0);
  __builtin_amdgcn_sched_barrier(0);
  fetch(rk, 1, K1);
  __builtin_amdgcn_sched_barrier(0);
  fetch(rk, 2, K2);
  __builtin_amdgcn_sched_barrier(0);
  fetch(rv, 0, V0);
  __builtin_amdgcn_sched_barrier(0);
  fetch(rk, 3, K3);
  __builtin_amdgcn_sched_barrier(0);
  fetch(rv, 1, V1);
  wait_vm<2 * T::LOADS>();  // K0, K1, K2 and V0 landed
  block_barrier();
  score_tile(K0 + gofs, sA);
  block_barrier();  // every wave is done with K0 before iteration 0 refills its slot

  u32x4 pre[4];
  iter(IC<0>{}, std::true_type{}, 0, sA, sB, pA, pB, pre);
  // Four iterations per trip (j = 1..4 mod 4) as one straight-line chain, so
  // ring slots and register roles are compile-time in every body.
  for (int j = 1; j < nkt_w; j += 4) {
    window_for(min(j + 7, nkt - 1));  // this trip fetches up to tile j + 7
    iter(IC<1>{}, std::false_type{}, j, sB, sA, pB, pA, pre);
    if (j + 1 >= nkt_w) break;
    iter(IC<2>{}, std::false_type{}, j + 1, sA, sB, pA, pB, pre);
    if (j + 2 >= nkt_w) break;
    iter(IC<3>{}, std::false_type{}, j + 2, sB, sA, pB, pA, pre);
    if (j + 3 >= nkt_w) break;
    iter(IC<0>{}, std::false_type{}, j + 3, sA, sB, pA, pB, pre);
  }

  // Value product of the wave's last tile: P(nkt_w-1) is in pB when nkt_w-1
  // is even.
  auto last_value = [&]() __attribute__((always_inline)) {
    const unsigned(&plast)[T::RB][T::NKB][8] = ((nkt_w - 1) & 1) ? pA : pB;
    switch ((nkt_w - 1) & 3) {
      case 0: value_tile(V0 + gofs, plast); break;
      case 1: value_tile(V1 + gofs, plast); break;
      case 2: value_tile(V2 + gofs, plast); break;
      default: value_tile(V3 + gofs, plast); break;
    }
  };
  if (nkt_w == nkt) {
    wait_vm<0>();
    block_barrier();
    last_value();
  } else {
    // V[nkt_w-1] landed before the barrier that closed iteration nkt_w-1,
    // and its slot is refilled only in iteration nkt_w+1, after the next
    // barrier: read it now.  Then iterations nkt_w..nkt-1 without products:
    // the same loads into the same slots, the same waits and barriers as
    // the waves that still compute, and the final barrier they take before
    // their last value product.
    last_value();
    for (int j = nkt_w; j < nkt; ++j) {
      char* ks = (j & 3) == 0 ? K0 : (j & 3) == 1 ? K1 : (j & 3) == 2 ? K2 : K3;
      char* vs = (j & 3) == 0 ? V2 : (j & 3) == 1 ? V3 : (j & 3) == 2 ? V0 : V1;
      fetch(rk, j + 4, ks);
      fetch(rv, j + 2, vs);
      wait_vm<2 * T::LOADS>();
      block_barrier();
    }
    wait_vm<0>();
    block_barrier();
  }
  }  // !SPARSE || nkt > 0

  if constexpr (SPLIT) {
    // ---- merge of the two key halves --------------------------------------------
    // Group 1's wave r writes its (reference, sum, accumulator) lane by lane
    // into ring slots K_r and V_r; group 0's wave r, which holds the same
    // rows, combines them with its own: M = max(m0, m1), l = l0 2^(m0-M) +
    // l1 2^(m1-M), acc likewise (always in this order).  The first barrier
    // covers the last value products' slot reads.
    static_assert(T::RB == 1 && T::DB * 16 * 64 * 4 <= NG * T::TILEB, "accumulator fits a slot");
    block_barrier();
    float* const kw = reinterpret_cast<float*>(wr == 0 ? K0 : wr == 1 ? K1 : wr == 2 ? K2 : K3);
    float* const vw = reinterpret_cast<float*>(wr == 0 ? V0 : wr == 1 ? V1 : wr == 2 ? V2 : V3);
    if (grp == 1) {
#pragma unroll
      for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) kw[(db * 16 + r) * 64 + lane] = oacc[0][db][r];
      vw[lane] = m[0];
      vw[64 + lane] = l[0];
    }
    block_barrier();
    if (grp == 1) return;  // no barrier follows
    if (nkt_all - nkt > 0) {  // the second half had tiles
      const float m1 = vw[lane], l1 = vw[64 + lane];
      const float M = fmaxf(m[0], m1);
      const float a0 = fast_exp2(m[0] - M), a1 = fast_exp2(m1 - M);
      l[0] = l[0] * a0 + l1 * a1;
#pragma unroll
      for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          oacc[0][db][r] = oacc[0][db][r] * a0 + kw[(db * 16 + r) * 64 + lane] * a1;
      m[0] = M;
    }
  }

  // ---- epilogue: O = acc / l, lse = (m + log2 l) * ln 2 ---------------------
#pragma unroll
  for (int rb = 0; rb < T::RB; ++rb) {
    const int qg = qw0 + 32 * rb + n;
    const float lt = halves_sum(l[rb]);
    // l = 0 only for block-sparse rows that see no key: O = 0, lse = -inf.
    const float inv = (SPARSE && lt == 0.f) ? 0.f : 1.f / lt;
    if (OUT_F32) {
      const auto ro = make_rsrc(static_cast<float*>(O) + qoff, (uint32_t)Lq * D * 4);
#pragma unroll
      for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          u32x4 v;
          v.x = __builtin_bit_cast(unsigned, oacc[rb][db][4 * g4 + 0] * inv);
          v.y = __builtin_bit_cast(unsigned, oacc[rb][db][4 * g4 + 1] * inv);
          v.z = __builtin_bit_cast(unsigned, oacc[rb][db][4 * g4 + 2] * inv);
          v.w = __builtin_bit_cast(unsigned, oacc[rb][db][4 * g4 + 3] * inv);
          store16(ro, (uint32_t)(qg * D + db * 32 + 8 * g4 + 4 * h) * 4, v);
        }
    } else {
      // bf16 O is staged for whole-row stores in the wave's ring slot (K_w,
      // or V_(w-4)).  Waves that computed to the last tile read its V slot
      // after the final barrier, so all waves meet once more first.
      static_assert(T::RB == 1 && 32 * 2 * D <= T::TILEB, "one wave's rows per ring slot");
      // (SPLIT: the merge's barriers already ordered every slot reader, and
      // group 1 has returned; wave r stages in K_r, which only it reads now.)
      if constexpr (!SPLIT) block_barrier();
      u32x2 po[T::DB][4];
#pragma unroll
      for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          po[db][g4].x = pack_bf16x2(oacc[rb][db][4 * g4 + 0] * inv, oacc[rb][db][4 * g4 + 1] * inv);
          po[db][g4].y = pack_bf16x2(oacc[rb][db][4 * g4 + 2] * inv, oacc[rb][db][4 * g4 + 3] * inv);
        }
      char* const st = w == 0 ? K0 : w == 1 ? K1 : w == 2 ? K2 : w == 3 ? K3
                     : w == 4 ? V0 : w == 5 ? V1 : w == 6 ? V2 : V3;
      store_rows_staged<D>(st, lane, po, make_rsrc(static_cast<uint16_t*>(O) + qoff, (uint32_t)Lq * D * 2),
                           qw0);
    }
    if (h == 0 && qg < Lq)
      LSE[(size_t)bh * Lq + qg] =
          (SPARSE && lt == 0.f) ? -INFINITY : (m[rb] + __log2f(lt)) * kLn2;
  }
}

template <int D, bool CAUSAL, bool OUT_F32, int MODE>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  using T = FwdTile<D, MODE != 0>;
  const int n_qt = (a.Lq + T::BR - 1) / T::BR;
  const dim3 grid((unsigned)(n_qt * a.BH));
  // c = |scale| log2(e), kept > 0 so masked (-inf) scores give exactly 0; a
  // zero scale uses a tiny c, which gives probabilities of exactly 1.0f.
  float c = fabsf(a.scale) * kLog2e;
  if (c < 1e-30f) c = 1e-30f;
  const unsigned qsign = a.scale < 0.f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, OUT_F32, MODE>), grid,
                     dim3(64 * T::NW * (MODE == 3 ? 2 : 1)), 0,
                     stream, static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                     static_cast<const uint16_t*>(a.V), a.O, a.lse, a.BH, a.Lq, a.Lk, n_qt, c,
                     qsign, a.block_mask, a.bm_stride, a.nqb, a.nkb);
  return hipGetLastError();
}

template <int D, int MODE>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
  if (a.causal)
    return a.out_f32 ? launch<D, true, true, MODE>(a, stream) : launch<D, true, false, MODE>(a, stream);
  return a.out_f32 ? launch<D, false, true, MODE>(a, stream) : launch<D, false, false, MODE>(a, stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  static_assert(FwdTile<128, false>::BR == kFwdBf16RowsPerBlock, "tile table out of sync");
  if (a.block_mask) return a.d == 64 ? launch_d<64, 2>(a, stream) : launch_d<128, 2>(a, stream);
  // 256-row workgroups unless that gives fewer than two per compute unit
  // (gfx950: 256 compute units); then 128-row ones, which also halve the
  // longest workgroup's work under a causal mask.
  const int64_t wgs256 = (int64_t)((a.Lq + 255) / 256) * a.BH;
  if (wgs256 < 2 * kComputeUnits) {
    // Causal launches whose longest row tile runs at least 128 key tiles
    // (the heavy tiles then bound the launch) split each workgroup's keys
    // over two wave groups: B1 H8 L8192 d128 140.4 -> 133.2 us.  Shorter
    // ones keep two 128-row workgroups per compute unit (the split's 128 KiB
    // of LDS allows one): B2 H16 L2048 d128 40.8 us against 42.3.
    const int bc = a.d == 128 ? FwdTile<128, true>::BC : FwdTile<64, true>::BC;
    if (a.causal && (a.Lk + bc - 1) / bc >= 128)
      return a.d == 64 ? launch_d<64, 3>(a, stream) : launch_d<128, 3>(a, stream);
    return a.d == 64 ? launch_d<64, 1>(a, stream) : launch_d<128, 1>(a, stream);
  }
  return a.d == 64 ? launch_d<64, 0>(a, stream) : launch_d<128, 0>(a, stream);
}

}  // namespace fa
