// Key-split forward for short query blocks against long key sequences (the
// decode shape), bf16 inputs, d in {64, 128}, gfx950.
//
// Generating one token attends a handful of query rows to every cached key:
// the work is a single pass over K and V, bound by memory traffic rather
// than arithmetic (blog page "What Is FlashAttention? ...", section "What it
// changes for you"; explainer page "Flash attention explained", section "Why
// this pattern keeps recurring").  A (slice, query block) pair alone would
// give one workgroup per slice, far too few to stream HBM at full rate, so
// the keys are cut into ranges ("splits") processed by separate workgroups,
// and a second kernel merges the per-range results through their softmax
// normalisers -- the running-statistics recurrence of the annotated-code
// page ("How Flash Attention Improves Transformer Memory Efficiency ...",
// section "The Three Running Statistics") applied once over finished ranges.
//
// Partial kernel.  One workgroup = one slice, 16 query rows, one key range;
// four waves.  64-key K and V tiles stream through a 4-stage LDS ring by
// direct-to-LDS buffer loads, three tiles ahead of use, so that up to 96 KiB
// per CU (d=128) are in flight; the loads are non-temporal, since nothing
// reads a K/V line twice.  Each wave owns 16 keys of every tile:
//   S^T (16 keys x 16 queries) = K_w Q^T    on v_mfma_f32_16x16x32_bf16
//   online softmax per query over the wave's keys (fp32; the probabilities
//   are rounded to bf16 for the value product, the running sum adds them
//   unrounded)
//   O^T (d x 16 queries) += V_w^T P^T        on v_mfma_f32_16x16x16_bf16
// The score product's output layout (lane l, register r: key 4(l/16)+r,
// query l%16) is exactly the B-operand layout of the value product, so the
// probabilities go from the accumulator to the next product without moving
// between lanes.  At the end the four waves' (m, l, O) are merged in LDS and
// the range's normalised output O_s and natural-log lse_s go to the
// workspace.  A row that sees no key of its range writes O_s = 0 and
// lse_s = -inf, which gives it weight zero in the merge.
//
// Merge kernel.  Per query row: lse = log sum_s exp(lse_s),
// O = sum_s exp(lse_s - lse) O_s, written in the output dtype.  Every row sees
// key 0, so at least one range has a finite lse.

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {
namespace {

// Cache-policy operand of the buffer-load builtins on gfx950: bit 1 is NT
// (non-temporal: the line is not kept for reuse).
constexpr int kCachePolicyNT = 2;

typedef short i16x4v __attribute__((ext_vector_type(4)));

template <int D>
struct SplitTile {
  static constexpr int NW = 4;                     // waves; wave w owns keys [16w, 16w+16) of a tile
  static constexpr int BC = kSplitKvKeysPerTile;   // keys per tile
  static constexpr int QR = kSplitKvRowsPerBlock;  // query rows per workgroup
  static constexpr int ROWB = D * 2;               // bytes per K/V row
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int TILEB = BC * ROWB;          // bytes per K (or V) tile
  static constexpr int RPK = 1024 / ROWB;          // rows per 1-KiB load instruction
  static constexpr int LOADS = TILEB / 1024 / NW;  // 1-KiB loads per wave per tensor per tile
  static_assert(LOADS >= 1 && LOADS <= 4, "immediate load offsets reach 3 KiB");
  static constexpr int KSTEP = D / 32;             // 32-deep steps of the score product
  static constexpr int DB = D / 16;                // 16-row blocks of O^T
  static constexpr int OPAD = D + 4;               // floats per query row in the wave merge
  static_assert(QR * OPAD * 4 <= TILEB, "one wave's partial output fits in one ring slot");
};

// Chunk swizzle of this kernel's K/V tiles (16-byte chunk c of row r is
// stored at c ^ split_swz(r)).  Its reads differ from the dense kernels':
// a K fragment read (ds_read_b128) takes chunks 4ks+g of rows 16w+u (lane
// 16g+u), and a V^T transposed read takes a 32-byte chunk pair of 8
// consecutive rows per 32 lanes.  For the transposed read the bank rule is
// the plain one (64 four-byte banks, 32 lanes at a time), which asks for the
// 8 rows' pairs at 8 distinct pair positions of a 256-byte line.  The
// 16-byte reads do not follow that rule (two lanes 16 apart reading one row
// conflict, two reading the same chunk of rows 16 apart do not), so among
// the swizzles that satisfy the transposed rule these were chosen by
// measuring the exact read patterns with the shader's LDS bank-conflict
// counter: zero conflict cycles for both reads, at d = 128 and d = 64.
template <int D>
__device__ __forceinline__ int split_swz(int r) {
  const int b0 = r & 1, b1 = (r >> 1) & 1, b2 = (r >> 2) & 1, b3 = (r >> 3) & 1;
  if (D == 128) return (b0 << 1) ^ (b1 << 2) ^ (b2 << 3) ^ (b3 * 9);
  return (b1 << 1) ^ (b2 * 6) ^ (b3 << 1);
}

__device__ __forceinline__ f32x4 mma16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16x16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4v, a),
                                                   __builtin_bit_cast(i16x4v, b), c, 0, 0, 0);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void splitkv_partial_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ Opart, float* __restrict__ LSEpart,
    int BH, int Lq, int Lk, int nsplit, int chunk, float c) {
  using T = SplitTile<D>;
  // One array per ring slot: the compiler then relates each LDS read only to
  // the direct-to-LDS loads of its own slot.
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
  const int lane = tid & 63, u = lane & 15, g = lane >> 4;

  // Workgroup -> (slice, key range, query block); consecutive workgroups take
  // different slices.
  const int bh = wg_id() % BH;
  const int rest = wg_id() / BH;
  const int s = rest % nsplit;
  const int q0 = (rest / nsplit) * T::QR;

  const int k_beg = s * chunk;
  int k_end = min(k_beg + chunk, Lk);
  if (CAUSAL) k_end = min(k_end, min(q0 + T::QR, Lq));  // no row of the block sees later keys
  const int nt = k_end > k_beg ? (k_end - k_beg + T::BC - 1) / T::BC : 0;

  const size_t qoff = (size_t)bh * Lq * D;
  const size_t koff = (size_t)bh * Lk * D;
  const auto rq = make_rsrc(Q + qoff, (uint32_t)Lq * D * 2);
  const auto rk = make_rsrc(K + koff, (uint32_t)Lk * D * 2);
  const auto rv = make_rsrc(V + koff, (uint32_t)Lk * D * 2);

  // ---- tile fetch: each wave moves LOADS KiB of the K (and V) tile -------
  // Lane l of load i writes LDS bytes [16 l, 16 l + 16) of KiB (w*LOADS + i)
  // of the slot and fetches the logical chunk the swizzle stores there.
  int fetch_off[T::LOADS];
#pragma unroll
  for (int i = 0; i < T::LOADS; ++i) {
    const int row = (w * T::LOADS + i) * T::RPK + lane / T::CPR;
    const int chunk16 = (lane % T::CPR) ^ split_swz<D>(row);
    fetch_off[i] = (row * D + chunk16 * 8) * 2;
  }
  auto fetch = [&](const __amdgpu_buffer_rsrc_t& r, int t, char* slot)
                   __attribute__((always_inline)) {
    // Tiles past the last re-fetch the last one, which keeps the number of
    // loads in flight the same every iteration.
    const int tt = min(t, nt - 1);
    const uint32_t base = (uint32_t)(k_beg + tt * T::BC) * T::ROWB;
    lds_void* dst = (lds_void*)(slot + w * T::LOADS * 1024);
    static_for<0, T::LOADS>([&](auto Ic) __attribute__((always_inline)) {
      constexpr int i = decltype(Ic)::value;
      // The explicit conversion matters: with an implicit one in this
      // argument the host pass drops the kernel's launch stub without a
      // diagnostic.  Every K/V byte is read once, so the loads carry the
      // non-temporal hint (cache-policy bit NT): streaming reads with it
      // reach ~7 TB/s on MI355X against ~5.8 without.
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, (uint32_t)(base + fetch_off[i] - i * 1024),
                                               0, i * 1024, kCachePolicyNT);
    });
  };

  // ---- per-lane LDS read offsets (slot-relative) ---------------------------
  // K (A operand of the score product): key row 16w + u, chunk 4ks + g.
  const int krow = 16 * w + u;
  int koffs[T::KSTEP];
#pragma unroll
  for (int ks = 0; ks < T::KSTEP; ++ks)
    koffs[ks] = krow * T::ROWB + (((4 * ks + g) ^ split_swz<D>(krow)) << 4);
  // V^T (A operand of the value product) by transposed reads: in lane group
  // g, lane u = 4j + t4 points at key row 16w + 4g + j, columns
  // 16db + 4t4 .. +3; lane u receives column 16db + u of the four rows.
  const int vrow = 16 * w + 4 * g + (u >> 2), t4 = u & 3;
  int voffs[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db)
    voffs[db] = vrow * T::ROWB + (((2 * db + (t4 >> 1)) ^ split_swz<D>(vrow)) << 4) + 8 * (t4 & 1);

  // ---- Q^T fragments (B operand of the score product) ----------------------
  // Lane l: query q0 + u, the same head-dimension chunks 4ks + g as K.
  u32x4 qf[T::KSTEP];
#pragma unroll
  for (int ks = 0; ks < T::KSTEP; ++ks)
    qf[ks] = load16(rq, (uint32_t)((q0 + u) * D + (4 * ks + g) * 8) * 2);

  f32x4 oacc[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  const int qrow = q0 + u;
  const int kvis_end = CAUSAL ? min(k_end, qrow + 1) : k_end;  // this lane's visible keys end here

  auto iter = [&](auto Rc, int t) __attribute__((always_inline)) {
    constexpr int R = decltype(Rc)::value;
    // Tile t landed for this wave (tiles t+1, t+2 may still be in flight),
    // then for every wave; every wave is also done with slot R+3 = R-1.
    wait_vm<4 * T::LOADS>();
    block_barrier();
    fetch(rk, t + 3, kslot(IC<(R + 3) % 4>{}));
    fetch(rv, t + 3, vslot(IC<(R + 3) % 4>{}));
    const char* kb = kslot(IC<R>{});
    const char* vb = vslot(IC<R>{});

    u32x4 ka[T::KSTEP];
#pragma unroll
    for (int ks = 0; ks < T::KSTEP; ++ks) ka[ks] = lds_read16(kb, koffs[ks]);
    u32x2 va[T::DB];
#pragma unroll
    for (int db = 0; db < T::DB; ++db) va[db] = lds_read_tr(vb, voffs[db]);

    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < T::KSTEP; ++ks) sc = mma16x32(ka[ks], qf[ks], sc);

    // Register r holds key k_beg + t*BC + 16w + 4g + r for query qrow.
    const int key = k_beg + t * T::BC + 16 * w + 4 * g;
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = (key + r < kvis_end) ? sc[r] * c : -INFINITY;
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m, mx);
    const float base = m_new == -INFINITY ? 0.f : m_new;  // no key seen yet: p and alpha are 0
    const float alpha = fast_exp2(m - base);
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = fast_exp2(x[r] - base);
    u32x2 pk;
    pk.x = pack_bf16x2(p[0], p[1]);
    pk.y = pack_bf16x2(p[2], p[3]);
    // The running sum adds the unrounded values: summing the bf16-rounded
    // ones moves lse by more than 1e-3 on rows that see few keys.
    float ps = (p[0] + p[1]) + (p[2] + p[3]);
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l = alpha * l + ps;
    m = m_new;
#pragma unroll
    for (int db = 0; db < T::DB; ++db) {
      oacc[db] *= alpha;
      oacc[db] = mma16x16(va[db], pk, oacc[db]);
    }
  };

  if (nt > 0) {
    fetch(rk, 0, K0);
    fetch(rv, 0, V0);
    fetch(rk, 1, K1);
    fetch(rv, 1, V1);
    fetch(rk, 2, K2);
    fetch(rv, 2, V2);
    for (int t = 0; t < nt; t += 4) {
      iter(IC<0>{}, t);
      if (t + 1 >= nt) break;
      iter(IC<1>{}, t + 1);
      if (t + 2 >= nt) break;
      iter(IC<2>{}, t + 2);
      if (t + 3 >= nt) break;
      iter(IC<3>{}, t + 3);
    }
    wait_vm<0>();
  }
  block_barrier();  // every wave is done with the ring: reuse it for the merge

  // ---- merge the four waves' (m, l, O) --------------------------------------
  // Wave w writes O^T (lane l, register r of block db: d = 16db + 4g + r,
  // query u) as rows [query][d] into ring slot K_w, and m, l into V0.
  {
    char* mine = w == 0 ? K0 : w == 1 ? K1 : w == 2 ? K2 : K3;
    float* ow = reinterpret_cast<float*>(mine);
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
      *reinterpret_cast<f32x4*>(ow + u * T::OPAD + 16 * db + 4 * g) = oacc[db];
    float* ml = reinterpret_cast<float*>(V0);
    if (g == 0) {
      ml[w * T::QR + u] = m;
      ml[(T::NW + w) * T::QR + u] = l;
    }
  }
  block_barrier();

  const float* ml = reinterpret_cast<const float*>(V0);
  const size_t part = (size_t)s * BH + bh;
  const auto ro = make_rsrc(Opart + part * Lq * D, (uint32_t)Lq * D * 4);
  const auto rl = make_rsrc(LSEpart + part * Lq, (uint32_t)Lq * 4);
  for (int idx = tid; idx < T::QR * (D / 4); idx += 64 * T::NW) {
    const int i = idx / (D / 4), d4 = idx % (D / 4);
    float mw[T::NW], M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < T::NW; ++ww) {
      mw[ww] = ml[ww * T::QR + i];
      M = fmaxf(M, mw[ww]);
    }
    const float base = M == -INFINITY ? 0.f : M;
    float L = 0.f;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    static_for<0, T::NW>([&](auto Wc) __attribute__((always_inline)) {
      constexpr int ww = decltype(Wc)::value;
      const float f = fast_exp2(mw[ww] - base);
      L += f * ml[(T::NW + ww) * T::QR + i];
      acc += f * *reinterpret_cast<const f32x4*>(
                     reinterpret_cast<const float*>(kslot(IC<ww>{})) + i * T::OPAD + 4 * d4);
    });
    // A row with no visible key in this range: O_s = 0, lse_s = -inf.
    const float inv = L > 0.f ? 1.f / L : 0.f;
    acc *= inv;
    store16(ro, (uint32_t)((q0 + i) * D + 4 * d4) * 4, __builtin_bit_cast(u32x4, acc));
    if (d4 == 0)
      store4f(rl, (uint32_t)(q0 + i) * 4, L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY);
  }
}

// Merge of the per-range results: one thread per 4 output columns of a row.
template <int D, bool OUT_F32>
__global__ __launch_bounds__(256) void splitkv_merge_kernel(
    const float* __restrict__ Opart, const float* __restrict__ LSEpart, void* __restrict__ O,
    float* __restrict__ LSE, int64_t rows, int nsplit) {
  constexpr int TPR = D / 4;  // threads per row
  const int tid = wi_id();
  const int64_t row = (int64_t)wg_id() * (256 / TPR) + tid / TPR;
  const int d4 = tid % TPR;
  if (row >= rows) return;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, LSEpart[(size_t)s * rows + row]);
  float L = 0.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsplit; ++s) {
    const float ls = LSEpart[(size_t)s * rows + row];
    const float f = fast_exp2((ls - M) * kLog2e);  // -inf (unseen range) gives 0
    L += f;
    acc += f * *reinterpret_cast<const f32x4*>(Opart + ((size_t)s * rows + row) * D + 4 * d4);
  }
  acc *= 1.f / L;
  if (OUT_F32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(O) + row * D + 4 * d4) = acc;
  } else {
    u32x2 p;
    p.x = pack_bf16x2(acc[0], acc[1]);
    p.y = pack_bf16x2(acc[2], acc[3]);
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(O) + row * D + 4 * d4) = p;
  }
  if (d4 == 0) LSE[row] = M + __logf(L);
}

template <int D, bool CAUSAL>
hipError_t launch_partial(const SplitKvArgs& a, hipStream_t stream) {
  const int nqb = (a.Lq + kSplitKvRowsPerBlock - 1) / kSplitKvRowsPerBlock;
  const unsigned grid = (unsigned)((int64_t)a.BH * nqb * a.nsplit);
  hipLaunchKernelGGL((splitkv_partial_kernel<D, CAUSAL>), dim3(grid), dim3(256), 0, stream,
                     (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V, a.Opart,
                     a.LSEpart, a.BH, a.Lq, a.Lk, a.nsplit, a.chunk, a.scale * kLog2e);
  return hipGetLastError();
}

template <int D, bool OUT_F32>
hipError_t launch_merge(const SplitKvArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.BH * a.Lq;
  const int64_t per = 256 / (D / 4);
  const unsigned grid = (unsigned)((rows + per - 1) / per);
  hipLaunchKernelGGL((splitkv_merge_kernel<D, OUT_F32>), dim3(grid), dim3(256), 0, stream,
                     a.Opart, a.LSEpart, a.O, a.lse, rows, a.nsplit);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_splitkv_bf16(const SplitKvArgs& a, unsigned stages, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (stages & kSplitKvPartial) {
    if (a.d == 128)
      e = a.causal ? launch_partial<128, true>(a, stream) : launch_partial<128, false>(a, stream);
    else
      e = a.causal ? launch_partial<64, true>(a, stream) : launch_partial<64, false>(a, stream);
    if (e != hipSuccess) return e;
  }
  if (stages & kSplitKvMerge) {
    if (a.d == 128)
      e = a.out_f32 ? launch_merge<128, true>(a, stream) : launch_merge<128, false>(a, stream);
    else
      e = a.out_f32 ? launch_merge<64, true>(a, stream) : launch_merge<64, false>(a, stream);
  }
  return e;
}

}  // namespace fa
