// C ABI of libfa (declared in include/fa.h): argument validation, workspace
// layout and dispatch to the gfx950 kernels.  Validation runs entirely on
// the host and returns before any HIP call, so an invalid call enqueues
// nothing.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "fa.h"
#include "fa_launch.h"

namespace {

constexpr int64_t kMaxSliceBytes = int64_t(1) << 31;  // per-slice byte offsets stay 32-bit

bool valid_dtype(int t) { return t == FA_F32 || t == FA_BF16; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Shape checks shared by forward, backward and workspace sizing.  Slices get
// one tile of slack so that in-kernel offsets of the last (ragged) tile stay
// representable.
// Every size is bounded before it enters a product, so no product below can
// overflow int64 whatever the caller passes.
fa_status check_shape(fa_dtype in_dtype, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d) {
  if (B < 0 || H < 0 || Lq < 0 || Lk < 0 || d <= 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (B > INT32_MAX || H > INT32_MAX || Lq > INT32_MAX || Lk > INT32_MAX) return FA_ERR_SHAPE;
  // All four are now below 2^31, so the products below stay below 2^62.
  if (B * H > INT32_MAX) return FA_ERR_SHAPE;
  if (B * H > 0 && Lq > 0 && Lk == 0) return FA_ERR_SHAPE;
  const int64_t slack = 256;
  const int64_t esz = 4;  // fp32 outputs and accumulators bound every path
  if ((Lq + slack) * d * esz >= kMaxSliceBytes || (Lk + slack) * d * esz >= kMaxSliceBytes)
    return FA_ERR_SHAPE;
  const int64_t bh = B * H;
  // Row counts bound the grids of the row-wise helper kernels.
  if (bh * Lq > (int64_t(1) << 34) || bh * Lk > (int64_t(1) << 34)) return FA_ERR_SHAPE;
  const int64_t rows_per_block =
      in_dtype == FA_BF16 ? fa::kBf16MinRowsPerBlock : fa::kF32RowsPerBlock;
  // Grid sizes (x dimension) of the largest launch, query- or key-side, must fit.
  if (bh * cdiv(Lq, rows_per_block) > INT32_MAX || bh * cdiv(Lk, rows_per_block) > INT32_MAX)
    return FA_ERR_SHAPE;
  // So must its work-item count (grid x workgroup size), which a dispatch
  // carries in 32 bits: at most D/8 threads per query row (the bf16 prepare
  // kernel; every other bf16 kernel uses 2-4) and 32 per row or key at fp32,
  // over the rows padded to a whole workgroup.  Only sizes near the device
  // memory (2^28 bf16 rows of d = 128) reach it.
  const int64_t threads_per_row = in_dtype == FA_BF16 ? d / 8 : 32;
  const int64_t longest = std::max(Lq, Lk) + 256;
  if (bh * longest * threads_per_row > int64_t(UINT32_MAX)) return FA_ERR_SHAPE;
  return FA_OK;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

extern "C" {

const char* fa_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: invalid or too large sizes (negative size, Lk = 0 with Lq > 0, over 2^31 bytes per slice, or over 2^32 threads in one launch)";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dimension or dtype combination not implemented (d must be 64 or 128)";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: a base pointer is not 16-byte aligned";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace NULL or smaller than the matching *_workspace_bytes() size";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime reported a launch error";
    case FA_ERR_ARG: return "FA_ERR_ARG: non-finite scale, unknown enum value or split count out of range";
  }
  return "unknown fa_status";
}

const char* fa_version(void) { return "libfa 0.1.0 gfx950"; }

fa_status fa_fwd(fa_dtype in_dtype, fa_dtype out_dtype, int64_t B, int64_t H, int64_t Lq,
                 int64_t Lk, int64_t d, const void* Q, const void* K, const void* V, float scale,
                 int causal, void* O, float* lse, hipStream_t stream) {
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype) || !std::isfinite(scale)) return FA_ERR_ARG;
  if (fa_status st = check_shape(in_dtype, B, H, Lq, Lk, d)) return st;
  if (in_dtype == FA_F32 && out_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if (B * H * Lq == 0) return FA_OK;
  if (!Q || !K || !V || !O || !lse) return FA_ERR_NULL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(lse))
    return FA_ERR_ALIGN;

  fa::FwdArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.lse = lse;
  a.BH = (int)(B * H);
  a.Lq = (int)Lq;
  a.Lk = (int)Lk;
  a.d = (int)d;
  a.scale = scale;
  a.causal = causal != 0;
  a.out_f32 = out_dtype == FA_F32;
  const hipError_t e = in_dtype == FA_BF16 ? fa::launch_fwd_bf16(a, stream) : fa::launch_fwd_f32(a, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd_blocksparse(fa_dtype in_dtype, fa_dtype out_dtype, int64_t B, int64_t H,
                             int64_t Lq, int64_t Lk, int64_t d, const void* Q, const void* K,
                             const void* V, float scale, int causal, const uint8_t* block_mask,
                             int64_t mask_slices, void* O, float* lse, hipStream_t stream) {
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype) || !std::isfinite(scale)) return FA_ERR_ARG;
  if (fa_status st = check_shape(in_dtype, B, H, Lq, Lk, d)) return st;
  if (in_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (mask_slices != 1 && mask_slices != B * H) return FA_ERR_ARG;
  const int64_t nqb = cdiv(Lq, fa::kSparseBlock), nkb = cdiv(Lk, fa::kSparseBlock);
  if (nkb > fa::kSparseMaxKeyBlocks) return FA_ERR_UNSUPPORTED;
  if (nqb * nkb > INT32_MAX || B * H * nqb > INT32_MAX) return FA_ERR_SHAPE;  // mask, grid
  if (B * H * Lq == 0) return FA_OK;
  if (!Q || !K || !V || !O || !lse || !block_mask) return FA_ERR_NULL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(lse))
    return FA_ERR_ALIGN;

  fa::FwdArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.lse = lse;
  a.BH = (int)(B * H);
  a.Lq = (int)Lq;
  a.Lk = (int)Lk;
  a.d = (int)d;
  a.scale = scale;
  a.causal = causal != 0;
  a.out_f32 = out_dtype == FA_F32;
  a.block_mask = block_mask;
  a.nqb = (int)nqb;
  a.nkb = (int)nkb;
  a.bm_stride = mask_slices == 1 ? 0 : (int)(nqb * nkb);
  const hipError_t e = fa::launch_fwd_bf16(a, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_bytes(fa_dtype in_dtype, int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                              int64_t d) {
  if (!valid_dtype(in_dtype) || check_shape(in_dtype, B, H, Lq, Lk, d) != FA_OK) return 0;
  const size_t rows = (size_t)(B * H * Lq);
  // D statistic and lse in base 2.
  return 2 * round_up(rows * sizeof(float), 256);
}

}  // extern "C"

namespace {

// Shared by fa_bwd and its three stages: validates exactly the pointers the
// requested stages touch, then enqueues those stages.
fa_status bwd_stages(unsigned stages, fa_dtype in_dtype, fa_dtype o_dtype, int64_t B, int64_t H,
                     int64_t Lq, int64_t Lk, int64_t d, const void* Q, const void* K, const void* V,
                     const void* O, const void* dO, const float* lse, float scale, int causal,
                     void* dQ, void* dK, void* dV, const void* workspace, size_t workspace_bytes,
                     hipStream_t stream, const uint8_t* block_mask = nullptr,
                     int64_t mask_slices = 0) {
  if (!valid_dtype(in_dtype) || !valid_dtype(o_dtype) || !std::isfinite(scale)) return FA_ERR_ARG;
  if (fa_status st = check_shape(in_dtype, B, H, Lq, Lk, d)) return st;
  // O is in the input dtype, or fp32 beside bf16 inputs (fa_fwd's outputs).
  if (in_dtype == FA_F32 && o_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  const bool has_q = B * H * Lq > 0, has_k = B * H * Lk > 0;
  if (!has_q && !has_k) return FA_OK;
  const bool pre = stages & fa::kBwdPrepare, kv = stages & fa::kBwdDkDv, dq = stages & fa::kBwdDq;
  // A slice with queries always has keys (check_shape), so has_q implies has_k.
  if (has_q && pre && (!O || !dO || !lse)) return FA_ERR_NULL;
  if (has_q && (kv || dq) && (!Q || !dO)) return FA_ERR_NULL;
  if (has_q && dq && (!K || !V || !dQ)) return FA_ERR_NULL;
  if (has_k && kv && (!K || !V || !dK || !dV)) return FA_ERR_NULL;
  const void* ptrs[] = {Q, K, V, O, dO, lse, dQ, dK, dV};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FA_ERR_ALIGN;
  const size_t need = fa_bwd_workspace_bytes(in_dtype, B, H, Lq, Lk, d);
  if (need > 0 && (!workspace || workspace_bytes < need)) return FA_ERR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return FA_ERR_ALIGN;

  const size_t rows = (size_t)(B * H * Lq);
  const size_t stat = round_up(rows * sizeof(float), 256);
  char* ws = static_cast<char*>(const_cast<void*>(workspace));
  fa::BwdArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.dO = dO;
  a.lse = lse;
  a.dQ = dQ;
  a.dK = dK;
  a.dV = dV;
  a.Dvec = reinterpret_cast<float*>(ws);
  a.lse2 = ws ? reinterpret_cast<float*>(ws + stat) : nullptr;
  a.BH = (int)(B * H);
  a.Lq = (int)Lq;
  a.Lk = (int)Lk;
  a.d = (int)d;
  a.scale = scale;
  a.causal = causal != 0;
  a.o_f32 = o_dtype == FA_F32;
  if (block_mask) {
    a.block_mask = block_mask;
    a.nqb = (int)cdiv(Lq, fa::kSparseBlock);
    a.nkb = (int)cdiv(Lk, fa::kSparseBlock);
    a.bm_stride = mask_slices == 1 ? 0 : a.nqb * a.nkb;
  }
  // Second line of defence: every pointer a launched kernel dereferences is
  // set (the checks above are per argument; this is per kernel).
  if (has_q && pre && !(a.O && a.dO && a.lse && a.Dvec && a.lse2)) return FA_ERR_NULL;
  if (has_k && kv && !(a.K && a.V && a.dK && a.dV)) return FA_ERR_NULL;
  if (has_q && kv && !(a.Q && a.dO && a.Dvec && a.lse2)) return FA_ERR_NULL;
  if (has_q && dq && !(a.Q && a.K && a.V && a.dO && a.dQ && a.Dvec && a.lse2)) return FA_ERR_NULL;
  const hipError_t e = in_dtype == FA_BF16 ? fa::launch_bwd_bf16(a, stages, stream)
                                           : fa::launch_bwd_f32(a, stages, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

fa_status fa_bwd(fa_dtype in_dtype, fa_dtype o_dtype, int64_t B, int64_t H, int64_t Lq,
                 int64_t Lk, int64_t d, const void* Q, const void* K, const void* V,
                 const void* O, const void* dO, const float* lse, float scale, int causal,
                 void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
  return bwd_stages(fa::kBwdAll, in_dtype, o_dtype, B, H, Lq, Lk, d, Q, K, V, O, dO, lse, scale,
                    causal, dQ, dK, dV, workspace, workspace_bytes, stream);
}

fa_status fa_bwd_prepare(fa_dtype in_dtype, fa_dtype o_dtype, int64_t B, int64_t H, int64_t Lq,
                         int64_t Lk, int64_t d, const void* O, const void* dO, const float* lse,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_stages(fa::kBwdPrepare, in_dtype, o_dtype, B, H, Lq, Lk, d, nullptr, nullptr, nullptr,
                    O, dO, lse, 1.f, 0, nullptr, nullptr, nullptr, workspace, workspace_bytes,
                    stream);
}

fa_status fa_bwd_dkdv(fa_dtype in_dtype, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d,
                      const void* Q, const void* K, const void* V, const void* dO, float scale,
                      int causal, void* dK, void* dV, const void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  return bwd_stages(fa::kBwdDkDv, in_dtype, in_dtype, B, H, Lq, Lk, d, Q, K, V, nullptr, dO,
                    nullptr, scale, causal, nullptr, dK, dV, workspace, workspace_bytes, stream);
}

fa_status fa_bwd_dq(fa_dtype in_dtype, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d,
                    const void* Q, const void* K, const void* V, const void* dO, float scale,
                    int causal, void* dQ, const void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  return bwd_stages(fa::kBwdDq, in_dtype, in_dtype, B, H, Lq, Lk, d, Q, K, V, nullptr, dO,
                    nullptr, scale, causal, dQ, nullptr, nullptr, workspace, workspace_bytes,
                    stream);
}

fa_status fa_bwd_prepare_dq(fa_dtype in_dtype, fa_dtype o_dtype, int64_t B, int64_t H,
                            int64_t Lq, int64_t Lk, int64_t d, const void* Q, const void* K,
                            const void* V, const void* O, const void* dO, const float* lse,
                            float scale, int causal, void* dQ, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  return bwd_stages(fa::kBwdPrepare | fa::kBwdDq, in_dtype, o_dtype, B, H, Lq, Lk, d, Q, K, V, O,
                    dO, lse, scale, causal, dQ, nullptr, nullptr, workspace, workspace_bytes,
                    stream);
}

}  // extern "C"

namespace {

constexpr int64_t kMaxSplits = 4096;

int64_t splitkv_chunk(int64_t Lk, int64_t nsplit) {
  const int64_t t = fa::kSplitKvKeysPerTile;
  return cdiv(cdiv(Lk, nsplit), t) * t;
}

// Shape and size checks of the key-split forward (sizes the merge needs
// too: Lk is only bounded through check_shape).
fa_status splitkv_check(int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d, int64_t nsplit) {
  if (fa_status st = check_shape(FA_BF16, B, H, Lq, Lk, d)) return st;
  if (nsplit < 1 || nsplit > kMaxSplits) return FA_ERR_ARG;
  const int64_t bh = B * H;
  if (bh * cdiv(Lq, fa::kSplitKvRowsPerBlock) * nsplit > INT32_MAX) return FA_ERR_SHAPE;
  if (cdiv(bh * Lq, 256 / (d / 4)) > INT32_MAX) return FA_ERR_SHAPE;
  return FA_OK;
}

size_t splitkv_opart_bytes(int64_t B, int64_t H, int64_t Lq, int64_t d, int64_t nsplit) {
  return round_up((size_t)(nsplit * B * H * Lq * d) * sizeof(float), 256);
}

size_t splitkv_ws_bytes(int64_t B, int64_t H, int64_t Lq, int64_t d, int64_t nsplit) {
  return splitkv_opart_bytes(B, H, Lq, d, nsplit) +
         round_up((size_t)(nsplit * B * H * Lq) * sizeof(float), 256);
}

fa_status splitkv_run(unsigned stages, fa_dtype in_dtype, fa_dtype out_dtype, int64_t B,
                      int64_t H, int64_t Lq, int64_t Lk, int64_t d, const void* Q, const void* K,
                      const void* V, float scale, int causal, int64_t nsplit, void* O, float* lse,
                      const void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype) || !std::isfinite(scale)) return FA_ERR_ARG;
  if (fa_status st = splitkv_check(B, H, Lq, Lk, d, nsplit)) return st;
  if (in_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (B * H * Lq == 0) return FA_OK;
  const bool part = stages & fa::kSplitKvPartial, merge = stages & fa::kSplitKvMerge;
  if (part && (!Q || !K || !V)) return FA_ERR_NULL;
  if (merge && (!O || !lse)) return FA_ERR_NULL;
  const void* ptrs[] = {Q, K, V, O, lse};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FA_ERR_ALIGN;
  if (!workspace || workspace_bytes < splitkv_ws_bytes(B, H, Lq, d, nsplit)) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;

  char* ws = static_cast<char*>(const_cast<void*>(workspace));
  fa::SplitKvArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.lse = lse;
  a.Opart = reinterpret_cast<float*>(ws);
  a.LSEpart = reinterpret_cast<float*>(ws + splitkv_opart_bytes(B, H, Lq, d, nsplit));
  a.BH = (int)(B * H);
  a.Lq = (int)Lq;
  a.Lk = (int)Lk;
  a.d = (int)d;
  a.nsplit = (int)nsplit;
  a.chunk = (int)splitkv_chunk(Lk, nsplit);
  a.scale = scale;
  a.causal = causal != 0;
  a.out_f32 = out_dtype == FA_F32;
  const hipError_t e = fa::launch_splitkv_bf16(a, stages, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

int64_t fa_fwd_splitkv_default_splits(int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d) {
  if (check_shape(FA_BF16, B, H, Lq, Lk, d) != FA_OK || B * H * Lq == 0) return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  const int64_t blocks = B * H * cdiv(Lq, fa::kSplitKvRowsPerBlock);
  int64_t n = cdiv(2 * (int64_t)cus, blocks);
  n = std::min(n, std::max<int64_t>(1, Lk / 256));
  return std::max<int64_t>(1, std::min(n, kMaxSplits));
}

size_t fa_fwd_splitkv_workspace_bytes(fa_dtype in_dtype, int64_t B, int64_t H, int64_t Lq,
                                      int64_t Lk, int64_t d, int64_t nsplit) {
  if (in_dtype != FA_BF16 || splitkv_check(B, H, Lq, Lk, d, nsplit) != FA_OK) return 0;
  return splitkv_ws_bytes(B, H, Lq, d, nsplit);
}

fa_status fa_fwd_splitkv(fa_dtype in_dtype, fa_dtype out_dtype, int64_t B, int64_t H, int64_t Lq,
                         int64_t Lk, int64_t d, const void* Q, const void* K, const void* V,
                         float scale, int causal, int64_t nsplit, void* O, float* lse,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return splitkv_run(fa::kSplitKvAll, in_dtype, out_dtype, B, H, Lq, Lk, d, Q, K, V, scale, causal,
                     nsplit, O, lse, workspace, workspace_bytes, stream);
}

fa_status fa_fwd_splitkv_partial(fa_dtype in_dtype, int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                                 int64_t d, const void* Q, const void* K, const void* V,
                                 float scale, int causal, int64_t nsplit, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  return splitkv_run(fa::kSplitKvPartial, in_dtype, FA_BF16, B, H, Lq, Lk, d, Q, K, V, scale,
                     causal, nsplit, nullptr, nullptr, workspace, workspace_bytes, stream);
}

fa_status fa_fwd_splitkv_merge(fa_dtype out_dtype, int64_t B, int64_t H, int64_t Lq, int64_t d,
                               int64_t nsplit, const void* workspace, size_t workspace_bytes,
                               void* O, float* lse, hipStream_t stream) {
  // The merge does not look at keys; one key keeps the shape checks valid.
  return splitkv_run(fa::kSplitKvMerge, FA_BF16, out_dtype, B, H, Lq, 1, d, nullptr, nullptr,
                     nullptr, 1.f, 0, nsplit, O, lse, workspace, workspace_bytes, stream);
}

}  // extern "C"

extern "C" {

fa_status fa_bwd_blocksparse(fa_dtype in_dtype, fa_dtype o_dtype, int64_t B, int64_t H,
                             int64_t Lq, int64_t Lk, int64_t d, const void* Q, const void* K, const void* V, const void* O,
                             const void* dO, const float* lse, float scale, int causal,
                             const uint8_t* block_mask, int64_t mask_slices, void* dQ, void* dK,
                             void* dV, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  if (!valid_dtype(in_dtype) || !valid_dtype(o_dtype) || !std::isfinite(scale)) return FA_ERR_ARG;
  if (fa_status st = check_shape(in_dtype, B, H, Lq, Lk, d)) return st;
  if (in_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (mask_slices != 1 && mask_slices != B * H) return FA_ERR_ARG;
  const int64_t nqb = cdiv(Lq, fa::kSparseBlock), nkb = cdiv(Lk, fa::kSparseBlock);
  if (nkb > fa::kSparseMaxKeyBlocks || nqb > fa::kSparseMaxKeyBlocks) return FA_ERR_UNSUPPORTED;
  if (B * H * (Lq + Lk) > 0 && !block_mask) return FA_ERR_NULL;
  return bwd_stages(fa::kBwdAll, in_dtype, o_dtype, B, H, Lq, Lk, d, Q, K, V, O, dO, lse, scale,
                    causal, dQ, dK, dV, workspace, workspace_bytes, stream, block_mask,
                    mask_slices);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Backward without a caller-provided workspace: the per-row statistics live
// in a fixed device array of this library instead.
// ---------------------------------------------------------------------------

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;  // D and base-2 lse for up to 2^21 rows
constexpr int kMaxDevices = 64;

// One copy per GPU the library runs on, held until the process ends.  Host
// code never passes the name itself to a kernel or a copy: on the host it
// names a stand-in, not device memory.  The device address comes from
// hipGetSymbolAddress, once per device (scratch_address).
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that owns `stream` (the current
// device for the NULL stream); looked up the first time with that device
// current, then reused.
fa_status scratch_address(hipStream_t stream, void** out) {
  int cur = 0, dev = 0;
  if (hipGetDevice(&cur) != hipSuccess) return FA_ERR_HIP;
  dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return FA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return FA_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return FA_ERR_HIP;
    if (e != hipSuccess || p == nullptr) return FA_ERR_HIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

size_t fa_bwd_noalloc_max_scratch_bytes(void) { return kScratchBytes; }

fa_status fa_bwd_noalloc(fa_dtype in_dtype, fa_dtype o_dtype, int64_t B, int64_t H, int64_t Lq,
                         int64_t Lk, int64_t d, const void* Q, const void* K, const void* V,
                         const void* O, const void* dO, const float* lse, float scale, int causal,
                         void* dQ, void* dK, void* dV, hipStream_t stream) {
  // The same checks as fa_bwd, in the same order, before the scratch
  // address is looked up: a call they reject makes no HIP call.
  if (!valid_dtype(in_dtype) || !valid_dtype(o_dtype) || !std::isfinite(scale)) return FA_ERR_ARG;
  if (fa_status st = check_shape(in_dtype, B, H, Lq, Lk, d)) return st;
  if (in_dtype == FA_F32 && o_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if (fa_bwd_workspace_bytes(in_dtype, B, H, Lq, Lk, d) > kScratchBytes) return FA_ERR_WORKSPACE;
  const bool has_q = B * H * Lq > 0, has_k = B * H * Lk > 0;
  if (!has_q && !has_k) return FA_OK;
  if (has_q && (!Q || !K || !V || !O || !dO || !lse || !dQ)) return FA_ERR_NULL;
  if (has_k && (!K || !V || !dK || !dV)) return FA_ERR_NULL;
  const void* ptrs[] = {Q, K, V, O, dO, lse, dQ, dK, dV};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FA_ERR_ALIGN;
  void* ws = nullptr;
  if (fa_status st = scratch_address(stream, &ws)) return st;
  return bwd_stages(fa::kBwdAll, in_dtype, o_dtype, B, H, Lq, Lk, d, Q, K, V, O, dO, lse, scale,
                    causal, dQ, dK, dV, ws, kScratchBytes, stream);
}

}  // extern "C"
