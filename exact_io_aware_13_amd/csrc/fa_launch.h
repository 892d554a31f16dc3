// Internal launchers behind the C ABI.  Arguments are already validated by
// fa_api.hip; every launcher enqueues on `stream` and returns
// hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* lse;
  int BH, Lq, Lk, d;
  float scale;
  bool causal;
  bool out_f32;
  // Block-sparse forward (bf16 only): NULL for the dense forward.  Mask
  // [mask slices][nqb][nkb] of kSparseBlock x kSparseBlock (query, key)
  // blocks, nonzero = visible; bm_stride = nqb*nkb per slice, or 0 when one
  // mask serves every slice.
  const uint8_t* block_mask = nullptr;
  int bm_stride = 0, nqb = 0, nkb = 0;
};
constexpr int kSparseBlock = 128;
constexpr int kSparseMaxKeyBlocks = 4096;

struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  const float* lse;
  void* dQ;
  void* dK;
  void* dV;
  float* Dvec;   // [BH, Lq] row statistic (workspace; bf16 path: -D, fp32 path: D)
  float* lse2;   // [BH, Lq] lse * log2(e) (workspace)
  int BH, Lq, Lk, d;
  float scale;
  bool causal;
  bool o_f32 = false;  // O is fp32 (beside bf16 inputs); else the input dtype
  // Block-sparse backward (bf16 only), as in FwdArgs; NULL for the dense one.
  const uint8_t* block_mask = nullptr;
  int bm_stride = 0, nqb = 0, nkb = 0;
};

// Backward stages, run in this order by the launchers for the stages set in
// `stages`: per-row statistics (D, and lse in base 2 for bf16) into the
// workspace, then dK/dV, then dQ.  The last two only read the statistics
// and are independent of each other.  The bf16 launcher runs the first and
// the last in one kernel when both are requested (and O is bf16), before
// dK/dV.
enum : unsigned { kBwdPrepare = 1u, kBwdDkDv = 2u, kBwdDq = 4u, kBwdAll = 7u };

// Key-split forward (short query blocks, long key sequences).  Split s
// covers keys [s*chunk, min((s+1)*chunk, Lk)); chunk is a multiple of
// kSplitKvKeysPerTile.  Opart [nsplit, BH, Lq, d] and LSEpart
// [nsplit, BH, Lq] (fp32, workspace) hold each range's normalised output and
// natural-log lse; the merge writes O (o dtype) and lse.
struct SplitKvArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* lse;
  float* Opart;
  float* LSEpart;
  int BH, Lq, Lk, d;
  int nsplit, chunk;
  float scale;
  bool causal;
  bool out_f32;
};
enum : unsigned { kSplitKvPartial = 1u, kSplitKvMerge = 2u, kSplitKvAll = 3u };
constexpr int kSplitKvKeysPerTile = 64;
constexpr int kSplitKvRowsPerBlock = 16;

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdArgs& a, unsigned stages, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_f32(const BwdArgs& a, unsigned stages, hipStream_t stream);
hipError_t launch_splitkv_bf16(const SplitKvArgs& a, unsigned stages, hipStream_t stream);

// Work decomposition shared by validation and the launchers.
constexpr int kComputeUnits = 256;  // MI355X (gfx950)
constexpr int kFwdBf16RowsPerBlock = 256;
constexpr int kBf16MinRowsPerBlock = 128;  // fewest query or key rows of any bf16 workgroup
constexpr int kBwdBf16KeysPerBlock = 128;
constexpr int kF32RowsPerBlock = 8;        // fewest rows of an fp32 workgroup (d = 128)

}  // namespace fa
