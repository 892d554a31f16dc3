// Device-side building blocks for the gfx950 attention kernels: vector
// types, bounds-checked buffer loads/stores, bf16 packing and the bf16
// matrix-core product.  Internal to libfa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Workgroup and work-item index read straight from the hardware registers.
// The blockIdx/threadIdx accessors go through small library functions that
// the inliner may leave out of line in a large kernel; their results then
// count as per-lane values, and every buffer descriptor derived from the
// workgroup index turns into a per-lane loop around each buffer access.
__device__ __forceinline__ int wg_id() { return (int)__builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ int wi_id() { return (int)__builtin_amdgcn_workitem_id_x(); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Buffer resource over [base, base + bytes): loads past the end return zero
// and stores past the end are dropped by the hardware range check.  This is
// how ragged tails (L not a multiple of the tile) are handled without
// branches.  Word 3 selects a raw 32-bit-format buffer on gfx9-family parts.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
__device__ __forceinline__ u32x2 load8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0));
}
__device__ __forceinline__ float load4f(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}
__device__ __forceinline__ void store16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, byte_off, 0, 0);
}
__device__ __forceinline__ void store8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, v), r, byte_off, 0, 0);
}
__device__ __forceinline__ void store4f(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), r, byte_off, 0, 0);
}

// fp32 -> bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32), two at a
// time; element a lands in the low half.
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(unsigned, v);
}
__device__ __forceinline__ float bf16_lo(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// D += A * B on the bf16 matrix cores, 32x32 output tile, 16-deep.
// Lane l supplies A[m = l%32][8 k-slots of half l/32] and B[same k-slots][n = l%32];
// the result holds, in lane l and register r, D[m = 8*(r/4) + 4*(l/32) + r%4][n = l%32].
__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Value held by lane l ^ 32.
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace fa
