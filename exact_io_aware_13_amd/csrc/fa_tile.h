// LDS tile helpers shared by the bf16 matrix-core kernels: chunk swizzle,
// plain and transposing LDS fragment reads, wait-count and barrier
// primitives, compile-time loops, and the wave-half exchange.  Internal to
// libfa.
#pragma once

#include "fa_device.h"

#include <type_traits>

namespace fa {

// Chunk swizzle: bijective on the row index mod 16 (d=128) or on row/2 mod 8
// (d=64), and spreads the 4 rows of a transposed read over all banks.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ u32x4 lds_read16(const char* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr(const char* base, int off) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(base + off));
  return __builtin_bit_cast(u32x2, v);
}

// s_waitcnt vmcnt(N) leaving expcnt and lgkmcnt unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

// Workgroup barrier that leaves buffer loads in flight: completes this wave's
// LDS reads (lgkmcnt(0)), then s_barrier.  The empty asm statements keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int N>
using IC = std::integral_constant<int, N>;

// Pins a value at this point of the instruction stream: the empty asm
// "modifies" it, so it must be computed before and cannot be sunk past it.
// Keeps the hand-placed softmax work between the matrix products it is meant
// to overlap (scheduling barriers alone do not stop code sinking).
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(unsigned& x) { asm volatile("" : "+v"(x)); }

// Calls f(IC<B>{}), ..., f(IC<E-1>{}): loop bodies with compile-time indices,
// so register arrays are never indexed at run time.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(IC<B>{});
    static_for<B + 1, E>(f);
  }
}

// Whole-row stores of one wave's 32 output rows of D bf16 columns held in
// the 32x32 accumulator layout: lane (n = lane % 32, h = lane / 32) holds,
// for each 32-wide column block db and group g, the 8-byte piece v[db][g] =
// columns 32db + 8g + 4h .. +3 of row n.  Stored directly, each store
// instruction would write 16 bytes into each of 32 rows.  The wave instead
// writes the pieces to its own LDS staging area st (32 * 2D bytes, not read
// by any other wave) and stores whole rows, 1 KiB per instruction, to rows
// row0 .. row0 + 31 of the buffer r (rows past its range are dropped by the
// range check).  It reads back only what it wrote, so no barrier is needed.
// Staging layout: 8-byte slot s of row r at slot s ^ x(r), x(r) = (r / rows
// per 256-byte bank line) mod slots per row, which spreads the 32 lanes of
// a write over all banks; a 16-byte chunk c then sits at chunk c ^ (x >> 1),
// its halves swapped when x is odd.
template <int D>
__device__ __forceinline__ void store_rows_staged(char* st, int lane, const u32x2 (&v)[D / 32][4],
                                                  __amdgpu_buffer_rsrc_t r, int row0) {
  constexpr int ROWB = 2 * D;           // bytes per row
  constexpr int SLOTS = D / 4;          // 8-byte slots per row
  constexpr int RPL = 256 / ROWB;       // rows per 256-byte bank line
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int RPK = 1024 / ROWB;      // rows per 1-KiB store instruction
  const int n = lane & 31, h = lane >> 5;
  const int xw = (n / RPL) & (SLOTS - 1);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<u32x2*>(st + n * ROWB + (((8 * db + 2 * g + h) ^ xw) << 3)) = v[db][g];
#pragma unroll
  for (int i = 0; i < 32 * ROWB / 1024; ++i) {
    const int rr = i * RPK + lane / CPR, cl = lane % CPR;
    const int xr = (rr / RPL) & (SLOTS - 1);
    u32x4 a = *reinterpret_cast<const u32x4*>(st + rr * ROWB + ((cl ^ (xr >> 1)) << 4));
    if (xr & 1) a = u32x4{a.z, a.w, a.x, a.y};
    store16(r, (uint32_t)((row0 + rr) * D + cl * 8) * 2, a);
  }
}

// Row max / row sum across the two wave halves (lanes l and l ^ 32 hold the
// two halves of one query row).  v_permlane32_swap exchanges the upper 32
// lanes of its first operand with the lower 32 lanes of its second; applied
// to two copies of x, every lane ends up with its own value in one register
// and its partner's in the other.  Issued as a single VALU instruction in
// asm: given identical operands, the compiler otherwise treats the two
// results of the builtin as equal and drops one.
__device__ __forceinline__ void halves_pair(float x, float& a, float& b) {
  a = x;
  b = x;
  // The nops give the wait states a VALU write needs before the swap reads
  // it (the compiler cannot see hazards inside asm).
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float halves_max(float x) {
  float a, b;
  halves_pair(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float halves_sum(float x) {
  float a, b;
  halves_pair(x, a, b);
  return a + b;
}

}  // namespace fa
