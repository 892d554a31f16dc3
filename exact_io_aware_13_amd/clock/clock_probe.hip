// Shader-clock probe for the benchmark (not part of the attention library):
// one wave spins for a given number of shader-clock cycles and records the
// shader cycle counter (s_memtime) and the constant 100 MHz real-time counter
// (s_memrealtime) at its start and end, so cycles / (ticks / 100 MHz) is the
// clock the chip ran at while the spin lasted -- alone, or beside other
// kernels on another stream.

#include <hip/hip_runtime.h>
#include <stdint.h>

__global__ __launch_bounds__(64) void clock_spin_kernel(unsigned long long* out,
                                                         long long cycles) {
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  unsigned long long t = t0;
  while ((long long)(t - t0) < cycles) t = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[0] = t0;
    out[1] = r0;
    out[2] = t;
    out[3] = r1;
  }
}

// Enqueues the spin on `stream`; `out` is 4 device uint64 values.  Returns
// the launch status (0 = hipSuccess).
extern "C" __attribute__((visibility("default"))) int fa_clock_spin(unsigned long long* out,
                                                                   long long cycles,
                                                                   hipStream_t stream) {
  if (!out || cycles <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(clock_spin_kernel, dim3(1), dim3(64), 0, stream, out, cycles);
  return (int)hipGetLastError();
}
