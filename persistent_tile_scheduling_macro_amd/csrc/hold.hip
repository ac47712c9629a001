// Benchmark aid: hold a number of CUs for a bounded time, so the tile
// schedulers can be measured when only part of the GPU is available (the
// case where the CUs actually available differ from the static
// assumption, KernelWiki "Persistent Kernels with Cluster Launch Control",
// "Choosing between static and CLC scheduling").
//
// Each workgroup allocates the whole 160 KiB of its CU's LDS, so no other
// workgroup that uses LDS (every GEMM workgroup does) can share that CU
// while it runs, and idles in s_sleep until the device's constant-rate
// clock (s_memrealtime) has advanced by `ticks`. The pass count is capped
// as well: each pass sleeps at least 127 x 64 cycles, so `ticks / 64 + 16`
// passes cover the wait at any clock rate the chip runs at, and the kernel
// ends even if the clock counter did not advance.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pgemm {

__global__ void __launch_bounds__(64) hold_cu_kernel(uint64_t ticks) {
  __shared__ __attribute__((aligned(16))) uint8_t hold[160 * 1024];
  asm volatile("" ::"v"(&hold[threadIdx.x]));  // keep the allocation
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t cap = ticks / 64 + 16;
  for (uint64_t i = 0; i < cap; ++i) {
    if (__builtin_amdgcn_s_memrealtime() - t0 >= ticks) break;
    __builtin_amdgcn_s_sleep(127);
  }
}

void launch_hold(int n, uint64_t ticks, hipStream_t stream) {
  hipLaunchKernelGGL(hold_cu_kernel, dim3(n), dim3(64), 0, stream, ticks);
}

} // namespace pgemm
