// Instantiations of the GEMM kernels for one element type.
#include "gemm_fast.h"
#include "gemm_generic.h"
#include "kernels.h"

namespace pgemm {

kernel_fn pick_kernel_f16(int sched, bool fast) {
  switch (sched) {
    case kNonPersistent:
      return fast ? fast::gemm_fast_kernel<kF16, kNonPersistent> : generic::gemm_generic_kernel<kF16, kNonPersistent>;
    case kStatic:
      return fast ? fast::gemm_fast_kernel<kF16, kStatic> : generic::gemm_generic_kernel<kF16, kStatic>;
    default:
      return fast ? fast::gemm_fast_kernel<kF16, kDynamic> : generic::gemm_generic_kernel<kF16, kDynamic>;
  }
}

} // namespace pgemm

namespace pgemm {
// Both output types are 16 bits wide and +0.0 is all-zero bits in both.
void launch_fill_zero(void* C, int64_t n, hipStream_t stream) {
  const int blocks = (int)(n / 256 + 1 < 4096 ? n / 256 + 1 : 4096);
  hipLaunchKernelGGL(generic::fill_zero_kernel<_Float16>, dim3(blocks), dim3(256), 0, stream,
                     reinterpret_cast<_Float16*>(C), n);
}
} // namespace pgemm
