// Instantiations of the GEMM kernels for one element type.
#include "gemm_fast.h"
#include "gemm_generic.h"
#include "kernels.h"

namespace pgemm {

kernel_fn pick_kernel_bf16(int sched, bool fast) {
  switch (sched) {
    case kNonPersistent:
      return fast ? fast::gemm_fast_kernel<kBF16, kNonPersistent> : generic::gemm_generic_kernel<kBF16, kNonPersistent>;
    case kStatic:
      return fast ? fast::gemm_fast_kernel<kBF16, kStatic> : generic::gemm_generic_kernel<kBF16, kStatic>;
    default:
      return fast ? fast::gemm_fast_kernel<kBF16, kDynamic> : generic::gemm_generic_kernel<kBF16, kDynamic>;
  }
}

} // namespace pgemm
