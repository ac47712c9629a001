// Instantiations of the GEMM kernels for one element type.
#include "gemm_fast.h"
#include "gemm_generic.h"
#include "kernels.h"

namespace pgemm {

kernel_fn pick_kernel_f8(int sched, bool fast) {
  switch (sched) {
    case kNonPersistent:
      return fast ? fast::gemm_fast_kernel<kF8E4M3, kNonPersistent> : generic::gemm_generic_kernel<kF8E4M3, kNonPersistent>;
    case kStatic:
      return fast ? fast::gemm_fast_kernel<kF8E4M3, kStatic> : generic::gemm_generic_kernel<kF8E4M3, kStatic>;
    default:
      return fast ? fast::gemm_fast_kernel<kF8E4M3, kDynamic> : generic::gemm_generic_kernel<kF8E4M3, kDynamic>;
  }
}

} // namespace pgemm
