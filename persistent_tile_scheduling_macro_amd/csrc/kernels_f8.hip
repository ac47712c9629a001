// Instantiations of the GEMM kernels for one element type.
#include "kernels_impl.h"

namespace pgemm {

kernel_fn pick_kernel_f8(int sched, int body, bool trace, bool bt) {
  return pick_for_dtype<kF8E4M3>(sched, body, trace, bt);
}
kernel_fn pick_fixup_f8(int body) { return pick_fixup_for_dtype<kF8E4M3>(body); }

} // namespace pgemm
