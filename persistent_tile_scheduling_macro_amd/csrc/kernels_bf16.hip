// Instantiations of the GEMM kernels for one element type.
#include "kernels_impl.h"

namespace pgemm {

kernel_fn pick_kernel_bf16(int sched, int body, bool trace, bool bt) {
  return pick_for_dtype<kBF16>(sched, body, trace, bt);
}
kernel_fn pick_fixup_bf16(int body) { return pick_fixup_for_dtype<kBF16>(body); }

} // namespace pgemm
