// Instantiations of the producer-wave GEMM kernels for one element type.
#include "kernels_pw_impl.h"

namespace pgemm {

kernel_fn pick_kernel_pw_f8(int sched, bool trace, bool bt) { return pick_pw_for_dtype<kF8E4M3>(sched, trace, bt); }

} // namespace pgemm
