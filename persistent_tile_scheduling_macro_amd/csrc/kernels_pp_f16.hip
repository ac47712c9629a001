// Instantiations of the ping-pong GEMM kernels for one element type.
#include "kernels_pp_impl.h"

namespace pgemm {

kernel_fn pick_kernel_pp_f16(int sched, bool trace, bool bt) { return pick_pp_for_dtype<kF16>(sched, trace, bt); }

} // namespace pgemm
