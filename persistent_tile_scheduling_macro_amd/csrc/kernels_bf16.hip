// Instantiations of the GEMM kernels for one element type.
#include "kernels_impl.h"

namespace pgemm {

kernel_fn pick_kernel_bf16(int sched, int body) { return pick_for_dtype<kBF16>(sched, body); }

} // namespace pgemm
