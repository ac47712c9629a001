// Instantiations of the GEMM kernels for one element type.
#include "kernels_impl.h"

namespace pgemm {

kernel_fn pick_kernel_f16(int sched, int body, bool trace, bool bt) {
  return pick_for_dtype<kF16>(sched, body, trace, bt);
}
kernel_fn pick_fixup_f16(int body) { return pick_fixup_for_dtype<kF16>(body); }

} // namespace pgemm

namespace pgemm {
// Both output types are 16 bits wide and +0.0 is all-zero bits in both.
void launch_fill_zero(void* C, int64_t rows, int64_t cols, int64_t ldc, hipStream_t stream) {
  const int64_t n = rows * cols;
  const int blocks = (int)(n / 256 + 1 < 4096 ? n / 256 + 1 : 4096);
  hipLaunchKernelGGL(generic::fill_zero_kernel<_Float16>, dim3(blocks), dim3(256), 0, stream,
                     reinterpret_cast<_Float16*>(C), rows, cols, ldc);
}
} // namespace pgemm
