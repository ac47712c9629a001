// Kernel selection across the per-dtype translation units.
#pragma once

#include "device_common.h"

namespace pgemm {

typedef void (*kernel_fn)(Params);

// Returns the kernel for (scheduling mode, fast or generic body).
kernel_fn pick_kernel_f16(int sched, bool fast);
kernel_fn pick_kernel_bf16(int sched, bool fast);
kernel_fn pick_kernel_f8(int sched, bool fast);

// K == 0: C = 0 (an empty sum). n = M * N output elements.
void launch_fill_zero(void* C, int64_t n, hipStream_t stream);

} // namespace pgemm
