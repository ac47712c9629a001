// Instantiation of the producer-wave kernels of one element type; included by
// that type's producer-wave translation unit only (kernels_pw_*.hip).
#pragma once

#include "gemm_producer.h"
#include "kernels.h"

namespace pgemm {

template <int DT, int SCHED>
kernel_fn pick_pw(bool trace, bool bt) {
  if (bt) return trace ? pw::gemm_pw_kernel<DT, SCHED, true, true> : pw::gemm_pw_kernel<DT, SCHED, false, true>;
  return trace ? pw::gemm_pw_kernel<DT, SCHED, true, false> : pw::gemm_pw_kernel<DT, SCHED, false, false>;
}

template <int DT>
kernel_fn pick_pw_for_dtype(int sched, bool trace, bool bt) {
  switch (sched) {
    case kNonPersistent: return pick_pw<DT, kNonPersistent>(trace, bt);
    case kStatic: return pick_pw<DT, kStatic>(trace, bt);
    case kDynamic: return pick_pw<DT, kDynamic>(trace, bt);
    case kCancel: return pick_pw<DT, kCancel>(trace, bt);
    default: return nullptr;
  }
}

} // namespace pgemm
