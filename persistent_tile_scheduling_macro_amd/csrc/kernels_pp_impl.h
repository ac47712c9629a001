// Instantiation of the ping-pong kernels of one element type; included by
// that type's ping-pong translation unit only (kernels_pp_*.hip).
#pragma once

#include "gemm_pingpong.h"
#include "kernels.h"

namespace pgemm {

template <int DT, int SCHED>
kernel_fn pick_pp(bool trace, bool bt) {
  if (bt) return trace ? pp::gemm_pp_kernel<DT, SCHED, true, true> : pp::gemm_pp_kernel<DT, SCHED, false, true>;
  return trace ? pp::gemm_pp_kernel<DT, SCHED, true, false> : pp::gemm_pp_kernel<DT, SCHED, false, false>;
}

template <int DT>
kernel_fn pick_pp_for_dtype(int sched, bool trace, bool bt) {
  switch (sched) {
    case kNonPersistent: return pick_pp<DT, kNonPersistent>(trace, bt);
    case kStatic: return pick_pp<DT, kStatic>(trace, bt);
    case kDynamic: return pick_pp<DT, kDynamic>(trace, bt);
    case kCancel: return pick_pp<DT, kCancel>(trace, bt);
    default: return nullptr;
  }
}

} // namespace pgemm
