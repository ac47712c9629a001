// Instantiation of every (scheduling mode, tile body) kernel of one element
// type; included by that type's translation unit only.
#pragma once

#include "gemm_fast.h"
#include "gemm_generic.h"
#include "kernels.h"

namespace pgemm {

template <int DT, int SCHED, int CFG>
kernel_fn pick_fast(bool trace, bool bt) {
  if (bt)
    return trace ? fast::gemm_fast_kernel<DT, SCHED, CFG, true, true> : fast::gemm_fast_kernel<DT, SCHED, CFG, false, true>;
  return trace ? fast::gemm_fast_kernel<DT, SCHED, CFG, true, false> : fast::gemm_fast_kernel<DT, SCHED, CFG, false, false>;
}

template <int DT, int SCHED>
kernel_fn pick_body(int body, bool trace, bool bt) {
  switch (body) {
    case kBodyTile256: return pick_fast<DT, SCHED, fast::kTile256>(trace, bt);
    case kBodyTile128: return pick_fast<DT, SCHED, fast::kTile128>(trace, bt);
    default: // the generic body has no stream-K split: it runs that mode as static
      return generic::gemm_generic_kernel<DT, SCHED == kStreamK ? kStatic : SCHED>;
  }
}

template <int DT>
kernel_fn pick_for_dtype(int sched, int body, bool trace, bool bt) {
  switch (sched) {
    case kNonPersistent: return pick_body<DT, kNonPersistent>(body, trace, bt);
    case kStatic: return pick_body<DT, kStatic>(body, trace, bt);
    case kDynamic: return pick_body<DT, kDynamic>(body, trace, bt);
    case kCancel: return pick_body<DT, kCancel>(body, trace, bt);
    default: return pick_body<DT, kStreamK>(body, trace, bt);
  }
}

template <int DT>
kernel_fn pick_fixup_for_dtype(int body) {
  switch (body) {
    case kBodyTile256: return fast::sk_fixup_kernel<DT, fast::kTile256>;
    case kBodyTile128: return fast::sk_fixup_kernel<DT, fast::kTile128>;
    default: return nullptr;
  }
}

} // namespace pgemm
