// Kernel selection across the per-dtype translation units.
#pragma once

#include "device_common.h"

namespace pgemm {

typedef void (*kernel_fn)(Params);

// Tile body of a launch: the fast kernel in one of its two macro-tile
// configurations (lockstep waves), the 256 x 256 ping-pong form of the fast
// kernel (gemm_pingpong.h), the 256 x 128 producer-wave form (copy waves and
// MFMA waves, gemm_producer.h), or the generic 64 x 64 body for unaligned
// operands.
enum Body : int { kBodyGeneric = 0, kBodyTile256 = 1, kBodyTile128 = 2, kBodyPingPong = 3, kBodyProducer = 4 };
constexpr int kNumBodies = 5;

// Returns the kernel for (scheduling mode, tile body); `trace` selects the
// fast bodies' instantiation that writes the tile trace, `bt` the one that
// takes B as N x K (the generic body reads Params::b_nk instead).
kernel_fn pick_kernel_f16(int sched, int body, bool trace, bool bt);
kernel_fn pick_kernel_bf16(int sched, int body, bool trace, bool bt);
kernel_fn pick_kernel_f8(int sched, int body, bool trace, bool bt);

// The ping-pong 256 x 256 kernel for the non-persistent, static, dynamic and
// cancel-and-reuse modes (kernels_pp_*.hip); nullptr for stream-K, whose
// tail launch takes the lockstep 256 x 256 body.
kernel_fn pick_kernel_pp_f16(int sched, bool trace, bool bt);
kernel_fn pick_kernel_pp_bf16(int sched, bool trace, bool bt);
kernel_fn pick_kernel_pp_f8(int sched, bool trace, bool bt);

// The producer-wave 256 x 128 kernel for the same four modes (kernels_pw_*.hip);
// nullptr for stream-K, which that body does not serve.
kernel_fn pick_kernel_pw_f16(int sched, bool trace, bool bt);
kernel_fn pick_kernel_pw_bf16(int sched, bool trace, bool bt);
kernel_fn pick_kernel_pw_f8(int sched, bool trace, bool bt);

// The stream-K fix-up kernel of a fast tile body (nullptr for the generic body).
kernel_fn pick_fixup_f16(int body);
kernel_fn pick_fixup_bf16(int body);
kernel_fn pick_fixup_f8(int body);

// K == 0: C = 0 (an empty sum), rows x cols elements with rows ldc elements apart.
void launch_fill_zero(void* C, int64_t rows, int64_t cols, int64_t ldc, hipStream_t stream);

// Benchmark aid (hold.hip): n workgroups that each hold a whole CU's LDS
// until the constant-rate clock has advanced by `ticks`.
void launch_hold(int n, uint64_t ticks, hipStream_t stream);

} // namespace pgemm
