// Producer-wave form of the fast tile body: a workgroup of eight waves in
// which four waves (4-7) only copy operand tiles global -> LDS and claim
// tiles, and four waves (0-3) only read fragments and run MFMAs -- the
// dedicated load warp of warp specialisation, and the producer side of a
// scheduler pipeline that requests the next work id ahead of its consumers
// (KernelWiki "Persistent Kernels with Cluster Launch Control", "Retained
// implementation excerpt" and the note under "Choosing between static and
// CLC scheduling").
//
// Shape. On CDNA every wave of a workgroup is given the same register
// budget, so a copy-only wave holds as many registers as an MFMA wave. At
// two waves per SIMD (256 registers per wave) a 256 x 256 tile needs all
// eight waves as MFMA waves (128 accumulators each); with four of them
// copying instead, the tile that fits is 256 x 128: each MFMA wave owns the
// same 128 x 64 sub-tile (8 x 4 blocks of 16 x 16) as in the 256 x 256
// bodies, arranged 2 x 2, and each SIMD runs one MFMA wave and one copy
// wave (waves w and w + 4 share a SIMD). A step moves 32 KiB of A and
// 16 KiB of B for half the flops of a 256 x 256 step, so this body needs
// 1.5 times the copy bandwidth per flop of the 256 x 256 bodies.
//
// LDS: three stages of 48 KiB (A: 256 rows of 128 bytes, B: 64 or 128 rows
// of 256 or 128 bytes, or 128 rows of 128 bytes when B is N x K), with the
// swizzles of the other fast bodies: A as in the 256 x 256 tile, B as in the
// 128 x 128 tile (both 64-column MFMA-wave layouts), so the fragment reads
// are bank-conflict-free and the MFMAs see the same operands in the same
// order -- C is bitwise the same as the other bodies'.
//
// Pipeline. Barrier j of a workgroup (j = 0, 1, ...) is passed once the
// copy of k-step j has landed, and once the MFMA waves have finished reading
// stage (j - 1) mod 3; after it the copy waves issue step j + 2 into that
// stage. The MFMA waves meet barrier j + 1 in the middle of step j (16-bit
// types: between the step's two MFMA k-groups, with the second k-group's
// fragments already in registers) or at its end (e4m3, one k-group per
// step). So each copy has two barrier intervals to land, and no MFMA wave
// ever issues a copy.
//
// Steps are counted over the workgroup's flattened (tile, k-step) sequence,
// so the copy waves run into the next tile while the MFMA waves store the
// current one. Tile sequences are the other bodies' (non-persistent, static,
// dynamic, cancel-and-reuse); the stream-K mode is not offered in this body.
// Claims are made by the copy waves' thread 256: the claim for tile q + 1 is
// issued just before the copies of tile q's second k-step (its fourth for
// cancel-and-reuse's first tile when a tile has four or more steps, so that
// no early workgroup takes a second tile before the late ones took a first)
// and written to the LDS ring after the copy waves' next wait, which the
// next barrier publishes. The copies of tile q + 1 begin two barriers later
// at the earliest, and the MFMA waves read the entry at the end of tile q.
#pragma once

#include "gemm_fast.h"

namespace pgemm {
namespace pw {

using fast::b_swz;
using fast::block_k;
using fast::Frag;
using fast::read_a;
using fast::read_b;
using fast::static_for;
using fast::wait_vmcnt;

// s_waitcnt lgkmcnt(0) (vmcnt and expcnt left at their maxima)
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// A workgroup barrier without a memory fence: each side waits for exactly
// the counters it needs first.
__device__ inline void barrier_raw() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

template <int DT, int SCHED, bool TRACE, bool BT>
__global__ void __launch_bounds__(512, 2) gemm_pw_kernel(Params p) {
  static_assert(SCHED == kNonPersistent || SCHED == kStatic || SCHED == kDynamic || SCHED == kCancel,
                "the producer-wave body serves the four tile-sequence modes, not stream-K");
  constexpr int BM = 256, BN = 128;
  constexpr int MB = 8, WN = 64, NB = 4;       // an MFMA wave's 128 x 64 sub-tile
  constexpr int ES = Traits<DT>::esize;
  constexpr int BK = block_k(ES);
  constexpr int KSUB = BK / Traits<DT>::kgroup; // MFMA k-groups per step (2, or 1 for e4m3)
  constexpr int A_ROW = 128;
  constexpr int A_BYTES = BM * A_ROW;           // 32 KiB
  constexpr int B_ROW = BT ? A_ROW : BN * ES;   // bytes per B row in LDS
  constexpr int B_BYTES = BT ? BN * A_ROW : BK * B_ROW;
  static_assert(B_BYTES == 16 * 1024, "16 B blocks of 1 KiB per step");
  constexpr int B_CPR = B_ROW / 16;
  constexpr int B_RPI = 1024 / B_ROW;           // B rows per 1 KiB copy block
  constexpr int STAGE = A_BYTES + B_BYTES;      // 48 KiB
  constexpr int LA = 8, LB = 4;                 // copy instructions per copy wave per step
  constexpr int L = LA + LB;
  typedef typename Traits<DT>::out_t out_t;
  typedef typename Frag<DT>::t frag_t;

  __shared__ __attribute__((aligned(1024))) uint8_t smem[3 * STAGE];
  __shared__ int s_ring[8]; // claiming modes: tile id of tile-sequence number q at q % 8

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = p.M, N = p.N, K = p.K, T = p.T, G = p.G;
  const int nk = ((K + BK - 1) / BK + 1) & ~1; // even, >= 2 (K >= 1)
  const int64_t lda = (int64_t)p.lda * ES;
  const int64_t ldb = (int64_t)p.ldb * ES;
  const int64_t ldc = p.ldc;

  // ---- the tile sequence --------------------------------------------------
  constexpr bool CLAIMS = SCHED == kDynamic || SCHED == kCancel;
  auto tile_of = [&](int q) __attribute__((always_inline)) -> int {
    if constexpr (SCHED == kNonPersistent) {
      return q == 0 ? (int)blockIdx.x : T;
    } else if constexpr (SCHED == kStatic) {
      const int64_t t = (int64_t)blockIdx.x + (int64_t)q * G;
      return t < T ? (int)t : T;
    } else {
      return __builtin_amdgcn_readfirstlane(s_ring[q & 7]);
    }
  };
  // k-step of tile q at which the claim for tile q + 1 is issued
  const bool defer_t1 = SCHED == kCancel && nk >= 4;
  auto claim_step = [&](int q) __attribute__((always_inline)) -> int { return (defer_t1 && q == 0) ? 3 : 1; };
  bool claim_live = false; // thread 256: the last claim got a tile
  if constexpr (CLAIMS) {
    if (tid == 256) {
      int t0 = (int)blockIdx.x;
      if constexpr (SCHED == kCancel) {
        t0 = claim_tile(p.counter, T, claim_offset<SCHED>(G), claim_total<SCHED>(T, G));
        claim_live = t0 < T;
      } else {
        // dynamic with G >= T: no tile lies beyond the grid's own, so no claim is made at all
        claim_live = G < T;
        if (!claim_live) s_ring[1] = T;
      }
      s_ring[0] = t0;
    }
    __syncthreads();
    if constexpr (SCHED == kCancel) {
      if ((unsigned)tile_of(0) >= (unsigned)T) return; // found no tile: the whole workgroup leaves at once
    }
  }

  if (wave >= 4) {
    // =========================== copy waves =====================================
    const int pw = wave - 4;
    // A: block q = pw + 4j (j < 8) holds rows 8q..8q+7; the lane fetches row
    // 8q + lane/8, the chunk the swizzle stores at lane % 8.
    const int a_row0 = 8 * pw + (lane >> 3);
    int a_chunk;
    if constexpr (ES == 2) {
      a_chunk = (lane & 7) ^ (lane >> 3);
    } else {
      const int r = lane >> 3;
      a_chunk = (lane & 7) ^ (((r >> 1) & 1) | (r & 4));
    }
    // B: block q = pw + 4j (j < 4) holds B rows B_RPI*q..; with N x K B the rows are n,
    // copied like A's. The K x N chunk also takes the rows' swizzle term, an XOR of
    // single row bits: the part from the block's row offset is a per-instruction constant.
    const int b_row0 = BT ? 8 * pw + (lane >> 3) : B_RPI * pw + lane / B_CPR;
    const int b_chunk0 = BT ? a_chunk : (lane % B_CPR) ^ b_swz<ES, B_ROW>(B_RPI * pw + lane / B_CPR);
    const uint32_t a_vbase = (uint32_t)a_row0 * (uint32_t)lda + 16u * (uint32_t)a_chunk;

    int u_q = 0, u_kt = 0; // tile sequence number and k-step of the next step to copy
    int issued = 0;        // steps copied so far
    bool u_done = false;   // the tile sequence has ended
    const uint8_t* u_a = nullptr;
    const uint8_t* u_b = nullptr;
    int u_m0 = 0, u_n0 = 0;
    int c_raw = 0, c_slot = 0; // thread 256: a claim in flight and the ring slot it fills
    bool c_pending = false;
    // copy of the next step into stage `stage`; returns false once the sequence has ended
    auto issue = [&](int stage) __attribute__((always_inline)) -> bool {
      if (u_done) return false;
      if (u_kt == 0) {
        const int t = tile_of(u_q);
        if ((unsigned)t >= (unsigned)T) { // any id outside [0, T) ends the sequence
          u_done = true;
          return false;
        }
        int pm, pn;
        tile_coords(t, p, &pm, &pn);
        u_m0 = pm * BM;
        u_n0 = pn * BN;
        u_a = p.A + (int64_t)u_m0 * lda;
        u_b = BT ? p.B + (int64_t)u_n0 * ldb : p.B + (int64_t)u_n0 * ES;
      }
      if constexpr (CLAIMS) {
        // issued ahead of this step's copies, so the wait that follows them covers it
        if (tid == 256 && claim_live && u_kt == claim_step(u_q)) {
          c_raw = claim_raw(p.counter);
          c_slot = u_q + 1;
          c_pending = true;
        }
      }
      const int m0 = u_m0, n0 = u_n0, k0 = u_kt * BK;
      int lda_s = (int)lda, ldb_s = (int)ldb, pw_s = pw * 1024, st_s = stage * STAGE;
      asm volatile("" : "+s"(lda_s), "+s"(ldb_s), "+s"(pw_s), "+s"(st_s));
      uint8_t* sA = smem + st_s;
      uint8_t* sB = smem + st_s + A_BYTES;
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(u_a + (int64_t)k0 * ES);
      const __amdgpu_buffer_rsrc_t rb = BT ? make_rsrc(u_b + (int64_t)k0 * ES) : make_rsrc(u_b + (int64_t)k0 * ldb);
      const int mrem = M - m0, krem = K - k0;
      const int nrem = BT ? N - n0 : (N - n0) * ES;
      const bool full = (mrem >= BM) & (krem >= BK) & (BT ? nrem >= BN : nrem >= BN * ES);
      const bool kval = full || (k0 * ES + 16 * a_chunk) < K * ES;
      static_for<LA>([&](auto jc) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value; // block pw + 4J: rows +32J
        const bool ok = full || (kval & (a_row0 + 32 * J < mrem));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, PGEMM_LDS(void, sA + 4 * J * 1024 + pw_s), 16, ok ? a_vbase : kOOB,
                                                 32 * J * lda_s, 0, 0);
      });
      static_for<LB>([&](auto jc) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;
        if constexpr (BT) {
          const bool ok = full || (kval & (b_row0 + 32 * J < nrem));
          const uint32_t base = (uint32_t)b_row0 * (uint32_t)ldb + 16u * (uint32_t)b_chunk0;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, PGEMM_LDS(void, sB + 4 * J * 1024 + pw_s), 16, ok ? base : kOOB,
                                                   32 * J * ldb_s, 0, 0);
        } else {
          constexpr int SW = b_swz<ES, B_ROW>(4 * B_RPI * J);
          const int Lc = b_chunk0 ^ SW;
          const bool ok = full || ((b_row0 + 4 * B_RPI * J < krem) & (16 * Lc < nrem));
          const uint32_t base = (uint32_t)b_row0 * (uint32_t)ldb + 16u * (uint32_t)Lc;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, PGEMM_LDS(void, sB + 4 * J * 1024 + pw_s), 16, ok ? base : kOOB,
                                                   4 * B_RPI * J * ldb_s, 0, 0);
        }
      });
      if (++u_kt == nk) {
        u_kt = 0;
        ++u_q;
      }
      ++issued;
      return true;
    };
    // after a wait that covers the claim in flight: write its result to the ring
    auto publish = [&]() __attribute__((always_inline)) {
      if constexpr (CLAIMS) {
        if (tid == 256 && c_pending) {
          const int t = claim_finish(p.counter, c_raw, T, claim_offset<SCHED>(G), claim_total<SCHED>(T, G));
          s_ring[c_slot & 7] = t;
          claim_live = t < T;
          c_pending = false;
        }
        wait_lgkm0();
      }
    };

    // steps 0 and 1 (one tile: nk >= 2), then barrier 0 once step 0 has landed
    issue(0);
    issue(1);
    wait_vmcnt<L>();
    publish();
    barrier_raw();
    int st = 2; // stage of step j + 2
    for (int j = 0;; ++j) {
      const bool more = issue(st);
      st = st == 2 ? 0 : st + 1;
      if (j + 1 >= issued) break; // step j was the last: no barrier j + 1
      if (more)
        wait_vmcnt<L>(); // step j + 1 has landed (and any claim issued before step j + 2's copies)
      else
        wait_vmcnt<0>();
      publish();
      barrier_raw();
    }
    return;
  }

  // ============================= MFMA waves =========================================
  const int wm = wave >> 1, wn = wave & 1; // 2 x 2 waves of 128 x 64
  const int g = lane >> 4, s16 = lane & 15;
  int a_off[KSUB][2];
#pragma unroll
  for (int kk = 0; kk < KSUB; ++kk) {
    const int r = wm * 128 + s16; // + mb * 16
    if constexpr (ES == 2) {
      a_off[kk][0] = r * A_ROW + 16 * ((4 * kk + g) ^ (s16 & 7));
      a_off[kk][1] = a_off[kk][0];
    } else {
      const int sw = ((s16 >> 1) & 1) | (s16 & 4);
      a_off[kk][0] = r * A_ROW + 16 * ((2 * g) ^ sw);
      a_off[kk][1] = r * A_ROW + 16 * ((2 * g + 1) ^ sw);
    }
  }
  int b_off[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if constexpr (BT) {
      if constexpr (ES == 2) {
        const int q = s16 >> 2;
        const int r = wn * WN + 32 * (nb >> 1) + 8 * q + 4 * ((nb + q) & 1) + (s16 & 3);
        b_off[nb] = r * A_ROW + 16 * (g ^ (r & 7));
      } else {
        const int r = wn * WN + nb * 16 + s16;
        b_off[nb] = r * A_ROW + 16 * ((2 * g) ^ (((r >> 1) & 1) | (r & 4)));
      }
    } else if constexpr (ES == 2) {
      const int k = 8 * g + (s16 >> 2);
      const int q = s16 & 3;
      const int Lc = wn * (WN / 8) + 4 * (nb >> 1) + q;
      b_off[nb] = k * B_ROW + 16 * (Lc ^ b_swz<ES, B_ROW>(k)) + 8 * ((nb + q) & 1);
    } else {
      const int k = 32 * g + (s16 >> 1);
      const int Lc = wn * (WN / 16) + nb;
      b_off[nb] = k * B_ROW + 16 * (Lc ^ b_swz<ES, B_ROW>(k)) + 8 * (s16 & 1);
    }
  }

  floatx4_t acc[MB][NB];
  frag_t af[2][MB], bf[2][NB];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    acc_drain();
  };
  auto stage_ptr = [&](int c) __attribute__((always_inline)) -> const uint8_t* {
    int off = c * STAGE;
    asm volatile("" : "+s"(off));
    return smem + off;
  };
  auto read_a_frag = [&](auto f, const uint8_t* sA, int kk, int mb) __attribute__((always_inline)) {
    constexpr int F = decltype(f)::value;
    af[F][mb] = read_a<DT>(sA + a_off[kk][0] + mb * 16 * A_ROW, sA + a_off[kk][1] + mb * 16 * A_ROW);
  };
  auto read_b_frag = [&](auto f, const uint8_t* sB, int kk, int nb) __attribute__((always_inline)) {
    constexpr int F = decltype(f)::value;
    if constexpr (BT) {
      if constexpr (ES == 2)
        bf[F][nb] = read_a<DT>(sB + (b_off[nb] ^ (64 * kk)), nullptr);
      else
        bf[F][nb] = read_a<DT>(sB + b_off[nb], sB + (b_off[nb] ^ 16));
    } else {
      bf[F][nb] = read_b<DT, B_ROW>(sB + b_off[nb] + kk * 32 * B_ROW);
    }
  };
  auto mfma_row = [&](auto f, int mb) __attribute__((always_inline)) {
    constexpr int F = decltype(f)::value;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) mfma_acc(acc[mb][nb], bf[F][nb], af[F][mb]);
  };
  typedef std::integral_constant<int, 0> I0;
  typedef std::integral_constant<int, 1> I1;

  long long t_begin = 0; // tile trace: when the current tile began

  // ---- epilogue: this wave's 128 x 64 block of the tile, rounded and stored --------
  auto epilogue = [&](int tile) __attribute__((always_inline)) {
    acc_drain();
    int pm, pn;
    tile_coords(tile, p, &pm, &pn);
    const int mrow = pm * BM + wm * 128 + s16;
    out_t* C = reinterpret_cast<out_t*>(p.C);
    if constexpr (ES == 2) {
      const int ncol8 = pn * BN + wn * WN + 8 * g;
      const bool odd = (g & 1) != 0;
      out_t* crow = C + (int64_t)mrow * ldc + ncol8;
      if ((pm * BM + BM <= M) & (pn * BN + BN <= N)) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          out_t* dst = crow + (int64_t)(16 * mb) * ldc;
#pragma unroll
          for (int P = 0; P < NB / 2; ++P)
            store8(dst + 32 * P, acc_read(acc[mb][2 * P]), acc_read(acc[mb][2 * P + 1]), odd);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          if (mrow + mb * 16 < M) {
            out_t* dst = crow + (int64_t)(16 * mb) * ldc;
#pragma unroll
            for (int P = 0; P < NB / 2; ++P)
              if (ncol8 + 32 * P < N) store8(dst + 32 * P, acc_read(acc[mb][2 * P]), acc_read(acc[mb][2 * P + 1]), odd);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
      // e4m3 inputs: dequantise the sum with the product of the per-tensor scales
      const float cs = p.c_scale;
      const int ncol = pn * BN + wn * WN + 4 * g;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int m = mrow + mb * 16;
        if (m < M) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const int n = ncol + nb * 16;
            out_t* dst = C + (int64_t)m * ldc + n;
            const floatx4_t v = acc_read(acc[mb][nb]) * cs;
            if (n + 3 < N) {
              store4(dst, v);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (n + e < N) dst[e] = to_out(v[e], (out_t*)nullptr);
            }
          }
        }
      }
    }
    if (tid == 0) {
      if (p.visits) atomicAdd(p.visits + tile, 1);
      if (p.owner) p.owner[tile] = blockIdx.x;
    }
    if constexpr (TRACE) {
      const long long te = trace_clock();
      if (tid == 0) trace_tile(p.trace, tile, blockIdx.x, t_begin, te);
      t_begin = te;
    }
  };

  barrier_raw(); // barrier 0: step 0 has landed
  if constexpr (TRACE) {
    t_begin = trace_clock();
    asm volatile("" ::"s"(t_begin));
  }
  int c = 0; // stage of the current step
  if constexpr (KSUB == 2) {
    const uint8_t* s0 = stage_ptr(0);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) read_b_frag(I0{}, s0 + A_BYTES, 0, nb);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) read_a_frag(I0{}, s0, 0, mb);
  }
  int q = 0;
  bool next = true;
  zero_acc();
  for (;;) {
    for (int kt = 0; kt < nk; ++kt) {
      const uint8_t* sA = stage_ptr(c);
      const uint8_t* sB = sA + A_BYTES;
      const int cn = c == 2 ? 0 : c + 1;
      // is there a step after this one? (the ring entry of tile q + 1 was published
      // at least one barrier ago)
      next = kt + 1 < nk || (unsigned)tile_of(q + 1) < (unsigned)T;
      if constexpr (KSUB == 2) {
        // k-group 0's MFMAs while k-group 1's fragments are read
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          mfma_row(I0{}, mb);
          if (mb < NB) read_b_frag(I1{}, sB, 1, mb);
          read_a_frag(I1{}, sA, 1, mb);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (next) {
          wait_lgkm0(); // this wave is done with stage c
          barrier_raw();
        }
        // k-group 1's MFMAs while the next step's k-group-0 fragments are read (stale but
        // harmless reads when there is no next step)
        const uint8_t* sAn = stage_ptr(cn);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          mfma_row(I1{}, mb);
          if (mb < NB) read_b_frag(I0{}, sAn + A_BYTES, 0, mb);
          read_a_frag(I0{}, sAn, 0, mb);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        // e4m3: the step's B fragments and A's first row block, then each further A row
        // block one MFMA row ahead
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) read_b_frag(I0{}, sB, 0, nb);
        read_a_frag(I0{}, sA, 0, 0);
        static_for<MB>([&](auto mbc) __attribute__((always_inline)) {
          constexpr int MBI = decltype(mbc)::value;
          if constexpr (MBI + 1 < MB) read_a_frag(I0{}, sA, 0, MBI + 1);
          mfma_row(I0{}, MBI);
          __builtin_amdgcn_sched_barrier(0);
        });
        if (next) {
          wait_lgkm0();
          barrier_raw();
        }
      }
      c = cn;
    }
    epilogue(tile_of(q));
    if (!next) break;
    zero_acc();
    ++q;
  }
}

} // namespace pw
} // namespace pgemm
