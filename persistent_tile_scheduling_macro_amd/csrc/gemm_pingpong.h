// Ping-pong form of the 256 x 256 fast tile body: the same eight waves of
// 128 x 64 (2 x 4), the same LDS swizzles, fragment reads and MFMAs as the
// lockstep body in gemm_fast.h -- so the same C bits -- but with the two
// waves of each SIMD in opposite phases instead of in lockstep.
//
// Waves 0-3 (group X, tile rows 0-127) and waves 4-7 (group Y, rows
// 128-255) share SIMDs pairwise (wave w and w + 4 run on one SIMD). Each
// k-step of a wave is two phases, separated by workgroup barriers:
//   memory phase:  issue the wave's global -> LDS copies for the next step,
//                  read the whole step's fragments (both k-groups) from LDS
//                  into registers, wait for the reads;
//   compute phase: the step's MFMAs, back to back, operands in registers.
// Group Y starts one phase late, so while the four X waves compute, the
// four Y waves copy and read, and the other way round: each SIMD's MFMA
// pipe is fed by one wave while its partner keeps the address unit and the
// LDS busy. No wave issues a copy inside its MFMA stream, so the address
// unit's queue can never hold up an MFMA (in the lockstep body every wave
// stalls in that queue right after the barrier, a third of each step). This
// is the forum thread's copy/compute overlap (first answer), arranged per
// SIMD instead of per workgroup; the roles alternate rather than being
// fixed to producer and consumer waves, because on CDNA every wave of a
// workgroup gets the same register budget, so a copy-only wave would waste
// the half of the register file that holds accumulators.
//
// Copy windows (two LDS stages of 64 KiB, one per step parity). Stage c of
// step s is free once both groups have read it, i.e. at the barrier that
// ends Y's memory phase of step s. In its memory phase of step s each group
// copies its part of step s + 1 into the other stage (free since both
// finished step s - 1):
//   X: A rows 0-127 and all of B, needed by X two phases later;
//   Y: A rows 128-255, needed by Y two phases later.
// Each wave waits for its own copies at the end of its compute phase, and
// the next barrier publishes them. (Giving Y part of B, so that both groups
// issue the same number of copies, was level or slower: those copies get
// only one phase to land.)
//
// LDS arrays are separate per stage and per A half, and the group and the
// stage are compile-time values in the loop, so the compiler can tell that
// a wave's reads of one stage do not alias the copies it has in flight into
// the other (it would otherwise wait for those copies before every read).
//
// Scheduling modes: non-persistent, static, dynamic and cancel-and-reuse,
// with the lockstep body's tile sequences and claim protocol. Claims are
// made by thread 0 (an X wave) at the first step of a tile, for the tile
// two ahead; the result is written to the LDS ring at the end of that
// step's compute phase and the next barrier publishes it, long before any
// wave needs that tile.
#pragma once

#include "gemm_fast.h"

namespace pgemm {
namespace pp {

using fast::b_swz;
using fast::block_k;
using fast::Frag;
using fast::read_a;
using fast::read_b;
using fast::static_for;
using fast::wait_vmcnt;

// s_waitcnt lgkmcnt(0) (vmcnt and expcnt left at their maxima)
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// A workgroup barrier without a memory fence: the caller waits for exactly
// the counters it needs (a fence would wait for every copy in flight).
__device__ inline void barrier_raw() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

template <int DT, int SCHED, bool TRACE, bool BT>
__global__ void __launch_bounds__(512, 2) gemm_pp_kernel(Params p) {
  static_assert(SCHED == kNonPersistent || SCHED == kStatic || SCHED == kDynamic || SCHED == kCancel,
                "stream-K runs its whole waves in the static kernel and its tail in the lockstep body");
  constexpr int BM = 256, BN = 256, MB = 8, WN = 64, NB = 4;
  constexpr int ES = Traits<DT>::esize;
  constexpr int BK = block_k(ES);
  constexpr int KSUB = BK / Traits<DT>::kgroup;
  constexpr int A_ROW = 128;
  constexpr int AH_BYTES = 128 * A_ROW;       // one A half: 128 rows of 128 B
  constexpr int B_ROW = BT ? A_ROW : BN * ES; // bytes per B row in LDS
  constexpr int B_BYTES = BT ? BN * A_ROW : BK * B_ROW;
  constexpr int B_CPR = B_ROW / 16;
  constexpr int B_RPI = 1024 / B_ROW;         // B rows per 1 KiB copy block
  static_assert(B_BYTES == 32 * 1024, "32 B blocks of 1 KiB per step");
  constexpr int XBW = 8; // B blocks per X wave per step (X copies all 32)
  typedef typename Traits<DT>::out_t out_t;
  typedef typename Frag<DT>::t frag_t;
  typedef std::integral_constant<int, 0> I0;
  typedef std::integral_constant<int, 1> I1;

  __shared__ __attribute__((aligned(1024))) uint8_t sAt0[AH_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sAt1[AH_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sAb0[AH_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sAb1[AH_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[B_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[B_BYTES];
  __shared__ int s_ring[8]; // claiming modes: tile id of tile-sequence number q at q % 8

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2; // 0 = X (rows 0-127), 1 = Y (rows 128-255)
  const int wl = wave & 3;   // wave column (64 columns each)
  const int M = p.M, N = p.N, K = p.K, T = p.T, G = p.G;
  const int nk = ((K + BK - 1) / BK + 1) & ~1; // even: every tile starts on stage 0
  const int64_t lda = (int64_t)p.lda * ES;
  const int64_t ldb = (int64_t)p.ldb * ES;
  const int64_t ldc = p.ldc;

  // ---- the tile sequence --------------------------------------------------
  // Sequence number q -> tile id; T past the workgroup's last tile.
  constexpr bool CLAIMS = SCHED == kDynamic || SCHED == kCancel;
  auto tile_of = [&](int q) __attribute__((always_inline)) -> int {
    if constexpr (SCHED == kNonPersistent) {
      return q == 0 ? (int)blockIdx.x : T;
    } else if constexpr (SCHED == kStatic) {
      const int64_t t = (int64_t)blockIdx.x + (int64_t)q * G;
      return t < T ? (int)t : T;
    } else {
      // claiming modes: every id comes from the ring, the dynamic mode's first
      // one (its own id) too; a per-q select between blockIdx.x and a ring read
      // made the compiler treat the tile id as divergent
      return __builtin_amdgcn_readfirstlane(s_ring[q & 7]);
    }
  };
  // Cancel-and-reuse with tiles of >= 4 k-steps claims tile 1 during tile 0
  // (steps 0-1) instead of in the prologue, so the first workgroups to start
  // cannot take a second tile before the last ones of the wave took a first
  // (the lockstep body's reason, measured there).
  const bool defer_t1 = SCHED == kCancel && nk >= 4;
  bool claim_live = false; // thread 0: the last claim got a tile
  if constexpr (CLAIMS) {
    if (tid == 0) {
      int t0 = (int)blockIdx.x;
      if constexpr (SCHED == kCancel) t0 = claim_tile(p.counter, T, claim_offset<SCHED>(G), claim_total<SCHED>(T, G));
      s_ring[0] = t0;
      // dynamic with G >= T: no tile lies beyond the grid's own, so no claim is made at all
      const bool may_claim = SCHED == kCancel || G < T;
      if (!defer_t1) {
        const int t1 = (t0 < T && may_claim) ? claim_tile(p.counter, T, claim_offset<SCHED>(G), claim_total<SCHED>(T, G)) : T;
        s_ring[1] = t1;
        claim_live = t1 < T;
      } else {
        claim_live = t0 < T;
      }
    }
    __syncthreads();
    if constexpr (SCHED == kCancel) {
      if ((unsigned)tile_of(0) >= (unsigned)T) return; // found no tile: the whole workgroup leaves at once
    }
  }

  // ---- copy lanes -----------------------------------------------------------
  // A half: block q = wl + 4j (j < 4) holds rows 8q..8q+7 of the half; the lane
  // fetches row 8q + lane/8, the chunk the swizzle stores at lane % 8.
  const int a_row0 = 8 * wl + (lane >> 3);
  int a_chunk;
  if constexpr (ES == 2) {
    a_chunk = (lane & 7) ^ (lane >> 3);
  } else {
    const int r = lane >> 3;
    a_chunk = (lane & 7) ^ (((r >> 1) & 1) | (r & 4));
  }
  // B (X waves only): block qb = wl + 4j (j < 8) holds B rows B_RPI*qb..; with
  // N x K B, rows are n and copied like A's.
  const int b_row0 = BT ? 8 * wl + (lane >> 3) : B_RPI * wl + lane / B_CPR;
  const int b_chunk0 = BT ? a_chunk : (lane % B_CPR) ^ b_swz<ES, B_ROW>(B_RPI * wl + lane / B_CPR);

  // ---- fragment lanes (the lockstep body's offsets, within one A half) -------
  const int g = lane >> 4, s16 = lane & 15;
  int a_off[KSUB][2];
#pragma unroll
  for (int kk = 0; kk < KSUB; ++kk) {
    if constexpr (ES == 2) {
      a_off[kk][0] = s16 * A_ROW + 16 * ((4 * kk + g) ^ (s16 & 7));
      a_off[kk][1] = a_off[kk][0];
    } else {
      const int sw = ((s16 >> 1) & 1) | (s16 & 4);
      a_off[kk][0] = s16 * A_ROW + 16 * ((2 * g) ^ sw);
      a_off[kk][1] = s16 * A_ROW + 16 * ((2 * g + 1) ^ sw);
    }
  }
  int b_off[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if constexpr (BT) {
      if constexpr (ES == 2) {
        const int q = s16 >> 2;
        const int r = wl * WN + 32 * (nb >> 1) + 8 * q + 4 * ((nb + q) & 1) + (s16 & 3);
        b_off[nb] = r * A_ROW + 16 * (g ^ (r & 7));
      } else {
        const int r = wl * WN + nb * 16 + s16;
        b_off[nb] = r * A_ROW + 16 * ((2 * g) ^ (((r >> 1) & 1) | (r & 4)));
      }
    } else if constexpr (ES == 2) {
      const int k = 8 * g + (s16 >> 2);
      const int q = s16 & 3;
      const int Lc = wl * (WN / 8) + 4 * (nb >> 1) + q;
      b_off[nb] = k * B_ROW + 16 * (Lc ^ b_swz<ES, B_ROW>(k)) + 8 * ((nb + q) & 1);
    } else {
      const int k = 32 * g + (s16 >> 1);
      const int Lc = wl * (WN / 16) + nb;
      b_off[nb] = k * B_ROW + 16 * (Lc ^ b_swz<ES, B_ROW>(k)) + 8 * (s16 & 1);
    }
  }

  // ---- producer: this wave's copies of the next step ---------------------------
  // An instruction's global offset is a per-lane base plus a per-instruction
  // row offset, which goes into the uniform soffset operand; masked lanes
  // (edges of M, N or K) take kOOB as their base and read zeros. A K x N B
  // copy's chunk also depends on its rows' swizzle term, a compile-time value
  // per instruction (the swizzle is an XOR of single row bits).
  const uint32_t a_vbase = (uint32_t)a_row0 * (uint32_t)lda + 16u * (uint32_t)a_chunk;
  int u_q = 0, u_kt = 0;  // tile sequence number and k-step of the next step to copy
  bool u_done = false;    // the tile sequence has ended
  const uint8_t* u_a = nullptr; // per-tile part of the copy addresses
  const uint8_t* u_b = nullptr;
  int u_m0 = 0, u_n0 = 0;
  auto copy_step = [&](auto grp_c, auto stage) __attribute__((always_inline)) {
    constexpr int GR = decltype(grp_c)::value, C = decltype(stage)::value;
    uint8_t* sAh = GR == 0 ? (C == 0 ? sAt0 : sAt1) : (C == 0 ? sAb0 : sAb1);
    uint8_t* sB = C == 0 ? sB0 : sB1;
    if (u_done) return;
    if (u_kt == 0) {
      const int t = tile_of(u_q);
      if ((unsigned)t >= (unsigned)T) { // any id outside [0, T) ends the sequence
        u_done = true;
        return;
      }
      int pm, pn;
      tile_coords(t, p, &pm, &pn);
      u_m0 = pm * BM + 128 * GR;
      u_n0 = pn * BN;
      u_a = p.A + (int64_t)u_m0 * lda;
      u_b = BT ? p.B + (int64_t)u_n0 * ldb : p.B + (int64_t)u_n0 * ES;
    }
    const int m0 = u_m0, n0 = u_n0, k0 = u_kt * BK;
    // Row strides and the wave's 1 KiB column of LDS blocks, made opaque here so
    // that every instruction's row offset (soffset) and LDS destination (M0) is
    // recomputed from them with one scalar operation instead of being hoisted out
    // of the loop: some 30 such invariants exhaust the SGPRs, after which the
    // compiler keeps offsets in VGPRs and wraps each copy in a readfirstlane loop.
    int lda_s = (int)lda, ldb_s = (int)ldb, wl_s = wl * 1024;
    asm volatile("" : "+s"(lda_s), "+s"(ldb_s), "+s"(wl_s));
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(u_a + (int64_t)k0 * ES);
    const int mrem = M - m0, krem = K - k0;
    // interior step: no lane of any copy is masked
    const int nrem = BT ? N - n0 : (N - n0) * ES;
    const bool full = (mrem >= 128) & (krem >= BK) & (BT ? nrem >= BN : nrem >= BN * ES);
    const bool kval = full || (k0 * ES + 16 * a_chunk) < K * ES;
    if constexpr (GR == 0) {
      const __amdgpu_buffer_rsrc_t rb = BT ? make_rsrc(u_b + (int64_t)k0 * ES) : make_rsrc(u_b + (int64_t)k0 * ldb);
      static_for<XBW>([&](auto jc) __attribute__((always_inline)) {
        constexpr int QOFF = 4 * decltype(jc)::value; // block qb = QOFF + wl
        if constexpr (BT) {
          const bool ok = full || (kval & (b_row0 + 8 * QOFF < nrem));
          const uint32_t base = (uint32_t)b_row0 * (uint32_t)ldb + 16u * (uint32_t)b_chunk0;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, PGEMM_LDS(void, sB + QOFF * 1024 + wl_s), 16, ok ? base : kOOB,
                                                   8 * QOFF * ldb_s, 0, 0);
        } else {
          constexpr int SW = b_swz<ES, B_ROW>(B_RPI * QOFF);
          const int Lc = b_chunk0 ^ SW;
          const bool ok = full || ((b_row0 + B_RPI * QOFF < krem) & (16 * Lc < nrem));
          const uint32_t base = (uint32_t)b_row0 * (uint32_t)ldb + 16u * (uint32_t)Lc;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, PGEMM_LDS(void, sB + QOFF * 1024 + wl_s), 16, ok ? base : kOOB,
                                                   B_RPI * QOFF * ldb_s, 0, 0);
        }
      });
    }
    static_for<4>([&](auto jc) __attribute__((always_inline)) {
      constexpr int J = decltype(jc)::value;
      const bool ok = full || (kval & (a_row0 + 32 * J < mrem));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, PGEMM_LDS(void, sAh + 4 * J * 1024 + wl_s), 16, ok ? a_vbase : kOOB,
                                               32 * J * lda_s, 0, 0);
    });
    if (++u_kt == nk) {
      u_kt = 0;
      ++u_q;
    }
  };

  // ---- accumulators, fragments --------------------------------------------------
  floatx4_t acc[MB][NB];
  frag_t af[KSUB][MB], bf[KSUB][NB];
  auto read_frags = [&](auto grp_c, auto stage) __attribute__((always_inline)) {
    constexpr int GR = decltype(grp_c)::value, C = decltype(stage)::value;
    const uint8_t* sAh = GR == 0 ? (C == 0 ? sAt0 : sAt1) : (C == 0 ? sAb0 : sAb1);
    const uint8_t* sB = C == 0 ? sB0 : sB1;
#pragma unroll
    for (int kk = 0; kk < KSUB; ++kk) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if constexpr (BT) {
          if constexpr (ES == 2)
            bf[kk][nb] = read_a<DT>(sB + (b_off[nb] ^ (64 * kk)), nullptr);
          else
            bf[kk][nb] = read_a<DT>(sB + b_off[nb], sB + (b_off[nb] ^ 16));
        } else {
          bf[kk][nb] = read_b<DT, B_ROW>(sB + b_off[nb] + kk * 32 * B_ROW);
        }
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        af[kk][mb] = read_a<DT>(sAh + a_off[kk][0] + mb * 16 * A_ROW, sAh + a_off[kk][1] + mb * 16 * A_ROW);
    }
  };
  // each accumulator takes k-group 0 then k-group 1 of the step, as in the lockstep body
  auto compute = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < KSUB; ++kk)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) mfma_acc(acc[mb][nb], bf[kk][nb], af[kk][mb]);
  };
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    acc_drain();
  };

  long long t_begin = 0; // tile trace: when group Y began the current tile

  // ---- epilogue: this wave's 128 x 64 block of the tile, rounded and stored ------
  auto epilogue = [&](auto grp_c, int tile) __attribute__((always_inline)) {
    constexpr int GR = decltype(grp_c)::value;
    acc_drain();
    // the lane's row and column group, recomputed here (a volatile read of the lane
    // id) rather than kept live in VGPRs through the whole k-loop
    int lane_e;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_e));
    const int s16 = lane_e & 15, g = lane_e >> 4;
    int pm, pn;
    tile_coords(tile, p, &pm, &pn);
    const int mrow = pm * BM + GR * 128 + s16;
    out_t* C = reinterpret_cast<out_t*>(p.C);
    if constexpr (ES == 2) {
      const int ncol8 = pn * BN + wl * WN + 8 * g;
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
      const int ncol = pn * BN + wl * WN + 4 * g;
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
    // Group Y stores the tile's second half one phase after X stored the first:
    // its wave 0 counts the visit, logs the owner and writes the trace.
    if constexpr (GR == 1) {
      if (tid == 256) {
        if (p.visits) atomicAdd(p.visits + tile, 1);
        if (p.owner) p.owner[tile] = blockIdx.x;
      }
      if constexpr (TRACE) {
        const long long te = trace_clock();
        if (tid == 256) trace_tile(p.trace, tile, blockIdx.x, t_begin, te);
        t_begin = te;
      }
    }
  };

  // ---- claims (thread 0, an X wave) ------------------------------------------------
  // At a tile's first step the claim for the tile two ahead is issued in the
  // memory phase and finished at the end of the same step's compute phase,
  // after the wave's wait for its memory operations; the barrier that follows
  // publishes the ring entry. Cancel-and-reuse with a deferred tile 1 makes two
  // claims in tile 0 (tiles 1 and 2, at steps 0 and 2).
  int c_raw = 0;
  auto claim_now = [&](int q, int kt) __attribute__((always_inline)) -> bool {
    return (kt & 1) == 0 && kt < (defer_t1 && q == 0 ? 4 : 2) && claim_live;
  };
  auto claim_issue = [&](int q, int kt) __attribute__((always_inline)) {
    if constexpr (CLAIMS) {
      if (tid == 0 && claim_now(q, kt)) c_raw = claim_raw(p.counter);
    }
  };
  auto claim_publish = [&](int q, int kt) __attribute__((always_inline)) {
    if constexpr (CLAIMS) {
      if (tid == 0 && claim_now(q, kt)) {
        const int t = claim_finish(p.counter, c_raw, T, claim_offset<SCHED>(G), claim_total<SCHED>(T, G));
        s_ring[(defer_t1 && q == 0 ? 1 + (kt >> 1) : q + 2) & 7] = t;
        claim_live = t < T;
      }
    }
  };

  // ---- the ping-pong, one instance per group ----------------------------------------
  auto run = [&](auto grp_c) __attribute__((always_inline)) {
    constexpr int GR = decltype(grp_c)::value;
    copy_step(grp_c, I0{}); // step 0 into stage 0 (this wave's part)
    wait_vmcnt<0>();
    barrier_raw();
    if constexpr (GR == 1) barrier_raw(); // Y runs one phase behind X
    if constexpr (TRACE && GR == 1) {
      t_begin = trace_clock();
      asm volatile("" ::"s"(t_begin));
    }
    int q = 0, kt = 0; // consumer: tile sequence number and k-step
    // One k-step: memory phase, barrier, compute phase, barrier. A tile's
    // epilogue follows its last step's final barrier, so it opens the wave's
    // next memory phase (no fragment is live across it).
    auto step = [&](auto stage) __attribute__((always_inline)) {
      typedef std::integral_constant<int, decltype(stage)::value ^ 1> NEXT;
      if constexpr (GR == 0) claim_issue(q, kt);
      copy_step(grp_c, NEXT{});
      read_frags(grp_c, stage);
      wait_lgkm0();
      barrier_raw();
      compute();
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<0>(); // this wave's copies of the next step (and its C stores) have landed
      if constexpr (GR == 0) claim_publish(q, kt);
      barrier_raw();
      ++kt;
    };
    zero_acc();
    for (;;) {
      for (kt = 0; kt < nk;) { // nk is even
        step(I0{});
        step(I1{});
      }
      if ((unsigned)tile_of(q + 1) >= (unsigned)T) break;
      epilogue(grp_c, tile_of(q));
      zero_acc();
      ++q;
    }
    if constexpr (GR == 0) barrier_raw(); // X matches Y's extra barrier
    epilogue(grp_c, tile_of(q));
  };
  if (grp == 0)
    run(I0{});
  else
    run(I1{});
}

} // namespace pp
} // namespace pgemm
