// The fast GEMM kernel for aligned operands (K and N multiples of 16 bytes
// of elements, 16-byte aligned A and B).
//
// Macro tile 256 x 256, 256 threads = 4 waves in a 2 x 2 arrangement, each
// wave owning a 128 x 128 sub-tile (8 x 8 blocks of 16 x 16 MFMA outputs,
// 256 fp32 accumulators per lane, kept in AGPRs). K is consumed in steps of
// BK (32 for fp16/bf16, 128 for fp8: one MFMA k-group per step). Each
// step's A (256 x BK) and B (BK x 256) slices are copied global -> LDS by
// buffer loads that write LDS directly (no register staging) into a ring of
// S stages (4 for 16-bit, 2 for fp8), so copies run S-1 steps ahead of the
// MFMAs -- the copy/compute overlap of the persistent-kernel forum thread
// (first answer). Per-CU L2 -> LDS bandwidth on this part is about the rate
// at which the MFMAs consume a 256 x 256 tile's operands, so the copies
// must run continuously and well ahead.
//
// Step s on stage c = s mod S:
//   1. MFMAs for rows 0..3 of the wave's 8 x 8 block grid (fragments of
//      step s were read into registers during step s-1);
//   2. wait for this wave's copy of step s+1, then one workgroup barrier:
//      after it, stage s+1 is complete and nobody reads stage c any more;
//   3. issue the copy of step s+S into stage c;
//   4. MFMAs for rows 4..7, interleaved with the LDS reads of step s+1's
//      fragments (so LDS latency hides under MFMAs at every step).
// One barrier per step.
//
// All three scheduling modes run this one body over the flattened sequence
// of (tile, k-step) pairs their scheduler produces. The copies cross tile
// boundaries freely, so in the persistent modes the next tile's first
// S-1 steps are in flight while the current tile's epilogue converts and
// stores C -- the pipelining across output tiles that the Triton
// persistent-matmul issue ("Describe the issue") expected persistence to
// buy. In the non-persistent mode a workgroup owns one tile.
//
// LDS layouts use 16-byte chunks, swizzled so that every fragment read is
// bank-conflict-free on gfx950 (64 banks; ds_read_b128 serves lanes
// {0-7,16-23}, {8-15,24-31}, ... per pass; transpose reads serve 32 lanes):
//   A, 16-bit: 256 rows (m) x 64 B; chunk c of row r at c ^ ((r >> 1) & 3).
//   A, fp8:    256 rows (m) x 128 B; chunk c of row r at c ^ sa8(r),
//              sa8(r) = ((r >> 1) & 1) | (r & 4).
//   B, 16-bit: 32 rows (k) x 512 B; chunk c of row r at
//              c ^ (2*(r & 3) + 8*((r >> 3) & 1)).
//   B, fp8:    128 rows (k) x 256 B; chunk c of row r at
//              c ^ ((r & 7) + 8*((r >> 5) & 1)).
// A fragments are plain 16-byte reads of consecutive k. B is n-contiguous
// in memory, so its fragments come from the gfx950 LDS transpose reads
// (ds_read_b64_tr_b16 / _b8), which hand each lane one column's
// consecutive k values.
//
// The MFMA is issued with B as its first operand, so each lane's four
// outputs are four consecutive columns of one row of C (8-byte stores).
#pragma once

#include "device_common.h"

namespace pgemm {
namespace fast {

constexpr int BM = 256, BN = 256, THREADS = 256;

__host__ __device__ constexpr int block_k(int esize) { return esize == 2 ? 32 : 128; }
__host__ __device__ constexpr int stages(int esize) { return esize == 2 ? 4 : 2; }

template <int DT>
struct Frag;
template <>
struct Frag<kF16> { typedef half8_t t; };
template <>
struct Frag<kBF16> { typedef bf16x8_t t; };
template <>
struct Frag<kF8E4M3> { typedef intx8_t t; };

// s_waitcnt vmcnt(n) (expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Read the B fragment of one 16-column block: lane (16g + s) ends up with
// column s of the block and the k values its A partner holds.
template <int DT>
__device__ inline typename Frag<DT>::t read_b(const uint8_t* base) {
  if constexpr (Traits<DT>::esize == 2) {
    // two transpose reads: k rows +0..3 and +4..7 of the lane group's 8 k
    fp16x4_raw_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16(PGEMM_LDS(fp16x4_raw_t, base));
    fp16x4_raw_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16(PGEMM_LDS(fp16x4_raw_t, base + 4 * 512));
    intx2_t l = __builtin_bit_cast(intx2_t, lo), h = __builtin_bit_cast(intx2_t, hi);
    intx4_t w = {l[0], l[1], h[0], h[1]};
    return __builtin_bit_cast(typename Frag<DT>::t, w);
  } else {
    // four transpose reads of 8 k each (k rows +0, +8, +16, +24)
    intx2_t r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(PGEMM_LDS(intx2_t, base));
    intx2_t r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(PGEMM_LDS(intx2_t, base + 8 * 256));
    intx2_t r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(PGEMM_LDS(intx2_t, base + 16 * 256));
    intx2_t r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(PGEMM_LDS(intx2_t, base + 24 * 256));
    return intx8_t{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
  }
}

template <int DT>
__device__ inline typename Frag<DT>::t read_a(const uint8_t* lo, const uint8_t* hi) {
  if constexpr (Traits<DT>::esize == 2) {
    (void)hi;
    return __builtin_bit_cast(typename Frag<DT>::t, *reinterpret_cast<const intx4_t*>(lo));
  } else {
    intx4_t a = *reinterpret_cast<const intx4_t*>(lo), b = *reinterpret_cast<const intx4_t*>(hi);
    return intx8_t{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
}

template <int DT, int SCHED>
__global__ void __launch_bounds__(THREADS) gemm_fast_kernel(Params p) {
  constexpr int ES = Traits<DT>::esize;
  constexpr int BK = block_k(ES);      // k elements per step
  constexpr int S = stages(ES);        // LDS ring depth
  constexpr int A_ROW = BK * ES;       // bytes per A row in LDS (64 or 128)
  constexpr int A_BYTES = BM * A_ROW;  // per stage
  constexpr int B_ROW = BN * ES;       // bytes per B row in LDS (512 or 256)
  constexpr int B_BYTES = BK * B_ROW;  // per stage
  constexpr int LA = A_BYTES / (THREADS * 16), LB = B_BYTES / (THREADS * 16);
  constexpr int L = LA + LB;           // copy instructions per thread per step
  constexpr int A_RPI = 1024 / A_ROW;  // A rows per copy instruction (16 or 8)
  static_assert(S == 2 || S == 4, "ring depth");
  static_assert((S - 1) * L < 64, "vmcnt range");
  typedef typename Traits<DT>::out_t out_t;
  typedef typename Frag<DT>::t frag_t;
  typedef std::integral_constant<int, 0> I0;
  typedef std::integral_constant<int, 1> I1;
  typedef std::integral_constant<int, (S > 2 ? 2 : 0)> I2;
  typedef std::integral_constant<int, (S > 2 ? 3 : 1)> I3;

  __shared__ __attribute__((aligned(1024))) uint8_t sA0[A_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[B_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[A_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[B_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sA2[S > 2 ? A_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t sB2[S > 2 ? B_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t sA3[S > 2 ? A_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t sB3[S > 2 ? B_BYTES : 16];
  __shared__ int s_ring[8]; // dynamic mode: tile id of tile-sequence number q at q % 8

  auto bufA = [&](auto c) __attribute__((always_inline)) -> uint8_t* {
    constexpr int C = decltype(c)::value;
    return C == 0 ? sA0 : C == 1 ? sA1 : C == 2 ? sA2 : sA3;
  };
  auto bufB = [&](auto c) __attribute__((always_inline)) -> uint8_t* {
    constexpr int C = decltype(c)::value;
    return C == 0 ? sB0 : C == 1 ? sB1 : C == 2 ? sB2 : sB3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // wave-uniform, lives in an SGPR
  const int wm = wave >> 1, wn = wave & 1;
  const int M = p.M, N = p.N, K = p.K, T = p.T, G = p.G;
  // k-steps per tile, rounded up to a multiple of S so that every tile starts
  // on stage 0 (the extra steps read zeros: they lie past K)
  const int nk = ((K + BK - 1) / BK + S - 1) / S * S;
  const int64_t lda = (int64_t)K * ES; // bytes per row of A
  const int64_t ldb = (int64_t)N * ES; // bytes per row of B
  const int64_t ldc = N;               // elements per row of C

  // ---- per-lane constants of the global -> LDS copy ------------------------
  // A: instruction q = wave + 4j covers A_RPI rows; lane -> row q*A_RPI +
  // lane/(A_ROW/16), physical chunk lane % (A_ROW/16); the swizzle depends
  // on the row's low bits only, which are lane-constant.
  int a_row0, a_chunk;
  if constexpr (ES == 2) {
    a_row0 = A_RPI * wave + (lane >> 2);
    a_chunk = (lane & 3) ^ ((lane >> 3) & 3); // row & 15 == lane >> 2
  } else {
    a_row0 = A_RPI * wave + (lane >> 3);
    const int r = lane >> 3;                  // row & 7
    a_chunk = (lane & 7) ^ (((r >> 1) & 1) | (r & 4));
  }
  // B: instruction q = wave + 4j covers 1024 / B_ROW rows.
  int b_row0, b_pchunk, b_h0;
  if constexpr (ES == 2) {
    b_row0 = 2 * wave + (lane >> 5);
    b_pchunk = lane & 31;
    b_h0 = 2 * (b_row0 & 3); // + 8 * (j & 1) per instruction
  } else {
    b_row0 = 4 * wave + (lane >> 4);
    b_pchunk = lane & 15;
    b_h0 = b_row0 & 7;       // + 8 * ((j >> 1) & 1) per instruction
  }

  // ---- per-lane constants of the fragment reads ----------------------------
  const int g = lane >> 4, s16 = lane & 15;
  int a_off[2];
  {
    const int r = wm * 128 + s16; // + mb * 16
    if constexpr (ES == 2) {
      a_off[0] = r * A_ROW + 16 * (g ^ ((s16 >> 1) & 3));
      a_off[1] = a_off[0];
    } else {
      const int sw = ((s16 >> 1) & 1) | (s16 & 4);
      a_off[0] = r * A_ROW + 16 * ((2 * g) ^ sw);
      a_off[1] = r * A_ROW + 16 * ((2 * g + 1) ^ sw);
    }
  }
  int b_off[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    if constexpr (ES == 2) {
      const int k = 8 * g + (s16 >> 2); // +4 for the second read
      const int Lc = wn * 16 + 2 * nb + ((s16 & 3) >> 1);
      const int h = 2 * (s16 >> 2) + 8 * (g & 1);
      b_off[nb] = k * B_ROW + 16 * (Lc ^ h) + 8 * (s16 & 1);
    } else {
      const int k = 32 * g + (s16 >> 1); // +8, +16, +24 for reads 1..3
      const int Lc = wn * 8 + nb;
      const int h = (s16 >> 1) + 8 * (g & 1);
      b_off[nb] = k * B_ROW + 16 * (Lc ^ h) + 8 * (s16 & 1);
    }
  }

  // ---- the tile sequence of this workgroup ---------------------------------
  // Sequence number q -> tile id. Static: blockIdx + q*G; non-persistent:
  // blockIdx for q = 0 only; dynamic: blockIdx for q = 0, then each tile's
  // successor is claimed when the producer starts copying that tile, and
  // published in s_ring before the next barrier.
  int claim_val = 0;
  bool claim_pending = false; // thread 0 only: a claim waiting to be published
  int claim_seq = 0;          // sequence number the pending claim is for
  auto tile_of = [&](int q) __attribute__((always_inline)) -> int {
    if constexpr (SCHED == kNonPersistent) {
      return q == 0 ? (int)blockIdx.x : T;
    } else if constexpr (SCHED == kStatic) {
      const int64_t t = (int64_t)blockIdx.x + (int64_t)q * G;
      return t < T ? (int)t : T;
    } else {
      return q == 0 ? (int)blockIdx.x : __builtin_amdgcn_readfirstlane(s_ring[q & 7]);
    }
  };
  auto publish_claim = [&]() __attribute__((always_inline)) {
    if constexpr (SCHED == kDynamic) {
      if (claim_pending) {
        s_ring[claim_seq & 7] = claim_val;
        claim_pending = false;
      }
    }
  };

  // ---- producer: copy of step `issued` into stage `issued % S` --------------
  // A copy is begun (tile and k of the step resolved, buffer resources
  // built) and then issued one 1 KiB instruction at a time, interleaved
  // with the MFMAs: a burst of copy instructions would stall this wave's
  // in-order issue behind the memory pipeline and starve the MFMAs.
  int issued = 0;      // copies begun
  int p_tile = 0;      // tile of the copy in progress
  bool p_done = false; // no more steps to copy
  bool p_busy = false; // a begun copy still has instructions to issue
  __amdgpu_buffer_rsrc_t ra, rb;
  bool p_kval = false;
  int p_mrem = 0, p_krem = 0, p_nrem = 0;
  uint32_t a_base = 0;
  auto begin_copy = [&]() __attribute__((always_inline)) {
    if (p_done) return;
    const int q = issued / nk, kt = issued - q * nk;
    if (kt == 0) {
      p_tile = tile_of(q);
      if (p_tile >= T) {
        p_done = true;
        return;
      }
      if constexpr (SCHED == kDynamic) {
        if (tid == 0) { // claim the successor now; published before the next barrier
          claim_val = claim_tile(p.counter, T, G);
          claim_seq = q + 1;
          claim_pending = true;
        }
      }
    }
    int pm, pn;
    tile_coords(p_tile, p, &pm, &pn);
    const int m0 = pm * BM, n0 = pn * BN, k0 = kt * BK;
    // A rebased at (m0, k0), B at (k0, n0); rows past M or K and chunks
    // past K or N read zeros.
    ra = make_rsrc(p.A + (int64_t)m0 * lda + (int64_t)k0 * ES);
    rb = make_rsrc(p.B + (int64_t)k0 * ldb + (int64_t)n0 * ES);
    p_mrem = M - m0;
    p_krem = K - k0;
    p_nrem = (N - n0) * ES;
    p_kval = (k0 * ES + 16 * a_chunk) < K * ES;
    a_base = (uint32_t)a_row0 * (uint32_t)lda + 16u * (uint32_t)a_chunk;
    p_busy = true;
    ++issued;
  };
  // instruction j (0 <= j < LA + LB) of the copy in progress, into stage (sA, sB)
  auto copy_part = [&](uint8_t* sA, uint8_t* sB, auto jc) __attribute__((always_inline)) {
    constexpr int J = decltype(jc)::value;
    if (!p_busy) return;
    if constexpr (J < LA) {
      const bool ok = p_kval & (a_row0 + 4 * A_RPI * J < p_mrem);
      const uint32_t off = ok ? a_base + (uint32_t)(4 * A_RPI * J) * (uint32_t)lda : kOOB;
      load16_to_lds(ra, sA + (wave + 4 * J) * 1024, off);
    } else {
      constexpr int JB = J - LA;
      int row, Lc;
      if constexpr (ES == 2) {
        row = b_row0 + 8 * JB;
        Lc = b_pchunk ^ (b_h0 + 8 * (JB & 1));
      } else {
        row = b_row0 + 16 * JB;
        Lc = b_pchunk ^ (b_h0 + 8 * ((JB >> 1) & 1));
      }
      const bool ok = (row < p_krem) & (16 * Lc < p_nrem);
      const uint32_t off = ok ? (uint32_t)row * (uint32_t)ldb + 16u * (uint32_t)Lc : kOOB;
      load16_to_lds(rb, sB + (wave + 4 * JB) * 1024, off);
    }
    if (J == LA + LB - 1) p_busy = false;
  };
  // a whole copy at once (prologue only)
  auto copy_all = [&](auto c) __attribute__((always_inline)) {
    begin_copy();
    uint8_t* sA = bufA(c);
    uint8_t* sB = bufB(c);
    copy_part(sA, sB, std::integral_constant<int, 0>{});
    copy_part(sA, sB, std::integral_constant<int, 1>{});
    copy_part(sA, sB, std::integral_constant<int, 2>{});
    copy_part(sA, sB, std::integral_constant<int, 3>{});
    copy_part(sA, sB, std::integral_constant<int, 4>{});
    copy_part(sA, sB, std::integral_constant<int, 5>{});
    copy_part(sA, sB, std::integral_constant<int, 6>{});
    copy_part(sA, sB, std::integral_constant<int, 7>{});
    if constexpr (L > 8) {
      copy_part(sA, sB, std::integral_constant<int, (L > 8 ? 8 : 0)>{});
      copy_part(sA, sB, std::integral_constant<int, (L > 8 ? 9 : 0)>{});
      copy_part(sA, sB, std::integral_constant<int, (L > 8 ? 10 : 0)>{});
      copy_part(sA, sB, std::integral_constant<int, (L > 8 ? 11 : 0)>{});
      copy_part(sA, sB, std::integral_constant<int, (L > 8 ? 12 : 0)>{});
      copy_part(sA, sB, std::integral_constant<int, (L > 8 ? 13 : 0)>{});
      copy_part(sA, sB, std::integral_constant<int, (L > 8 ? 14 : 0)>{});
      copy_part(sA, sB, std::integral_constant<int, (L > 8 ? 15 : 0)>{});
    }
  };

  // ---- accumulators and fragments -------------------------------------------
  floatx4_t acc[8][8];
  frag_t af[2][8], bf[2][8];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    acc_drain(); // accvgpr writes -> MFMA srcC reads
  };
  auto read_frags = [&](auto f, auto c, int mb) __attribute__((always_inline)) {
    constexpr int F = decltype(f)::value;
    const uint8_t* sA = bufA(c);
    const uint8_t* sB = bufB(c);
    bf[F][mb] = read_b<DT>(sB + b_off[mb]);
    af[F][mb] = read_a<DT>(sA + a_off[0] + mb * 16 * A_ROW, sA + a_off[1] + mb * 16 * A_ROW);
  };
  auto mfma_row = [&](auto f, int mb) __attribute__((always_inline)) {
    constexpr int F = decltype(f)::value;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) mfma_acc(acc[mb][nb], bf[F][nb], af[F][mb]);
  };

  // ---- epilogue: round to the output type and store one tile ---------------
  auto epilogue = [&](int tile) __attribute__((always_inline)) {
    acc_drain();
    int pm, pn;
    tile_coords(tile, p, &pm, &pn);
    const int mrow = pm * BM + wm * 128 + s16;
    const int ncol = pn * BN + wn * 128 + 4 * g;
    out_t* C = reinterpret_cast<out_t*>(p.C);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const int m = mrow + mb * 16;
      if (m < M) {
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          const int n = ncol + nb * 16;
          out_t* dst = C + (int64_t)m * ldc + n;
          if (n + 3 < N) {
            store4(dst, acc[mb][nb]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < N) dst[e] = to_out(acc[mb][nb][e], (out_t*)nullptr);
          }
        }
      }
    }
    if (tid == 0) {
      if (p.visits) atomicAdd(p.visits + tile, 1);
      if (p.owner) p.owner[tile] = blockIdx.x;
    }
  };

  // ---- prologue: copies of steps 0..S-1, fragments of step 0 ----------------
  // nk is a multiple of S, so all S prologue copies belong to the first tile
  copy_all(I0{});
  copy_all(I1{});
  if constexpr (S > 2) {
    copy_all(I2{});
    copy_all(I3{});
  }
  publish_claim();
  // step 0's copy is the oldest; `issued - 1` newer steps may stay in flight
  if (issued == S) {
    wait_vmcnt<(S - 1) * L>();
  } else {
    wait_vmcnt<0>();
  }
  __syncthreads();
  zero_acc();
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) read_frags(I0{}, I0{}, mb);

  int cs = 0;           // consumer step
  bool stores_pending = false;
  bool has_next = true;

  // One consumer step on stage C (compile time), fragment set C & 1.
  // Copy instructions: the second half of the copy begun in the previous
  // step (into stage C-1) rides along rows 0..3; the first half of the copy
  // begun at this step's barrier (into stage C) rides along rows 4..7.
  constexpr int HALF = L / 2;       // copy instructions per half step (4 or 8)
  constexpr int PER_ROW = HALF / 4; // per MFMA row (1 or 2)
  auto step = [&](auto cst) __attribute__((always_inline)) {
    constexpr int C = decltype(cst)::value;
    constexpr int F = C & 1, FN = F ^ 1, CN = (C + 1) % S, CP = (C + S - 1) % S;
    typedef std::integral_constant<int, F> IF;
    typedef std::integral_constant<int, FN> IFN;
    typedef std::integral_constant<int, CN> ICN;
    typedef std::integral_constant<int, CP> ICP;
    typedef std::integral_constant<int, C> IC;
    has_next = issued > cs + 1;
    auto first_row = [&](auto mbc) __attribute__((always_inline)) {
      constexpr int MB = decltype(mbc)::value;
      mfma_row(IF{}, MB);
      copy_part(bufA(ICP{}), bufB(ICP{}), std::integral_constant<int, HALF + PER_ROW * MB>{});
      if constexpr (PER_ROW > 1)
        copy_part(bufA(ICP{}), bufB(ICP{}), std::integral_constant<int, HALF + PER_ROW * MB + PER_ROW - 1>{});
      __builtin_amdgcn_sched_barrier(0);
    };
    first_row(std::integral_constant<int, 0>{});
    first_row(std::integral_constant<int, 1>{});
    first_row(std::integral_constant<int, 2>{});
    first_row(std::integral_constant<int, 3>{});
    if (has_next) {
      // wait for this wave's copy of step cs+1 (newer copies may stay in flight)
      const int after = issued - (cs + 2); // steps copied after step cs+1
      if (stores_pending || after <= 0) {
        wait_vmcnt<0>();
        stores_pending = false;
      } else if (S == 4 && after >= 2) {
        wait_vmcnt<(S == 4 ? 2 * L : 0)>();
      } else {
        wait_vmcnt<L>();
      }
      __syncthreads();
      begin_copy(); // step cs + S into stage C, which nobody reads any more
    }
    // the next step's fragments (harmless stale reads when there is no next step)
    auto second_row = [&](auto mbc) __attribute__((always_inline)) {
      constexpr int MB = decltype(mbc)::value; // 4..7
      read_frags(IFN{}, ICN{}, 2 * (MB - 4));
      mfma_row(IF{}, MB);
      copy_part(bufA(IC{}), bufB(IC{}), std::integral_constant<int, PER_ROW * (MB - 4)>{});
      if constexpr (PER_ROW > 1)
        copy_part(bufA(IC{}), bufB(IC{}), std::integral_constant<int, PER_ROW * (MB - 4) + PER_ROW - 1>{});
      read_frags(IFN{}, ICN{}, 2 * (MB - 4) + 1);
      __builtin_amdgcn_sched_barrier(0);
    };
    second_row(std::integral_constant<int, 4>{});
    second_row(std::integral_constant<int, 5>{});
    second_row(std::integral_constant<int, 6>{});
    second_row(std::integral_constant<int, 7>{});
    publish_claim();
    ++cs;
  };

  int c_q = 0; // consumer tile sequence number
  int c_tile = blockIdx.x;
  for (;;) {
    for (int kt = 0; kt < nk; kt += S) {
      step(I0{});
      step(I1{});
      if constexpr (S > 2) {
        step(I2{});
        step(I3{});
      }
    }
    // tile finished: store it while the next tile's copies are in flight
    epilogue(c_tile);
    stores_pending = true;
    if (!has_next) break;
    c_tile = tile_of(++c_q);
    zero_acc();
  }
}

} // namespace fast
} // namespace pgemm
