// The fast GEMM kernel for aligned operands (K and N multiples of 16 bytes
// of elements, 16-byte aligned A and B), in two macro-tile configurations:
//
//   kTile256: 256 x 256 tile, 512 threads = 8 waves (two per SIMD) in a
//             2 x 4 arrangement, each wave owning a 128 x 64 sub-tile
//             (8 x 4 blocks of 16 x 16 MFMA outputs, 128 fp32 accumulators
//             per lane, kept in AGPRs); one workgroup per CU.
//   kTile128: 128 x 128 tile, 256 threads = 4 waves in 2 x 2, each wave
//             owning a 64 x 64 sub-tile (4 x 4 blocks, 64 accumulators);
//             two workgroups per CU, so a problem has four times the tiles
//             (a 4096 x 4096 C has 1024, two per persistent workgroup).
//
// K is consumed in steps of 128 bytes of elements (BK = 64 for fp16/bf16,
// 128 for fp8). Each step's A (BM x BK) and B (BK x BN) slices are copied
// global -> LDS by buffer loads that write LDS directly (no register
// staging) into a two-stage ring, so the copy of step s+1 overlaps the
// MFMAs of step s (the copy/compute overlap of the persistent-kernel forum
// thread, first answer). Both configurations copy 4 + 4 KiB-sized
// instructions per thread per step (the body is written for waves of 64 or
// 128 columns and any even copy count).
//
// Why this shape on gfx950 (measured on the part, not taken from the
// pages): a 256 x 256 tile's MFMAs need 32 B/clk of operand copies at full
// rate, which the CU's global -> LDS path (about 46 B/clk for whole-line
// copies) sustains. What binds is the LDS: it serves the fragment reads
// (256 B/clk for 16-byte reads, 172 B/clk for the transposing reads) and
// takes the copies' writes, and at this kernel's mix its read throughput
// falls to about 110 B/clk, near the 96 B/clk the fragment reads need at
// full MFMA rate. Two waves per SIMD overlap that with the MFMAs far
// better than one: four waves of 128 x 128, which read a third less from
// LDS, measured 9-20% slower. Copy rows must be whole 128-byte lines
// (half-line rows cut the copy path's throughput at full occupancy).
//
// Step s on stage c = s mod 2 (16-bit: two MFMA k-groups per step):
//   1. MFMAs of k-group 0 (fragments read during step s-1) while the
//      fragments of k-group 1 are read from stage c;
//   2. wait for this wave's copy of step s+1, one workgroup barrier: stage
//      c^1 is complete, and every wave has read all of stage c;
//   3. issue the whole copy of step s+2 into stage c at once (eight 1 KiB
//      instructions; measured faster than spreading them over MFMA rows);
//   4. MFMAs of k-group 1 while the k-group-0 fragments of step s+1 are
//      read from stage c^1.
// So every LDS read has MFMAs to hide behind, and there is one barrier per
// step. fp8 steps are a single k-group: the barrier sits at the top of the
// step, the next copy is issued right after it, and the step's fragments
// are read after it. (A variant with a second barrier per step, freeing
// each stage as soon as its fragments are in registers, measured slower on
// this part: the extra barrier costs more than the earlier copies buy.)
//
// All scheduling modes run this one body over the flattened sequence of
// (tile, k-step) pairs their scheduler produces. Copies cross tile
// boundaries freely, so in the persistent modes the next tile's first copy
// is in flight while the current tile's epilogue converts and stores C --
// the pipelining across output tiles the Triton persistent-matmul issue
// ("Describe the issue") expected persistence to buy. In the
// non-persistent mode a workgroup owns one tile. In the stream-K mode a
// work unit is a k-range of a tile (a whole tile in the first waves, a
// piece of one at the tail); pieces store fp32 partial tiles that
// sk_fixup_kernel adds up.
//
// LDS layouts use 16-byte chunks, swizzled so that the fragment reads are
// bank-conflict-free on gfx950 (measured: 64 banks; ds_read_b128 serves
// lanes {0-7,16-23}, {8-15,24-31}, ... per pass; transpose reads serve 32
// lanes per pass):
//   A, 16-bit: BM rows (m) x 128 B; chunk c of row r at c ^ (r & 7).
//   A, fp8:    BM rows (m) x 128 B; chunk c of row r at c ^ sa8(r),
//              sa8(r) = ((r >> 1) & 1) | (r & 4).
//   B, 16-bit: 64 rows (k) x 2*BN B; chunk c of row r at
//              c ^ ((r & 1) + 4*((r >> 1) & 1) + 8*((r >> 3) & 1)).
//   B, fp8:    128 rows (k) x BN B; chunk c of row r at
//              c ^ ((r & 7) + 8*((r >> 5) & 1))          (BN = 256)
//              c ^ (((r >> 1) & 3) + 4*((r >> 5) & 1))   (BN = 128).
// A fragments are plain 16-byte reads of consecutive k. B is n-contiguous
// in memory, so its fragments come from the gfx950 LDS transpose reads
// (ds_read_b64_tr_b16 / _b8), which hand each lane one column's
// consecutive k values.
//
// The MFMA is issued with B as its first operand, so each lane's four
// outputs of a block are four columns of one row of C. For the 16-bit types
// the columns behind each MFMA block are permuted (n-position 4q + r of
// block nb is wave column 32*(nb/2) + 8q + 4*((nb + q) & 1) + r) so that a
// lane's outputs of blocks 2P and 2P+1 are eight consecutive columns: one
// 16-byte store each, and two store instructions cover 64 bytes of each of
// 16 rows. The transpose reads still fetch four consecutive columns per
// source lane; the B swizzle above keeps them conflict-free with this
// order. fp8 keeps the plain order (its transpose read hands out eight
// consecutive columns per source lane) and stores 8 bytes per block.
#pragma once

#include "device_common.h"

namespace pgemm {
namespace fast {

__host__ __device__ constexpr int block_k(int esize) { return 128 / esize; }

enum TileConfig : int { kTile256 = 0, kTile128 = 1 };

template <int CFG>
struct Tile;
template <>
struct Tile<kTile256> {
  static constexpr int BM = 256, BN = 256, WAVES = 8, WGM = 2, WGN = 4;
  static constexpr int MIN_WAVES_PER_SIMD = 2;
};
template <>
struct Tile<kTile128> {
  static constexpr int BM = 128, BN = 128, WAVES = 4, WGM = 2, WGN = 2;
  static constexpr int MIN_WAVES_PER_SIMD = 2; // two workgroups per CU
};

// Compile-time loop: f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>).
template <class F, int... I>
__device__ __attribute__((always_inline)) inline void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __attribute__((always_inline)) inline void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Swizzle of B's LDS rows: row k's chunk c is stored at chunk c ^ b_swz(k).
template <int ES, int B_ROW>
__host__ __device__ constexpr int b_swz(int k) {
  return ES == 2 ? (k & 1) + 4 * ((k >> 1) & 1) + 8 * ((k >> 3) & 1)
                 : (B_ROW == 256 ? (k & 7) + 8 * ((k >> 5) & 1) : ((k >> 1) & 3) + 4 * ((k >> 5) & 1));
}

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
template <int DT, int B_ROW>
__device__ inline typename Frag<DT>::t read_b(const uint8_t* base) {
  if constexpr (Traits<DT>::esize == 2) {
    // two transpose reads: k rows +0..3 and +4..7 of the lane group's 8 k
    fp16x4_raw_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16(PGEMM_LDS(fp16x4_raw_t, base));
    fp16x4_raw_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16(PGEMM_LDS(fp16x4_raw_t, base + 4 * B_ROW));
    intx2_t l = __builtin_bit_cast(intx2_t, lo), h = __builtin_bit_cast(intx2_t, hi);
    intx4_t w = {l[0], l[1], h[0], h[1]};
    return __builtin_bit_cast(typename Frag<DT>::t, w);
  } else {
    // four transpose reads of 8 k each (k rows +0, +8, +16, +24)
    intx2_t r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(PGEMM_LDS(intx2_t, base));
    intx2_t r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(PGEMM_LDS(intx2_t, base + 8 * B_ROW));
    intx2_t r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(PGEMM_LDS(intx2_t, base + 16 * B_ROW));
    intx2_t r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(PGEMM_LDS(intx2_t, base + 24 * B_ROW));
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

// TRACE selects the instantiation that writes the tile trace (p.trace); the
// timed kernels carry no trace code at all, so their register allocation is
// untouched by it. BT selects B given as N x K row-major (K contiguous, the
// layout of a linear layer's weight): B's tile is then copied and swizzled
// exactly like A's (BN rows of 128 bytes), and its fragments are plain
// 16-byte reads instead of LDS transpose reads. Each lane reads the B row
// that the permuted column order gives its n-position, so the MFMAs see the
// same operands as with K x N B and C is bitwise the same.
template <int DT, int SCHED, int CFG, bool TRACE, bool BT>
__global__ void __launch_bounds__(Tile<CFG>::WAVES * 64, Tile<CFG>::MIN_WAVES_PER_SIMD) gemm_fast_kernel(Params p) {
  constexpr int BM = Tile<CFG>::BM, BN = Tile<CFG>::BN;
  constexpr int WAVES = Tile<CFG>::WAVES, THREADS = WAVES * 64;
  constexpr int WGN = Tile<CFG>::WGN;             // waves along n
  constexpr int WTM = BM / Tile<CFG>::WGM;        // rows of a wave's sub-tile
  constexpr int MB = WTM / 16;                    // 16-row MFMA blocks per wave (8 or 4)
  constexpr int WN = BN / WGN;                    // columns of a wave's sub-tile
  constexpr int NB = WN / 16;                     // 16-column MFMA blocks per wave (4 or 8)
  static_assert(NB == 4 || NB == 8, "a wave owns 64 or 128 columns");
  constexpr int ES = Traits<DT>::esize;
  constexpr int BK = block_k(ES);                // k elements per step
  constexpr int KSUB = BK / Traits<DT>::kgroup;  // MFMA k-groups per step (2 or 1)
  constexpr int A_ROW = 128;                     // bytes per A row in LDS
  constexpr int A_BYTES = BM * A_ROW;            // 32 or 16 KiB per stage
  constexpr int B_ROW = BN * ES;                 // bytes per B row in LDS (512, 256 or 128)
  constexpr int B_BYTES = BK * B_ROW;            // 32 or 16 KiB per stage
  constexpr int B_CPR = B_ROW / 16;              // 16-byte chunks per B row
  constexpr int B_RPI = 1024 / B_ROW;            // B rows per 1 KiB copy instruction
  constexpr int LA = A_BYTES / (THREADS * 16), LB = B_BYTES / (THREADS * 16);
  constexpr int L = LA + LB;                     // copy instructions per thread per step
  static_assert(LA * THREADS * 16 == A_BYTES && LB * THREADS * 16 == B_BYTES && (L & 1) == 0,
                "each thread copies whole 16-byte chunks, in pairs of instructions");
  static_assert(L / 2 <= MB, "the fp8 step issues one copy pair per MFMA row");
  static_assert(MB <= 8, "fragment arrays sized for at most 8 row blocks");
  typedef typename Traits<DT>::out_t out_t;
  typedef typename Frag<DT>::t frag_t;
  typedef std::integral_constant<int, 0> I0;
  typedef std::integral_constant<int, 1> I1;

  __shared__ __attribute__((aligned(1024))) uint8_t sA0[A_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[B_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[A_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[B_BYTES];
  __shared__ int s_ring[8]; // claiming modes: tile id of tile-sequence number q at q % 8

  auto bufA = [&](auto c) __attribute__((always_inline)) -> uint8_t* {
    return decltype(c)::value == 0 ? sA0 : sA1;
  };
  auto bufB = [&](auto c) __attribute__((always_inline)) -> uint8_t* {
    return decltype(c)::value == 0 ? sB0 : sB1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // wave-uniform, lives in an SGPR
  const int wm = wave / WGN, wn = wave % WGN;                // WGM x WGN waves of WTM x 64
  const int M = p.M, N = p.N, K = p.K, T = p.T, G = p.G;
  // k-steps per tile, rounded up to even so that every tile starts on stage
  // 0 (an extra step reads zeros: it lies past K)
  const int nk = ((K + BK - 1) / BK + 1) & ~1;
  const int64_t lda = (int64_t)p.lda * ES; // bytes per row of A
  const int64_t ldb = (int64_t)p.ldb * ES; // bytes per row of B (K x N, or N x K when BT)
  const int64_t ldc = p.ldc;               // elements per row of C

  // ---- per-lane constants of the global -> LDS copy ------------------------
  // Instruction q = wave + WAVES*j fills one 1 KiB block of a stage: A rows
  // 8q..8q+7 (lane -> row 8q + lane/8, physical chunk lane % 8); B rows
  // B_RPI*q .. B_RPI*q + B_RPI-1 (lane -> row B_RPI*q + lane/B_CPR, physical
  // chunk lane % B_CPR). Each lane fetches the global chunk that the swizzle
  // stores at its physical position (the swizzles are XOR involutions). They
  // depend on row bits that are constant per lane and wave, and for fp8 B
  // also on the parity of j.
  const int a_row0 = 8 * wave + (lane >> 3); // + 8*WAVES j
  int a_chunk;
  if constexpr (ES == 2) {
    a_chunk = (lane & 7) ^ (lane >> 3);
  } else {
    const int r = lane >> 3;
    a_chunk = (lane & 7) ^ (((r >> 1) & 1) | (r & 4));
  }
  const int b_row0 = B_RPI * wave + lane / B_CPR; // + B_RPI*WAVES j
  // Instruction JB adds B_RPI*WAVES*JB rows, which only sets row bits above those of b_row0;
  // the swizzle is a sum of single-bit terms, so its value for the sum is the XOR of the two.
  const int b_chunk0 = (lane % B_CPR) ^ b_swz<ES, B_ROW>(b_row0);

  // ---- per-lane constants of the fragment reads ----------------------------
  const int g = lane >> 4, s16 = lane & 15;
  int a_off[KSUB][2];
  {
    const int r = wm * WTM + s16; // + mb * 16
#pragma unroll
    for (int kk = 0; kk < KSUB; ++kk) {
      if constexpr (ES == 2) {
        a_off[kk][0] = r * A_ROW + 16 * ((4 * kk + g) ^ (s16 & 7));
        a_off[kk][1] = a_off[kk][0];
      } else {
        const int sw = ((s16 >> 1) & 1) | (s16 & 4);
        a_off[kk][0] = r * A_ROW + 16 * ((2 * g) ^ sw);
        a_off[kk][1] = r * A_ROW + 16 * ((2 * g + 1) ^ sw);
      }
    }
  }
  int b_off[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if constexpr (BT) {
      // N x K B: this lane's B row is the wave column of its n-position s16
      // (16-bit: the permuted order below; fp8: plain), stored like an A row
      if constexpr (ES == 2) {
        const int q = s16 >> 2;
        const int r = wn * WN + 32 * (nb >> 1) + 8 * q + 4 * ((nb + q) & 1) + (s16 & 3);
        b_off[nb] = r * A_ROW + 16 * (g ^ (r & 7)); // k-group 1: chunk 4 + g, i.e. offset ^ 64
      } else {
        const int r = wn * WN + nb * 16 + s16;
        b_off[nb] = r * A_ROW + 16 * ((2 * g) ^ (((r >> 1) & 1) | (r & 4))); // second chunk: ^ 16
      }
      continue;
    }
    // the swizzle is the same for every row this lane reads from here
    // (+4 and +32 rows for 16-bit, +8/+16/+24 for fp8)
    if constexpr (ES == 2) {
      // source lane q = s16 & 3 of a row reads the four columns at wave
      // column 32*(nb/2) + 8q + 4*((nb + q) & 1) (permuted order)
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

  // ---- the tile sequence of this workgroup ---------------------------------
  // Sequence number q -> tile id. Static: blockIdx + q*G; non-persistent:
  // blockIdx for q = 0 only; dynamic: blockIdx for q = 0; cancel-and-reuse:
  // claimed for q = 0 too. In the claiming modes thread 0 claims tile 1 (and
  // tile 0) before the pipeline starts and then, in each tile's epilogue,
  // the tile two ahead: the claim is issued before the C stores and its
  // result written to s_ring after them, so the atomic's latency hides
  // behind the stores, and the next barrier publishes it before the copy
  // of that tile can begin. Keeping the claim code out of the k-loop keeps
  // its registers out of the loop too. (Stream-K does not use tile_of: its
  // work units come from the walkers below.)
  constexpr bool CLAIMS = SCHED == kDynamic || SCHED == kCancel;
  bool claim_live = false;    // thread 0 only: the last claim got a tile
  // Cancel-and-reuse with tiles of >= 4 k-steps: the claim of tile sequence number 1 is
  // issued after the first k-step's barrier and finished at the second's, not in the
  // prologue. Made in the prologue, the claims of the first workgroups to start took tiles
  // before the last workgroups of the same wave had made their first claim (measured at
  // 4096^3, 256 tiles on 256 workgroups: 16 workgroups ran two tiles and 16 none, doubling
  // the run). The producer needs tile 1 only from step nk - 2 >= 2 on.
  const bool defer_t1 = SCHED == kCancel && nk >= 4;
  int t1_raw = 0; // thread 0: the deferred claim's counter value
  auto tile_of = [&](int q) __attribute__((always_inline)) -> int {
    if constexpr (SCHED == kNonPersistent) {
      return q == 0 ? (int)blockIdx.x : T;
    } else if constexpr (SCHED == kStatic) {
      const int64_t t = (int64_t)blockIdx.x + (int64_t)q * G;
      return t < T ? (int)t : T;
    } else if constexpr (SCHED == kDynamic) {
      return q == 0 ? (int)blockIdx.x : __builtin_amdgcn_readfirstlane(s_ring[q & 7]);
    } else {
      return __builtin_amdgcn_readfirstlane(s_ring[q & 7]);
    }
  };

  // stream-K: the producer and the consumer each walk this workgroup's
  // work units (tile, k-step range); tile T past the last
  constexpr bool SK = SCHED == kStreamK;
  SkWalker p_walk, c_walk;
  if constexpr (SK) {
    p_walk.init((int)blockIdx.x, G, p.sk_waves, T, p.sk_tiles, p.sk_groups, nk >> 1);
    c_walk = p_walk;
  }
  auto next_unit = [&](SkWalker& wk, int* kb, int* ke) __attribute__((always_inline)) -> int {
    int t;
    return wk.next(&t, kb, ke) ? t : T;
  };

  // ---- producer: the copy of step `issued` ----------------------------------
  // begin_copy() resolves the step's tile and k and builds the buffer
  // resources; copy_part<J>() issues its J-th 1 KiB instruction.
  int issued = 0;      // copies begun
  int p_tile = 0;      // tile of the copy in progress
  bool p_done = false; // no more steps to copy
  bool p_busy = false; // the begun copy has instructions left
  __amdgpu_buffer_rsrc_t ra, rb;
  bool p_kval = false;
  int p_mrem = 0, p_krem = 0, p_nrem = 0;
  const uint32_t a_base = (uint32_t)a_row0 * (uint32_t)lda + 16u * (uint32_t)a_chunk;
  int p_kt = 0, p_ke = 0; // stream-K: next step, end of the unit's k-step range
  // Row strides and the wave's LDS block column, made opaque at each step so the
  // per-instruction offsets and LDS destinations are recomputed from them with
  // one scalar operation each instead of being hoisted out of the loop as some
  // two dozen loop invariants (which exhaust the SGPRs and push values to VGPRs).
  int lda_s = (int)lda, ldb_s = (int)ldb, wv_s = wave * 1024;
  auto begin_copy = [&]() __attribute__((always_inline)) {
    asm volatile("" : "+s"(lda_s), "+s"(ldb_s), "+s"(wv_s));
    if (p_done) return;
    int kt;
    if constexpr (SK) {
      if (p_kt == p_ke) {
        p_tile = next_unit(p_walk, &p_kt, &p_ke);
        if ((unsigned)p_tile >= (unsigned)T) {
          p_done = true;
          return;
        }
      }
      kt = p_kt++;
    } else {
      const int q = issued / nk;
      kt = issued - q * nk;
      if (kt == 0) {
        p_tile = tile_of(q);
        // any id outside [0, T) ends the sequence (a ring entry is only ever a tile id or
        // T; the unsigned compare keeps even a corrupt negative value off the tile grid)
        if ((unsigned)p_tile >= (unsigned)T) {
          p_done = true;
          return;
        }
      }
    }
    int pm, pn;
    tile_coords(p_tile, p, &pm, &pn);
    const int m0 = pm * BM, n0 = pn * BN, k0 = kt * BK;
    // A rebased at (m0, k0), B at (k0, n0); rows past M or K and chunks past
    // K or N read zeros.
    ra = make_rsrc(p.A + (int64_t)m0 * lda + (int64_t)k0 * ES);
    rb = BT ? make_rsrc(p.B + (int64_t)n0 * ldb + (int64_t)k0 * ES) : make_rsrc(p.B + (int64_t)k0 * ldb + (int64_t)n0 * ES);
    p_mrem = M - m0;
    p_krem = K - k0;
    p_nrem = BT ? N - n0 : (N - n0) * ES; // BT: rows of N x K B left
    p_kval = (k0 * ES + 16 * a_chunk) < K * ES;
    p_busy = true;
    ++issued;
  };
  auto copy_part = [&](uint8_t* sA, uint8_t* sB, auto jc) __attribute__((always_inline)) {
    constexpr int J = decltype(jc)::value;
    if (!p_busy) return;
    // per-lane base in voffset (kOOB when masked), the instruction's row offset in soffset
    if constexpr (J < LA) {
      const bool ok = p_kval & (a_row0 + 8 * WAVES * J < p_mrem);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, PGEMM_LDS(void, sA + WAVES * J * 1024 + wv_s), 16, ok ? a_base : kOOB,
                                               8 * WAVES * J * lda_s, 0, 0);
    } else {
      constexpr int JB = J - LA;
      if constexpr (BT) {
        // rows n of N x K B, copied like A's rows m (same lanes, chunks and swizzle)
        const bool ok = p_kval & (a_row0 + 8 * WAVES * JB < p_nrem);
        const uint32_t base = (uint32_t)a_row0 * (uint32_t)ldb + 16u * (uint32_t)a_chunk;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, PGEMM_LDS(void, sB + WAVES * JB * 1024 + wv_s), 16, ok ? base : kOOB,
                                                 8 * WAVES * JB * ldb_s, 0, 0);
      } else {
        const int row = b_row0 + B_RPI * WAVES * JB;
        const int Lc = b_chunk0 ^ b_swz<ES, B_ROW>(B_RPI * WAVES * JB);
        const bool ok = (row < p_krem) & (16 * Lc < p_nrem);
        const uint32_t base = (uint32_t)b_row0 * (uint32_t)ldb + 16u * (uint32_t)Lc;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, PGEMM_LDS(void, sB + WAVES * JB * 1024 + wv_s), 16, ok ? base : kOOB,
                                                 B_RPI * WAVES * JB * ldb_s, 0, 0);
      }
    }
    if (J == L - 1) p_busy = false;
  };
  auto copy_pair = [&](auto c, auto pc) __attribute__((always_inline)) {
    constexpr int P = decltype(pc)::value;
    copy_part(bufA(c), bufB(c), std::integral_constant<int, 2 * P>{});
    copy_part(bufA(c), bufB(c), std::integral_constant<int, 2 * P + 1>{});
  };

  // ---- accumulators and fragments -------------------------------------------
  floatx4_t acc[MB][NB];
  frag_t af[2][MB], bf[2][NB];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    acc_drain(); // accvgpr writes -> MFMA srcC reads
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

  // tile trace: when the current unit began (each clock value is consumed at
  // once, so no scalar read is outstanding in the k-loop)
  long long t_begin = 0;

  // ---- epilogue: round to the output type and store one tile ---------------
  auto epilogue = [&](int tile) __attribute__((always_inline)) {
    acc_drain();
    int pm, pn;
    tile_coords(tile, p, &pm, &pn);
    const int mrow = pm * BM + wm * WTM + s16;
    out_t* C = reinterpret_cast<out_t*>(p.C);
    if constexpr (ES == 2) {
      // permuted order: blocks 2P and 2P+1 give this lane columns
      // 32P + 8g .. +7 (block 2P + (g & 1) the first four). N is a multiple
      // of 8, so each 16-byte store is wholly inside or outside C. Interior
      // tiles (the uniform common case) store without masks; the schedule
      // barriers keep each row block's accumulator reads next to its stores.
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

  // ---- stream-K: store the fp32 partial tile of a piece ---------------------
  // Workspace slot `slot` holds a BM x BN fp32 tile, row-major; each lane
  // writes its accumulator blocks at the rows and columns the epilogue
  // would give them in C.
  auto store_partial = [&](int slot) __attribute__((always_inline)) {
    acc_drain();
    float* base = p.work + (int64_t)slot * (BM * BN);
    const int r0 = wm * WTM + s16;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      float* row = base + (r0 + mb * 16) * BN + wn * WN;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = ES == 2 ? 32 * (nb >> 1) + 8 * g + 4 * ((nb & 1) ^ (g & 1)) : nb * 16 + 4 * g;
        *reinterpret_cast<floatx4_t*>(row + col) = acc_read(acc[mb][nb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (TRACE) {
      t_begin = trace_clock();
      asm volatile("" ::"s"(t_begin));
    }
  };

  // ---- one k-step on stage C --------------------------------------------------
  int cs = 0; // consumer step
  bool has_next = true;
  // fp8 step: barrier at the top, next copy right after it. The B fragments
  // and A's first row block are read before the first MFMA row; each further
  // A row block is read one MFMA row ahead (a burst of all reads was slower).
  auto step_top = [&](auto cst) __attribute__((always_inline)) {
    constexpr int C = decltype(cst)::value;
    typedef std::integral_constant<int, C ^ 1> ICN;
    const uint8_t* sA = bufA(cst);
    const uint8_t* sB = bufB(cst);
    wait_vmcnt<0>();
    if constexpr (SCHED == kCancel) {
      if (defer_t1 && cs == 1 && tid == 0) { // the deferred claim has returned: publish it
        const int t1 = claim_finish(p.counter, t1_raw, T, claim_offset<SCHED>(G), claim_total<SCHED>(T, G));
        s_ring[1] = t1;
        claim_live = t1 < T;
      }
    }
    __syncthreads();
    if constexpr (SCHED == kCancel) {
      if (defer_t1 && cs == 0 && tid == 0) t1_raw = claim_raw(p.counter);
    }
    begin_copy();
    has_next = p_busy;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) read_b_frag(I0{}, sB, 0, nb);
    read_a_frag(I0{}, sA, 0, 0);
    static_for<MB>([&](auto mbc) __attribute__((always_inline)) {
      constexpr int MBI = decltype(mbc)::value;
      if constexpr (MBI + 1 < MB) read_a_frag(I0{}, sA, 0, MBI + 1); // one row ahead
      mfma_row(I0{}, MBI);
      if constexpr (MBI < L / 2) copy_pair(ICN{}, std::integral_constant<int, MBI>{});
      __builtin_amdgcn_sched_barrier(0);
    });
    ++cs;
  };
  // mid-step variant (16-bit): the barrier sits between the two k-groups.
  // Before it: MFMAs of k-group 0 while k-group 1's fragments are read.
  // After it: the copy of step s+2 goes into this (now free) stage and the
  // next step's k-group-0 fragments are read during k-group 1's MFMAs.
  auto step_mid = [&](auto cst) __attribute__((always_inline)) {
    constexpr int C = decltype(cst)::value;
    typedef std::integral_constant<int, C ^ 1> ICN;
    const uint8_t* sA = bufA(cst);
    const uint8_t* sB = bufB(cst);
    const uint8_t* sAn = bufA(ICN{});
    const uint8_t* sBn = bufB(ICN{});
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      mfma_row(I0{}, mb);
      if (mb < NB) read_b_frag(I1{}, sB, 1, mb);
      read_a_frag(I1{}, sA, 1, mb);
      __builtin_amdgcn_sched_barrier(0);
    }
    has_next = issued > cs + 1;
    if (has_next) {
      wait_vmcnt<0>(); // this wave's copy of step cs+1 (and any older stores) landed
      if constexpr (SCHED == kCancel) {
        if (defer_t1 && cs == 1 && tid == 0) { // the deferred claim has returned: publish it
          const int t1 = claim_finish(p.counter, t1_raw, T, claim_offset<SCHED>(G), claim_total<SCHED>(T, G));
          s_ring[1] = t1;
          claim_live = t1 < T;
        }
      }
      __syncthreads(); // every wave's; and every wave has read all of stage C
      if constexpr (SCHED == kCancel) {
        if (defer_t1 && cs == 0 && tid == 0) t1_raw = claim_raw(p.counter);
      }
      begin_copy();    // step cs + 2 into stage C
      static_for<L / 2>([&](auto pc) __attribute__((always_inline)) { copy_pair(cst, pc); });
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      mfma_row(I1{}, mb);
      if (mb < NB) read_b_frag(I0{}, sBn, 0, mb); // stale but harmless without a next step
      read_a_frag(I0{}, sAn, 0, mb);
      __builtin_amdgcn_sched_barrier(0);
    }
    ++cs;
  };
  auto step = [&](auto cst) __attribute__((always_inline)) {
    if constexpr (KSUB == 2) step_mid(cst); else step_top(cst);
  };

  // ---- the (tile, k-step) pipeline -----------------------------------------
  auto copy_whole = [&](auto c) __attribute__((always_inline)) {
    begin_copy();
    static_for<L / 2>([&](auto pc) __attribute__((always_inline)) { copy_pair(c, pc); });
  };
  if constexpr (CLAIMS) {
    if (tid == 0) {
      int t0 = (int)blockIdx.x;
      if constexpr (SCHED == kCancel) {
        t0 = claim_tile(p.counter, T, claim_offset<SCHED>(G), claim_total<SCHED>(T, G));
        s_ring[0] = t0;
      }
      // dynamic with G >= T: no tile lies beyond the grid's own, so no claim is made at all
      // (the counter is left at 0); cancel-and-reuse always claims
      const bool may_claim = SCHED == kCancel || G < T;
      if (!defer_t1) {
        const int t1 = (t0 < T && may_claim) ? claim_tile(p.counter, T, claim_offset<SCHED>(G), claim_total<SCHED>(T, G)) : T;
        s_ring[1] = t1;
        claim_live = t1 < T;
      }
    }
    __syncthreads();
    if constexpr (SCHED == kCancel) {
      // a workgroup that found no tile left exits here, all of it at once
      if ((unsigned)tile_of(0) >= (unsigned)T) return;
    }
  }
  int c_kb = 0, c_ke = nk; // k-step range of the consumer's unit
  int c_tile = 0;
  if constexpr (SK) {
    c_tile = next_unit(c_walk, &c_kb, &c_ke);
    if (c_tile >= T) return; // a workgroup without work units (none are launched so; kept as a guard)
  }
  copy_whole(I0{}); // step 0 into stage 0
  if constexpr (KSUB == 2) {
    copy_whole(I1{}); // step 1 into stage 1 (nk >= 2: same tile)
    wait_vmcnt<L>();  // step 0's copy landed; step 1's may still fly
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) read_b_frag(I0{}, sB0, 0, nb);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) read_a_frag(I0{}, sA0, 0, mb);
  }
  int c_q = 0; // consumer tile sequence number
  if constexpr (!SK) c_tile = tile_of(0);
  if constexpr (TRACE) {
    t_begin = trace_clock();
    asm volatile("" ::"s"(t_begin));
  }
  for (;;) {
    zero_acc();
    for (int kt = c_kb; kt < c_ke; kt += 2) {
      step(I0{});
      step(I1{});
    }
    // tile finished: store it while the next tile's copies are in flight
    // (claiming modes: and claim the tile two ahead meanwhile)
    int claimed = T;
    if constexpr (CLAIMS) {
      if (tid == 0 && claim_live) {
        claimed = claim_tile(p.counter, T, claim_offset<SCHED>(G), claim_total<SCHED>(T, G));
        claim_live = claimed < T;
      }
    }
    if (SK && (c_kb != 0 || c_ke != nk))
      store_partial((int)blockIdx.x + c_tile - (T - p.sk_tiles));
    else
      epilogue(c_tile);
    if constexpr (CLAIMS) {
      if (tid == 0) s_ring[(c_q + 2) & 7] = claimed;
    }
    if (!has_next) break;
    if constexpr (SK) c_tile = next_unit(c_walk, &c_kb, &c_ke); else c_tile = tile_of(++c_q);
    // the producer resolved the same published entry and began this tile only if it lies in
    // [0, T); the consumer checks it too, so the two can never disagree on a corrupt entry
    if ((unsigned)c_tile >= (unsigned)T) break;
  }
}

// ---- stream-K fix-up ----------------------------------------------------------
// One launch after the stream-K kernel, on the same stream. Workgroup
// (s, y) finishes rows y*ROWS .. y*ROWS+ROWS-1 of split tile s: it adds the
// tile's partials slot by slot in k order (workgroups w0..w1 of the split
// in ascending order, so every run adds the same values in the same
// order), rounds the sum to nearest even and stores it. Each thread covers
// eight consecutive columns of one row: two 16-byte partial loads per slot
// and one 16-byte store. A tile that one workgroup computed whole (w0 ==
// w1) was stored by that workgroup and is skipped.
template <int DT, int CFG>
__global__ void __launch_bounds__(256) sk_fixup_kernel(Params p) {
  constexpr int BM = Tile<CFG>::BM, BN = Tile<CFG>::BN;
  constexpr int ES = Traits<DT>::esize, BK = block_k(ES);
  constexpr int TPR = BN / 8;       // threads per row
  constexpr int ROWS = 256 / TPR;   // rows per workgroup
  typedef typename Traits<DT>::out_t out_t;
  const int s = blockIdx.x;
  if (s >= p.sk_tiles) return;
  const int kp = (((p.K + BK - 1) / BK + 1) & ~1) >> 1;
  const int64_t S = (int64_t)p.sk_tiles * kp;
  const int w0 = sk_owner((int64_t)s * kp, S, p.sk_groups);
  const int w1 = sk_owner((int64_t)(s + 1) * kp - 1, S, p.sk_groups);
  if (w0 == w1) return;
  const int tile = p.T - p.sk_tiles + s;
  long long t_begin = 0;
  if (p.trace) {
    t_begin = trace_clock();
    asm volatile("" ::"s"(t_begin));
  }
  int pm, pn;
  tile_coords(tile, p, &pm, &pn);
  const int r = blockIdx.y * ROWS + (int)threadIdx.x / TPR;
  const int c = ((int)threadIdx.x % TPR) * 8;
  const int m = pm * BM + r, n = pn * BN + c;
  if (r < BM && m < p.M && n < p.N) { // N is a multiple of 8: the 8 columns are all inside
    const float* src = p.work + (int64_t)(w0 + s) * (BM * BN) + r * BN + c;
    floatx4_t lo = *reinterpret_cast<const floatx4_t*>(src);
    floatx4_t hi = *reinterpret_cast<const floatx4_t*>(src + 4);
    for (int w = w0 + 1; w <= w1; ++w) {
      src += (int64_t)BM * BN;
      lo += *reinterpret_cast<const floatx4_t*>(src);
      hi += *reinterpret_cast<const floatx4_t*>(src + 4);
    }
    if constexpr (ES == 1) { // e4m3 inputs: the partials are unscaled sums
      lo *= p.c_scale;
      hi *= p.c_scale;
    }
    store8(reinterpret_cast<out_t*>(p.C) + (int64_t)m * p.ldc + n, lo, hi, false);
  }
  if (blockIdx.y == 0 && threadIdx.x == 0) {
    if (p.visits) atomicAdd(p.visits + tile, 1);
    if (p.owner) p.owner[tile] = -1 - s; // stored by the fix-up, not by a workgroup of the GEMM grid
    if (p.trace) trace_tile(p.trace, tile, -1 - s, t_begin, trace_clock());
  }
}

} // namespace fast
} // namespace pgemm
