// The fast GEMM kernel for aligned operands (K and N multiples of 16 bytes
// of elements, 16-byte aligned bases).
//
// Macro tile 256 x 256, 256 threads = 4 waves in a 2 x 2 arrangement, each
// wave owning a 128 x 128 sub-tile (8 x 8 blocks of 16 x 16 MFMA outputs,
// 256 fp32 accumulators per lane). K is consumed in steps of 128 bytes of
// elements (64 fp16/bf16 or 128 fp8). Each step's A (256 x 128 B) and B
// (128 B x 256 cols) slices are copied global -> LDS by buffer loads that
// write LDS directly (no register staging), into a two-stage LDS ring, so
// the copy of step s+1 overlaps the MFMAs of step s (the copy/compute
// overlap of the persistent-kernel forum thread, first answer).
//
// All three scheduling modes run this one body over a flattened sequence
// of (tile, k-step) pairs. The producer side (the loads) runs one step
// ahead of the MFMAs and crosses tile boundaries freely, so in the
// persistent modes the next tile's first loads are in flight while the
// current tile's epilogue converts and stores C -- the pipelining across
// output tiles the Triton persistent-matmul issue ("Describe the issue")
// expected persistence to buy. In the non-persistent mode a workgroup owns
// exactly one tile and the sequence ends there.
//
// LDS layouts (16-byte chunks, XOR-swizzled so the fragment reads below are
// bank-conflict-free whether the LDS serves 8 or 16 lanes of 16 bytes per
// cycle):
//   A stage: 256 rows (m) x 128 B (k); chunk c of row r sits at
//            c ^ fa(r), fa(r) = (r & 7) ^ ((r >> 3) & 1).
//   B stage, 16-bit: 64 rows (k) x 512 B (n); chunk c of row r sits at
//            c ^ (2*(r & 3) + 8*((r >> 3) & 1)).
//   B stage, fp8: 128 rows (k) x 256 B (n); chunk c of row r sits at
//            c ^ ((r & 7) + 8*((r >> 5) & 1)).
// A fragments are plain 16-byte reads of 8 (or 16) consecutive k. B is
// n-contiguous in memory, so its fragments come from the gfx950 LDS
// transpose reads (ds_read_b64_tr_b16 / _b8), which hand each lane one
// column's consecutive k values.
//
// The MFMA is issued with B as its first operand, so each lane's four
// outputs are four consecutive columns of one row of C (8-byte stores).
#pragma once

#include "device_common.h"

namespace pgemm {
namespace fast {

constexpr int BM = 256, BN = 256, THREADS = 256;
constexpr int STAGE_BYTES = 32768; // per operand per stage
constexpr int ROW_A = 128;         // bytes of k per A row in LDS

__host__ __device__ constexpr int block_k(int esize) { return 128 / esize; }

__device__ inline int fa(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int DT>
struct Frag;
template <>
struct Frag<kF16> { typedef half8_t t; };
template <>
struct Frag<kBF16> { typedef bf16x8_t t; };
template <>
struct Frag<kF8E4M3> { typedef intx8_t t; };

// Read the B fragment of one 16-column block: lane (16g + s) ends up with
// column (s) of the block and the k values its A partner holds.
template <int DT>
__device__ inline typename Frag<DT>::t read_b(const uint8_t* base) {
  typename Frag<DT>::t f;
  if constexpr (Traits<DT>::esize == 2) {
    // two transpose reads, rows +0..3 and +4..7 of the lane group's 8 k
    fp16x4_raw_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16(PGEMM_LDS(fp16x4_raw_t, base));
    fp16x4_raw_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16(PGEMM_LDS(fp16x4_raw_t, base + 4 * 512));
    intx2_t l = __builtin_bit_cast(intx2_t, lo), h = __builtin_bit_cast(intx2_t, hi);
    intx4_t w = {l[0], l[1], h[0], h[1]};
    f = __builtin_bit_cast(typename Frag<DT>::t, w);
  } else {
    // four transpose reads of 8 k each (rows +0, +8, +16, +24)
    intx2_t r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(PGEMM_LDS(intx2_t, base));
    intx2_t r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(PGEMM_LDS(intx2_t, base + 8 * 256));
    intx2_t r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(PGEMM_LDS(intx2_t, base + 16 * 256));
    intx2_t r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(PGEMM_LDS(intx2_t, base + 24 * 256));
    f = intx8_t{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
  }
  return f;
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
  constexpr int BK = block_k(ES);                 // k elements per step
  constexpr int KSUB = BK / Traits<DT>::kgroup;   // MFMA k-groups per step (2 or 1)
  constexpr int ROW_B = BN * ES;                  // bytes per B row in LDS (512 or 256)
  typedef typename Traits<DT>::out_t out_t;
  typedef typename Frag<DT>::t frag_t;

  __shared__ __attribute__((aligned(1024))) uint8_t sA0[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[STAGE_BYTES];
  __shared__ int s_claim[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // wave-uniform, lives in an SGPR
  const int wm = wave >> 1, wn = wave & 1;
  const int M = p.M, N = p.N, K = p.K, T = p.T;
  const int nk = (K + BK - 1) / BK;
  const int64_t lda = (int64_t)K * ES; // bytes per row of A
  const int64_t ldb = (int64_t)N * ES; // bytes per row of B
  const int64_t ldc = N;               // elements per row of C

  // ---- per-lane constants of the global -> LDS copy ------------------------
  // A: instruction q = wave + 4j (j < 8) fills rows 8q .. 8q+7; lane -> row
  // 8q + lane/8, physical chunk lane%8, logical chunk (lane%8) ^ fa(row).
  const int a_row0 = 8 * wave + (lane >> 3);                    // row for j = 0 (+32 per j)
  const int a_chunk = (lane & 7) ^ ((lane >> 3) ^ (wave & 1));  // fa(row) is the same for all j
  // B, 16-bit: instruction q fills rows 2q, 2q+1 (512 B each); fp8: rows 4q..4q+3 (256 B).
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

  // ---- per-lane constants of the fragment reads ------------------------------
  const int g = lane >> 4, s16 = lane & 15;
  // A: lane (16g + i) reads row wm*128 + mb*16 + i; fa depends on i only.
  int a_off[KSUB][2];
  {
    const int r = wm * 128 + s16;
    const int f = fa(s16);
#pragma unroll
    for (int kk = 0; kk < KSUB; ++kk) {
      if constexpr (ES == 2) {
        a_off[kk][0] = r * ROW_A + 16 * ((4 * kk + g) ^ f);
        a_off[kk][1] = a_off[kk][0];
      } else {
        a_off[kk][0] = r * ROW_A + 16 * ((2 * g) ^ f);
        a_off[kk][1] = r * ROW_A + 16 * ((2 * g + 1) ^ f);
      }
    }
  }
  // B: source lane (16g + s) supplies the address of one 8-byte piece.
  int b_off[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    if constexpr (ES == 2) {
      const int k = 8 * g + (s16 >> 2);                       // + 32*kk (+4 for the second read)
      const int L = wn * 16 + 2 * nb + ((s16 & 3) >> 1);
      const int h = 2 * (s16 >> 2) + 8 * (g & 1);
      b_off[nb] = k * ROW_B + 16 * (L ^ h) + 8 * (s16 & 1);
    } else {
      const int k = 32 * g + (s16 >> 1);                      // +8, +16, +24 for reads 1..3
      const int L = wn * 8 + nb;
      const int h = (s16 >> 1) + 8 * (g & 1);
      b_off[nb] = k * ROW_B + 16 * (L ^ h) + 8 * (s16 & 1);
    }
  }

  // ---- producer: issue the copy of one (tile, k-step) into a stage ----------
  auto issue_loads = [&](int tile, int kt, uint8_t* sA, uint8_t* sB) __attribute__((always_inline)) {
    int pm, pn;
    tile_coords(tile, p, &pm, &pn);
    const int m0 = pm * BM, n0 = pn * BN, k0 = kt * BK;
    // A: rebased at (m0, k0); offsets stay below 256 * lda. Rows past M and
    // k chunks past K read zeros.
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A + (int64_t)m0 * lda + (int64_t)k0 * ES);
    const int mrem = M - m0;
    const bool kval = (k0 * ES + 16 * a_chunk) < K * ES;
    const uint32_t a_base = (uint32_t)a_row0 * (uint32_t)lda + 16u * (uint32_t)a_chunk;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool ok = kval & (a_row0 + 32 * j < mrem);
      const uint32_t off = ok ? a_base + (uint32_t)(32 * j) * (uint32_t)lda : kOOB;
      load16_to_lds(ra, sA + (wave + 4 * j) * 1024, off);
    }
    // B: rebased at (k0, n0); offsets stay below BK * ldb.
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B + (int64_t)k0 * ldb + (int64_t)n0 * ES);
    const int krem = K - k0;
    const int nrem_bytes = (N - n0) * ES;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int row, L;
      if constexpr (ES == 2) {
        row = b_row0 + 8 * j;
        L = b_pchunk ^ (b_h0 + 8 * (j & 1));
      } else {
        row = b_row0 + 16 * j;
        L = b_pchunk ^ (b_h0 + 8 * ((j >> 1) & 1));
      }
      const bool ok = (row < krem) & (16 * L < nrem_bytes);
      const uint32_t off = ok ? (uint32_t)row * (uint32_t)ldb + 16u * (uint32_t)L : kOOB;
      load16_to_lds(rb, sB + (wave + 4 * j) * 1024, off);
    }
  };

  // ---- consumer: MFMAs of one stage ------------------------------------------
  floatx4_t acc[8][8];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    acc_drain(); // accvgpr writes -> MFMA srcC reads
  };
  // Fragments are software-pipelined: while the 64 MFMAs of k-group kk run,
  // the LDS reads of k-group kk+1 are issued in eight chunks, one after each
  // row of MFMAs. sched_barrier pins that order (the MFMAs are inline asm,
  // whose latency the compiler cannot see).
  auto read_a_frag = [&](const uint8_t* sA, int kk, int mb) __attribute__((always_inline)) {
    return read_a<DT>(sA + a_off[kk][0] + mb * 16 * ROW_A, sA + a_off[kk][1] + mb * 16 * ROW_A);
  };
  auto read_b_frag = [&](const uint8_t* sB, int kk, int nb) __attribute__((always_inline)) {
    return read_b<DT>(sB + b_off[nb] + kk * 32 * ROW_B);
  };
  auto compute = [&](const uint8_t* sA, const uint8_t* sB) __attribute__((always_inline)) {
    frag_t af[2][8], bf[2][8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) bf[0][nb] = read_b_frag(sB, 0, nb);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) af[0][mb] = read_a_frag(sA, 0, mb);
#pragma unroll
    for (int kk = 0; kk < KSUB; ++kk) {
      const int c = kk & 1, n = c ^ 1;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) mfma_acc(acc[mb][nb], bf[c][nb], af[c][mb]);
        if (kk + 1 < KSUB) {
          bf[n][mb] = read_b_frag(sB, kk + 1, mb);
          af[n][mb] = read_a_frag(sA, kk + 1, mb);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
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

  // ---- the (tile, k-step) pipeline -----------------------------------------
  // The producer runs one k-step ahead of the MFMAs. On a tile's last
  // k-step it already issues the next tile's first copy, so that copy is in
  // flight while the epilogue below stores the finished tile. In the dynamic
  // mode thread 0 claims tile j+1 in the step that starts copying tile j and
  // publishes the claim through one of two LDS slots after that step's
  // MFMAs; the claim is read one or more barriers later, so its latency is
  // hidden behind a whole k-step.
  int tile = blockIdx.x;
  int claim_slot = 0; // slot holding the claim for the tile after `tile`
  if constexpr (SCHED == kDynamic) {
    if (tid == 0) s_claim[0] = claim_tile(p.counter, T, p.G);
  }
  issue_loads(tile, 0, sA0, sB0);
  int start = 0; // stage holding the current tile's first k-step

  // One k-step on stage S; returns the tile the producer moved to (or T).
  auto step = [&](auto stage, int kt, int next) __attribute__((always_inline)) -> int {
    constexpr int S = decltype(stage)::value;
    uint8_t* sAc = S == 0 ? sA0 : sA1;
    uint8_t* sBc = S == 0 ? sB0 : sB1;
    uint8_t* sAn = S == 0 ? sA1 : sA0;
    uint8_t* sBn = S == 0 ? sB1 : sB0;
    __builtin_amdgcn_s_waitcnt(0x0F70); // vmcnt(0): this wave's copies into stage S landed
    __syncthreads();                    // ... and every wave's; nobody still reads stage 1-S
    int claim_val = 0;
    bool pending = false;
    if (kt + 1 < nk) {
      issue_loads(tile, kt + 1, sAn, sBn);
    } else {
      if constexpr (SCHED == kNonPersistent) {
        next = T;
      } else if constexpr (SCHED == kStatic) {
        next = tile + p.G;
      } else {
        next = __builtin_amdgcn_readfirstlane(s_claim[claim_slot]);
      }
      if (next < T) {
        if constexpr (SCHED == kDynamic) {
          if (tid == 0) {
            claim_val = claim_tile(p.counter, T, p.G);
            pending = true;
          }
        }
        issue_loads(next, 0, sAn, sBn);
      }
    }
    compute(sAc, sBc);
    if constexpr (SCHED == kDynamic) {
      if (pending) s_claim[claim_slot ^ 1] = claim_val;
    }
    return next;
  };

  for (;;) {
    zero_acc();
    int next = T;
    int kt = 0;
    if (start == 1) {
      next = step(std::integral_constant<int, 1>{}, kt, next);
      ++kt;
    }
    for (; kt + 1 < nk; kt += 2) {
      next = step(std::integral_constant<int, 0>{}, kt, next);
      next = step(std::integral_constant<int, 1>{}, kt + 1, next);
    }
    if (kt < nk) next = step(std::integral_constant<int, 0>{}, kt, next);
    epilogue(tile);
    if (next >= T) break;
    tile = next;
    start = (start + nk) & 1;
    if constexpr (SCHED == kDynamic) claim_slot ^= 1;
  }
}

} // namespace fast
} // namespace pgemm
