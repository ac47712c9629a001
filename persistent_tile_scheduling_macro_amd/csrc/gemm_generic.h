// The generic GEMM kernel: any M, N, K and any element alignment. It is
// the correctness path for shapes the fast kernel cannot take (K or N not a
// multiple of 16 bytes of elements, or unaligned bases), not a speed path.
//
// Macro tile 64 x 64, 256 threads = 4 waves of 32 x 32 (2 x 2 MFMA blocks).
// Each k-step copies one MFMA k-group of A (64 x kgroup) and B (kgroup x 64)
// element by element through registers with bounds checks (zero outside
// the matrix), storing A as [m][k] and B transposed as [n][k] in LDS so
// both fragments are contiguous reads. The tile schedulers are the same
// three as the fast kernel's: one tile per workgroup, a static stride of G
// over the tile order, or claims from the work counter (dynamic and
// cancel-and-reuse).
#pragma once

#include "device_common.h"

namespace pgemm {
namespace generic {

constexpr int BM = 64, BN = 64, THREADS = 256;

template <int DT, int SCHED>
__global__ void __launch_bounds__(THREADS) gemm_generic_kernel(Params p) {
  constexpr int ES = Traits<DT>::esize;
  constexpr int KG = Traits<DT>::kgroup;      // k per step
  constexpr int ROWB = KG * ES + 16;          // padded LDS row bytes
  typedef typename Traits<DT>::out_t out_t;

  __shared__ __attribute__((aligned(16))) uint8_t sA[BM * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t sB[BN * ROWB]; // B transposed: [n][k]
  __shared__ int s_claim;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4, s16 = lane & 15;
  const int nk = (p.K + KG - 1) / KG;
  typedef typename std::conditional<ES == 2, uint16_t, uint8_t>::type elem_t;
  const elem_t* A = reinterpret_cast<const elem_t*>(p.A);
  const elem_t* B = reinterpret_cast<const elem_t*>(p.B);
  out_t* C = reinterpret_cast<out_t*>(p.C);

  int tile = blockIdx.x;
  if constexpr (SCHED == kCancel) { // the first tile is claimed too
    if (tid == 0) s_claim = claim_tile(p.counter, p.T, claim_offset<SCHED>(p.G), claim_total<SCHED>(p.T, p.G));
    __syncthreads();
    tile = __builtin_amdgcn_readfirstlane(s_claim);
    __syncthreads();
  }
  while (tile < p.T) {
    long long t_begin = 0;
    if (p.trace) {
      t_begin = trace_clock();
      asm volatile("" ::"s"(t_begin));
    }
    int pm, pn;
    tile_coords(tile, p, &pm, &pn);
    const int m0 = pm * BM, n0 = pn * BN;
    floatx4_t acc[2][2];
    for (int i = 0; i < 2; ++i)
      for (int j = 0; j < 2; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    for (int kt = 0; kt < nk; ++kt) {
      const int k0 = kt * KG;
      for (int e = tid; e < BM * KG; e += THREADS) {
        const int r = e / KG, k = e % KG;
        const int gm = m0 + r, gk = k0 + k;
        elem_t v = (gm < p.M && gk < p.K) ? A[(int64_t)gm * p.lda + gk] : (elem_t)0;
        *reinterpret_cast<elem_t*>(sA + r * ROWB + k * ES) = v;
      }
      for (int e = tid; e < BN * KG; e += THREADS) {
        const int k = e / BN, c = e % BN;
        const int gk = k0 + k, gn = n0 + c;
        elem_t v = (gk < p.K && gn < p.N) ? B[p.b_nk ? (int64_t)gn * p.ldb + gk : (int64_t)gk * p.ldb + gn] : (elem_t)0;
        *reinterpret_cast<elem_t*>(sB + c * ROWB + k * ES) = v;
      }
      __syncthreads();
      for (int i = 0; i < 2; ++i) {
        for (int j = 0; j < 2; ++j) {
          const uint8_t* pa = sA + (wm * 32 + i * 16 + s16) * ROWB;
          const uint8_t* pb = sB + (wn * 32 + j * 16 + s16) * ROWB;
          if constexpr (ES == 2) {
            intx4_t a = *reinterpret_cast<const intx4_t*>(pa + 16 * g);
            intx4_t b = *reinterpret_cast<const intx4_t*>(pb + 16 * g);
            if constexpr (DT == kF16)
              acc[i][j] = mfma(__builtin_bit_cast(half8_t, b), __builtin_bit_cast(half8_t, a), acc[i][j]);
            else
              acc[i][j] = mfma(__builtin_bit_cast(bf16x8_t, b), __builtin_bit_cast(bf16x8_t, a), acc[i][j]);
          } else {
            intx4_t a0 = *reinterpret_cast<const intx4_t*>(pa + 32 * g);
            intx4_t a1 = *reinterpret_cast<const intx4_t*>(pa + 32 * g + 16);
            intx4_t b0 = *reinterpret_cast<const intx4_t*>(pb + 32 * g);
            intx4_t b1 = *reinterpret_cast<const intx4_t*>(pb + 32 * g + 16);
            intx8_t a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            intx8_t b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
            acc[i][j] = mfma(b, a, acc[i][j]);
          }
        }
      }
      __syncthreads();
    }
    // epilogue: lane holds C[m][n..n+3] of each 16 x 16 block
    for (int i = 0; i < 2; ++i) {
      const int m = m0 + wm * 32 + i * 16 + s16;
      if (m >= p.M) continue;
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + wn * 32 + j * 16 + 4 * g;
        for (int e = 0; e < 4; ++e)
          if (n + e < p.N)
            C[(int64_t)m * p.ldc + n + e] = to_out(ES == 1 ? acc[i][j][e] * p.c_scale : acc[i][j][e], (out_t*)nullptr);
      }
    }
    if (tid == 0) {
      if (p.visits) atomicAdd(p.visits + tile, 1);
      if (p.owner) p.owner[tile] = blockIdx.x;
      if (p.trace) trace_tile(p.trace, tile, blockIdx.x, t_begin, trace_clock());
    }
    if constexpr (SCHED == kNonPersistent) {
      break;
    } else if constexpr (SCHED == kStatic) {
      tile += p.G;
    } else if (SCHED == kDynamic && p.G >= p.T) {
      break; // no tile lies beyond the grid's own: no claim is made (the counter stays 0)
    } else {
      if (tid == 0) s_claim = claim_tile(p.counter, p.T, claim_offset<SCHED>(p.G), claim_total<SCHED>(p.T, p.G));
      __syncthreads();
      tile = __builtin_amdgcn_readfirstlane(s_claim);
      __syncthreads();
    }
  }
}

// C = 0 for K = 0 (an empty sum): rows x cols outputs, rows ldc elements apart.
template <class OutT>
__global__ void fill_zero_kernel(OutT* C, int64_t rows, int64_t cols, int64_t ldc) {
  const int64_t n = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    C[(i / cols) * ldc + i % cols] = (OutT)0.0f;
}

} // namespace generic
} // namespace pgemm
