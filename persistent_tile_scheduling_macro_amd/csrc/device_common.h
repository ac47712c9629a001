// Device-side building blocks shared by the GEMM kernels: element traits,
// fragment types, buffer resources and zero-filling LDS loads, the tile
// order, the tile schedulers' claim protocol and the stream-K split.
//
// The operation is the GEMM of the persistent-kernel forum thread
// (question): C = A*B cut into output tiles, each tile handed to one
// workgroup by a tile scheduler. Layouts: A is M x K row-major, B is K x N
// row-major, C is M x N row-major.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace pgemm {

// ---------------------------------------------------------------- types
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef int intx8_t __attribute__((ext_vector_type(8)));
typedef int intx4_t __attribute__((ext_vector_type(4)));
typedef int intx2_t __attribute__((ext_vector_type(2)));
typedef __fp16 fp16x4_raw_t __attribute__((__vector_size__(8)));

#define PGEMM_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

enum DType : int { kF16 = 0, kBF16 = 1, kF8E4M3 = 2 };
enum Sched : int { kNonPersistent = 0, kStatic = 1, kDynamic = 2, kCancel = 3, kStreamK = 4 };

// Per-dtype facts used by the kernels. A "k-group" is the reduction depth
// of one MFMA: 32 for the 16-bit types (v_mfma_f32_16x16x32_{f16,bf16}),
// 128 for OCP e4m3 (v_mfma_f32_16x16x128_f8f6f4). Each lane of a 16x16
// MFMA holds 16 bytes (16-bit types) or 32 bytes (fp8) of one row of A and
// of one column of B.
template <int DT> struct Traits;
template <> struct Traits<kF16> {
  static constexpr int esize = 2;   // bytes per input element
  static constexpr int kgroup = 32; // k per MFMA
  typedef _Float16 out_t;
};
template <> struct Traits<kBF16> {
  static constexpr int esize = 2;
  static constexpr int kgroup = 32;
  typedef __bf16 out_t;
};
template <> struct Traits<kF8E4M3> {
  static constexpr int esize = 1;
  static constexpr int kgroup = 128;
  typedef __bf16 out_t;
};

// ------------------------------------------------------- kernel arguments
struct Params {
  const uint8_t* A;
  const uint8_t* B;
  uint8_t* C;
  int M, N, K;
  int lda, ldb, ldc; // leading dimensions in elements (A rows, B rows in its layout, C rows)
  int n_m, n_n, T; // tile grid and tile count
  int G;           // workgroups launched
  int group_m;     // GROUP_SIZE_M of the tile order (>= 1)
  int xcd_chunk;   // >0: XCD-aware remap inside chunks of this many tiles
  int* counter;    // dynamic scheduler's work counter (reads 0 between launches)
  int* visits;     // optional int32[T] tile-visit counter
  int* owner;      // optional int32[T] owner log (workgroup id per tile)
  long long* trace; // optional int64[4T] tile trace {workgroup, XCD, start, end}
  int b_nk;         // 1: B is N x K row-major (K contiguous); 0: K x N row-major
  float c_scale;    // e4m3 inputs: product of the per-tensor scales of A and B (else 1)
  // stream-K only (zero otherwise): the first T - sk_tiles tiles run whole,
  // sk_waves per workgroup; the k-step pairs of the last sk_tiles tiles are
  // split over workgroups 0 .. sk_groups-1; pieces that do not cover their
  // whole tile leave fp32 partial tiles in `work` for the fix-up kernel.
  int sk_waves, sk_tiles, sk_groups;
  float* work;
};

// ------------------------------------------------------------ tile order
// Tile id t -> (pid_m, pid_n). Two steps, applied identically in every
// scheduling mode so that only the scheduling differs between modes:
//
// 1. XCD-aware remap. Workgroup ids are dealt round-robin over the 8 XCDs
//    (from a starting XCD that carries over between launches), and in the
//    persistent modes workgroup w owns tiles t = w (mod G) with G a multiple
//    of the CU count, so all tiles with the same t mod 8 run on one XCD.
//    Inside each full chunk of `xcd_chunk` tiles the remap makes each such
//    class consecutive, so step 2 gives every XCD a compact block of the
//    output (shared operand rows and columns stay in that XCD's L2).
// 2. Grouped order (the GROUP_SIZE_M knob of the Triton persistent-matmul
//    issue, "What I've tried" / follow-up comment): walk down groups of
//    group_m tile rows column by column. group_m = 1 is plain row-major.
__host__ __device__ inline int xcd_remap(int t, int T, int chunk) {
  if (chunk <= 0 || (chunk & 7) != 0) return t;
  int base = t - t % chunk;
  if (base + chunk > T) return t; // partial last chunk keeps the identity order
  int u = t - base;
  return base + (u & 7) * (chunk >> 3) + (u >> 3);
}

__host__ __device__ inline void grouped_tile(int t, int n_m, int n_n, int group_m, int* pm, int* pn) {
  int width = group_m * n_n;
  int group = t / width;
  int first_m = group * group_m;
  int gs = n_m - first_m < group_m ? n_m - first_m : group_m;
  int r = t - group * width;
  *pm = first_m + r % gs;
  *pn = r / gs;
}

__host__ __device__ inline void tile_coords(int t, const Params& p, int* pm, int* pn) {
  grouped_tile(xcd_remap(t, p.T, p.xcd_chunk), p.n_m, p.n_n, p.group_m, pm, pn);
}

// ---------------------------------------------------- dynamic work counter
// Claim protocol of the two claiming modes, the AMD analogue of cluster
// launch control (KernelWiki "Persistent Kernels with Cluster Launch
// Control", intro): the grid defines the candidate ids, a claim returns the
// next unstarted id, and a failed claim means the worker never claims again.
//
// * dynamic persistent (grid G): every workgroup starts on tile blockIdx.x
//   without a claim; claim value c names tile c + G.
// * cancel-and-reuse (grid T): every workgroup claims even its first tile;
//   claim value c names tile c. A workgroup that starts after every tile is
//   taken fails its first claim and exits at once -- the stand-in for a
//   cluster whose launch was cancelled and whose id was reused.
//
// Each workgroup makes exactly one failing claim, so a launch makes exactly
// `total` claims (T for dynamic, T + G for cancel-and-reuse) and they return
// the counter values 0..total-1 once each (a dynamic launch with G >= T, where
// every workgroup has at most its own tile, makes no claim at all); the claim that returns total-1 is
// the launch's last and resets the counter to 0 for the next launch on the
// stream. A value outside [0, total) cannot come from this protocol and is
// treated as a failed claim, so a corrupted counter never names a tile
// outside the grid. (Claims are handed out in the order they arrive, which
// at a launch's start is close to workgroup order, so the tiles a
// workgroup gets are close to the ones the static mode would give it.
// Separate per-XCD counters measured slower.) Host-callable too, so a CPU test can race it.
__host__ __device__ inline int claim_raw(int* counter) {
  return __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The rest of a claim once its counter value c is back: the last claim of the launch resets
// the counter; c names tile c + offset, or none (T). Split from claim_raw so that a kernel
// can issue the atomic and finish the claim later, when the value has returned.
__host__ __device__ inline int claim_finish(int* counter, int c, int T, int offset, int total) {
  if (c == total - 1) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return (c < 0 || c >= total || c + offset >= T) ? T : c + offset;
}
__host__ __device__ inline int claim_tile(int* counter, int T, int offset, int total) {
  return claim_finish(counter, claim_raw(counter), T, offset, total);
}

// Claim parameters of a scheduling mode: (offset, total) of claim_tile.
template <int SCHED>
__host__ __device__ inline int claim_offset(int G) { return SCHED == kCancel ? 0 : G; }
template <int SCHED>
__host__ __device__ inline int claim_total(int T, int G) { return SCHED == kCancel ? T + G : T; }

// ------------------------------------------------------ stream-K split
// Tail handling that adds work units instead of idling CUs. With T = W*G + R
// tiles on G workgroups the static mapping leaves the last wave R/G full;
// the static and dynamic schedulers cannot fix that, because neither
// creates more independent work than the tiles (KernelWiki "Persistent
// Kernels with Cluster Launch Control", "Choosing between static and CLC
// scheduling"). Here the first W*G tiles in tile order run whole (workgroup
// w takes w, w+G, ..., as in the static mode) and the k-steps of the last R
// tiles are laid end to end, in pairs (kp pairs per tile, so every piece
// starts on stage 0 of the two-stage ring), and cut into sk_groups
// contiguous ranges of equal length, one per workgroup:
//   range of workgroup w: pair positions [w*S/Gs, (w+1)*S/Gs), S = R*kp.
// A range crosses tile boundaries, so it is a sequence of pieces, each the
// part of one tile's k-range that lies in it. A piece that is a whole tile
// is stored to C as usual; any other piece stores its fp32 partial tile in
// workspace slot w + s (s = tile - W*G): along the pair positions each new
// piece starts at a workgroup boundary or a tile boundary, so w + s grows
// by at least one from piece to piece and the slots of distinct pieces
// differ. A fix-up launch then adds each split tile's partials in k order
// (deterministic: the same bits on every run) and rounds them to C. The
// split needs 1 <= Gs <= S, so that every range holds at least one pair
// and the workgroups w0..w1 of a split tile all left a partial in it.

// Workgroup whose range holds pair position x: the w with
// floor(w*S/Gs) <= x < floor((w+1)*S/Gs), i.e. ceil((x+1)*Gs/S) - 1.
__host__ __device__ inline int sk_owner(int64_t x, int64_t S, int Gs) {
  return (int)(((x + 1) * Gs + S - 1) / S - 1);
}
__host__ __device__ inline int64_t sk_range_begin(int w, int64_t S, int Gs) { return (int64_t)w * S / Gs; }

// Work unit q of workgroup w: sets tile, and the k-step range [kb, ke) of
// it (even numbers; nk = 2*kp is a whole tile); returns false past the
// workgroup's last unit. G = launch grid, W = whole-tile waves.
__host__ __device__ inline bool sk_unit(int q, int w, int G, int W, int T, int R, int Gs, int kp, int* tile,
                                        int* kb, int* ke) {
  if (q < W) {
    *tile = q * G + w;
    *kb = 0;
    *ke = 2 * kp;
    return true;
  }
  if (R == 0 || w >= Gs) return false;
  const int64_t S = (int64_t)R * kp;
  const int64_t b = sk_range_begin(w, S, Gs), e = sk_range_begin(w + 1, S, Gs);
  const int64_t s = b / kp + (q - W);
  if (b >= e || s * kp >= e) return false; // empty range (only if Gs > S), or past its end
  const int64_t lo = b > s * kp ? b : s * kp;
  const int64_t hi = e < (s + 1) * kp ? e : (s + 1) * kp;
  *tile = (T - R) + (int)s;
  *kb = (int)(2 * (lo - s * kp));
  *ke = (int)(2 * (hi - s * kp));
  return true;
}

// The same unit sequence, walked incrementally: the 64-bit divisions happen
// once per workgroup (init); next() then costs a few 32-bit operations, so
// a kernel can resolve units inside its k-loop. A workgroup's tail range
// is at most ceil(S/Gs) pairs, which the host keeps below 2^30.
struct SkWalker {
  int q, W, G, w, tail0, kp; // unit index; whole waves; grid; workgroup; first tail tile id; pairs per tile
  int s, off, rem;           // next tail tile index, first pair in it, pairs left in the range
  __host__ __device__ void init(int w_, int G_, int W_, int T, int R, int Gs, int kp_) {
    q = 0;
    W = W_;
    G = G_;
    w = w_;
    kp = kp_;
    tail0 = T - R;
    s = off = rem = 0;
    if (R > 0 && w < Gs) {
      const int64_t S = (int64_t)R * kp;
      const int64_t b = sk_range_begin(w, S, Gs), e = sk_range_begin(w + 1, S, Gs);
      s = (int)(b / kp);
      off = (int)(b - (int64_t)s * kp);
      rem = (int)(e - b);
    }
  }
  // Next unit: tile and k-step range [kb, ke); false when none is left.
  __host__ __device__ bool next(int* tile, int* kb, int* ke) {
    if (q < W) {
      *tile = q * G + w;
      *kb = 0;
      *ke = 2 * kp;
      ++q;
      return true;
    }
    if (rem <= 0) return false;
    const int n = kp - off < rem ? kp - off : rem;
    *tile = tail0 + s;
    *kb = 2 * off;
    *ke = 2 * (off + n);
    rem -= n;
    off = 0;
    ++s;
    ++q;
    return true;
  }
};

// ------------------------------------------------------- tile trace
// Optional per-tile record of who ran a tile, where and when: entry t holds
// {workgroup id, XCD id, start, end}, the times in ticks of the device's
// constant-rate clock. Kernels consume each clock read at once (an empty
// asm use or a store), so no scalar memory read stays outstanding across
// a k-loop.
__device__ inline long long trace_clock() { return (long long)__builtin_amdgcn_s_memrealtime(); }
__device__ inline int xcd_id() {
  int v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 15;
}
__device__ inline void trace_tile(long long* trace, int t, int wg, long long start, long long end) {
  long long* e = trace + 4 * (long long)t;
  e[0] = wg;
  e[1] = xcd_id();
  e[2] = start;
  e[3] = end;
}

// ------------------------------------------------ buffer loads into LDS
// gfx9 buffer resource word 3 for raw (untyped) dword access.
constexpr int kRsrcWord3 = 0x00020000;
// Any lane offset >= num_records reads zeros; masked lanes use this offset.
constexpr uint32_t kOOB = 0x80000000u;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, kRsrcWord3);
}

// One wave-wide 16-byte-per-lane load straight into LDS: lane l's 16 bytes
// land at lds + 16*l (a contiguous 1 KiB per wave). Offsets >= 2^31 read 0.
__device__ inline void load16_to_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, PGEMM_LDS(void, lds), 16, voffset, 0, 0, 0);
}

// --------------------------------------------------------------- MFMA
// 16x16 output block; lane l holds rows 4*(l/16)+r, column l%16 of D, r<4.
// Both operands: lane l holds row (or column) l%16 and the k-slots of group
// l/16; the pairing of A and B k-slots is positional, so any k order that
// both operands share gives the same sum.
__device__ inline floatx4_t mfma(const half8_t& a, const half8_t& b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ inline floatx4_t mfma(const bf16x8_t& a, const bf16x8_t& b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline floatx4_t mfma(const intx8_t& a, const intx8_t& b, floatx4_t c) {
  // format codes 0/0: both operands OCP fp8 e4m3; zero scale operands select
  // the unscaled instruction (per-tensor scale 1.0)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The same MFMAs with the accumulator pinned to AGPRs and tied (dst ==
// srcC). Used for the 256-register accumulator tile of the fast kernel,
// where the compiler otherwise renames accumulators between the two
// register files on every MFMA. Not volatile, so LDS reads and buffer loads
// still schedule around them. Callers must leave >= 24 wait states between
// the last MFMA and any read of the accumulators (see acc_drain()).
__device__ inline void mfma_acc(floatx4_t& c, const half8_t& a, const half8_t& b) {
  asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ inline void mfma_acc(floatx4_t& c, const bf16x8_t& a, const bf16x8_t& b) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ inline void mfma_acc(floatx4_t& c, const intx8_t& a, const intx8_t& b) {
  asm("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// Wait states between MFMAs issued as inline asm and a VALU / accvgpr read
// of their results (the compiler cannot see the asm's latency).
__device__ inline void acc_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// Read an accumulator block out of its AGPRs at this point of the program.
// (Left to itself the compiler copies the whole 128-register accumulator
// tile into VGPRs ahead of the epilogue and spills around it.)
__device__ inline floatx4_t acc_read(const floatx4_t& a) {
  floatx4_t v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v[0]) : "a"(a[0]));
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v[1]) : "a"(a[1]));
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v[2]) : "a"(a[2]));
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v[3]) : "a"(a[3]));
  return v;
}

// --------------------------------------------------------- output rounding
// fp32 -> fp16 / bf16, IEEE round to nearest even.
__device__ inline _Float16 to_out(float x, _Float16*) { return (_Float16)x; }
__device__ inline __bf16 to_out(float x, __bf16*) { return (__bf16)x; }

template <class OutT>
__device__ inline void store4(OutT* dst, floatx4_t v) {
  typedef OutT v4 __attribute__((ext_vector_type(4)));
  v4 o;
  o[0] = to_out(v[0], (OutT*)nullptr);
  o[1] = to_out(v[1], (OutT*)nullptr);
  o[2] = to_out(v[2], (OutT*)nullptr);
  o[3] = to_out(v[3], (OutT*)nullptr);
  *reinterpret_cast<v4*>(dst) = o;
}

// Eight consecutive outputs from two 4-wide accumulator blocks: a's values
// first, or b's first when `swap`; one 16-byte store (dst 16-byte aligned).
template <class OutT>
__device__ inline void store8(OutT* dst, floatx4_t a, floatx4_t b, bool swap) {
  typedef OutT v4 __attribute__((ext_vector_type(4)));
  v4 oa, ob;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    oa[e] = to_out(a[e], (OutT*)nullptr);
    ob[e] = to_out(b[e], (OutT*)nullptr);
  }
  const intx2_t wa = __builtin_bit_cast(intx2_t, oa), wb = __builtin_bit_cast(intx2_t, ob);
  intx4_t w;
  w[0] = swap ? wb[0] : wa[0];
  w[1] = swap ? wb[1] : wa[1];
  w[2] = swap ? wa[0] : wb[0];
  w[3] = swap ? wa[1] : wb[1];
  *reinterpret_cast<intx4_t*>(dst) = w;
}

} // namespace pgemm
