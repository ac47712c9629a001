// Host side of the library: argument validation, kernel selection, grid
// sizing, the work counter, and the C-ABI entry points declared in
// include/pgemm.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <mutex>
#include <thread>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>

#include "../../include/pgemm.h"
#include "kernels.h"

using namespace pgemm;

struct pgemm_ctx {
  int device = 0;
  hipStream_t stream = nullptr;
  int cus = 0;
  int* counter = nullptr; // work counter of the claiming modes (device int32)
  int32_t* visits = nullptr;
  int64_t n_visits = 0;
  int32_t* owner = nullptr;
  int64_t n_owner = 0;
  int64_t* trace = nullptr;
  int64_t n_trace = 0;
  int b_nk = 0; // layout of B: 0 = K x N row-major, 1 = N x K row-major
  float scale_a = 1.0f, scale_b = 1.0f; // per-tensor scales of e4m3 A and B
  // Tile-order defaults measured on MI355X (8192^3 and 4096^3 fp16, round-robin
  // timing): GROUP_SIZE_M between 1 and 16 moved throughput by a few percent
  // at most. The XCD remap (-1 = automatic: on when a launch has more tiles
  // than CUs) leaves the time level at 8192^3 and cuts the L2-miss fetches
  // there by a third (each XCD reads fewer operand panels); with one wave of
  // tiles it fetches the same bytes and measured slightly slower, so it stays
  // off there.
  int group_m = 4;
  int xcd_remap = -1;
  int tile = PGEMM_TILE_AUTO; // macro-tile choice of the fast kernel
  int mainloop = PGEMM_MAINLOOP_AUTO; // lockstep, ping-pong or producer waves for the 256-row tile
  // Stream-K: shortest piece, in k-step pairs, a split may cut (tiles with
  // fewer pairs are not split).
  int sk_min_pairs = 4;
  float* work = nullptr; // stream-K partial tiles, grown on demand
  size_t work_bytes = 0;
  int occ_cache[3][5][kNumBodies] = {}; // occupancy per (dtype, mode, body); 0 = not queried yet
  char last_error[512] = {0};
};

// ---- device scratch of the allocation-free entry point -----------------------------
// pgemm_run_noalloc takes the stream-K partial tiles from this file-scope array
// instead of a workspace the handle grows with hipMalloc. Each device that the
// library runs on holds its own copy until the process ends. In host code
// `scratch` is only a host-side stand-in for the symbol: its device address is
// looked up once per device (hipGetSymbolAddress, in pgemm_create) and only that
// address is ever handed to kernels.
static __device__ __align__(256) float scratch[PGEMM_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
float* g_scratch[kMaxDevices] = {}; // device address of `scratch` per device id

// With `device` current: look up its copy of `scratch` once.
hipError_t scratch_setup(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[device]) return hipSuccess;
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!ptr) return hipErrorInvalidSymbol;
  g_scratch[device] = static_cast<float*>(ptr);
  return hipSuccess;
}

float* scratch_of(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch[device];
}

} // namespace

namespace {

int fail(pgemm_ctx* h, int status, const char* fmt, ...) {
  if (h) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(h->last_error, sizeof(h->last_error), fmt, ap);
    va_end(ap);
  }
  return status;
}

// Macro-tile facts of the kernel bodies (the kernels themselves live in the
// per-dtype translation units).
struct BodyShape {
  int bm, bn, threads;
};
BodyShape body_shape(int body) {
  switch (body) {
    case kBodyTile256:
    case kBodyPingPong: return {256, 256, 512};
    case kBodyProducer: return {256, 128, 512};
    case kBodyTile128: return {128, 128, 256};
    default: return {64, 64, 256};
  }
}
int fast_block_k(int dtype) { return dtype == kF8E4M3 ? 128 : 64; }

kernel_fn pick_kernel(int dtype, int sched, int body, bool trace = false, bool bt = false) {
  if (body == kBodyPingPong) {
    // stream-K's tail launch takes the lockstep body (its whole waves run as a static launch)
    if (sched == kStreamK) return pick_kernel(dtype, sched, kBodyTile256, trace, bt);
    switch (dtype) {
      case kF16: return pick_kernel_pp_f16(sched, trace, bt);
      case kBF16: return pick_kernel_pp_bf16(sched, trace, bt);
      default: return pick_kernel_pp_f8(sched, trace, bt);
    }
  }
  if (body == kBodyProducer) {
    switch (dtype) {
      case kF16: return pick_kernel_pw_f16(sched, trace, bt);
      case kBF16: return pick_kernel_pw_bf16(sched, trace, bt);
      default: return pick_kernel_pw_f8(sched, trace, bt);
    }
  }
  switch (dtype) {
    case kF16: return pick_kernel_f16(sched, body, trace, bt);
    case kBF16: return pick_kernel_bf16(sched, body, trace, bt);
    default: return pick_kernel_f8(sched, body, trace, bt);
  }
}

kernel_fn pick_fixup(int dtype, int body) {
  if (body == kBodyPingPong) body = kBodyTile256; // same tile geometry
  switch (dtype) {
    case kF16: return pick_fixup_f16(body);
    case kBF16: return pick_fixup_bf16(body);
    default: return pick_fixup_f8(body);
  }
}

// Tile body for an aligned problem. Automatic choice: the 256 x 256 tile
// moves the fewest operand bytes per flop and measured faster whenever it
// gives every CU a tile (4096^2 to 8200^2, every K); when it would leave CUs
// idle, the 128 x 128 tile (two workgroups per CU, four times the tiles)
// fills the chip. The 256 x 256 tile runs its waves in ping-pong (each
// SIMD's two waves in opposite copy/compute phases) once a tile has enough
// k-steps; shorter k-loops take the lockstep form, whose tile prologue and
// epilogue cost less. Measured per K on MI355X (M = N = 4096 and 8192, every
// scheduling mode): 16-bit ping-pong is 2-17% slower up to 16 k-steps
// (K <= 1024), level at 18-20 and 2-14% faster from there; fp8 ping-pong is
// already 10% faster at 8 k-steps (8192^2 x 1024) and 2-3% slower at 2.
constexpr int kPingPongMinSteps16 = 20; // fp16 / bf16: K >= 1217
constexpr int kPingPongMinSteps8 = 8;   // e4m3: K >= 897

int choose_body(const pgemm_ctx* h, int64_t M, int64_t N, int64_t K, int dtype, int sched, bool fast) {
  if (!fast) return kBodyGeneric;
  int body;
  if (h->tile == PGEMM_TILE_256) {
    body = kBodyTile256;
  } else if (h->tile == PGEMM_TILE_128) {
    body = kBodyTile128;
  } else {
    const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
    body = t256 < (int64_t)h->cus ? kBodyTile128 : kBodyTile256;
  }
  if (body != kBodyTile256 || h->mainloop == PGEMM_MAINLOOP_LOCKSTEP) return body;
  if (h->mainloop == PGEMM_MAINLOOP_PINGPONG) return kBodyPingPong;
  // the producer-wave body takes the place of the 256 x 256 tile in the tile-sequence
  // modes; stream-K keeps the lockstep 256 x 256 body (its tail kernel and fix-up)
  if (h->mainloop == PGEMM_MAINLOOP_PRODUCER) return sched == kStreamK ? kBodyTile256 : kBodyProducer;
  const int64_t bk = dtype == kF8E4M3 ? 128 : 64;
  const int64_t nk = ((K + bk - 1) / bk + 1) & ~(int64_t)1;
  return nk >= (dtype == kF8E4M3 ? kPingPongMinSteps8 : kPingPongMinSteps16) ? kBodyPingPong : kBodyTile256;
}

int esize_of(int dtype) { return dtype == kF8E4M3 ? 1 : 2; }

bool sizes_fast(int dtype, int64_t N, int64_t K) {
  const int per16 = 16 / esize_of(dtype); // elements per 16 bytes
  return (K % per16) == 0 && (N % per16) == 0;
}

bool ptrs_fast(const void* A, const void* B, const void* C) {
  return ((uintptr_t)A % 16) == 0 && ((uintptr_t)B % 16) == 0 && ((uintptr_t)C % 16) == 0;
}

struct Plan {
  bool fast;
  int body, threads;
  int bm, bn, bk;
  int64_t n_m, n_n, T;
  int occupancy;
  int64_t G;
  // stream-K split (all zero in the other modes)
  int sk_waves = 0, sk_tiles = 0, sk_groups = 0, sk_split = 0; // sk_split: tiles cut into pieces
  size_t work_bytes = 0;
};

// Stream-K split of a fast launch (the helpers' comment in device_common.h
// gives the scheme): W = T / G whole-tile waves on G = mult * CUs
// workgroups, the R = T mod G tail tiles' S = R * kp pairs cut into
// Gs = min(G, S / min(kp, min_pairs)) ranges. The grid is G when W >= 1,
// else Gs.
void plan_streamk(const pgemm_ctx* h, int64_t K, int64_t G_full, Plan* pl) {
  const int64_t nk = ((K + pl->bk - 1) / pl->bk + 1) & ~(int64_t)1;
  const int64_t kp = nk / 2;
  const int64_t W = pl->T / G_full, R = pl->T % G_full;
  pl->sk_waves = (int)W;
  pl->sk_tiles = (int)R;
  int64_t Gs = 0;
  if (R > 0) {
    const int64_t S = R * kp;
    const int64_t minp = std::max<int64_t>(1, std::min<int64_t>(kp, h->sk_min_pairs));
    Gs = std::max<int64_t>(1, std::min<int64_t>(G_full, S / minp));
  }
  pl->sk_groups = (int)Gs;
  pl->G = W >= 1 ? G_full : Gs;
  int split = 0;
  for (int64_t s = 0; s < R; ++s) {
    const int64_t S = R * kp;
    if (sk_owner(s * kp, S, (int)Gs) != sk_owner((s + 1) * kp - 1, S, (int)Gs)) ++split;
  }
  pl->sk_split = split;
  pl->work_bytes = split ? (size_t)(Gs + R) * (size_t)pl->bm * (size_t)pl->bn * sizeof(float) : 0;
}

int plan_launch(pgemm_ctx* h, int64_t M, int64_t N, int64_t K, int dtype, int sched, int grid_multiple,
                bool fast, Plan* pl) {
  pl->fast = fast;
  pl->body = choose_body(h, M, N, K, dtype, sched, fast);
  const BodyShape bs = body_shape(pl->body);
  pl->threads = bs.threads;
  pl->bm = bs.bm;
  pl->bn = bs.bn;
  pl->bk = fast ? fast_block_k(dtype) : (dtype == kF8E4M3 ? 128 : 32);
  pl->n_m = (M + pl->bm - 1) / pl->bm;
  pl->n_n = (N + pl->bn - 1) / pl->bn;
  pl->T = pl->n_m * pl->n_n;
  // tile ids and claims (< T + G <= 2T) stay inside int32
  if (pl->T >= ((int64_t)1 << 30))
    return fail(h, PGEMM_ERR_UNSUPPORTED, "tile count %lld exceeds 2^30-1", (long long)pl->T);
  if (fast) {
    // per-tile A offsets reach BM rows of K elements; per-step B offsets reach BK rows of N
    const int64_t es = esize_of(dtype);
    if ((int64_t)pl->bm * K * es >= ((int64_t)1 << 31) || (int64_t)pl->bk * N * es >= ((int64_t)1 << 31))
      return fail(h, PGEMM_ERR_UNSUPPORTED, "operand rows too long for 32-bit buffer offsets");
  }
  // occupancy of the kernel, queried once per handle (it depends on the kernel and the device only)
  int& cached = h->occ_cache[dtype][sched][pl->body];
  if (cached == 0) {
    kernel_fn k = pick_kernel(dtype, sched, pl->body);
    int q = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&q, reinterpret_cast<const void*>(k), pl->threads, 0);
    if (e != hipSuccess) return fail(h, PGEMM_ERR_HIP, "occupancy query: %s", hipGetErrorString(e));
    cached = q < 1 ? 1 : q;
  }
  const int occ = cached;
  pl->occupancy = occ;
  const int64_t mult = grid_multiple <= 0 ? occ : grid_multiple;
  if (sched == kNonPersistent || sched == kCancel) {
    pl->G = pl->T; // one workgroup per tile (cancel-and-reuse: late ones find none left)
  } else if (sched == kStreamK && fast) {
    // pair positions (< T * kp) and the owner arithmetic stay inside int64
    const int64_t kp = (((K + pl->bk - 1) / pl->bk + 1) & ~(int64_t)1) / 2;
    if (pl->T * kp >= ((int64_t)1 << 40) || mult * h->cus >= ((int64_t)1 << 20))
      return fail(h, PGEMM_ERR_UNSUPPORTED, "stream-K split too large (tiles x k-steps or grid)");
    plan_streamk(h, K, mult * h->cus, pl);
    // a workgroup's tail range (in k-step pairs) must fit the kernel's 32-bit walker
    if (pl->sk_tiles && ((int64_t)pl->sk_tiles * kp + pl->sk_groups - 1) / pl->sk_groups >= ((int64_t)1 << 30))
      return fail(h, PGEMM_ERR_UNSUPPORTED, "stream-K range per workgroup too long");
  } else {
    pl->G = std::min<int64_t>(mult * h->cus, pl->T); // static, dynamic; stream-K on the generic body
  }
  return PGEMM_OK;
}

int check_common(pgemm_ctx* h, int64_t M, int64_t N, int64_t K, int dtype, int sched) {
  if (!h) return PGEMM_ERR_INVALID_ARG;
  if (M < 0 || N < 0 || K < 0)
    return fail(h, PGEMM_ERR_INVALID_ARG, "negative size M=%lld N=%lld K=%lld", (long long)M, (long long)N,
                (long long)K);
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
    return fail(h, PGEMM_ERR_UNSUPPORTED, "sizes must be below 2^31");
  if (dtype < PGEMM_F16 || dtype > PGEMM_F8E4M3_BF16) return fail(h, PGEMM_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (sched < PGEMM_SCHED_NONPERSISTENT || sched > PGEMM_SCHED_STREAMK)
    return fail(h, PGEMM_ERR_INVALID_ARG, "unknown sched_mode %d", sched);
  return PGEMM_OK;
}

} // namespace

namespace {
int run_impl(pgemm_handle_t h, const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
             int64_t M, int64_t N, int64_t K, int dtype, int sched_mode, int grid_multiple, bool noalloc);
} // namespace

extern "C" {

int pgemm_create(pgemm_handle_t* out, int device) {
  if (!out) return PGEMM_ERR_INVALID_ARG;
  *out = nullptr;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev) return PGEMM_ERR_INVALID_ARG;
  pgemm_ctx* h = new (std::nothrow) pgemm_ctx();
  if (!h) return PGEMM_ERR_OOM;
  h->device = device;
  if (hipSetDevice(device) != hipSuccess || hipDeviceGetAttribute(&h->cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) {
    delete h;
    return PGEMM_ERR_HIP;
  }
  // The counter gets a 256-byte allocation of its own so no other data shares its cache line.
  if (hipMalloc(&h->counter, 256) != hipSuccess) {
    delete h;
    return PGEMM_ERR_OOM;
  }
  if (hipMemset(h->counter, 0, 256) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    (void)hipFree(h->counter);
    delete h;
    return PGEMM_ERR_HIP;
  }
  if (scratch_setup(device) != hipSuccess) { // the allocation-free entry point's device scratch
    (void)hipGetLastError();
    (void)hipFree(h->counter);
    delete h;
    return PGEMM_ERR_HIP;
  }
  if (const char* g = getenv("PGEMM_GROUP_M")) h->group_m = std::max(1, atoi(g));
  if (const char* x = getenv("PGEMM_XCD_REMAP")) h->xcd_remap = atoi(x) < 0 ? -1 : atoi(x) != 0;
  if (const char* m = getenv("PGEMM_SK_MIN_PAIRS")) h->sk_min_pairs = std::max(1, atoi(m));
  if (const char* t = getenv("PGEMM_TILE")) {
    const int v = atoi(t);
    h->tile = v == 256 ? PGEMM_TILE_256 : v == 128 ? PGEMM_TILE_128 : PGEMM_TILE_AUTO;
  }
  if (const char* m = getenv("PGEMM_MAINLOOP")) {
    const int v = atoi(m);
    h->mainloop = v == PGEMM_MAINLOOP_LOCKSTEP || v == PGEMM_MAINLOOP_PINGPONG || v == PGEMM_MAINLOOP_PRODUCER
                      ? v
                      : PGEMM_MAINLOOP_AUTO;
  }
  *out = h;
  return PGEMM_OK;
}

int pgemm_set_stream(pgemm_handle_t h, void* hip_stream) {
  if (!h) return PGEMM_ERR_INVALID_ARG;
  h->stream = reinterpret_cast<hipStream_t>(hip_stream);
  return PGEMM_OK;
}

int pgemm_run(pgemm_handle_t h, const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
              int dtype, int sched_mode, int grid_multiple) {
  if (!h) return PGEMM_ERR_INVALID_ARG;
  return pgemm_run_ld(h, A, K, B, h->b_nk ? K : N, C, N, M, N, K, dtype, sched_mode, grid_multiple);
}

int pgemm_run_ld(pgemm_handle_t h, const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                 int64_t M, int64_t N, int64_t K, int dtype, int sched_mode, int grid_multiple) {
  return run_impl(h, A, lda, B, ldb, C, ldc, M, N, K, dtype, sched_mode, grid_multiple, false);
}

int pgemm_run_noalloc(pgemm_handle_t h, const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                      int dtype, int sched_mode, int grid_multiple) {
  if (!h) return PGEMM_ERR_INVALID_ARG;
  return run_impl(h, A, K, B, h->b_nk ? K : N, C, N, M, N, K, dtype, sched_mode, grid_multiple, true);
}

} // extern "C"

namespace {

// pgemm_run_ld, and with `noalloc` pgemm_run_noalloc: the stream-K workspace is then the
// device's `scratch` array (at most PGEMM_NOALLOC_SCRATCH_BYTES) instead of the handle's.
int run_impl(pgemm_handle_t h, const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
             int64_t M, int64_t N, int64_t K, int dtype, int sched_mode, int grid_multiple, bool noalloc) {
  int rc = check_common(h, M, N, K, dtype, sched_mode);
  if (rc != PGEMM_OK) return rc;
  h->last_error[0] = 0;
  if (M == 0 || N == 0) return PGEMM_OK;
  if (!C) return fail(h, PGEMM_ERR_INVALID_ARG, "C is NULL");
  // a leading dimension covers its row and stays below 2^31 elements
  const int64_t brow = h->b_nk ? K : N;
  if (ldc < N || (K > 0 && (lda < K || ldb < brow)) || lda > INT32_MAX || ldb > INT32_MAX || ldc > INT32_MAX)
    return fail(h, PGEMM_ERR_INVALID_ARG, "leading dimensions lda=%lld ldb=%lld ldc=%lld too small or too large",
                (long long)lda, (long long)ldb, (long long)ldc);
  if (hipSetDevice(h->device) != hipSuccess) return fail(h, PGEMM_ERR_HIP, "hipSetDevice failed");
  if (K == 0) {
    launch_fill_zero(C, M, N, ldc, h->stream);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? PGEMM_OK : fail(h, PGEMM_ERR_HIP, "zero-fill launch: %s", hipGetErrorString(e));
  }
  if (!A || !B) return fail(h, PGEMM_ERR_INVALID_ARG, "A or B is NULL");
  const int64_t per16 = 16 / esize_of(dtype); // elements per 16 bytes
  const bool fast = sizes_fast(dtype, N, K) && ptrs_fast(A, B, C) && lda % per16 == 0 && ldb % per16 == 0 &&
                    ldc % 8 == 0;
  Plan pl;
  rc = plan_launch(h, M, N, K, dtype, sched_mode, grid_multiple, fast, &pl);
  if (rc != PGEMM_OK) return rc;
  if (fast) {
    // per-tile A (and N x K B) offsets reach BM (BN) rows; per-step K x N B offsets reach BK rows
    const int64_t es = esize_of(dtype), lim = (int64_t)1 << 31;
    const int64_t b_span = h->b_nk ? (int64_t)pl.bn * ldb * es : (int64_t)pl.bk * ldb * es;
    if ((int64_t)pl.bm * lda * es >= lim || b_span >= lim)
      return fail(h, PGEMM_ERR_UNSUPPORTED, "leading dimensions too long for 32-bit buffer offsets");
  }
  if (h->visits && pl.T > h->n_visits)
    return fail(h, PGEMM_ERR_INVALID_ARG, "tile counter holds %lld entries, run has %lld tiles",
                (long long)h->n_visits, (long long)pl.T);
  if (h->owner && pl.T > h->n_owner)
    return fail(h, PGEMM_ERR_INVALID_ARG, "owner log holds %lld entries, run has %lld tiles", (long long)h->n_owner,
                (long long)pl.T);
  if (h->trace && pl.T > h->n_trace)
    return fail(h, PGEMM_ERR_INVALID_ARG, "tile trace holds %lld tiles, run has %lld tiles", (long long)h->n_trace,
                (long long)pl.T);
  Params p;
  p.A = static_cast<const uint8_t*>(A);
  p.B = static_cast<const uint8_t*>(B);
  p.C = static_cast<uint8_t*>(C);
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.lda = (int)lda;
  p.ldb = (int)ldb;
  p.ldc = (int)ldc;
  p.n_m = (int)pl.n_m;
  p.n_n = (int)pl.n_n;
  p.T = (int)pl.T;
  p.G = (int)pl.G;
  p.group_m = h->group_m;
  p.xcd_chunk = (h->xcd_remap > 0 || (h->xcd_remap < 0 && pl.T > h->cus)) ? h->cus : 0;
  p.counter = h->counter;
  p.visits = h->visits;
  p.owner = h->owner;
  p.trace = reinterpret_cast<long long*>(h->trace);
  p.b_nk = h->b_nk;
  p.c_scale = dtype == kF8E4M3 ? h->scale_a * h->scale_b : 1.0f;
  p.sk_waves = pl.sk_waves;
  p.sk_tiles = pl.sk_tiles;
  p.sk_groups = pl.sk_groups;
  p.work = nullptr;
  if (pl.work_bytes && noalloc) {
    if (pl.work_bytes > PGEMM_NOALLOC_SCRATCH_BYTES)
      return fail(h, PGEMM_ERR_UNSUPPORTED,
                  "stream-K split needs %zu bytes of partial tiles, more than the %zu-byte device scratch of "
                  "pgemm_run_noalloc (use pgemm_run)",
                  pl.work_bytes, (size_t)PGEMM_NOALLOC_SCRATCH_BYTES);
    p.work = scratch_of(h->device);
    if (!p.work) return fail(h, PGEMM_ERR_HIP, "device scratch of device %d was not set up", h->device);
  } else if (pl.work_bytes) {
    if (pl.work_bytes > h->work_bytes) {
      // grow the workspace: wait for launches that may still use the old one
      if (hipStreamSynchronize(h->stream) != hipSuccess) return fail(h, PGEMM_ERR_HIP, "stream synchronize failed");
      if (h->work) (void)hipFree(h->work);
      h->work = nullptr;
      h->work_bytes = 0;
      if (hipMalloc(&h->work, pl.work_bytes) != hipSuccess) {
        h->work = nullptr;
        (void)hipGetLastError();
        return fail(h, PGEMM_ERR_OOM, "stream-K workspace of %zu bytes", pl.work_bytes);
      }
      h->work_bytes = pl.work_bytes;
    }
    p.work = h->work;
  }
  if (sched_mode != kStreamK || !pl.fast) {
    kernel_fn k = pick_kernel(dtype, sched_mode, pl.body, p.trace != nullptr, p.b_nk != 0);
    hipLaunchKernelGGL(k, dim3((unsigned)pl.G), dim3(pl.threads), 0, h->stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(h, PGEMM_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
    return PGEMM_OK;
  }
  // Stream-K as up to three launches on the stream: (1) the W whole waves, by
  // the static kernel over the first W*G tiles of the tile order (its tile
  // sequence, unchanged: tile coordinates do not depend on T, and the XCD
  // remap's chunk, the CU count, divides W*G); (2) the R tail tiles' split,
  // by the stream-K kernel on its own grid of Gs workgroups; (3) the fix-up
  // of split tiles. Keeping the whole waves in the static kernel keeps them
  // at its speed: the stream-K kernel's partial-tile stores make the compiler
  // add a wait for every outstanding global->LDS copy inside its k-loop
  // (measured 8% slower at 8192^3).
  if (pl.sk_waves > 0) {
    Params pd = p;
    pd.T = (int)(pl.T - pl.sk_tiles); // W * G
    pd.sk_waves = pd.sk_tiles = pd.sk_groups = 0;
    pd.work = nullptr;
    hipLaunchKernelGGL(pick_kernel(dtype, kStatic, pl.body, p.trace != nullptr, p.b_nk != 0), dim3((unsigned)pl.G),
                       dim3(pl.threads), 0, h->stream, pd);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(h, PGEMM_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  }
  if (pl.sk_tiles > 0) {
    Params ps = p;
    ps.sk_waves = 0;
    ps.G = pl.sk_groups;
    hipLaunchKernelGGL(pick_kernel(dtype, kStreamK, pl.body, p.trace != nullptr, p.b_nk != 0),
                       dim3((unsigned)pl.sk_groups), dim3(pl.threads), 0, h->stream, ps);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(h, PGEMM_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
    if (pl.sk_split) {
      // 256 threads cover 8 columns each: 256 / (bn / 8) rows per workgroup
      const unsigned rows_per_wg = 256u / (unsigned)(pl.bn / 8);
      hipLaunchKernelGGL(pick_fixup(dtype, pl.body), dim3((unsigned)pl.sk_tiles, (unsigned)pl.bm / rows_per_wg),
                         dim3(256), 0, h->stream, ps);
      e = hipGetLastError();
      if (e != hipSuccess) return fail(h, PGEMM_ERR_HIP, "fix-up launch: %s", hipGetErrorString(e));
    }
  }
  return PGEMM_OK;
}

} // namespace

extern "C" {

int pgemm_destroy(pgemm_handle_t h) {
  if (!h) return PGEMM_OK;
  int rc = PGEMM_OK;
  if (hipSetDevice(h->device) != hipSuccess) rc = PGEMM_ERR_HIP;
  if (hipStreamSynchronize(h->stream) != hipSuccess) rc = PGEMM_ERR_HIP;
  if (hipFree(h->counter) != hipSuccess) rc = PGEMM_ERR_HIP;
  if (h->work && hipFree(h->work) != hipSuccess) rc = PGEMM_ERR_HIP;
  delete h;
  return rc;
}

int pgemm_wait(pgemm_handle_t h, int timeout_ms) {
  if (!h || timeout_ms < 0) return PGEMM_ERR_INVALID_ARG;
  if (hipSetDevice(h->device) != hipSuccess) return fail(h, PGEMM_ERR_HIP, "hipSetDevice failed");
  const auto deadline = std::chrono::steady_clock::now() + std::chrono::milliseconds(timeout_ms);
  for (;;) {
    const hipError_t e = hipStreamQuery(h->stream);
    if (e == hipSuccess) return PGEMM_OK;
    if (e != hipErrorNotReady) return fail(h, PGEMM_ERR_HIP, "stream query: %s", hipGetErrorString(e));
    if (std::chrono::steady_clock::now() >= deadline)
      return fail(h, PGEMM_ERR_TIMEOUT, "stream still busy after %d ms", timeout_ms);
    std::this_thread::sleep_for(std::chrono::microseconds(50));
  }
}

const char* pgemm_status_string(int status) {
  switch (status) {
    case PGEMM_OK: return "PGEMM_OK";
    case PGEMM_ERR_INVALID_ARG: return "PGEMM_ERR_INVALID_ARG";
    case PGEMM_ERR_UNSUPPORTED: return "PGEMM_ERR_UNSUPPORTED";
    case PGEMM_ERR_HIP: return "PGEMM_ERR_HIP";
    case PGEMM_ERR_OOM: return "PGEMM_ERR_OOM";
    case PGEMM_ERR_TIMEOUT: return "PGEMM_ERR_TIMEOUT";
    default: return "PGEMM_ERR_UNKNOWN";
  }
}

const char* pgemm_last_error(pgemm_handle_t h) { return h ? h->last_error : "invalid handle"; }

int pgemm_set_tile_counter(pgemm_handle_t h, int32_t* dev_visits, int64_t n_tiles) {
  if (!h) return PGEMM_ERR_INVALID_ARG;
  if (dev_visits && n_tiles <= 0) return fail(h, PGEMM_ERR_INVALID_ARG, "n_tiles must be positive");
  h->visits = dev_visits;
  h->n_visits = dev_visits ? n_tiles : 0;
  return PGEMM_OK;
}

int pgemm_set_owner_log(pgemm_handle_t h, int32_t* dev_owner, int64_t n_tiles) {
  if (!h) return PGEMM_ERR_INVALID_ARG;
  if (dev_owner && n_tiles <= 0) return fail(h, PGEMM_ERR_INVALID_ARG, "n_tiles must be positive");
  h->owner = dev_owner;
  h->n_owner = dev_owner ? n_tiles : 0;
  return PGEMM_OK;
}

int pgemm_set_tile_trace(pgemm_handle_t h, int64_t* dev_trace, int64_t n_tiles) {
  if (!h) return PGEMM_ERR_INVALID_ARG;
  if (dev_trace && n_tiles <= 0) return fail(h, PGEMM_ERR_INVALID_ARG, "n_tiles must be positive");
  h->trace = dev_trace;
  h->n_trace = dev_trace ? n_tiles : 0;
  return PGEMM_OK;
}

int pgemm_set_b_layout(pgemm_handle_t h, int layout) {
  if (!h) return PGEMM_ERR_INVALID_ARG;
  if (layout != PGEMM_B_KN && layout != PGEMM_B_NK) return fail(h, PGEMM_ERR_INVALID_ARG, "unknown B layout %d", layout);
  h->b_nk = layout == PGEMM_B_NK;
  return PGEMM_OK;
}

int pgemm_set_fp8_scales(pgemm_handle_t h, float scale_a, float scale_b) {
  if (!h) return PGEMM_ERR_INVALID_ARG;
  if (!std::isfinite(scale_a) || !std::isfinite(scale_b) || !std::isfinite(scale_a * scale_b))
    return fail(h, PGEMM_ERR_INVALID_ARG, "fp8 scales must be finite with a finite product");
  h->scale_a = scale_a;
  h->scale_b = scale_b;
  return PGEMM_OK;
}

int pgemm_clock_khz(int device, int* khz) {
  if (!khz) return PGEMM_ERR_INVALID_ARG;
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeWallClockRate, device) != hipSuccess || v <= 0)
    return PGEMM_ERR_HIP;
  *khz = v;
  return PGEMM_OK;
}

int pgemm_query_launch(pgemm_handle_t h, int64_t M, int64_t N, int64_t K, int dtype, int sched_mode,
                       int grid_multiple, int* tiles, int* grid, int* occupancy, int* bm, int* bn, int* bk,
                       int* body) {
  int rc = check_common(h, M, N, K, dtype, sched_mode);
  if (rc != PGEMM_OK) return rc;
  // the plan may query the kernel's occupancy: on the handle's device
  if (hipSetDevice(h->device) != hipSuccess) return fail(h, PGEMM_ERR_HIP, "hipSetDevice failed");
  Plan pl;
  rc = plan_launch(h, M, N, K, dtype, sched_mode, grid_multiple, sizes_fast(dtype, N, K), &pl);
  if (rc != PGEMM_OK) return rc;
  if (tiles) *tiles = (int)pl.T;
  if (grid) *grid = (int)pl.G;
  if (occupancy) *occupancy = pl.occupancy;
  if (bm) *bm = pl.bm;
  if (bn) *bn = pl.bn;
  if (bk) *bk = pl.bk;
  if (body) {
    // the tile body of the launch that does the GEMM's whole tiles: 0 generic, 1 lockstep,
    // 2 ping-pong, 3 producer waves
    *body = !pl.fast ? 0 : pl.body == kBodyPingPong ? 2 : pl.body == kBodyProducer ? 3 : 1;
  }
  return PGEMM_OK;
}

int pgemm_query_streamk(pgemm_handle_t h, int64_t M, int64_t N, int64_t K, int dtype, int grid_multiple,
                        int* whole_tiles, int* split_tiles, int* split_groups, int* pieces_split,
                        int64_t* workspace_bytes) {
  int rc = check_common(h, M, N, K, dtype, PGEMM_SCHED_STREAMK);
  if (rc != PGEMM_OK) return rc;
  if (hipSetDevice(h->device) != hipSuccess) return fail(h, PGEMM_ERR_HIP, "hipSetDevice failed");
  Plan pl;
  rc = plan_launch(h, M, N, K, dtype, PGEMM_SCHED_STREAMK, grid_multiple, sizes_fast(dtype, N, K), &pl);
  if (rc != PGEMM_OK) return rc;
  if (whole_tiles) *whole_tiles = (int)(pl.T - pl.sk_tiles);
  if (split_tiles) *split_tiles = pl.sk_tiles;
  if (split_groups) *split_groups = pl.sk_groups;
  if (pieces_split) *pieces_split = pl.sk_split;
  if (workspace_bytes) *workspace_bytes = (int64_t)pl.work_bytes;
  return PGEMM_OK;
}

int pgemm_set_tile_order(pgemm_handle_t h, int group_m, int xcd_remap) {
  if (!h) return PGEMM_ERR_INVALID_ARG;
  if (group_m < 1) return fail(h, PGEMM_ERR_INVALID_ARG, "group_m must be >= 1");
  h->group_m = group_m;
  h->xcd_remap = xcd_remap < 0 ? -1 : xcd_remap != 0;
  return PGEMM_OK;
}

int pgemm_set_tile_config(pgemm_handle_t h, int tile) {
  if (!h) return PGEMM_ERR_INVALID_ARG;
  if (tile < PGEMM_TILE_AUTO || tile > PGEMM_TILE_128) return fail(h, PGEMM_ERR_INVALID_ARG, "unknown tile config %d", tile);
  h->tile = tile;
  return PGEMM_OK;
}

int pgemm_set_mainloop(pgemm_handle_t h, int mainloop) {
  if (!h) return PGEMM_ERR_INVALID_ARG;
  if (mainloop < PGEMM_MAINLOOP_AUTO || mainloop > PGEMM_MAINLOOP_PRODUCER)
    return fail(h, PGEMM_ERR_INVALID_ARG, "unknown mainloop %d", mainloop);
  h->mainloop = mainloop;
  return PGEMM_OK;
}

int pgemm_tile_coords(int64_t t, int64_t n_m, int64_t n_n, int group_m, int cu_chunk, int* pid_m, int* pid_n) {
  if (n_m <= 0 || n_n <= 0 || group_m < 1 || t < 0 || n_m * n_n >= ((int64_t)1 << 31) || t >= n_m * n_n || !pid_m ||
      !pid_n)
    return PGEMM_ERR_INVALID_ARG;
  const int T = (int)(n_m * n_n);
  grouped_tile(xcd_remap((int)t, T, cu_chunk), (int)n_m, (int)n_n, group_m, pid_m, pid_n);
  return PGEMM_OK;
}

int pgemm_hold_cus(void* hip_stream, int device, int n_cus, int microseconds) {
  if (n_cus < 0 || n_cus > 65536 || microseconds < 0 || microseconds > 1000000) return PGEMM_ERR_INVALID_ARG;
  if (n_cus == 0 || microseconds == 0) return PGEMM_OK;
  if (hipSetDevice(device) != hipSuccess) return PGEMM_ERR_INVALID_ARG;
  int khz = 0; // rate of the s_memrealtime clock
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, device) != hipSuccess || khz <= 0) khz = 100000;
  launch_hold(n_cus, (uint64_t)microseconds * (uint64_t)khz / 1000u, reinterpret_cast<hipStream_t>(hip_stream));
  return hipGetLastError() == hipSuccess ? PGEMM_OK : PGEMM_ERR_HIP;
}

int pgemm_read_work_counter(pgemm_handle_t h, int32_t* value) {
  if (!h || !value) return PGEMM_ERR_INVALID_ARG;
  if (hipSetDevice(h->device) != hipSuccess) return fail(h, PGEMM_ERR_HIP, "hipSetDevice failed");
  hipError_t e = hipMemcpyAsync(value, h->counter, sizeof(int32_t), hipMemcpyDeviceToHost, h->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(h->stream);
  return e == hipSuccess ? PGEMM_OK : fail(h, PGEMM_ERR_HIP, "counter read: %s", hipGetErrorString(e));
}

} // extern "C"
