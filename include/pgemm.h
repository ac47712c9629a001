/*
 * pgemm.h -- persistent-tile-scheduled GEMM for AMD Instinct MI355X (gfx950).
 *
 * C-ABI boundary of the library: plain pointers and sizes, no C++ or torch
 * types. All matrix pointers are DEVICE pointers (hipMalloc'd or torch
 * tensors' data_ptr()); everything else is host memory.
 *
 * The operation (persistent-kernel forum thread, question): the GEMM
 *     C[i][j] = sum_k A[i][k] * B[k][j]
 * with A: M x K row-major (leading dimension K), B: K x N row-major
 * (leading dimension N) -- or, after pgemm_set_b_layout(h, PGEMM_B_NK),
 * N x K row-major (leading dimension K, i.e. B stored transposed, the layout
 * of a linear layer's weight) -- and C: M x N row-major (leading dimension
 * N), all contiguous, accumulated in fp32. The output is cut into macro tiles and
 * a tile scheduler hands tiles to workgroups (same question). Scheduling
 * never changes the value of C: modes NONPERSISTENT..CANCEL run the same
 * tile body, so C is bitwise identical across them and across reruns
 * (KernelWiki "Persistent Kernels with Cluster Launch Control", "Choosing
 * between static and CLC scheduling": neither scheduler adds work).
 * STREAMK adds work (split tiles' partial sums), so its C may differ from
 * theirs in the last bits; it is bitwise identical across its own reruns.
 *
 * Errors: every entry point returns a pgemm_status_t. No C++ exception
 * crosses this boundary. Launches are asynchronous on the handle's stream;
 * errors of the launch itself are returned as PGEMM_ERR_HIP, with detail
 * in pgemm_last_error(). A handle is not thread-safe: use one handle per
 * stream used concurrently (the dynamic scheduler's work counter is per
 * handle; DYNAMIC and CANCEL share it).
 */
#ifndef PGEMM_H
#define PGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pgemm_ctx* pgemm_handle_t;

typedef enum {
  PGEMM_OK = 0,
  PGEMM_ERR_INVALID_ARG = 1, /* null pointer with non-zero size, negative size, bad enum */
  PGEMM_ERR_UNSUPPORTED = 2, /* size beyond the 32-bit tile/offset limits */
  PGEMM_ERR_HIP = 3,         /* a HIP runtime call failed; see pgemm_last_error() */
  PGEMM_ERR_OOM = 4,         /* device or host allocation failed */
  PGEMM_ERR_TIMEOUT = 5      /* pgemm_wait: the stream's work did not finish in time */
} pgemm_status_t;

/* Element formats. The pages name fp16 and fp8 (Triton persistent-matmul
 * issue: "--prec fp16", and the fp8 example on H100); bf16 is the other
 * 16-bit format of the same MFMA family. fp8 is OCP E4M3 ("fn": bias 7,
 * max 448, no infinities) with a per-tensor scale for each of A and B: 1.0
 * by default, any finite value through pgemm_set_fp8_scales. */
typedef enum {
  PGEMM_F16 = 0,         /* A, B, C: IEEE binary16 */
  PGEMM_BF16 = 1,        /* A, B, C: bfloat16 */
  PGEMM_F8E4M3_BF16 = 2  /* A, B: OCP e4m3 (1 byte); C: bfloat16 */
} pgemm_dtype_t;

/* Tile scheduling modes.
 * NONPERSISTENT: one workgroup per output tile (forum thread, question:
 *   "a thread block for each tile"); grid = number of tiles T.
 * STATIC: a persistent grid of G workgroups (forum thread, question: block
 *   count set to the SM count; first answer: sized so all blocks stay
 *   resident); workgroup w computes tiles w, w+G, w+2G, ... of the tile
 *   order, a deterministic mapping (KernelWiki, "Choosing between static
 *   and CLC scheduling").
 * DYNAMIC: a persistent grid of G workgroups; workgroup w starts on tile
 *   w, then claims further tile ids from a device-wide atomic work counter
 *   until a claim fails, after which it never claims again -- the AMD
 *   analogue of cluster launch control's cancel-and-reuse (KernelWiki,
 *   intro), not a port of it. With G >= T there is nothing to claim and no
 *   claim is made.
 * CANCEL: the grid is one workgroup per tile (T), as in NONPERSISTENT, but
 *   every workgroup claims its tiles -- the first one too -- from the work
 *   counter and keeps claiming until a claim fails. Workgroups that run
 *   early take over the tiles of workgroups that have not started; those
 *   find no tile left when they start and exit at once. This is the closer
 *   analogue of cancel-and-reuse (a grid whose not-yet-launched members'
 *   ids are taken over, same page, intro) and needs no co-residency
 *   assumption; grid_multiple is ignored.
 * STREAMK: tail handling that creates work instead of idling CUs, for
 *   tile counts T that the grid G does not divide (the case the KernelWiki
 *   page's static-vs-CLC guidance leaves open: neither of its schedulers
 *   creates work at the tail). With T = W*G + R, the first W*G tiles of the
 *   tile order run whole, as in STATIC; the k-steps of the last R tiles are
 *   split evenly over the G workgroups (over fewer when pieces would drop
 *   below a minimum length), so every workgroup gets about W + R/G tiles
 *   of work. A workgroup whose piece covers only part of a tile's k-range
 *   writes an fp32 partial tile to a workspace the handle owns. A second
 *   launch on the same stream then adds each split tile's partials in k
 *   order, rounds the sum and stores the tile. G as in STATIC, without the
 *   clamp to T: with T < G (W = 0) the split spreads even a few tiles over
 *   the whole chip. The whole waves run as one STATIC launch over the first
 *   W*G tiles, the tail as a second launch on its own grid, then the fix-up:
 *   up to three launches per run, all on the handle's stream. R = 0 is
 *   exactly STATIC (one launch). Operands that take the generic kernel
 *   (below) run this mode as STATIC. */
typedef enum {
  PGEMM_SCHED_NONPERSISTENT = 0,
  PGEMM_SCHED_STATIC = 1,
  PGEMM_SCHED_DYNAMIC = 2,
  PGEMM_SCHED_CANCEL = 3,
  PGEMM_SCHED_STREAMK = 4
} pgemm_sched_t;

/* Macro-tile configurations of the fast kernel (the Triton persistent-
 * matmul issue tunes BLOCK_SIZE_M/N per problem, "What I've tried").
 * TILE_256: 256 x 256 tiles, 512 threads, one workgroup per CU: the fewest
 *   operand bytes per flop, for problems with many tiles.
 * TILE_128: 128 x 128 tiles, 256 threads, two workgroups per CU: four times
 *   the tiles, so small problems fill the chip and persistent workgroups
 *   get several tiles each.
 * AUTO (default): TILE_128 when 256 x 256 tiles would number fewer than the
 *   CUs (some CUs would idle), else TILE_256. The environment variable PGEMM_TILE (256 or 128)
 *   overrides the default at pgemm_create. */
typedef enum {
  PGEMM_TILE_AUTO = 0,
  PGEMM_TILE_256 = 1,
  PGEMM_TILE_128 = 2
} pgemm_tile_t;

/* Wave schedule of the 256-row fast tile (pgemm_set_mainloop). The value of
 * C does not depend on it: every schedule gives every accumulator the same
 * MFMAs on the same operands in the same order, so C is bitwise the same.
 * LOCKSTEP: all eight waves of a workgroup copy, read and multiply in step,
 *   one barrier per k-step; each step's global -> LDS copy is issued right
 *   after its barrier (the copy/compute overlap of the persistent-kernel
 *   forum thread's first answer, per workgroup).
 * PINGPONG: the two waves of each SIMD run opposite phases: while one issues
 *   copies and reads the next fragments from LDS, the other runs its MFMAs,
 *   and they swap at each barrier (the same overlap, per SIMD; the load role
 *   alternates between the waves instead of being given to a producer wave,
 *   KernelWiki "Persistent Kernels with Cluster Launch Control", tutorial
 *   note on warp specialization).
 * PRODUCER: a dedicated load role (the KernelWiki page's producer-side
 *   request pipeline and its warp-specialization note): waves 4-7 of the
 *   workgroup only copy operand tiles into a three-stage LDS ring and make
 *   the tile claims of the claiming modes, waves 0-3 only read fragments and
 *   run MFMAs. Every wave of a workgroup gets the same register budget on
 *   CDNA, so with four waves copying the tile shrinks to 256 x 128 (T is
 *   counted in those tiles). STREAMK keeps the lockstep 256 x 256 body.
 *   Offered for measurement; AUTO never picks it (measured slower).
 * AUTO (default): PINGPONG for tiles of at least 20 k-steps of 64 for
 *   fp16/bf16 (K >= 1217) and 8 k-steps of 128 for fp8 (K >= 897), LOCKSTEP
 *   below, where its cheaper tile prologue and epilogue win (measured).
 *   The 128 x 128 tile, the generic body and the split tail of STREAMK
 *   always run lockstep. The environment variable PGEMM_MAINLOOP (1, 2 or 3)
 *   overrides the default at pgemm_create. */
typedef enum {
  PGEMM_MAINLOOP_AUTO = 0,
  PGEMM_MAINLOOP_LOCKSTEP = 1,
  PGEMM_MAINLOOP_PINGPONG = 2,
  PGEMM_MAINLOOP_PRODUCER = 3
} pgemm_mainloop_t;

/* Storage of B (pgemm_set_b_layout). The value of C does not depend on it:
 * both layouts feed the MFMAs the same operands in the same order, so C is
 * bitwise the same. */
typedef enum {
  PGEMM_B_KN = 0, /* B[k][n] at B + k*N + n (default) */
  PGEMM_B_NK = 1  /* B[k][n] at B + n*K + k */
} pgemm_b_layout_t;

/* Create a handle on HIP device `device` (which becomes current). Allocates
 * the claiming modes' device work counter (zeroed) and caches the CU count.
 * The handle starts on the null stream. *out is NULL on failure.
 * pgemm_create, pgemm_run and pgemm_destroy are this library's stated
 * interface (the pages specify no API; they fix the operation: forum
 * thread, question); the other entry points complete it. PGEMM_ERR_INVALID_ARG
 * for a NULL out or a device outside [0, device count); PGEMM_ERR_OOM if the
 * handle or the counter cannot be allocated; PGEMM_ERR_HIP if the device
 * cannot be queried. */
int pgemm_create(pgemm_handle_t* out, int device);

/* Bind a hipStream_t (passed as void*; NULL = null stream). Later runs
 * enqueue on it; the caller keeps ownership of the stream, which must
 * outlive its use by the handle. Part of the stated interface's completion
 * (asynchronous runs on a caller's stream). PGEMM_ERR_INVALID_ARG for a
 * NULL handle. */
int pgemm_set_stream(pgemm_handle_t h, void* hip_stream);

/* Enqueue C = A * B on the handle's stream; returns without waiting.
 *   A, B, C: device pointers to contiguous row-major matrices (layouts
 *     above); they must not alias and must stay valid until the work is
 *     done. The caller owns them.
 *   M, N, K: sizes, each in [0, 2^31 - 1]. M == 0 or N == 0: no work, OK.
 *     K == 0: C is filled with zeros (an empty sum).
 *   dtype: pgemm_dtype_t.
 *   sched_mode: pgemm_sched_t.
 *   grid_multiple: persistent modes only (ignored for NONPERSISTENT and
 *     CANCEL).
 *     <= 0: G = occupancy x CU count (all workgroups co-resident, the
 *     sizing of the forum thread's first answer); > 0: G = grid_multiple x
 *     CU count (the NUM_SMS multiple of the Triton issue's follow-up
 *     comment), which may exceed co-residency -- no workgroup waits on
 *     another, so that stays correct. G is clamped to the tile count T
 *     (except in STREAMK, see above).
 * Operands whose K and N are multiples of 16 bytes of elements (8 for
 * fp16/bf16, 16 for fp8) with 16-byte-aligned A, B and C
 * take the fast kernel (256 x 256 or 128 x 128 tiles, pgemm_tile_t);
 * others take a generic 64 x 64 tile kernel with the same schedulers
 * (correct, slower).
 * STREAMK workspace: a run whose split needs more workspace than the handle
 * holds (pgemm_query_streamk) first waits for the handle's stream, frees
 * the old workspace and hipMallocs the new one (PGEMM_ERR_OOM if that
 * fails); later runs of the same or smaller need allocate nothing. Under
 * stream capture, make one such run before capturing. Two runs in flight
 * on one handle share the workspace, which the one-stream-per-handle rule
 * above already orders. */
int pgemm_run(pgemm_handle_t h, const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
              int dtype, int sched_mode, int grid_multiple);

/* Wait for the handle's stream, free the work counter, the stream-K
 * workspace and the handle (stated interface). NULL is accepted (no-op).
 * Returns PGEMM_ERR_HIP if the wait or a free failed; the handle is freed
 * either way and must not be used again. */
int pgemm_destroy(pgemm_handle_t h);

/* Size in bytes of the device scratch that pgemm_run_noalloc uses for
 * STREAMK partial tiles (one copy per device, held until the process ends). */
#define PGEMM_NOALLOC_SCRATCH_BYTES (96u << 20)

/* pgemm_run that allocates nothing, for callers that cannot call hipMalloc
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). Same arguments, semantics, errors and results (bitwise) as
 * pgemm_run, except for where STREAMK keeps its fp32 partial tiles: in a
 * file-scope device array of PGEMM_NOALLOC_SCRATCH_BYTES per device (set up
 * by pgemm_create on the handle's device), not in the handle's workspace.
 * A STREAMK split that needs more (pgemm_query_streamk's workspace_bytes)
 * fails with PGEMM_ERR_UNSUPPORTED before any launch; no other mode needs
 * scratch. The partial tiles are fully written before they are read, so the
 * array needs no clearing between calls. All calls on one device share its
 * array: two STREAMK calls whose work overlaps on the device (on different
 * streams, or different handles) race on it; serialize them (one stream).
 * The call makes no hipMalloc, hipFree or stream synchronization. */
int pgemm_run_noalloc(pgemm_handle_t h, const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                      int dtype, int sched_mode, int grid_multiple);

/* pgemm_run with leading dimensions, for operands that are row-major views
 * inside larger allocations: A[i][k] at A + i*lda + k, B[k][n] at
 * B + k*ldb + n (or, with PGEMM_B_NK, at B + n*ldb + k), C[i][j] at
 * C + i*ldc + j, all counted in elements. pgemm_run is this call with
 * lda = K, ldb = N (K for PGEMM_B_NK) and ldc = N. Requires ldc >= N and,
 * when K > 0, lda >= K and ldb >= the length of B's rows (N, or K for
 * PGEMM_B_NK); each below 2^31; else PGEMM_ERR_INVALID_ARG. Only the M x N
 * window of C is written. The fast kernel additionally needs lda and ldb
 * to be multiples of 16 bytes of elements and ldc a multiple of 8 (16-byte
 * rows of C); otherwise the generic kernel runs. Leading dimensions whose
 * tile spans exceed 32-bit buffer offsets give PGEMM_ERR_UNSUPPORTED.
 * Everything else is as for pgemm_run. */
int pgemm_run_ld(pgemm_handle_t h, const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                 int64_t M, int64_t N, int64_t K, int dtype, int sched_mode, int grid_multiple);

/* Watchdog wait: poll the handle's stream (hipStreamQuery, about every
 * 50 microseconds) until all work enqueued on it has finished, or until
 * timeout_ms milliseconds have passed. Returns PGEMM_OK when the stream is
 * idle, PGEMM_ERR_TIMEOUT when the deadline passed first (the work keeps
 * running; the caller may wait again), PGEMM_ERR_HIP if the stream reports
 * an error (e.g. a kernel fault), PGEMM_ERR_INVALID_ARG for a NULL handle
 * or a negative timeout. Lets a harness notice a kernel that never ends
 * instead of blocking in a synchronize. */
int pgemm_wait(pgemm_handle_t h, int timeout_ms);

/* Static text for a status code (never NULL; unknown codes give
 * "PGEMM_ERR_UNKNOWN"). Error reporting of the stated interface: every
 * entry point returns a status instead of raising. */
const char* pgemm_status_string(int status);

/* Detail of the last failure on this handle ("" if none; "invalid handle"
 * for NULL). Owned by the handle, valid until the next call on it. Error
 * reporting of the stated interface. */
const char* pgemm_last_error(pgemm_handle_t h);

/* ---- checking and reporting (not for timed runs) ---------------------- */

/* Attach a caller-owned device int32 array of n_tiles entries. Each run
 * then atomically adds 1 to visits[t] after tile t's C store, so after a
 * run from zeroed memory every entry must read exactly 1 (every tile
 * written exactly once). dev_visits == NULL detaches. Runs whose tile
 * count exceeds n_tiles fail with PGEMM_ERR_INVALID_ARG. */
int pgemm_set_tile_counter(pgemm_handle_t h, int32_t* dev_visits, int64_t n_tiles);

/* Attach a caller-owned device int32 array of n_tiles entries; each run
 * writes owner[t] = the id of the workgroup that computed tile t. NULL
 * detaches. Same size rule as the visit counter. In STREAMK the W*G
 * whole-wave tiles are logged by workgroup id of that launch (t mod G), a
 * tail tile computed whole by the id of its workgroup in the tail launch,
 * and a split tile, stored by the fix-up launch, as -1 - s (s = the tile's
 * index among the R tail tiles); the visit counter counts that store, so
 * every tile still reads 1. */
int pgemm_set_owner_log(pgemm_handle_t h, int32_t* dev_owner, int64_t n_tiles);

/* Attach a caller-owned device int64 array of 4 * n_tiles entries: the
 * tile trace, used to draw per-workgroup timelines of the tail effect
 * (KernelWiki "Persistent Kernels with Cluster Launch Control", "Choosing
 * between static and CLC scheduling": the last wave of tiles leaves part
 * of the chip idle). Each run writes, for every tile t,
 *   trace[4t+0]  id of the workgroup that stored tile t (the owner-log
 *                convention: -1 - s for a STREAMK split tile, which the
 *                fix-up launch stores),
 *   trace[4t+1]  id of the XCD (0..7) whose CU ran that workgroup,
 *   trace[4t+2]  start: when that workgroup began the tile (its k-loop),
 *   trace[4t+3]  end: after the tile's C store was issued,
 * the times in ticks of the device's constant-rate clock (see
 * pgemm_clock_khz). For a split tile, start and end bracket its fix-up.
 * The trace adds a clock read and a few stores per tile: leave it off in
 * timed runs. NULL detaches. Runs whose tile count exceeds n_tiles fail
 * with PGEMM_ERR_INVALID_ARG before launching. */
int pgemm_set_tile_trace(pgemm_handle_t h, int64_t* dev_trace, int64_t n_tiles);

/* Rate in kHz of the constant-rate clock that stamps the tile trace, for
 * device `device`. PGEMM_ERR_INVALID_ARG if khz is NULL, PGEMM_ERR_HIP if
 * the device cannot be queried. */
int pgemm_clock_khz(int device, int* khz);

/* Report how pgemm_run would launch this problem, without launching:
 * tile count, grid size, occupancy (workgroups per CU), macro tile
 * (bm x bn, k-step bk in elements), and the tile body of the launch that
 * computes the whole tiles: 0 = the generic kernel (unaligned sizes),
 * 1 = the fast kernel with lockstep waves, 2 = the fast kernel in ping-pong,
 * 3 = the fast kernel with producer waves (pgemm_mainloop_t). Output
 * pointers may be NULL. Alignment is judged from
 * the sizes only (pointers assumed 16-byte aligned). */
int pgemm_query_launch(pgemm_handle_t h, int64_t M, int64_t N, int64_t K, int dtype, int sched_mode,
                       int grid_multiple, int* tiles, int* grid, int* occupancy, int* bm, int* bn, int* bk,
                       int* body);

/* Report the STREAMK split pgemm_run would use for this problem, without
 * launching: whole_tiles = W*G tiles run whole, split_tiles = R tail
 * tiles whose k-steps are split, split_groups = workgroups sharing them,
 * pieces_split = tail tiles actually cut into two or more pieces (0: no
 * fix-up launch), workspace_bytes = the workspace the run needs (0 when
 * nothing is cut). Output pointers may be NULL. Operands that take the
 * generic kernel report split_tiles = 0. */
int pgemm_query_streamk(pgemm_handle_t h, int64_t M, int64_t N, int64_t K, int dtype, int grid_multiple,
                        int* whole_tiles, int* split_tiles, int* split_groups, int* pieces_split,
                        int64_t* workspace_bytes);

/* Tile-order knobs: GROUP_SIZE_M of the grouped order (default 4; the
 * Triton issue's setting is 8; 1 = row-major), and the XCD-aware remap
 * (1 = on; 0 = off; -1 = automatic, the default: on for launches with more
 * tiles than the device has CUs, off otherwise). Both apply identically to
 * all modes and never change C's bits, only which workgroup computes which
 * tile. The environment variables PGEMM_GROUP_M and PGEMM_XCD_REMAP override
 * the defaults at pgemm_create. */
int pgemm_set_tile_order(pgemm_handle_t h, int group_m, int xcd_remap);

/* Choose the fast kernel's macro tile for later runs on this handle
 * (pgemm_tile_t). Unaligned operands always take the generic 64 x 64 body.
 * Returns PGEMM_ERR_INVALID_ARG for an unknown value. */
int pgemm_set_tile_config(pgemm_handle_t h, int tile);

/* Per-tensor scales of e4m3 A and B for later PGEMM_F8E4M3_BF16 runs on this
 * handle: the stored codes represent scale_a * dec(a) and scale_b * dec(b),
 * so C[i][j] = scale_a * scale_b * sum_k dec(A[i][k]) * dec(B[k][j]). The
 * epilogue multiplies the fp32 sum by the fp32 product scale_a * scale_b and
 * rounds to bf16 (nearest-even); with power-of-two scales that product and
 * multiplication are exact. Default 1.0 and 1.0 (exact: C unchanged). Other
 * dtypes ignore the scales. PGEMM_ERR_INVALID_ARG for a NULL handle, a
 * non-finite scale or a non-finite product. */
int pgemm_set_fp8_scales(pgemm_handle_t h, float scale_a, float scale_b);

/* Choose the wave schedule of the 256-row tile for later runs on this
 * handle (pgemm_mainloop_t; C's bits do not depend on it). Returns
 * PGEMM_ERR_INVALID_ARG for a NULL handle or an unknown value. */
int pgemm_set_mainloop(pgemm_handle_t h, int mainloop);

/* Choose how B is stored for later runs on this handle (pgemm_b_layout_t;
 * default PGEMM_B_KN). With PGEMM_B_NK the fast kernel copies B's tile like
 * A's (rows of 128 bytes) and reads its fragments with plain 16-byte LDS
 * reads instead of LDS transpose reads. The fast-kernel size rule is the
 * same in both layouts (K and N multiples of 16 bytes of elements).
 * Returns PGEMM_ERR_INVALID_ARG for a NULL handle or an unknown value. */
int pgemm_set_b_layout(pgemm_handle_t h, int layout);

/* Host mirror of the device tile order: (pid_m, pid_n) of tile t for an
 * n_m x n_n tile grid, with the same knobs and CU-count chunking the
 * device uses (cu_chunk = CU count, or 0 for no XCD remap). Pure function,
 * no GPU needed. */
int pgemm_tile_coords(int64_t t, int64_t n_m, int64_t n_n, int group_m, int cu_chunk, int* pid_m,
                      int* pid_n);

/* Read the device work counter of the claiming modes (synchronizes the
 * handle's stream). It reads 0 between launches -- each launch's last claim
 * resets it -- so any other value means a launch was cut short. */
int pgemm_read_work_counter(pgemm_handle_t h, int32_t* value);

/* Benchmark aid, not part of the GEMM: make about `n_cus` CUs of device
 * `device` unavailable for about `microseconds`, asynchronously on the HIP
 * stream `hip_stream` (NULL = null stream). It launches n_cus workgroups
 * that each hold a whole CU's LDS (so no GEMM workgroup can share that CU)
 * and idle until the device's constant-rate clock has advanced by the
 * given time; the wait is also capped by a pass count, so the kernel ends
 * even if that clock stalled. Used to measure the schedulers when only part
 * of the GPU is available (KernelWiki "Persistent Kernels with Cluster
 * Launch Control", "Choosing between static and CLC scheduling"). n_cus in
 * [0, 65536], microseconds in [0, 10^6], else PGEMM_ERR_INVALID_ARG; 0 for
 * either launches nothing. */
int pgemm_hold_cus(void* hip_stream, int device, int n_cus, int microseconds);

#ifdef __cplusplus
}
#endif

#endif /* PGEMM_H */
