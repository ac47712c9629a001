"""Python binding of libpgemm (persistent-tile-scheduled GEMM for MI355X).

Argument marshalling only: every step of the GEMM runs in the HIP kernels
behind the C ABI declared in include/pgemm.h, and the functions here carry
the same names as its entry points. torch is used only to hand over device
memory (``tensor.data_ptr()``) and streams. There is no fallback: if the
HIP library has not been built, importing this package raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpgemm.so")

PGEMM_OK = 0
PGEMM_ERR_INVALID_ARG = 1
PGEMM_ERR_UNSUPPORTED = 2
PGEMM_ERR_HIP = 3
PGEMM_ERR_OOM = 4
PGEMM_ERR_TIMEOUT = 5

PGEMM_F16 = 0
PGEMM_BF16 = 1
PGEMM_F8E4M3_BF16 = 2

PGEMM_SCHED_NONPERSISTENT = 0
PGEMM_SCHED_STATIC = 1
PGEMM_SCHED_DYNAMIC = 2
PGEMM_SCHED_CANCEL = 3
PGEMM_SCHED_STREAMK = 4

PGEMM_TILE_AUTO = 0
PGEMM_TILE_256 = 1
PGEMM_TILE_128 = 2

PGEMM_B_KN = 0
PGEMM_B_NK = 1

PGEMM_MAINLOOP_AUTO = 0
PGEMM_MAINLOOP_LOCKSTEP = 1
PGEMM_MAINLOOP_PINGPONG = 2
PGEMM_MAINLOOP_PRODUCER = 3

DTYPE_NAMES = {"f16": PGEMM_F16, "bf16": PGEMM_BF16, "e4m3fn": PGEMM_F8E4M3_BF16}
SCHED_NAMES = {"nonpersistent": PGEMM_SCHED_NONPERSISTENT, "static": PGEMM_SCHED_STATIC,
               "dynamic": PGEMM_SCHED_DYNAMIC, "cancel": PGEMM_SCHED_CANCEL, "streamk": PGEMM_SCHED_STREAMK}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python -m persistent_tile_scheduling_macro_amd.build` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)
_vp, _i64, _i32, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
_ip = ctypes.POINTER(ctypes.c_int)


def _sig(name, restype, *argtypes):
    f = getattr(_lib, name)
    f.restype = restype
    f.argtypes = list(argtypes)
    return f


_create = _sig("pgemm_create", _int, ctypes.POINTER(_vp), _int)
_set_stream = _sig("pgemm_set_stream", _int, _vp, _vp)
_run = _sig("pgemm_run", _int, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _int)
_run_noalloc = _sig("pgemm_run_noalloc", _int, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _int)
_run_ld = _sig("pgemm_run_ld", _int, _vp, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _int, _int, _int)
_destroy = _sig("pgemm_destroy", _int, _vp)
_status_string = _sig("pgemm_status_string", ctypes.c_char_p, _int)
_last_error = _sig("pgemm_last_error", ctypes.c_char_p, _vp)
_set_tile_counter = _sig("pgemm_set_tile_counter", _int, _vp, _vp, _i64)
_set_owner_log = _sig("pgemm_set_owner_log", _int, _vp, _vp, _i64)
_set_tile_trace = _sig("pgemm_set_tile_trace", _int, _vp, _vp, _i64)
_clock_khz = _sig("pgemm_clock_khz", _int, _int, _ip)
_wait = _sig("pgemm_wait", _int, _vp, _int)
_query_launch = _sig("pgemm_query_launch", _int, _vp, _i64, _i64, _i64, _int, _int, _int,
                     _ip, _ip, _ip, _ip, _ip, _ip, _ip)
_query_streamk = _sig("pgemm_query_streamk", _int, _vp, _i64, _i64, _i64, _int, _int, _ip, _ip, _ip, _ip,
                      ctypes.POINTER(_i64))
_set_tile_order = _sig("pgemm_set_tile_order", _int, _vp, _int, _int)
_set_tile_config = _sig("pgemm_set_tile_config", _int, _vp, _int)
_set_b_layout = _sig("pgemm_set_b_layout", _int, _vp, _int)
_set_mainloop = _sig("pgemm_set_mainloop", _int, _vp, _int)
_set_fp8_scales = _sig("pgemm_set_fp8_scales", _int, _vp, ctypes.c_float, ctypes.c_float)
_tile_coords = _sig("pgemm_tile_coords", _int, _i64, _i64, _i64, _int, _int, _ip, _ip)
_read_work_counter = _sig("pgemm_read_work_counter", _int, _vp, ctypes.POINTER(_i32))
_hold_cus = _sig("pgemm_hold_cus", _int, _vp, _int, _int, _int)


class PgemmError(RuntimeError):
    def __init__(self, status: int, detail: str = ""):
        self.status = status
        msg = pgemm_status_string(status)
        super().__init__(f"{msg}: {detail}" if detail else msg)


def _check(status: int, h=None) -> None:
    if status != PGEMM_OK:
        raise PgemmError(status, pgemm_last_error(h) if h else "")


def _ptr(x) -> int:
    """Device address of a torch tensor (or an int address / None)."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def pgemm_status_string(status: int) -> str:
    return _status_string(int(status)).decode()


def pgemm_last_error(h) -> str:
    return _last_error(h).decode()


def pgemm_create(device: int = 0):
    """Create a handle on `device`; returns an opaque handle (ctypes c_void_p)."""
    h = _vp()
    _check(_create(ctypes.byref(h), int(device)))
    return h


def _stream_ptr(stream):
    """hipStream_t of a torch.cuda.Stream, a raw int handle, or None (null stream)."""
    if stream is not None and not isinstance(stream, int):
        stream = int(stream.cuda_stream)
    return stream or None


def pgemm_set_stream(h, stream) -> None:
    """Bind a stream: a torch.cuda.Stream, a raw hipStream_t int, or None (null stream)."""
    _check(_set_stream(h, _stream_ptr(stream)), h)


def pgemm_run(h, A, B, C, M: int, N: int, K: int, dtype: int, sched_mode: int, grid_multiple: int = 0) -> None:
    """Enqueue C = A @ B (device pointers or tensors) on the handle's stream."""
    _check(_run(h, _ptr(A), _ptr(B), _ptr(C), int(M), int(N), int(K), int(dtype), int(sched_mode),
                int(grid_multiple)), h)


def pgemm_run_noalloc(h, A, B, C, M: int, N: int, K: int, dtype: int, sched_mode: int,
                      grid_multiple: int = 0) -> None:
    """pgemm_run that allocates nothing (stream-K partial tiles in the device's fixed scratch)."""
    _check(_run_noalloc(h, _ptr(A), _ptr(B), _ptr(C), int(M), int(N), int(K), int(dtype), int(sched_mode),
                        int(grid_multiple)), h)


PGEMM_NOALLOC_SCRATCH_BYTES = 96 << 20


def pgemm_run_ld(h, A, lda: int, B, ldb: int, C, ldc: int, M: int, N: int, K: int, dtype: int,
                 sched_mode: int, grid_multiple: int = 0) -> None:
    """pgemm_run with leading dimensions (in elements) for row-major views; pointers or tensors
    (a tensor's data_ptr() is the view's first element)."""
    _check(_run_ld(h, _ptr(A), int(lda), _ptr(B), int(ldb), _ptr(C), int(ldc), int(M), int(N), int(K),
                   int(dtype), int(sched_mode), int(grid_multiple)), h)


def pgemm_destroy(h) -> None:
    _check(_destroy(h))


def pgemm_set_tile_counter(h, visits, n_tiles: int = 0) -> None:
    """Attach an int32 device buffer of n_tiles visit counters (tensor or pointer); None detaches."""
    if visits is not None and not isinstance(visits, int) and not n_tiles:
        n_tiles = visits.numel()
    _check(_set_tile_counter(h, _ptr(visits) or None, int(n_tiles)), h)


def pgemm_set_owner_log(h, owner, n_tiles: int = 0) -> None:
    if owner is not None and not isinstance(owner, int) and not n_tiles:
        n_tiles = owner.numel()
    _check(_set_owner_log(h, _ptr(owner) or None, int(n_tiles)), h)


def pgemm_set_tile_trace(h, trace, n_tiles: int = 0) -> None:
    """trace: int64 device tensor of 4 * n_tiles entries ({wg, xcd, start, end} per tile), or None."""
    if trace is not None and not isinstance(trace, int) and not n_tiles:
        n_tiles = trace.numel() // 4
    _check(_set_tile_trace(h, _ptr(trace) or None, int(n_tiles)), h)


def pgemm_wait(h, timeout_ms: int) -> None:
    """Watchdog wait on the handle's stream; raises PgemmError(PGEMM_ERR_TIMEOUT) past the deadline."""
    _check(_wait(h, int(timeout_ms)), h)


def pgemm_clock_khz(device: int = 0) -> int:
    v = ctypes.c_int()
    _check(_clock_khz(int(device), ctypes.byref(v)))
    return v.value


def pgemm_query_launch(h, M: int, N: int, K: int, dtype: int, sched_mode: int, grid_multiple: int = 0) -> dict:
    out = [ctypes.c_int() for _ in range(7)]
    _check(_query_launch(h, int(M), int(N), int(K), int(dtype), int(sched_mode), int(grid_multiple),
                         *[ctypes.byref(o) for o in out]), h)
    keys = ["tiles", "grid", "occupancy", "bm", "bn", "bk", "body"]
    d = {k: o.value for k, o in zip(keys, out)}
    d["fast_path"] = int(d["body"] != 0)  # 0: generic kernel; body 1 lockstep, 2 ping-pong, 3 producer waves
    return d


def pgemm_query_streamk(h, M: int, N: int, K: int, dtype: int, grid_multiple: int = 0) -> dict:
    out = [ctypes.c_int() for _ in range(4)]
    ws = _i64()
    _check(_query_streamk(h, int(M), int(N), int(K), int(dtype), int(grid_multiple),
                          *[ctypes.byref(o) for o in out], ctypes.byref(ws)), h)
    keys = ["whole_tiles", "split_tiles", "split_groups", "pieces_split"]
    d = {k: o.value for k, o in zip(keys, out)}
    d["workspace_bytes"] = ws.value
    return d


def pgemm_set_tile_order(h, group_m: int = 8, xcd_remap=True) -> None:
    """xcd_remap: True/1 on, False/0 off, None/-1 automatic (on when a launch has more tiles than CUs)."""
    if xcd_remap is None or (not isinstance(xcd_remap, bool) and int(xcd_remap) < 0):
        v = -1
    else:
        v = int(bool(xcd_remap))
    _check(_set_tile_order(h, int(group_m), v), h)


def pgemm_set_tile_config(h, tile: int) -> None:
    _check(_set_tile_config(h, int(tile)), h)


def pgemm_set_mainloop(h, mainloop: int) -> None:
    """Wave schedule of the 256-row tile: PGEMM_MAINLOOP_AUTO, _LOCKSTEP, _PINGPONG or _PRODUCER."""
    _check(_set_mainloop(h, int(mainloop)), h)


def pgemm_set_fp8_scales(h, scale_a: float, scale_b: float) -> None:
    """Per-tensor scales of e4m3 A and B (C = scale_a * scale_b * sum of decoded products)."""
    _check(_set_fp8_scales(h, float(scale_a), float(scale_b)), h)


def pgemm_set_b_layout(h, layout: int) -> None:
    """PGEMM_B_KN: B is K x N row-major (default); PGEMM_B_NK: B is N x K row-major."""
    _check(_set_b_layout(h, int(layout)), h)


def pgemm_tile_coords(t: int, n_m: int, n_n: int, group_m: int = 8, cu_chunk: int = 0):
    pm, pn = ctypes.c_int(), ctypes.c_int()
    _check(_tile_coords(int(t), int(n_m), int(n_n), int(group_m), int(cu_chunk), ctypes.byref(pm),
                        ctypes.byref(pn)))
    return pm.value, pn.value


def pgemm_read_work_counter(h) -> int:
    v = ctypes.c_int32()
    _check(_read_work_counter(h, ctypes.byref(v)), h)
    return v.value


def pgemm_hold_cus(stream, device: int, n_cus: int, microseconds: int) -> None:
    """Benchmark aid: hold about n_cus CUs for about `microseconds` on `stream`."""
    _check(_hold_cus(_stream_ptr(stream), int(device), int(n_cus), int(microseconds)))


def matmul(A, B, C=None, *, sched: str | int = "static", grid_multiple: int = 0, handle=None):
    """C = A @ B for 2-D CUDA tensors (fp16, bf16, or float8_e4m3fn with a bf16 C).

    Marshals shapes and pointers into pgemm_run; no arithmetic happens here.
    """
    import torch  # the binding itself does not need torch; this helper does

    dtypes = {torch.float16: PGEMM_F16, torch.bfloat16: PGEMM_BF16, torch.float8_e4m3fn: PGEMM_F8E4M3_BF16}
    if A.dtype != B.dtype or A.dtype not in dtypes:
        raise TypeError(f"unsupported dtypes {A.dtype}, {B.dtype}")
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shape mismatch {tuple(A.shape)} @ {tuple(B.shape)}")
    if not (A.is_cuda and B.is_cuda and A.is_contiguous() and B.is_contiguous()):
        raise ValueError("A and B must be contiguous device tensors")
    M, K = A.shape
    N = B.shape[1]
    out_dtype = torch.bfloat16 if A.dtype == torch.float8_e4m3fn else A.dtype
    if C is None:
        C = torch.empty((M, N), dtype=out_dtype, device=A.device)
    elif C.shape != (M, N) or C.dtype != out_dtype or not C.is_contiguous():
        raise ValueError("C has the wrong shape, dtype or layout")
    own = handle is None
    h = pgemm_create(A.device.index or 0) if own else handle
    try:
        if own:
            pgemm_set_stream(h, torch.cuda.current_stream(A.device))
        s = SCHED_NAMES[sched] if isinstance(sched, str) else int(sched)
        pgemm_run(h, A, B, C, M, N, K, dtypes[A.dtype], s, grid_multiple)
    finally:
        if own:
            pgemm_destroy(h)
    return C
