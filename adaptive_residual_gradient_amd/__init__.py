"""AdaComp for AMD Instinct MI355X: Python binding of ``libadacomp.so``.

A thin ctypes layer over the C ABI declared in ``include/adacomp.h``: it
marshals torch tensors (device memory) and the current HIP stream into plain
pointers and sizes.  Every step of compression and decoding runs in the HIP
kernels of the library; nothing here computes.  If the library is not built,
every call raises ``HipLibraryMissing``; there is no fallback.

Method: "AdaComp (Adaptive Residual Gradient Compression)", AIMech curated
page, definition paragraph and Mechanism claim on local-bin soft threshold
and mean-g_max quantization (Algorithm 2).
"""
from __future__ import annotations

import ctypes
import pathlib
from typing import Iterable, List, Optional, Sequence

_HERE = pathlib.Path(__file__).resolve().parent
LIB_PATH = _HERE / "libadacomp.so"

OK = 0
NUM_STAGES = 11
STAGES = ("tile_pass", "chunk_scan", "finalize", "encode",
          "decode_count", "decode_base", "decode_apply", "compress_call", "decode_call",
          "decode_sgd_call", "decode_adam_call")
MAX_MESSAGES = 256
MAX_BIN_LEN = 32768
SEG_LS = 1   # segment flag: hard local selection (see include/adacomp.h)
PLAN_SEPARATE_FINISH = 1   # plan flag: finish with three kernels whatever the table
PLAN_SINGLE_LAUNCH = 2     # plan flag: a small table in one launch (slower; for comparison)
PLAN_DECODE_RECORDS = 4    # plan flag: plain sums always take the entry-record decode
SMALL_TABLE_MAX_SPAN = 1 << 21     # tables up to this span and this many segments
SMALL_TABLE_MAX_SEGMENTS = 256     # finish in one launch after the tile pass
NOALLOC_SCRATCH_BYTES = 128 << 20  # largest compress workspace compress_noalloc takes
CHUNK_FINISH_MAX_TILES = 1 << 20   # larger tables of <= 256 segments and this many tiles: two


class HipLibraryMissing(RuntimeError):
    pass


class AdaCompError(RuntimeError):
    def __init__(self, where: str, status: int):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} ({status})")


class _Segment(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_uint64), ("numel", ctypes.c_uint64),
                ("bin_len", ctypes.c_uint32), ("flags", ctypes.c_uint32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("nseg", ctypes.c_uint32), ("plan_hash", ctypes.c_uint32),
                ("total_numel", ctypes.c_uint64), ("span", ctypes.c_uint64),
                ("total_bins", ctypes.c_uint64), ("ntiles", ctypes.c_uint64),
                ("header_bytes", ctypes.c_uint64), ("message_capacity", ctypes.c_uint64),
                ("compress_workspace_bytes", ctypes.c_uint64),
                ("decode_workspace_bytes_per_message", ctypes.c_uint64),
                ("decode_workspace_bytes_fixed", ctypes.c_uint64),
                ("compress_launches", ctypes.c_uint64)]

    def as_dict(self):
        return {name: int(getattr(self, name)) for name, _ in self._fields_}

    def decode_workspace_bytes(self, K: int) -> int:
        return int(self.decode_workspace_bytes_fixed) + K * int(self.decode_workspace_bytes_per_message)


class Sgd(ctypes.Structure):
    """One step of SGD with momentum: g = scale*sum (+ weight_decay*w),
    m = momentum*m + g, w = w - lr*m."""
    _fields_ = [("lr", ctypes.c_float), ("momentum", ctypes.c_float),
                ("weight_decay", ctypes.c_float), ("scale", ctypes.c_float)]


class Adam(ctypes.Structure):
    """One Adam step (bias-corrected moments); see include/adacomp.h."""
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("scale", ctypes.c_float), ("step", ctypes.c_uint32)]


# Every exported symbol, with its C signature (argtypes, restype).
_P = ctypes.c_void_p
_U32, _U64, _INT = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int
SIGNATURES = {
    "adacomp_plan_query": ([ctypes.POINTER(_Segment), _U32, ctypes.POINTER(PlanInfo)], _INT),
    "adacomp_plan_create": ([ctypes.POINTER(_Segment), _U32, ctypes.POINTER(_P)], _INT),
    "adacomp_plan_create_ex": ([ctypes.POINTER(_Segment), _U32, _U32, ctypes.POINTER(_P)], _INT),
    "adacomp_plan_destroy": ([_P], _INT),
    "adacomp_plan_get_info": ([_P, ctypes.POINTER(PlanInfo)], _INT),
    "adacomp_compress": ([_P, _P, _P, _U64, _P, _U64, _P, _U64, _P, _P], _INT),
    "adacomp_compress_noalloc": ([_P, _P, _P, _U64, _P, _U64, _P, _P], _INT),
    "adacomp_decode_accumulate": ([_P, ctypes.POINTER(_P), _U32, _P, _U64, _INT, _P, _U64, _P], _INT),
    "adacomp_compress_timed": ([_P, _P, _P, _U64, _P, _U64, _P, _U64, _P, _P, _P], _INT),
    "adacomp_decode_accumulate_timed": ([_P, ctypes.POINTER(_P), _U32, _P, _U64, _INT, _P, _U64,
                                         _P, _P], _INT),
    "adacomp_decode_sgd": ([_P, ctypes.POINTER(_P), _U32, _P, _P, _U64, ctypes.POINTER(Sgd), _P, _U64,
                            _P], _INT),
    "adacomp_decode_sgd_timed": ([_P, ctypes.POINTER(_P), _U32, _P, _P, _U64, ctypes.POINTER(Sgd), _P,
                                  _U64, _P, _P], _INT),
    "adacomp_decode_sgd_workspace_bytes": ([_P, _U32, ctypes.POINTER(_U64)], _INT),
    "adacomp_decode_adam": ([_P, ctypes.POINTER(_P), _U32, _P, _P, _P, _U64, ctypes.POINTER(Adam), _P,
                             _U64, _P], _INT),
    "adacomp_decode_adam_timed": ([_P, ctypes.POINTER(_P), _U32, _P, _P, _P, _U64, ctypes.POINTER(Adam),
                                   _P, _U64, _P, _P], _INT),
    "adacomp_timer_create": ([ctypes.POINTER(_P)], _INT),
    "adacomp_timer_destroy": ([_P], _INT),
    "adacomp_timer_read": ([_P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_U64), _U32], _INT),
    "adacomp_timer_reset": ([_P], _INT),
    "adacomp_status_str": ([_INT], ctypes.c_char_p),
}

_lib = None


def lib():
    """The loaded HIP library; raises HipLibraryMissing if it is not built."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise HipLibraryMissing(
                f"{LIB_PATH} is not built; build it with __graft_entry__.build() "
                "(hipcc --offload-arch=gfx950)")
        h = ctypes.CDLL(str(LIB_PATH))
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.argtypes = args
            fn.restype = res
        _lib = h
    return _lib


def status_str(status: int) -> str:
    try:
        return lib().adacomp_status_str(int(status)).decode()
    except HipLibraryMissing:
        return "unknown"


def _check(where: str, st: int) -> None:
    if st != OK:
        raise AdaCompError(where, st)


def _segments(segments: Iterable[Sequence[int]]):
    segs = list(segments)
    arr = (_Segment * max(1, len(segs)))()
    for i, s in enumerate(segs):
        arr[i] = _Segment(int(s[0]), int(s[1]), int(s[2]), int(s[3]) if len(s) > 3 else 0)
    return arr, len(segs)


def plan_query(segments) -> PlanInfo:
    """Host-only: validate a segment table and return the sizes of its plan."""
    arr, n = _segments(segments)
    info = PlanInfo()
    _check("adacomp_plan_query", lib().adacomp_plan_query(arr, n, ctypes.byref(info)))
    return info


def _stream_handle(stream) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _f32_ptr(t, name: str) -> int:
    import torch
    if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous float32 CUDA tensor")
    return t.data_ptr()


def _u8_ptr(t, name: str) -> int:
    import torch
    if t.dtype != torch.uint8 or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous uint8 CUDA tensor")
    return t.data_ptr()


class Timer:
    """Per-kernel-stage device time recorded with HIP events on the stream."""

    def __init__(self):
        h = _P()
        _check("adacomp_timer_create", lib().adacomp_timer_create(ctypes.byref(h)))
        self.handle = h

    def read(self):
        ms = (ctypes.c_double * NUM_STAGES)()
        n = (_U64 * NUM_STAGES)()
        _check("adacomp_timer_read", lib().adacomp_timer_read(self.handle, ms, n, NUM_STAGES))
        return {STAGES[i]: (float(ms[i]), int(n[i])) for i in range(NUM_STAGES)}

    def reset(self):
        _check("adacomp_timer_reset", lib().adacomp_timer_reset(self.handle))

    def close(self):
        if self.handle:
            lib().adacomp_timer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Plan:
    """A segment table made into device tile tables on the current device.

    ``segments``: (offset, numel, bin_len) or (offset, numel, bin_len, flags)
    per layer, offsets in elements of the flat float32 buffers (multiples of
    4); flags 0 (AdaComp) or SEG_LS.  ``plan_flags``: 0, PLAN_SEPARATE_FINISH
    or PLAN_SINGLE_LAUNCH (``info.compress_launches`` says how many launches
    a compress call makes)."""

    def __init__(self, segments, plan_flags: int = 0):
        self.segments = [tuple(int(x) for x in s) for s in segments]
        arr, n = _segments(self.segments)
        h = _P()
        _check("adacomp_plan_create_ex",
               lib().adacomp_plan_create_ex(arr, n, int(plan_flags), ctypes.byref(h)))
        self.handle = h
        info = PlanInfo()
        _check("adacomp_plan_get_info", lib().adacomp_plan_get_info(h, ctypes.byref(info)))
        self.info = info

    def close(self):
        if getattr(self, "handle", None):
            lib().adacomp_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # Buffer helpers (torch allocations are 256-byte aligned).
    def message_buffer(self, device="cuda"):
        import torch
        return torch.empty(int(self.info.message_capacity), dtype=torch.uint8, device=device)

    def compress_workspace(self, device="cuda"):
        import torch
        return torch.empty(int(self.info.compress_workspace_bytes), dtype=torch.uint8, device=device)

    def decode_workspace(self, K: int, device="cuda"):
        import torch
        return torch.empty(self.info.decode_workspace_bytes(K), dtype=torch.uint8, device=device)

    def decode_sgd_workspace_bytes(self, K: int) -> int:
        n = _U64(0)
        _check("adacomp_decode_sgd_workspace_bytes",
               lib().adacomp_decode_sgd_workspace_bytes(self.handle, int(K), ctypes.byref(n)))
        return int(n.value)

    def decode_sgd_workspace(self, K: int, device="cuda"):
        import torch
        return torch.empty(self.decode_sgd_workspace_bytes(K), dtype=torch.uint8, device=device)


def compress(plan: Plan, residue, dW, msg, ws, bin_max_out=None, stream=None,
             timer: Optional[Timer] = None) -> None:
    """One AdaComp step: residue updated in place, message written to msg."""
    bm = _f32_ptr(bin_max_out, "bin_max_out") if bin_max_out is not None else None
    if bin_max_out is not None and bin_max_out.numel() < plan.info.total_bins:
        raise ValueError("bin_max_out shorter than the plan's total_bins")
    n = min(residue.numel(), dW.numel())
    st = lib().adacomp_compress_timed(
        plan.handle, _f32_ptr(residue, "residue"), _f32_ptr(dW, "dW"), n,
        _u8_ptr(msg, "msg"), msg.numel(), _u8_ptr(ws, "ws"), ws.numel(), bm,
        _stream_handle(stream), timer.handle if timer is not None else None)
    _check("adacomp_compress", st)


def compress_noalloc(plan: Plan, residue, dW, msg, bin_max_out=None, stream=None) -> None:
    """One AdaComp step as compress(), its workspace the library's own
    per-GPU scratch: the call allocates no device memory.  Calls that may
    overlap on one GPU race on that scratch."""
    bm = _f32_ptr(bin_max_out, "bin_max_out") if bin_max_out is not None else None
    if bin_max_out is not None and bin_max_out.numel() < plan.info.total_bins:
        raise ValueError("bin_max_out shorter than the plan's total_bins")
    n = min(residue.numel(), dW.numel())
    st = lib().adacomp_compress_noalloc(
        plan.handle, _f32_ptr(residue, "residue"), _f32_ptr(dW, "dW"), n,
        _u8_ptr(msg, "msg"), msg.numel(), bm, _stream_handle(stream))
    _check("adacomp_compress_noalloc", st)


def decode_accumulate(plan: Plan, msgs: List, out, accumulate: bool, ws, stream=None,
                      timer: Optional[Timer] = None) -> None:
    """Sum the messages (in list order) into out."""
    ptrs = (_P * max(1, len(msgs)))(*[_u8_ptr(m, "msgs[k]") for m in msgs])
    st = lib().adacomp_decode_accumulate_timed(
        plan.handle, ptrs, len(msgs), _f32_ptr(out, "out"), out.numel(),
        1 if accumulate else 0, _u8_ptr(ws, "ws"), ws.numel(), _stream_handle(stream),
        timer.handle if timer is not None else None)
    _check("adacomp_decode_accumulate", st)


def decode_sgd(plan: Plan, msgs: List, weights, momentum, lr: float, momentum_coef: float,
               ws, weight_decay: float = 0.0, scale: float = 1.0, stream=None,
               timer: Optional[Timer] = None) -> None:
    """Sum the messages (in list order) and take one SGD-with-momentum step on
    weights and momentum (in place), without writing the sum."""
    ptrs = (_P * max(1, len(msgs)))(*[_u8_ptr(m, "msgs[k]") for m in msgs])
    n = min(weights.numel(), momentum.numel())
    p = Sgd(lr, momentum_coef, weight_decay, scale)
    st = lib().adacomp_decode_sgd_timed(
        plan.handle, ptrs, len(msgs), _f32_ptr(weights, "weights"), _f32_ptr(momentum, "momentum"),
        n, ctypes.byref(p), _u8_ptr(ws, "ws"), ws.numel(), _stream_handle(stream),
        timer.handle if timer is not None else None)
    _check("adacomp_decode_sgd", st)


def decode_adam(plan: Plan, msgs: List, weights, m, v, lr: float, beta1: float, beta2: float,
                eps: float, step: int, ws, weight_decay: float = 0.0, scale: float = 1.0,
                stream=None, timer: Optional[Timer] = None) -> None:
    """Sum the messages (in list order) and take Adam step number ``step``
    (>= 1) on weights, m and v (in place), without writing the sum.  ws as
    for decode_sgd (Plan.decode_sgd_workspace)."""
    ptrs = (_P * max(1, len(msgs)))(*[_u8_ptr(x, "msgs[k]") for x in msgs])
    n = min(weights.numel(), m.numel(), v.numel())
    p = Adam(lr, beta1, beta2, eps, weight_decay, scale, int(step))
    st = lib().adacomp_decode_adam_timed(
        plan.handle, ptrs, len(msgs), _f32_ptr(weights, "weights"), _f32_ptr(m, "m"),
        _f32_ptr(v, "v"), n, ctypes.byref(p), _u8_ptr(ws, "ws"), ws.numel(),
        _stream_handle(stream), timer.handle if timer is not None else None)
    _check("adacomp_decode_adam", st)


def message_header(plan: Plan, msg):
    """Copy a message's header and directory to the host (synchronizes):
    (total_bytes, total_survivors, [(s, nsurv, entries_offset)] per segment)."""
    from .stats import read_header
    raw = bytes(msg[: int(plan.info.header_bytes)].cpu().numpy().tobytes())
    return read_header(raw, int(plan.info.nseg))
