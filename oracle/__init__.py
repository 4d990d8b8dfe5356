"""AdaComp CPU oracle -- TEST INFRASTRUCTURE ONLY.

A ctypes wrapper around ``adacomp_oracle.c``: a plain, slow, single-threaded C
implementation of the AdaComp compressor (the per-layer residual-gradient
compression step, Algorithm 2) and of the decode-accumulate of several
messages.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package.  It shares no code with the HIP
library under ``adaptive_residual_gradient_amd``; the two meet only in the
seeded input generators of ``workloads``.

Method source: "AdaComp (Adaptive Residual Gradient Compression)", AIMech
curated page, definition paragraph and the Mechanism claim on local-bin soft
threshold and mean-g_max quantization (Algorithm 2); word widths from the
Application claim (Table 2).  The readings taken where the page is silent are
listed in the header comment of ``adacomp_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import pathlib
import subprocess

import numpy as np

_HERE = pathlib.Path(__file__).resolve().parent
_SRC = _HERE / "adacomp_oracle.c"
_LIB_PATH = _HERE / "libadacomp_oracle.so"
# A test may point the wrapper at another build of an oracle source (the
# mutation test loads deliberately broken copies this way); such a library is
# loaded as it is and never rebuilt here.
_LIB_OVERRIDE = os.environ.get("ADACOMP_ORACLE_LIB")

# Plain C, IEEE single and double arithmetic, no contraction into fused
# multiply-adds, no fast-math, no flush-to-zero.
CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build() -> pathlib.Path:
    """Compile the oracle with gcc into ``oracle/libadacomp_oracle.so``."""
    tmp = _LIB_PATH.with_suffix(".so.tmp")
    subprocess.run(["gcc", *CFLAGS, "-o", str(tmp), str(_SRC), "-lm"], check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Seg(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_uint64), ("numel", ctypes.c_uint64),
                ("bin_len", ctypes.c_uint32), ("flags", ctypes.c_uint32)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            path = pathlib.Path(_LIB_OVERRIDE)
            if not path.exists():
                raise OracleError(f"ADACOMP_ORACLE_LIB names a missing file: {path}")
        else:
            path = _LIB_PATH
            if not path.exists():
                build()
        lib = ctypes.CDLL(str(path))
        P = ctypes.POINTER
        lib.oracle_plan_hash.argtypes = [P(_Seg), ctypes.c_uint32]
        lib.oracle_plan_hash.restype = ctypes.c_uint32
        lib.oracle_message_capacity.argtypes = [P(_Seg), ctypes.c_uint32, P(ctypes.c_uint64)]
        lib.oracle_message_capacity.restype = ctypes.c_int
        lib.oracle_compress.argtypes = [P(_Seg), ctypes.c_uint32, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                        ctypes.c_void_p, P(ctypes.c_uint64)]
        lib.oracle_compress.restype = ctypes.c_int
        lib.oracle_decode_accumulate.argtypes = [P(_Seg), ctypes.c_uint32,
                                                 P(ctypes.c_void_p), ctypes.c_uint32,
                                                 ctypes.c_void_p, ctypes.c_int]
        lib.oracle_decode_accumulate.restype = ctypes.c_int
        lib.oracle_decode_sgd.argtypes = [P(_Seg), ctypes.c_uint32, P(ctypes.c_void_p),
                                          ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                          ctypes.c_float]
        lib.oracle_decode_sgd.restype = ctypes.c_int
        lib.oracle_decode_adam.argtypes = [P(_Seg), ctypes.c_uint32, P(ctypes.c_void_p),
                                           ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p] + [ctypes.c_float] * 6 + [ctypes.c_uint32]
        lib.oracle_decode_adam.restype = ctypes.c_int
        _lib = lib
    return _lib


class OracleError(RuntimeError):
    pass


def _segs(segments):
    """segments: iterable of (offset, numel, bin_len) or (offset, numel, bin_len, flags)."""
    segments = list(segments)
    arr = (_Seg * max(1, len(segments)))()
    for i, sg in enumerate(segments):
        off, numel, lt = int(sg[0]), int(sg[1]), int(sg[2])
        flags = int(sg[3]) if len(sg) > 3 else 0
        arr[i] = _Seg(off, numel, lt, flags)
    return arr, len(segments)


def plan_hash(segments) -> int:
    arr, n = _segs(segments)
    return int(_load().oracle_plan_hash(arr, n))


def message_capacity(segments) -> int:
    arr, n = _segs(segments)
    cap = ctypes.c_uint64(0)
    st = _load().oracle_message_capacity(arr, n, ctypes.byref(cap))
    if st != 0:
        raise OracleError(f"oracle_message_capacity failed: {st}")
    return int(cap.value)


def total_bins(segments) -> int:
    return sum((int(s[1]) + int(s[2]) - 1) // int(s[2]) for s in segments)


def compress(segments, residue: np.ndarray, dW: np.ndarray):
    """One compression step.  ``residue`` (float32, contiguous) is updated in
    place.  Returns ``(message, gmax)``: the message bytes (uint8, exactly
    total_bytes long) and every bin maximum (float32, segments in order)."""
    if residue.dtype != np.float32 or dW.dtype != np.float32:
        raise TypeError("residue and dW must be float32")
    if not (residue.flags.c_contiguous and dW.flags.c_contiguous):
        raise ValueError("residue and dW must be contiguous")
    arr, n = _segs(segments)
    span = max(int(s[0]) + int(s[1]) for s in segments)
    if residue.size < span or dW.size < span:
        raise ValueError("buffers shorter than the segment table's span")
    cap = message_capacity(segments)
    msg = np.zeros(cap, dtype=np.uint8)
    gmax = np.zeros(total_bins(segments), dtype=np.float32)
    nbytes = ctypes.c_uint64(0)
    st = _load().oracle_compress(arr, n, residue.ctypes.data, dW.ctypes.data,
                                 msg.ctypes.data, cap, gmax.ctypes.data,
                                 ctypes.byref(nbytes))
    if st != 0:
        raise OracleError(f"oracle_compress failed: {st}")
    return msg[: nbytes.value].copy(), gmax


def decode_accumulate(segments, messages, out: np.ndarray, accumulate: bool) -> None:
    """Sum the messages (in list order) into ``out`` (float32, in place)."""
    if out.dtype != np.float32 or not out.flags.c_contiguous:
        raise TypeError("out must be contiguous float32")
    arr, n = _segs(segments)
    span = max(int(s[0]) + int(s[1]) for s in segments)
    if out.size < span:
        raise ValueError("out shorter than the segment table's span")
    keep = [np.frombuffer(bytes(m), dtype=np.uint8) if isinstance(m, (bytes, bytearray, memoryview))
            else np.ascontiguousarray(m, dtype=np.uint8) for m in messages]
    ptrs = (ctypes.c_void_p * max(1, len(keep)))(*[m.ctypes.data for m in keep])
    st = _load().oracle_decode_accumulate(arr, n, ptrs, len(keep), out.ctypes.data,
                                          1 if accumulate else 0)
    if st != 0:
        raise OracleError(f"oracle_decode_accumulate failed: {st}")


def decode_sgd(segments, messages, w: np.ndarray, m: np.ndarray, lr: float, momentum: float,
               weight_decay: float = 0.0, scale: float = 1.0) -> None:
    """Sum the messages and take one SGD-with-momentum step on ``w`` and ``m``
    (float32, in place): g = scale*sum (+ weight_decay*w), m = momentum*m + g,
    w = w - lr*m, every operation rounded to float32."""
    for a in (w, m):
        if a.dtype != np.float32 or not a.flags.c_contiguous:
            raise TypeError("w and m must be contiguous float32")
    arr, n = _segs(segments)
    span = max(int(s[0]) + int(s[1]) for s in segments)
    if w.size < span or m.size < span:
        raise ValueError("w or m shorter than the segment table's span")
    keep = [np.frombuffer(bytes(x), dtype=np.uint8) if isinstance(x, (bytes, bytearray, memoryview))
            else np.ascontiguousarray(x, dtype=np.uint8) for x in messages]
    ptrs = (ctypes.c_void_p * max(1, len(keep)))(*[x.ctypes.data for x in keep])
    st = _load().oracle_decode_sgd(arr, n, ptrs, len(keep), w.ctypes.data, m.ctypes.data,
                                   float(lr), float(momentum), float(weight_decay), float(scale))
    if st != 0:
        raise OracleError(f"oracle_decode_sgd failed: {st}")


def decode_adam(segments, messages, w: np.ndarray, m: np.ndarray, v: np.ndarray, lr: float,
                beta1: float, beta2: float, eps: float, step: int, weight_decay: float = 0.0,
                scale: float = 1.0) -> None:
    """Sum the messages and take Adam step number ``step`` (>= 1) on w, m, v
    (float32, in place); the formula is in ``adacomp_oracle.c``."""
    for a in (w, m, v):
        if a.dtype != np.float32 or not a.flags.c_contiguous:
            raise TypeError("w, m and v must be contiguous float32")
    arr, n = _segs(segments)
    span = max(int(s[0]) + int(s[1]) for s in segments)
    if min(w.size, m.size, v.size) < span:
        raise ValueError("w, m or v shorter than the segment table's span")
    keep = [np.frombuffer(bytes(x), dtype=np.uint8) if isinstance(x, (bytes, bytearray, memoryview))
            else np.ascontiguousarray(x, dtype=np.uint8) for x in messages]
    ptrs = (ctypes.c_void_p * max(1, len(keep)))(*[x.ctypes.data for x in keep])
    st = _load().oracle_decode_adam(arr, n, ptrs, len(keep), w.ctypes.data, m.ctypes.data,
                                    v.ctypes.data, float(lr), float(beta1), float(beta2), float(eps),
                                    float(weight_decay), float(scale), int(step))
    if st != 0:
        raise OracleError(f"oracle_decode_adam failed: {st}")
