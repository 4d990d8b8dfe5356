"""Test-side parser of the AdaComp message format.

Written independently of both the HIP library and the C oracle, so that the
tests can check any message's structure (header, directory, count and entry
regions, alignment and zero padding) and read back the transmitted set.

Layout (little-endian, every region 16-byte aligned, padding zero):
  header (32 B): u32 magic 0x43414441, u16 version 1, u16 0, u32 nseg,
                 u32 plan_hash, u64 total_bytes, u64 total_survivors
  directory: nseg x {f32 s, u32 nsurv, u64 entries_offset}
  count regions: per segment, B words of w bits
  entry regions: per segment, nsurv words of w bits: sign << (w-1) | index
  w = 8 if L_T < 64 else 16
"""
from __future__ import annotations

import struct
from dataclasses import dataclass
from typing import List, Sequence

import numpy as np

MAGIC = 0x43414441


def fnv1a32(data: bytes) -> int:
    h = 0x811C9DC5
    for b in data:
        h ^= b
        h = (h * 0x01000193) & 0xFFFFFFFF
    return h


def table_hash(segments) -> int:
    raw = b"".join(struct.pack("<QQII", int(s[0]), int(s[1]), int(s[2]),
                               int(s[3]) if len(s) > 3 else 0) for s in segments)
    return fnv1a32(raw)


def align16(x: int) -> int:
    return (x + 15) // 16 * 16


def word_bytes(bin_len: int) -> int:
    return 1 if bin_len < 64 else 2


@dataclass
class SegmentMsg:
    s: float
    s_bits: int
    nsurv: int
    entries_offset: int
    counts: np.ndarray      # int64 [B]
    words: np.ndarray       # int64 [nsurv], raw entry words
    index: np.ndarray       # int64 [nsurv], element index within the segment
    negative: np.ndarray    # bool [nsurv]


@dataclass
class Message:
    nseg: int
    plan_hash: int
    total_bytes: int
    total_survivors: int
    segs: List[SegmentMsg]


class FormatError(AssertionError):
    pass


def _check(cond, what):
    if not cond:
        raise FormatError(what)


def as_bytes(buf) -> bytes:
    if isinstance(buf, (bytes, bytearray, memoryview)):
        return bytes(buf)
    return np.ascontiguousarray(buf, dtype=np.uint8).tobytes()


def parse(buf, segments: Sequence, strict: bool = True) -> Message:
    """Parse ``buf`` (bytes-like or uint8 array) against the segment table.
    With ``strict`` every structural rule is checked, padding included."""
    b = as_bytes(buf)
    _check(len(b) >= 32, "message shorter than its header")
    magic, ver, zero, nseg, phash, total, nsurv_all = struct.unpack_from("<IHHIIQQ", b, 0)
    _check(magic == MAGIC, f"bad magic {magic:#x}")
    _check(ver == 1 and zero == 0, "bad version field")
    _check(nseg == len(segments), "nseg does not match the table")
    if strict:
        _check(phash == table_hash(segments), "plan hash mismatch")
        _check(total % 16 == 0, "total_bytes not 16-aligned")
        _check(len(b) >= total, "buffer shorter than total_bytes")
    count_at = align16(32 + 16 * nseg)
    if strict:
        _check(all(x == 0 for x in b[32 + 16 * nseg:count_at]), "directory padding not zero")
    count_offs = []
    for (_, n, lt, *rest) in segments:
        nb = (n + lt - 1) // lt
        count_offs.append(count_at)
        end = count_at + nb * word_bytes(lt)
        if strict:
            _check(all(x == 0 for x in b[end:align16(end)]), "count padding not zero")
        count_at = align16(end)
    entry_at = count_at
    segs = []
    surv_sum = 0
    for i, (off, n, lt, *rest) in enumerate(segments):
        wb = word_bytes(lt)
        nb = (n + lt - 1) // lt
        s_bits, nsurv, eoff = struct.unpack_from("<IIQ", b, 32 + 16 * i)
        s = struct.unpack("<f", struct.pack("<I", s_bits))[0]
        dt = np.uint8 if wb == 1 else np.dtype("<u2")
        counts = np.frombuffer(b, dtype=dt, count=nb, offset=count_offs[i]).astype(np.int64)
        if strict:
            _check(eoff == entry_at, f"segment {i}: entries_offset {eoff} != {entry_at}")
            _check(int(counts.sum()) == nsurv, f"segment {i}: counts do not sum to nsurv")
        words = np.frombuffer(b, dtype=dt, count=nsurv, offset=eoff).astype(np.int64)
        sign_bit = 1 << (8 * wb - 1)
        negative = (words & sign_bit) != 0
        idx = words & (sign_bit - 1)
        bins = np.repeat(np.arange(nb, dtype=np.int64), counts)
        if strict:
            blen = np.minimum(lt, n - bins * lt)
            _check(bool(np.all(idx < blen)), f"segment {i}: in-bin index out of range")
            starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
            # ascending in-bin index inside every bin
            if nsurv > 1:
                same_bin = bins[1:] == bins[:-1]
                _check(bool(np.all(idx[1:][same_bin] > idx[:-1][same_bin])),
                       f"segment {i}: indices not strictly ascending within a bin")
            del starts
        end = eoff + nsurv * wb
        if strict:
            _check(all(x == 0 for x in b[end:align16(end)]), "entry padding not zero")
        entry_at = align16(end)
        segs.append(SegmentMsg(s, s_bits, nsurv, eoff, counts, words,
                               bins * lt + idx, negative))
        surv_sum += nsurv
    if strict:
        _check(total == entry_at, f"total_bytes {total} != {entry_at}")
        _check(nsurv_all == surv_sum, "total_survivors mismatch")
    return Message(nseg, phash, total, nsurv_all, segs)


def dense_quantized(msg: Message, segments, length: int) -> np.ndarray:
    """The transmitted G_q as a dense float32 vector (zeros elsewhere)."""
    out = np.zeros(length, dtype=np.float32)
    for sm, (off, n, lt, *rest) in zip(msg.segs, segments):
        vals = np.where(sm.negative, -np.float32(sm.s), np.float32(sm.s)).astype(np.float32)
        out[off + sm.index] = vals
    return out


def sent_mask(msg: Message, segments, length: int) -> np.ndarray:
    m = np.zeros(length, dtype=bool)
    for sm, (off, n, lt, *rest) in zip(msg.segs, segments):
        m[off + sm.index] = True
    return m


def single_segment_message(buf, segments, i: int) -> bytes:
    """Re-pack segment i of a message as a one-segment message for the table
    [(0, numel_i, bin_len_i)] (used to check samples of very large messages
    against the oracle segment by segment)."""
    b = as_bytes(buf)
    msg = parse(b, segments, strict=False)
    sm = msg.segs[i]
    _, n, lt, *rest = segments[i]
    wb = word_bytes(lt)
    nb = (n + lt - 1) // lt
    sub = [(0, n, lt, *rest)]
    count_at = align16(32 + 16)
    entry_at = align16(count_at + nb * wb)
    dt = np.uint8 if wb == 1 else np.dtype("<u2")
    counts = sm.counts.astype(dt).tobytes()
    words = sm.words.astype(dt).tobytes()
    total = align16(entry_at + len(words))
    out = bytearray(total)
    struct.pack_into("<IHHIIQQ", out, 0, MAGIC, 1, 0, 1, table_hash(sub), total, sm.nsurv)
    struct.pack_into("<IIQ", out, 32, sm.s_bits, sm.nsurv, entry_at)
    out[count_at:count_at + len(counts)] = counts
    out[entry_at:entry_at + len(words)] = words
    return bytes(out)
