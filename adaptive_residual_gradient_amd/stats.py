"""Host-side reporting helpers: compression ratios of an AdaComp message.

The payload ratio follows the arithmetic behind the figures on the "AdaComp"
AIMech page (Application claim, Table 2; Mechanism claim on self-adjusting
sparsity, Figures 4-6): a layer of N float32 values (32 bits each) sent as
n_sent index words of w bits compresses by 32*N / (w*n_sent).  With about 5
words sent per bin of L_T values that is 32*L_T/(5*w): 40x for conv layers
(L_T = 50, 8-bit words), 200x for FC/LSTM layers (L_T = 500, 16-bit words)
and 2000x at L_T = 5000.  The wire ratio also counts what the payload ratio
leaves out: the header, the directory and the per-bin counts.
"""
from __future__ import annotations

import struct
from typing import Iterable, Sequence, Tuple


def word_bits(bin_len: int) -> int:
    """Index word width: 8 bits when L_T < 64, 16 bits otherwise."""
    return 8 if bin_len < 64 else 16


def payload_ratio(numel: int, sent: Iterable[Tuple[int, int]]) -> float:
    """32*numel / sum(w * n_sent) over (n_sent, w) pairs; inf if nothing sent."""
    bits = sum(int(n) * int(w) for n, w in sent)
    return float("inf") if bits == 0 else 32.0 * numel / bits


def per_bin_ratio(bin_len: int, sent_per_bin: float) -> float:
    """Payload ratio of one full bin with ``sent_per_bin`` words sent."""
    return 32.0 * bin_len / (word_bits(bin_len) * sent_per_bin)


def wire_ratio(numel: int, total_bytes: int) -> float:
    return 4.0 * numel / total_bytes


def read_header(raw: bytes, nseg: int):
    """Header and directory of a message: (total_bytes, total_survivors,
    [(s, nsurv, entries_offset)] * nseg).  ``raw`` holds at least the first
    32 + 16*nseg bytes."""
    magic, ver, _, n, _, total, surv = struct.unpack_from("<IHHIIQQ", raw, 0)
    if magic != 0x43414441 or ver != 1 or n != nseg:
        raise ValueError("not an AdaComp message for this segment table")
    dirs = [struct.unpack_from("<fIQ", raw, 32 + 16 * i) for i in range(nseg)]
    return total, surv, dirs


def message_ratios(segments: Sequence, raw: bytes):
    """(payload ratio, wire ratio, total_bytes, total_survivors)."""
    total, surv, dirs = read_header(raw, len(segments))
    numel = sum(int(s[1]) for s in segments)
    pr = payload_ratio(numel, ((d[1], word_bits(int(s[2]))) for d, s in zip(dirs, segments)))
    return pr, wire_ratio(numel, total), total, surv
