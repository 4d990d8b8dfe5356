"""Pure-Python brute force of one AdaComp compression step, for tiny layers.

Element by element, straight from the definition on the "AdaComp" AIMech page
(definition paragraph; Mechanism claim on local-bin soft threshold and
mean-g_max quantization, Algorithm 2): G = residue + dW, H = G + dW (both
rounded to float32), g_max of each bin of L_T elements, transmit |H| >= g_max
(and G != 0, since a sign bit cannot carry a zero), s = exact mean of the bin
maxima rounded once to float32 (computed here with exact rationals), residue
<- G - sign(G)*s for transmitted elements and G otherwise.

It shares nothing with the C oracle: scalar numpy.float32 arithmetic,
fractions.Fraction for the mean, and the message bytes packed with struct.

Segments with flag 1 use hard Local Selection (the baseline the same page's
Mechanism claim "self-adjusting sparsity prevents residual explosion"
contrasts AdaComp with): per bin only the first element whose |G| equals the
bin maximum is sent, none when the maximum is 0; s and the residue update are
unchanged.
"""
from __future__ import annotations

import struct
from fractions import Fraction

import numpy as np

from msgparse import align16, table_hash, word_bytes

F32 = np.float32


def rn_f32(q: Fraction) -> np.float32:
    """Round an exact rational to the nearest float32, ties to even."""
    if q == 0:
        return F32(0.0)
    guess = F32(float(q))          # float(Fraction) is correctly rounded to double
    cands = {float(guess), float(np.nextafter(guess, F32(np.inf))),
             float(np.nextafter(guess, F32(-np.inf)))}
    best = None
    for c in cands:
        c32 = F32(c)
        if not np.isfinite(c32):
            continue
        err = abs(Fraction(float(c32)) - q)
        key = (err, int(np.frombuffer(c32.tobytes(), dtype=np.uint32)[0]) & 1)
        if best is None or key < best[0]:
            best = (key, c32)
    return best[1]


def ulp_distance(a: np.float32, b: np.float32) -> int:
    ia = int(np.array(a, dtype=np.float32).view(np.int32))
    ib = int(np.array(b, dtype=np.float32).view(np.int32))
    if ia < 0:
        ia = -(ia & 0x7FFFFFFF)
    if ib < 0:
        ib = -(ib & 0x7FFFFFFF)
    return abs(ia - ib)


def compress_segment(r, dw, bin_len, ls=False):
    """Returns (new_residue list, gmax list, s, sent list of (idx, negative))."""
    n = len(r)
    G = [F32(F32(r[j]) + F32(dw[j])) for j in range(n)]
    H = [F32(G[j] + F32(dw[j])) for j in range(n)]
    nb = (n + bin_len - 1) // bin_len
    gmax = []
    for b in range(nb):
        members = [j for j in range(n) if j // bin_len == b]
        gmax.append(max(abs(G[j]) for j in members))
    s = rn_f32(sum((Fraction(float(g)) for g in gmax), Fraction(0)) / nb)
    # LS: the first index of each bin holding the bin maximum (bins with a
    # zero maximum send nothing)
    first = {}
    for j in range(n):
        b = j // bin_len
        if gmax[b] > 0 and abs(G[j]) == gmax[b] and b not in first:
            first[b] = j
    new_r = []
    sent = []
    for j in range(n):
        g = gmax[j // bin_len]
        chosen = first.get(j // bin_len) == j if ls else (abs(H[j]) >= g and G[j] != 0)
        if chosen:
            q = s if G[j] > 0 else -s
            new_r.append(F32(G[j] - q))
            sent.append((j, bool(G[j] < 0)))
        else:
            new_r.append(G[j])
    return new_r, gmax, s, sent


def compress(segments, residue: np.ndarray, dW: np.ndarray):
    """Brute-force step over a segment table.  Returns
    (new_residue array, gmax array, message bytes, list of s)."""
    out_r = residue.astype(np.float32).copy()
    nseg = len(segments)
    count_at = align16(32 + 16 * nseg)
    count_offs = []
    for (_, n, lt, *rest) in segments:
        count_offs.append(count_at)
        count_at = align16(count_at + ((n + lt - 1) // lt) * word_bytes(lt))
    entry_at = count_at
    body = bytearray(entry_at)
    gm_all, s_all = [], []
    entry_blobs = []
    total = 0
    for i, (off, n, lt, *rest) in enumerate(segments):
        wb = word_bytes(lt)
        flags = rest[0] if rest else 0
        r_new, gmax, s, sent = compress_segment(list(residue[off:off + n]),
                                                list(dW[off:off + n]), lt, ls=bool(flags & 1))
        out_r[off:off + n] = np.array(r_new, dtype=np.float32)
        gm_all += gmax
        s_all.append(s)
        nb = len(gmax)
        counts = [0] * nb
        words = []
        for j, neg in sent:
            counts[j // lt] += 1
            words.append(((1 if neg else 0) << (8 * wb - 1)) | (j % lt))
        fmt = "<B" if wb == 1 else "<H"
        for b, c in enumerate(counts):
            struct.pack_into(fmt, body, count_offs[i] + b * wb, c)
        blob = b"".join(struct.pack(fmt, w) for w in words)
        struct.pack_into("<fIQ", body, 32 + 16 * i, float(s), len(words), entry_at)
        blob += bytes(align16(len(blob)) - len(blob))
        entry_blobs.append(blob)
        entry_at += len(blob)
        total += len(words)
    struct.pack_into("<IHHIIQQ", body, 0, 0x43414441, 1, 0, nseg,
                     table_hash(segments), entry_at, total)
    msg = bytes(body) + b"".join(entry_blobs)
    assert len(msg) == entry_at
    return out_r, np.array(gm_all, dtype=np.float32), msg, s_all
