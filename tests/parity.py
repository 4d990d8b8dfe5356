"""Comparison of the HIP path against the CPU oracle, step-locked.

Tolerances (the AdaComp definition fixes every integer and selection result;
only the scale s involves a rounded sum):
  - bin maxima, selection masks, per-bin counts, entry words, directory
    survivor counts and offsets, header totals, message length: bit-exact;
  - s: relative difference <= 1e-6 (the float64 sum of bin maxima may be
    taken in a different order on each side before the single rounding to
    float32; in practice the two agree bit for bit);
  - residue: bit-exact where nothing was sent; where an element was sent,
    |difference| <= 1e-6 * max(|residue_ref|, s_ref), which is bit-exact
    whenever the two s agree;
  - message bytes: identical whenever every s agrees.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

import msgparse as mp
import oracle

S_RTOL = 1e-6
R_RTOL = 1e-6


def bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


@dataclass
class StepReport:
    segments: int = 0
    s_exact: int = 0
    survivors: int = 0
    msg_identical: bool = False
    notes: list = field(default_factory=list)


def compare_step(segments, r_in: np.ndarray, dW: np.ndarray, r_gpu: np.ndarray,
                 msg_gpu: np.ndarray, gmax_gpu: np.ndarray | None = None) -> StepReport:
    """Run the oracle on (r_in, dW) and compare with the GPU's outputs."""
    r_ref = r_in.copy()
    msg_ref, gmax_ref = oracle.compress(segments, r_ref, dW)
    rep = StepReport(segments=len(segments))
    if gmax_gpu is not None:
        np.testing.assert_array_equal(bits(gmax_gpu), bits(gmax_ref), err_msg="bin maxima")
    m_ref = mp.parse(msg_ref, segments)
    m_gpu = mp.parse(msg_gpu, segments)           # strict structural check of the GPU message
    assert m_gpu.total_bytes == m_ref.total_bytes, "total_bytes"
    assert m_gpu.total_survivors == m_ref.total_survivors, "total_survivors"
    assert m_gpu.plan_hash == m_ref.plan_hash
    all_s_equal = True
    for i, (a, b) in enumerate(zip(m_gpu.segs, m_ref.segs)):
        assert a.nsurv == b.nsurv, f"segment {i}: nsurv"
        assert a.entries_offset == b.entries_offset, f"segment {i}: entries_offset"
        np.testing.assert_array_equal(a.counts, b.counts, err_msg=f"segment {i}: counts")
        np.testing.assert_array_equal(a.words, b.words, err_msg=f"segment {i}: entry words")
        if a.s_bits == b.s_bits:
            rep.s_exact += 1
        else:
            all_s_equal = False
            rel = abs(float(a.s) - float(b.s)) / max(abs(float(b.s)), 1e-45)
            assert rel <= S_RTOL, f"segment {i}: s {a.s!r} vs {b.s!r}"
            rep.notes.append(f"segment {i}: s differs by {rel:.2e} relative")
    rep.survivors = m_ref.total_survivors
    g = mp.as_bytes(msg_gpu)[: m_ref.total_bytes]
    rep.msg_identical = bytes(g) == bytes(msg_ref)
    if all_s_equal:
        assert rep.msg_identical, "message bytes differ although every s agrees"
    # residue
    span = r_in.size
    sent = mp.sent_mask(m_ref, segments, span)
    keep = ~sent
    np.testing.assert_array_equal(bits(r_gpu[keep]), bits(r_ref[keep]),
                                  err_msg="residue where nothing was sent (and gaps)")
    if sent.any():
        s_ref = np.zeros(span, np.float32)
        for (off, n, _lt, *rest), sm in zip(segments, m_ref.segs):
            s_ref[off:off + n] = sm.s
        tol = R_RTOL * np.maximum(np.abs(r_ref[sent]), s_ref[sent])
        diff = np.abs(r_gpu[sent].astype(np.float64) - r_ref[sent].astype(np.float64))
        assert np.all(diff <= tol), "residue of sent elements"
        if all_s_equal:
            np.testing.assert_array_equal(bits(r_gpu[sent]), bits(r_ref[sent]))
    return rep
