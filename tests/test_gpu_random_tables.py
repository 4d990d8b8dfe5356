"""Seeded random segment tables against the CPU oracle.

Each case draws a table mixing every bin-length class (per-element maxima
below 4, 8-bit words below 64, register tiles up to 4093, streamed long bins
up to 32768), hard local selection layers, one-element and ragged layers and
gaps between layers, with spans on both sides of the small-table limit and,
now and then, more layers than the small-table finish takes; and a value mix
(normal at a random scale, a small set with ties, +-0 and a denormal, or
magnitudes spread over 60 decades).  Four compress steps from a random
residue run with three finishes (the default: small-table or two-kernel,
whichever the table takes; three-kernel; single launch where it applies):
their messages, residues and bin maxima must be equal byte for byte, and
the default's first two must match the oracle (tests/parity.py).  Then the
case's four messages, with a foreign one among them, are decoded
(accumulate into a random start; summed from +0 by the default decode and by
the entry-record decode the three-kernel plan's flag selects), decoded with
an SGD step and with an Adam step, each against the oracle bit for bit."""
import sys

import numpy as np
import pytest
import torch

import adaptive_residual_gradient_amd as A
import oracle
from parity import bits, compare_step

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CASES = 48


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def random_table(rng):
    many = rng.random() < 0.15
    nseg = int(rng.integers(200, 300)) if many else int(rng.integers(1, 24))
    segs, off = [], 4 * int(rng.integers(0, 3))
    for _ in range(nseg):
        r = rng.random()
        if many or r < 0.3:
            numel = int(rng.integers(1, 70))
        elif r < 0.8:
            numel = int(rng.integers(70, 20000))
        elif r < 0.96:
            numel = int(rng.integers(20000, 400000))
        else:
            numel = int(rng.integers(1_000_000, 3_000_000))
        r = rng.random()
        if r < 0.35:
            lt = int(rng.integers(1, 64))
        elif r < 0.8:
            lt = int(rng.integers(64, 4094))
        else:
            lt = int(rng.integers(4094, 32769))
        flags = A.SEG_LS if rng.random() < 0.2 else 0
        segs.append((off, numel, lt, flags))
        off += (numel + 3) // 4 * 4 + 4 * int(rng.integers(0, 3))
    return segs, off + 4


def random_values(rng, n, kind, scale):
    if kind == "normal":
        return (rng.standard_normal(n) * scale).astype(np.float32)
    if kind == "ties":
        return rng.choice(np.float32([0, -0.0, 0.5, -0.5, 1, -1, 0.25, 2, -2, 1e-40]), n)
    mag = 10.0 ** rng.uniform(-30, 30, n)
    return (mag * rng.choice([-1.0, 1.0], n)).astype(np.float32)


@pytest.mark.parametrize("seed", range(CASES))
def test_random_table(seed):
    rng = np.random.default_rng(1000 + seed)
    segs, span = random_table(rng)
    kind = ["normal", "ties", "wide"][seed % 3]
    scale = float(10.0 ** rng.uniform(-6, 0))
    plans = [A.Plan(segs), A.Plan(segs, plan_flags=A.PLAN_SEPARATE_FINISH | A.PLAN_DECODE_RECORDS),
             A.Plan(segs, plan_flags=A.PLAN_SINGLE_LAUNCH)]
    info = plans[0].info
    say(f"  seed {seed}: {len(segs)} layers, span {span}, {info.ntiles} tiles, {kind}, "
        f"launches {[int(p.info.compress_launches) for p in plans]}")
    bufs = [dict(msg=p.message_buffer(DEV), ws=p.compress_workspace(DEV),
                 g=torch.empty(int(info.total_bins), dtype=torch.float32, device=DEV)) for p in plans]
    r_host = random_values(rng, span, kind, scale)
    residues = [torch.from_numpy(r_host.copy()).to(DEV) for _ in plans]
    msgs = []
    for step in range(4):
        d = random_values(rng, span, kind, scale)
        d_dev = torch.from_numpy(d).to(DEV)
        r_in = residues[0].cpu().numpy()
        for p, b, r in zip(plans, bufs, residues):
            A.compress(p, r, d_dev, b["msg"], b["ws"], bin_max_out=b["g"])
        torch.cuda.synchronize()
        outs = []
        for p, b, r in zip(plans, bufs, residues):
            total, _, _ = A.message_header(p, b["msg"])
            outs.append((b["msg"][:total].cpu().numpy(), r.cpu().numpy(), b["g"].cpu().numpy()))
        for name, o in zip(("three-kernel finish", "single launch or default"), outs[1:]):
            assert np.array_equal(o[0], outs[0][0]), f"{name}: message differs"
            assert np.array_equal(bits(o[1]), bits(outs[0][1])), f"{name}: residue differs"
            assert np.array_equal(bits(o[2]), bits(outs[0][2])), f"{name}: bin maxima differ"
        if step < 2:
            compare_step(segs, r_in, d, outs[0][1], outs[0][0], outs[0][2])
        msgs.append(outs[0][0])

    # Decode the four messages with a foreign one (wrong magic) among them.
    foreign = msgs[1].copy()
    foreign[0] ^= 0xFF
    pos = int(rng.integers(0, len(msgs) + 1))
    dev_msgs = [torch.from_numpy(m).to(DEV) for m in msgs]
    dev_msgs.insert(pos, torch.from_numpy(foreign).to(DEV))
    K = len(dev_msgs)
    plan = plans[0]
    start = random_values(rng, span, "normal", scale)
    out = torch.from_numpy(start.copy()).to(DEV)
    A.decode_accumulate(plan, dev_msgs, out, True, plan.decode_workspace(K, DEV))
    want = start.copy()
    oracle.decode_accumulate(segs, msgs, want, True)
    assert np.array_equal(bits(out.cpu().numpy()), bits(want)), "decode_accumulate"
    # the plain sum, also on the entry-record decode (the second plan carries that flag)
    for pl in (plans[0], plans[1]):
        out = torch.from_numpy(start.copy()).to(DEV)
        A.decode_accumulate(pl, dev_msgs, out, False, pl.decode_workspace(K, DEV))
        want = start.copy()
        oracle.decode_accumulate(segs, msgs, want, False)
        assert np.array_equal(bits(out.cpu().numpy()), bits(want)), "decode (sum)"

    ws = plan.decode_sgd_workspace(K, DEV)
    w0 = random_values(rng, span, "normal", 1.0)
    m0 = random_values(rng, span, "normal", 0.1)
    w, m = torch.from_numpy(w0.copy()).to(DEV), torch.from_numpy(m0.copy()).to(DEV)
    A.decode_sgd(plan, dev_msgs, w, m, 0.05, 0.9, ws, weight_decay=1e-4, scale=0.25)
    wh, mh = w0.copy(), m0.copy()
    oracle.decode_sgd(segs, msgs, wh, mh, 0.05, 0.9, weight_decay=1e-4, scale=0.25)
    assert np.array_equal(bits(w.cpu().numpy()), bits(wh)), "decode_sgd weights"
    assert np.array_equal(bits(m.cpu().numpy()), bits(mh)), "decode_sgd momentum"

    v0 = np.abs(random_values(rng, span, "normal", 0.01))
    w, m, v = (torch.from_numpy(x.copy()).to(DEV) for x in (w0, m0, v0))
    A.decode_adam(plan, dev_msgs, w, m, v, 1e-3, 0.9, 0.999, 1e-8, 3, ws, weight_decay=1e-4,
                  scale=0.25)
    wh, mh, vh = w0.copy(), m0.copy(), v0.copy()
    oracle.decode_adam(segs, msgs, wh, mh, vh, 1e-3, 0.9, 0.999, 1e-8, 3, weight_decay=1e-4,
                       scale=0.25)
    assert np.array_equal(bits(w.cpu().numpy()), bits(wh)), "decode_adam weights"
    assert np.array_equal(bits(m.cpu().numpy()), bits(mh)), "decode_adam m"
    assert np.array_equal(bits(v.cpu().numpy()), bits(vh)), "decode_adam v"
    for p in plans:
        p.close()
