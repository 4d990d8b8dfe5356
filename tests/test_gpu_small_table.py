"""The compress of small tables (span at most 2^21 elements, at most 256
segments): after the tile pass, one finish kernel instead of three, and the
single-launch variant (a plan flag).  Each is checked against the CPU oracle
step-locked and byte for byte against the three-kernel finish of the same
table (PLAN_SEPARATE_FINISH): they round only where that one does, in the
same order.  Also: the single launch's ticket word at the start of the
workspace, whatever the workspace held before."""
import sys

import numpy as np
import pytest
import torch

import adaptive_residual_gradient_amd as A
import workloads as W
from parity import bits, compare_step

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SYNC_IDLE = 0xFFF1ADAC0DE5 << 16   # the ticket word a finished call leaves


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def sync_word(ws) -> int:
    return int(ws[:8].cpu().numpy().view(np.uint64)[0])


class Paths:
    """The same table compressed by every path, each with its own buffers:
    the default (small-table finish), the single launch where the table
    allows it, and the three-kernel finish (the reference)."""

    def __init__(self, segs, r0: np.ndarray, single: bool = True):
        self.segs = segs
        shapes = A.plan_query(segs).compress_launches - 1   # tile-pass launches
        self.small = A.Plan(segs)
        self.plans = [self.small]
        assert self.small.info.compress_launches == shapes + 1
        self.single = None
        if single:
            self.single = A.Plan(segs, plan_flags=A.PLAN_SINGLE_LAUNCH)
            assert self.single.info.compress_launches == 1
            self.plans.append(self.single)
        self.separate = A.Plan(segs, plan_flags=A.PLAN_SEPARATE_FINISH)
        assert self.separate.info.compress_launches == shapes + 3
        self.plans.append(self.separate)
        self.bufs = []
        for plan in self.plans:
            self.bufs.append(dict(
                plan=plan, r=torch.from_numpy(r0.copy()).to(DEV), msg=plan.message_buffer(DEV),
                ws=plan.compress_workspace(DEV),
                g=torch.empty(int(plan.info.total_bins), dtype=torch.float32, device=DEV)))

    def step(self, d: np.ndarray, oracle_check: bool = True):
        d_dev = torch.from_numpy(d).to(DEV)
        r_in = self.bufs[0]["r"].cpu().numpy()
        for b in self.bufs:
            A.compress(b["plan"], b["r"], d_dev, b["msg"], b["ws"], bin_max_out=b["g"])
        torch.cuda.synchronize()
        outs = []
        for b in self.bufs:
            total, surv, _ = A.message_header(b["plan"], b["msg"])
            outs.append((b["msg"][:total].cpu().numpy(), b["r"].cpu().numpy(), b["g"].cpu().numpy(),
                         surv))
        m_ref, r_ref, g_ref, _ = outs[-1]   # the three-kernel finish
        for i, (m, r, g, _) in enumerate(outs[:-1]):
            name = "small-table finish" if i == 0 else "single launch"
            assert np.array_equal(m, m_ref), f"{name}: message differs from the three-kernel finish"
            assert np.array_equal(bits(r), bits(r_ref)), f"{name}: residue differs"
            assert np.array_equal(bits(g), bits(g_ref)), f"{name}: bin maxima differ"
        if self.single is not None:
            assert sync_word(self.bufs[1]["ws"]) == SYNC_IDLE
        if oracle_check:
            compare_step(self.segs, r_in, d, outs[0][1], outs[0][0], outs[0][2])
        return outs[0][3]

    def close(self):
        for plan in self.plans:
            plan.close()


def test_fc_workload_every_path():
    """The 100x1000 layer (L_T 500) for its 10 steps from zero residue."""
    wl = W.workload("fc")
    p = Paths(wl.segments, np.zeros(W.alloc_len(wl), np.float32))
    for step in range(1, 11):
        surv = p.step(W.make_dw(wl, 0, step).numpy())
        say(f"  fc step {step}: {surv} survivors, every path identical, oracle parity")
    p.close()


def _values(rng, n, kind):
    if kind == "normal":
        return (rng.standard_normal(n) * 1e-3).astype(np.float32)
    return rng.choice(np.float32([0, -0.0, 0.5, -0.5, 1, -1, 0.25, 2, -2, 1e-40]), n)


@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_mixed_table_every_path(kind):
    """Both register tile shapes in one table (L_T <= 2045 and 2046..4093),
    hard local selection next to AdaComp layers, 8- and 16-bit words, ragged
    last bins, one-element and unaligned-length segments, gaps."""
    layers = [(100003, 500, 0), (7, 3, 0), (4097, 4093, 0), (36861, 50, A.SEG_LS), (1, 1, 0),
              (65, 64, 0), (5000, 2046, A.SEG_LS), (40003, 7, 0), (4093, 4093, A.SEG_LS)]
    segs, off = [], 8
    for n, lt, fl in layers:
        segs.append((off, n, lt, fl))
        off += (n + 3) // 4 * 4 + 12
    span = off + 4
    rng = np.random.default_rng(11 if kind == "normal" else 12)
    p = Paths(segs, _values(rng, span, kind))
    for step in range(3):
        surv = p.step(_values(rng, span, kind))
        say(f"  mixed {kind} step {step}: {surv} survivors")
    p.close()


def test_long_bins_small_table():
    """Bins longer than 4093 (one streamed bin per tile) next to register
    tiles: the small-table finish takes them; the single launch does not
    (its plan flag leaves such a table on the small-table finish)."""
    segs = [(0, 20000, 5000), (20000, 4097, 50), (24100, 32768, 32768), (56868, 9000, 4094)]
    span = 65868
    rng = np.random.default_rng(21)
    assert A.Plan(segs, plan_flags=A.PLAN_SINGLE_LAUNCH).info.compress_launches == \
        A.Plan(segs).info.compress_launches
    p = Paths(segs, _values(rng, span, "normal"), single=False)
    for step in range(3):
        p.step(_values(rng, span, "normal"))
    p.close()


@pytest.mark.parametrize("case", ["span_limit", "segment_limit", "one_tile"])
def test_size_limits(case):
    """The largest tables the small-table finish takes (span 2^21; 256
    segments of 4 one-bin tiles each, 1024 tiles) and the smallest (one tile:
    in the single launch its workgroup is also the last); one step past the
    span limit the plan takes the two-kernel finish, past the segment limit
    the three-kernel one."""
    if case == "span_limit":
        segs = [(0, (1 << 21) - 4, 500), ((1 << 21) - 4, 4, 3)]
        past, past_launches = [(0, (1 << 21) + 4, 500)], 3
    elif case == "segment_limit":
        segs = [(4100 * i, 4100, 1025) for i in range(255)] + [(4100 * 255, 3076, 1025)]
        past, past_launches = [(4 * i, 4, 4) for i in range(257)], 4
    else:
        segs = [(0, 1000, 500)]
        past = None
    span = max(o + n for o, n, _ in segs)
    rng = np.random.default_rng(3)
    p = Paths(segs, np.zeros((span + 3) // 4 * 4, np.float32))
    say(f"  {case}: {p.small.info.ntiles} tiles, span {p.small.info.span}")
    for _ in range(2):
        p.step(_values(rng, (span + 3) // 4 * 4, "normal"))
    p.close()
    if past is not None:
        info = A.plan_query(past)
        assert info.compress_launches == past_launches
        assert A.Plan(past, plan_flags=A.PLAN_SINGLE_LAUNCH).info.compress_launches == past_launches


@pytest.mark.parametrize("kind", ["no_survivors", "all_survive"])
def test_survivor_extremes(kind):
    """No survivor at all (all-zero input: s = 0, empty entry regions), and
    every element sent (L_T = 1 from a zero residue: |2 dW| >= |dW|), which
    leaves all 65536 entries to the last workgroup's four wavefronts."""
    segs = [(0, 65536, 1)] if kind == "all_survive" else [(0, 60000, 50), (60000, 5536, 500)]
    span = 65536
    rng = np.random.default_rng(7)
    p = Paths(segs, np.zeros(span, np.float32))
    d = np.zeros(span, np.float32) if kind == "no_survivors" else _values(rng, span, "normal")
    if kind == "all_survive":
        d[d == 0] = 1e-3
    surv = p.step(d)
    assert surv == (0 if kind == "no_survivors" else span)
    p.close()


@pytest.mark.parametrize("fill", ["random", "zeros", "ones", "idle", "tag_in_low_half"])
def test_workspace_contents_do_not_matter(fill):
    """Single launch: the ticket word may hold anything but the tag with a
    nonzero count: random bytes, zeros, all ones, the idle word a previous
    call left, the tag's bytes at the wrong place.  Each call gives the
    reference result and leaves the idle word."""
    wl = W.workload("fc")
    n = W.alloc_len(wl)
    plan = A.Plan(wl.segments, plan_flags=A.PLAN_SINGLE_LAUNCH)
    d = W.make_dw(wl, 0, 1, DEV)
    r_ref = torch.zeros(n, dtype=torch.float32, device=DEV)
    m_ref, w_ref = plan.message_buffer(DEV), plan.compress_workspace(DEV)
    A.compress(plan, r_ref, d, m_ref, w_ref)
    torch.cuda.synchronize()
    total, _, _ = A.message_header(plan, m_ref)
    rng = np.random.default_rng(5)
    ws_host = rng.integers(0, 256, int(plan.info.compress_workspace_bytes), dtype=np.uint8)
    word = {"random": None, "zeros": 0, "ones": (1 << 64) - 1, "idle": SYNC_IDLE,
            "tag_in_low_half": SYNC_IDLE >> 16}[fill]
    if word is not None:
        ws_host[:8] = np.array([word], dtype=np.uint64).view(np.uint8)
    for call in range(3):
        ws = torch.from_numpy(ws_host.copy()).to(DEV) if call == 0 else ws
        r = torch.zeros(n, dtype=torch.float32, device=DEV)
        msg = plan.message_buffer(DEV)
        A.compress(plan, r, d, msg, ws)
        torch.cuda.synchronize()
        assert torch.equal(msg[:total], m_ref[:total]), f"call {call}: message"
        assert torch.equal(r.view(torch.int32), r_ref.view(torch.int32)), f"call {call}: residue"
        assert sync_word(ws) == SYNC_IDLE
    plan.close()
