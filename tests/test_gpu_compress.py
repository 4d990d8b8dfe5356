"""GPU parity of adacomp_compress against the CPU oracle (step-locked), on the
synthetic workloads at their full sizes and on edge-case segment tables.
Tolerances are documented in tests/parity.py."""
import sys

import numpy as np
import pytest
import torch

import adaptive_residual_gradient_amd as A
import msgparse as mp
import oracle
import workloads as W
from parity import bits, compare_step

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_gpu_step(plan, r_dev, d_dev, msg, ws, gmax):
    A.compress(plan, r_dev, d_dev, msg, ws, bin_max_out=gmax)
    torch.cuda.synchronize()
    total, _, _ = A.message_header(plan, msg)
    return msg[:total].cpu().numpy(), r_dev.cpu().numpy(), gmax.cpu().numpy()


def run_workload(wl, steps, learner=0):
    plan = A.Plan(wl.segments)
    n = W.alloc_len(wl)
    r_dev = torch.zeros(n, dtype=torch.float32, device=DEV)
    d_dev = torch.empty(n, dtype=torch.float32, device=DEV)
    msg = plan.message_buffer(DEV)
    ws = plan.compress_workspace(DEV)
    gmax = torch.empty(int(plan.info.total_bins), dtype=torch.float32, device=DEV)
    reports = []
    for step in range(1, steps + 1):
        W.fill_dw(d_dev, wl, learner, step)
        r_in = r_dev.cpu().numpy()
        d = d_dev.cpu().numpy()
        say(f"  {wl.name} step {step}: compress {wl.numel} elements")
        m, r_out, g = run_gpu_step(plan, r_dev, d_dev, msg, ws, gmax)
        reports.append(compare_step(wl.segments, r_in, d, r_out, m, g))
    plan.close()
    return reports


@pytest.mark.parametrize("name,steps", [("fc", 10), ("conv", 50), ("resnet50", 20),
                                        ("fc_lstm", 50)])
def test_workload_parity(name, steps):
    wl = W.workload(name)
    reps = run_workload(wl, steps)
    s_total = sum(r.segments for r in reps)
    s_exact = sum(r.s_exact for r in reps)
    say(f"{name}: {steps} steps, s bit-exact {s_exact}/{s_total}, "
        f"messages identical {sum(r.msg_identical for r in reps)}/{steps}, "
        f"survivors first/last {reps[0].survivors}/{reps[-1].survivors}")
    assert s_exact >= s_total - 1


def _values(rng, n, kind):
    if kind == "normal":
        return (rng.standard_normal(n) * 1e-3).astype(np.float32)
    if kind == "ties":
        return rng.choice(np.float32([0, -0.0, 0.5, -0.5, 1, -1, 0.25, 2, -2, 1e-40]), n)
    if kind == "zero":
        return np.zeros(n, np.float32)
    raise ValueError(kind)


EDGE_BINS = [1, 2, 3, 4, 5, 7, 50, 63, 64, 65, 500, 4093, 4094, 5000, 32767, 32768]
EDGE_NUMEL = [1, 2, 3, 5, 7, 63, 65, 4093, 4097, 36861, 40003]


# Tables this small finish with one kernel by default; they also run with the
# three-kernel finish and (bins held in registers, L_T <= 4093) in one launch.
EDGE_CASES = ([(lt, 0) for lt in EDGE_BINS] + [(lt, A.PLAN_SEPARATE_FINISH) for lt in EDGE_BINS] +
              [(lt, A.PLAN_SINGLE_LAUNCH) for lt in EDGE_BINS if lt <= 4093])


@pytest.mark.parametrize("lt,plan_flags", EDGE_CASES)
def test_edge_bin_lengths(lt, plan_flags):
    """Every bin length class (per-element path L_T < 4, two-run path, 8/16-bit
    switch at 64, register tiles / streamed long bins at 4093/4094, the 16-bit
    maximum), ragged last bins, tiny segments, gaps between segments, ties
    and +-0."""
    rng = np.random.default_rng(lt)
    segs, off = [], 4
    for n in EDGE_NUMEL:
        segs.append((off, n, lt))
        off += (n + 3) // 4 * 4 + 8
    span = off + 4
    plan = A.Plan(segs, plan_flags=plan_flags)
    say(f"  L_T={lt}: {plan.info.compress_launches} compress launches")
    msg, ws = plan.message_buffer(DEV), plan.compress_workspace(DEV)
    gmax = torch.empty(int(plan.info.total_bins), dtype=torch.float32, device=DEV)
    for kind in ("normal", "ties"):
        r = _values(rng, span, kind)
        d = _values(rng, span, kind)
        r_dev = torch.from_numpy(r.copy()).to(DEV)
        d_dev = torch.from_numpy(d).to(DEV)
        say(f"  L_T={lt} {kind}: {len(segs)} segments")
        m, r_out, g = run_gpu_step(plan, r_dev, d_dev, msg, ws, gmax)
        compare_step(segs, r, d, r_out, m, g)
        # a second step from the updated residue
        d2 = _values(rng, span, kind)
        r_dev2 = torch.from_numpy(r_out.copy()).to(DEV)
        m, r_out2, g = run_gpu_step(plan, r_dev2, torch.from_numpy(d2).to(DEV), msg, ws, gmax)
        compare_step(segs, r_out, d2, r_out2, m, g)
    plan.close()


def test_degenerate_inputs():
    """All-zero layer (nothing sent, s = 0); dW = 0 (exactly the bin maxima and
    their ties are sent); zero residue (H = 2 dW)."""
    segs = [(0, 10000, 50), (10000, 7001, 500)]
    span = 17004
    plan = A.Plan(segs)
    msg, ws = plan.message_buffer(DEV), plan.compress_workspace(DEV)
    gmax = torch.empty(int(plan.info.total_bins), dtype=torch.float32, device=DEV)
    rng = np.random.default_rng(1)
    cases = {
        "all_zero": (np.zeros(span, np.float32), np.zeros(span, np.float32)),
        "dw_zero": (rng.choice(np.float32([-1, -0.5, 0, 0.5, 1]), span), np.zeros(span, np.float32)),
        "residue_zero": (np.zeros(span, np.float32), (rng.standard_normal(span) * 1e-3).astype(np.float32)),
        "negative_zero": (np.full(span, -0.0, np.float32), np.full(span, -0.0, np.float32)),
    }
    for name, (r, d) in cases.items():
        say(f"  degenerate {name}")
        m, r_out, g = run_gpu_step(plan, torch.from_numpy(r.copy()).to(DEV),
                                   torch.from_numpy(d).to(DEV), msg, ws, gmax)
        compare_step(segs, r, d, r_out, m, g)
        pm = mp.parse(m, segs)
        if name in ("all_zero", "negative_zero"):
            assert pm.total_survivors == 0 and all(sm.s == 0.0 for sm in pm.segs)
            np.testing.assert_array_equal(bits(r_out[:span]), bits((r + d)[:span]))
    plan.close()


def test_survivor_distribution_extremes():
    """The encode shares survivors out evenly among wavefronts, so its start
    search and tile walk must hold for both extremes: a few survivors spread
    over long runs of empty tiles (most bins all zero), and a first step from
    a zero residue where a large share of the elements survive."""
    segs = [(0, 3000000, 50), (3000000, 1000000, 500), (4000000, 2000003, 7),
            (6000004, 4096, 4093)]
    span = 6000004 + 4096
    plan = A.Plan(segs)
    msg, ws = plan.message_buffer(DEV), plan.compress_workspace(DEV)
    gmax = torch.empty(int(plan.info.total_bins), dtype=torch.float32, device=DEV)
    rng = np.random.default_rng(11)
    # sparse: only every 997th bin of each layer is nonzero
    r = np.zeros(span, np.float32)
    d = np.zeros(span, np.float32)
    for off, n, lt in segs:
        for b0 in range(0, n, 997 * lt):
            e = min(b0 + lt, n)
            d[off + b0:off + e] = (rng.standard_normal(e - b0) * 1e-3).astype(np.float32)
    say("  sparse survivors")
    m, r_out, g = run_gpu_step(plan, torch.from_numpy(r.copy()).to(DEV), torch.from_numpy(d).to(DEV),
                               msg, ws, gmax)
    rep = compare_step(segs, r, d, r_out, m, g)
    say(f"    survivors {rep.survivors}")
    # dense: first step from zero residue
    d = (rng.standard_normal(span) * 1e-3).astype(np.float32)
    say("  dense first step")
    m, r_out, g = run_gpu_step(plan, torch.from_numpy(r.copy()).to(DEV), torch.from_numpy(d).to(DEV),
                               msg, ws, gmax)
    rep = compare_step(segs, r, d, r_out, m, g)
    say(f"    survivors {rep.survivors}")
    assert rep.survivors > span // 20
    plan.close()


@pytest.mark.parametrize("values", ["normal", "ties"])
def test_local_selection_parity(values):
    """Hard local selection (segment flag 1) next to AdaComp layers, over every
    tile shape (bins of 1 to 32768 elements, the 1024-thread tiles included),
    ragged last bins and ties of the bin maximum; three steps each, then the
    LS messages summed by decode_accumulate."""
    lts = [1, 3, 50, 500, 4093, 5000, 32768]
    segs, off = [], 0
    for i, lt in enumerate(lts):
        n = lt * 5 + 3 if lt > 1000 else 40003
        segs.append((off, n, lt, A.SEG_LS if i % 2 == 0 else 0))
        segs.append((off + (n + 3) // 4 * 4, 4097, lt, A.SEG_LS if i % 2 == 1 else 0))
        off += (n + 3) // 4 * 4 + 4100
    span = off
    plan = A.Plan(segs)
    msg, ws = plan.message_buffer(DEV), plan.compress_workspace(DEV)
    gmax = torch.empty(int(plan.info.total_bins), dtype=torch.float32, device=DEV)
    rng = np.random.default_rng(17)
    r = np.zeros(span, np.float32)
    host_msgs, dev_msgs = [], []
    for step in range(3):
        d = _values(rng, span, values)
        say(f"  LS table, {values}, step {step}")
        m, r_out, g = run_gpu_step(plan, torch.from_numpy(r.copy()).to(DEV),
                                   torch.from_numpy(d).to(DEV), msg, ws, gmax)
        rep = compare_step(segs, r, d, r_out, m, g)
        pm = mp.parse(m, segs)
        for (o, n, lt, fl), sm in zip(segs, pm.segs):
            if fl == A.SEG_LS:
                assert int(sm.counts.max()) <= 1
        host_msgs.append(m.copy())
        dev_msgs.append(torch.from_numpy(m.copy()).to(DEV))
        r = r_out
    say(f"    survivors {rep.survivors}")
    out = torch.zeros(span, dtype=torch.float32, device=DEV)
    A.decode_accumulate(plan, dev_msgs, out, False, plan.decode_workspace(3, DEV))
    want = np.zeros(span, np.float32)
    oracle.decode_accumulate(segs, host_msgs, want, False)
    np.testing.assert_array_equal(bits(out.cpu().numpy()), bits(want))
    plan.close()


def test_local_selection_conv_workload():
    """The conv workload (L_T = 50) with every layer under hard local
    selection, 20 steps with the residue carried over."""
    wl = W.workload("conv")
    segs = [(o, n, lt, A.SEG_LS) for (o, n, lt) in wl.segments]
    plan = A.Plan(segs)
    n = W.alloc_len(wl)
    r_dev = torch.zeros(n, dtype=torch.float32, device=DEV)
    d_dev = torch.empty(n, dtype=torch.float32, device=DEV)
    msg, ws = plan.message_buffer(DEV), plan.compress_workspace(DEV)
    gmax = torch.empty(int(plan.info.total_bins), dtype=torch.float32, device=DEV)
    for step in range(1, 21):
        W.fill_dw(d_dev, wl, 0, step)
        r_in, d = r_dev.cpu().numpy(), d_dev.cpu().numpy()
        m, r_out, g = run_gpu_step(plan, r_dev, d_dev, msg, ws, gmax)
        rep = compare_step(segs, r_in, d, r_out, m, g)
    say(f"  conv under LS: survivors at step 20 {rep.survivors} (bins {wl.bins})")
    assert rep.survivors <= wl.bins
    plan.close()


def test_table_order_differs_from_memory_order():
    """Layers listed in another order than they lie in memory (message
    regions follow the table, elements the offsets), with gaps; compress and
    a decode of two such messages."""
    segs = [(60000, 5003, 50), (0, 40001, 500), (48008, 7, 3), (40004, 8000, 4094)]
    span = 65004
    plan = A.Plan(segs)
    msg, ws = plan.message_buffer(DEV), plan.compress_workspace(DEV)
    gmax = torch.empty(int(plan.info.total_bins), dtype=torch.float32, device=DEV)
    rng = np.random.default_rng(23)
    host_msgs, dev_msgs = [], []
    for k in range(2):
        r = (rng.standard_normal(span) * 1e-3).astype(np.float32)
        d = (rng.standard_normal(span) * 1e-3).astype(np.float32)
        m, r_out, g = run_gpu_step(plan, torch.from_numpy(r.copy()).to(DEV),
                                   torch.from_numpy(d).to(DEV), msg, ws, gmax)
        compare_step(segs, r, d, r_out, m, g)
        host_msgs.append(m.copy())
        dev_msgs.append(torch.from_numpy(m.copy()).to(DEV))
    out = torch.full((span,), 7.0, dtype=torch.float32, device=DEV)
    A.decode_accumulate(plan, dev_msgs, out, False, plan.decode_workspace(2, DEV))
    want = np.full(span, 7.0, np.float32)
    oracle.decode_accumulate(segs, host_msgs, want, False)
    np.testing.assert_array_equal(bits(out.cpu().numpy()), bits(want))
    plan.close()


def test_one_layer_of_many_scan_chunks():
    """A single layer of 2^28 elements (131072 tiles, 128 scan chunks in one
    layer): the chunk-level offsets and the encode's start search across
    chunks, checked in full against the oracle over two steps."""
    n = 1 << 28
    segs = [(0, n, 500)]
    plan = A.Plan(segs)
    msg, ws = plan.message_buffer(DEV), plan.compress_workspace(DEV)
    gmax = torch.empty(int(plan.info.total_bins), dtype=torch.float32, device=DEV)
    r_dev = torch.zeros(n, dtype=torch.float32, device=DEV)
    d_dev = torch.empty(n, dtype=torch.float32, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(29)
    for step in range(2):
        d_dev.normal_(0.0, 1e-3, generator=gen)
        r_in, d = r_dev.cpu().numpy(), d_dev.cpu().numpy()
        say(f"  one layer of {n} elements, step {step}")
        m, r_out, g = run_gpu_step(plan, r_dev, d_dev, msg, ws, gmax)
        rep = compare_step(segs, r_in, d, r_out, m, g)
        say(f"    survivors {rep.survivors}")
    plan.close()
    del r_dev, d_dev, msg, ws, gmax
    torch.cuda.empty_cache()


def test_layer_past_two_to_the_31():
    """One layer of 2^31 + 5 elements (ragged last bin): every element index,
    tile offset and survivor count past the signed 32-bit range, compared in
    full with the oracle; then decoded (K = 1) and compared."""
    n = (1 << 31) + 5
    segs = [(0, n, 500)]
    plan = A.Plan(segs)
    span = int(plan.info.span)
    msg, ws = plan.message_buffer(DEV), plan.compress_workspace(DEV)
    r_dev = torch.empty(span, dtype=torch.float32, device=DEV)
    d_dev = torch.empty(span, dtype=torch.float32, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(31)
    r_dev.normal_(0.0, 1e-3, generator=gen)
    d_dev.normal_(0.0, 1e-3, generator=gen)
    r_in, d = r_dev.cpu().numpy(), d_dev.cpu().numpy()
    say(f"  one layer of {n} elements")
    A.compress(plan, r_dev, d_dev, msg, ws)
    torch.cuda.synchronize()
    total, surv, _ = A.message_header(plan, msg)
    m = msg[:total].cpu().numpy()
    del ws
    rep = compare_step(segs, r_in, d, r_dev.cpu().numpy(), m)
    say(f"    survivors {rep.survivors}, message {total} bytes")
    del r_dev, d_dev, r_in, d
    out = torch.empty(span, dtype=torch.float32, device=DEV)
    A.decode_accumulate(plan, [msg], out, False, plan.decode_workspace(1, DEV))
    want = np.empty(span, np.float32)
    oracle.decode_accumulate(segs, [m], want, False)
    np.testing.assert_array_equal(bits(out[:n].cpu().numpy()), bits(want[:n]))
    plan.close()
    del out, msg
    torch.cuda.empty_cache()


def test_determinism_and_resume():
    """Two runs give the same bits; 5 steps + residue checkpoint + 5 steps equal
    10 straight steps."""
    wl = W.workload("conv")
    plan = A.Plan(wl.segments)
    n = W.alloc_len(wl)
    msg, ws = plan.message_buffer(DEV), plan.compress_workspace(DEV)
    dws = [W.make_dw(wl, 0, s, DEV) for s in range(1, 11)]

    def run(r, steps):
        out = []
        for d in steps:
            A.compress(plan, r, d, msg, ws)
            total, _, _ = A.message_header(plan, msg)
            out.append(bytes(msg[:total].cpu().numpy()))
        return out

    r1 = torch.zeros(n, dtype=torch.float32, device=DEV)
    m1 = run(r1, dws)
    r2 = torch.zeros(n, dtype=torch.float32, device=DEV)
    m2 = run(r2, dws)
    assert m1 == m2 and torch.equal(r1.view(torch.int32), r2.view(torch.int32))
    r3 = torch.zeros(n, dtype=torch.float32, device=DEV)
    m3 = run(r3, dws[:5])
    saved = r3.cpu().clone()
    r4 = saved.to(DEV)
    m3 += run(r4, dws[5:])
    assert m3 == m1
    assert torch.equal(r4.view(torch.int32), r1.view(torch.int32))
    plan.close()


def test_argument_errors():
    segs = [(0, 1000, 50)]
    plan = A.Plan(segs)
    r = torch.zeros(1008, dtype=torch.float32, device=DEV)
    d = torch.zeros(1008, dtype=torch.float32, device=DEV)
    msg, ws = plan.message_buffer(DEV), plan.compress_workspace(DEV)
    with pytest.raises(A.AdaCompError) as e:
        A.compress(plan, r, d, msg[:100], ws)
    assert e.value.status == -5
    with pytest.raises(A.AdaCompError) as e:
        A.compress(plan, r, d, msg, ws[:64])
    assert e.value.status == -5
    with pytest.raises(A.AdaCompError) as e:
        A.compress(plan, r[1:], d[1:], msg, ws)
    assert e.value.status == -3
    with pytest.raises(A.AdaCompError) as e:
        A.compress(plan, r[:500], d[:500], msg, ws)
    assert e.value.status == -5
    with pytest.raises(A.AdaCompError) as e:
        A.compress(plan, r, r, msg, ws)
    assert e.value.status == -1
    plan.close()


@pytest.mark.parametrize("name,plan_flags", [("fc", A.PLAN_SEPARATE_FINISH), ("fc", 0),
                                             ("fc", A.PLAN_SINGLE_LAUNCH), ("conv", 0)])
def test_timer_reports_every_stage(name, plan_flags):
    """The three-kernel finish reports its four kernels and the whole call;
    the small-table finish (100x1000 table) the tile pass, its one finish
    kernel (as the encode stage) and the call; the two-kernel finish (conv
    table) the tile pass, the chunk scan, its finish kernel (as the encode
    stage) and the call; the single launch only the call."""
    wl = W.workload(name)
    plan = A.Plan(wl.segments, plan_flags=plan_flags)
    r = torch.zeros(W.alloc_len(wl), dtype=torch.float32, device=DEV)
    d = W.make_dw(wl, 0, 1, DEV)
    msg, ws = plan.message_buffer(DEV), plan.compress_workspace(DEV)
    t = A.Timer()
    for _ in range(3):
        A.compress(plan, r, d, msg, ws, timer=t)
    rd = t.read()
    kernels = ("tile_pass", "chunk_scan", "finalize", "encode")
    recorded = {A.PLAN_SEPARATE_FINISH: kernels, 0: ("tile_pass", "encode"),
                A.PLAN_SINGLE_LAUNCH: ()}[plan_flags]
    if name == "conv":
        recorded = ("tile_pass", "chunk_scan", "encode")
    assert rd["compress_call"][1] == 3 and rd["compress_call"][0] > 0
    for st in kernels:
        if st in recorded:
            assert rd[st][1] == 3 and rd[st][0] > 0
        else:
            assert rd[st][1] == 0 and rd[st][0] == 0
    parts = sum(rd[st][0] for st in kernels)
    assert rd["compress_call"][0] >= 0.9 * parts
    t.close()
    plan.close()
