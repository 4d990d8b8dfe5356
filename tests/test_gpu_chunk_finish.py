"""The two-kernel finish of tables past the small-table limit (at most 256
segments and 2^20 tiles): after the tile pass, the chunk scan and one kernel
in which every workgroup forms s, the entry regions and the directory from
the chunk sums in LDS and encodes its share of the survivors.  Each table is
compressed by it and by the three-kernel finish (PLAN_SEPARATE_FINISH) from
the same residue: messages, residues and bin maxima must be equal byte for
byte, and the first must match the CPU oracle step-locked."""
import sys

import numpy as np
import pytest
import torch

import adaptive_residual_gradient_amd as A
import workloads as W
from parity import bits, compare_step

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_both(segs, r0, ds, oracle_steps):
    """Compress len(ds) steps with both finishes; the first oracle_steps are
    also checked against the oracle.  Returns the survivors per step."""
    plans = [A.Plan(segs), A.Plan(segs, plan_flags=A.PLAN_SEPARATE_FINISH)]
    shapes = A.plan_query(segs).compress_launches - 2
    assert plans[0].info.compress_launches == shapes + 2, "not the two-kernel finish"
    assert plans[1].info.compress_launches == shapes + 3
    bufs = [dict(r=torch.from_numpy(r0.copy()).to(DEV), msg=p.message_buffer(DEV),
                 ws=p.compress_workspace(DEV),
                 g=torch.empty(int(p.info.total_bins), dtype=torch.float32, device=DEV)) for p in plans]
    survivors = []
    for step, d in enumerate(ds):
        d_dev = torch.from_numpy(d).to(DEV)
        r_in = bufs[0]["r"].cpu().numpy() if step < oracle_steps else None
        for p, b in zip(plans, bufs):
            A.compress(p, b["r"], d_dev, b["msg"], b["ws"], bin_max_out=b["g"])
        torch.cuda.synchronize()
        outs = []
        for p, b in zip(plans, bufs):
            total, surv, _ = A.message_header(p, b["msg"])
            outs.append((b["msg"][:total].cpu().numpy(), b["r"].cpu().numpy(), b["g"].cpu().numpy(), surv))
        (m, r, g, surv), (m3, r3, g3, _) = outs
        assert np.array_equal(m, m3), f"step {step}: message differs from the three-kernel finish"
        assert np.array_equal(bits(r), bits(r3)), f"step {step}: residue differs"
        assert np.array_equal(bits(g), bits(g3)), f"step {step}: bin maxima differ"
        if r_in is not None:
            compare_step(segs, r_in, d, r, m, g)
        survivors.append(surv)
    for p in plans:
        p.close()
    return survivors


@pytest.mark.parametrize("name", ["conv", "fc_lstm", "resnet50"])
def test_workloads_both_finishes(name):
    """The conv, FC/LSTM and ResNet-50 tables, 3 steps from zero residue."""
    wl = W.workload(name)
    n = W.alloc_len(wl)
    ds = [W.make_dw(wl, 0, step).numpy() for step in range(1, 4)]
    surv = run_both(wl.segments, np.zeros(n, np.float32), ds, oracle_steps=1)
    say(f"  {name}: survivors {surv}")


def _values(rng, n, scale=1e-3):
    return (rng.standard_normal(n) * scale).astype(np.float32)


def test_mixed_table_at_the_segment_limit():
    """256 segments past the small-table span: hard local selection next to
    AdaComp, every tile shape (register tiles of both sizes, streamed bins),
    8- and 16-bit words, a segment of three scan chunks, one-element and
    ragged segments, gaps."""
    rng = np.random.default_rng(41)
    lts = [1, 3, 7, 50, 63, 64, 500, 2046, 4093, 4094, 9000, 32768]
    segs, off = [], 8
    for i in range(255):
        n = int(rng.integers(1, 9000)) if i % 7 else 1
        segs.append((off, n, lts[i % len(lts)], A.SEG_LS if i % 5 == 0 else 0))
        off += (n + 3) // 4 * 4 + 4 * (i % 3)
    segs.append((off, 5_000_003, 1021, 0))   # 2446 tiles: three scan chunks
    span = off + 5_000_004
    assert len(segs) == 256 and span > A.SMALL_TABLE_MAX_SPAN
    ds = [_values(rng, span) for _ in range(3)]
    surv = run_both(segs, _values(rng, span), ds, oracle_steps=2)
    say(f"  256 segments, span {span}: survivors {surv}")


@pytest.mark.parametrize("kind", ["no_survivors", "all_survive"])
def test_survivor_extremes(kind):
    """No survivor (all-zero input, s = 0) and every element sent (L_T = 1
    from a zero residue), 3 * 2^20 elements in two segments."""
    segs = [(0, 2 << 20, 1 if kind == "all_survive" else 500), (2 << 20, 1 << 20, 1)]
    span = 3 << 20
    rng = np.random.default_rng(43)
    if kind == "no_survivors":
        d = np.zeros(span, np.float32)
    else:
        d = _values(rng, span)
        d[d == 0] = 1e-3
    surv = run_both(segs, np.zeros(span, np.float32), [d], oracle_steps=1)
    assert surv == [0 if kind == "no_survivors" else span]


def test_tile_limit():
    """The largest table the two-kernel finish takes: one layer of 2^20
    tiles (L_T 1025, one bin per tile; 1024 scan chunks in the layer),
    compared in full with the oracle; one tile more takes three kernels."""
    n = (1 << 20) * 1025
    segs = [(0, n, 1025)]
    assert A.plan_query([(0, n + 4, 1025)]).compress_launches == 4
    plan = A.Plan(segs)
    assert plan.info.ntiles == A.CHUNK_FINISH_MAX_TILES and plan.info.compress_launches == 3
    msg, ws = plan.message_buffer(DEV), plan.compress_workspace(DEV)
    gmax = torch.empty(int(plan.info.total_bins), dtype=torch.float32, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(47)
    r_dev = torch.empty(n, dtype=torch.float32, device=DEV).normal_(0.0, 1e-3, generator=gen)
    d_dev = torch.empty(n, dtype=torch.float32, device=DEV).normal_(0.0, 1e-3, generator=gen)
    r_in, d = r_dev.cpu().numpy(), d_dev.cpu().numpy()
    say(f"  one layer of {n} elements, {plan.info.ntiles} tiles")
    A.compress(plan, r_dev, d_dev, msg, ws, bin_max_out=gmax)
    torch.cuda.synchronize()
    total, surv, _ = A.message_header(plan, msg)
    del ws, d_dev
    rep = compare_step(segs, r_in, d, r_dev.cpu().numpy(), msg[:total].cpu().numpy(), gmax.cpu().numpy())
    say(f"    survivors {rep.survivors}, message {total} bytes")
    plan.close()
    del r_dev, msg, gmax
    torch.cuda.empty_cache()
