"""adacomp_compress_noalloc (the compress entry point that takes its workspace
from the library's per-GPU scratch) against adacomp_compress with a caller
workspace: the same message bytes, residue and bin maxima, bit for bit, on
two calls in a row -- a conv-sized table, then a smaller single-launch table
(whose ticket counter lives in the scratch's first bytes and must be left
reusable) -- and a third call repeating the first table.  A plan whose
workspace exceeds the scratch is refused before any work."""
import sys

import numpy as np
import pytest
import torch

import adaptive_residual_gradient_amd as A
import workloads as W
from parity import bits

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    return t.cpu().numpy()


def both_ways(plan, segs, n, seed, steps=2):
    """Run `steps` compress steps from the same residue through both entry
    points; compare every step."""
    rng = np.random.default_rng(seed)
    r0 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    r_a = torch.from_numpy(r0.copy()).to(DEV)
    r_b = torch.from_numpy(r0.copy()).to(DEV)
    msg_a, msg_b = plan.message_buffer(DEV), plan.message_buffer(DEV)
    msg_b.fill_(0xCD)
    ws = plan.compress_workspace(DEV)
    nb = int(plan.info.total_bins)
    g_a = torch.empty(nb, dtype=torch.float32, device=DEV)
    g_b = torch.full((nb,), -1.0, dtype=torch.float32, device=DEV)
    for step in range(steps):
        d = torch.from_numpy((rng.standard_normal(n) * 1e-3).astype(np.float32)).to(DEV)
        A.compress(plan, r_a, d, msg_a, ws, bin_max_out=g_a)
        A.compress_noalloc(plan, r_b, d, msg_b, bin_max_out=g_b)
        torch.cuda.synchronize()
        ta, sa, _ = A.message_header(plan, msg_a)
        tb, sb, _ = A.message_header(plan, msg_b)
        assert (ta, sa) == (tb, sb)
        np.testing.assert_array_equal(host(msg_a[:ta]), host(msg_b[:tb]))
        np.testing.assert_array_equal(bits(host(r_a)), bits(host(r_b)))
        np.testing.assert_array_equal(bits(host(g_a)), bits(host(g_b)))
        say(f"  step {step + 1}: {sa} survivors, {ta} bytes, identical")


def test_noalloc_matches_compress_twice_then_smaller():
    wl = W.workload("conv")
    say(f"  noalloc call 1: conv table, {W.alloc_len(wl)} elements")
    plan = A.Plan(wl.segments)
    assert plan.info.compress_workspace_bytes <= A.NOALLOC_SCRATCH_BYTES
    both_ways(plan, wl.segments, W.alloc_len(wl), 11)
    plan.close()

    segs = [(0, 70000, 50), (70000, 30001, 500), (100004, 999, 7)]
    say("  noalloc call 2: a smaller single-launch table, 101003 elements")
    small = A.Plan(segs, plan_flags=A.PLAN_SINGLE_LAUNCH)
    both_ways(small, segs, 101004, 12, steps=3)
    small.close()

    say("  noalloc call 3: the conv table again")
    plan = A.Plan(wl.segments)
    both_ways(plan, wl.segments, W.alloc_len(wl), 13, steps=1)
    plan.close()


def test_noalloc_refuses_plans_past_the_scratch():
    n = A.NOALLOC_SCRATCH_BYTES // 4          # the staging alone would fill the scratch
    plan = A.Plan([(0, n, 500)])
    assert plan.info.compress_workspace_bytes > A.NOALLOC_SCRATCH_BYTES
    r = torch.zeros(16, dtype=torch.float32, device=DEV)
    msg = torch.zeros(64, dtype=torch.uint8, device=DEV)
    with pytest.raises(A.AdaCompError) as e:
        A.compress_noalloc(plan, r, r.clone(), msg)
    assert e.value.status == -8
    plan.close()
