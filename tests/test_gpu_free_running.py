"""Free-running comparison with the CPU oracle, the secondary signal beside
the step-locked parity tests: the GPU and the oracle each carry their own
residue from zero through a workload's whole step sequence, and each step's
message and residue are compared byte for byte.  Both sides round s once from
a float64 sum, so they stay identical unless a sum rounds differently (the
tolerance allows s to differ by 1e-6 relative); the test fails on any
divergence not caused by such an s difference, and reports how many steps
stayed identical."""
import sys

import numpy as np
import pytest
import torch

import adaptive_residual_gradient_amd as A
import msgparse as mp
import oracle
import workloads as W
from parity import S_RTOL, bits

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("name,steps", [("fc", 10), ("conv", 50), ("fc_lstm", 50), ("resnet50", 20)])
def test_free_running(name, steps):
    wl = W.workload(name)
    plan = A.Plan(wl.segments)
    n = W.alloc_len(wl)
    r_dev = torch.zeros(n, dtype=torch.float32, device=DEV)
    d_dev = torch.empty(n, dtype=torch.float32, device=DEV)
    msg, ws = plan.message_buffer(DEV), plan.compress_workspace(DEV)
    r_host = np.zeros(n, np.float32)
    identical = 0
    for step in range(1, steps + 1):
        W.fill_dw(d_dev, wl, 0, step)
        A.compress(plan, r_dev, d_dev, msg, ws)
        torch.cuda.synchronize()
        total, _, _ = A.message_header(plan, msg)
        m_gpu = msg[:total].cpu().numpy()
        m_ref, _ = oracle.compress(wl.segments, r_host, d_dev.cpu().numpy())
        same_msg = m_gpu.size == m_ref.size and np.array_equal(m_gpu, m_ref)
        same_res = np.array_equal(bits(r_dev.cpu().numpy()), bits(r_host))
        if same_msg and same_res:
            identical += 1
            continue
        # Diverged: only a different rounding of some s may cause it.
        a, b = mp.parse(m_gpu, wl.segments), mp.parse(m_ref, wl.segments)
        diff_s = [i for i, (x, y) in enumerate(zip(a.segs, b.segs)) if x.s_bits != y.s_bits]
        assert diff_s, f"step {step}: diverged with every s equal"
        for i in diff_s:
            rel = abs(float(a.segs[i].s) - float(b.segs[i].s)) / abs(float(b.segs[i].s))
            assert rel <= S_RTOL, f"step {step}, segment {i}: s differs by {rel:.2e}"
        say(f"  {name}: diverged at step {step} through s of segments {diff_s}")
        break
    say(f"  {name}: {identical} of {steps} steps identical free-running")
    plan.close()
