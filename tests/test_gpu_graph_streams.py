"""Use patterns of the C ABI on the GPU: capture in a graph and replay, and one
plan shared by calls on two streams at once.  Checked against the same calls
made eagerly on one stream (bit for bit: the library is deterministic)."""
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


@pytest.mark.parametrize("name,flags,launches", [("conv", 0, 3), ("conv", A.PLAN_SEPARATE_FINISH, 4),
                                                  ("fc", 0, 2), ("fc", A.PLAN_SINGLE_LAUNCH, 1)])
def test_compress_and_decode_in_a_graph(name, flags, launches):
    """compress then decode_accumulate captured once and replayed five times
    on new gradients (copied into the captured input buffer between replays,
    with eager work and synchronisations in between); every replay's residue,
    message and decoded sum equal the eager calls'.  The 100x1000 table takes
    the small-table finish (or, with its flag, the single launch, whose
    ticket word lives in the captured workspace), the conv table the
    two-kernel one (or, with its flag, the three-kernel one)."""
    wl = W.workload(name)
    plan = A.Plan(wl.segments, plan_flags=flags)
    assert plan.info.compress_launches == launches
    n = W.alloc_len(wl)
    msg, ws = plan.message_buffer(DEV), plan.compress_workspace(DEV)
    dws = plan.decode_workspace(1, DEV)
    d_static = torch.empty(n, dtype=torch.float32, device=DEV)
    r_graph = torch.zeros(n, dtype=torch.float32, device=DEV)
    out_graph = torch.empty(n, dtype=torch.float32, device=DEV)
    # eager reference on its own buffers
    r_ref = torch.zeros(n, dtype=torch.float32, device=DEV)
    msg_ref, ws_ref = plan.message_buffer(DEV), plan.compress_workspace(DEV)
    out_ref = torch.empty(n, dtype=torch.float32, device=DEV)
    dws_ref = plan.decode_workspace(1, DEV)

    W.fill_dw(d_static, wl, 0, 1)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            A.compress(plan, r_graph, d_static, msg, ws)
            A.decode_accumulate(plan, [msg], out_graph, False, dws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    r_graph.zero_()   # capture did not run the kernels; start both from zero
    for step in range(1, 6):
        W.fill_dw(d_static, wl, 0, step)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        A.compress(plan, r_ref, d_static, msg_ref, ws_ref)
        A.decode_accumulate(plan, [msg_ref], out_ref, False, dws_ref)
        torch.cuda.synchronize()
        total, _, _ = A.message_header(plan, msg_ref)
        assert torch.equal(msg[:total], msg_ref[:total]), f"message, replay {step}"
        assert torch.equal(r_graph.view(torch.int32), r_ref.view(torch.int32)), f"residue, replay {step}"
        assert torch.equal(out_graph.view(torch.int32), out_ref.view(torch.int32)), f"decode, replay {step}"
        say(f"  replay {step}: {total} message bytes, identical")
    plan.close()


@pytest.mark.parametrize("name,launches", [("fc_lstm", 3), ("fc", 2)])
def test_one_plan_on_two_streams(name, launches):
    """Two learners compress with one shared plan on two streams at once (each
    with its own buffers), then decode on the two streams; results equal the
    same calls made one after the other (the 100x1000 table with the
    small-table finish, fc_lstm with the two-kernel one)."""
    wl = W.workload(name)
    plan = A.Plan(wl.segments)
    assert plan.info.compress_launches == launches
    n = W.alloc_len(wl)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    bufs = []
    for k in range(2):
        bufs.append(dict(r=torch.zeros(n, dtype=torch.float32, device=DEV),
                         d=W.make_dw(wl, k, 1, DEV), msg=plan.message_buffer(DEV),
                         ws=plan.compress_workspace(DEV), out=torch.empty(n, dtype=torch.float32, device=DEV),
                         dws=plan.decode_workspace(2, DEV)))
    ref = []
    for k in range(2):
        b = bufs[k]
        r = torch.zeros(n, dtype=torch.float32, device=DEV)
        m, w = plan.message_buffer(DEV), plan.compress_workspace(DEV)
        for step in range(3):
            A.compress(plan, r, b["d"], m, w)
        ref.append((r, m))
    torch.cuda.synchronize()
    for step in range(3):
        for k in range(2):
            b = bufs[k]
            A.compress(plan, b["r"], b["d"], b["msg"], b["ws"], stream=streams[k])
    for s in streams:
        s.synchronize()
    for k in range(2):
        total, _, _ = A.message_header(plan, ref[k][1])
        assert torch.equal(bufs[k]["msg"][:total], ref[k][1][:total])
        assert torch.equal(bufs[k]["r"].view(torch.int32), ref[k][0].view(torch.int32))
    msgs = [bufs[0]["msg"], bufs[1]["msg"]]
    for k in range(2):
        A.decode_accumulate(plan, msgs, bufs[k]["out"], False, bufs[k]["dws"], stream=streams[k])
    for s in streams:
        s.synchronize()
    assert torch.equal(bufs[0]["out"].view(torch.int32), bufs[1]["out"].view(torch.int32))
    plan.close()
