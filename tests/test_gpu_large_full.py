"""The 1.07-billion-element workload (64 layers of 4096 x 4096, L_T = 500,
bursty N(0, 1e-3) gradients) at full size, in the launch configuration the
benchmark times, against the oracle on every layer:

  - compress: learner 0's ten steps from zero residue, step-locked (the
    oracle consumes the GPU's residue each step); every bin maximum, every
    layer's count words, entry words, s and survivor count, and the residue
    of every element, each step;
  - decode: the step-10 messages of 16 learners (own seeds each) summed by
    one K = 16 call, fused with one SGD step, and fused with one Adam step;
    every element of every layer bit for bit.

The oracle runs layer by layer (layers are independent: one s per layer, bins
never cross layers) on a pool of host threads; the GPU message is cut into
one-layer messages for it.  Tolerances are those of tests/parity.py."""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

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
STEPS = 10
K = 16
THREADS = max(1, min(16, os.cpu_count() or 1))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    return t.cpu().numpy()


def bin_offsets(segments):
    out, b = [], 0
    for (_, c, lt) in segments:
        out.append(b)
        b += (c + lt - 1) // lt
    return out


def test_large_compress_all_layers_ten_steps():
    wl = W.workload("large")
    segs = wl.segments
    plan = A.Plan(segs)
    n = W.alloc_len(wl)
    r_dev = torch.zeros(n, dtype=torch.float32, device=DEV)
    d_dev = torch.empty(n, dtype=torch.float32, device=DEV)
    msg, ws = plan.message_buffer(DEV), plan.compress_workspace(DEV)
    gmax = torch.empty(int(plan.info.total_bins), dtype=torch.float32, device=DEV)
    b0 = bin_offsets(segs)
    s_exact = 0
    with ThreadPoolExecutor(max_workers=THREADS) as pool:
        for step in range(1, STEPS + 1):
            W.fill_dw(d_dev, wl, 0, step)
            r_in = host(r_dev)
            d = host(d_dev)
            A.compress(plan, r_dev, d_dev, msg, ws, bin_max_out=gmax)
            torch.cuda.synchronize()
            total, surv, _ = A.message_header(plan, msg)
            m = host(msg[:total])
            pm = mp.parse(m, segs)   # strict structure check of the whole message
            assert pm.total_survivors == surv
            r_out = host(r_dev)
            g_all = host(gmax)

            def layer(i):
                o, c, lt = segs[i]
                g = g_all[b0[i]:b0[i] + (c + lt - 1) // lt]
                return compare_step([(0, c, lt)], r_in[o:o + c], d[o:o + c], r_out[o:o + c],
                                    mp.single_segment_message(m, segs, i), g)

            reps = list(pool.map(layer, range(len(segs))))
            s_exact += sum(r.s_exact for r in reps)
            say(f"  step {step}: {surv} survivors, {total} bytes, all {len(segs)} layers match")
            del r_in, d, r_out
    say(f"  s bit-exact on {s_exact} of {STEPS * len(segs)} layer-steps")
    plan.close()
    del r_dev, d_dev, msg, ws, gmax
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def learner_messages():
    """The step-10 messages of learners 0..15 (each from zero residue with its
    own seeds), on the device and on the host."""
    wl = W.workload("large")
    plan = A.Plan(wl.segments)
    n = W.alloc_len(wl)
    ws = plan.compress_workspace(DEV)
    d = torch.empty(n, dtype=torch.float32, device=DEV)
    r = torch.empty(n, dtype=torch.float32, device=DEV)
    msg = plan.message_buffer(DEV)
    dev_msgs, host_msgs = [], []
    say("  building 16 learner messages at full size (10 steps each)")
    for k in range(K):
        r.zero_()
        for s in range(1, STEPS + 1):
            W.fill_dw(d, wl, k, s)
            A.compress(plan, r, d, msg, ws)
        total, _, _ = A.message_header(plan, msg)
        dev_msgs.append(msg[:total].clone())
        host_msgs.append(host(dev_msgs[-1]))
    del d, r, msg, ws
    torch.cuda.empty_cache()
    yield wl, plan, dev_msgs, host_msgs
    plan.close()
    del dev_msgs
    torch.cuda.empty_cache()


def per_layer(segs, host_msgs):
    """Each learner's message cut into one-layer messages, per layer."""
    return [[mp.single_segment_message(hm, segs, i) for hm in host_msgs] for i in range(len(segs))]


def test_large_decode_all_layers(learner_messages):
    wl, plan, dev_msgs, host_msgs = learner_messages
    segs = wl.segments
    n = W.alloc_len(wl)
    out = torch.empty(n, dtype=torch.float32, device=DEV)
    ws = plan.decode_workspace(K, DEV)
    say("  decode K=16 full size")
    A.decode_accumulate(plan, dev_msgs, out, False, ws)
    torch.cuda.synchronize()
    assert int(host(ws[:4]).view(np.uint32)[0]) == 0
    got = host(out)
    subs = per_layer(segs, host_msgs)

    def layer(i):
        o, c, lt = segs[i]
        want = np.zeros(c, np.float32)
        oracle.decode_accumulate([(0, c, lt)], subs[i], want, False)
        np.testing.assert_array_equal(bits(got[o:o + c]), bits(want), err_msg=f"layer {i}")
        return int(np.count_nonzero(want))

    with ThreadPoolExecutor(max_workers=THREADS) as pool:
        nz = sum(pool.map(layer, range(len(segs))))
    say(f"  all {len(segs)} layers bit-exact; {nz} elements received a sum")
    del out, ws
    torch.cuda.empty_cache()


def test_large_decode_sgd_all_layers(learner_messages):
    wl, plan, dev_msgs, host_msgs = learner_messages
    segs = wl.segments
    n = W.alloc_len(wl)
    w = torch.empty(n, dtype=torch.float32, device=DEV)
    w.normal_(0.0, 0.05, generator=torch.Generator(device=DEV).manual_seed(5))
    m = torch.empty(n, dtype=torch.float32, device=DEV)
    m.normal_(0.0, 1e-3, generator=torch.Generator(device=DEV).manual_seed(6))
    w0, m0 = host(w), host(m)
    ws = plan.decode_sgd_workspace(K, DEV)
    lr, mu, wd, scale = 0.01, 0.9, 1e-4, 1.0 / K
    say("  decode+SGD K=16 full size")
    A.decode_sgd(plan, dev_msgs, w, m, lr, mu, ws, weight_decay=wd, scale=scale)
    torch.cuda.synchronize()
    w1, m1 = host(w), host(m)
    subs = per_layer(segs, host_msgs)

    def layer(i):
        o, c, lt = segs[i]
        w_ref, m_ref = w0[o:o + c].copy(), m0[o:o + c].copy()
        oracle.decode_sgd([(0, c, lt)], subs[i], w_ref, m_ref, lr, mu, weight_decay=wd, scale=scale)
        np.testing.assert_array_equal(bits(w1[o:o + c]), bits(w_ref), err_msg=f"layer {i} weights")
        np.testing.assert_array_equal(bits(m1[o:o + c]), bits(m_ref), err_msg=f"layer {i} momentum")

    with ThreadPoolExecutor(max_workers=THREADS) as pool:
        list(pool.map(layer, range(len(segs))))
    say(f"  all {len(segs)} layers bit-exact")
    del w, m, ws
    torch.cuda.empty_cache()


def test_large_decode_adam_all_layers(learner_messages):
    wl, plan, dev_msgs, host_msgs = learner_messages
    segs = wl.segments
    n = W.alloc_len(wl)
    w = torch.empty(n, dtype=torch.float32, device=DEV)
    w.normal_(0.0, 0.05, generator=torch.Generator(device=DEV).manual_seed(7))
    m = torch.empty(n, dtype=torch.float32, device=DEV)
    m.normal_(0.0, 1e-3, generator=torch.Generator(device=DEV).manual_seed(8))
    v = torch.empty(n, dtype=torch.float32, device=DEV)
    v.uniform_(0.0, 1e-6, generator=torch.Generator(device=DEV).manual_seed(9))
    w0, m0, v0 = host(w), host(m), host(v)
    ws = plan.decode_sgd_workspace(K, DEV)
    lr, b1, b2, eps, wd, scale, step = 1e-3, 0.9, 0.999, 1e-8, 0.0, 1.0 / K, 3
    say("  decode+Adam K=16 full size")
    A.decode_adam(plan, dev_msgs, w, m, v, lr, b1, b2, eps, step, ws, weight_decay=wd, scale=scale)
    torch.cuda.synchronize()
    w1, m1, v1 = host(w), host(m), host(v)
    subs = per_layer(segs, host_msgs)

    def layer(i):
        o, c, lt = segs[i]
        w_ref, m_ref, v_ref = w0[o:o + c].copy(), m0[o:o + c].copy(), v0[o:o + c].copy()
        oracle.decode_adam([(0, c, lt)], subs[i], w_ref, m_ref, v_ref, lr, b1, b2, eps, step,
                           weight_decay=wd, scale=scale)
        np.testing.assert_array_equal(bits(w1[o:o + c]), bits(w_ref), err_msg=f"layer {i} weights")
        np.testing.assert_array_equal(bits(m1[o:o + c]), bits(m_ref), err_msg=f"layer {i} m")
        np.testing.assert_array_equal(bits(v1[o:o + c]), bits(v_ref), err_msg=f"layer {i} v")

    with ThreadPoolExecutor(max_workers=THREADS) as pool:
        list(pool.map(layer, range(len(segs))))
    say(f"  all {len(segs)} layers bit-exact")
    del w, m, v, ws
    torch.cuda.empty_cache()
