"""GPU parity of adacomp_decode_accumulate against the CPU oracle: bit-exact,
messages summed in order, for K = 1..16 messages, both accumulate modes,
edge-case tables, and messages whose header does not match the plan (the
full-size 1.07-billion-element workload: tests/test_gpu_large_full.py)."""
import sys

import numpy as np
import pytest
import torch

import adaptive_residual_gradient_amd as A
import msgparse as mp
import oracle
import workloads as W
from parity import bits

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def learner_messages(wl, plan, K, steps=2):
    """K learners, each `steps` compress steps from a zero residue with its
    own seeds; returns the device messages of the last step."""
    n = W.alloc_len(wl)
    ws = plan.compress_workspace(DEV)
    d = torch.empty(n, dtype=torch.float32, device=DEV)
    msgs = []
    for k in range(K):
        r = torch.zeros(n, dtype=torch.float32, device=DEV)
        msg = plan.message_buffer(DEV)
        for s in range(1, steps + 1):
            W.fill_dw(d, wl, k, s)
            A.compress(plan, r, d, msg, ws)
        total, _, _ = A.message_header(plan, msg)
        msgs.append(msg[:max(total, 16)].clone() if total < msg.numel() else msg)
    return msgs


def host(t):
    return t.cpu().numpy()


# flags: the default kernel choice, and plain sums forced onto the entry-record
# kernel (taken by default only by tables of at least 65536 tiles)
FLAGS = [0, A.PLAN_DECODE_RECORDS]


@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("name,K", [("fc", 1), ("fc", 3), ("conv", 4), ("resnet50", 16),
                                    ("fc_lstm", 2)])
def test_decode_parity(name, K, flags):
    wl = W.workload(name)
    plan = A.Plan(wl.segments, plan_flags=flags)
    n = W.alloc_len(wl)
    msgs = learner_messages(wl, plan, K)
    host_msgs = [host(m) for m in msgs]
    ws = plan.decode_workspace(K, DEV)
    rng = np.random.default_rng(K)
    for accumulate in (False, True):
        start = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        start[::5] = -0.0
        out = torch.from_numpy(start.copy()).to(DEV)
        say(f"  decode {name} K={K} accumulate={accumulate}")
        A.decode_accumulate(plan, msgs, out, accumulate, ws)
        got = host(out)
        want = start.copy()
        oracle.decode_accumulate(wl.segments, host_msgs, want, accumulate)
        np.testing.assert_array_equal(bits(got), bits(want))
        assert int(host(ws[:4]).view(np.uint32)[0]) == 0
    plan.close()


@pytest.mark.parametrize("flags", FLAGS)
def test_decode_dense_many_tiles(flags):
    """One layer of 2^28 elements at L_T = 50: 66281 decode tiles of 81 bins
    with 8-bit words, past the tile count from which the decode count reads a
    tile's count blocks together; three learners' second-step messages, both
    accumulate modes, compared in full with the oracle."""
    n = 1 << 28
    segs = [(0, n, 50)]
    plan = A.Plan(segs, plan_flags=flags)
    msg_ws = plan.compress_workspace(DEV)
    d = torch.empty(n, dtype=torch.float32, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(50)
    msgs = []
    for k in range(3):
        r = torch.zeros(n, dtype=torch.float32, device=DEV)
        msg = plan.message_buffer(DEV)
        for _ in range(2):
            d.normal_(0.0, 1e-3, generator=gen)
            A.compress(plan, r, d, msg, msg_ws)
        total, surv, _ = A.message_header(plan, msg)
        say(f"  learner {k}: {surv} survivors, {total} bytes")
        msgs.append(msg[:total].clone())
        del r, msg
    del d, msg_ws
    torch.cuda.empty_cache()
    host_msgs = [host(m) for m in msgs]
    ws = plan.decode_workspace(len(msgs), DEV)
    for accumulate in (False, True):
        start = np.full(n, 0.5, np.float32)
        start[::7] = -0.0
        out = torch.from_numpy(start).to(DEV)
        say(f"  decode 2^28 elements at L_T 50, accumulate={accumulate}")
        A.decode_accumulate(plan, msgs, out, accumulate, ws)
        got = host(out)
        del out
        oracle.decode_accumulate(segs, host_msgs, start, accumulate)
        np.testing.assert_array_equal(bits(got), bits(start))
        assert int(host(ws[:4]).view(np.uint32)[0]) == 0
        del got, start
    plan.close()
    del msgs, ws
    torch.cuda.empty_cache()


@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("lt", [1, 3, 7, 50, 64, 500, 1021, 4093, 4094, 9000, 18432, 18433, 32768])
def test_decode_edge_tables(lt, flags):
    """Every decode tile shape: LDS tiles (L_T <= 4093), long bins with at
    least two bins per tile accumulated in LDS (4094 .. 18432) and one bin
    per tile accumulated in place (18433 and up); ragged and one-element
    layers; accumulate from zero and from a random start."""
    segs, off = [], 0
    for n in (1, 5, 63, 4097, 40003):
        segs.append((off, n, lt))
        off += (n + 3) // 4 * 4 + 4
    span = off
    plan = A.Plan(segs, plan_flags=flags)
    rng = np.random.default_rng(lt)
    cws = plan.compress_workspace(DEV)
    msgs = []
    for k in range(3):
        r = torch.from_numpy((rng.standard_normal(span) * 1e-3).astype(np.float32)).to(DEV)
        d = torch.from_numpy((rng.standard_normal(span) * 1e-3).astype(np.float32)).to(DEV)
        m = plan.message_buffer(DEV)
        A.compress(plan, r, d, m, cws)
        msgs.append(m)
    host_msgs = []
    for m in msgs:
        total, _, _ = A.message_header(plan, m)
        host_msgs.append(host(m[:total]))
    ws = plan.decode_workspace(3, DEV)
    for accumulate in (False, True):
        start = rng.standard_normal(span).astype(np.float32)
        out = torch.from_numpy(start.copy()).to(DEV)
        say(f"  decode L_T={lt} accumulate={accumulate}")
        A.decode_accumulate(plan, msgs, out, accumulate, ws)
        want = start.copy()
        oracle.decode_accumulate(segs, host_msgs, want, accumulate)
        np.testing.assert_array_equal(bits(host(out)), bits(want))
    plan.close()


@pytest.mark.parametrize("K,dense", [(2, True), (3, True), (16, False), (5, "mixed")])
def test_decode_bin_table_limits(K, dense):
    """Plain decodes of a small table of 8-bit words (L_T 50), where entry
    bins come from the LDS bin-start table when a tile's runs fit it: every
    element sent by every message (all values of a bin equal in magnitude),
    with K = 2 (runs of 8100 words per tile: inside the table) and K = 3
    (12150: past it, so the tiles take the prefix search); sparse messages;
    and a mix of both, in both accumulate modes."""
    segs = [(0, 1000050, 50), (1000052, 123457, 50)]
    span = 1000052 + 123460
    plan = A.Plan(segs)
    rng = np.random.default_rng(1000 + K)
    cws = plan.compress_workspace(DEV)
    msgs, host_msgs = [], []
    for k in range(K):
        full = dense is True or (dense == "mixed" and k % 2 == 0)
        if full:   # r = 0, |dW| equal: |H| = 2|dW| >= g_max = |dW| everywhere
            d = (np.where(rng.random(span) < 0.5, -1.0, 1.0) * 1e-3).astype(np.float32)
        else:
            d = (rng.standard_normal(span) * 1e-3).astype(np.float32)
        r = torch.zeros(span, dtype=torch.float32, device=DEV)
        m = plan.message_buffer(DEV)
        A.compress(plan, r, torch.from_numpy(d).to(DEV), m, cws)
        total, surv, _ = A.message_header(plan, m)
        if full:
            assert surv == 1000050 + 123457
        msgs.append(m)
        host_msgs.append(host(m[:total]))
    ws = plan.decode_workspace(K, DEV)
    for accumulate in (False, True):
        start = rng.standard_normal(span).astype(np.float32)
        out = torch.from_numpy(start.copy()).to(DEV)
        say(f"  decode K={K} dense={dense} accumulate={accumulate}")
        A.decode_accumulate(plan, msgs, out, accumulate, ws)
        want = start.copy()
        oracle.decode_accumulate(segs, host_msgs, want, accumulate)
        np.testing.assert_array_equal(bits(host(out)), bits(want))
    plan.close()


@pytest.mark.parametrize("flags", FLAGS)
def test_decode_skips_foreign_messages(flags):
    """A message made for another segment table contributes nothing and is
    counted in the status word."""
    segs = [(0, 5000, 50)]
    other = [(0, 5000, 500)]
    plan, plan2 = A.Plan(segs, plan_flags=flags), A.Plan(other)
    r = torch.zeros(5000, dtype=torch.float32, device=DEV)
    d = torch.from_numpy((np.random.default_rng(0).standard_normal(5000) * 1e-3)
                         .astype(np.float32)).to(DEV)
    m1, m2 = plan.message_buffer(DEV), plan2.message_buffer(DEV)
    A.compress(plan, r.clone(), d, m1, plan.compress_workspace(DEV))
    A.compress(plan2, r.clone(), d, m2, plan2.compress_workspace(DEV))
    ws = plan.decode_workspace(2, DEV)
    out = torch.zeros(5000, dtype=torch.float32, device=DEV)
    A.decode_accumulate(plan, [m1, m2], out, False, ws)
    ref = torch.zeros(5000, dtype=torch.float32, device=DEV)
    A.decode_accumulate(plan, [m1], ref, False, plan.decode_workspace(1, DEV))
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
    assert int(host(ws[:4]).view(np.uint32)[0]) == 1
    plan.close()
    plan2.close()


def _put(buf, at, dtype, value):
    n = np.dtype(dtype).itemsize
    buf[at:at + n] = np.frombuffer(np.array(value, dtype).tobytes(), np.uint8)


def _get(buf, at, dtype):
    return np.frombuffer(buf[at:at + np.dtype(dtype).itemsize].tobytes(), dtype)[0]


@pytest.mark.parametrize("flags", FLAGS)
def test_decode_rejects_inconsistent_messages(flags):
    """Messages whose header matches the plan but whose body is inconsistent,
    every offset still inside the buffer, are refused one by one: the others
    are summed as the oracle sums them alone, and the refused ones are
    counted in the status word, for the plain sum, the accumulate mode and
    the fused SGD step.  Corruptions: a directory survivor count one too
    high; one count word one too high; an entry offset off its 16-byte
    alignment; a total length past the plan's capacity."""
    segs = [(0, 6000, 50), (6000, 9000, 500)]
    wl_n = 15000
    plan = A.Plan(segs, plan_flags=flags)
    ws_c = plan.compress_workspace(DEV)
    rng = np.random.default_rng(77)
    good = []
    for k in range(6):
        r = torch.zeros(wl_n, dtype=torch.float32, device=DEV)
        d = torch.from_numpy((rng.standard_normal(wl_n) * 1e-3).astype(np.float32)).to(DEV)
        msg = plan.message_buffer(DEV)
        A.compress(plan, r, d, msg, ws_c)
        good.append(host(msg).copy())
    info = plan.info
    cap = int(info.message_capacity)
    bad = [m.copy() for m in good]
    _put(bad[1], 32 + 16 + 4, np.uint32, _get(bad[1], 32 + 16 + 4, np.uint32) + 1)
    cnt0 = ((32 + 16 * 2) + 15) // 16 * 16          # first count word of segment 0 (8-bit)
    bad[2][cnt0] += 1
    _put(bad[3], 32 + 8, np.uint64, _get(bad[3], 32 + 8, np.uint64) + 8)
    _put(bad[4], 16, np.uint64, cap + 16)
    dev = [torch.from_numpy(m).to(DEV) for m in bad]
    keep = [bad[0][:int(_get(bad[0], 16, np.uint64))], bad[5][:int(_get(bad[5], 16, np.uint64))]]
    for m in bad[1:3]:          # the oracle refuses the two count mismatches as well
        with pytest.raises(oracle.OracleError):
            oracle.decode_accumulate(segs, [m], np.zeros(wl_n, np.float32), False)

    ws = plan.decode_workspace(6, DEV)
    out = torch.full((wl_n,), 3.0, dtype=torch.float32, device=DEV)
    A.decode_accumulate(plan, dev, out, False, ws)
    torch.cuda.synchronize()
    assert int(host(ws[:4]).view(np.uint32)[0]) == 4
    want = np.zeros(wl_n, np.float32)
    oracle.decode_accumulate(segs, keep, want, False)
    np.testing.assert_array_equal(bits(host(out)), bits(want))

    start = (rng.standard_normal(wl_n) * 1e-2).astype(np.float32)
    out = torch.from_numpy(start.copy()).to(DEV)
    A.decode_accumulate(plan, dev, out, True, ws)
    torch.cuda.synchronize()
    assert int(host(ws[:4]).view(np.uint32)[0]) == 4
    want = start.copy()
    oracle.decode_accumulate(segs, keep, want, True)
    np.testing.assert_array_equal(bits(host(out)), bits(want))

    w0 = (rng.standard_normal(wl_n) * 0.05).astype(np.float32)
    m0 = (rng.standard_normal(wl_n) * 1e-3).astype(np.float32)
    w, m = torch.from_numpy(w0.copy()).to(DEV), torch.from_numpy(m0.copy()).to(DEV)
    ws2 = plan.decode_sgd_workspace(6, DEV)
    A.decode_sgd(plan, dev, w, m, 0.01, 0.9, ws2, weight_decay=1e-4, scale=0.5)
    torch.cuda.synchronize()
    assert int(host(ws2[:4]).view(np.uint32)[0]) == 4
    w_ref, m_ref = w0.copy(), m0.copy()
    oracle.decode_sgd(segs, keep, w_ref, m_ref, 0.01, 0.9, weight_decay=1e-4, scale=0.5)
    np.testing.assert_array_equal(bits(host(w)), bits(w_ref))
    np.testing.assert_array_equal(bits(host(m)), bits(m_ref))
    plan.close()


@pytest.mark.parametrize("K,lt", [(70, 50), (256, 500), (20, 1)])
def test_decode_many_messages(K, lt):
    """Message groups: more messages than one group holds (64 at most, fewer
    when the bin prefixes of a tile are long), up to the 256-message limit."""
    segs = [(0, 3001, lt), (3004, 517, lt)]
    span = 3524
    plan = A.Plan(segs)
    rng = np.random.default_rng(K + lt)
    cws = plan.compress_workspace(DEV)
    msgs, host_msgs = [], []
    for k in range(K):
        r = torch.from_numpy((rng.standard_normal(span) * 1e-3).astype(np.float32)).to(DEV)
        d = torch.from_numpy((rng.standard_normal(span) * 1e-3 * (1 + k % 3)).astype(np.float32)).to(DEV)
        m = plan.message_buffer(DEV)
        A.compress(plan, r, d, m, cws)
        total, _, _ = A.message_header(plan, m)
        msgs.append(m[:total].clone())
        host_msgs.append(host(msgs[-1]))
    ws = plan.decode_workspace(K, DEV)
    start = rng.standard_normal(span).astype(np.float32)
    out = torch.from_numpy(start.copy()).to(DEV)
    say(f"  decode K={K} L_T={lt}")
    A.decode_accumulate(plan, msgs, out, True, ws)
    want = start.copy()
    oracle.decode_accumulate(segs, host_msgs, want, True)
    np.testing.assert_array_equal(bits(host(out)), bits(want))
    plan.close()


def test_decode_rejects_too_many_messages():
    segs = [(0, 100, 50)]
    plan = A.Plan(segs)
    m = plan.message_buffer(DEV)
    out = torch.zeros(100, dtype=torch.float32, device=DEV)
    with pytest.raises(A.AdaCompError) as e:
        A.decode_accumulate(plan, [m] * 257, out, False, plan.decode_workspace(257, DEV))
    assert e.value.status == -1
    with pytest.raises(A.AdaCompError) as e:
        A.decode_accumulate(plan, [m], out, False, plan.decode_workspace(1, DEV)[:16])
    assert e.value.status == -5
    plan.close()


# --------------------------------------------------------------------------
# decode fused with one SGD-with-momentum step
# --------------------------------------------------------------------------

def _sgd_check(plan, segs, msgs, host_msgs, w_host, m_host, lr, mu, wd, scale, steps=3):
    """Run `steps` fused steps on the GPU and the oracle from the same w, m;
    compare bit for bit after each step (the oracle consumes its own state,
    which stays equal to the GPU's while they agree)."""
    K = len(msgs)
    ws = plan.decode_sgd_workspace(K, DEV)
    w_dev = torch.from_numpy(w_host.copy()).to(DEV)
    m_dev = torch.from_numpy(m_host.copy()).to(DEV)
    w_ref, m_ref = w_host.copy(), m_host.copy()
    for step in range(steps):
        A.decode_sgd(plan, msgs, w_dev, m_dev, lr, mu, ws, weight_decay=wd, scale=scale)
        oracle.decode_sgd(segs, host_msgs, w_ref, m_ref, lr, mu, wd, scale)
        np.testing.assert_array_equal(bits(host(m_dev)), bits(m_ref), err_msg=f"momentum, step {step}")
        np.testing.assert_array_equal(bits(host(w_dev)), bits(w_ref), err_msg=f"weights, step {step}")
    assert int(host(ws[:4]).view(np.uint32)[0]) == 0


@pytest.mark.parametrize("name,K,wd", [("fc", 2, 0.0), ("conv", 4, 1e-4), ("resnet50", 16, 5e-4),
                                       ("fc_lstm", 3, 0.0)])
def test_decode_sgd_parity(name, K, wd):
    wl = W.workload(name)
    plan = A.Plan(wl.segments)
    n = W.alloc_len(wl)
    msgs = learner_messages(wl, plan, K)
    host_msgs = [host(m) for m in msgs]
    rng = np.random.default_rng(K)
    w = (rng.standard_normal(n) * 0.05).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    say(f"  decode+SGD {name} K={K} wd={wd}")
    _sgd_check(plan, wl.segments, msgs, host_msgs, w, m, 0.01, 0.9, wd, 1.0 / K)
    plan.close()


@pytest.mark.parametrize("lt", [1, 7, 50, 500, 4093, 4094, 32768])
def test_decode_sgd_edge_tables(lt):
    """Every bin-length class, including bins longer than 4093 (summed in the
    workspace scratch, then stepped), ragged sizes and gaps between layers
    (never written)."""
    segs, off = [], 4
    for n in (1, 5, 63, 4097, 40003):
        segs.append((off, n, lt))
        off += (n + 3) // 4 * 4 + 8
    span = off + 4
    plan = A.Plan(segs)
    rng = np.random.default_rng(lt + 1)
    cws = plan.compress_workspace(DEV)
    msgs, host_msgs = [], []
    for k in range(3):
        r = torch.from_numpy((rng.standard_normal(span) * 1e-3).astype(np.float32)).to(DEV)
        d = torch.from_numpy((rng.standard_normal(span) * 1e-3).astype(np.float32)).to(DEV)
        mm = plan.message_buffer(DEV)
        A.compress(plan, r, d, mm, cws)
        total, _, _ = A.message_header(plan, mm)
        msgs.append(mm[:total].clone())
        host_msgs.append(host(msgs[-1]))
    w = rng.standard_normal(span).astype(np.float32)
    m = (rng.standard_normal(span) * 1e-2).astype(np.float32)
    say(f"  decode+SGD L_T={lt}")
    _sgd_check(plan, segs, msgs, host_msgs, w, m, 0.05, 0.5, 1e-3, 1.0 / 3.0)
    plan.close()


def test_decode_sgd_argument_errors():
    segs = [(0, 100, 50)]
    plan = A.Plan(segs)
    mm = plan.message_buffer(DEV)
    w = torch.zeros(100, dtype=torch.float32, device=DEV)
    m = torch.zeros(100, dtype=torch.float32, device=DEV)
    ws = plan.decode_sgd_workspace(1, DEV)
    with pytest.raises(A.AdaCompError) as e:
        A.decode_sgd(plan, [mm], w, m, 0.1, 0.9, ws[:16])
    assert e.value.status == -5
    with pytest.raises(A.AdaCompError) as e:
        A.decode_sgd(plan, [mm], w, w, 0.1, 0.9, ws)
    assert e.value.status == -1
    with pytest.raises(A.AdaCompError) as e:
        A.decode_sgd(plan, [mm], w[1:], m[1:], 0.1, 0.9, ws)
    assert e.value.status == -3
    plan.close()


# --------------------------------------------------------------------------
# decode fused with one Adam step
# --------------------------------------------------------------------------

def _adam_check(plan, segs, msgs, host_msgs, w_host, m_host, v_host, lr, b1, b2, eps, wd, scale,
                steps=3):
    K = len(msgs)
    ws = plan.decode_sgd_workspace(K, DEV)
    dev = [torch.from_numpy(a.copy()).to(DEV) for a in (w_host, m_host, v_host)]
    ref = [a.copy() for a in (w_host, m_host, v_host)]
    for t in range(1, steps + 1):
        A.decode_adam(plan, msgs, dev[0], dev[1], dev[2], lr, b1, b2, eps, t, ws,
                      weight_decay=wd, scale=scale)
        oracle.decode_adam(segs, host_msgs, ref[0], ref[1], ref[2], lr, b1, b2, eps, t, wd, scale)
        for name, d, r in zip(("weights", "m", "v"), dev, ref):
            np.testing.assert_array_equal(bits(host(d)), bits(r), err_msg=f"{name}, step {t}")


@pytest.mark.parametrize("name,K,wd", [("fc", 2, 0.0), ("conv", 4, 1e-4), ("resnet50", 16, 1e-2),
                                       ("fc_lstm", 3, 0.0)])
def test_decode_adam_parity(name, K, wd):
    wl = W.workload(name)
    plan = A.Plan(wl.segments)
    n = W.alloc_len(wl)
    msgs = learner_messages(wl, plan, K)
    host_msgs = [host(x) for x in msgs]
    rng = np.random.default_rng(K + 100)
    w = (rng.standard_normal(n) * 0.05).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = (rng.random(n) * 1e-7).astype(np.float32)
    say(f"  decode+Adam {name} K={K} wd={wd}")
    _adam_check(plan, wl.segments, msgs, host_msgs, w, m, v, 1e-3, 0.9, 0.999, 1e-8, wd, 1.0 / K)
    plan.close()


@pytest.mark.parametrize("lt", [1, 50, 4093, 4094, 32768])
def test_decode_adam_edge_tables(lt):
    segs, off = [], 4
    for n in (1, 5, 63, 4097, 40003):
        segs.append((off, n, lt))
        off += (n + 3) // 4 * 4 + 8
    span = off + 4
    plan = A.Plan(segs)
    rng = np.random.default_rng(lt + 7)
    cws = plan.compress_workspace(DEV)
    msgs, host_msgs = [], []
    for k in range(2):
        r = torch.from_numpy((rng.standard_normal(span) * 1e-3).astype(np.float32)).to(DEV)
        d = torch.from_numpy((rng.standard_normal(span) * 1e-3).astype(np.float32)).to(DEV)
        mm = plan.message_buffer(DEV)
        A.compress(plan, r, d, mm, cws)
        total, _, _ = A.message_header(plan, mm)
        msgs.append(mm[:total].clone())
        host_msgs.append(host(msgs[-1]))
    w = rng.standard_normal(span).astype(np.float32)
    m = np.zeros(span, np.float32)
    v = np.zeros(span, np.float32)
    say(f"  decode+Adam L_T={lt}")
    _adam_check(plan, segs, msgs, host_msgs, w, m, v, 1e-2, 0.9, 0.99, 1e-6, 0.0, 0.5)
    plan.close()


def test_decode_adam_argument_errors():
    plan = A.Plan([(0, 100, 50)])
    mm = plan.message_buffer(DEV)
    w, m, v = (torch.zeros(100, dtype=torch.float32, device=DEV) for _ in range(3))
    ws = plan.decode_sgd_workspace(1, DEV)
    with pytest.raises(A.AdaCompError) as e:
        A.decode_adam(plan, [mm], w, m, v, 1e-3, 0.9, 0.999, 1e-8, 0, ws)
    assert e.value.status == -1
    with pytest.raises(A.AdaCompError) as e:
        A.decode_adam(plan, [mm], w, m, m, 1e-3, 0.9, 0.999, 1e-8, 1, ws)
    assert e.value.status == -1
    plan.close()
