"""Benchmark of the AdaComp hot path on one MI355X.

One step = one adacomp_compress of a learner's full gradient (the
1.07-billion-element workload: 64 layers of 4096 x 4096, L_T = 500, 16-bit
words, bursty N(0, 1e-3) gradients with 5% of bins scaled x100) followed by
one adacomp_decode_accumulate of K = 16 learners' messages into a dense float32
sum.  Every input is generated on the device before the timed region; the
residue carries over from step to step.  The step sequence first runs once
untimed from zero residue (its messages kept), then again from zero residue:
warm-up steps, then the timed steps, each call after a 1 GiB scratch read
that evicts the 256 MB last-level cache (a read leaves no dirty lines to
write back inside the timed call) and timed with device events; every
message of the rerun must equal the first run's byte for byte.

Printed: one JSON line.  ``value`` is compress throughput in Gelem/s (device
time of the compress calls inside the timed steps); ``roofline`` rates the
dominant kernel (the dense tile pass) against MI355X's 8 TB/s HBM peak;
``cpu_baseline`` is the plain C oracle timed on this host's cores on a sample
of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import pathlib
import statistics
import sys
import time

ROOT = pathlib.Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBPS = 8000.0
METRIC = "AdaComp compress Gelem/s & % of HBM roofline; compression ratio; decode GB/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# The sources the dense tile pass is built from (its HBM counters stay valid
# while these are unchanged).
TILE_PASS_SOURCES = ("layout.hpp", "common.hpp", "tile_pass.hpp")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in TILE_PASS_SOURCES:
        h.update((ROOT / "adaptive_residual_gradient_amd" / "csrc" / name).read_bytes())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str):
    """HBM bytes per tile-pass launch measured with rocprofv3 counters, if the
    kernel sources have not changed since they were taken."""
    p = ROOT / "profiles" / f"tile_pass_{workload}_traffic.json"
    if not p.exists():
        return None
    try:
        rec = json.loads(p.read_text())
    except ValueError:
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(wl, dws_host_fn, max_steps: int, seconds: float = 15.0):
    """Time the oracle on whole layers of the workload, as it stands: single
    threaded, and with one call per layer on a pool of host threads (the
    oracle call releases the interpreter lock, so layers run on separate
    cores; at most 16 threads, the host share of one GPU)."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    segs = wl.segments
    take = min(24, len(segs))
    sub, off = [], 0
    for (_, n, lt) in segs[:take]:
        sub.append((off, n, lt))
        off += (n + 3) // 4 * 4
    per_layer = [[(0, n, lt)] for (_, n, lt) in sub]
    elems_per_step = sum(n for _, n, _ in sub)

    def run(threads):
        r = np.zeros(off, np.float32)
        steps, t_used = 0, 0.0
        pool = ThreadPoolExecutor(max_workers=threads) if threads > 1 else None
        while t_used < seconds / 2 and steps < max_steps:
            d = dws_host_fn(steps, off)
            t0 = time.perf_counter()
            if pool is None:
                oracle.compress(sub, r, d)
            else:
                views = [(r[o:o + n], d[o:o + n]) for (o, n, _) in sub]
                list(pool.map(lambda i: oracle.compress(per_layer[i], views[i][0], views[i][1]),
                              range(len(sub))))
            t_used += time.perf_counter() - t0
            steps += 1
        if pool is not None:
            pool.shutdown()
        return steps, t_used

    threads = max(1, min(16, os.cpu_count() or 1, take))
    s1, t1 = run(1)
    sn, tn = run(threads) if threads > 1 else (s1, t1)
    v1, vn = s1 * elems_per_step / t1 / 1e9, sn * elems_per_step / tn / 1e9
    best, cores = (vn, threads) if vn > v1 else (v1, 1)   # whichever the host does faster
    return {
        "value": round(best, 4),
        "unit": "Gelem/s",
        "cores": cores,
        "threads": threads,
        "host_cores": os.cpu_count(),
        "kind": "oracle",
        "single_thread_value": round(v1, 4),
        "threaded_value": round(vn, 4),
        "sample": f"{take} of {len(segs)} layers ({elems_per_step} elements), compress steps from zero "
                  f"residue on the benchmark's own gradients: {sn} steps in {tn:.1f} s with one layer "
                  f"per thread on {threads} threads; single-threaded {s1} steps in {t1:.1f} s",
    }


def measure_copy(dev, reps: int = 5) -> dict:
    """Device-to-device copies of 1 GiB (read + write 2 GiB per copy), GB/s,
    two ways: the runtime's copy (`copy_`) and an elementwise kernel
    (`mul(src, 1, out=dst)`).  The faster is the practical streaming
    ceiling, a second denominator beside the HBM peak."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    fns = {"copy_": lambda: dst.copy_(src), "elementwise": lambda: torch.mul(src, 1.0, out=dst)}
    res = {}
    for name, fn in fns.items():
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        res[name] = 2.0 * (1 << 30) / (a.elapsed_time(b) / reps * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return res


def measure_decode_sgd(A, plan, msgs, n_alloc, N, K, dev):
    """After the timed steps: decode fused with one SGD-with-momentum step
    (reads and writes weights and momentum, 16 B/element + messages) against
    decode_accumulate followed by the same step as separate torch operations
    (which also write and re-read the sum: 24 B/element + messages), and
    decode fused with one Adam step (24 B/element + messages)."""
    import torch
    w = torch.zeros(n_alloc, dtype=torch.float32, device=dev)
    m = torch.zeros(n_alloc, dtype=torch.float32, device=dev)
    out = torch.empty(n_alloc, dtype=torch.float32, device=dev)
    ws = plan.decode_sgd_workspace(K, dev)
    lr, mu, scale = 0.01, 0.9, 1.0 / K

    def fused():
        A.decode_sgd(plan, msgs, w, m, lr, mu, ws, scale=scale)

    def unfused():
        A.decode_accumulate(plan, msgs, out, False, ws)
        m.mul_(mu).add_(out, alpha=scale)
        w.add_(m, alpha=-lr)

    def time_it(fn, reps=6):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    v = torch.zeros(n_alloc, dtype=torch.float32, device=dev)
    step = [0]

    def adam():
        step[0] += 1
        A.decode_adam(plan, msgs, w, m, v, 1e-3, 0.9, 0.999, 1e-8, step[0], ws, scale=scale)

    t_f, t_u, t_a = time_it(fused), time_it(unfused), time_it(adam)
    mbytes = float(sum(x.numel() for x in msgs))
    del w, m, v, out, ws
    torch.cuda.empty_cache()
    return {"messages": K, "fused_ms": round(t_f, 4),
            "fused_GBps": round((mbytes + 16.0 * N) / (t_f * 1e-3) / 1e9, 1),
            "decode_then_torch_sgd_ms": round(t_u, 4),
            "fused_adam_ms": round(t_a, 4),
            "fused_adam_GBps": round((mbytes + 24.0 * N) / (t_a * 1e-3) / 1e9, 1)}


def measure_small_table(A, W, dev):
    """The 100 x 1000 layer (L_T 500), launch-latency bound: one compress call
    per step over its 10 seeded gradients, timed per call with events
    (median of 100 calls), back to back (mean of 500) and replayed from a HIP
    graph of the 10 calls (mean of 20 replays), for each finish:
    the default small-table finish (tile pass + one finish kernel), the
    three-kernel finish and the single launch."""
    import time

    import torch
    wl = W.workload("fc")
    n = W.alloc_len(wl)
    dws = [W.make_dw(wl, 0, s, dev) for s in range(1, wl.steps + 1)]
    out = {"workload": "fc_100x1000", "elements": wl.numel}
    for label, flags in (("default", 0), ("separate_finish", A.PLAN_SEPARATE_FINISH),
                         ("single_launch", A.PLAN_SINGLE_LAUNCH)):
        plan = A.Plan(wl.segments, plan_flags=flags)
        msg, ws = plan.message_buffer(dev), plan.compress_workspace(dev)
        r = torch.zeros(n, dtype=torch.float32, device=dev)
        for i in range(20):
            A.compress(plan, r, dws[i % len(dws)], msg, ws)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(100)]
        for i, (a, b) in enumerate(ev):
            a.record()
            A.compress(plan, r, dws[i % len(dws)], msg, ws)
            b.record()
        torch.cuda.synchronize()
        per = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
        t0 = time.perf_counter()
        for i in range(500):
            A.compress(plan, r, dws[i % len(dws)], msg, ws)
        torch.cuda.synchronize()
        b2b = (time.perf_counter() - t0) * 1e6 / 500
        # The 10 steps captured once in a HIP graph and replayed 20 times (no host
        # launch per kernel): events around the replays, per call.
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for d in dws:
                    A.compress(plan, r, d, msg, ws)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(20):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        graph_us = a.elapsed_time(b) * 1e3 / (20 * len(dws))
        del g
        out[label] = {"launches": int(plan.info.compress_launches), "call_us": round(per[50], 2),
                      "back_to_back_us": round(b2b, 2), "graph_replay_us": round(graph_us, 2)}
        plan.close()
    return out


def measure_other_workloads(A, W, dev):
    """The three other parity workloads at full size (context; the metric is
    the 1.07e9-element workload's): each runs its first 10 steps from zero
    residue on its own seeded gradients, all resident before timing; steps
    6-10 are timed one call at a time with events (median), then again with
    the 10 calls enqueued back to back (compress_us_queued: the host's
    launches no longer wait for the previous call).  Then the decode of 16
    learners' third-step messages, timed one call at a time after a 1 GiB
    read each."""
    import torch
    out = {}
    for name in ("conv", "fc_lstm", "resnet50"):
        wl = W.workload(name)
        n = W.alloc_len(wl)
        plan = A.Plan(wl.segments)
        dws = [W.make_dw(wl, 0, s, dev) for s in range(1, 11)]
        msg, ws = plan.message_buffer(dev), plan.compress_workspace(dev)
        r = torch.zeros(n, dtype=torch.float32, device=dev)
        times = []
        for s, d in enumerate(dws):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            A.compress(plan, r, d, msg, ws)
            b.record()
            torch.cuda.synchronize()
            if s >= 5:
                times.append(a.elapsed_time(b))
        t = sorted(times)[len(times) // 2]
        total, surv, _ = A.message_header(plan, msg)
        # The same 10 steps again from zero residue, enqueued back to back (no
        # synchronisation between calls, so the host's launches run ahead of the
        # GPU): events around each call, steps 6-10, median.
        r.zero_()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in dws]
        torch.cuda.synchronize()
        for (a, b), d in zip(ev, dws):
            a.record()
            A.compress(plan, r, d, msg, ws)
            b.record()
        torch.cuda.synchronize()
        tq = sorted(a.elapsed_time(b) for a, b in ev[5:])[2]
        del dws
        # Decode of K = 16 messages: learner k's third step from zero residue,
        # each timed call after a 1 GiB read (median of 5).
        msgs = []
        for k in range(16):
            rk = torch.zeros(n, dtype=torch.float32, device=dev)
            for s in range(1, 4):
                A.compress(plan, rk, W.make_dw(wl, k, s, dev), msg, ws)
            tk, _, _ = A.message_header(plan, msg)
            msgs.append(msg[:tk].clone())
            del rk
        dsum = torch.empty(n, dtype=torch.float32, device=dev)
        dws = plan.decode_workspace(len(msgs), dev)
        evict = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dt = []
        for i in range(7):
            evict.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            A.decode_accumulate(plan, msgs, dsum, False, dws)
            b.record()
            torch.cuda.synchronize()
            if i >= 2:
                dt.append(a.elapsed_time(b))
        td = sorted(dt)[len(dt) // 2]
        mbytes = sum(int(m.numel()) for m in msgs)
        out[wl.name] = {"elements": wl.numel, "layers": len(wl.segments),
                        "compress_launches": int(plan.info.compress_launches),
                        "compress_us": round(t * 1e3, 1),
                        "compress_us_queued": round(tq * 1e3, 1),
                        "Gelem_per_s": round(wl.numel / (t * 1e-3) / 1e9, 1),
                        "GBps": round((12.0 * wl.numel + total) / (t * 1e-3) / 1e9, 1),
                        "survivors_step10": int(surv),
                        "decode_messages": len(msgs), "decode_message_bytes": mbytes,
                        "decode_us": round(td * 1e3, 1),
                        "decode_GBps": round((4.0 * wl.numel + mbytes) / (td * 1e-3) / 1e9, 1)}
        plan.close()
        del r, msg, ws, msgs, dsum, dws, evict
    torch.cuda.empty_cache()
    return out


def measure_ls(A, W, dev, wl, dws, n_alloc):
    """Hard local selection (segment flag SEG_LS), after the timed steps:
    (1) compress of the benchmark workload with every layer flagged, on the
    benchmark's own resident gradients (steps 1-10 from zero residue; steps
    6-10 timed one call at a time with events, each after the 1 GiB read
    that evicts the last-level cache, median: the protocol of the bin-length
    sweep and the other workloads); (2) the residue
    contrast the AIMech page's Mechanism claim "self-adjusting sparsity
    prevents residual explosion" draws: the FC/LSTM workload for 50 steps
    from zero residue under AdaComp and under LS on the same seeded
    gradients, max |residue| after steps 1, 10, 20, 30, 40, 50."""
    import torch
    plan = A.Plan([(o, n, b, A.SEG_LS) for (o, n, b) in wl.segments])
    msg, ws = plan.message_buffer(dev), plan.compress_workspace(dev)
    r = torch.zeros(n_alloc, dtype=torch.float32, device=dev)
    evict = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
    times = []
    for i in range(10):
        evict.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        A.compress(plan, r, dws[i % len(dws)], msg, ws)
        b.record()
        torch.cuda.synchronize()
        if i >= 5:
            times.append(a.elapsed_time(b))
    t = statistics.median(times)
    total, surv, _ = A.message_header(plan, msg)
    out = {"workload": wl.name, "compress_ms": round(t, 4),
           "Gelem_per_s": round(wl.numel / (t * 1e-3) / 1e9, 1),
           "compress_frac_of_peak": round(12.0 * wl.numel / (t * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
           "survivors_step10": int(surv)}
    plan.close()
    del r, msg, ws, evict
    torch.cuda.empty_cache()

    demo = W.workload("fc_lstm")
    n = W.alloc_len(demo)
    growth = {}
    for label, flag in (("adacomp", 0), ("ls", A.SEG_LS)):
        plan = A.Plan([(o, k, b, flag) for (o, k, b) in demo.segments])
        msg, ws = plan.message_buffer(dev), plan.compress_workspace(dev)
        r = torch.zeros(n, dtype=torch.float32, device=dev)
        d = torch.empty(n, dtype=torch.float32, device=dev)
        trace = {}
        for step in range(1, 51):
            W.fill_dw(d, demo, 0, step)
            A.compress(plan, r, d, msg, ws)
            if step in (1, 10, 20, 30, 40, 50):
                trace[step] = float(r.abs().max())
        growth[label] = trace
        plan.close()
        del r, d, msg, ws
    out["residue_growth"] = {"workload": demo.name, "max_abs_residue": growth}
    return out


def lt_sweep(args):
    """Bin-length sweep (not the default run): the same 64 x 4096 x 4096
    layers and the same gradient stream compressed with L_T = 50, 500 and 5000
    (8-bit words at 50, 16-bit otherwise), 10 steps each from a zero residue.
    One JSON line per L_T: compress time and HBM fraction over steps 6..10,
    payload and wire compression ratio and the largest |residue| at step 10."""
    import torch
    import adaptive_residual_gradient_amd as A
    import workloads as W
    from adaptive_residual_gradient_amd import stats

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = W.workload(args.workload)
    n_alloc, N = W.alloc_len(wl), wl.numel
    steps = 10
    dws = []
    for s in range(1, steps + 1):
        t = torch.empty(n_alloc, dtype=torch.float32, device=dev)
        W.fill_dw(t, wl, 0, s)
        dws.append(t)
    for lt in (50, 500, 5000):
        segs = [(o, n, lt) for (o, n, _) in wl.segments]
        plan = A.Plan(segs)
        msg, ws = plan.message_buffer(dev), plan.compress_workspace(dev)
        residue = torch.zeros(n_alloc, dtype=torch.float32, device=dev)
        timer = A.Timer()
        for i in range(steps):
            if i == 5:
                torch.cuda.synchronize()
                timer.reset()
            A.compress(plan, residue, dws[i], msg, ws, timer=timer if i >= 5 else None)
        torch.cuda.synchronize()
        st = timer.read()
        call = st["compress_call"][0] / st["compress_call"][1]
        tile = st["tile_pass"][0] / st["tile_pass"][1]
        total, surv, _ = A.message_header(plan, msg)
        pr, wr, _, _ = stats.message_ratios(segs, bytes(msg[: int(plan.info.header_bytes)].cpu().numpy()))
        rmax = float(residue.abs().max().item())
        # decode of K learners' step-10 messages (learners 1..K, own seeds)
        K = args.learners
        msgs = []
        lr = torch.empty(n_alloc, dtype=torch.float32, device=dev)
        for k in range(1, K + 1):
            lr.zero_()
            for s in range(1, steps + 1):
                W.fill_dw(dws[0], wl, k, s)
                A.compress(plan, lr, dws[0], msg, ws)
            t_k, _, _ = A.message_header(plan, msg)
            msgs.append(msg[:t_k].clone())
        W.fill_dw(dws[0], wl, 0, 1)
        out = torch.empty(n_alloc, dtype=torch.float32, device=dev)
        dws_dec = plan.decode_workspace(K, dev)
        timer.reset()
        for i in range(6):
            A.decode_accumulate(plan, msgs, out, False, dws_dec, timer=timer if i >= 2 else None)
        torch.cuda.synchronize()
        dst = timer.read()
        dec = dst["decode_call"][0] / dst["decode_call"][1]
        dec_bytes = float(sum(m.numel() for m in msgs)) + 4.0 * N
        del msgs, lr, out, dws_dec
        print(json.dumps({
            "sweep": "bin_len", "workload": wl.name, "bin_len": lt,
            "index_bits": 8 if lt < 64 else 16, "steps": steps,
            "compress_ms": round(call, 4), "Gelem_per_s": round(N / (call * 1e-3) / 1e9, 2),
            "compress_frac_of_peak": round(12.0 * N / (call * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "tile_pass_ms": round(tile, 4),
            "tile_pass_frac_of_peak": round(12.0 * N / (tile * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "survivors_step10": int(surv), "message_bytes_step10": int(total),
            "payload_ratio": round(pr, 1), "wire_ratio": round(wr, 1),
            "max_abs_residue_step10": rmax,
            "decode_messages": K, "decode_ms": round(dec, 4),
            "decode_GBps": round(dec_bytes / (dec * 1e-3) / 1e9, 1),
        }), flush=True)
        timer.close()
        plan.close()
        del msg, ws, residue
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="large")
    ap.add_argument("--learners", type=int, default=16)
    ap.add_argument("--learner-steps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--lt-sweep", action="store_true",
                    help="instead of the benchmark, compress the workload with L_T = 50, 500 "
                         "and 5000 and print one JSON line per bin length")
    ap.add_argument("--no-small-table", action="store_true",
                    help="leave the small-table, other-workload and LS measurements out of the default run "
                         "(profiling runs that select the benchmark's own tile-pass dispatches by order)")
    ap.add_argument("--small-table", action="store_true",
                    help="instead of the benchmark, time the compress of the 100 x 1000 layer "
                         "with each finish (default, three-kernel, single launch); one JSON line")
    ap.add_argument("--other-workloads", action="store_true",
                    help="instead of the benchmark, time the compress (steps 6-10 from zero "
                         "residue) and a K = 16 decode of the conv-stack, FC/LSTM and ResNet-50 "
                         "tables; one JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain device copy of 1 GiB (a known-size reference "
                         "for rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this build measures one GPU: the compressor runs per learner "
                                   "on its own GPU; multi-GPU exchange is not built (run with --gpus 1)"}))
        sys.exit(2)
    if args.lt_sweep:
        lt_sweep(args)
        return
    if args.small_table:
        import torch

        import adaptive_residual_gradient_amd as A
        import workloads as W
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        print(json.dumps(measure_small_table(A, W, dev)), flush=True)
        return
    if args.other_workloads:
        import torch

        import adaptive_residual_gradient_amd as A
        import workloads as W
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        print(json.dumps(measure_other_workloads(A, W, dev)), flush=True)
        return

    import numpy as np
    import torch

    import adaptive_residual_gradient_amd as A
    import workloads as W
    from adaptive_residual_gradient_amd import stats

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    wl = W.workload(args.workload)
    n_alloc = W.alloc_len(wl)
    N = wl.numel
    plan = A.Plan(wl.segments)
    info = plan.info
    log(f"workload {wl.name}: {N} elements, {len(wl.segments)} layers, {info.total_bins} bins")

    # Decode inputs: K learners, each running its own steps from zero residue.
    K = args.learners
    msg = plan.message_buffer(dev)
    ws = plan.compress_workspace(dev)
    dbuf = torch.empty(n_alloc, dtype=torch.float32, device=dev)
    learner_msgs, learner_bytes = [], []
    for k in range(1, K + 1):
        r = torch.zeros(n_alloc, dtype=torch.float32, device=dev)
        for s in range(1, args.learner_steps + 1):
            W.fill_dw(dbuf, wl, k, s)
            A.compress(plan, r, dbuf, msg, ws)
        total, _, _ = A.message_header(plan, msg)
        learner_msgs.append(msg[:total].clone())
        learner_bytes.append(total)
        del r
    log(f"built {K} learner messages, {sum(learner_bytes) / 1e6:.1f} MB in total")

    # The benchmarked learner (learner 0): all step gradients resident in HBM.
    nsteps = args.warmup + args.steps
    dws = []
    for s in range(1, nsteps + 1):
        t = torch.empty(n_alloc, dtype=torch.float32, device=dev)
        W.fill_dw(t, wl, 0, s)
        dws.append(t)
    residue = torch.zeros(n_alloc, dtype=torch.float32, device=dev)
    out = torch.empty(n_alloc, dtype=torch.float32, device=dev)
    dws_dec = plan.decode_workspace(K, dev)
    copy_gbps = measure_copy(dev)

    # First run, untimed: every step from zero residue; its messages kept.
    ref_msgs = []
    for i in range(nsteps):
        A.compress(plan, residue, dws[i], msg, ws)
        total_i, _, _ = A.message_header(plan, msg)
        ref_msgs.append(msg[:total_i].clone())
    ratios = [stats.message_ratios(wl.segments, bytes(m[: int(info.header_bytes)].cpu().numpy()))[:2]
              for m in ref_msgs]

    # The rerun: zero residue again, warm-up steps, then the timed steps.
    residue.zero_()
    evict = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
    timers = [A.Timer() for _ in range(args.steps)]
    rerun_msgs = []
    torch.cuda.synchronize()

    def step(i, tm):
        evict.sum()
        A.compress(plan, residue, dws[i], msg, ws, timer=tm)
        rerun_msgs.append(msg[: ref_msgs[i].numel()].clone())
        evict.sum()
        A.decode_accumulate(plan, learner_msgs, out, False, dws_dec, timer=tm)

    for i in range(args.warmup):
        step(i, None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, nsteps):
        step(i, timers[i - args.warmup])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    reads = [t.read() for t in timers]
    for t in timers:
        t.close()
    del evict
    rerun_identical = all(torch.equal(a, b) for a, b in zip(ref_msgs, rerun_msgs))
    st = {k: (sum(r[k][0] for r in reads), sum(r[k][1] for r in reads)) for k in reads[0]}
    per_compress = [r["compress_call"][0] for r in reads]
    per_decode = [r["decode_call"][0] for r in reads]

    # Message of the last timed step (for the compression ratio).
    total, surv, dirs = A.message_header(plan, msg)
    bin_lens = sorted({int(seg[2]) for seg in wl.segments})
    pr, wr, _, _ = stats.message_ratios(wl.segments, bytes(msg[: int(info.header_bytes)].cpu().numpy()))

    ms = {k: v[0] / max(v[1], 1) for k, v in st.items()}
    launches = {k: v[1] for k, v in st.items()}
    compress_ms = ms["compress_call"]    # whole call: kernels and the gaps between them
    decode_ms = ms["decode_call"]
    tile_bytes = 12.0 * N                       # read residue + dW, write residue
    achieved = tile_bytes / (ms["tile_pass"] * 1e-3) / 1e9
    compress_bytes = 12.0 * N + total
    decode_bytes = float(sum(learner_bytes)) + 4.0 * N
    traffic = traffic_from_profiles(args.workload)

    res = {
        "metric": METRIC,
        "value": round(N / (compress_ms * 1e-3) / 1e9, 3),
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": len(wl.segments), "numel": N,
                   "bin_len": bin_lens[0] if len(bin_lens) == 1 else bin_lens,
                   "index_bits": sorted({8 if b < 64 else 16 for b in bin_lens}) if len(bin_lens) > 1
                   else (8 if bin_lens[0] < 64 else 16),
                   "decode_messages": K, "learner_steps": args.learner_steps},
        "roofline": {"bound": "hbm", "kernel": "tile_pass",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic},
        "compress_ms": round(compress_ms, 4),
        "compress_GBps": round(compress_bytes / (compress_ms * 1e-3) / 1e9, 1),
        "compress_frac_of_peak": round(compress_bytes / (compress_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "decode_ms": round(decode_ms, 4),
        "decode_GBps": round(decode_bytes / (decode_ms * 1e-3) / 1e9, 1),
        "stage_ms": {k: round(v, 4) for k, v in ms.items()},
        "stage_launches": launches,
        "last_message": {"bytes": int(total), "survivors": int(surv),
                         "payload_ratio": round(pr, 2), "wire_ratio": round(wr, 2)},
        "compress_ms_median": round(statistics.median(per_compress), 4),
        "decode_ms_median": round(statistics.median(per_decode), 4),
        "per_step": {"compress_ms": [round(x, 4) for x in per_compress],
                     "decode_ms": [round(x, 4) for x in per_decode],
                     "payload_ratio": [round(x[0], 2) for x in ratios[args.warmup:]],
                     "wire_ratio": [round(x[1], 2) for x in ratios[args.warmup:]]},
        "rerun_identical": rerun_identical,
        "cache_eviction": "1 GiB scratch read before every timed compress and decode call",
        "copy_bw": {"GBps": round(max(copy_gbps.values()), 1),
                    "by_method": {k: round(v, 1) for k, v in copy_gbps.items()},
                    "tile_pass_frac_of_copy": round(achieved / max(copy_gbps.values()), 4)},
    }
    res["decode_sgd"] = measure_decode_sgd(A, plan, learner_msgs, n_alloc, N, K, dev)
    res["small_table"] = None if args.no_small_table else measure_small_table(A, W, dev)
    res["other_workloads"] = None if args.no_small_table else measure_other_workloads(A, W, dev)
    res["ls"] = None if args.no_small_table else measure_ls(A, W, dev, wl, dws, n_alloc)

    if not args.no_cpu_baseline:
        def host_dw(step_idx, length):
            # the benchmarked learner's gradient of step step_idx+1, first layers
            return dws[min(step_idx, nsteps - 1)][:length].cpu().numpy().copy()
        res["cpu_baseline"] = cpu_baseline(wl, host_dw, nsteps)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
