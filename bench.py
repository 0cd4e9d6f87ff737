#!/usr/bin/env python3
"""Benchmark: one 1-bit LAMB compression-stage step over the BERT-Large
tensor table (385 fp32 tensors, N = 333,563,904 parameters) with W = 8
simulated workers on one MI355X.

A step is the whole hot path through the C ABI: every worker's
error-compensated 1-bit compression of its momentum, the server average
and recompression, the reconstructed gradient and fresh variance, the
per-tensor rescale with soft thresholds, and the parameter update.  Inputs
are synthetic (seeded counter-based generator) and already resident in HBM
when the timed region starts; the gradient buffers are filled once and
reused by every step (the optimizer state still evolves step to step).

Prints one JSON line.  `value` is parameters per second for the step with
fp32 momentum; `packed_momentum` times the same step with the momentum kept
as the server's packed output (bit-identical results); `roofline` is the
dominant kernel (phase 1: compression, average, rescale statistics) timed
with HIP events on its stream; `runtime_copy` is the runtime's own 1 GiB
device-to-device copy timed on the same machine, as a reference rate;
`cpu_baseline` is the single-threaded CPU oracle on a bounded window of the
same workload.  `--method adam` and
`--method sparse` time the 1-bit Adam mode and the SLAMB-style sparse stage
on the same buffers instead.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "params/sec and achieved HBM GB/s (% of peak) per 1-bit LAMB step"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def step_bytes(N, K, C, W):
    """Algorithmic bytes of the step, every array touched once: momentum
    read and written, each worker's gradient read and error read and
    written, the server error read and written, the frozen variance read,
    the fresh variance and the parameters read and written, and the packed
    signs and scales of the W workers and the server written."""
    packed = (W + 1) * K * (C // 8 + 4)
    return N * (12 * W + 36) + packed


def step_bytes_packed(N, K, C, W):
    """The same step with packed momentum: the momentum is read as the
    previous server signs and scales instead of fp32, and not written."""
    packed = (W + 1) * K * (C // 8 + 4)
    return N * (12 * W + 28) + packed + K * (C // 8 + 4)


def phase1_bytes(N, K, C, W):
    """Algorithmic bytes of the phase-1 kernel: m read; per worker g read,
    e read and written; e_s read and written; v_fresh read and written;
    v_frozen read; (W+1) packed sign arrays and scales written."""
    packed = (W + 1) * K * (C // 8 + 4)
    return N * (12 * W + 24) + packed


def adam_bytes(N, K, C, W):
    """Algorithmic bytes of one 1-bit Adam compression step, both kernels:
    the allreduce (m read; per worker g read, e read and written; e_s read
    and written; (W+1) packed sign arrays and scales written), then the
    update (the server's packed output read back; x read and written;
    v_frozen read; m written)."""
    packed = K * (C // 8 + 4)
    return N * (12 * W + 12) + (W + 1) * packed + N * 16 + packed


def sparse_bytes(N, K, C, W, nsel):
    """Algorithmic bytes of the sparse-stage kernel: m read and written; per
    worker g read, e read and written; on the transmitted fraction
    f = nsel*64/C: x and v_fresh read and written, v_frozen read, W + 1
    transmitted values written; the selection read."""
    f = nsel * 64 / C
    return int(N * (12 * W + 8) + N * f * (20 + 4 * (W + 1)) + 4 * K)


def copy_ceiling(torch, stream, nbytes=1 << 30, reps=10):
    """torch's device-to-device copy of nbytes on the same stream, timed with
    HIP events: a reference rate of this machine, reported beside the 8 TB/s
    peak.  Returns GB/s counting the bytes read and written."""
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        b.copy_(a)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    del a, b
    return 2 * nbytes / (ms * 1e-3) / 1e9


def _ceiling(torch, stream, achieved):
    copy_gbps = copy_ceiling(torch, stream)
    log(f"[bench] runtime copy {copy_gbps:.0f} GB/s")
    return {"copy_GBps": copy_gbps, "copy_frac_of_peak": copy_gbps / PEAK_HBM_GBPS,
            "kernel_frac_of_copy": achieved / copy_gbps,
            "note": "1 GiB device-to-device copy by the runtime (torch copy_) on the same stream "
                    "after the timed steps, read plus written bytes; a reference rate of the machine, "
                    "not an upper bound (a tuned streaming copy runs faster)"}


def _ceiling_lib():
    import ctypes
    path = os.path.join(ROOT, "communication_compressed_optimizer_amd", "libonebit_ceiling.so")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.onebit_ceiling_read.argtypes = [ctypes.c_int64, P, P, P]
    lib.onebit_ceiling_copy.argtypes = [ctypes.c_int64, P, P, P]
    lib.onebit_ceiling_phase1.argtypes = [ctypes.c_int64, ctypes.c_int32, P, P, P, P, P, P, P, P,
                                          ctypes.c_uint32, ctypes.c_int32, ctypes.c_int32, P]
    return lib


def pattern_ceiling(torch, stream, wl, g, e, err_s, m, v, vf, bits_w, bits_s, achieved,
                    reps=10):
    """The machine's practical ceiling, measured in the same run on the step's own
    buffers by pure-traffic kernels with the step's loads, stores and launch
    shape (libonebit_ceiling.so): phase 1's exact stream set (m read; per
    worker g and e read, e and the sign words written, a workgroup barrier per
    worker; e_s read and written; v_fresh and v_frozen read, v_fresh written;
    the server's sign words written), a streaming read and a streaming copy.
    The written arrays get their own bits back, so the state is unchanged.
    Returns the rates (GB/s of bytes read plus written) and phase 1's
    fraction of its own pattern's rate."""
    import ctypes
    lib = _ceiling_lib()
    N, W = wl.N, wl.W
    n = (N // 4096) * 4096                         # the kernels' whole 4096-element chunks
    P = ctypes.c_void_p
    ga = (P * W)(*[t.data_ptr() for t in g])
    ea = (P * W)(*[t.data_ptr() for t in e])
    ba = (P * W)(*[t.data_ptr() for t in bits_w])
    tmp = torch.empty(N, dtype=torch.float32, device="cuda")
    sink = torch.empty(N // 4096 + 1, dtype=torch.float32, device="cuda")
    st = stream.cuda_stream
    pbytes = n * (12 * W + 24) + (W + 1) * n // 8
    calls = {
        "phase1_pattern": (lambda: lib.onebit_ceiling_phase1(
            n, W, m.data_ptr(), ga, ea, ba, err_s.data_ptr(), v.data_ptr(), vf.data_ptr(),
            bits_s.data_ptr(), 0, 0, 0, st), pbytes),
        # the same pattern at one workgroup per CU, the launch shape of the
        # persistent pass A
        "phase1_pattern_1_per_cu": (lambda: lib.onebit_ceiling_phase1(
            n, W, m.data_ptr(), ga, ea, ba, err_s.data_ptr(), v.data_ptr(), vf.data_ptr(),
            bits_s.data_ptr(), 0, 0, _LDS_CAPS[1], st), pbytes),
        "stream_read": (lambda: lib.onebit_ceiling_read(n, g[0].data_ptr(), sink.data_ptr(), st),
                        4 * n),
        "stream_copy": (lambda: lib.onebit_ceiling_copy(n, g[0].data_ptr(), tmp.data_ptr(), st),
                        8 * n),
    }
    out = {}
    for name, (fn, nbytes) in calls.items():
        for _ in range(2):
            assert fn() == 0, name
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(reps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / reps
        out[name + "_GBps"] = nbytes / (ms * 1e-3) / 1e9
    del tmp, sink
    out["phase1_frac_of_pattern"] = achieved / out["phase1_pattern_GBps"]
    best = max(out["phase1_pattern_GBps"], out["phase1_pattern_1_per_cu_GBps"])
    out["phase1_frac_of_best_pattern"] = achieved / best
    out["note"] = ("pure-traffic kernels on the step's own buffers after the timed steps "
                   "(libonebit_ceiling.so): phase 1's stream set with its barriers and no "
                   "arithmetic, with one workgroup per chunk and at one workgroup per CU, a "
                   "streaming read, a streaming copy; bytes read plus written")
    log("[bench] ceiling: " + ", ".join(f"{k} {v:.0f}" for k, v in out.items()
                                        if k.endswith("GBps")) +
        f" GB/s; phase 1 at {out['phase1_frac_of_pattern']:.3f} of its pattern, "
        f"{out['phase1_frac_of_best_pattern']:.3f} of the faster of the two")
    return out


def graph_replay(torch, fn, steps, warm=2):
    """ms per call of fn (which enqueues on torch's current stream) when it is
    captured once in a HIP graph and replayed: `warm` untimed replays, then
    `steps` replays between two events."""
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    for _ in range(warm):
        g.replay()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    cur = torch.cuda.current_stream()
    ev[0].record(cur)
    for _ in range(steps):
        g.replay()
    ev[1].record(cur)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    del g
    return ms


def cpu_baseline(wl, n_chunks, method="lamb", nsel=1, by_step=None):
    """The oracle (single-threaded C, as it stands) on the window of the
    first n_chunks chunks of the workload: one compression step.  With
    by_step (a dict, LAMB only), the same window's other step types are
    timed into it too: the LAMB warmup step, the workers' compression
    (onebit_compress_ef's rule, one worker) and the server's average and
    recompression (onebit_average_packed's rule, W workers)."""
    import oracle
    from tests.harness import HostRun
    hi = min(wl.N, n_chunks * wl.chunk)
    h = HostRun(wl, 0, hi)
    h.fill_grads(0)
    t0 = time.perf_counter()
    if method == "adam":
        h.adam_compressed_step(0, fill=False)
    elif method == "sparse":
        h.sparse_step(0, nsel, fill=False)
    else:
        h.compressed_step(0, fill=False)
    dt = time.perf_counter() - t0
    what = {"adam": "1-bit Adam", "sparse": f"sparse ({nsel} block(s) of 64 per chunk)"}.get(
        method, "1-bit LAMB")
    sample = (f"elements [0, {hi}) of the {wl.name} table (first {-(-hi // wl.chunk)} chunks, "
              f"W={wl.W})")
    if by_step is not None and method == "lamb":
        def timed(fn):
            t = time.perf_counter()
            fn()
            return time.perf_counter() - t
        out = h.out
        h.fill_grads(1)                       # untimed, like the compression step's
        steps = {
            "compressed_step": dt,
            "compress_ef": timed(lambda: oracle.compress_ef(h.g[0], h.e[0], wl.chunk)),
            "average_packed": timed(lambda: oracle.average_packed(out["bits_w"], out["scales_w"],
                                                                  h.err_s, wl.chunk)),
            "warmup_step": timed(lambda: h.warmup_step(1, fill=False)),
        }
        for k, t in steps.items():
            by_step[k] = {"value": hi / t, "unit": "params/s", "seconds": t, "cores": 1,
                          "kind": "oracle", "sample": sample}
    return {"value": hi / dt, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"one {what} compression step on {sample}; {dt:.2f} s"}


def cpu_baseline_by_config(max_chunks=8192):
    """The oracle (as it stands, one core) on each configuration of the
    workload set: the whole table where it is small (Tiny, Single), else its
    first max_chunks chunks (Mixed, BERT-XL; BERT-Large is the main
    baseline's window).  Configurations that start with a warmup time one
    warmup step, then (after the freeze) one compression step; the others
    one compression step.  Gradients are filled before each timed call."""
    from synth.workloads import WORKLOADS
    from tests.harness import HostRun
    out = {}
    for name in ("tiny", "single", "mixed", "bert_xl"):
        wl = WORKLOADS[name]
        hi = min(wl.N, max_chunks * wl.chunk)
        h = HostRun(wl, 0, hi)
        entry = {"elements": hi, "W": wl.W, "cores": 1, "kind": "oracle",
                 "sample": f"elements [0, {hi}) of the {name} table"
                           + (" (whole)" if hi == wl.N else f" (first {-(-hi // wl.chunk)} chunks)")}
        if wl.init == "fresh":
            h.fill_grads(0)
            t0 = time.perf_counter()
            h.warmup_step(0, fill=False)
            entry["warmup_step_params_per_s"] = hi / (time.perf_counter() - t0)
            h.freeze(1)
        h.fill_grads(1)
        t0 = time.perf_counter()
        h.compressed_step(1, fill=False)
        entry["compressed_step_params_per_s"] = hi / (time.perf_counter() - t0)
        out[name] = entry
        del h
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="bert_large")
    ap.add_argument("--chunk", type=int, default=0,
                    help="elements per compression chunk (0 = the workload's own, 4096); a "
                         "power of two in [64, 16384]")
    ap.add_argument("--method", choices=("lamb", "adam", "sparse", "share"), default="lamb",
                    help="1-bit LAMB (the default), the 1-bit Adam mode, the SLAMB-style "
                         "sparse stage, or one GPU's share of a W-GPU 1-bit LAMB step, on the "
                         "same buffers")
    ap.add_argument("--nsel", type=int, default=1,
                    help="sparse stage: transmitted 64-element blocks per chunk")
    ap.add_argument("--cpu-chunks", type=int, default=40960,
                    help="chunks of the workload the CPU oracle baseline runs (0 = skip)")
    ap.add_argument("--ceiling-sweep", action="store_true",
                    help="time the real phase 1 against the pure-traffic kernel of its stream "
                         "pattern at several caps on the workgroups per CU, and the pattern's "
                         "loads alone and stores alone (overwrites the state; one JSON line)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 2^28 floats (1 GiB) three times, the "
                         "reference for scaling HBM byte counters")
    args = ap.parse_args()

    if args.calibrate_copy:
        import torch
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("[bench] copied 3 x 1 GiB")
        return

    if args.gpus != 1:
        log(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the W workers are "
            "simulated as W buffers on one device, so there is no multi-GPU run to measure")
        sys.exit(2)

    need = [os.path.join(ROOT, "communication_compressed_optimizer_amd", "libonebit.so"),
            os.path.join(ROOT, "communication_compressed_optimizer_amd", "libonebit_ceiling.so"),
            os.path.join(ROOT, "synth", "libsynth_dev.so"), os.path.join(ROOT, "oracle", "liboracle.so")]
    if not all(os.path.exists(p) for p in need):
        import __graft_entry__
        __graft_entry__.build()

    import torch
    import communication_compressed_optimizer_amd as ob
    from synth.workloads import HPARAMS, WORKLOADS

    wl = WORKLOADS[args.workload]
    if args.chunk:
        import dataclasses
        wl = dataclasses.replace(wl, chunk=args.chunk)
    C, N, W, K, L = wl.chunk, wl.N, wl.W, wl.K, wl.L
    torch.cuda.set_device(0)
    dev = "cuda"
    log(f"[bench] workload {wl.name}: N={N} L={L} K={K} W={W} chunk={C}; allocating state")
    table = ob.LayerTable(wl.numels, C)

    def f():
        return torch.empty(N, dtype=torch.float32, device=dev)

    x, m, v, vf = f(), f(), f(), f()
    err_s = torch.zeros(N, dtype=torch.float32, device=dev)
    g = [f() for _ in range(W)]
    e = [torch.zeros(N, dtype=torch.float32, device=dev) for _ in range(W)]
    words = K * C // 32
    bits_w = [torch.zeros(words, dtype=torch.int32, device=dev) for _ in range(W)]
    scales_w = [torch.zeros(K, dtype=torch.float32, device=dev) for _ in range(W)]
    bits_s = torch.zeros(words, dtype=torch.int32, device=dev)
    scales_s = torch.zeros(K, dtype=torch.float32, device=dev)
    c_avg = torch.ones(L, dtype=torch.float32, device=dev)
    f_prev = torch.ones(L, dtype=torch.float32, device=dev)
    c_out = torch.zeros(L, dtype=torch.float32, device=dev)
    ws = torch.empty(table.workspace_size(W), dtype=torch.uint8, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    hp = ob.onebit_hparams(**HPARAMS)
    wl.fill("x", x)
    wl.fill("m", m)
    wl.fill("v", v)
    vf.copy_(v)
    for w in range(W):
        wl.fill("g", g[w], 0, 0, w)
    torch.cuda.synchronize()
    log("[bench] inputs resident; warming up")

    stream = torch.cuda.current_stream()

    if args.ceiling_sweep:
        return ceiling_sweep(args, wl, ob, torch, table, hp, g, e, err_s, m, v, vf, bits_w,
                             scales_w, bits_s, scales_s, ws, status, stream)
    if args.method == "adam":
        return bench_adam(args, wl, ob, torch, hp, g, e, err_s, x, m, v, bits_w, scales_w, bits_s,
                          scales_s, status, stream)
    if args.method == "sparse":
        return bench_sparse(args, wl, ob, torch, table, hp, g, e, x, m, v, vf, c_avg, status,
                            stream)
    if args.method == "share":
        return bench_share(args, wl, ob, torch, table, hp, g, e, err_s, x, m, v, vf, bits_w,
                           scales_w, bits_s, scales_s, c_avg, f_prev, c_out, ws, status, stream)

    def step(ev=None, mm=m, st=stream):
        if ev is not None:
            ev[0].record(st)
        ob.onebit_lamb_compress_average(table, W, g, e, err_s, mm, v, vf, bits_w, scales_w, bits_s,
                                        scales_s, hp, ws, status, st)
        if ev is not None:
            ev[1].record(st)
        ob.onebit_lamb_rescale_update(table, bits_s, scales_s, x, mm, v, c_avg, f_prev, c_out, hp,
                                      ws, status, st)
        if ev is not None:
            ev[2].record(st)

    def timed(mm):
        """ms per step over `steps` steps with nothing between them (the step
        time), then the two phases' mean times from HIP events recorded
        around each phase of `steps` further steps (events between kernels
        cost the stream a little, so they stay out of the step time)."""
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(None, mm)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        for i in range(args.steps):
            step(evs[i], mm)
        torch.cuda.synchronize()
        p1 = [a.elapsed_time(b) for a, b, _ in evs]
        p2 = [b.elapsed_time(c) for _, b, c in evs]
        timed.p1 = sorted(p1)
        return (t1 - t0) * 1e3 / args.steps, sum(p1) / len(p1), sum(p2) / len(p2)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms_per_step, p1_ms, p2_ms = timed(m)
    p1_sorted = timed.p1
    st = int(status.item())
    if st:
        log(f"[bench] WARNING: status flags {st} (non-finite scale or statistic)")
    log(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step (phase1 {p1_ms:.3f} ms, "
        f"phase2 {p2_ms:.3f} ms)")
    # context: the same steps with packed momentum (m = NULL: the momentum is
    # the previous server output, bit-identical results, no fp32 copy)
    # (the fused step takes no packed momentum at chunks over 16384)
    long_chunk = C > 16384
    if not long_chunk:
        pm_ms, pm_p1, pm_p2 = timed(None)
        log(f"[bench] packed momentum {args.steps} steps: {pm_ms:.3f} ms/step (phase1 "
            f"{pm_p1:.3f} ms, phase2 {pm_p2:.3f} ms)")
    # context: the fp32-momentum step captured once in a HIP graph and
    # replayed, as a training loop with fixed hyper-parameters can run it; it
    # takes the host's per-call work (argument checks, launches) off the
    # step, which is what bounds the step on small tables
    gr_ms = graph_replay(torch, lambda: step(st=torch.cuda.current_stream()), args.steps)
    log(f"[bench] graph replay {args.steps} steps: {gr_ms:.3f} ms/step")

    # context: the LAMB warmup step on the same table (after the timed
    # compression steps; it reuses the same buffers), carrying the
    # parameters' squared norm from step to step as a warmup loop would
    c_sum = torch.zeros(L, dtype=torch.float32, device=dev)
    x_sq = torch.zeros(table.n_segments, dtype=torch.float64, device=dev)
    for i in range(2):
        ob.onebit_lamb_warmup_step_carry(table, W, g, x, m, v, c_sum, c_out, x_sq, int(i > 0), hp,
                                         ws, status, stream)
    wev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    wsteps = 5
    wev[0].record(stream)
    for _ in range(wsteps):
        ob.onebit_lamb_warmup_step_carry(table, W, g, x, m, v, c_sum, c_out, x_sq, 1, hp, ws,
                                         status, stream)
    wev[1].record(stream)
    torch.cuda.synchronize()
    warm_ms = wev[0].elapsed_time(wev[1]) / wsteps
    warm_bytes = N * (4 * W + 24)          # each array once: the algorithmic count
    warm_moved = N * (4 * W + 32)          # the two passes: m, v and x read again by the update

    sbytes = step_bytes(N, K, C, W)
    pm_bytes = None if long_chunk else step_bytes_packed(N, K, C, W)
    abytes = phase1_bytes(N, K, C, W)
    achieved = abytes / (p1_ms * 1e-3) / 1e9
    step_gbps = sbytes / (ms_per_step * 1e-3) / 1e9
    traffic = _measured_traffic("traffic_compress_average_bert_large.txt") \
        if wl.name == "bert_large" else None
    cpu = None
    cpu_by_step = {}
    cpu_by_config = None
    if args.cpu_chunks > 0:
        log("[bench] CPU oracle baseline ...")
        cpu = cpu_baseline(wl, args.cpu_chunks, by_step=cpu_by_step)
        log(f"[bench] oracle: {cpu['value']:.3e} params/s ({cpu['sample']})")
        log("[bench] oracle by step: " + ", ".join(f"{k} {v['value']:.3e} params/s"
                                                   for k, v in cpu_by_step.items()))
        cpu_by_config = cpu_baseline_by_config()
        log("[bench] oracle by config: " + ", ".join(
            f"{k} {v['compressed_step_params_per_s']:.3e}" for k, v in cpu_by_config.items()))

    out = {
        "metric": METRIC,
        "value": N / (ms_per_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: 1-bit LAMB compression-stage step, {L} tensors, "
                               f"N={N}, W={W} simulated workers, chunk {C}",
                   "N": N, "W": W, "tensors": L, "chunk": C},
        "achieved_GBps": step_gbps,
        "frac_of_peak": step_gbps / PEAK_HBM_GBPS,
        "step_bytes": sbytes,
        "phase_ms": {"compress_average": p1_ms, "rescale_update": p2_ms},
        "phase1_ms_per_step": {"min": p1_sorted[0], "median": p1_sorted[len(p1_sorted) // 2],
                               "max": p1_sorted[-1]},
        "warmup_step": {"ms": warm_ms, "params_per_s": N / (warm_ms * 1e-3),
                        "GBps": warm_bytes / (warm_ms * 1e-3) / 1e9,
                        "frac_of_peak": warm_bytes / (warm_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                        "bytes": warm_bytes, "moved_bytes": warm_moved,
                        "moved_GBps": warm_moved / (warm_ms * 1e-3) / 1e9,
                        "note": "onebit_lamb_warmup_step_carry, norm carried; GBps counts each "
                                "array once (4W+24 B/elem), moved_GBps the two passes' traffic "
                                "(4W+32: the update rereads m, v and x)"},
        "packed_momentum": {
            "note": "not taken by the fused step at chunks over 16384 elements"} if long_chunk
        else {
            "ms_per_step": pm_ms, "params_per_s": N / (pm_ms * 1e-3),
            "phase_ms": {"compress_average": pm_p1, "rescale_update": pm_p2},
            "step_bytes": pm_bytes, "GBps": pm_bytes / (pm_ms * 1e-3) / 1e9,
            "note": "same step with m = NULL: the momentum is the previous server output "
                    "(bits_s, scales_s), outputs bit-identical to the fp32-momentum step"},
        "graph_replay": {
            "ms_per_step": gr_ms, "params_per_s": N / (gr_ms * 1e-3),
            "GBps": sbytes / (gr_ms * 1e-3) / 1e9,
            "note": "the same fp32-momentum step captured once in a HIP graph and replayed "
                    "(the hyper-parameters are fixed at capture); no host work per step"},
        "roofline": {"bound": "hbm",
                     # the library's choice of pass-A kernel (persistent ring at
                     # 4096-element chunks from seven workers up)
                     "kernel": "k_compressed_pass_a_ring<4096>" if C == 4096 and W >= 7 else
                     ("k_big_workers_compress, k_big_average_packed, k_big_rescale_stats"
                      if long_chunk else f"k_compressed_pass_a<{C}>"),
                     "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic,
                     "algorithmic_bytes": abytes},
        "ceiling": pattern_ceiling(torch, stream, wl, g, e, err_s, m, v, vf, bits_w, bits_s,
                                   achieved),
        "runtime_copy": _ceiling(torch, stream, achieved),
        "cpu_baseline": cpu,
        "cpu_baseline_by_step": cpu_by_step or None,
        "cpu_baseline_by_config": cpu_by_config,
        "readings": "the compression-stage rescale (reconstructed gradient, fresh variance, "
                    "rho as the per-tensor maximum of the ratio, the soft thresholds) is a "
                    "reading of the 1-bit LAMB page's prose, which prints no formula for it; "
                    "GPU and oracle agree on that reading, not on a printed equation",
    }
    print(json.dumps(out), flush=True)


# Dynamic LDS per workgroup that caps the workgroups resident on a CU (160 KiB
# of LDS per CU; the pattern kernel's own 2 KiB added): 1, 2, 3, 4 per CU.
_LDS_CAPS = {1: 84 * 1024, 2: 56 * 1024, 3: 44 * 1024, 4: 36 * 1024}


def ceiling_sweep(args, wl, ob, torch, table, hp, g, e, err_s, m, v, vf, bits_w, scales_w,
                  bits_s, scales_s, ws, status, stream, reps=8, rounds=3):
    """What the phase-1 access pattern costs on this machine, from committed
    kernels only: the real phase-1 kernel, interleaved with the pure-traffic
    kernel of its stream set (libonebit_ceiling.so) uncapped and at 1-4
    workgroups per CU, then that pattern's loads alone and its stores alone,
    a streaming read and a streaming copy.  Medians over `rounds` rounds of
    `reps` launches.  The stores-only kernel overwrites the state, so it
    runs last."""
    import ctypes
    lib = _ceiling_lib()
    C, N, W = wl.chunk, wl.N, wl.W
    n = (N // C) * C
    P = ctypes.c_void_p
    ga = (P * W)(*[t.data_ptr() for t in g])
    ea = (P * W)(*[t.data_ptr() for t in e])
    ba = (P * W)(*[t.data_ptr() for t in bits_w])
    st = stream.cuda_stream
    pbytes = n * (12 * W + 24) + (W + 1) * n // 8

    def pattern(mode, lds):
        return lambda: lib.onebit_ceiling_phase1(n, W, m.data_ptr(), ga, ea, ba, err_s.data_ptr(),
                                                 v.data_ptr(), vf.data_ptr(), bits_s.data_ptr(), 0,
                                                 mode, lds, st)

    def phase1():
        ob.onebit_lamb_compress_average(table, W, g, e, err_s, m, v, vf, bits_w, scales_w, bits_s,
                                        scales_s, hp, ws, status, stream)

    tmp = torch.empty(N, dtype=torch.float32, device="cuda")
    sink = torch.empty(N // 4096 + 1, dtype=torch.float32, device="cuda")
    cases = {"phase1_kernel": (phase1, phase1_bytes(wl.N, wl.K, C, W)),
             "pattern": (pattern(0, 0), pbytes)}
    for per_cu, lds in _LDS_CAPS.items():
        cases[f"pattern_{per_cu}_per_cu"] = (pattern(0, lds), pbytes)
    cases["pattern_loads_only"] = (pattern(1, 0), n * (8 * W + 16))
    cases["stream_read"] = (lambda: lib.onebit_ceiling_read(n, g[0].data_ptr(), sink.data_ptr(), st),
                            4 * n)
    cases["stream_copy"] = (lambda: lib.onebit_ceiling_copy(n, g[0].data_ptr(), tmp.data_ptr(), st),
                            8 * n)
    times = {k: [] for k in cases}
    for _ in range(rounds):
        for name, (fn, _) in cases.items():
            fn()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            for i in range(reps):
                ev[i].record(stream)
                fn()
            ev[reps].record(stream)
            torch.cuda.synchronize()
            times[name] += [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]
    # last: the stores alone (they overwrite the state)
    fn = pattern(2, 0)
    fn()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    for i in range(reps):
        ev[i].record(stream)
        fn()
    ev[reps].record(stream)
    torch.cuda.synchronize()
    times["pattern_stores_only"] = [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]
    sbytes = n * (4 * W + 8) + (W + 1) * n // 8
    out = {"metric": "phase-1 access pattern on this machine (pure-traffic kernels)",
           "workload": f"{wl.name}: N={N}, W={W}, chunk {C}", "unit": "ms, GB/s",
           "note": "medians; *_per_cu caps the resident workgroups per CU with dynamic LDS; "
                   "loads_only/stores_only are the pattern's reads or writes alone"}
    for name, ts in times.items():
        nbytes = cases[name][1] if name in cases else sbytes
        med = sorted(ts)[len(ts) // 2]
        out[name] = {"ms": med, "GBps": nbytes / (med * 1e-3) / 1e9}
        log(f"[sweep] {name:28s} {med:8.3f} ms  {nbytes / (med * 1e-3) / 1e9:7.0f} GB/s")
    out["mix_penalty"] = out["pattern"]["ms"] / (out["pattern_loads_only"]["ms"] +
                                                out["pattern_stores_only"]["ms"])
    out["phase1_frac_of_pattern"] = out["pattern"]["ms"] / out["phase1_kernel"]["ms"]
    print(json.dumps(out), flush=True)


def bench_adam(args, wl, ob, torch, hp, g, e, err_s, x, m, v, bits_w, scales_w, bits_s, scales_s,
               status, stream):
    """The 1-bit Adam mode on the same table, flattened: one
    onebit_adam_compressed_step per compression step, i.e. the allreduce
    kernel and the update kernel (v is the frozen variance)."""
    C, N, W, K = wl.chunk, wl.N, wl.W, wl.K

    def step(mm=m):
        ob.onebit_adam_compressed_step(N, C, W, g, e, err_s, x, mm, v, bits_w, scales_w, bits_s,
                                       scales_s, hp, status, stream)

    def timed(mm):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record(stream)
        for _ in range(args.steps):
            step(mm)
        ev[1].record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return (t1 - t0) * 1e3 / args.steps, ev[0].elapsed_time(ev[1]) / args.steps

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms_per_step, k_ms = timed(m)
    if int(status.item()):
        log(f"[bench] WARNING: status flags {int(status.item())}")
    log(f"[bench] adam {args.steps} steps: {ms_per_step:.3f} ms/step (kernels {k_ms:.3f} ms)")
    pm_ms, pm_k = timed(None)
    log(f"[bench] adam packed momentum {args.steps} steps: {pm_ms:.3f} ms/step "
        f"(kernels {pm_k:.3f} ms)")
    pm_bytes = adam_bytes(N, K, C, W) - 8 * N + K * (C // 8 + 4)

    for _ in range(2):
        ob.onebit_adam_warmup_step(N, W, g, x, m, v, hp, stream)
    wev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    wsteps = 5
    wev[0].record(stream)
    for _ in range(wsteps):
        ob.onebit_adam_warmup_step(N, W, g, x, m, v, hp, stream)
    wev[1].record(stream)
    torch.cuda.synchronize()
    warm_ms = wev[0].elapsed_time(wev[1]) / wsteps
    warm_bytes = N * (4 * W + 24)

    abytes = adam_bytes(N, K, C, W)
    achieved = abytes / (k_ms * 1e-3) / 1e9
    traffic = _measured_traffic("traffic_adam_step_bert_large.txt") \
        if wl.name == "bert_large" else None
    cpu = None
    if args.cpu_chunks > 0:
        log("[bench] CPU oracle baseline ...")
        cpu = cpu_baseline(wl, args.cpu_chunks, "adam")
        log(f"[bench] oracle: {cpu['value']:.3e} params/s ({cpu['sample']})")
    step_gbps = abytes / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": "params/sec and achieved HBM GB/s (% of peak) per 1-bit Adam step",
        "value": N / (ms_per_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name} (flattened): 1-bit Adam compression-stage step, "
                               f"N={N}, W={W} simulated workers, chunk {C}",
                   "N": N, "W": W, "chunk": C},
        "achieved_GBps": step_gbps,
        "frac_of_peak": step_gbps / PEAK_HBM_GBPS,
        "step_bytes": abytes,
        "warmup_step": {"ms": warm_ms, "params_per_s": N / (warm_ms * 1e-3),
                        "GBps": warm_bytes / (warm_ms * 1e-3) / 1e9, "bytes": warm_bytes},
        "packed_momentum": {
            "ms_per_step": pm_ms, "params_per_s": N / (pm_ms * 1e-3), "kernel_ms": pm_k,
            "step_bytes": pm_bytes, "GBps": pm_bytes / (pm_k * 1e-3) / 1e9,
            "note": "same step with m = NULL: the momentum is the previous server output, "
                    "outputs bit-identical"},
        "roofline": {"bound": "hbm",
                     "kernel": "k_adam_allreduce<4096> + k_adam_update<4096> (one call)",
                     "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic,
                     "algorithmic_bytes": abytes},
        "runtime_copy": _ceiling(torch, stream, achieved),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def share_bytes(N, K, C, W):
    """Algorithmic bytes of one GPU's share of a W-GPU step, per kernel:
    worker compression (g read, e read and written, m read, signs and
    scales written), serving 1/W of the chunks (W workers' signs and scales
    read, server error read and written, signs and scales written),
    receiver statistics (signs and scales, m and v_frozen read, v_fresh read
    and written) and the update (signs and scales, v_frozen read, x read and
    written, m written)."""
    pk = K * (C // 8 + 4)
    ks = -(-K // W)
    n_s = min(ks * C, N)
    pk_s = ks * (C // 8 + 4)
    return {"worker": 16 * N + pk, "server": (W + 1) * pk_s + 8 * n_s,
            "stats": 16 * N + pk, "update": 16 * N + pk}


def _time_calls(torch, stream, fns, reps):
    """Average HIP-event time of each call in fns, run in order reps times
    (after two untimed rounds)."""
    for _ in range(2):
        for f in fns:
            f()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(reps)]
    for ev in evs:
        ev[0].record(stream)
        for j, f in enumerate(fns):
            f()
            ev[j + 1].record(stream)
    torch.cuda.synchronize()
    return [sum(ev[j].elapsed_time(ev[j + 1]) for ev in evs) / reps for j in range(len(fns))]


def _other_shares(wl, ob, torch, table, hp, g, e, err_s, x, m, v, vf, bits_w, scales_w, bits_s,
                  scales_s, c_avg, status, stream, reps):
    """Context for the share bench: one GPU's share of a W-GPU 1-bit Adam
    step (its worker, 1/W of the chunks as server, onebit_adam_update) and
    of a sparse-stage step (onebit_sparse_worker, onebit_sparse_average on
    its range of transmitted values, onebit_sparse_update; one 64-element
    block of 64 per chunk), on the same buffers."""
    C, N, W, K = wl.chunk, wl.N, wl.W, wl.K
    ks = -(-K // W)
    n_s = min(ks * C, N)
    wq = ks * C // 32
    pk = K * (C // 8 + 4)
    pk_s = ks * (C // 8 + 4)
    worker = lambda: ob.onebit_worker_compress(N, C, g[0], e[0], m, None, None, bits_w[0],  # noqa
                                               scales_w[0], hp, status, stream)
    server = lambda: ob.onebit_average_packed(n_s, C, W, [b[:wq] for b in bits_w],  # noqa
                                              [s_[:ks] for s_ in scales_w], err_s[:n_s],
                                              bits_s[:wq], scales_s[:ks], status, stream)
    update = lambda: ob.onebit_adam_update(N, C, bits_s, scales_s, x, m, v, hp, stream)  # noqa
    t = _time_calls(torch, stream, [worker, server, update], reps)
    a_by = {"worker": 16 * N + pk, "server": (W + 1) * pk_s + 8 * n_s, "update": 16 * N + pk}
    a_ms = dict(zip(("worker", "server", "update"), t))
    adam = {"ms_per_step": sum(t), "kernel_ms": a_ms, "kernel_bytes": a_by,
            "GBps": sum(a_by.values()) / (sum(t) * 1e-3) / 1e9}
    log(f"[bench] adam share: {sum(t):.3f} ms/step (" +
        ", ".join(f"{k} {a_ms[k]:.3f}" for k in a_ms) + " ms)")
    per = 64                                  # one block of 64 transmitted per chunk
    sel = torch.from_numpy(wl.selection(0)).cuda()
    vals_w = [torch.zeros(K * per, dtype=torch.float32, device="cuda") for _ in range(W)]
    vals_s = torch.zeros(K * per, dtype=torch.float32, device="cuda")
    for w in range(1, W):                     # the other workers' values, filled once
        ob.onebit_sparse_worker(N, C, 1, sel, g[w], e[w], m, vals_w[w], hp, stream)
    s_worker = lambda: ob.onebit_sparse_worker(N, C, 1, sel, g[0], e[0], m, vals_w[0], hp,  # noqa
                                               stream)
    s_server = lambda: ob.onebit_sparse_average(ks * per, W, [t_[:ks * per] for t_ in vals_w],  # noqa
                                                vals_s[:ks * per], stream)
    s_update = lambda: ob.onebit_sparse_update(table, 1, sel, vals_s, x, m, v, vf, c_avg, hp,  # noqa
                                               status, stream)
    t = _time_calls(torch, stream, [s_worker, s_server, s_update], reps)
    f = per / C
    s_by = {"worker": int(16 * N + 4 * f * N + 4 * K), "server": 4 * (W + 1) * ks * per,
            "update": int(4 * N + 28 * f * N + 4 * K)}
    s_ms = dict(zip(("worker", "server", "update"), t))
    sparse = {"ms_per_step": sum(t), "kernel_ms": s_ms, "kernel_bytes": s_by,
              "GBps": sum(s_by.values()) / (sum(t) * 1e-3) / 1e9}
    log(f"[bench] sparse share: {sum(t):.3f} ms/step (" +
        ", ".join(f"{k} {s_ms[k]:.3f}" for k in s_ms) + " ms)")
    return adam, sparse


def bench_share(args, wl, ob, torch, table, hp, g, e, err_s, x, m, v, vf, bits_w, scales_w,
                bits_s, scales_s, c_avg, f_prev, c_out, ws, status, stream):
    """One GPU's share of a W-GPU 1-bit LAMB compression step at its real
    shape, the exchange left out: this GPU's worker compresses its momentum
    over the whole buffer, serves the first 1/W of the chunks (the other
    workers' packed chunks, as the all-to-all would deliver them, are the
    simulated workers' arrays), then forms the rescale statistics and
    updates its replica."""
    C, N, W, K = wl.chunk, wl.N, wl.W, wl.K
    ks = -(-K // W)                       # chunks this GPU serves: [0, ks)
    n_s = min(ks * C, N)
    wq = ks * C // 32
    # the other workers' packed chunks for this range, filled once
    for w in range(1, W):
        ob.onebit_worker_compress(N, C, g[w], e[w], m, None, None, bits_w[w], scales_w[w], hp,
                                  status, stream)
    names = ("worker", "server", "stats", "update")

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        ob.onebit_worker_compress(N, C, g[0], e[0], m, None, None, bits_w[0], scales_w[0], hp,
                                  status, stream)
        mark(1)
        ob.onebit_average_packed(n_s, C, W, [b[:wq] for b in bits_w], [s[:ks] for s in scales_w],
                                 err_s[:n_s], bits_s[:wq], scales_s[:ks], status, stream)
        mark(2)
        ob.onebit_lamb_rescale_stats(table, bits_s, scales_s, m, None, None, v, vf, hp, ws, stream)
        mark(3)
        ob.onebit_lamb_rescale_update(table, bits_s, scales_s, x, m, v, c_avg, f_prev, c_out, hp,
                                      ws, status, stream)
        mark(4)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if int(status.item()):
        log(f"[bench] WARNING: status flags {int(status.item())}")
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    k_ms = {nm: sum(ev[j].elapsed_time(ev[j + 1]) for ev in evs) / args.steps
            for j, nm in enumerate(names)}
    log(f"[bench] share {args.steps} steps: {ms_per_step:.3f} ms/step (" +
        ", ".join(f"{nm} {k_ms[nm]:.3f}" for nm in names) + " ms)")
    by = share_bytes(N, K, C, W)
    sbytes = sum(by.values())
    adam_share, sparse_share = _other_shares(wl, ob, torch, table, hp, g, e, err_s, x, m, v, vf,
                                             bits_w, scales_w, bits_s, scales_s, c_avg, status,
                                             stream, args.steps)
    achieved = by["worker"] / (k_ms["worker"] * 1e-3) / 1e9
    step_gbps = sbytes / (ms_per_step * 1e-3) / 1e9
    traffic = _measured_traffic("traffic_worker_compress_bert_large.txt") \
        if wl.name == "bert_large" else None
    out = {
        "metric": "params/sec and achieved HBM GB/s (% of peak) per GPU for one GPU's share of a "
                  "W-GPU 1-bit LAMB step (the exchange left out)",
        "value": N / (ms_per_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: one GPU's share of a {W}-GPU 1-bit LAMB compression "
                               f"step (its worker, 1/{W} of the chunks as server, its replica's "
                               f"update), N={N}, chunk {C}",
                   "N": N, "W": W, "chunk": C},
        "achieved_GBps": step_gbps,
        "frac_of_peak": step_gbps / PEAK_HBM_GBPS,
        "step_bytes": sbytes,
        "kernel_ms": k_ms,
        "kernel_bytes": by,
        "adam_share": adam_share,
        "sparse_share": sparse_share,
        "roofline": {"bound": "hbm", "kernel": "k_worker_compress<4096>",
                     "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic,
                     "algorithmic_bytes": by["worker"]},
        "runtime_copy": _ceiling(torch, stream, achieved),
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def bench_sparse(args, wl, ob, torch, table, hp, g, e, x, m, v, vf, c_avg, status, stream):
    """The SLAMB-style sparse stage on the same table: one fused kernel per
    step, a fresh seeded block selection per step (uploaded before timing)."""
    C, N, W, K, L = wl.chunk, wl.N, wl.W, wl.K, wl.L
    nsel = args.nsel
    per = nsel * 64
    vals_w = [torch.zeros(K * per, dtype=torch.float32, device="cuda") for _ in range(W)]
    vals_s = torch.zeros(K * per, dtype=torch.float32, device="cuda")
    total = args.warmup + args.steps
    sels = [torch.from_numpy(wl.selection(i)).cuda() for i in range(total)]
    torch.cuda.synchronize()

    def step(i):
        ob.onebit_sparse_compressed_step(table, W, nsel, sels[i], g, e, x, m, v, vf, c_avg, vals_w,
                                         vals_s, hp, status, stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.warmup, total):
        step(i)
    ev[1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if int(status.item()):
        log(f"[bench] WARNING: status flags {int(status.item())}")
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    k_ms = ev[0].elapsed_time(ev[1]) / args.steps
    log(f"[bench] sparse {args.steps} steps: {ms_per_step:.3f} ms/step (kernel {k_ms:.3f} ms)")
    abytes = sparse_bytes(N, K, C, W, nsel)
    achieved = abytes / (k_ms * 1e-3) / 1e9
    cpu = None
    if args.cpu_chunks > 0:
        log("[bench] CPU oracle baseline ...")
        cpu = cpu_baseline(wl, args.cpu_chunks, "sparse", nsel)
        log(f"[bench] oracle: {cpu['value']:.3e} params/s ({cpu['sample']})")
    step_gbps = abytes / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": "params/sec and achieved HBM GB/s (% of peak) per sparse-stage step",
        "value": N / (ms_per_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: SLAMB-style sparse compression step, {L} tensors, "
                               f"N={N}, W={W} simulated workers, chunk {C}, {nsel} of {C // 64} "
                               f"blocks transmitted",
                   "N": N, "W": W, "tensors": L, "chunk": C, "nsel": nsel},
        "achieved_GBps": step_gbps,
        "frac_of_peak": step_gbps / PEAK_HBM_GBPS,
        "step_bytes": abytes,
        "roofline": {"bound": "hbm", "kernel": "k_sparse_step<4096>",
                     "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": _measured_traffic("traffic_sparse_step_bert_large.txt")
                     if wl.name == "bert_large" and nsel == 1 else None,
                     "algorithmic_bytes": abytes},
        "runtime_copy": _ceiling(torch, stream, achieved),
        "cpu_baseline": cpu,
        "readings": "the sparse stage is a reading of the SLAMB page's abstract (a masked "
                    "momentum, error compensation on each worker, an element-wise rescale), "
                    "which gives no algorithm in detail; GPU and oracle agree on that reading",
    }
    print(json.dumps(out), flush=True)


def _kernel_sha():
    import hashlib
    h = hashlib.sha256()
    for p in ("communication_compressed_optimizer_amd/csrc/onebit_kernels.hpp",
              "communication_compressed_optimizer_amd/csrc/onebit.hip"):
        with open(os.path.join(ROOT, p), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _measured_traffic(name):
    """HBM bytes per launch of the dominant kernel from a committed counter
    summary, or None if the kernels changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for ln in fh:
            if ":" in ln and not ln.startswith("#"):
                k, v = ln.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha") != _kernel_sha():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


if __name__ == "__main__":
    main()
