#!/usr/bin/env python3
"""Benchmark of the Longformer sparse self-attention forward on one MI355X.

One step = one lf_attn_fwd call over the whole hot path (band tiles of
every dilation class, global-key columns, split global rows and their
combine) on one batch of seeded synthetic input already resident in HBM.

Prints one JSON line:
  value      useful TFLOP/s (4*d per allowed (query, key) pair) of the path
  roofline   the tile kernel against the bf16 dense MFMA peak (2.5 PFLOP/s)
  cpu_baseline  the fp64 oracle on the host cores (a baseline, not a target)

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

--profile-mode runs only W + K eager calls plus a copy of known size (the
calibration kernel for rocprofv3 HBM-byte counters) and prints no JSON.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HEADLINE = "bf16-b1h12t4096-r256-g1"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
SETTLE_MS = 100           # untimed graph replays before the timed one (clock ramp)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "tile_kernel_hbm_traffic.json")


def measured_traffic(workload):
    from sparse_long_sequence_lf_amd.profiling import kernel_sha
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or was taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload)
    if not e or e.get("kernel_sha") != kernel_sha():
        return None
    return e.get("hbm_bytes_per_launch")


def mfma_achievable_tflops(stream):
    """The dense bf16 MFMA rate this GPU reaches in a loop of nothing but
    MFMAs (libmfmapeak.so, built beside the library), or None if absent."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "sparse_long_sequence_lf_amd", "libmfmapeak.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.lf_mfma_peak_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.lf_mfma_peak_launch.restype = ctypes.c_int
    lib.lf_mfma_peak_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.lf_mfma_peak_flops.restype = ctypes.c_double
    blocks, iters = 256 * 8, 2048
    sptr = ctypes.c_void_p(stream.cuda_stream)
    if lib.lf_mfma_peak_launch(blocks, iters, None, sptr) != 0:
        return None
    torch.cuda.synchronize()
    best = None
    for _ in range(3):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        lib.lf_mfma_peak_launch(blocks, iters, None, sptr)
        b.record(stream)
        torch.cuda.synchronize()
        t = lib.lf_mfma_peak_flops(blocks, iters) / (a.elapsed_time(b) * 1e-3) / 1e12
        best = t if best is None else max(best, t)
    return best


def cpu_baseline(inp, flops, seconds):
    """The fp64 oracle, unmodified, on the host cores: whole-workload passes
    repeated until about `seconds` of wall time."""
    import oracle
    reps = 0
    t0 = time.perf_counter()
    threads = 0
    while True:
        _, threads = oracle.fwd(inp.q, inp.k, inp.v, inp.r, inp.dilation, inp.global_idx,
                                inp.key_padding_mask, return_threads=True, one_sided=inp.one_sided,
                                random_blocks=inp.random_blocks)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1024:
            break
    return {"value": flops * reps / el / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole workload ({inp.q.shape[0] * inp.q.shape[1] * inp.q.shape[2]} query rows), "
                      f"{reps} passes in {el:.1f} s, fp64"}


def global_rows_bytes(inp):
    """Algorithmic HBM bytes of the global rows alone: every valid K and V row
    of each (b, h) read once, plus the global rows' q read and out written."""
    B, H, T, d = inp.q.shape
    es = inp.q.element_size()
    lengths = inp.lengths if inp.lengths is not None else [T] * B
    if inp.key_padding_mask is not None and inp.lengths is None:
        lengths = [int((inp.key_padding_mask[b] == 0).sum()) for b in range(B)]
    n_g = len(set(inp.global_idx))
    return sum(lengths) * H * 2 * d * es + 2 * B * H * n_g * d * es


def bench_global_rows(args, lf, W, metrics):
    """lf_attn_fwd_global_rows on the workload (the global rows alone, the
    same tasks the whole forward runs for them): W warmup calls, SETTLE_MS of
    untimed calls, then K back-to-back calls timed with events on the call
    stream.  Bound: HBM (each global row group streams every valid K and V
    row of its head)."""
    import torch
    w = W.workload(args.workload)
    inp = W.make_inputs(w)
    if not inp.global_idx:
        raise SystemExit(f"{w.name} has no global rows")
    dev = torch.device("cuda:0")
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    kpm = None if inp.key_padding_mask is None else inp.key_padding_mask.to(dev)
    B, H, T, d = q.shape
    stream = torch.cuda.current_stream(dev)
    out = torch.zeros_like(q)
    G = list(inp.global_idx)

    def call():
        lf.attn_fwd_global_rows(q, k, v, G, key_padding_mask=kpm, out=out, stream=stream)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    n_untimed = args.warmup
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < SETTLE_MS:
        for _ in range(20):
            call()
        torch.cuda.synchronize()
        n_untimed += 20
    if args.profile_mode:
        for _ in range(args.steps):
            call()
        torch.cuda.synchronize()
        from sparse_long_sequence_lf_amd.profiling import COPY_BYTES
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"profile mode: {n_untimed} untimed global-row calls then {args.steps} of {w.name}, "
              f"one {COPY_BYTES} B copy", flush=True)
        return
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nbytes = global_rows_bytes(inp)
    gbps = nbytes / (ms * 1e-3) / 1e9
    traffic = measured_traffic(w.name + "-globalrows")
    line = {
        "metric": "HBM GB/s of the global rows alone (lf_attn_fwd_global_rows)", "value": round(gbps, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v; no dataset, no weights)",
        "config": {"workload": w.name, "pass": "global rows", "B": B, "H": H, "T": T, "d": d,
                   "n_global": len(set(G)), "padded": kpm is not None, "algorithmic_bytes": nbytes,
                   "timing": f"eager back-to-back calls after {n_untimed} untimed calls"},
        "roofline": {"bound": "hbm", "kernel": "tile_kernel, global-row tasks and their combine",
                     "achieved": round(gbps, 1), "peak": 8000.0, "unit": "GB/s", "frac": round(gbps / 8000.0, 4),
                     "traffic": traffic},
    }
    print(json.dumps(line), flush=True)


PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA


def bench_backward(args, lf, W, metrics):
    """The gradients on the workload, given the forward's output and lse
    (lf_attn_bwd_ex, as a training step calls it after its forward): W
    warmup calls, SETTLE_MS of untimed calls, then K back-to-back calls
    timed with events on the call stream; then K calls of lf_attn_bwd, which
    runs the forward itself.  Useful FLOPs: 10 d per allowed pair (s = q.k,
    dP = dy.v, dv, dq, dk), against the bf16 matrix-core peak."""
    import torch
    w = W.workload(args.workload)
    inp = W.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    dy = W.make_grad(inp, w.seed + 17).to(dev)
    kpm = None if inp.key_padding_mask is None else inp.key_padding_mask.to(dev)
    B, H, T, d = q.shape
    stream = torch.cuda.current_stream(dev)
    outs = tuple(torch.empty_like(q) for _ in range(3))
    lse = torch.empty(B, H, T, dtype=torch.float32, device=dev)
    y = lf.attn_fwd(q, k, v, inp.r, inp.dilation, inp.global_idx, key_padding_mask=kpm, lse=lse, stream=stream,
                    one_sided=inp.one_sided, random_blocks=inp.random_blocks)

    def call(given=True):
        lf.attn_bwd(q, k, v, dy, inp.r, inp.dilation, inp.global_idx, key_padding_mask=kpm, out=outs,
                    stream=stream, one_sided=inp.one_sided, random_blocks=inp.random_blocks,
                    y=y if given else None, lse=lse if given else None)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    n_untimed = args.warmup
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < SETTLE_MS:
        call()
        torch.cuda.synchronize()
        n_untimed += 1
    if args.profile_mode:
        for _ in range(args.steps):
            call()
        torch.cuda.synchronize()
        print(f"profile mode: {n_untimed} untimed backward calls then {args.steps} of {w.name}", flush=True)
        return

    def timed(given):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            call(given)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms = timed(True)
    ms_with_fwd = timed(False)
    pairs = metrics.useful_pairs(B, H, T, inp.r, inp.dilation, inp.global_idx, inp.key_padding_mask,
                                 one_sided=inp.one_sided, random_blocks=inp.random_blocks)
    flops = 10 * d * pairs
    tf = flops / (ms * 1e-3) / 1e12
    bf16 = w.dtype == "bf16"
    line = {
        "metric": "useful TFLOP/s of the backward pass (dq, dk, dv), 10 d FLOP per allowed pair",
        "value": round(tf, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "ms_per_step_with_forward": round(ms_with_fwd, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic (seeded N(0,1) q/k/v/dy; no dataset, no weights)",
        "config": {"workload": w.name, "pass": "backward", "B": B, "H": H, "T": T, "d": d, "r": inp.r,
                   "one_sided": inp.one_sided, "dilation": inp.dilation, "n_global": len(set(inp.global_idx)),
                   "n_rand": 0 if inp.random_blocks is None else int(inp.random_blocks.shape[2]),
                   "padded": inp.key_padding_mask is not None, "useful_pairs": pairs,
                   "timing": f"eager back-to-back calls after {n_untimed} untimed calls; value and "
                             "ms_per_step with the forward's output and lse given (lf_attn_bwd_ex), "
                             "ms_per_step_with_forward running it too (lf_attn_bwd)"},
        "roofline": {"bound": "mfma" if bf16 else "alu",
                     "kernel": "whole call: statistics, global rows and keys, dq and dk/dv band kernels",
                     "achieved": round(tf, 3), "peak": PEAK_BF16_TFLOPS if bf16 else 157.3, "unit": "TFLOP/s",
                     "frac": round(tf / (PEAK_BF16_TFLOPS if bf16 else 157.3), 4), "traffic": None,
                     "algorithmic_flops": flops},
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-mode", action="store_true")
    ap.add_argument("--global-rows", action="store_true",
                    help="time lf_attn_fwd_global_rows (the global rows alone) on the workload")
    ap.add_argument("--backward", action="store_true",
                    help="time lf_attn_bwd (dq, dk, dv) on the workload instead of the forward")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only; --gpus must be 1 "
              "(sharding the (batch, head) pairs across GPUs is not built)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_long_sequence_lf_amd as lf
    from sparse_long_sequence_lf_amd import metrics
    from sparse_long_sequence_lf_amd import workloads as W

    if args.global_rows:
        torch.cuda.set_device(0)
        bench_global_rows(args, lf, W, metrics)
        return

    if args.backward:
        torch.cuda.set_device(0)
        bench_backward(args, lf, W, metrics)
        return

    w = W.workload(args.workload)
    inp = W.make_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    kpm = None if inp.key_padding_mask is None else inp.key_padding_mask.to(dev)
    B, H, T, d = q.shape
    stream = torch.cuda.current_stream(dev)
    call = lf.Prepared(q, k, v, inp.r, inp.dilation, inp.global_idx, kpm, stream=stream,
                       one_sided=inp.one_sided, random_blocks=inp.random_blocks)

    if args.profile_mode:
        # warmup calls, then more untimed calls for at least SETTLE_MS (the
        # clock ramp), then the K calls a profile's steady-state figure uses
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        n_untimed = args.warmup
        t_settle = time.perf_counter()
        while (time.perf_counter() - t_settle) * 1e3 < SETTLE_MS:
            for _ in range(20):
                call()
            torch.cuda.synchronize()
            n_untimed += 20
        for _ in range(args.steps):
            call()
        torch.cuda.synchronize()
        from sparse_long_sequence_lf_amd.profiling import COPY_BYTES
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"profile mode: {n_untimed} untimed calls then {args.steps} calls of {w.name}, "
              f"one {COPY_BYTES} B copy", flush=True)
        return

    pairs = metrics.useful_pairs(B, H, T, inp.r, inp.dilation, inp.global_idx, inp.key_padding_mask,
                                 one_sided=inp.one_sided, random_blocks=inp.random_blocks)
    flops = 4 * d * pairs

    # eager: back-to-back calls, events on the call stream (after the warmup
    # calls and SETTLE_MS more of untimed calls for the clock ramp)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < SETTLE_MS:
        for _ in range(20):
            call()
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_eager = e0.elapsed_time(e1) / args.steps
    ref_out = call.out.clone()

    # the same K calls captured in one HIP graph and replayed (no host launch gaps)
    ms_graph = None
    graph_ok = False
    settle_replays = 0
    try:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            gcall = lf.Prepared(q, k, v, inp.r, inp.dilation, inp.global_idx, kpm, out=call.out, stream=side,
                                one_sided=inp.one_sided, random_blocks=inp.random_blocks)
            gcall()   # the workspace for this stream is allocated outside capture
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=side):
                for _ in range(args.steps):
                    gcall()
        torch.cuda.synchronize()
        call.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        graph_ok = torch.equal(call.out, ref_out)
        # The GPU's clock rises over the first tens of milliseconds of
        # sustained load: untimed replays of the same graph for at least
        # SETTLE_MS come first, so that the timed replay sees the steady clock.
        t_settle = time.perf_counter()
        while True:
            g.replay()
            torch.cuda.synchronize()
            settle_replays += 1
            if (time.perf_counter() - t_settle) * 1e3 >= SETTLE_MS:
                break
        e2 = torch.cuda.Event(enable_timing=True)
        e3 = torch.cuda.Event(enable_timing=True)
        e2.record(stream)
        g.replay()
        e3.record(stream)
        torch.cuda.synchronize()
        ms_graph = e2.elapsed_time(e3) / args.steps
    except Exception as ex:  # graph capture is an optimisation of the timing loop only
        print(f"bench.py: graph capture unavailable ({ex}); reporting the eager loop", file=sys.stderr)

    # per-launch event pairs (each includes the launch's own dispatch gap):
    # reported beside the timed-region figure, not used for the roofline
    n_each = min(args.steps, 200)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_each)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    ms_launch = sum(a.elapsed_time(b) for a, b in ev) / n_each

    # cold caches: before each timed call, 512 MiB are written so that the
    # L2s and the MALL hold none of q, k, v; the events bracket the call only
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    n_cold = min(args.steps, 20)
    evc = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_cold)]
    torch.cuda.synchronize()
    for a, b in evc:
        flush.zero_()
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    ms_cold = sum(a.elapsed_time(b) for a, b in evc) / n_cold
    del flush
    achievable = mfma_achievable_tflops(stream)

    use_graph = ms_graph is not None and graph_ok
    ms = ms_graph if use_graph else ms_eager
    tflops = flops / (ms * 1e-3) / 1e12
    # The tile kernel's average duration: the timed region (events on the
    # call stream around K back-to-back calls) over K.  bf16 calls launch the
    # tile kernel alone; fp32 calls also run the hi/lo plane split first, so
    # there the figure is an upper bound on the tile kernel's own duration.
    ms_kernel = ms

    traffic = measured_traffic(w.name)
    line = {
        "metric": "useful TFLOP/s + % bf16 MFMA peak, sliding-window+global attn fwd T=4096",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) q/k/v; no dataset, no weights)",
        "config": {"workload": w.name, "B": B, "H": H, "T": T, "d": d, "r": inp.r,
                   "one_sided": inp.one_sided,
                   "n_rand": 0 if inp.random_blocks is None else int(inp.random_blocks.shape[2]),
                   "dilation": inp.dilation, "n_global": len(set(inp.global_idx)),
                   "padded": inp.key_padding_mask is not None, "useful_pairs": pairs,
                   "useful_gflop": round(flops / 1e9, 4), "parallelism": "single GPU",
                   "timing": (f"hip graph of K calls, timed after {settle_replays} untimed replays "
                              f"(>= {SETTLE_MS} ms of load to settle the clock)") if use_graph
                             else "eager back-to-back calls"},
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "ms_per_step_eager": round(ms_eager, 5),
        "ms_per_step_graph": None if ms_graph is None else round(ms_graph, 5),
        "ms_per_step_cold": round(ms_cold, 5),
        "wall_s_eager_loop": round(wall, 4),
        "roofline": {"bound": "mfma", "kernel": "lfk::tile_kernel",
                     "achieved": round(flops / (ms_kernel * 1e-3) / 1e12, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops / (ms_kernel * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "kernel_us": round(ms_kernel * 1e3, 3),
                     "kernel_us_source": "timed region / K" + (" (includes the fp32 plane split)" if w.dtype != "bf16" else ""),
                     "launch_us_event_pairs": round(ms_launch * 1e3, 3),
                     "achievable_peak": None if achievable is None else round(achievable, 1),
                     "frac_of_achievable": None if achievable is None else
                     round(flops / (ms_kernel * 1e-3) / 1e12 / achievable, 4),
                     "algorithmic_flops": flops,
                     "algorithmic_bytes": metrics.algorithmic_bytes(B, H, T, d, q.element_size(),
                                                                    inp.key_padding_mask)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, flops, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
