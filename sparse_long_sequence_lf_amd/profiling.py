"""Summaries of rocprofv3 output for the tile kernel (the text files under
profiles/ and the HBM-traffic record bench.py reads).

    python -m sparse_long_sequence_lf_amd.profiling stats DIR --workload W --cmd "..." --out FILE
    python -m sparse_long_sequence_lf_amd.profiling traffic FETCH_DIR WRITE_DIR --workload W \
        --cmd "..." --out-json profiles/tile_kernel_hbm_traffic.json --out-txt FILE
    python -m sparse_long_sequence_lf_amd.profiling counters DIR --workload W --cmd "..." --out FILE \
        [--useful-flops F --kernel-us U --hbm-bytes B]
    python -m sparse_long_sequence_lf_amd.profiling take --workload W [--backward] [--out-dir profiles]

`take` runs the rocprofv3 passes itself (each a child process under a time
limit) and writes every summary of the workload.

DIR, FETCH_DIR, WRITE_DIR are rocprofv3 output directories written with
`-f csv` (kernel trace with --stats; one --pmc FETCH_SIZE run; one --pmc
WRITE_SIZE run) of `bench.py --profile-mode`, whose calls end with one copy of
COPY_BYTES bytes.  FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the tile
kernel are scaled by what the same counter reads for that copy: a copy of N
bytes fetches N and writes N.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import subprocess
import sys
from types import SimpleNamespace
from typing import Dict, List

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
# the kernels and the host code that plans their tasks (the plan decides
# what a launch runs: split counts, task order)
KERNEL_SOURCES = ["sparse_long_sequence_lf_amd/csrc/lf_fwd_kernels.hip",
                  "sparse_long_sequence_lf_amd/csrc/lf_host.cpp",
                  "sparse_long_sequence_lf_amd/csrc/lf_kernels.h",
                  "sparse_long_sequence_lf_amd/csrc/lf_device.h",
                  "sparse_long_sequence_lf_amd/csrc/lf_decode.h"]
BWD_SOURCES = ["sparse_long_sequence_lf_amd/csrc/lf_bwd_mfma.hip",
               "sparse_long_sequence_lf_amd/csrc/lf_bwd_kernels.hip",
               "sparse_long_sequence_lf_amd/csrc/lf_bwd.h"] + KERNEL_SOURCES
KERNEL_NAME = "tile_kernel"
COPY_BYTES = 1 << 28   # the calibration copy in bench.py --profile-mode


def kernel_sha(sources=None) -> str:
    """Digest of the kernel sources: a traffic record taken on other sources is stale."""
    h = hashlib.sha256()
    for p in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise SystemExit(f"no file matches {pattern}")
    return hits[0]


def kernel_durations(d: str) -> Dict[str, List[int]]:
    """Kernel name -> list of dispatch durations (ns) from a kernel trace."""
    out: Dict[str, List[int]] = {}
    with open(_one(os.path.join(d, "**", "*kernel_trace.csv"))) as f:
        for r in csv.DictReader(f):
            out.setdefault(r["Kernel_Name"], []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return out


def counter_per_dispatch(d: str, counter: str) -> Dict[int, tuple]:
    """Dispatch id -> (kernel name, counter value summed over its instances)."""
    out: Dict[int, list] = {}
    with open(_one(os.path.join(d, "**", "*counter_collection.csv"))) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            e = out.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], 0.0])
            e[1] += float(r["Counter_Value"])
    return {k: tuple(v) for k, v in out.items()}


def _copy_value(vals: Dict[int, tuple]) -> float:
    # the calibration copy is the largest non-tile dispatch of the run
    cands = [v for (name, v) in vals.values() if KERNEL_NAME not in name]
    if not cands:
        raise SystemExit("no calibration copy dispatch found")
    return max(cands)


def cmd_stats(a) -> None:
    durs = kernel_durations(a.dir)
    lines = [f"# rocprofv3 kernel trace: {a.workload}", "", "command:", f"    {a.cmd}", "",
             f"{'kernel':70s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
    for name, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        short = name if len(name) <= 70 else name[:67] + "..."
        lines.append(f"{short:70s} {len(v):6d} {statistics.mean(v) / 1e3:9.2f} {min(v) / 1e3:9.2f} {max(v) / 1e3:9.2f}")
    tile = [x for n, v in durs.items() if KERNEL_NAME in n for x in v]
    steady_us = None
    if getattr(a, "backward", False):
        bwd = {n: v for n, v in durs.items() if "bwd" in n or "lfb" in n}
        lines += ["", "The tile_kernel line is the one forward call that makes the output and lse handed to every",
                  f"backward call.  Sum of the backward kernels' averages: "
                  f"{sum(statistics.mean(v) for v in bwd.values()) / 1e3:.2f} us per call.",
                  f"backward kernel sources sha: {kernel_sha(BWD_SOURCES)}"]
        tile = []
    if tile:
        steady = tile[a.skip:] if len(tile) > a.skip else tile
        lines += ["", f"tile kernel average duration: {statistics.mean(tile) / 1e3:.2f} us over {len(tile)} dispatches",
                  f"tile kernel steady-state average (first {a.skip} dispatches, the untimed warmup and clock-settle calls, left out): "
                  f"{statistics.mean(steady) / 1e3:.2f} us over {len(steady)}, median {statistics.median(steady) / 1e3:.2f} us",
                  f"kernel sources sha: {kernel_sha()}"]
        steady_us = statistics.mean(steady) / 1e3
    text = "\n".join(lines) + "\n"
    with open(a.out, "w") as f:
        f.write(text)
    sys.stdout.write(text)
    return steady_us


def cmd_traffic(a) -> None:
    fetch = counter_per_dispatch(a.fetch_dir, "FETCH_SIZE")
    write = counter_per_dispatch(a.write_dir, "WRITE_SIZE")
    f_copy, w_copy = _copy_value(fetch), _copy_value(write)
    f_scale = COPY_BYTES / (f_copy * 1024.0)
    w_scale = COPY_BYTES / (w_copy * 1024.0)
    f_tile = [v for (n, v) in fetch.values() if KERNEL_NAME in n]
    w_tile = [v for (n, v) in write.values() if KERNEL_NAME in n]
    if not f_tile or not w_tile:
        raise SystemExit("no tile kernel dispatches in the counter runs")
    fetch_b = statistics.mean(f_tile) * 1024.0 * f_scale
    write_b = statistics.mean(w_tile) * 1024.0 * w_scale
    rec = {"kernel_sha": kernel_sha(), "hbm_bytes_per_launch": int(round(fetch_b + write_b)),
           "fetch_bytes": int(round(fetch_b)), "write_bytes": int(round(write_b)),
           "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5),
           "dispatches": [len(f_tile), len(w_tile)], "command": a.cmd}
    table = {}
    if os.path.exists(a.out_json):
        with open(a.out_json) as f:
            table = json.load(f)
    table[a.workload] = rec
    with open(a.out_json, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")
    text = (f"# HBM traffic of the tile kernel: {a.workload}\n\ncommand (one run per counter):\n    {a.cmd}\n\n"
            f"calibration copy of {COPY_BYTES} B: FETCH_SIZE {f_copy:.0f} KiB, WRITE_SIZE {w_copy:.0f} KiB\n"
            f"scale factors (bytes per counted KiB / 1024): fetch {f_scale:.5f}, write {w_scale:.5f}\n\n"
            f"tile kernel per launch ({len(f_tile)} / {len(w_tile)} dispatches):\n"
            f"    fetched {fetch_b / 1e6:.3f} MB, written {write_b / 1e6:.3f} MB, total {(fetch_b + write_b) / 1e6:.3f} MB\n"
            f"kernel sources sha: {kernel_sha()}\n")
    with open(a.out_txt, "w") as f:
        f.write(text)
    sys.stdout.write(text)
    return fetch_b + write_b


COUNTER_SET = ["MfmaUtil", "VALUBusy", "SALUBusy", "MfmaFlopsBF16", "LDSBankConflict"]


def cmd_counters(a) -> None:
    """Utilisation counters of the tile kernel (median over its dispatches),
    next to the useful work of one launch."""
    vals: Dict[int, Dict[str, float]] = {}
    names: Dict[int, str] = {}
    with open(_one(os.path.join(a.dir, "**", "*counter_collection.csv"))) as f:
        for r in csv.DictReader(f):
            d = int(r["Dispatch_Id"])
            names[d] = r["Kernel_Name"]
            vals.setdefault(d, {}).setdefault(r["Counter_Name"], 0.0)
            vals[d][r["Counter_Name"]] += float(r["Counter_Value"])
    tile = [v for d, v in vals.items() if KERNEL_NAME in names[d]]
    if not tile:
        raise SystemExit("no tile kernel dispatches in the counter run")
    med = {k: statistics.median(v[k] for v in tile if k in v) for k in tile[0]}
    lines = [f"# rocprofv3 utilisation counters of the tile kernel: {a.workload}", "", "command:", f"    {a.cmd}", "",
             f"median over {len(tile)} dispatches (rocprofv3's derived metrics of this GPU):"]
    for k in sorted(med):
        lines.append(f"    {k:18s} {med[k]:16.4f}")
    if "MfmaFlopsBF16" in med and a.useful_flops:
        lines += ["", f"useful FLOPs per launch (the allowed (query, key) pairs x 4 d): {a.useful_flops:.4e}",
                  f"MFMA FLOPs issued per launch: {med['MfmaFlopsBF16']:.4e} "
                  f"(useful share {a.useful_flops / med['MfmaFlopsBF16']:.3f}; the rest is masked or padded "
                  f"work inside 32x32 blocks)"]
    if a.kernel_us and a.hbm_bytes:
        lines.append(f"HBM traffic {a.hbm_bytes / 1e6:.2f} MB per launch over {a.kernel_us:.2f} us: "
                     f"{a.hbm_bytes / (a.kernel_us * 1e-6) / 1e9:.0f} GB/s")
    lines.append(f"kernel sources sha: {kernel_sha()}")
    text = "\n".join(lines) + "\n"
    with open(a.out, "w") as f:
        f.write(text)
    sys.stdout.write(text)


def _profile_run(a, work, tag, prof_args, steps, warmup):
    """One rocprofv3 run of bench.py --profile-mode (a child process, under
    `timeout -s KILL`); returns its output directory, the untimed calls
    bench.py reported and the command as the summaries state it."""
    d = os.path.join(work, f"{_name(a)}{'_bwd' if a.backward else ''}_{tag}")
    tail = ["--profile-mode", "--workload", a.workload, "--steps", str(steps), "--warmup", str(warmup)]
    if a.backward:
        tail.insert(0, "--backward")
    if a.global_rows:
        tail.insert(0, "--global-rows")
    cmd = ["timeout", "-s", "KILL", str(a.timeout), "rocprofv3", *prof_args, "-f", "csv", "-d", d, "-o", tag, "--",
           sys.executable, os.path.join(ROOT, "bench.py"), *tail]
    shown = f"cd /tmp && rocprofv3 {' '.join(prof_args)} -f csv -d <out> -o {tag} -- python3 <repo>/bench.py {' '.join(tail)}"
    print(f"step: {tag}: {shown}", flush=True)
    p = subprocess.run(cmd, cwd="/tmp", env=dict(os.environ, TMPDIR="/tmp"), capture_output=True, text=True)
    with open(d + ".log", "w") as f:
        f.write(p.stdout + p.stderr)
    done = [ln for ln in p.stdout.splitlines() if ln.startswith("profile mode:")]
    if not done:
        raise SystemExit(f"{tag}: bench.py did not finish (exit {p.returncode}); see {d}.log")
    if p.returncode != 0:
        # rocprofv3 itself can exit abnormally after a complete run
        print(f"  note: rocprofv3 exited {p.returncode} after bench.py finished", flush=True)
    return d, int(done[0].split()[2]), shown


def _name(a) -> str:
    """The workload's name in the summaries (-globalrows: the global rows alone)."""
    return a.workload + ("-globalrows" if a.global_rows else "")


def cmd_take(a) -> None:
    """Kernel trace, HBM bytes (FETCH_SIZE, then WRITE_SIZE) and utilisation
    counters of one workload, each from its own rocprofv3 run, and their
    summaries under --out-dir."""
    from sparse_long_sequence_lf_amd import metrics
    from sparse_long_sequence_lf_amd import workloads as W
    work = os.path.abspath(a.work_dir)
    out = os.path.abspath(a.out_dir)
    os.makedirs(work, exist_ok=True)
    os.makedirs(out, exist_ok=True)
    made_by = f"python -m sparse_long_sequence_lf_amd.profiling take --workload {a.workload}" + \
        (" --backward" if a.backward else "") + (" --global-rows" if a.global_rows else "")
    name = _name(a)
    if a.backward:
        d, skip, shown = _profile_run(a, work, "kt", ["--kernel-trace", "--stats"], 20, 3)
        cmd_stats(SimpleNamespace(dir=d, workload=a.workload + " (backward)", cmd=f"{shown}\n    (run by: {made_by})",
                                  out=os.path.join(out, f"bwd_kernels_{a.workload}_trace.txt"), skip=0,
                                  backward=True))
        return
    d, skip, shown = _profile_run(a, work, "kt", ["--kernel-trace", "--stats"], 50, 10)
    kernel_us = cmd_stats(SimpleNamespace(dir=d, workload=name, cmd=f"{shown}\n    (run by: {made_by})",
                                          out=os.path.join(out, f"tile_kernel_{name}_trace.txt"), skip=skip))
    fd, _, shown_f = _profile_run(a, work, "f", ["--pmc", "FETCH_SIZE"], 10, 2)
    wd, _, _ = _profile_run(a, work, "w", ["--pmc", "WRITE_SIZE"], 10, 2)
    hbm = cmd_traffic(SimpleNamespace(fetch_dir=fd, write_dir=wd, workload=name,
                                      cmd=shown_f.replace("--pmc FETCH_SIZE", "--pmc FETCH_SIZE (then WRITE_SIZE)") +
                                      f"\n    (run by: {made_by})",
                                      out_json=os.path.join(out, "tile_kernel_hbm_traffic.json"),
                                      out_txt=os.path.join(out, f"tile_kernel_{name}_hbm.txt")))
    ud, _, shown_u = _profile_run(a, work, "u", ["--pmc", *COUNTER_SET], 10, 2)
    w = W.workload(a.workload)
    inp = W.make_inputs(w)
    B, H, T, dd = inp.q.shape
    useful = 0.0
    if not a.global_rows:
        pairs = metrics.useful_pairs(B, H, T, inp.r, inp.dilation, inp.global_idx, inp.key_padding_mask,
                                     one_sided=inp.one_sided, random_blocks=inp.random_blocks)
        useful = 4.0 * dd * pairs
    cmd_counters(SimpleNamespace(dir=ud, workload=name, cmd=f"{shown_u}\n    (run by: {made_by})",
                                 out=os.path.join(out, f"tile_kernel_{name}_util.txt"),
                                 useful_flops=useful, kernel_us=kernel_us or 0.0, hbm_bytes=hbm))
    if a.global_rows:
        sys.path.insert(0, ROOT)
        import bench
        alg = bench.global_rows_bytes(inp)
        text = (f"# HBM rate of the global rows alone: {a.workload}\n\n"
                f"lf_attn_fwd_global_rows runs the global-row tasks of the tile kernel (the same tasks, and\n"
                f"the same combine, as the whole forward runs for those rows) and nothing else.\n\n"
                f"run by: {made_by}\n\n"
                f"tile kernel steady-state average: {kernel_us:.2f} us per launch\n"
                f"algorithmic bytes (every valid K and V row of each (b, h) once, plus the global rows'\n"
                f"q read and out written): {alg / 1e6:.3f} MB -> {alg / (kernel_us * 1e-6) / 1e9:.0f} GB/s\n"
                f"counter bytes (FETCH_SIZE + WRITE_SIZE, scaled by the calibration copy): {hbm / 1e6:.3f} MB -> "
                f"{hbm / (kernel_us * 1e-6) / 1e9:.0f} GB/s ({hbm / alg:.2f} x algorithmic)\n"
                f"kernel sources sha: {kernel_sha()}\n")
        with open(os.path.join(out, "global_rows_hbm_rate.txt"), "w") as f:
            f.write(text)
        sys.stdout.write(text)

def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--workload", required=True)
    s.add_argument("--cmd", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--skip", type=int, default=0, help="leading tile dispatches (untimed warmup and clock-settle calls) left out of the steady-state figures")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--workload", required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--out-json", required=True)
    t.add_argument("--out-txt", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--workload", required=True)
    c.add_argument("--cmd", required=True)
    c.add_argument("--out", required=True)
    c.add_argument("--useful-flops", type=float, default=0.0)
    c.add_argument("--kernel-us", type=float, default=0.0)
    c.add_argument("--hbm-bytes", type=float, default=0.0)
    k = sub.add_parser("take")
    k.add_argument("--workload", required=True)
    k.add_argument("--backward", action="store_true", help="kernel trace of the backward call only")
    k.add_argument("--global-rows", action="store_true", help="the global rows alone (lf_attn_fwd_global_rows)")
    k.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"))
    k.add_argument("--work-dir", default=os.path.join(ROOT, "gpurun_out", "prof"))
    k.add_argument("--timeout", type=int, default=150, help="seconds per rocprofv3 run")
    a = ap.parse_args(argv)
    {"stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters, "take": cmd_take}[a.what](a)


if __name__ == "__main__":
    main()
