"""Summarise rocprofv3 CSV output into the short text kept under profiles/.

  python -m speculative_pipeline_decoding_amd.profile_summary stats DIR \
         [--kernel K --group G --skip S]
      per-kernel dispatch count, total and average duration (kernel trace); with
      --kernel, also K's average over one phase of the run (below)
  python -m speculative_pipeline_decoding_amd.profile_summary traffic FETCH_DIR WRITE_DIR \
         --calib-mib 1024 [--kernel gemv_gate_up --group G --skip S]
      FETCH_SIZE and WRITE_SIZE per dispatch (KiB), each scaled by what the same
      counter reads for a plain device-to-device copy of known size (the largest
      copy dispatch in the run, of --calib-mib MiB), as HBM bytes per launch; the
      kernel's bytes per launch are taken over one phase.

A phase of a kernel is the run of its dispatches between two prefills (any prefill
GEMM dispatch ends one): in bench.py's default run, phase 0 holds the headline steps,
phase 1 the same steps replayed with per-launch events (what its kernel table and
roofline time), phase 2 the autoregressive reference. --skip drops the phase's
warm-up dispatches.

  python -m speculative_pipeline_decoding_amd.profile_summary mfma COUNTER_DIR TRACE_DIR
      per kernel with matrix-core work: bf16 MFMA flops per dispatch (MfmaFlopsBF16),
      their rate over the kernel-trace mean duration, and MfmaUtil.

Every summary records the SHA-256 of the GEMV source it measured, so a later
reader can tell whether the numbers still describe the current kernel.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
GEMV_SOURCE = os.path.join(HERE, "csrc", "gemv.hip")


def source_hash(path: str = GEMV_SOURCE) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def short_name(n: str) -> str:
    n = n.replace("spd::(anonymous namespace)::", "").replace("void ", "")
    n = n.replace("unsigned short", "bf16")
    base = n.split("(")[0]
    return base[:60]


def _find(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits[0]


def kernel_durations(trace_dir: str):
    rows = list(csv.DictReader(open(_find(trace_dir, "kernel_trace.csv"))))
    agg = collections.defaultdict(list)
    for r in rows:
        agg[short_name(r["Kernel_Name"])].append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return agg


def _matches(name: str, kernel: str) -> bool:
    """A kernel given by its full short name, or by its base name: every instantiation
    (a GEMV role's launches take different kernel kinds as their vector counts change)."""
    return name == kernel or ("<" not in kernel and name.startswith(kernel + "<"))


def _phase(values, names, kernel, group, skip, sep="gemm_x3_kernel"):
    """Values of one kernel's dispatches in one phase of a run, in dispatch order: phases
    are the runs of that kernel's dispatches between prefills (any `sep` dispatch ends a
    phase); `skip` leading dispatches of the phase are dropped (the warm-up steps)."""
    phases, cur = [], []
    for n, v in zip(names, values):
        if n == sep:
            if cur:
                phases.append(cur)
                cur = []
        elif _matches(n, kernel):
            cur.append(v)
    if cur:
        phases.append(cur)
    if group >= len(phases):
        raise SystemExit(f"{kernel}: {len(phases)} phases, no phase {group}")
    return phases[group][skip:]


def trace_sequence(trace_dir: str):
    """(kernel names, durations in us) of every dispatch, in dispatch order."""
    rows = sorted(csv.DictReader(open(_find(trace_dir, "kernel_trace.csv"))),
                  key=lambda r: int(r["Dispatch_Id"]))
    return ([short_name(r["Kernel_Name"]) for r in rows],
            [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows])


def counter_sequence(d: str, counter: str):
    """(kernel names, values) of one counter over every dispatch, in dispatch order."""
    rows = sorted((r for r in csv.DictReader(open(_find(d, "counter_collection.csv")))
                   if r["Counter_Name"] == counter), key=lambda r: int(r["Dispatch_Id"]))
    return [short_name(r["Kernel_Name"]) for r in rows], [float(r["Counter_Value"]) for r in rows]


def _kernel_label(names, kernel):
    hits = sorted({n for n in names if _matches(n, kernel)})
    if not hits:
        raise SystemExit(f"no dispatch of {kernel}")
    return hits[0] if len(hits) == 1 else f"{kernel} ({', '.join(hits)})"


def counter_values(d: str, counter: str):
    rows = list(csv.DictReader(open(_find(d, "counter_collection.csv"))))
    agg = collections.defaultdict(list)
    for r in rows:
        if r["Counter_Name"] == counter:
            agg[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return agg


def cmd_stats(a):
    agg = kernel_durations(a.dir)
    tot = sum(sum(v) for v in agg.values())
    print(f"gemv source sha256[:16]: {source_hash()}")
    print(f"{'kernel':62s} {'calls':>7s} {'total_ms':>10s} {'avg_us':>9s} {'share':>6s}")
    for k, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        print(f"{k:62s} {len(v):7d} {sum(v) / 1e3:10.3f} {sum(v) / len(v):9.2f} {100 * sum(v) / tot:5.1f}%")
    if a.kernel:
        names, durs = trace_sequence(a.dir)
        k = _kernel_label(names, a.kernel)
        v = _phase(durs, names, a.kernel, a.group, a.skip)
        print(f"phase {a.group} of {k} (dispatches after {a.skip} warm-up ones): "
              f"{len(v)} calls, avg_us {sum(v) / len(v):.2f}")


def cmd_traffic(a):
    f = counter_values(a.fetch_dir, "FETCH_SIZE")
    w = counter_values(a.write_dir, "WRITE_SIZE")
    copy_name = next((k for k in f if "copyBuffer" in k), None)
    if copy_name is None:
        raise SystemExit("no copy dispatch in the FETCH_SIZE run (pass --calib-copy-mib to bench.py)")
    known = a.calib_mib * 1024.0           # KiB moved each way by the calibration copy
    fscale = known / max(f[copy_name])
    wscale = known / max(w[copy_name])
    print(f"gemv source sha256[:16]: {source_hash()}")
    print(f"calibration copy {a.calib_mib} MiB: FETCH_SIZE reads {max(f[copy_name]):.1f} KiB "
          f"(scale {fscale:.4f}), WRITE_SIZE reads {max(w[copy_name]):.1f} KiB (scale {wscale:.4f})")
    print(f"{'kernel':62s} {'calls':>6s} {'fetch_MB':>10s} {'write_MB':>9s} (per dispatch, scaled)")
    for k in sorted(f, key=lambda k: -sum(f[k])):
        fv, wv = f[k], w.get(k, [0.0])
        fb = sum(fv) / len(fv) * 1024 * fscale
        wb = sum(wv) / len(wv) * 1024 * wscale
        print(f"{k:62s} {len(fv):6d} {fb / 1e6:10.2f} {wb / 1e6:9.2f}")
    if a.kernel:
        fn, fv = counter_sequence(a.fetch_dir, "FETCH_SIZE")
        wn, wv = counter_sequence(a.write_dir, "WRITE_SIZE")
        k = _kernel_label(fn, a.kernel)
        fp = _phase(fv, fn, a.kernel, a.group, a.skip)
        wp = _phase(wv, wn, a.kernel, a.group, a.skip)
        fb = sum(fp) / len(fp) * 1024 * fscale
        wb = sum(wp) / len(wp) * 1024 * wscale
        print(f"phase {a.group} of {k} (dispatches after {a.skip} warm-up ones): {len(fp)} calls, "
              f"fetch_MB {fb / 1e6:.2f}, write_MB {wb / 1e6:.2f}")
        print(f"traffic_bytes_per_launch {k} {fb + wb:.0f}")


def cmd_mfma(a):
    """Matrix-core use per kernel: MfmaFlopsBF16 (bf16 MFMA operations x 512) and MfmaUtil
    (percent of SIMD cycles with the MFMA unit busy, over the dispatch's active cycles) from
    one counter run, and the mean duration from a kernel trace of the same command."""
    flops = counter_values(a.counter_dir, "MfmaFlopsBF16")
    util = counter_values(a.counter_dir, "MfmaUtil")
    dur = kernel_durations(a.trace_dir)
    print(f"gemv source sha256[:16]: {source_hash()}")
    print(f"{'kernel':44s} {'calls':>6s} {'avg_us':>8s} {'MFMA_GFLOP':>11s} {'TFLOP/s':>8s} "
          f"{'of_2.5P':>7s} {'MfmaUtil%':>9s}")
    for k in sorted(flops, key=lambda k: -sum(flops[k])):
        fv = flops[k]
        if sum(fv) == 0:
            continue
        uv = util.get(k, [0.0])
        d = dur.get(k)
        avg_us = sum(d) / len(d) if d else float("nan")
        f_avg = sum(fv) / len(fv)
        tf = f_avg / (avg_us * 1e-6) / 1e12 if d else float("nan")
        print(f"{k:44s} {len(fv):6d} {avg_us:8.2f} {f_avg / 1e9:11.3f} {tf:8.1f} "
              f"{tf / 2500.0:7.3f} {sum(uv) / len(uv):9.2f}")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--kernel", default=None)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--calib-mib", type=int, required=True)
    t.add_argument("--kernel", default="gemv_gate_up")
    for q in (s, t):
        q.add_argument("--group", type=int, default=0,
                       help="phase of --kernel: its dispatches between the run's n-th and "
                            "next prefill (0 = before the second prefill)")
        q.add_argument("--skip", type=int, default=0,
                       help="leading dispatches of the phase to drop (warm-up steps)")
    m = sub.add_parser("mfma")
    m.add_argument("counter_dir")
    m.add_argument("trace_dir")
    a = ap.parse_args(argv)
    {"stats": cmd_stats, "traffic": cmd_traffic, "mfma": cmd_mfma}[a.cmd](a)


if __name__ == "__main__":
    main(sys.argv[1:])
