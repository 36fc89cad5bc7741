#!/usr/bin/env python3
"""Committed tokens/s of Speculative Pipeline Decoding on one MI355X.

A bench "step" is one SPD pipeline step (spd_step + spd_verify_commit): the
stage-0 embedding, the PDM (anchor gather, k*d -> d projection, Ls layers,
LM head, draft), every in-flight token's stage slice (QKV + RoPE + KV write,
staircase attention, O, SwiGLU FFN, residual + anchor capture), and the
streaming verification with commit / truncate / flush / reseed.

Default workload: dense 32-layer bf16 decoder, d=2560, 32 q / 8 kv heads x 80,
SwiGLU 9728, vocab 151936, SPD n=8, Ls=4, anchors {0,8,16,24,31}, context 2048
(1792-token prompt + 256 generated), T=1 with rejection-sampling verification
and top-p 1.0 (--t0-run adds the greedy, lossless T=0 run).
Weights are seeded random N(0, 0.02) and the prompt is uniform random ids:
synthetic data of the workload's shape.

Timed region: W warm-up steps, then exactly K steps between two device
synchronisations, with inputs resident in HBM. value = committed tokens / s.
step_us is each step's full cycle as a caller sees it (enqueue, GPU execution and
verdict read-back), taken on the host between successive verify_commit returns.
Per-launch durations for the roofline come from HIP start/stop events that the
library binds to each launch's dispatch packet (hipExtLaunchKernel), on the
stream the launch runs on, over the timed steps of a second pass that replays
the same warm-up and timed steps from a fresh prefill (the events cost ~15% of
step time, so the headline region runs without them). The CPU baseline is the
float32 oracle on the host cores: the same workload and prompt, a bounded number
of steps, its own committed tokens over the steps' wall time.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC_FMT = "committed tokens/s (1 seq, 1 GPU) + step µs + % HBM roofline, n={n}"
# the arithmetic type of every kernel on the path: fp32 FMAs and fp32 accumulation, on bf16
# (or fp32) weights and a bf16 (or fp32) KV cache
ARITH_DTYPE = "f32"
HBM_PEAK_GBS = 8000.0
FP32_MATRIX_PEAK_TFLOPS = 157.3     # MI355X dense fp32 matrix-core peak
BF16_MATRIX_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix-core peak


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def pct(xs, q):
    xs = sorted(xs)
    if not xs:
        return None
    i = min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))
    return xs[i]


def hbm_ceiling():
    """Measured streaming rates of plain library kernels on 1 GiB (best of five, host-timed):
    a device-to-device copy (read + write) and a sum (read only)."""
    import torch
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)

    def best(fn):
        b = None
        for _ in range(5):
            torch.cuda.synchronize()
            t = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            dt = time.perf_counter() - t
            b = dt if b is None else min(b, dt)
        return b

    copy = 2.0 * (1 << 30) / best(lambda: dst.copy_(src)) / 1e9
    read = 1.0 * (1 << 30) / best(lambda: src.sum()) / 1e9
    del src, dst
    return {"kind": "torch copy_ and sum over 1 GiB, best of 5, host-timed",
            "copy_GBps": copy, "read_GBps": read,
            "frac_of_peak": max(copy, read) / HBM_PEAK_GBS}


def prefill_flops(cfg, P):
    """Matrix flops of a P-token prefill: target layers, prefix aggregation, PDM layers,
    causal attention (QK and PV), and the head for the last row."""
    d, F, hd = cfg.d_model, cfg.d_ffn, cfg.head_dim
    qo, kvd = cfg.n_q_heads * hd, cfg.n_kv_heads * hd
    soft = d * (qo + 2 * kvd) + qo * d + 3 * d * F
    lin = 4 * d * qo + 3 * d * F
    k = len(cfg.anchors)
    w = sum(lin if kind else soft for kind in cfg.kinds)
    w += k * d * d + cfg.pdm_layers * soft
    attn_layers = sum(1 for kind in cfg.kinds if not kind) + cfg.pdm_layers
    attn = attn_layers * 2 * qo * P * (P + 1)            # QK^T and PV, causal
    lin_flops = sum(1 for kind in cfg.kinds if kind) * P * cfg.n_q_heads * 4 * hd * hd
    return 2.0 * P * w + attn + lin_flops + 2.0 * cfg.vocab * d


def prefill_rate(cfg, dW, prompt):
    """Prefill of the workload's prompt, timed warm (the second of two), with its matrix
    flops (the whole prefill, GEMMs and the rest). The bf16-weight GEMMs run each fp32
    product as three bf16 products, so their ceiling is a third of the bf16 peak."""
    import torch
    from speculative_pipeline_decoding_amd import SPD
    spd = SPD(cfg, dW, stream=torch.cuda.current_stream())
    spd.prefill(prompt)
    torch.cuda.synchronize()
    spd.reset()
    t = time.perf_counter()
    spd.prefill(prompt)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t
    spd.close()
    fl = prefill_flops(cfg, len(prompt))
    tf = fl / dt / 1e12
    peak = BF16_MATRIX_PEAK_TFLOPS / 3.0 if cfg.dtype == "bf16" else FP32_MATRIX_PEAK_TFLOPS
    return {"tokens": len(prompt), "seconds": dt, "tokens_per_s": len(prompt) / dt,
            "matrix_tflops": tf, "peak_tflops": peak, "frac": tf / peak,
            "frac_of_fp32_matrix_peak": tf / FP32_MATRIX_PEAK_TFLOPS,
            "note": "bf16 weights: fp32 activations split into three bf16 terms on the bf16 "
                    "matrix cores (peak = bf16 peak / 3); the time includes norms, RoPE, "
                    "attention and the host's chunk loop"}


def run_spd(cfg, dW, prompt, T, seed, warmup, steps, kernel_timing, top_p=1.0,
            speculate_from="input", lookahead=True):
    import torch
    from speculative_pipeline_decoding_amd import SPD
    stream = torch.cuda.current_stream()
    spd = SPD(cfg, dW, temperature=T, top_p=top_p, seed=seed, stream=stream,
              speculate_from=speculate_from, draft_width=cfg.draft_width)
    # a refill step's successor is enqueued together with it (the library skips this while
    # per-launch timing is on)
    spd.lookahead(lookahead)
    t = time.perf_counter()
    spd.prefill(prompt)
    torch.cuda.synchronize()
    prefill_s = time.perf_counter() - t
    out = {"prefill_s": prefill_s}
    for _ in range(warmup):
        spd.step()
        spd.verify_commit()

    def region():
        # Step latency is taken on the host, between successive verify_commit returns: one
        # full cycle of enqueue, GPU execution and verdict read-back, as a caller sees it.
        s0 = spd.stats()
        kinds, host, step_ms = [], [], []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        t_prev = t0
        for _ in range(steps):
            h0 = time.perf_counter()
            spd.step()
            host.append(time.perf_counter() - h0)
            c = spd.verify_commit()
            t_now = time.perf_counter()
            step_ms.append(1e3 * (t_now - t_prev))
            t_prev = t_now
            kinds.append(bool(c.verified))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        s1 = spd.stats()
        return s1, {"wall_s": wall, "N": s1.N - s0.N, "K": s1.K - s0.K, "step_ms": step_ms,
                    "host_step_us": 1e6 * float(np.median(host)),
                    "full": [m for m, k in zip(step_ms, kinds) if k],
                    "refill": [m for m, k in zip(step_ms, kinds) if not k]}

    s1, out["timed"] = region()
    if kernel_timing:
        # The same steps again from a fresh prefill (same seed, so the same sequence of
        # steps), with start/stop events bound to each launch's dispatch packet (kernel
        # durations without the command processor's gaps) over exactly the timed steps.
        # They are kept out of the headline region, which runs without them. Lookahead is
        # off here (the library skips it while timing anyway); results are bit-identical.
        spd.reset()
        spd.lookahead(False)
        spd.prefill(prompt)
        for _ in range(warmup):
            spd.step()
            spd.verify_commit()
        spd.timing(True)
        _, kt = region()
        out["kernels"] = spd.timing_read()
        out["kernel_steps"] = steps
        out["kernel_region"] = {"N": kt["N"], "K": kt["K"]}
        spd.timing(False)
    out["alpha_total"], out["s0_total"] = s1.alpha, s1.s0
    spd.close()
    return out


def traffic_from_profile(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, or None
    when there is none or it was taken on a different GEMV source than the current one."""
    from speculative_pipeline_decoding_amd.profile_summary import source_hash
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    digest, value = None, None
    for line in open(path):
        if line.startswith("gemv source sha256[:16]:"):
            digest = line.split()[-1]
        if line.startswith("traffic_bytes_per_launch"):
            value = float(line.split()[-1])
    if digest != source_hash() or value is None:
        return None
    return value


def cpu_info():
    """CPU model, logical CPUs and BLAS threads of the host running this process."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
            "blas_threads": int(threads)}


def cpu_baseline(cfg, W, prompt, T, seed, budget_s, top_p=1.0, speculate_from="input"):
    """The oracle as it stands, in float32, on the host cores: the workload's own prompt,
    then as many SPD steps as fit the budget; value = the oracle's own committed tokens
    over the wall time of its steps (its prefill is set-up, as the GPU's is)."""
    import numpy as np
    from oracle.spd import SPD as OracleSPD
    from oracle.sampling import Sampling
    info = cpu_info()
    t = time.perf_counter()
    o = OracleSPD(cfg, W, Sampling(temperature=T, top_p=top_p, seed=seed), ft=np.float32,
                  speculate_from=speculate_from, record_logits=False, W=cfg.draft_width)
    o.prefill(np.asarray(prompt))
    setup = time.perf_counter() - t
    log(f"cpu baseline: float32 oracle prefill of {len(prompt)} tokens in {setup:.1f}s "
        f"(weights upcast once; untimed)")
    t0 = time.perf_counter()
    # bounded by the budget and by the workload's own length (G tokens, the context)
    while (o.K < 2 or time.perf_counter() - t0 < budget_s) and 1 + o.N < cfg.gen_len \
            and o.F[-1][0] + 1 < cfg.max_ctx:
        o.step()
        if o.K % 8 == 0:
            log(f"cpu baseline: oracle step {o.K} (N={o.N}) at {time.perf_counter() - t0:.1f}s")
    dt = time.perf_counter() - t0
    return {"value": o.N / dt, "unit": "tokens/s", "cores": info["blas_threads"],
            "kind": "oracle",
            "sample": (f"the float32 numpy oracle on the same n={o.n} workload: prefill of its "
                       f"{len(prompt)}-token prompt (untimed), then {o.K} SPD steps in "
                       f"{dt:.1f} s committing N={o.N} tokens (alpha={o.alpha:.3f}); value = N "
                       f"over the steps' wall time"),
            "N": o.N, "K": o.K, "seconds": dt, "steps_per_s": o.K / dt, "alpha": o.alpha,
            "prefill_s": setup, **info}


def forced_sweep(cfg, dW, prompt, ps, warmup, steps, lookahead=True):
    """Throughput at controlled acceptance (T=0 forced mode): each draft at position x is
    the target's own greedy token with probability p, else a wrong one, so every
    verification accepts with probability p. The reference stream is the library's own
    greedy decode at n = 1 (autoregressive). Under this reading p = 0.77 gives the pages'
    alpha n = 3.04 at n = 8."""
    import torch
    from speculative_pipeline_decoding_amd import SPD
    stream = torch.cuda.current_stream()
    ar = SPD(cfg, dW, n=1, stream=stream)
    ref, _ = ar.generate(prompt, warmup + steps + cfg.n_stages + 8)
    ar.close()
    out = []
    for p in ps:
        spd = SPD(cfg, dW, forced_p=p, forced_ref=ref, stream=stream)
        spd.lookahead(lookahead)
        spd.prefill(prompt)
        for _ in range(warmup):
            spd.step()
            spd.verify_commit()
        s0 = spd.stats()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            spd.step()
            spd.verify_commit()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        s1 = spd.stats()
        spd.close()
        N, K = s1.N - s0.N, s1.K - s0.K
        out.append({"p": p, "alpha": N / K, "s0": N / K * cfg.n_stages,
                    "tokens_per_s": N / wall, "ms_per_step": 1e3 * wall / K})
    return out


def ar_reference(cfg, dW, prompt, T, seed, warmup, steps):
    """Context: the same library at n = 1 with a one-layer PDM, i.e. autoregressive decoding
    on the same kernels. Each step runs all L layers for one token and the head sweep and
    commits exactly one token (the draft it makes is verified in the same step). On one GPU
    SPD cannot beat this: every commit costs at least one sweep of the weights; the paper's
    speedup needs a GPU per stage."""
    import torch
    from speculative_pipeline_decoding_amd import SPD
    stream = torch.cuda.current_stream()
    spd = SPD(cfg, dW, temperature=T, seed=seed, n=1, Ls=1, stream=stream)
    spd.lookahead(True)
    spd.prefill(prompt)
    for _ in range(warmup):
        spd.step()
        spd.verify_commit()
    s0 = spd.stats()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        spd.step()
        spd.verify_commit()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    s1 = spd.stats()
    spd.close()
    N = s1.N - s0.N
    return {"n": 1, "pdm_layers": 1, "temperature": T, "tokens_per_s": N / wall,
            "ms_per_token": 1e3 * wall / max(N, 1), "N": N}


def stage_plan_report(cfg, dW, prompt, steps):
    """Per-layer cost of one token through each target layer (the library at n = 1, where
    every sub-layer launch serves one layer), and the stage split balanced on it against
    the default split: per-stage time and its spread. With one GPU per stage, a pipeline
    step lasts as long as its slowest stage."""
    import numpy as np
    from speculative_pipeline_decoding_amd import SPD, balance_stages
    spd = SPD(cfg, dW, temperature=0.0, n=1)
    spd.prefill(prompt)
    spd.timing(True, serial=True)     # no launch shares the GPU with the PDM chain
    for _ in range(steps):
        spd.step()
        spd.verify_commit()
    ms, passes = spd.timing_read_layers()
    spd.close()
    us = 1e3 * ms / np.maximum(passes, 1)
    n = cfg.n_stages

    def stages(sizes):
        b = np.concatenate([[0], np.cumsum(sizes)])
        t = [float(us[b[i]:b[i + 1]].sum()) for i in range(n)]
        return {"sizes": [int(x) for x in sizes], "stage_us": [round(x, 1) for x in t],
                "max_us": round(max(t), 1), "spread": round(max(t) / min(t) - 1.0, 4)}

    default = [len(a) for a in np.array_split(np.arange(cfg.n_layers), n)]
    balanced = balance_stages(us, n)
    kinds = np.asarray(cfg.kinds)
    per_kind = {("linear" if k else "softmax"): round(float(us[kinds == k].mean()), 1)
                for k in sorted(set(kinds.tolist()))}
    return {"layer_us_per_token": per_kind, "passes": int(passes.min()),
            "default": stages(default), "balanced": stages(balanced)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="cfg3")
    ap.add_argument("--temperature", type=float, default=None,
                    help="sampling temperature (default: the workload's first one)")
    ap.add_argument("--top-p", type=float, default=None,
                    help="top-p of the sampled run (default: the workload's, 1.0)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--speculate-from", choices=["input", "output"], default="input",
                    help="input: the PDM beside the step on its input states (the method); "
                         "output: after the step on its output states (the ablation)")
    ap.add_argument("--t0-run", action="store_true",
                    help="also time the same steps at T=0 (greedy, lossless) and report them")
    ap.add_argument("--stage-plan", action="store_true",
                    help="also time one token through each layer (n = 1) and report the "
                         "stage split balanced on those costs against the default split")
    ap.add_argument("--forced-sweep", action="store_true",
                    help="also time T=0 forced-acceptance runs at p = 0.5, 0.77, 0.9")
    ap.add_argument("--no-lookahead", action="store_true",
                    help="enqueue every step only after the previous one's verdict (no "
                         "lookahead launch of a refill step's successor)")
    ap.add_argument("--kv-f32", action="store_true",
                    help="store the KV caches in fp32 (kv_dtype SPD_KV_F32) instead of bf16")
    ap.add_argument("--draft-width", type=int, default=None,
                    help="draft candidates per position for the headline run (default: the "
                         "workload's, 1)")
    ap.add_argument("--tree-width", type=int, default=4,
                    help="also time the same steps with draft trees of this width (the "
                         "paper's W = 4; 0 or 1 skips it; softmax-only models)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0,
                    help="seconds of oracle steps in the CPU baseline (its prefill is extra)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run one device-to-device copy of this many MiB: a kernel of "
                         "known traffic, to scale hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the library runs the "
              "SPD hot path on a single MI355X and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from spd_inputs import get, make_prompt, make_weights, weight_bytes
    from speculative_pipeline_decoding_amd import upload_weights

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cfg = get(args.workload)
    if args.kv_f32:
        cfg = cfg.with_(kv_dtype="f32")
    if args.draft_width is not None:
        cfg = cfg.with_(draft_width=args.draft_width)
    if args.temperature is None:
        args.temperature = float(cfg.temperatures[0])
    if args.top_p is None:
        args.top_p = float(cfg.top_p)
    if args.warmup + args.steps > cfg.gen_len:
        print(f"warmup + steps must be <= {cfg.gen_len} (the workload generates {cfg.gen_len} "
              "tokens; each step commits at most one)", file=sys.stderr)
        sys.exit(2)
    t = time.perf_counter()
    W = make_weights(cfg)
    log(f"weights drawn in {time.perf_counter() - t:.1f}s ({weight_bytes(cfg) / 1e9:.2f} GB)")
    dW = upload_weights(cfg, W)
    torch.cuda.synchronize()
    prompt = make_prompt(cfg)
    log(f"weights resident on {torch.cuda.get_device_name(0)}")
    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.calib_copy_mib} MiB read + {args.calib_copy_mib} MiB written")
        del src, dst

    lookahead = not args.no_lookahead
    main_run = run_spd(cfg, dW, prompt, args.temperature, args.seed, args.warmup, args.steps, True,
                       args.top_p, args.speculate_from, lookahead)
    tm = main_run["timed"]
    log(f"T={args.temperature}: prefill {main_run['prefill_s']:.2f}s, timed {tm['K']} steps in "
        f"{tm['wall_s'] * 1e3:.1f} ms, N={tm['N']}")
    t0_run = None
    if args.t0_run and args.temperature != 0.0:
        r = run_spd(cfg, dW, prompt, 0.0, args.seed, args.warmup, args.steps, False,
                    speculate_from=args.speculate_from, lookahead=lookahead)
        rt = r["timed"]
        t0_run = {"temperature": 0.0, "tokens_per_s": rt["N"] / rt["wall_s"], "N": rt["N"],
                  "K": rt["K"], "alpha": rt["N"] / rt["K"], "s0": rt["N"] / rt["K"] * cfg.n_stages,
                  "ms_per_step": rt["wall_s"] * 1e3 / rt["K"],
                  "step_us_median": 1e3 * statistics.median(rt["step_ms"])}
        log(f"T=0: timed {rt['K']} steps, N={rt['N']}")
    tree_run = None
    tree_ok = (args.tree_width > 1 and cfg.draft_width == 1 and not any(cfg.kinds)
               and args.speculate_from == "input" and args.top_p >= 1.0)
    if tree_ok:
        # the same workload with draft trees (W candidates per draft position), same seed
        r = run_spd(cfg.with_(draft_width=args.tree_width), dW, prompt, args.temperature,
                    args.seed, args.warmup, args.steps, False, lookahead=lookahead)
        rt = r["timed"]
        tree_run = {"draft_width": args.tree_width, "temperature": args.temperature,
                    "tokens_per_s": rt["N"] / rt["wall_s"], "N": rt["N"], "K": rt["K"],
                    "alpha": rt["N"] / rt["K"], "s0": rt["N"] / rt["K"] * cfg.n_stages,
                    "ms_per_step": rt["wall_s"] * 1e3 / rt["K"],
                    "step_us_median": 1e3 * statistics.median(rt["step_ms"]),
                    "full_median_us": 1e3 * statistics.median(rt["full"]) if rt["full"] else None,
                    "refill_median_us": (1e3 * statistics.median(rt["refill"])
                                         if rt["refill"] else None)}
        log(f"W={args.tree_width}: timed {rt['K']} steps, N={rt['N']}")

    value = tm["N"] / tm["wall_s"]
    ms_per_step = tm["wall_s"] * 1e3 / tm["K"]
    alpha = tm["N"] / tm["K"]
    kern = main_run["kernels"]
    ik = main_run["kernel_steps"]
    # algorithmic bytes of the timed steps (the replay runs the same steps)
    step_bytes = sum(v["bytes"] for v in kern.values()) / ik
    dominant = max((k for k in kern if k.startswith("gemv") and kern[k]["count"]),
                   key=lambda k: kern[k]["ms"])
    d = kern[dominant]
    achieved = (d["bytes"] / d["count"]) / (d["ms"] / d["count"] * 1e-3) / 1e9
    kernels = {k: {"launches": v["count"], "avg_us": 1e3 * v["ms"] / v["count"],
                   "GBps": (v["bytes"] / (v["ms"] * 1e-3) / 1e9) if v["bytes"] else None,
                   "bytes_per_launch": v["bytes"] / v["count"]}
               for k, v in kern.items() if v["count"]}
    res = {
        "metric": METRIC_FMT.format(n=cfg.n_stages),
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ARITH_DTYPE,
        "data": "synthetic",
        "config": {"workload": cfg.name, "n": cfg.n_stages, "Ls": cfg.pdm_layers,
                   "anchors": list(cfg.anchors), "context": cfg.prompt_len + cfg.gen_len,
                   "prompt": cfg.prompt_len, "temperature": args.temperature, "top_p": args.top_p,
                   "speculate_from": args.speculate_from, "lookahead": lookahead,
                   "draft_width": cfg.draft_width,
                   "weights": f"{cfg.dtype} N(0,{cfg.weight_std}) seeded",
                   "kv_cache": cfg.dtype if cfg.kv_dtype == "auto" else cfg.kv_dtype,
                   "arithmetic": "fp32 FMA, fp32 accumulation",
                   "prompt_ids": "uniform random"},
        "commits": tm["N"],
        "timed_steps": tm["K"],
        "value_note": (f"{tm['N']} commits in {tm['K']} timed steps: with random weights the "
                       "acceptance is a random walk, so a short run's tokens/s carries alpha's "
                       "noise; step_us and step_hbm_roofline do not depend on alpha"),
        "roofline": {"bound": "hbm", "kernel": dominant,
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic_from_profile(cfg.name, dominant),
                     "algorithmic_bytes_per_launch": d["bytes"] / d["count"],
                     "avg_launch_us": 1e3 * d["ms"] / d["count"]},
        "step_us": {"median": 1e3 * statistics.median(tm["step_ms"]),
                    "p10": 1e3 * pct(tm["step_ms"], 0.1), "p90": 1e3 * pct(tm["step_ms"], 0.9),
                    "full_median": 1e3 * statistics.median(tm["full"]) if tm["full"] else None,
                    "refill_median": 1e3 * statistics.median(tm["refill"]) if tm["refill"] else None,
                    "full_steps": len(tm["full"]), "refill_steps": len(tm["refill"]),
                    "host_enqueue_median": tm["host_step_us"]},
        "alpha": alpha,
        "s0": alpha * cfg.n_stages,
        "step_hbm_roofline": {"algorithmic_bytes_per_step": step_bytes,
                              "achieved_GBps": step_bytes / (ms_per_step * 1e-3) / 1e9,
                              "frac": step_bytes / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
                              "over": "the timed steps: their algorithmic bytes (per-launch "
                                      "accounting of the same steps replayed) over ms_per_step"},
        "kernels": kernels,
        "t0_run": t0_run,
        "tree_run": tree_run,
        "prefill_s": main_run["prefill_s"],
        "device": torch.cuda.get_device_name(0),
    }
    res["ar_reference"] = ar_reference(cfg, dW, prompt, args.temperature, args.seed, 8,
                                       min(64, cfg.gen_len - 8))
    log(f"AR reference (n=1): {res['ar_reference']['tokens_per_s']:.1f} tokens/s")
    res["hbm_ceiling"] = hbm_ceiling()
    res["prefill"] = prefill_rate(cfg, dW, prompt)
    log(f"HBM copy {res['hbm_ceiling']['copy_GBps']:.0f} GB/s, read {res['hbm_ceiling']['read_GBps']:.0f}"
        f" GB/s; prefill "
        f"{res['prefill']['tokens_per_s']:.0f} tok/s, {res['prefill']['matrix_tflops']:.1f} TFLOP/s")
    if args.forced_sweep:
        res["forced_sweep"] = forced_sweep(cfg, dW, prompt, (0.5, 0.77, 0.9), args.warmup,
                                           args.steps, lookahead)
        log(f"forced sweep: {res['forced_sweep']}")
    if args.stage_plan:
        res["stage_plan"] = stage_plan_report(cfg, dW, prompt, 24)
        log(f"stage plan: {res['stage_plan']}")
    if not args.no_cpu_baseline:
        del dW
        torch.cuda.empty_cache()
        res["cpu_baseline"] = cpu_baseline(cfg, W, prompt, args.temperature, args.seed,
                                           args.cpu_budget, args.top_p, args.speculate_from)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
