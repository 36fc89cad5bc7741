"""Host-side pieces of bench.py (no GPU)."""
import os

from conftest import ROOT


def test_traffic_is_read_from_the_committed_counter_summary():
    import bench
    from speculative_pipeline_decoding_amd.profile_summary import source_hash
    wl = "dense_bf16_L32_d2560_n8_ctx2048"
    path = os.path.join(ROOT, "profiles", f"gemv_gate_up_traffic_{wl}.txt")
    lines = open(path).read().splitlines()
    digest = [ln.split()[-1] for ln in lines if ln.startswith("gemv source sha256[:16]:")]
    value = [float(ln.split()[-1]) for ln in lines if ln.startswith("traffic_bytes_per_launch")]
    got = bench.traffic_from_profile(wl, "gemv_gate_up")
    if digest and digest[0] == source_hash():
        assert got == value[0]
    else:
        assert got is None           # counters taken on another GEMV source are not reported


def test_more_than_one_gpu_is_refused():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def _write_csv(path, header, rows):
    import csv
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_profile_phases_pick_the_timed_replay(tmp_path, capsys):
    """A kernel's phase is the run of its dispatches between two prefills (prefill GEMM
    dispatches end one), counted in dispatch order, not file order; --skip drops warm-up."""
    from speculative_pipeline_decoding_amd import profile_summary as ps
    gemm, gu, other = "gemm_x3_kernel", "spd::(anonymous namespace)::gemv_gate_up<unsigned short, 0>(x)", "k2"
    # dispatch id, kernel, duration (ns): prefill, phase 0 (2 launches), prefill, phase 1 (3),
    # prefill, phase 2 (1); written out of order
    seq = [(1, gemm, 5), (2, gu, 100), (3, other, 7), (4, gu, 100), (5, gemm, 5), (6, gemm, 5),
           (7, gu, 10), (8, other, 7), (9, gu, 20), (10, gu, 30), (11, gemm, 5), (12, gu, 999)]
    rows = [["KERNEL_DISPATCH", d, k, 1000, 1000 + ns] for d, k, ns in reversed(seq)]
    _write_csv(str(tmp_path / "t" / "run_kernel_trace.csv"),
               ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    ps.main(["stats", str(tmp_path / "t"), "--kernel", "gemv_gate_up", "--group", "1", "--skip", "1"])
    last = capsys.readouterr().out.strip().splitlines()[-1]
    assert "phase 1" in last and "2 calls" in last and "avg_us 0.03" in last   # (20 + 30) / 2 ns
    ps.main(["stats", str(tmp_path / "t"), "--kernel", "gemv_gate_up", "--group", "0"])
    assert "2 calls, avg_us 0.10" in capsys.readouterr().out.strip().splitlines()[-1]
    # a base name covers every kind of the kernel (launches change kind with their vector
    # counts); a full name, one kind
    gu4 = "spd::(anonymous namespace)::gemv_gate_up<unsigned short, 6>(x)"
    rows = [["KERNEL_DISPATCH", d, gu4 if d == 8 else k, 1000, 1000 + (40 if d == 8 else ns)]
            for d, k, ns in seq]
    _write_csv(str(tmp_path / "t2" / "run_kernel_trace.csv"),
               ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    ps.main(["stats", str(tmp_path / "t2"), "--kernel", "gemv_gate_up", "--group", "1"])
    assert "4 calls, avg_us 0.03" in capsys.readouterr().out.strip().splitlines()[-1]   # 100/4 ns
    ps.main(["stats", str(tmp_path / "t2"), "--kernel", "gemv_gate_up<bf16, 6>", "--group", "0"])
    assert "1 calls, avg_us 0.04" in capsys.readouterr().out.strip().splitlines()[-1]
    # counters: FETCH_SIZE / WRITE_SIZE per dispatch, scaled by a calibration copy
    copy = "__amd_rocclr_copyBuffer"
    cseq = seq + [(13, copy, 0)]
    for d, cnt, scale in (("f", "FETCH_SIZE", 2.0), ("w", "WRITE_SIZE", 1.0)):
        rows = []
        for i, k, ns in cseq:
            kib = 1024.0 / scale if k == copy else (ns * 1000.0 if k == gu else 1.0)
            rows.append([i, k, cnt, kib])
        _write_csv(str(tmp_path / d / "run_counter_collection.csv"),
                   ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    ps.main(["traffic", str(tmp_path / "f"), str(tmp_path / "w"), "--calib-mib", "1",
             "--kernel", "gemv_gate_up", "--group", "1", "--skip", "1"])
    out = capsys.readouterr().out.strip().splitlines()
    # phase 1 after one warm-up: counters 20000 and 30000 KiB, fetch scaled x2, write x1
    want = (25000 * 2.0 + 25000 * 1.0) * 1024
    assert out[-1].startswith("traffic_bytes_per_launch") and abs(float(out[-1].split()[-1]) - want) < 1
