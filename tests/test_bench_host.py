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
