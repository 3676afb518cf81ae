"""Host-side checks of the benchmark script (no GPU): one GPU only, and the
work and roofline bookkeeping it reports."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_prefill_work_of_the_t8192_workload():
    flops, nbytes = bench.prefill_work(1, 16, 8192, 64, 128)
    # per head-token: 2d(C+1) + 4d^2 + d^2/C flops; 10d bytes; plus 8d^2 per head
    assert flops == 16 * 8192 * (2 * 128 * 65 + 4 * 128 * 128 + 128 * 128 / 64)
    assert nbytes == 16 * 8192 * 10 * 128 + 16 * 8 * 128 * 128 == 169869312


def test_decode_bytes_of_the_decode_workload():
    assert bench.decode_bytes(256, 32, 128) == 8192 * (8 * 128 * 128 + 10 * 128) == 1084227584


def test_continuation_roofline_picks_the_binding_bound():
    # plain T=16: bytes need more time than FMAs at the peaks -> HBM
    r = bench.tokens_roofline("k", 1_241_513_984, 256 * 32 * 16 * 2 * 128 * 128, 0.225)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and abs(r["frac"] - r["hbm_frac"]) < 1e-12
    # grouped T=16, four query heads per state: the FMAs bind -> vector ALU
    r = bench.tokens_roofline("k", 385_875_968, 256 * (8 + 32) * 16 * 128 * 128, 0.127)
    assert r["bound"] == "alu" and r["unit"] == "TFLOP/s" and abs(r["frac"] - r["alu_frac"]) < 1e-12
    assert 0.5 < r["frac"] < 0.6


def test_spread_of_step_times():
    s = bench.spread([3.0, 1.0, 2.0, 10.0, 4.0])
    assert s["median_ms"] == 3.0 and s["min_ms"] == 1.0 and s["max_ms"] == 10.0 and s["n"] == 5
    assert s["mean_ms"] == 4.0 and s["p10_ms"] == 1.0 and s["p90_ms"] == 10.0


def test_oracle_threads_follow_the_host(monkeypatch):
    monkeypatch.delenv("OMP_NUM_THREADS", raising=False)
    threads, host = bench.host_cores()
    assert threads == len(os.sched_getaffinity(0)) == host["cpus_in_affinity"]
    assert host["logical_cpus"] == os.cpu_count()
    monkeypatch.setenv("OMP_NUM_THREADS", "2")
    threads, host = bench.host_cores()
    assert threads == min(2, len(os.sched_getaffinity(0))) and host["omp_num_threads"] == 2


def test_hbm_roofline_takes_the_launch_gap_off():
    r = bench.hbm_roofline("k", 169869312, 0.0435, 0.0017, traffic=1.8e8, timing="t")
    assert abs(r["kernel_ms"] - 0.0418) < 1e-12 and r["kernel_ms_back_to_back"] == 0.0435
    assert abs(r["achieved"] - 169869312 / 0.0418e-3 / 1e9) < 1e-6
    assert abs(r["frac"] - r["achieved"] / 8000.0) < 1e-12 and r["frac_back_to_back"] < r["frac"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["traffic"] == 1.8e8
