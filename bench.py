"""Benchmark: causal linear-attention prefill and decode on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Prints ONE JSON line.  ``value`` is prefill throughput in tokens/s (B*T per
second) on the T=8192 workload (B=1, H=16, C=64, d_k=d_v=128, bf16 Q/K/V,
fp32 state and output); the decode workload (256 sequences x 32 heads,
d=128, state from a seeded T=4096 prefill) is reported under ``decode`` in
steps/s.

Prefill is timed cold: the timed steps rotate over several input/output
sets whose total exceeds the 256 MB Infinity Cache, so each step's inputs
come from HBM; a warm figure (one set repeated) is given for context.  Each
step calls the three prefill phases in order (exactly what lla_prefill
does) with HIP events between them on the launch stream, which gives the
per-kernel duration of the dominant kernel (the chunk walk) for the
roofline.  Decode steps are timed the same way, one event pair per step.

The CPU baseline is the float64 oracle (the token-by-token recurrence) on
the host cores, timed on a bounded sample of the same workloads.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 matrix cores, TFLOP/s
METRIC = "prefill tokens/s + % bf16 MFMA peak; decode steps/s + % HBM BW (1 GPU)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "chunk_walk_T8192_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "decode_lla_prefill_amd", "csrc", f)
                  for f in ("lla_prefill.hip", "lla_device.h")]


def prefill_work(B, H, T, C, d):
    """Algorithmic flops and bytes of one prefill (kept triangle only).

    flops per head-token: 2d(C+1) (scores + masked scores x V over the kept
    triangle) + 4d^2 (Q S and K^T V) + d^2/C (the state add per chunk);
    bytes per head-token: 6d (bf16 Q, K, V) + 4d (fp32 O); plus 8d^2 per
    (b,h) for reading S_0 and writing S_T.
    """
    ht = B * H * T
    flops = ht * (2 * d * (C + 1) + 4 * d * d + d * d / C)
    nbytes = ht * 10 * d + B * H * 8 * d * d
    return flops, nbytes


def decode_bytes(B, H, d):
    """Per step: fp32 state read + write (8d^2), bf16 q,k,v (6d), fp32 o (4d)."""
    return B * H * (8 * d * d + 10 * d)


def kernel_source_sha():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic():
    """HBM bytes per chunk-walk launch from the committed counter summary,
    or None if it is missing or was taken on a different kernel source."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if "=" in line and not line.startswith("#"):
                    key, val = line.split("=", 1)
                    kv[key.strip()] = val.strip()
        if kv.get("kernel_source_sha") != kernel_source_sha():
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def time_oracle_prefill(q, k, v, threads):
    import oracle
    t0 = time.perf_counter()
    oracle.recurrence(q, k, v, nthreads=threads)
    return time.perf_counter() - t0


def bench_prefill(args, torch, lla, workloads):
    cfg = workloads.CONFIGS[args.prefill_config]
    dev = torch.device("cuda:0")
    B, H, T, C, d = cfg.B, cfg.H, cfg.T, cfg.C, cfg.dk
    q0, k0, v0 = workloads.config_inputs(cfg, device=dev)
    sets = []
    for r in range(args.rotate):
        q, k, v = (x.clone() for x in (q0, k0, v0)) if r else (q0, k0, v0)
        S = lla.state_init(B, H, d, d, device=dev)
        o = torch.empty((B, H, T, d), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, lla.prefill_workspace_size(B, H, T, d, d, C) // 4),
                         dtype=torch.float32, device=dev)
        sets.append((q, k, v, S, o, ws))
    stream = torch.cuda.current_stream(dev)

    def step(i, ev=None):
        q, k, v, S, o, ws = sets[i % len(sets)]
        lla.state_init(B, H, d, d, out=S)
        if ev is not None:
            ev[0].record(stream)
        lla.prefill_segment_states(k, v, C, ws)
        if ev is not None:
            ev[1].record(stream)
        lla.prefill_state_scan(S, T, C, ws)
        if ev is not None:
            ev[2].record(stream)
        lla.prefill_chunks(q, k, v, S, C, workspace=ws, out=o)
        if ev is not None:
            ev[3].record(stream)

    def run(n_steps, n_sets_used):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n_steps):
            step(i % n_sets_used, evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        phase = [[e[j].elapsed_time(e[j + 1]) for e in evs] for j in range(3)]
        per_step = [e[0].elapsed_time(e[3]) for e in evs]
        return wall, phase, per_step

    for i in range(args.warmup):
        step(i)
    wall, phase, per_step = run(args.steps, len(sets))
    _, phase_w, per_step_w = run(args.steps, 1)
    flops, nbytes = prefill_work(B, H, T, C, d)
    ms_step = wall * 1e3 / args.steps
    gpu_ms = sum(per_step) / len(per_step)
    walk_ms = sum(phase[2]) / len(phase[2])
    achieved = nbytes / (walk_ms * 1e-3) / 1e9
    traffic = stored_traffic()
    res = {
        "config": {"workload": cfg.name, "B": B, "H": H, "T": T, "C": C, "dk": d, "dv": d,
                   "inputs": "bf16 N(0,1)/sqrt(128), K rows L2-normalised; fp32 state and output",
                   "cache": "cold: %d rotating input/output sets (%.0f MB each)" % (
                       len(sets), (nbytes + 0) / 1e6)},
        "value": B * T / (ms_step * 1e-3),
        "ms_per_step": ms_step,
        "gpu_ms_per_step": gpu_ms,
        "phase_ms": {"segment_states": sum(phase[0]) / len(phase[0]),
                     "state_scan": sum(phase[1]) / len(phase[1]),
                     "chunk_walk": walk_ms},
        "mfma_frac": flops / (ms_step * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
        "hbm_gbs": nbytes / (ms_step * 1e-3) / 1e9,
        "roofline": {"kernel": "k_chunk_walk<bf16,64,128>", "bound": "hbm",
                     "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic,
                     "algorithmic_bytes": nbytes,
                     "algorithmic_flops": flops},
        "warm": {"gpu_ms_per_step": sum(per_step_w) / len(per_step_w),
                 "tokens_per_s": B * T / (sum(per_step_w) / len(per_step_w) * 1e-3),
                 "chunk_walk_ms": sum(phase_w[2]) / len(phase_w[2]),
                 "mfma_frac": flops / (sum(per_step_w) / len(per_step_w) * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)},
    }
    if not args.no_cpu_baseline:
        threads = args.cpu_threads
        qc, kc, vc = (x.cpu() for x in (q0, k0, v0))
        secs = time_oracle_prefill(qc, kc, vc, threads)
        res["cpu_baseline"] = {"value": B * T / secs, "unit": "tokens/s", "cores": threads,
                               "kind": "oracle", "seconds": secs,
                               "sample": "the whole workload (%d heads x %d tokens), float64 "
                                         "token-by-token recurrence, one head per thread" % (B * H, T)}
    del sets
    torch.cuda.empty_cache()
    return res


def bench_decode(args, torch, lla, workloads):
    cfg = workloads.CONFIGS["c5"]
    dev = torch.device("cuda:0")
    B, H, T, C, d = cfg.B, cfg.H, cfg.T, cfg.C, cfg.dk
    S = lla.state_init(B, H, d, d, device=dev)
    # state from the seeded T=4096 prefill, in batch slices to bound memory
    slice_b = 32
    qa, ka, va = workloads.config_inputs(cfg, device=dev)
    o_tmp = torch.empty((slice_b, H, T, d), dtype=torch.float32, device=dev)
    for b0 in range(0, B, slice_b):
        lla.prefill(qa[b0:b0 + slice_b], ka[b0:b0 + slice_b], va[b0:b0 + slice_b],
                    S[b0:b0 + slice_b], chunk=C, out=o_tmp)
    torch.cuda.synchronize()
    S_start = S[:8].cpu()
    del qa, ka, va, o_tmp
    torch.cuda.empty_cache()
    n = args.decode_steps
    qd, kd, vd = workloads.decode_inputs(cfg, n + args.warmup, device=dev)
    o = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        lla.decode_step(qd[n + i], kd[n + i], vd[n + i], S, out=o)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(n):
        lla.decode_step(qd[i], kd[i], vd[i], S, out=o)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(n)]
    ms_step = wall * 1e3 / n
    kern_ms = sum(per) / n
    nbytes = decode_bytes(B, H, d)
    res = {
        "workload": cfg.name, "B": B, "H": H, "dk": d, "dv": d, "steps": n,
        "value": n / wall, "unit": "steps/s", "ms_per_step": ms_step,
        "tokens_per_s": B * n / wall,
        "hbm_frac": nbytes / (ms_step * 1e-3) / (PEAK_HBM_GBS * 1e9),
        "roofline": {"kernel": "k_decode_step<bf16,4,16>", "bound": "hbm",
                     "achieved": nbytes / (kern_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": nbytes / (kern_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "traffic": None, "algorithmic_bytes": nbytes},
    }
    if not args.no_cpu_baseline:
        # n decode steps of one (b,h) are n iterations of the recurrence from
        # its state: time the oracle on 8 sequences x all heads x 128 steps.
        import oracle
        nb, ns = 8, min(128, n)
        qs, ks, vs = (x[:ns, :nb].permute(1, 2, 0, 3).contiguous().cpu() for x in (qd, kd, vd))
        threads = args.cpu_threads
        t0 = time.perf_counter()
        oracle.recurrence(qs, ks, vs, S_start[:nb], nthreads=threads)
        secs = time.perf_counter() - t0
        head_steps_per_s = nb * H * ns / secs
        res["cpu_baseline"] = {"value": head_steps_per_s / (B * H), "unit": "steps/s",
                               "cores": threads, "kind": "oracle", "seconds": secs,
                               "sample": "%d sequences x %d heads x %d decode steps (float64), "
                                         "scaled to the %d states of one step" % (nb, H, ns, B * H)}
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=512)
    ap.add_argument("--rotate", type=int, default=4, help="input/output sets cycled (cold cache)")
    ap.add_argument("--prefill-config", default="c3")
    ap.add_argument("--cpu-threads", type=int, default=min(16, os.cpu_count() or 1))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-decode", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: every (b,h) stream is independent, so the "
              "multi-GPU path shards (b,h) with no communication; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import decode_lla_prefill_amd as lla
    import workloads
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    lla.library()
    torch.cuda.set_device(0)

    pre = bench_prefill(args, torch, lla, workloads)
    line = {
        "metric": METRIC, "value": pre["value"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "config": pre["config"], "mfma_frac": pre["mfma_frac"],
        "hbm_gbs": pre["hbm_gbs"], "gpu_ms_per_step": pre["gpu_ms_per_step"],
        "phase_ms": pre["phase_ms"], "roofline": pre["roofline"], "warm": pre["warm"],
    }
    if "cpu_baseline" in pre:
        line["cpu_baseline"] = pre["cpu_baseline"]
    if not args.skip_decode:
        line["decode"] = bench_decode(args, torch, lla, workloads)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
