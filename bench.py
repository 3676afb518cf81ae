"""Benchmark: causal linear-attention prefill and decode on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Prints ONE JSON line.  ``value`` is prefill throughput in tokens/s (B*T per
second) on the T=8192 workload (B=1, H=16, C=64, d_k=d_v=128, bf16 Q/K/V,
fp32 state and output); the decode workload (256 sequences x 32 heads,
d=128, state from a seeded T=4096 prefill) is reported under ``decode`` in
steps/s.  The same two workloads with query heads grouped four to a
key/value head (shared states) are reported under ``grouped_heads``, with
FP8 (E4M3) inputs under ``fp8_inputs``, and with a decayed state (one gate
per head and token, S_t = g_t S_{t-1} + k_t v_t^T) under ``gated_state``.

Prefill is timed cold: the timed steps rotate over several input/output
sets whose total exceeds the 256 MB Infinity Cache, so each step's inputs
come from HBM; a warm figure (one set repeated) is given for context.  A
second pass calls the three prefill phases one by one with HIP events
between them on the launch stream (per-phase times, launch gaps included),
and a third times back-to-back launches of the dominant kernel, the chunk
walk, for the roofline.  The decode step is one kernel: HIP events around
the timed steps give its launch time.  Every back-to-back launch also waits
out the dispatch gap in front of it; the run measures that gap once
(near-empty launches replayed from a HIP graph) and each roofline takes it
off, keeping the raw back-to-back figure beside it.

``roofline.traffic`` is the HBM traffic per launch that the hardware
counters measured (FETCH_SIZE + WRITE_SIZE, calibrated against a plain
copy), read from the committed counter summary under profiles/ when that
was taken on the current kernel source, else null.

The CPU baseline is the float64 oracle (the token-by-token recurrence) on
the host cores, timed on a bounded sample of the same workloads.

``measured_peaks`` holds what this GPU sustains on a plain 1 GiB stream and a
large bf16 GEMM (both through torch); the headline fractions are given
against those too (``frac_of_measured_stream``, ``mfma_frac_of_measured_gemm``)
beside the fractions of the published peaks.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 matrix cores, TFLOP/s
# fp32 vector FMA without packed instructions (the kernels are built without
# them): 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz; the published
# 157.3 TFLOP/s counts packed FMA
PEAK_F32_VALU_TFLOPS = 78.6
METRIC = "prefill tokens/s + % bf16 MFMA peak; decode steps/s + % HBM BW (1 GPU)"
def prefill_work(B, H, T, C, d, Hkv=None, in_bytes=2):
    """Algorithmic flops and bytes of one prefill (kept triangle only), with
    H query heads on Hkv key/value heads (default: one each) and inputs of
    `in_bytes` bytes per element (2: bf16, 1: FP8).

    flops per query-head token: 2d(C+1) (scores + masked scores x V over the
    kept triangle) + 2d^2 (Q S); per key/value-head token: 2d^2 (K^T V) +
    d^2/C (the state add per chunk).  bytes per query-head token: Q (d
    elements) + 4d (fp32 O); per key/value-head token: K and V (2d
    elements); plus 8d^2 per key/value head for reading S_0 and writing S_T.
    """
    Hkv = Hkv or H
    tq, tkv = B * H * T, B * Hkv * T
    flops = tq * (2 * d * (C + 1) + 2 * d * d) + tkv * (2 * d * d + d * d / C)
    nbytes = tq * (in_bytes + 4) * d + tkv * 2 * in_bytes * d + B * Hkv * 8 * d * d
    return flops, nbytes


def decode_bytes(B, H, d, Hkv=None, in_bytes=2):
    """Per step: per key/value head the fp32 state read + write (8d^2) and
    k, v (2d elements); per query head q (d elements) and fp32 o (4d)."""
    Hkv = Hkv or H
    return B * Hkv * (8 * d * d + 2 * in_bytes * d) + B * H * (in_bytes + 4) * d


def tokens_roofline(kernel, nbytes, fmas, ms):
    """Roofline of a fused short continuation: its HBM bytes against the
    HBM peak and its fp32 FMAs (state updates and reads, on the vector ALU)
    against the vector peak; the bound is whichever needs more time."""
    secs = ms * 1e-3
    t_hbm, t_alu = nbytes / (PEAK_HBM_GBS * 1e9), 2 * fmas / (PEAK_F32_VALU_TFLOPS * 1e12)
    hbm = {"achieved": nbytes / secs / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    alu = {"achieved": 2 * fmas / secs / 1e12, "peak": PEAK_F32_VALU_TFLOPS, "unit": "TFLOP/s"}
    r = dict(alu if t_alu > t_hbm else hbm)
    r.update({"kernel": kernel, "bound": "alu" if t_alu > t_hbm else "hbm",
              "frac": r["achieved"] / r["peak"], "hbm_frac": hbm["achieved"] / PEAK_HBM_GBS,
              "alu_frac": alu["achieved"] / PEAK_F32_VALU_TFLOPS, "algorithmic_bytes": nbytes,
              "fp32_fmas": fmas, "kernel_ms": ms, "timing": "HIP events around back-to-back calls"})
    return r


def repeat_for(fn, min_seconds):
    """Runs fn() until at least min_seconds have passed; returns (calls, seconds)."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        secs = time.perf_counter() - t0
        if secs >= min_seconds:
            return reps, secs


def _timed(torch, fn, n_steps):
    """Wall clock and GPU-event time of n_steps calls of fn(i), synchronised on both sides."""
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(n_steps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return time.perf_counter() - t0, e0.elapsed_time(e1) * 1e-3


def _step_events(torch, fn, n_steps):
    """GPU time of each of n_steps calls of fn(i), in ms: one HIP event on the
    launch stream between consecutive calls (so each interval also holds the
    gap before its call).  A pass of its own, after the wall-clock one."""
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(n_steps):
        fn(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    return [evs[i].elapsed_time(evs[i + 1]) for i in range(n_steps)]


def spread(ms):
    """Median and spread of per-step times (ms)."""
    s = sorted(ms)
    pick = lambda f: s[min(len(s) - 1, int(round(f * (len(s) - 1))))]
    return {"median_ms": statistics.median(s), "mean_ms": sum(s) / len(s), "min_ms": s[0],
            "p10_ms": pick(0.1), "p90_ms": pick(0.9), "max_ms": s[-1], "n": len(s),
            "timing": "HIP events between consecutive steps on the launch stream"}


def host_cores():
    """Threads for the CPU oracle, and the host's core counts.  All cores this
    process may run on, except where the environment sets a CPU share per
    process (OMP_NUM_THREADS, as a GPU machine does for its one GPU): more
    threads than that share would only oversubscribe it."""
    affinity = len(os.sched_getaffinity(0))
    share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = min(affinity, share) if share > 0 else affinity
    return threads, {"logical_cpus": os.cpu_count(), "cpus_in_affinity": affinity,
                     "omp_num_threads": share or None,
                     "why": "all cores in this process's affinity mask, capped by OMP_NUM_THREADS "
                            "(the CPU share the environment gives this process) when it is set"}


def launch_gap_ms(torch, lla, n=64, reps=10):
    """GPU time per launch of back-to-back launches of an almost empty kernel
    (lla_state_init on one 4 x 4 state: one workgroup), replayed from a HIP
    graph so that host launch overhead stays out: the dispatch gap that timing
    back-to-back launches adds to each kernel, plus that tiny kernel itself."""
    dev = torch.device("cuda:0")
    S = torch.empty((1, 1, 4, 4), device=dev)
    lla.state_init(1, 1, 4, 4, out=S)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            lla.state_init(1, 1, 4, 4, out=S)
    for _ in range(3):
        g.replay()
    _, secs = _timed(torch, lambda i: g.replay(), reps)
    del g
    return secs * 1e3 / (n * reps)


def hbm_roofline(kernel, nbytes, b2b_ms, gap_ms, traffic=None, timing="", **extra):
    """Roofline of an HBM-bound kernel: algorithmic bytes per launch over its
    launch duration.  b2b_ms is the per-launch time of back-to-back launches
    between HIP events on the launch stream; each of those launches also
    waits out the dispatch gap before it, measured separately (launch_gap_ms),
    so the launch duration is b2b_ms - gap_ms -- what a kernel trace reports
    for the kernel.  Both raw figures are kept."""
    ms = b2b_ms - gap_ms
    r = {"kernel": kernel, "bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
         "unit": "GB/s", "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "traffic": traffic,
         "algorithmic_bytes": nbytes, "kernel_ms": ms, "kernel_ms_back_to_back": b2b_ms,
         "launch_gap_ms": gap_ms, "frac_back_to_back": nbytes / (b2b_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
         "timing": timing + "; kernel_ms = kernel_ms_back_to_back - launch_gap_ms"}
    r.update(extra)
    return r


def measure_peaks(torch):
    """Achievable peaks of this GPU, measured for context beside the published
    ones.  HBM: the best of two plain streams over 1 GiB fp32 (torch's
    out-of-place add, which reads 1 GiB and writes 1 GiB, and torch's
    device-to-device copy).  Matrix cores: torch.mm in bf16 (fp32
    accumulate), 16384 x 16384 x 16384 with the second operand transposed,
    the layout the GEMM library runs fastest."""
    dev = torch.device("cuda:0")
    n, reps = 1 << 28, 20
    src = torch.ones(n, device=dev)
    dst = torch.empty_like(src)
    streams = {}
    for name, fn in (("add", lambda i: torch.add(src, 1.0, out=dst)), ("copy", lambda i: dst.copy_(src))):
        for i in range(3):
            fn(i)
        _, secs = _timed(torch, fn, reps)
        streams[name] = 2 * n * 4 * reps / secs / 1e9
    del src, dst
    m, mreps = 16384, 10
    g = torch.Generator(device=dev).manual_seed(0)
    a = torch.randn((m, m), generator=g, device=dev).bfloat16()
    bt = torch.randn((m, m), generator=g, device=dev).bfloat16()
    c = torch.empty((m, m), dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        torch.mm(a, bt.t(), out=c)
    _, secs = _timed(torch, lambda i: torch.mm(a, bt.t(), out=c), mreps)
    gemm_tflops = 2 * m ** 3 * mreps / secs / 1e12
    del a, bt, c
    torch.cuda.empty_cache()
    stream_gbs = max(streams.values())
    return {
        "stream_gbs": stream_gbs, "stream_frac_of_spec": stream_gbs / PEAK_HBM_GBS,
        "stream_by_kind_gbs": streams,
        "bf16_gemm_tflops": gemm_tflops, "bf16_gemm_frac_of_spec": gemm_tflops / PEAK_BF16_TFLOPS,
        "how": "stream: best of torch add (out of place) and copy over 1 GiB fp32, %d calls each, "
               "bytes read + written; GEMM: torch.mm bf16 %d^3 (A times B transposed), %d calls; "
               "HIP events around each batch" % (reps, m, mreps),
    }


# the walk kernel of each prefill workload: (label, key of its counter summary,
# whether a fresh-prompt step is that one kernel alone -- the one-launch walk,
# whose workgroups sum the earlier segments themselves)
WALK_OF_CONFIG = {
    "prefill_T8192": ("k_chunk_walk_wide<64> (bf16, d=128)", "chunk_walk", False),
    "prefill_B4_T1024": ("k_chunk_walk<bf16,64,64,64,...,one launch> (four waves, d=64, C=64; the whole "
                         "fresh-prompt step)", "chunk_walk_T1024", True),
    "prefill_T131072": ("k_chunk_walk_wide<64> (bf16, d=128; C=128 run as two 64-token chunks)",
                        "chunk_walk_T131072", False),
}


def bench_prefill(args, torch, lla, workloads, profiling):
    cfg = workloads.CONFIGS[args.prefill_config]
    dev = torch.device("cuda:0")
    B, H, T, C, d = cfg.B, cfg.H, cfg.T, cfg.C, cfg.dk
    q0, k0, v0 = workloads.config_inputs(cfg, device=dev)
    sets, ins = [], []
    for r in range(args.rotate):
        q, k, v = (x.clone() for x in (q0, k0, v0)) if r else (q0, k0, v0)
        S = lla.state_init(B, H, d, d, device=dev)
        sets.append(lla.PreparedPrefill(q, k, v, S, C))
        ins.append((q, k, v))
    n_sets = len(sets)

    # One step = one fresh-prompt prefill: lla_prefill_ex with the zero-state
    # option (S_0 = 0 without reading S; S receives S_T).
    def step(i):
        sets[i % n_sets](zero_state=True)

    for i in range(args.warmup):
        step(i)
    wall, gpu = _timed(torch, step, args.steps)
    wall_w, gpu_w = _timed(torch, lambda i: sets[0](zero_state=True), args.steps)
    cold_spread = spread(_step_events(torch, step, args.steps))
    warm_spread = spread(_step_events(torch, lambda i: sets[0](zero_state=True), args.steps))

    # Per-phase durations: the same work with HIP events between the three
    # phases (what lla_prefill enqueues; the state is zeroed by lla_state_init
    # before them), on the launch stream.  An interval between two events
    # also holds the launch gap in front of the kernel.
    stream = torch.cuda.current_stream(dev)
    evs = []
    torch.cuda.synchronize()
    for i in range(args.steps):
        st = sets[i % n_sets]
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        st.zero_state()
        ev[0].record(stream)
        st.segment_states()
        ev[1].record(stream)
        st.state_scan()
        ev[2].record(stream)
        st.chunks()
        ev[3].record(stream)
        evs.append(ev)
    torch.cuda.synchronize()
    phase = [[ev[j].elapsed_time(ev[j + 1]) for ev in evs] for j in range(3)]

    # The chunk walk's launch duration: back-to-back walks over the rotating
    # sets between two events.  Every set's workspace holds its segment
    # states from the pass above, and a walk reads only those, q, k and v, so
    # the repeated walks are the same work as the one inside a step.
    # A workload whose fresh-prompt step is the one-launch walk times the
    # steps themselves.
    one_launch = WALK_OF_CONFIG.get(args.prefill_config, (None, None, False))[2]
    n_walk = max(args.steps, 4 * n_sets)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(n_walk):
        if one_launch:
            sets[i % n_sets](zero_state=True)
        else:
            sets[i % n_sets].chunks()
    e1.record(stream)
    torch.cuda.synchronize()
    walk_launch_ms = e0.elapsed_time(e1) / n_walk
    gap_ms = args.gap_ms
    flops, nbytes = prefill_work(B, H, T, C, d)
    ms_step = wall * 1e3 / args.steps
    walk_ms = sum(phase[2]) / len(phase[2])
    res = {
        "config": {"workload": cfg.name, "B": B, "H": H, "T": T, "C": C, "dk": d, "dv": d,
                   "inputs": "bf16 N(0,1)/sqrt(128), K rows L2-normalised; fp32 state and output",
                   "cache": "cold: %d rotating input/output sets of %.0f MB" % (n_sets, nbytes / 1e6),
                   "step": "one fresh-prompt lla_prefill_ex (S_0 = 0): " + (
                       "one launch, each segment's walk summing the earlier segments' K^T V" if one_launch
                       else "per-segment K^T V, segment scan, chunk walk")},
        "value": B * T / (ms_step * 1e-3),
        "ms_per_step": ms_step,
        "gpu_ms_per_step": gpu * 1e3 / args.steps,
        "step_spread": cold_spread,
        "phase_ms": {"segment_states": sum(phase[0]) / len(phase[0]),
                     "state_scan": sum(phase[1]) / len(phase[1]),
                     "chunk_walk": walk_ms},
        "head_tokens_per_s": B * H * T / (ms_step * 1e-3),
        "tflops": flops / (ms_step * 1e-3) / 1e12,  # algorithmic (kept triangle)
        "mfma_frac": flops / (ms_step * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
        "hbm_gbs": nbytes / (ms_step * 1e-3) / 1e9,
        # the step against its attainable roofline: min(MFMA peak, AI x HBM peak)
        "attainable": {"ms_at_roof": max(flops / (PEAK_BF16_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBS * 1e9)) * 1e3,
                       "frac": max(flops / (PEAK_BF16_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBS * 1e9))
                               / (ms_step * 1e-3),
                       "bound": "hbm" if nbytes / (PEAK_HBM_GBS * 1e9) > flops / (PEAK_BF16_TFLOPS * 1e12)
                                else "mfma"},
        "roofline": hbm_roofline(WALK_OF_CONFIG.get(args.prefill_config, ("chunk walk", None))[0], nbytes,
                                 walk_launch_ms, gap_ms,
                                 profiling.stored_traffic(WALK_OF_CONFIG[args.prefill_config][1])
                                 if args.prefill_config in WALK_OF_CONFIG else None,
                                 "HIP events around %d back-to-back walk launches" % n_walk,
                                 algorithmic_flops=flops),
        "warm": {"ms_per_step": wall_w * 1e3 / args.steps,
                 "tokens_per_s": B * T / (wall_w / args.steps),
                 "mfma_frac": flops / (wall_w / args.steps) / (PEAK_BF16_TFLOPS * 1e12),
                 "step_spread": warm_spread,
                 "cache": "warm: one input/output set repeated (Infinity-Cache resident)"},
    }
    if not args.no_cpu_baseline:
        import oracle
        threads = args.cpu_threads
        qc, kc, vc = (x.cpu() for x in (q0, k0, v0))
        reps, secs = repeat_for(lambda: oracle.recurrence(qc, kc, vc, nthreads=threads),
                                args.cpu_seconds)
        res["cpu_baseline"] = {"value": reps * B * T / secs, "unit": "tokens/s", "cores": threads,
                               "host": args.host, "kind": "oracle", "seconds": secs,
                               "sample": "the whole workload (%d heads x %d tokens) %d times over, "
                                         "float64 token-by-token recurrence, one head per thread"
                                         % (B * H, T, reps)}
        # one core: one head of the workload, scaled to all B*H heads
        q1, k1, v1 = (x[:1, :1] for x in (qc, kc, vc))
        reps1, secs1 = repeat_for(lambda: oracle.recurrence(q1, k1, v1, nthreads=1), 2.0)
        res["cpu_baseline"]["single_thread"] = {
            "value": reps1 * T / secs1 / (B * H) * B, "unit": "tokens/s", "cores": 1,
            "seconds": secs1, "sample": "one head (%d tokens) %d times over, scaled to the %d heads"
                                        % (T, reps1, B * H)}
    del sets
    torch.cuda.empty_cache()
    return res


def bench_decode(args, torch, lla, workloads, profiling):
    cfg = workloads.CONFIGS["decode_B256"]
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
    calls = [lla.PreparedDecode(qd[i], kd[i], vd[i], S, out=o) for i in range(n + args.warmup)]
    for i in range(args.warmup):
        calls[n + i]()
    # The step is one kernel, so the events around the timed steps give its
    # per-launch duration directly.
    wall, gpu = _timed(torch, lambda i: calls[i](), n)
    kern_ms = gpu * 1e3 / n
    ms_step = wall * 1e3 / n
    nbytes = decode_bytes(B, H, d)
    # per-step spread over a second pass (the steps continue from the state)
    n_sp = min(n, 100)
    dec_spread = spread(_step_events(torch, lambda i: calls[i](), n_sp))
    res = {
        "workload": cfg.name, "B": B, "H": H, "dk": d, "dv": d, "steps": n,
        "value": n / wall, "unit": "steps/s", "ms_per_step": ms_step,
        "gpu_ms_per_step": gpu * 1e3 / n,
        "tokens_per_s": B * n / wall,
        "step_spread": dec_spread,
        "hbm_frac": nbytes / (ms_step * 1e-3) / (PEAK_HBM_GBS * 1e9),
        "roofline": hbm_roofline("k_decode_step_sq<bf16,128,512>", nbytes, kern_ms, args.gap_ms,
                                 profiling.stored_traffic("decode_step"), "HIP events around the timed steps"),
    }
    # Short continuations from the same states: T tokens per call through
    # lla_prefill (the fused path for T <= 16).
    res["continuation"] = []
    for tc in (4, 16):
        qc, kc, vc = (x.permute(1, 2, 0, 3).contiguous()
                      for x in workloads.decode_inputs(cfg, tc, device=dev))
        call = lla.PreparedPrefill(qc, kc, vc, S, C)
        for _ in range(3):
            call()
        nc = 50
        wall_c, gpu_c = _timed(torch, lambda i: call(), nc)
        ms_c = gpu_c * 1e3 / nc
        cbytes = B * H * (8 * d * d + tc * 10 * d)
        fmas = B * H * tc * 2 * d * d  # per head and token: the update and the read
        res["continuation"].append({
            "tokens_per_call": tc, "value": B * tc * nc / wall_c, "unit": "tokens/s",
            "ms_per_call": wall_c * 1e3 / nc, "gpu_ms_per_call": ms_c,
            "roofline": tokens_roofline("k_decode_tokens<bf16,128,512>", cbytes, fmas, ms_c)})
        del call, qc, kc, vc

    # Speculative decoding at k = 4 draft tokens: the verify pass
    # (lla_prefill_ex with LLA_PREFILL_KEEP_STATE: S read, not written) and
    # the commit of each sequence's accepted prefix (lla_state_commit; the
    # accepted counts m_b, uniform in 0..4 from a fixed seed, stay on the
    # device).  Together they equal m_b decode steps bit for bit.
    kd_ = 4
    qs, ks, vs = (x.permute(1, 2, 0, 3).contiguous() for x in workloads.decode_inputs(cfg, kd_, device=dev))
    acc = torch.randint(0, kd_ + 1, (B,), generator=torch.Generator(device=dev).manual_seed(cfg.seed_base + 7),
                        device=dev, dtype=torch.int32)
    n_acc = int(acc.sum())
    S_spec = S.clone()
    verify = lla.PreparedPrefill(qs, ks, vs, S_spec, C)
    for _ in range(3):
        verify(keep_state=True)
        lla.state_commit(ks, vs, S_spec, acc)
    ns = 50
    _, v_s = _timed(torch, lambda i: verify(keep_state=True), ns)
    _, c_s = _timed(torch, lambda i: lla.state_commit(ks, vs, S_spec, acc), ns)
    wall_p, gpu_p = _timed(torch, lambda i: (verify(keep_state=True), lla.state_commit(ks, vs, S_spec, acc)), ns)
    v_ms, c_ms = v_s * 1e3 / ns, c_s * 1e3 / ns
    n_commit = int((acc > 0).sum())
    v_bytes = B * H * (4 * d * d + kd_ * 10 * d)  # S read; q, k, v bf16 and fp32 o per token
    c_bytes = n_commit * H * 8 * d * d + n_acc * H * 4 * d  # S read + written where m_b > 0; k, v of accepted tokens
    res["speculative"] = {
        "draft_tokens": kd_, "accepted_tokens_per_call": n_acc, "sequences_committing": n_commit,
        "accepted": "m_b uniform in 0..%d per sequence (seed %d), on the device" % (kd_, cfg.seed_base + 7),
        "value": n_acc * ns / wall_p, "unit": "accepted tokens/s",
        "draft_tokens_per_s": B * kd_ * ns / wall_p, "ms_per_call_pair": wall_p * 1e3 / ns,
        "gpu_ms_per_call_pair": gpu_p * 1e3 / ns,
        "verify": hbm_roofline("k_decode_tokens<bf16,128,512> (keep state)", v_bytes, v_ms, args.gap_ms, None,
                               "HIP events around %d back-to-back verify calls" % ns),
        "commit": hbm_roofline("k_state_commit_sq<bf16,128,512>", c_bytes, c_ms, args.gap_ms, None,
                               "HIP events around %d back-to-back commits" % ns),
    }
    del verify, qs, ks, vs, S_spec

    if not args.no_cpu_baseline:
        # n decode steps of one (b,h) are n iterations of the recurrence from
        # its state: time the oracle on 8 sequences x all heads x 128 steps.
        import oracle
        nb, ns = 8, min(128, n)
        qs, ks, vs = (x[:ns, :nb].permute(1, 2, 0, 3).contiguous().cpu() for x in (qd, kd, vd))
        threads = args.cpu_threads
        reps, secs = repeat_for(lambda: oracle.recurrence(qs, ks, vs, S_start[:nb], nthreads=threads),
                                args.cpu_seconds)
        head_steps_per_s = reps * nb * H * ns / secs
        res["cpu_baseline"] = {"value": head_steps_per_s / (B * H), "unit": "steps/s",
                               "cores": threads, "host": args.host, "kind": "oracle", "seconds": secs,
                               "sample": "%d sequences x %d heads x %d decode steps (float64), "
                                         "%d times over, scaled to the %d states of one step"
                                         % (nb, H, ns, reps, B * H)}
    return res


def bench_other_prefills(args, torch, lla, workloads, profiling):
    """The small (B=4, H=8, T=1024, d=64) and the very long (B=1, H=32,
    T=131072, C=128) prefill workloads: cold fresh-prompt steps over rotating
    input sets, back-to-back walks for the walk kernel's roofline, and the
    oracle on the whole workload."""
    import oracle
    dev = torch.device("cuda:0")
    out = []
    walks = WALK_OF_CONFIG
    for name, rotate, steps in (("prefill_B4_T1024", 16, args.steps), ("prefill_T131072", 2, 6)):
        cfg = workloads.CONFIGS[name]
        B, H, T, C, d = cfg.B, cfg.H, cfg.T, cfg.C, cfg.dk
        q0, k0, v0 = workloads.config_inputs(cfg, device=dev)
        sets = []
        for r in range(rotate):
            q, k, v = (x.clone() for x in (q0, k0, v0)) if r else (q0, k0, v0)
            sets.append(lla.PreparedPrefill(q, k, v, lla.state_init(B, H, d, d, device=dev), C))
        for i in range(max(2, args.warmup if name == "prefill_B4_T1024" else 1)):
            sets[i % rotate](zero_state=True)
        wall, gpu = _timed(torch, lambda i: sets[i % rotate](zero_state=True), steps)
        cold_spread = spread(_step_events(torch, lambda i: sets[i % rotate](zero_state=True), steps))
        wall_w, _ = _timed(torch, lambda i: sets[0](zero_state=True), steps)
        warm_spread = spread(_step_events(torch, lambda i: sets[0](zero_state=True), steps))
        n_walk = max(steps, 2 * rotate)
        if walks[name][2]:  # the step is the walk
            _, walk_s = _timed(torch, lambda i: sets[i % rotate](zero_state=True), n_walk)
        else:
            _, walk_s = _timed(torch, lambda i: sets[i % rotate].chunks(), n_walk)
        walk_ms = walk_s * 1e3 / n_walk
        flops, nbytes = prefill_work(B, H, T, C, d)
        step_s = gpu / steps
        line = {"workload": cfg.name, "B": B, "H": H, "T": T, "C": C, "dk": d, "dv": d,
                "value": B * T / (wall / steps), "unit": "tokens/s", "steps": steps,
                "ms_per_step": wall * 1e3 / steps, "gpu_ms_per_step": step_s * 1e3,
                "step_spread": cold_spread,
                "warm": {"ms_per_step": wall_w * 1e3 / steps, "tokens_per_s": B * T / (wall_w / steps),
                         "step_spread": warm_spread,
                         "cache": "warm: one input/output set repeated"},
                "mfma_frac": flops / step_s / (PEAK_BF16_TFLOPS * 1e12),
                "hbm_frac": nbytes / step_s / (PEAK_HBM_GBS * 1e9),
                "cache": "cold: %d rotating input/output sets of %.0f MB" % (rotate, nbytes / 1e6),
                "roofline": hbm_roofline(walks[name][0], nbytes, walk_ms, args.gap_ms,
                                         profiling.stored_traffic(walks[name][1]),
                                         "HIP events around %d back-to-back %s" % (
                                             n_walk, "fresh-prompt steps (one launch each)" if walks[name][2]
                                             else "walk launches"))}
        del sets
        torch.cuda.empty_cache()
        if not args.no_cpu_baseline:
            qc, kc, vc = (x.cpu() for x in (q0, k0, v0))
            t0 = time.perf_counter()
            oracle.recurrence(qc, kc, vc, nthreads=args.cpu_threads)
            secs = time.perf_counter() - t0
            line["cpu_baseline"] = {"value": B * T / secs, "unit": "tokens/s", "cores": args.cpu_threads,
                                    "host": args.host, "kind": "oracle", "seconds": secs,
                                    "sample": "the whole workload once (%d heads x %d tokens), float64 "
                                              "token-by-token recurrence" % (B * H, T)}
            del qc, kc, vc
        del q0, k0, v0
        torch.cuda.empty_cache()
        out.append(line)
    return out


def bench_grouped(args, torch, lla, workloads, profiling):
    """Shared-state heads: the T=8192 prefill with 16 query heads on 4
    key/value heads, and the decode batch with 32 query heads on 8."""
    dev = torch.device("cuda:0")
    cfg = workloads.CONFIGS["prefill_T8192_gqa"]
    B, H, Hkv, T, C, d = cfg.B, cfg.H, cfg.kv_heads, cfg.T, cfg.C, cfg.dk
    q0, k0, v0 = workloads.config_inputs(cfg, device=dev)
    sets = []
    for r in range(args.rotate):
        q, k, v = (x.clone() for x in (q0, k0, v0)) if r else (q0, k0, v0)
        sets.append(lla.PreparedPrefill(q, k, v, lla.state_init(B, Hkv, d, d, device=dev), C))
    for i in range(args.warmup):
        sets[i % len(sets)](zero_state=True)
    wall, gpu = _timed(torch, lambda i: sets[i % len(sets)](zero_state=True), args.steps)
    flops, nbytes = prefill_work(B, H, T, C, d, Hkv)
    step_s = gpu / args.steps
    pre = {"workload": cfg.name, "B": B, "Hq": H, "Hkv": Hkv, "T": T, "C": C, "dk": d, "dv": d,
           "value": B * T / (wall / args.steps), "unit": "tokens/s",
           "ms_per_step": wall * 1e3 / args.steps, "gpu_ms_per_step": step_s * 1e3,
           "mfma_frac": flops / step_s / (PEAK_BF16_TFLOPS * 1e12),
           "hbm_frac": nbytes / step_s / (PEAK_HBM_GBS * 1e9),
           "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
           "timing": "HIP events around the timed steps (fresh-prompt lla_prefill_ex), "
                     "%d rotating input sets" % len(sets)}
    del sets, q0, k0, v0
    torch.cuda.empty_cache()

    cfg = workloads.CONFIGS["decode_B256_gqa"]
    B, H, Hkv, d = cfg.B, cfg.H, cfg.kv_heads, cfg.dk
    # The grouped states (134 MB) would fit in the 256 MB Infinity Cache:
    # the steps cycle over three state sets so that every step reads its
    # states from HBM, as the layers of a model would.
    S0 = workloads.random_state(cfg, device=dev)
    S = [S0] + [S0.clone() for _ in range(2)]
    n = args.decode_steps
    qd, kd, vd = workloads.decode_inputs(cfg, n + args.warmup, device=dev)
    o = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    calls = [lla.PreparedDecode(qd[i], kd[i], vd[i], S[i % 3], out=o) for i in range(n + args.warmup)]
    for i in range(args.warmup):
        calls[n + i]()
    wall, gpu = _timed(torch, lambda i: calls[i](), n)
    kern_ms = gpu * 1e3 / n
    nbytes = decode_bytes(B, H, d, Hkv)
    dec = {"workload": cfg.name, "B": B, "Hq": H, "Hkv": Hkv, "dk": d, "dv": d, "steps": n,
           "value": n / wall, "unit": "steps/s", "ms_per_step": wall * 1e3 / n,
           "gpu_ms_per_step": kern_ms, "tokens_per_s": B * n / wall,
           "roofline": hbm_roofline("k_decode_group<bf16,128,512>", nbytes, kern_ms, args.gap_ms,
                                    profiling.stored_traffic("decode_group"),
                                    "HIP events around the timed steps, cycling over 3 state sets")}
    # Short continuations with shared-state heads: T tokens per call through
    # lla_prefill_gqa (T * G <= 64: fused grouped decode steps below 8
    # tokens, one chunk on the matrix cores from 8 on), from the cycled
    # state sets.
    dec["continuation"] = []
    for tc in (4, 16):
        qc, kc, vc = (x.permute(1, 2, 0, 3).contiguous()
                      for x in workloads.decode_inputs(cfg, tc, device=dev))
        cont = [lla.PreparedPrefill(qc, kc, vc, S[i], cfg.C) for i in range(3)]
        for i in range(3):
            cont[i]()
        nc = 48
        wall_c, gpu_c = _timed(torch, lambda i: cont[i % 3](), nc)
        ms_c = gpu_c * 1e3 / nc
        cbytes = B * Hkv * (8 * d * d + tc * 4 * d) + B * H * tc * 6 * d
        # the method's flops per call: per state K^T V (2 d^2 T); per query
        # head and token the state read (2 d^2) and the kept scores times V
        # (about 2 d t for token t)
        flops = B * Hkv * 2 * d * d * tc + B * H * (2 * d * d * tc + 2 * d * tc * (tc + 1) // 2 * 2)
        matrix = tc >= 8
        kname = "k_tokens_grouped_pipe<bf16> (matrix cores)" if matrix else \
            "k_decode_tokens<bf16> (fused decode steps)"
        r = hbm_roofline(kname, cbytes, ms_c, args.gap_ms,
                         profiling.stored_traffic("tokens_grouped") if tc == 16 else None,
                         "HIP events around %d back-to-back calls cycling over 3 state sets" % nc)
        r["algorithmic_flops"] = flops
        if matrix:
            r["mfma_frac"] = flops / (r["kernel_ms"] * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)
        dec["continuation"].append({
            "tokens_per_call": tc, "value": B * tc * nc / wall_c, "unit": "tokens/s",
            "gpu_ms_per_call": ms_c, "roofline": r})
        del cont, qc, kc, vc
    del calls, qd, kd, vd, S, S0
    torch.cuda.empty_cache()
    return {"prefill": pre, "decode": dec}


def bench_fp8(args, torch, lla, workloads, profiling):
    """FP8 (E4M3) inputs: the T=8192 prefill and the 256 x 32 decode batch."""
    dev = torch.device("cuda:0")
    cfg = workloads.CONFIGS["prefill_T8192_fp8"]
    B, H, T, C, d = cfg.B, cfg.H, cfg.T, cfg.C, cfg.dk
    q0, k0, v0 = workloads.config_inputs(cfg, device=dev)
    sets = []
    for r in range(args.rotate):
        q, k, v = (x.clone() for x in (q0, k0, v0)) if r else (q0, k0, v0)
        sets.append(lla.PreparedPrefill(q, k, v, lla.state_init(B, H, d, d, device=dev), C))
    for i in range(args.warmup):
        sets[i % len(sets)](zero_state=True)
    wall, gpu = _timed(torch, lambda i: sets[i % len(sets)](zero_state=True), args.steps)
    # the walk alone, back to back (every set's workspace holds its segment states)
    n_walk = max(args.steps, 4 * len(sets))
    _, walk_s = _timed(torch, lambda i: sets[i % len(sets)].chunks(), n_walk)
    walk_ms = walk_s * 1e3 / n_walk
    flops, nbytes = prefill_work(B, H, T, C, d, in_bytes=1)
    step_s = gpu / args.steps
    pre = {"workload": cfg.name, "B": B, "H": H, "T": T, "C": C, "dk": d, "dv": d,
           "inputs": "FP8 E4M3 N(0,1); fp32 state and output",
           "value": B * T / (wall / args.steps), "unit": "tokens/s",
           "ms_per_step": wall * 1e3 / args.steps, "gpu_ms_per_step": step_s * 1e3,
           "mfma_frac": flops / step_s / (PEAK_BF16_TFLOPS * 1e12),
           "hbm_frac": nbytes / step_s / (PEAK_HBM_GBS * 1e9),
           "roofline": hbm_roofline("k_chunk_walk_wide<64, fp8e4m3>", nbytes, walk_ms, args.gap_ms,
                                    profiling.stored_traffic("chunk_walk_fp8"),
                                    "HIP events around %d back-to-back walk launches" % n_walk),
           "timing": "HIP events around the timed steps (fresh-prompt lla_prefill_ex), "
                     "%d rotating input sets" % len(sets)}
    del sets, q0, k0, v0
    torch.cuda.empty_cache()

    cfg = workloads.CONFIGS["decode_B256_fp8"]
    B, H, d = cfg.B, cfg.H, cfg.dk
    S = workloads.random_state(cfg, device=dev)  # 512 MB: larger than the Infinity Cache
    n = args.decode_steps
    qd, kd, vd = workloads.decode_inputs(cfg, n + args.warmup, device=dev)
    o = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    calls = [lla.PreparedDecode(qd[i], kd[i], vd[i], S, out=o) for i in range(n + args.warmup)]
    for i in range(args.warmup):
        calls[n + i]()
    wall, gpu = _timed(torch, lambda i: calls[i](), n)
    kern_ms = gpu * 1e3 / n
    nbytes = decode_bytes(B, H, d, in_bytes=1)
    dec = {"workload": cfg.name, "B": B, "H": H, "dk": d, "dv": d, "steps": n,
           "value": n / wall, "unit": "steps/s", "ms_per_step": wall * 1e3 / n,
           "gpu_ms_per_step": kern_ms, "tokens_per_s": B * n / wall,
           "roofline": hbm_roofline("k_decode_step_sq<fp8e4m3,128,512>", nbytes, kern_ms, args.gap_ms,
                                    None, "HIP events around the timed steps")}
    del calls, qd, kd, vd, S
    torch.cuda.empty_cache()
    return {"prefill": pre, "decode": dec}


def bench_gated(args, torch, lla, workloads, profiling):
    """Gated (decayed) state, S_t = g_t S_{t-1} + k_t v_t^T with gates in
    [0.9, 1]: the T=8192 prefill and the 256 x 32 decode batch."""
    dev = torch.device("cuda:0")
    cfg = workloads.CONFIGS["prefill_T8192"]
    B, H, T, C, d = cfg.B, cfg.H, cfg.T, cfg.C, cfg.dk
    q0, k0, v0 = workloads.config_inputs(cfg, device=dev)
    g0 = workloads.gates(B, H, T, seed=cfg.seed_base + 9, device=dev)
    sets = []
    for r in range(args.rotate):
        q, k, v, g = (x.clone() for x in (q0, k0, v0, g0)) if r else (q0, k0, v0, g0)
        sets.append(lla.PreparedGatedPrefill(q, k, v, g, torch.empty((B, H, d, d), device=dev), C))
    for i in range(args.warmup):
        sets[i % len(sets)](zero_state=True)
    wall, gpu = _timed(torch, lambda i: sets[i % len(sets)](zero_state=True), args.steps)
    flops, nbytes = prefill_work(B, H, T, C, d)
    nbytes += B * H * T * 4  # the gates
    step_ms = gpu * 1e3 / args.steps
    pre = {"workload": cfg.name + "_gated", "B": B, "H": H, "T": T, "C": C, "dk": d, "dv": d,
           "gates": "uniform in [0.9, 1], one per (b,h) and token",
           "value": B * T / (wall / args.steps), "unit": "tokens/s",
           "ms_per_step": wall * 1e3 / args.steps, "gpu_ms_per_step": step_ms,
           "mfma_frac": flops / (step_ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
           # the whole step (segment pass, scan, walk) against the step's algorithmic bytes
           "roofline": hbm_roofline("fresh-prompt lla_prefill_gated step (k_gated_segment_states, "
                                    "k_gated_state_scan, k_gated_walk<bf16,64,128,64>)", nbytes, step_ms,
                                    0.0, None, "HIP events around %d back-to-back steps, %d rotating input sets"
                                    % (args.steps, len(sets))),
           "timing": "HIP events around the timed steps"}
    del sets, q0, k0, v0, g0
    torch.cuda.empty_cache()

    cfg = workloads.CONFIGS["decode_B256"]
    B, H, d = cfg.B, cfg.H, cfg.dk
    S = workloads.random_state(cfg, device=dev)
    n = args.decode_steps
    qd, kd, vd = workloads.decode_inputs(cfg, n + args.warmup, device=dev)
    gd = workloads.gates(n + args.warmup, B, H, seed=cfg.seed_base + 9, device=dev)
    o = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    calls = [lla.PreparedGatedDecode(qd[i], kd[i], vd[i], gd[i], S, out=o) for i in range(n + args.warmup)]
    for i in range(args.warmup):
        calls[n + i]()
    wall, gpu = _timed(torch, lambda i: calls[i](), n)
    kern_ms = gpu * 1e3 / n
    nbytes = decode_bytes(B, H, d) + B * H * 4
    dec = {"workload": cfg.name + "_gated", "B": B, "H": H, "dk": d, "dv": d, "steps": n,
           "value": n / wall, "unit": "steps/s", "ms_per_step": wall * 1e3 / n,
           "gpu_ms_per_step": kern_ms, "tokens_per_s": B * n / wall,
           "roofline": hbm_roofline("k_decode_step_sq<bf16,128,512,gated>", nbytes, kern_ms, args.gap_ms,
                                    profiling.stored_traffic("gated_decode"), "HIP events around the timed steps")}
    del calls, qd, kd, vd, gd, S
    torch.cuda.empty_cache()
    return {"prefill": pre, "decode": dec}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=512)
    ap.add_argument("--rotate", type=int, default=4, help="input/output sets cycled (cold cache)")
    ap.add_argument("--prefill-config", default="prefill_T8192")
    ap.add_argument("--cpu-threads", type=int, default=None,
                    help="oracle threads (default: every core this process may use, see host_cores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum oracle time of each CPU baseline (the sample is repeated)")
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--skip-grouped", action="store_true")
    ap.add_argument("--skip-other", action="store_true", help="skip the B=4 T=1024 and T=131072 prefills")
    ap.add_argument("--skip-fp8", action="store_true")
    ap.add_argument("--skip-gated", action="store_true")
    args = ap.parse_args()
    threads, args.host = host_cores()
    if args.cpu_threads is None:
        args.cpu_threads = threads

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: every (b,h) stream is independent, so the "
              "multi-GPU path shards (b,h) with no communication; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import decode_lla_prefill_amd as lla
    from decode_lla_prefill_amd import profiling
    import workloads
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    lla.library()
    torch.cuda.set_device(0)
    args.gap_ms = launch_gap_ms(torch, lla)

    pre = bench_prefill(args, torch, lla, workloads, profiling)
    line = {
        "metric": METRIC, "value": pre["value"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "config": pre["config"], "head_tokens_per_s": pre["head_tokens_per_s"],
        "tflops": pre["tflops"], "mfma_frac": pre["mfma_frac"], "launch_gap_ms": args.gap_ms,
        "hbm_gbs": pre["hbm_gbs"], "attainable": pre["attainable"],
        "gpu_ms_per_step": pre["gpu_ms_per_step"],
        "phase_ms": pre["phase_ms"], "roofline": pre["roofline"], "warm": pre["warm"],
        "step_spread": pre["step_spread"],
        "timing": "value and ms_per_step: wall clock over the timed steps (synchronised on both "
                  "sides); gpu_ms_per_step: HIP events around them; step_spread: a HIP event "
                  "between consecutive steps in a pass of its own (median, p10/p90, min/max); "
                  "phase_ms: HIP events between the phases in a second pass of the same steps "
                  "(launch gaps included); roofline kernel_ms: HIP events around back-to-back "
                  "launches, less the launch gap (back-to-back near-empty launches replayed from "
                  "a HIP graph), which every back-to-back launch also waits out",
    }
    if "cpu_baseline" in pre:
        line["cpu_baseline"] = pre["cpu_baseline"]
    if not args.skip_other:
        line["other_prefills"] = bench_other_prefills(args, torch, lla, workloads, profiling)
    if not args.skip_decode:
        line["decode"] = bench_decode(args, torch, lla, workloads, profiling)
    if not args.skip_grouped:
        line["grouped_heads"] = bench_grouped(args, torch, lla, workloads, profiling)
    if not args.skip_fp8:
        line["fp8_inputs"] = bench_fp8(args, torch, lla, workloads, profiling)
    if not args.skip_gated:
        line["gated_state"] = bench_gated(args, torch, lla, workloads, profiling)
    peaks = measure_peaks(torch)
    line["measured_peaks"] = peaks
    # the same figures against what this GPU measurably sustains
    line["roofline"]["frac_of_measured_stream"] = line["roofline"]["achieved"] / peaks["stream_gbs"]
    line["mfma_frac_of_measured_gemm"] = line["mfma_frac"] * PEAK_BF16_TFLOPS / peaks["bf16_gemm_tflops"]
    if "decode" in line:
        r = line["decode"]["roofline"]
        r["frac_of_measured_stream"] = r["achieved"] / peaks["stream_gbs"]
    print(json.dumps(line))


if __name__ == "__main__":
    main()
