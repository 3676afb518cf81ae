"""Kernel runs for rocprofv3 passes, and summaries of rocprofv3 output.

    python -m decode_lla_prefill_amd.profiling run [--launches N] [--workloads W,W,...]
        On cuda:0, for each workload W (default: every key of WORKLOADS) N
        steps over rotating input sets: fresh-prompt prefills (the
        per-segment K^T V, the segment scan and the chunk walk, as the
        benchmark times them) or decode steps.  Then N device-to-device copies
        of 1 GiB, the reference of known size for the HBM byte counters.
        Meant to run under ``rocprofv3 --pmc`` or ``--kernel-trace``.

    python -m decode_lla_prefill_amd.profiling stats OUT_DIR
        Per-kernel launch durations from a ``rocprofv3 --kernel-trace --stats
        --output-format csv`` directory: the tool's own per-name table, then
        the trace split by grid size (one kernel can run on several shapes).

    python -m decode_lla_prefill_amd.profiling traffic KERNEL FETCH_DIR WRITE_DIR
        HBM bytes per launch of KERNEL (a key of KERNELS) from a FETCH_SIZE
        pass and a WRITE_SIZE pass of ``run``: each counter is scaled by what
        it reads for the 1 GiB copy, whose true traffic is 1 GiB read and
        1 GiB written.  Prints ``key = value`` lines; bench.py reads
        ``hbm_bytes_per_launch`` while ``kernel_source_sha`` still matches the
        kernel's sources.

    python -m decode_lla_prefill_amd.profiling counters KERNEL DIR [DIR ...] [--duration-us T]
        Per-dispatch means of every counter the ``--pmc`` directories hold for
        KERNEL, and what follows from them: MFMA utilisation (rocprofiler's
        MfmaUtil), the executed bf16 matrix-core flops (MfmaFlopsBF16) and,
        given the kernel's duration, their rate against the bf16 peak; the
        LDS and issue counters as shares of the wave cycles.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import os
import re
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(_HERE)
CSRC = os.path.join(_HERE, "csrc")
PROFILES = os.path.join(ROOT, "profiles")

COPY_BYTES = 1 << 30

# The workloads ``run`` can drive (keys of workloads.CONFIGS).
WORKLOADS = ("prefill_T8192", "prefill_T8192_fp8", "prefill_B4_T1024", "prefill_T131072",
             "decode_B256", "decode_B256_gqa", "decode_B256_gqa_T16", "prefill_T8192_gated",
             "decode_B256_gated")
# Workloads whose measured kernel has the name and the grid of another's
# (the T=131072 walk is the T=8192 walk's kernel on 256 workgroups too):
# their counters come from a run of their own, never from the default run.
RUN_ALONE = ("prefill_T131072",)
DEFAULT_RUN = tuple(w for w in WORKLOADS if w not in RUN_ALONE)

# what decides a prefill kernel's work: its code and the plan that cuts the
# shape into segments
PREFILL_SOURCES = ("lla_prefill.hip", "lla_device.h", "lla_plan.cpp", "lla_internal.h")

# measured kernel -> (name fragments as the trace shows them (mangled or
# demangled), launch grid in threads of its workload, counter summary file,
# sources that define the kernel, workload).  Grids follow from the plan
# (tests/test_profiling_host.py recomputes them).
KERNELS = {
    "chunk_walk": (("k_chunk_walk_wideILi64EDF16bLb0E", "k_chunk_walk_wide<64, __bf16, false>"), 16 * 16 * 512,
                   "chunk_walk_T8192_traffic.txt", PREFILL_SOURCES, "prefill_T8192"),
    "segment_states": (("k_segment_states_wideILi64EDF16bLb0E", "k_segment_states_wide<64, __bf16, false>"),
                       16 * 15 * 512, "segment_states_T8192_traffic.txt",
                       PREFILL_SOURCES, "prefill_T8192"),
    "state_scan": (("k_state_scan",), 16 * 16 * 256, "state_scan_T8192_traffic.txt",
                   PREFILL_SOURCES, "prefill_T8192"),
    "chunk_walk_fp8": (("k_chunk_walk_wideILi64ENS_7fp8e4m3ELb0E", "k_chunk_walk_wide<64, lla::fp8e4m3, false>"),
                       16 * 16 * 512, "chunk_walk_T8192_fp8_traffic.txt",
                       PREFILL_SOURCES, "prefill_T8192_fp8"),
    # a fresh T=1024 prompt is one launch: the four-wave walk whose
    # workgroups sum the earlier segments themselves (the last template flag)
    "chunk_walk_T1024": (("k_chunk_walkIDF16bLi64ELi64ELi64ELb1ELi4ELb1E",
                          "k_chunk_walk<__bf16, 64, 64, 64, true, 4, true>"),
                         32 * 8 * 256, "chunk_walk_B4_T1024_traffic.txt",
                         PREFILL_SOURCES, "prefill_B4_T1024"),
    # chunks of 128 run as two of 64 on the wide walk (counters from a run of
    # this workload alone: the kernel and grid are chunk_walk's)
    "chunk_walk_T131072": (("k_chunk_walk_wideILi64EDF16bLb0E", "k_chunk_walk_wide<64, __bf16, false>"),
                           32 * 8 * 512, "chunk_walk_T131072_traffic.txt",
                           PREFILL_SOURCES, "prefill_T131072"),
    "decode_step": (("k_decode_step_sqIDF16bLi128ELi512ELb0E", "k_decode_step_sq<__bf16, 128, 512, false>"),
                    256 * 32 * 512, "decode_step_B256_H32_traffic.txt",
                    ("lla_decode.hip", "lla_device.h"), "decode_B256"),
    "decode_group": (("k_decode_groupIDF16bLi128E", "k_decode_group<__bf16, 128,"), 256 * 8 * 512, "decode_group_B256_Hq32_Hkv8_traffic.txt",
                     ("lla_decode.hip", "lla_device.h"), "decode_B256_gqa"),
    # 16-token continuations of the grouped states: one persistent 8-wave
    # workgroup per compute unit, walking the key/value heads
    "tokens_grouped": (("k_tokens_grouped_pipeIDF16bE", "k_tokens_grouped_pipe<__bf16>"),
                       256 * 512, "tokens_grouped_B256_Hq32_Hkv8_T16_traffic.txt",
                       PREFILL_SOURCES, "decode_B256_gqa_T16"),
    # the gated (decayed) state: the T=8192 prefill's walk and segment pass
    # (the plain kernels with the GATED flag), and the decode step.  The
    # trace demangles the bf16-with-flag names as "<64, bool _Accum, bool, E>".
    "gated_walk": (("k_chunk_walk_wideILi64EDF16bLb1E", "k_chunk_walk_wide<64, __bf16, true>",
                    "k_chunk_walk_wide<64, bool _Accum, bool, E>"), 16 * 16 * 512,
                   "gated_walk_T8192_traffic.txt", PREFILL_SOURCES, "prefill_T8192_gated"),
    "gated_segment_states": (("k_segment_states_wideILi64EDF16bLb1E", "k_segment_states_wide<64, __bf16, true>",
                              "k_segment_states_wide<64, bool _Accum, bool, E>"),
                             16 * 15 * 512, "gated_segment_states_T8192_traffic.txt", PREFILL_SOURCES,
                             "prefill_T8192_gated"),
    "gated_decode": (("k_decode_step_sqIDF16bLi128ELi512ELb1E", "k_decode_step_sq<__bf16, 128, 512, true>"),
                     256 * 32 * 512, "gated_decode_B256_H32_traffic.txt", ("lla_decode.hip", "lla_device.h"),
                     "decode_B256_gated"),
}

SIMD_NUM = 256 * 4  # MI355X: 256 compute units of 4 SIMDs (the SIMD_NUM of MfmaUtil)
PEAK_BF16_TFLOPS = 2516.6


def matches(name: str, kernel: str) -> bool:
    return any(f in name for f in KERNELS[kernel][0])


def code_only(text: str) -> str:
    """C/C++ source without its comments, one space for each run of
    whitespace: what the compiler sees, so a reworded comment does not
    invalidate counters taken on the same code."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":  # string or character literal, copied whole
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_sha(kernel: str) -> str:
    """Digest of the code (comments and layout aside) of the sources that
    define `kernel` (a key of KERNELS)."""
    h = hashlib.sha256()
    for name in KERNELS[kernel][3]:
        with open(os.path.join(CSRC, name)) as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_summary(path: str) -> dict:
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                key, val = line.split("=", 1)
                kv[key.strip()] = val.strip()
    return kv


def stored_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from its committed counter summary,
    or None when that is missing or was taken on other kernel sources."""
    try:
        kv = read_summary(os.path.join(PROFILES, KERNELS[kernel][2]))
        if kv.get("kernel_source_sha") != kernel_source_sha(kernel):
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


# ---- the counter workload -------------------------------------------------------

def run(launches: int, which=DEFAULT_RUN) -> None:
    import torch
    sys.path.insert(0, ROOT)
    import workloads
    from . import (PreparedDecode, PreparedGatedDecode, PreparedGatedPrefill, PreparedPrefill, library,
                   state_init)

    library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    for name in which:
        cfg = workloads.CONFIGS.get(name)
        if name.startswith("prefill") and not name.endswith("_gated"):
            rotate = 2 if cfg.T >= 65536 else 4
            q0, k0, v0 = workloads.config_inputs(cfg, device=dev)
            sets = []
            for r in range(rotate):
                q, k, v = (x.clone() for x in (q0, k0, v0)) if r else (q0, k0, v0)
                S = torch.empty((cfg.B, cfg.kv_heads, cfg.dk, cfg.dv), device=dev)
                sets.append(PreparedPrefill(q, k, v, S, cfg.C))
            for i in range(launches):
                sets[i % rotate](zero_state=True)  # a fresh prompt: K^T V, scan, walk (or the one-launch walk)
            torch.cuda.synchronize()
            del sets, q0, k0, v0
        elif name == "decode_B256":
            S = state_init(cfg.B, cfg.H, cfg.dk, cfg.dv, device=dev)
            qd, kd, vd = workloads.decode_inputs(cfg, launches, device=dev)
            calls = [PreparedDecode(qd[i], kd[i], vd[i], S) for i in range(launches)]
            for c in calls:
                c()
            torch.cuda.synchronize()
            del calls, S, qd, kd, vd
        elif name == "prefill_T8192_gated":
            # the T=8192 prefill with a decayed state, gates in [0.9, 1]
            cfg = workloads.CONFIGS["prefill_T8192"]
            q0, k0, v0 = workloads.config_inputs(cfg, device=dev)
            g0 = workloads.gates(cfg.B, cfg.H, cfg.T, seed=cfg.seed_base + 9, device=dev)
            sets = []
            for r in range(4):
                q, k, v, g = (x.clone() for x in (q0, k0, v0, g0)) if r else (q0, k0, v0, g0)
                S = torch.empty((cfg.B, cfg.H, cfg.dk, cfg.dv), device=dev)
                sets.append(PreparedGatedPrefill(q, k, v, g, S, cfg.C))
            for i in range(launches):
                sets[i % 4](zero_state=True)
            torch.cuda.synchronize()
            del sets, q0, k0, v0, g0
        elif name == "decode_B256_gated":
            cfg = workloads.CONFIGS["decode_B256"]
            S = state_init(cfg.B, cfg.H, cfg.dk, cfg.dv, device=dev)
            qd, kd, vd = workloads.decode_inputs(cfg, launches, device=dev)
            gd = workloads.gates(launches, cfg.B, cfg.H, seed=cfg.seed_base + 9, device=dev)
            calls = [PreparedGatedDecode(qd[i], kd[i], vd[i], gd[i], S) for i in range(launches)]
            for c in calls:
                c()
            torch.cuda.synchronize()
            del calls, S, qd, kd, vd, gd
        elif name == "decode_B256_gqa_T16":
            # 16-token continuations of the grouped states, cycling over
            # three state sets (lla_prefill_gqa, short-prompt route)
            cfg = workloads.CONFIGS["decode_B256_gqa"]
            S0 = workloads.random_state(cfg, device=dev)
            states = [S0] + [S0.clone() for _ in range(2)]
            qc, kc, vc = (x.permute(1, 2, 0, 3).contiguous()
                          for x in workloads.decode_inputs(cfg, 16, device=dev))
            calls = [PreparedPrefill(qc, kc, vc, states[i], cfg.C) for i in range(3)]
            for i in range(launches):
                calls[i % 3]()
            torch.cuda.synchronize()
            del calls, states, S0, qc, kc, vc
        elif name == "decode_B256_gqa":
            # three state sets, so that each step reads its states from HBM
            S0 = workloads.random_state(cfg, device=dev)
            states = [S0] + [S0.clone() for _ in range(2)]
            qd, kd, vd = workloads.decode_inputs(cfg, launches, device=dev)
            calls = [PreparedDecode(qd[i], kd[i], vd[i], states[i % 3]) for i in range(launches)]
            for c in calls:
                c()
            torch.cuda.synchronize()
            del calls, states, S0, qd, kd, vd
        else:
            raise SystemExit("unknown workload %s" % name)
        torch.cuda.empty_cache()
        print("%s: %d steps" % (name, launches), flush=True)

    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(launches):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("copy: %d x %d bytes" % (launches, COPY_BYTES), flush=True)


# ---- rocprofv3 csv summaries ----------------------------------------------------

def _find(directory: str, suffix: str):
    files = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit("no *%s under %s" % (suffix, directory))
    return files


def _short(name: str) -> str:
    """Readable kernel name: demangled names lose their argument list."""
    return re.sub(r"\((?!anonymous).*", "", name)[:90]


def _grid(row: dict) -> int:
    for key in ("Grid_Size", "Grid_Size_X"):
        if key in row and row[key]:
            g = int(float(row[key]))
            for extra in ("Grid_Size_Y", "Grid_Size_Z"):
                if extra in row and row[extra]:
                    g *= int(float(row[extra]))
            return g
    return -1


def stats(directory: str) -> None:
    print("# per-name table (rocprofv3 --stats, kernel_stats.csv)")
    print("%-90s %6s %12s %10s %10s %10s" % ("kernel", "calls", "total_us", "avg_us", "min_us",
                                            "max_us"))
    for f in _find(directory, "kernel_stats.csv"):
        for r in csv.DictReader(open(f)):
            print("%-90s %6s %12.1f %10.2f %10.2f %10.2f" % (
                _short(r["Name"]), r["Calls"], float(r["TotalDurationNs"]) / 1e3,
                float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    print()
    print("# per (kernel, grid) from kernel_trace.csv; grid in threads")
    acc = collections.defaultdict(list)
    for f in _find(directory, "kernel_trace.csv"):
        for r in csv.DictReader(open(f)):
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            acc[(_short(r["Kernel_Name"]), _grid(r))].append(dur)
    print("%-90s %10s %6s %10s %10s %10s" % ("kernel", "grid", "calls", "avg_us", "min_us",
                                            "max_us"))
    for (name, grid), d in sorted(acc.items(), key=lambda kv: -sum(kv[1])):
        print("%-90s %10d %6d %10.2f %10.2f %10.2f" % (name, grid, len(d), sum(d) / len(d),
                                                      min(d), max(d)))


def _counter_means(directory: str, counter: str):
    """Mean counter value per (kernel, grid) over all dispatches."""
    acc = collections.defaultdict(list)
    for f in _find(directory, "counter_collection.csv"):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                acc[(r["Kernel_Name"], _grid(r))].append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def _copy_mean(directory: str, counter: str) -> float:
    """Mean counter value of the 1 GiB copies.  The runtime's copy kernel
    also serves smaller copies (tensor clones) on the same grid, so only the
    dispatches within a factor of two of the largest count are kept."""
    vals = []
    for f in _find(directory, "counter_collection.csv"):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and "copyBuffer" in r["Kernel_Name"]:
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit("no copy dispatches with %s under %s" % (counter, directory))
    big = [v for v in vals if v >= 0.5 * max(vals)]
    return sum(big) / len(big)


def _pick(means: dict, kernel: str, grid: int | None):
    hits = [(k, v) for k, v in means.items() if matches(k[0], kernel) and (grid is None or k[1] == grid)]
    if len(hits) != 1:
        raise SystemExit("expected one (kernel, grid) matching %r grid %s, found %d"
                         % (KERNELS[kernel][0], grid, len(hits)))
    return hits[0]


def traffic(kernel: str, fetch_dir: str, write_dir: str) -> None:
    grid = KERNELS[kernel][1]
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")
    (kname, _), (f_kib, f_n) = _pick(fetch, kernel, grid)
    _, (w_kib, w_n) = _pick(write, kernel, grid)
    cf_kib = _copy_mean(fetch_dir, "FETCH_SIZE")
    cw_kib = _copy_mean(write_dir, "WRITE_SIZE")
    f_scale = cf_kib * 1024.0 / COPY_BYTES   # counter bytes per true byte
    w_scale = cw_kib * 1024.0 / COPY_BYTES
    read_b = f_kib * 1024.0 / f_scale
    write_b = w_kib * 1024.0 / w_scale
    print("kernel = %s" % _short(kname))
    print("grid_threads = %d" % grid)
    print("kernel_source_sha = %s" % kernel_source_sha(kernel))
    print("dispatches_fetch = %d" % f_n)
    print("dispatches_write = %d" % w_n)
    print("fetch_kib_per_launch = %.1f" % f_kib)
    print("write_kib_per_launch = %.1f" % w_kib)
    print("copy_fetch_kib = %.1f" % cf_kib)
    print("copy_write_kib = %.1f" % cw_kib)
    print("copy_fetch_scale = %.4f" % f_scale)
    print("copy_write_scale = %.4f" % w_scale)
    print("hbm_read_bytes_per_launch = %.0f" % read_b)
    print("hbm_write_bytes_per_launch = %.0f" % write_b)
    print("hbm_bytes_per_launch = %.0f" % (read_b + write_b))


def _all_counter_means(directories, kernel: str):
    """{counter: (mean per dispatch, dispatches)} of KERNEL (at its workload's
    grid) over every counter_collection.csv under the directories."""
    grid = KERNELS[kernel][1]
    acc = collections.defaultdict(list)
    name = None
    for d in directories:
        for f in _find(d, "counter_collection.csv"):
            for r in csv.DictReader(open(f)):
                if matches(r["Kernel_Name"], kernel) and _grid(r) == grid:
                    acc[r["Counter_Name"]].append(float(r["Counter_Value"]))
                    name = r["Kernel_Name"]
    if not acc:
        raise SystemExit("no dispatches of %s (grid %d) under %s" % (kernel, grid, directories))
    return name, {c: (sum(v) / len(v), len(v)) for c, v in acc.items()}


def counters(kernel: str, directories, duration_us=None) -> None:
    kname, means = _all_counter_means(directories, kernel)
    print("kernel = %s" % _short(kname))
    print("grid_threads = %d" % KERNELS[kernel][1])
    print("kernel_source_sha = %s" % kernel_source_sha(kernel))
    for c in sorted(means):
        print("%s = %.6g    # mean of %d dispatches" % (c, means[c][0], means[c][1]))
    m = {c: v for c, (v, _) in means.items()}
    if "MfmaUtil" in m:
        print("mfma_util_percent = %.2f    # rocprofiler's MfmaUtil: sum of SQ_VALU_MFMA_BUSY_CYCLES "
              "/ (max GRBM_GUI_ACTIVE x %d SIMDs)" % (m["MfmaUtil"], SIMD_NUM))
    if "MfmaFlopsBF16" in m:
        print("mfma_flops_bf16_per_launch = %.6g    # executed: SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512"
              % m["MfmaFlopsBF16"])
        if duration_us:
            tf = m["MfmaFlopsBF16"] / (duration_us * 1e-6) / 1e12
            print("kernel_duration_us = %.3f" % duration_us)
            print("mfma_tflops_bf16 = %.2f" % tf)
            print("mfma_frac_of_bf16_peak = %.4f    # of %.1f TFLOP/s" % (tf / PEAK_BF16_TFLOPS, PEAK_BF16_TFLOPS))
    wave = m.get("SQ_WAVE_CYCLES")
    if wave:
        for c in ("SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
                  "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VALU", "SQ_INST_CYCLES_VMEM"):
            if c in m and c != "SQ_BUSY_CYCLES":
                print("%s_share_of_wave_cycles = %.4f" % (c.lower(), m[c] / wave))


def main(argv=None):
    ap = argparse.ArgumentParser(prog="python -m decode_lla_prefill_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--launches", type=int, default=8)
    r.add_argument("--workloads", default=",".join(DEFAULT_RUN),
                   help="comma-separated, of %s" % ",".join(WORKLOADS))
    s = sub.add_parser("stats")
    s.add_argument("directory")
    t = sub.add_parser("traffic")
    t.add_argument("kernel", choices=sorted(KERNELS))
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    c = sub.add_parser("counters")
    c.add_argument("kernel", choices=sorted(KERNELS))
    c.add_argument("directories", nargs="+")
    c.add_argument("--duration-us", type=float, default=None,
                   help="the kernel's average duration (kernel trace), for the MFMA rate")
    a = ap.parse_args(argv)
    if a.cmd == "run":
        run(a.launches, [w for w in a.workloads.split(",") if w])
    elif a.cmd == "stats":
        stats(a.directory)
    elif a.cmd == "traffic":
        traffic(a.kernel, a.fetch_dir, a.write_dir)
    else:
        counters(a.kernel, a.directories, a.duration_us)


if __name__ == "__main__":
    main()
