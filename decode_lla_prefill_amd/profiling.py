"""Kernel runs for hardware-counter passes, and summaries of rocprofv3 output.

    python -m decode_lla_prefill_amd.profiling run [--launches N]
        On cuda:0: N prefill steps of the T=8192 workload (B=1, H=16, C=64,
        d=128; state init and the three phases, over rotating input sets),
        N decode steps of the 256 x 32 x 128 x 128 state, N grouped decode
        steps (256 sequences, 32 query heads on 8 key/value heads, three
        rotating state sets), and N device-to-device copies of 1 GiB, the
        reference of known size for the HBM byte counters.  Meant to run
        under ``rocprofv3 --pmc``.

    python -m decode_lla_prefill_amd.profiling stats OUT_DIR
        Per-kernel launch durations from a ``rocprofv3 --kernel-trace --stats
        --output-format csv`` directory: the tool's own per-name table, then
        the trace split by grid size (one kernel can run on several shapes).

    python -m decode_lla_prefill_amd.profiling traffic KERNEL FETCH_DIR WRITE_DIR
        HBM bytes per launch of KERNEL (a key of KERNELS) from a
        FETCH_SIZE pass and a WRITE_SIZE pass of ``run``: each counter is
        scaled by what it reads for the 1 GiB copy, whose true traffic is
        1 GiB read and 1 GiB written.  Prints ``key = value`` lines; bench.py
        reads ``hbm_bytes_per_launch`` while ``kernel_source_sha`` still
        matches the kernel's sources.
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

# measured kernel -> (name fragment in the trace, launch grid in threads of
# the bench workload, counter summary file, sources that define the kernel)
KERNELS = {
    "chunk_walk": ("k_chunk_walk", 16 * 16 * 2 * 256, "chunk_walk_T8192_traffic.txt",
                   ("lla_prefill.hip", "lla_device.h")),
    "decode_step": ("k_decode_step", 256 * 32 * 512, "decode_step_B256_H32_traffic.txt",
                    ("lla_decode.hip", "lla_device.h")),
    "decode_group": ("k_decode_group", 256 * 8 * 512, "decode_group_B256_Hq32_Hkv8_traffic.txt",
                     ("lla_decode.hip", "lla_device.h")),
}


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

def run(launches: int) -> None:
    import torch
    sys.path.insert(0, ROOT)
    import workloads
    from . import PreparedDecode, PreparedPrefill, library, state_init

    library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = workloads.CONFIGS["prefill_T8192"]
    q0, k0, v0 = workloads.config_inputs(cfg, device=dev)
    sets, keep = [], []
    for r in range(4):
        q, k, v = (x.clone() for x in (q0, k0, v0)) if r else (q0, k0, v0)
        S = state_init(cfg.B, cfg.H, cfg.dk, cfg.dv, device=dev)
        sets.append(PreparedPrefill(q, k, v, S, cfg.C))
        keep.append((q, k, v))
    for i in range(launches):
        st = sets[i % len(sets)]
        st.zero_state()
        st.segment_states()
        st.state_scan()
        st.chunks()
    torch.cuda.synchronize()
    print("prefill: %d steps" % launches, flush=True)
    del sets, keep
    torch.cuda.empty_cache()

    dc = workloads.CONFIGS["decode_B256"]
    S = state_init(dc.B, dc.H, dc.dk, dc.dv, device=dev)
    qd, kd, vd = workloads.decode_inputs(dc, launches, device=dev)
    calls = [PreparedDecode(qd[i], kd[i], vd[i], S) for i in range(launches)]
    for c in calls:
        c()
    torch.cuda.synchronize()
    print("decode: %d steps" % launches, flush=True)
    del calls, S
    torch.cuda.empty_cache()

    gc = workloads.CONFIGS["decode_B256_gqa"]
    S0 = workloads.random_state(gc, device=dev)
    states = [S0] + [S0.clone() for _ in range(2)]
    qd, kd, vd = workloads.decode_inputs(gc, launches, device=dev)
    calls = [PreparedDecode(qd[i], kd[i], vd[i], states[i % 3]) for i in range(launches)]
    for c in calls:
        c()
    torch.cuda.synchronize()
    print("grouped decode: %d steps" % launches, flush=True)
    del calls, states, S0
    torch.cuda.empty_cache()

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


def _pick(means: dict, fragment: str, grid: int | None):
    hits = [(k, v) for k, v in means.items() if fragment in k[0] and (grid is None or k[1] == grid)]
    if len(hits) != 1:
        raise SystemExit("expected one (kernel, grid) matching %r grid %s, found %d"
                         % (fragment, grid, len(hits)))
    return hits[0]


def traffic(kernel: str, fetch_dir: str, write_dir: str) -> None:
    frag, grid, _, _ = KERNELS[kernel]
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")
    (kname, _), (f_kib, f_n) = _pick(fetch, frag, grid)
    _, (w_kib, w_n) = _pick(write, frag, grid)
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


def main(argv=None):
    ap = argparse.ArgumentParser(prog="python -m decode_lla_prefill_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--launches", type=int, default=8)
    s = sub.add_parser("stats")
    s.add_argument("directory")
    t = sub.add_parser("traffic")
    t.add_argument("kernel", choices=sorted(KERNELS))
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    a = ap.parse_args(argv)
    if a.cmd == "run":
        run(a.launches)
    elif a.cmd == "stats":
        stats(a.directory)
    else:
        traffic(a.kernel, a.fetch_dir, a.write_dir)


if __name__ == "__main__":
    main()
