"""Build liblla.so (HIP, gfx950) in-tree.

    python -m decode_lla_prefill_amd.build

Every translation unit is compiled with hipcc for gfx950 only, with packed
fp32 vector instructions disabled (``-target-feature -packed-fp32-ops``; the
host pass warns that it does not know that feature, which is harmless), then
linked into ``decode_lla_prefill_amd/liblla.so`` next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "liblla.so")
BUILD_DIR = os.path.join(ROOT, "_build", "lla")

SOURCES = ["lla_abi.cpp", "lla_plan.cpp", "lla_prefill.hip", "lla_decode.hip", "lla_noalloc.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def _compile(src: str, extra=()) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(extra_flags=(), out: str = OUT, verbose: bool = False) -> str:
    """Compile all sources (in parallel) and link ``liblla.so``."""
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        raise RuntimeError("hipcc not found (%s)" % HIPCC)
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra_flags), SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


# Host-side sources: argument checking, status codes and the plan.  They hold
# no kernels, so a plain host compiler builds them.
HOST_SOURCES = ["lla_abi.cpp", "lla_plan.cpp"]
SANITIZE_DIR = os.path.join(ROOT, "_build", "asan")
CLANGXX = os.environ.get("LLA_CLANGXX", "/opt/rocm/llvm/bin/clang++")


def _newest_source() -> float:
    import glob
    files = glob.glob(os.path.join(CSRC, "*")) + [os.path.join(ROOT, "include", "lla.h")]
    return max(os.path.getmtime(f) for f in files)


def asan_runtime() -> str:
    """The address-sanitizer runtime of the ROCm clang (to preload into a
    process that loads a sanitized build)."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no clang address-sanitizer runtime under /opt/rocm/llvm")
    return hits[-1]


def build_sanitized(out_dir: str = SANITIZE_DIR) -> str:
    """A copy of liblla.so whose host code (HOST_SOURCES) is built with the
    address and undefined-behaviour sanitizers (clang++, no recovery: the
    first finding aborts), linked with the kernel objects of the regular
    build.  For CPU tests of the host-side paths, run with asan_runtime()
    preloaded; device code is not sanitized."""
    os.makedirs(out_dir, exist_ok=True)
    kernel_objs = [os.path.join(BUILD_DIR, s + ".o") for s in SOURCES if s not in HOST_SOURCES]
    stale = any(not os.path.exists(o) or os.path.getmtime(o) < _newest_source() for o in kernel_objs)
    if stale:
        build()  # the kernel objects under BUILD_DIR
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(out_dir, src + ".o")
        cmd = [CLANGXX, "-O1", "-g", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
               "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
               "-I" + CSRC, "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-fno-omit-frame-pointer", "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("sanitized compile failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
        objs.append(obj)
    objs += kernel_objs
    out = os.path.join(out_dir, "liblla.so")
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitized link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    return out


if __name__ == "__main__":
    build(extra_flags=sys.argv[1:], verbose=True)
