"""The host-side code under the address and undefined-behaviour sanitizers
(CPU only, no GPU call).

The oracle (lla_oracle.c) and the library's host code (argument checking,
status strings, the plan) are rebuilt with -fsanitize=address,undefined and
no recovery, so the first finding aborts.  A child process with the
sanitizer runtime preloaded then runs the oracle's pins (test_oracle.py,
test_oracle_gated.py) and the C ABI's host checks (test_abi_host.py,
test_gated_host.py) against those builds.  A planted
out-of-bounds read in a throwaway C function, built and loaded the same way,
must abort, which shows the sanitizers are live in that setting."""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN_OPTIONS = "detect_leaks=0:halt_on_error=1"
UBSAN_OPTIONS = "halt_on_error=1:print_stacktrace=1"


@pytest.fixture(scope="module")
def sanitized():
    from decode_lla_prefill_amd import build as lla_build
    import oracle
    out = os.path.join(ROOT, "_build", "asan")
    lib = lla_build.build_sanitized(out)
    olib = oracle.build_sanitized(out)
    env = dict(os.environ, LD_PRELOAD=lla_build.asan_runtime(), LLA_LIBRARY=lib,
               LLA_ORACLE_LIBRARY=olib, ASAN_OPTIONS=ASAN_OPTIONS, UBSAN_OPTIONS=UBSAN_OPTIONS)
    return lib, olib, env


def _child(env, *args, timeout=600):
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


def test_the_sanitized_builds_are_the_ones_loaded(sanitized):
    lib, olib, env = sanitized
    r = _child(env, "-c", "import decode_lla_prefill_amd as l, oracle; l.library(); oracle._load(); "
                          "print(open('/proc/self/maps').read())")
    assert r.returncode == 0, r.stderr[-2000:]
    assert lib in r.stdout and olib in r.stdout
    assert "libclang_rt.asan" in r.stdout


def test_a_planted_out_of_bounds_read_aborts(sanitized, tmp_path):
    _, _, env = sanitized
    src = tmp_path / "planted.c"
    src.write_text(textwrap.dedent("""
        int planted(int n) { int a[4] = {1, 2, 3, 4}; volatile int *p = a; return p[n]; }
    """))
    so = tmp_path / "libplanted.so"
    subprocess.run(["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-fPIC", "-shared",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", str(so), str(src)],
                   check=True)
    r = _child(env, "-c", "import ctypes; print(ctypes.CDLL(%r).planted(4))" % str(so))
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr


def test_oracle_pins_and_abi_host_checks_under_sanitizers(sanitized):
    _, _, env = sanitized
    r = _child(env, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
               "tests/test_oracle.py", "tests/test_abi_host.py", "tests/test_oracle_gated.py",
               "tests/test_gated_host.py")
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout and "error" not in r.stdout.splitlines()[-1]
