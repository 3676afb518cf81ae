"""The boundary is a C ABI: a plain C99 program includes include/lla.h
(compiled with -pedantic -Werror), links against liblla.so and calls the
host-only entry points -- the planners, an argument check that fails before
any HIP call, and the status strings.  No GPU is touched."""
import os
import shutil
import subprocess

import pytest

import decode_lla_prefill_amd as lla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include "lla.h"
#include <stdio.h>

int main(void) {
    size_t ws = lla_prefill_workspace_size(1, 16, 8192, 128, 128, 64);
    size_t ws_gqa = lla_prefill_gqa_workspace_size(1, 16, 4, 8192, 128, 128, 64);
    long long G = (long long)lla_prefill_segment_chunks(1, 16, 8192, 128, 128, 64);
    lla_status null_q = lla_prefill(NULL, NULL, NULL, LLA_BF16, 1, 1, 8, 2, 2, 4,
                                    NULL, NULL, NULL, 0, NULL);
    lla_status bad_flags = lla_prefill_ex((void *)16, (void *)32, (void *)48, LLA_BF16, 1, 1, 1, 8,
                                          2, 2, 4, 4u, (float *)64, (float *)80, NULL, 0, NULL);
    lla_status null_s = lla_state_commit((void *)16, (void *)32, LLA_BF16, 1, 1, 4, 64, 64, NULL, NULL, NULL);
    printf("%zu %zu %lld %d %d %d %d|%s\n", ws, ws_gqa, G, (int)null_q, (int)bad_flags, (int)null_s,
           lla_last_device_error(), lla_status_string(LLA_ERR_SHAPE));
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_plain_c_program_uses_the_library(tmp_path):
    src = tmp_path / "consumer.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(lla.library_path)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I" + os.path.join(ROOT, "include"), str(src), "-L" + libdir, "-llla",
                    "-Wl,-rpath," + libdir, "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.strip()
    nums, text = out.split("|")
    ws, ws_gqa, G, null_q, bad_flags, null_s, dev_err = (int(x) for x in nums.split())
    assert ws == 16 * 16 * 128 * 128 * 4   # 16 heads x 16 segments x one fp32 state
    assert ws_gqa == 4 * 16 * 128 * 128 * 4  # the segment states belong to the 4 key/value heads
    assert G == 8
    assert null_q == 1 and bad_flags == 4 and null_s == 1  # LLA_ERR_NULL, LLA_ERR_UNSUPPORTED
    assert dev_err == 0
    assert text == lla.library().lla_status_string(2).decode()
