"""lla_prefill_noalloc (the prefill with the workspace in the library's static
per-device array, for callers that cannot allocate) against lla_prefill_ex
with a caller workspace, through the C ABI: bit for bit, on two calls in a row
whose second input is smaller than the first (the array keeps the first
call's states), then a third with shared-state heads and an incoming state."""
import numpy as np
import pytest
import torch

import decode_lla_prefill_amd as lla
import workloads
from gpu_util import need_gpu, np64

pytestmark = pytest.mark.gpu


def _both(q, k, v, S0, C, zero_state, dev):
    """(o, S) from lla_prefill_noalloc and from lla_prefill_ex on the same inputs."""
    q, k, v = (x.to(dev).contiguous() for x in (q, k, v))
    S_a, S_b = S0.to(dev).clone(), S0.to(dev).clone()
    o_a = lla.prefill_noalloc(q, k, v, S_a, chunk=C, zero_state=zero_state)
    o_b = lla.prefill(q, k, v, S_b, chunk=C, zero_state=zero_state)
    torch.cuda.synchronize()
    return (np64(o_a), np64(S_a)), (np64(o_b), np64(S_b))


def test_noalloc_equals_caller_workspace_on_two_calls_the_second_smaller():
    dev = need_gpu()
    # 1) 4 heads x 64 segments of 64 KiB = 16 MiB of segment states
    B, H, T, d, C = 1, 4, 4096, 128, 64
    assert lla.prefill_workspace_size(B, H, T, d, d, C) == 16 << 20
    print("noalloc call 1", B, H, T, d, C, flush=True)
    q, k, v = workloads.gaussian(B, H, T, d, d, seed_base=500, scale=d ** -0.5)
    a, b = _both(q, k, v, torch.full((B, H, d, d), float("nan")), C, True, dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.isfinite(a[0]).all()
    # 2) smaller: 2 heads x 16 segments at d = 64, integer inputs from a nonzero S_0
    B, H, T, d, C = 1, 2, 1000, 64, 64
    assert 0 < lla.prefill_workspace_size(B, H, T, d, d, C) < 16 << 20
    print("noalloc call 2", B, H, T, d, C, flush=True)
    q, k, v = workloads.integers(B, H, T, d, d, seed=501)
    S0 = torch.randint(-20, 21, (B, H, d, d), generator=torch.Generator().manual_seed(502)).float()
    a, b = _both(q, k, v, S0, C, False, dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_noalloc_grouped_heads_and_short_prompts():
    dev = need_gpu()
    print("noalloc grouped", flush=True)
    q, k, v = workloads.gaussian(2, 8, 700, 128, 128, seed_base=510, scale=128 ** -0.5, Hkv=2)
    S0 = torch.randn((2, 2, 128, 128), generator=torch.Generator().manual_seed(511))
    a, b = _both(q, k, v, S0, 64, False, dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # a short prompt (fused decode steps: no workspace) and an empty one
    q, k, v = workloads.gaussian(1, 4, 5, 128, 128, seed_base=512, scale=128 ** -0.5)
    a, b = _both(q, k, v, S0[:1, :1].expand(1, 4, 128, 128).contiguous(), 64, False, dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    q, k, v = (x[:, :, :0] for x in (q, k, v))
    a, b = _both(q, k, v, torch.ones((1, 4, 128, 128)), 64, True, dev)
    assert np.array_equal(a[1], b[1]) and (a[1] == 0).all()


def test_noalloc_one_launch_published_sums_on_calls_in_a_row():
    """Fresh prompts on the one-launch route, whose segments publish their
    sums in the static array: three calls in a row with new inputs and other
    layouts (the array keeps the earlier calls' sums and flags), each bit for
    bit the call with a caller workspace."""
    dev = need_gpu()
    for r, (B, H, T, d, C) in enumerate(((4, 8, 1024, 64, 64), (2, 8, 1024, 64, 64), (4, 8, 1024, 64, 64))):
        print("noalloc one launch", r, B, H, T, d, C, flush=True)
        q, k, v = workloads.gaussian(B, H, T, d, d, seed_base=520 + r, scale=d ** -0.5)
        a, b = _both(q, k, v, torch.full((B, H, d, d), float("nan")), C, True, dev)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), r
