"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Bar: bit-exact on small-integer inputs (the deck's trace, its {0,1} toy
variants, {-1,0,1} inputs across tile counts, ragged tails and segment
counts); max|err|/max|ref| <= 2e-3 for bf16 inputs (all heads of the T=1024
and T=8192 shapes, four sampled heads of the T=131072 shape).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import TOL, gpu_prefill, need_gpu, np64, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def test_worked_trace_exact(dev):
    q, k, v = workloads.toy(0)
    o, S = gpu_prefill(q, k, v, C=4)
    assert np.array_equal(np64(o)[0, 0], [[2, 3], [5, 1], [3, 4], [5, 5], [3, 5], [7, 7], [4, 5], [7, 7]])
    assert np.array_equal(np64(S)[0, 0], [[4, 5], [7, 7]])


def test_toy_variants_exact(dev):
    for variant in range(0, 101):
        q, k, v = workloads.toy(variant)
        o, S = gpu_prefill(q, k, v, C=4)
        O_ref, S_ref = oracle.recurrence(q, k, v)
        assert np.array_equal(np64(o), O_ref), "variant %d outputs" % variant
        assert np.array_equal(np64(S), S_ref), "variant %d state" % variant


INT_CASES = [
    # B, H, T, dk, dv, C, dtype
    (2, 3, 200, 64, 64, 64, torch.bfloat16),
    (1, 2, 1000, 128, 128, 64, torch.bfloat16),
    (2, 2, 300, 128, 128, 128, torch.bfloat16),
    (1, 1, 7, 4, 4, 4, torch.bfloat16),
    (1, 3, 129, 5, 7, 16, torch.bfloat16),
    (3, 5, 64, 96, 80, 48, torch.bfloat16),
    (1, 1, 1, 128, 128, 64, torch.bfloat16),
    (1, 4, 12800, 128, 128, 64, torch.bfloat16),
    (1, 2, 65536, 32, 32, 64, torch.bfloat16),
    (1, 2, 2000, 64, 32, 32, torch.float32),
    (2, 1, 333, 128, 128, 64, torch.float32),
    (1, 1, 50, 3, 2, 7, torch.float32),
    (1, 2, 37, 16, 16, 1, torch.bfloat16),      # C = 1: the recurrence itself
    (2, 1, 300, 24, 40, 128, torch.bfloat16),   # C = 128 with odd head dims
    (1, 3, 500, 128, 128, 32, torch.bfloat16),  # C = 32 at d = 128
    (2, 2, 260, 104, 120, 20, torch.bfloat16),  # ragged chunks, partial columns
]


@pytest.mark.parametrize("B,H,T,dk,dv,C,dtype", INT_CASES)
def test_integer_inputs_exact(dev, B, H, T, dk, dv, C, dtype):
    q, k, v = workloads.integers(B, H, T, dk, dv, seed=T + dk + C, dtype=dtype)
    o, S = gpu_prefill(q, k, v, C=C)
    O_ref, S_ref = oracle.recurrence(q, k, v, nthreads=8)
    assert np.array_equal(np64(S), S_ref)
    assert np.array_equal(np64(o), O_ref)


def test_integer_inputs_with_incoming_state_exact(dev):
    q, k, v = workloads.integers(2, 3, 700, 64, 64, seed=5)
    g = torch.Generator().manual_seed(6)
    S0 = torch.randint(-40, 41, (2, 3, 64, 64), generator=g).float()
    o, S = gpu_prefill(q, k, v, C=64, S0=S0)
    O_ref, S_ref = oracle.recurrence(q, k, v, S0, nthreads=6)
    assert np.array_equal(np64(o), O_ref) and np.array_equal(np64(S), S_ref)


def _check_config(name, dev, heads=None, device_inputs=False, nthreads=16):
    cfg = workloads.CONFIGS[name]
    q, k, v = workloads.config_inputs(cfg, device=dev if device_inputs else "cpu")
    o, S = gpu_prefill(q, k, v, C=cfg.C)
    if heads is None:
        O_ref, S_ref = oracle.recurrence(q, k, v, nthreads=nthreads)
        got_o, got_s = np64(o), np64(S)
    else:
        sel = lambda x: x[:, heads].cpu()
        O_ref, S_ref = oracle.recurrence(sel(q), sel(k), sel(v), nthreads=nthreads)
        got_o, got_s = np64(o[:, heads]), np64(S[:, heads])
    e_o, e_s = rel_err(got_o, O_ref), rel_err(got_s, S_ref)
    print("%s: rel err O %.3e  S %.3e" % (name, e_o, e_s))
    assert e_o <= TOL and e_s <= TOL


def test_config_T1024_all_heads(dev):
    _check_config("prefill_B4_T1024", dev)


def test_config_T8192_all_heads(dev):
    _check_config("prefill_T8192", dev)


def test_config_T131072_sampled_heads(dev):
    _check_config("prefill_T131072", dev, heads=[0, 13, 22, 31], device_inputs=True)


def test_gaussian_with_random_incoming_state(dev):
    q, k, v = workloads.gaussian(1, 4, 3000, 128, 128, seed_base=70, scale=128 ** -0.5)
    g = torch.Generator().manual_seed(77)
    S0 = torch.randn((1, 4, 128, 128), generator=g) * 3.0
    o, S = gpu_prefill(q, k, v, C=64, S0=S0)
    O_ref, S_ref = oracle.recurrence(q, k, v, S0, nthreads=4)
    assert rel_err(np64(o), O_ref) <= TOL and rel_err(np64(S), S_ref) <= TOL


def test_fp32_gaussian_is_fp32_accurate(dev):
    q, k, v = workloads.gaussian(2, 2, 500, 64, 64, seed_base=80, scale=0.125, dtype=torch.float32)
    o, S = gpu_prefill(q, k, v, C=64)
    O_ref, S_ref = oracle.recurrence(q, k, v, nthreads=4)
    assert rel_err(np64(o), O_ref) <= 1e-5 and rel_err(np64(S), S_ref) <= 1e-5
