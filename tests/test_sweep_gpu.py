"""A seeded sweep over the dispatch space: random shapes (batch, query and
key/value heads, sequence length, head dims, chunk size, input type, fresh
prompt or not) drawn once from a fixed seed, each run through the C ABI on
integer inputs and compared with the oracle bit for bit.  Every kernel
variant the plan can pick is reached: the eight-wave double-buffered walk
(d = 128), the four-wave walks (vector and element paths), chunks of more
than 64 tokens (run as two sub-chunks), one or several segments,
grouped heads, the fused short-prompt route, bf16, fp32 and FP8 inputs.
A second draw runs gaussian inputs from a gaussian state and holds every
path to the floating-point bar on these shapes."""
import numpy as np
import pytest
import torch

import decode_lla_prefill_amd as lla
import oracle
import workloads
from gpu_util import need_gpu, np64, rel_err

pytestmark = pytest.mark.gpu

DTYPES = [torch.bfloat16, torch.float32, torch.float8_e4m3fn]


def _draw_prefill_cases(n, seed):
    rng = np.random.RandomState(seed)
    cases = []
    while len(cases) < n:
        dtype = DTYPES[rng.randint(3)]
        dk = int(rng.choice([128, 128, 64, 32, 16, 40, 72, 96, 120, 8, 1, 3]))
        dv = dk if rng.rand() < 0.7 else int(rng.choice([128, 64, 48, 8, 5]))
        C = int(rng.choice([64, 64, 128, 32, 16, 1, 7, 48, 100]))
        Hkv = int(rng.choice([1, 2, 3, 4]))
        G = int(rng.choice([1, 1, 2, 4]))
        B = int(rng.choice([1, 2, 3]))
        T = int(rng.choice([1, 5, 16, 17, 64, 65, 200, 333, 700, 1500]))
        if B * Hkv * G * T * max(dk, dv) > 1_500_000:  # keep the oracle fast
            continue
        cases.append((B, Hkv * G, Hkv, T, dk, dv, C, dtype, bool(rng.rand() < 0.3)))
    return cases


PREFILL_CASES = _draw_prefill_cases(48, 20240611)


@pytest.mark.parametrize("B,Hq,Hkv,T,dk,dv,C,dtype,fresh", PREFILL_CASES)
def test_sweep_prefill_integers_exact(B, Hq, Hkv, T, dk, dv, C, dtype, fresh):
    dev = need_gpu()
    print("sweep prefill", B, Hq, Hkv, T, dk, dv, C, dtype, fresh, flush=True)
    q, k, v = workloads.integers(B, Hq, T, dk, dv, seed=T * 7 + dk + C, dtype=dtype, Hkv=Hkv)
    gen = torch.Generator().manual_seed(T + C)
    S0 = torch.zeros(B, Hkv, dk, dv) if fresh else torch.randint(-50, 51, (B, Hkv, dk, dv), generator=gen).float()
    S = torch.full((B, Hkv, dk, dv), float("nan")) if fresh else S0.clone()
    S = S.to(dev).contiguous()
    o = lla.prefill(q.to(dev).contiguous(), k.to(dev).contiguous(), v.to(dev).contiguous(), S, chunk=C,
                    zero_state=fresh)
    torch.cuda.synchronize()
    O_ref, S_ref = oracle.grouped_recurrence(q, k, v, S0, nthreads=8)
    assert np.array_equal(np64(o), O_ref)
    assert np.array_equal(np64(S), S_ref)


def _draw_decode_cases(n, seed):
    rng = np.random.RandomState(seed)
    cases = []
    for _ in range(n):
        dtype = DTYPES[rng.randint(3)]
        G = int(rng.choice([1, 1, 2, 4, 8, 16]))
        d = int(rng.choice([128, 64]))
        if G == 1:
            dk = int(rng.choice([128, 64, 32, 40, 96, 7]))
            dv = dk if rng.rand() < 0.6 else int(rng.choice([128, 12, 64, 3]))
        else:
            dk = dv = d
        cases.append((int(rng.choice([1, 3, 17])), G * int(rng.choice([1, 2, 3])), dk, dv, G, dtype))
    return cases


DECODE_CASES = _draw_decode_cases(24, 424242)


def _draw_grouped_any_cases(n, seed):
    """Shared-state heads at any group size and head dims: the square
    kernels past one LDS batch of 16 query rows, and the general grouped
    kernel (4 or 1 value columns per thread)."""
    rng = np.random.RandomState(seed)
    cases = []
    for _ in range(n):
        dtype = DTYPES[rng.randint(3)]
        G = int(rng.choice([2, 3, 5, 8, 17, 24, 40]))
        dk = int(rng.choice([128, 64, 1, 7, 40, 96, 128]))
        dv = dk if rng.rand() < 0.4 else int(rng.choice([128, 100, 64, 12, 3, 1]))
        cases.append((int(rng.choice([1, 2, 5])), G * int(rng.choice([1, 2])), dk, dv, G, dtype))
    return cases


DECODE_CASES_ANY = _draw_grouped_any_cases(16, 77077)


@pytest.mark.parametrize("B,Hq,dk,dv,G,dtype", DECODE_CASES + DECODE_CASES_ANY)
def test_sweep_decode_steps_integers_exact(B, Hq, dk, dv, G, dtype):
    """Four decode steps in a row from an integer state, exact against the oracle."""
    dev = need_gpu()
    print("sweep decode", B, Hq, dk, dv, G, dtype, flush=True)
    Hkv = Hq // G
    gen = torch.Generator().manual_seed(Hq * 31 + dk + dv)
    S0 = torch.randint(-100, 101, (B, Hkv, dk, dv), generator=gen).float()
    S = S0.to(dev).contiguous()
    S_ref = S0.double().numpy()
    for step in range(4):
        q = torch.randint(-2, 3, (B, Hq, dk), generator=gen).to(dtype)
        k = torch.randint(-2, 3, (B, Hkv, dk), generator=gen).to(dtype)
        v = torch.randint(-2, 3, (B, Hkv, dv), generator=gen).to(dtype)
        o = lla.decode_step(q.to(dev), k.to(dev), v.to(dev), S)
        torch.cuda.synchronize()
        o_ref, S_ref = oracle.grouped_decode_step(q, k, v, S_ref)
        assert np.array_equal(np64(o), o_ref), step
    assert np.array_equal(np64(S), S_ref)


def _draw_float_cases(n, seed):
    rng = np.random.RandomState(seed)
    cases = []
    while len(cases) < n:
        dtype = DTYPES[rng.randint(3)]
        dk = int(rng.choice([128, 128, 64, 32, 40, 96, 8]))
        dv = dk if rng.rand() < 0.7 else int(rng.choice([128, 64, 24]))
        C = int(rng.choice([64, 64, 128, 32, 16, 48]))
        Hkv = int(rng.choice([1, 2, 3]))
        G = int(rng.choice([1, 1, 2, 4]))
        B = int(rng.choice([1, 2]))
        T = int(rng.choice([3, 16, 17, 100, 333, 1000, 2500]))
        if B * Hkv * G * T * max(dk, dv) > 1_500_000:
            continue
        cases.append((B, Hkv * G, Hkv, T, dk, dv, C, dtype))
    return cases


FLOAT_CASES = _draw_float_cases(24, 777)


@pytest.mark.parametrize("B,Hq,Hkv,T,dk,dv,C,dtype", FLOAT_CASES)
def test_sweep_prefill_gaussian_within_the_bar(B, Hq, Hkv, T, dk, dv, C, dtype):
    """Gaussian inputs (scaled 1/sqrt(dk); unit scale for FP8, whose range
    allows it) and a gaussian S_0, against the oracle: max|err|/max|ref| within
    2e-3 for bf16 and FP8 inputs, 1e-5 for fp32."""
    dev = need_gpu()
    print("float sweep prefill", B, Hq, Hkv, T, dk, dv, C, dtype, flush=True)
    scale = 1.0 if dtype == torch.float8_e4m3fn else dk ** -0.5
    q, k, v = workloads.gaussian(B, Hq, T, dk, dv, seed_base=T * 11 + dk + C, scale=scale, dtype=dtype, Hkv=Hkv)
    S0 = torch.randn((B, Hkv, dk, dv), generator=torch.Generator().manual_seed(T + dv))
    S = S0.to(dev).contiguous()
    o = lla.prefill(q.to(dev).contiguous(), k.to(dev).contiguous(), v.to(dev).contiguous(), S, chunk=C)
    torch.cuda.synchronize()
    O_ref, S_ref = oracle.grouped_recurrence(q, k, v, S0, nthreads=8)
    bar = 1e-5 if dtype == torch.float32 else 2e-3
    e_o, e_s = rel_err(np64(o), O_ref), rel_err(np64(S), S_ref)
    assert e_o <= bar and e_s <= bar, (e_o, e_s)
