"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Bar: bit-exact on small-integer inputs (the deck's trace, its {0,1} toy
variants, {-1,0,1} inputs across tile counts, ragged tails and segment
counts, and {-8..8} queries and keys whose scores reach 8192);
max|err|/max|ref| <= 2e-3 for bf16 inputs (all heads of the T=1024
and T=8192 shapes, four sampled heads of the T=131072 shape).
"""
import numpy as np
import pytest
import torch

import decode_lla_prefill_amd as lla
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
    (1, 2, 2000, 64, 64, 128, torch.float32),   # fp32 with C > 64: sub-chunks of 64
    (2, 1, 333, 128, 128, 100, torch.float32),  # sub-chunks of 50
    (1, 3, 70, 40, 24, 65, torch.float32),      # sub-chunks of 33, one segment
    (1, 2, 37, 16, 16, 1, torch.bfloat16),      # C = 1: the recurrence itself
    (2, 1, 300, 24, 40, 128, torch.bfloat16),   # C = 128 with odd head dims
    (1, 2, 1000, 64, 64, 101, torch.bfloat16),  # odd C > 64: two sub-chunks of 51
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


# Scores beyond what one bf16 value holds exactly: q, k in {-8..8} at d_k up
# to 128 give |q . k| up to 8192 (one bf16 value is exact only up to 256;
# the high + low pair to 2^16), with v in {-1, 0, 1} so that every partial sum
# stays below 2^24 for T < 2048 (|P V| <= 8192 C, |S| <= 8 T, |Q S| <= 8192 T):
# the results are exact integers, the same at every chunk size.
LARGE_SCORE_CASES = [
    # B, Hq, Hkv, T, dk, dv, C, dtype
    (1, 2, 2, 1000, 128, 128, 128, torch.bfloat16),      # chunks of 128 (run as two of 64)
    (1, 2, 2, 1000, 128, 128, 64, torch.bfloat16),       # double-buffered eight-wave walk
    (1, 2, 2, 500, 128, 128, 32, torch.bfloat16),
    (2, 2, 2, 700, 128, 128, 128, torch.float8_e4m3fn),  # E4M3 holds {-8..8} exactly
    (1, 3, 3, 900, 64, 64, 128, torch.bfloat16),         # four-wave walk
    (2, 1, 1, 300, 40, 72, 100, torch.bfloat16),         # element path
    (1, 4, 2, 600, 128, 128, 64, torch.bfloat16),        # shared-state heads
    (1, 4, 2, 600, 128, 128, 128, torch.bfloat16),
]


@pytest.mark.parametrize("B,Hq,Hkv,T,dk,dv,C,dtype", LARGE_SCORE_CASES)
def test_integer_inputs_with_large_scores_exact(dev, B, Hq, Hkv, T, dk, dv, C, dtype):
    q, k, v = workloads.integers(B, Hq, T, dk, dv, seed=3 * T + C, lo=-8, hi=8, dtype=dtype, Hkv=Hkv,
                                 v_range=(-1, 1))
    # the case does reach scores that one bf16 value cannot hold
    G = Hq // Hkv
    P = torch.tril(q.float() @ k.float().repeat_interleave(G, dim=1).transpose(-1, -2))
    assert P.abs().max() <= 2 ** 16 and (P != P.bfloat16().float()).any()
    S = torch.zeros((B, Hkv, dk, dv), device=dev)
    o = lla.prefill(q.to(dev), k.to(dev), v.to(dev), S, chunk=C)
    torch.cuda.synchronize()
    O_ref, S_ref = oracle.grouped_recurrence(q, k, v, np.zeros((B, Hkv, dk, dv)), nthreads=8)
    assert np.array_equal(np64(S), S_ref)
    assert np.array_equal(np64(o), O_ref)


@pytest.mark.parametrize("B,Hq,Hkv,T,dk,dv,C,dtype", [
    (1, 3, 3, 900, 64, 64, 128, torch.bfloat16),     # 14 chunks of 64 before the last segment
    (2, 4, 2, 700, 64, 64, 64, torch.float8_e4m3fn),  # shared-state heads, FP8
])
def test_integer_fresh_prompt_with_large_scores_one_launch_exact(dev, B, Hq, Hkv, T, dk, dv, C, dtype):
    """A fresh prompt on the one-launch walk (the walks sum the earlier
    segments themselves) with scores past one bf16 value: exact."""
    q, k, v = workloads.integers(B, Hq, T, dk, dv, seed=5 * T + C, lo=-8, hi=8, dtype=dtype, Hkv=Hkv,
                                 v_range=(-1, 1))
    S = torch.full((B, Hkv, dk, dv), float("nan"), device=dev)
    o = lla.prefill(q.to(dev), k.to(dev), v.to(dev), S, chunk=C, zero_state=True)
    torch.cuda.synchronize()
    O_ref, S_ref = oracle.grouped_recurrence(q, k, v, np.zeros((B, Hkv, dk, dv)), nthreads=8)
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


@pytest.mark.parametrize("C", [64, 100, 128])
def test_fp32_gaussian_is_fp32_accurate(dev, C):
    q, k, v = workloads.gaussian(2, 2, 500, 64, 64, seed_base=80, scale=0.125, dtype=torch.float32)
    o, S = gpu_prefill(q, k, v, C=C)
    O_ref, S_ref = oracle.recurrence(q, k, v, nthreads=4)
    assert rel_err(np64(o), O_ref) <= 1e-5 and rel_err(np64(S), S_ref) <= 1e-5


def test_fp32_chunks_over_64_with_state_and_workspace(dev):
    # several segments at d = 128: the sub-chunk plan runs in the workspace
    # the dtype-less size function gives
    q, k, v = workloads.gaussian(1, 4, 3000, 128, 128, seed_base=90, scale=128 ** -0.5, dtype=torch.float32)
    S0 = torch.randn((1, 4, 128, 128), generator=torch.Generator().manual_seed(91))
    assert lla.prefill_workspace_size(1, 4, 3000, 128, 128, 128) > 0
    o, S = gpu_prefill(q, k, v, C=128, S0=S0)
    O_ref, S_ref = oracle.recurrence(q, k, v, S0, nthreads=4)
    assert rel_err(np64(o), O_ref) <= 1e-5 and rel_err(np64(S), S_ref) <= 1e-5


@pytest.mark.parametrize("C,dtype", [(128, torch.float32), (101, torch.float32), (101, torch.bfloat16)])
def test_phases_at_chunks_over_64_equal_the_one_call(dev, C, dtype):
    # chunks over 64 tokens run as two sub-chunks of c = ceil(C/2) in every
    # call; segment s starts after s G c tokens (G = prefill_segment_chunks)
    B, H, T, d = 1, 3, 6000, 64
    q, k, v = (x.to(dev) for x in workloads.integers(B, H, T, d, d, seed=C, dtype=dtype))
    G = lla.prefill_segment_chunks(B, H, T, d, d, C)
    c = (C + 1) // 2
    n_seg = -(-(-(-T // c)) // G)
    assert n_seg > 1
    S_a = lla.state_init(B, H, d, d, device=dev)
    o_a = lla.prefill(q, k, v, S_a, chunk=C)
    S_b = lla.state_init(B, H, d, d, device=dev)
    ws = lla.prefill_segment_states(k, v, C, None)
    lla.prefill_state_scan(S_b, T, C, ws)
    o_b = lla.prefill_chunks(q, k, v, S_b, C, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(S_a, S_b)
    O_ref, S_ref, ck = oracle.recurrence(q.cpu(), k.cpu(), v.cpu(), ckpt_every=G * c, nthreads=3)
    assert np.array_equal(np64(o_a), O_ref) and np.array_equal(np64(S_a), S_ref)
    slots = np64(ws.view(B, H, n_seg, d, d))
    assert np.array_equal(slots[:, :, 1:], ck[:, :, :n_seg - 1])
