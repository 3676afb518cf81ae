"""Speculative decoding's verify and commit, through the C ABI: a prefill of
k draft tokens with LLA_PREFILL_KEEP_STATE gives every draft token's output
and leaves the state as it was; lla_state_commit then advances each
sequence's state by its accepted prefix m (0..k, read on the device).
On the fused short-prompt route they equal m decode steps bit for bit --
outputs of all k tokens, state after the commit -- and, on integer inputs,
the oracle's recurrence exactly.  Longer drafts and other shapes run the
chunked prefill without its state write: the prefill's outputs, the same
commit."""
import numpy as np
import pytest
import torch

import decode_lla_prefill_amd as lla
import oracle
import workloads
from gpu_util import need_gpu, np64

pytestmark = pytest.mark.gpu
FP8 = torch.float8_e4m3fn

CASES = [
    # B, Hq, Hkv, k (draft tokens), d, dtype
    (8, 4, 4, 4, 128, torch.bfloat16),
    (17, 2, 2, 16, 64, torch.bfloat16),
    (5, 8, 2, 4, 128, FP8),
    (6, 3, 3, 5, 64, torch.float32),
    (9, 8, 2, 8, 128, torch.bfloat16),   # shared-state heads: T * G = 32
    (2, 2, 2, 1, 128, torch.bfloat16),
]


def _inputs(B, Hq, Hkv, k, d, dtype, integer, seed):
    if integer:
        q, kk, v = workloads.integers(B, Hq, k, d, d, seed=seed, lo=-2, hi=2, dtype=dtype, Hkv=Hkv)
        S0 = torch.randint(-20, 21, (B, Hkv, d, d), generator=torch.Generator().manual_seed(seed)).float()
    else:
        scale = 1.0 if dtype == FP8 else d ** -0.5
        q, kk, v = workloads.gaussian(B, Hq, k, d, d, seed_base=seed, scale=scale, dtype=dtype, Hkv=Hkv)
        S0 = torch.randn((B, Hkv, d, d), generator=torch.Generator().manual_seed(seed))
    return q, kk, v, S0


def _verify_commit(q, kk, v, S0, accepted, dev):
    S = S0.to(dev).clone()
    o = lla.prefill(q.to(dev), kk.to(dev), v.to(dev), S, chunk=64, keep_state=True)
    torch.cuda.synchronize()
    kept = np64(S)
    acc = None if accepted is None else torch.tensor(accepted, dtype=torch.int32, device=dev)
    lla.state_commit(kk.to(dev), v.to(dev), S, acc)
    torch.cuda.synchronize()
    return np64(o), kept, np64(S)


@pytest.mark.parametrize("B,Hq,Hkv,k,d,dtype", CASES)
def test_verify_and_commit_equal_decode_steps_bit_for_bit(B, Hq, Hkv, k, d, dtype):
    dev = need_gpu()
    print("speculative decode-step equality", B, Hq, Hkv, k, d, dtype, flush=True)
    q, kk, v, S0 = _inputs(B, Hq, Hkv, k, d, dtype, False, 600 + k + d)
    accepted = [b % (k + 1) for b in range(B)]  # every m in 0..k appears
    o, kept, S = _verify_commit(q, kk, v, S0, accepted, dev)
    assert np.array_equal(kept, S0.double().numpy())  # the verify pass wrote nothing
    # the same tokens as k decode steps, keeping each sequence's state after its m steps
    Sd = S0.to(dev).clone()
    want = np.empty_like(S)
    for b in range(B):
        if accepted[b] == 0:
            want[b] = S0[b].double().numpy()
    for t in range(k):
        ot = lla.decode_step(q[:, :, t].contiguous().to(dev), kk[:, :, t].contiguous().to(dev),
                             v[:, :, t].contiguous().to(dev), Sd)
        torch.cuda.synchronize()
        assert np.array_equal(o[:, :, t], np64(ot)), t
        for b in range(B):
            if accepted[b] == t + 1:
                want[b] = np64(Sd[b])
    assert np.array_equal(S, want)


@pytest.mark.parametrize("B,Hq,Hkv,k,d,dtype", CASES)
def test_verify_and_commit_exact_against_the_oracle(B, Hq, Hkv, k, d, dtype):
    dev = need_gpu()
    print("speculative oracle", B, Hq, Hkv, k, d, dtype, flush=True)
    q, kk, v, S0 = _inputs(B, Hq, Hkv, k, d, dtype, True, 700 + k + d)
    accepted = [(3 * b + 1) % (k + 1) for b in range(B)]
    o, kept, S = _verify_commit(q, kk, v, S0, accepted, dev)
    O_ref, _ = oracle.grouped_recurrence(q, kk, v, S0, nthreads=8)
    assert np.array_equal(o, O_ref)
    for b in range(B):
        m = accepted[b]
        _, S_ref = oracle.grouped_recurrence(q[b:b + 1, :, :m], kk[b:b + 1, :, :m], v[b:b + 1, :, :m],
                                             S0[b:b + 1], nthreads=4)
        assert np.array_equal(S[b:b + 1], S_ref), b


def test_all_accepted_and_clamped_counts():
    dev = need_gpu()
    B, H, k, d = 4, 4, 6, 128
    q, kk, v, S0 = _inputs(B, H, H, k, d, torch.bfloat16, False, 800)
    # accepted = None: all k tokens, the state of the plain (fused) prefill
    _, _, S_all = _verify_commit(q, kk, v, S0, None, dev)
    S_plain = S0.to(dev).clone()
    lla.prefill(q.to(dev), kk.to(dev), v.to(dev), S_plain, chunk=64)
    torch.cuda.synchronize()
    assert np.array_equal(S_all, np64(S_plain))
    # counts outside [0, k] clamp: -3 -> 0 (state untouched), k + 5 -> k
    _, _, S_cl = _verify_commit(q, kk, v, S0, [-3, k + 5, 0, k], dev)
    assert np.array_equal(S_cl[0], S0[0].double().numpy()) and np.array_equal(S_cl[2], S0[2].double().numpy())
    assert np.array_equal(S_cl[1], S_all[1]) and np.array_equal(S_cl[3], S_all[3])


def test_commit_of_longer_drafts_and_odd_head_dims():
    """lla_state_commit takes any T and head dims: 40 draft tokens at dk = 24,
    dv = 7 (no vector path) against the oracle."""
    dev = need_gpu()
    B, H, T, dk, dv = 3, 2, 40, 24, 7
    q, kk, v = workloads.integers(B, H, T, dk, dv, seed=900, lo=-2, hi=2)
    S0 = torch.randint(-9, 10, (B, H, dk, dv), generator=torch.Generator().manual_seed(901)).float()
    S = S0.to(dev).clone()
    acc = torch.tensor([40, 17, 0], dtype=torch.int32, device=dev)
    lla.state_commit(kk.to(dev), v.to(dev), S, acc)
    torch.cuda.synchronize()
    for b, m in enumerate([40, 17, 0]):
        _, S_ref = oracle.recurrence(q[b:b + 1, :, :m], kk[b:b + 1, :, :m], v[b:b + 1, :, :m], S0[b:b + 1])
        assert np.array_equal(np64(S[b:b + 1]), S_ref), b


# Verify passes off the fused short-prompt route run the chunked prefill
# without its final state write: longer drafts, other head dims, T * G > 64.
CHUNKED_CASES = [
    # B, Hq, Hkv, k (draft tokens), dk, dv, C, dtype
    (3, 2, 2, 40, 64, 64, 64, torch.bfloat16),      # one segment: the walk reads S itself
    (2, 4, 2, 24, 128, 128, 64, torch.bfloat16),    # shared-state heads, T * G = 48 > 16 tokens
    (1, 32, 4, 16, 128, 128, 64, torch.bfloat16),   # T * G = 128 > 64
    (2, 3, 3, 30, 40, 24, 16, torch.float32),       # other head dims, several chunks
    (1, 2, 2, 3000, 128, 128, 128, FP8),            # several segments (workspace), C = 128
]


@pytest.mark.parametrize("B,Hq,Hkv,k,dk,dv,C,dtype", CHUNKED_CASES)
def test_chunked_verify_pass_leaves_the_state_and_commits_exactly(B, Hq, Hkv, k, dk, dv, C, dtype):
    """The outputs equal those of the same prefill without the option (bit
    for bit) and the oracle's (integers, exact); S is not written; the commit
    of each sequence's accepted prefix is exact against the oracle."""
    dev = need_gpu()
    print("speculative chunked verify", B, Hq, Hkv, k, dk, dv, C, dtype, flush=True)
    q, kk, v = workloads.integers(B, Hq, k, dk, dv, seed=1000 + k, lo=-1, hi=1, dtype=dtype, Hkv=Hkv)
    S0 = torch.randint(-20, 21, (B, Hkv, dk, dv), generator=torch.Generator().manual_seed(k)).float()
    qd, kd, vd = (x.to(dev) for x in (q, kk, v))
    S = S0.to(dev).clone()
    o = lla.prefill(qd, kd, vd, S, chunk=C, keep_state=True)
    S_plain = S0.to(dev).clone()
    o_plain = lla.prefill(qd, kd, vd, S_plain, chunk=C)
    torch.cuda.synchronize()
    assert torch.equal(o, o_plain)
    assert np.array_equal(np64(S), S0.double().numpy())  # the verify pass wrote nothing
    O_ref, _ = oracle.grouped_recurrence(q, kk, v, S0, nthreads=8)
    assert np.array_equal(np64(o), O_ref)
    accepted = [(5 * b + 3) % (k + 1) for b in range(B)]
    lla.state_commit(kd, vd, S, torch.tensor(accepted, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    for b, m in enumerate(accepted):
        _, S_ref = oracle.grouped_recurrence(q[b:b + 1, :, :m], kk[b:b + 1, :, :m], v[b:b + 1, :, :m],
                                             S0[b:b + 1], nthreads=4)
        assert np.array_equal(np64(S[b:b + 1]), S_ref), b


def test_chunked_verify_pass_of_a_fresh_prompt_reads_and_writes_nothing():
    """KEEP_STATE with ZERO_STATE off the fused route: outputs of the fresh
    prompt, S (NaN here) neither read nor written."""
    dev = need_gpu()
    B, H, k, d = 1, 4, 700, 64
    q, kk, v = (x.to(dev) for x in workloads.integers(B, H, k, d, d, seed=77))
    S = torch.full((B, H, d, d), float("nan"), device=dev)
    o = lla.prefill(q, kk, v, S, chunk=64, zero_state=True, keep_state=True)
    torch.cuda.synchronize()
    O_ref, _ = oracle.recurrence(q.cpu(), kk.cpu(), v.cpu(), nthreads=4)
    assert np.array_equal(np64(o), O_ref)
    assert torch.isnan(S).all()
