"""Short continuations: a prompt of a few tokens from an existing state (the
regime where prefill behaves like decode).  lla_prefill runs T <= 16 tokens
with square heads of 64 or 128 as T fused decode steps; checked against the
oracle, against T separate decode steps (same arithmetic: identical bits),
and against the chunked path of the same call at larger T."""
import numpy as np
import pytest
import torch

import decode_lla_prefill_amd as lla
import oracle
import workloads
from gpu_util import TOL, need_gpu, np64, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def _inputs(B, H, T, d, dtype, seed, integer):
    g = torch.Generator().manual_seed(seed)
    if integer:
        q, k, v = (torch.randint(-2, 3, (B, H, T, d), generator=g).to(dtype) for _ in range(3))
        S = torch.randint(-300, 301, (B, H, d, d), generator=g).float()
    else:
        q, k, v = (torch.randn((B, H, T, d), generator=g).mul(d ** -0.5).to(dtype) for _ in range(3))
        S = torch.randn((B, H, d, d), generator=g) * 3
    return q, k, v, S


@pytest.mark.parametrize("T", [1, 2, 5, 16])
@pytest.mark.parametrize("d,dtype", [(128, torch.bfloat16), (64, torch.bfloat16), (128, torch.float32)])
def test_short_prompt_equals_decode_steps(dev, T, d, dtype):
    q, k, v, S0 = _inputs(2, 3, T, d, dtype, seed=T * 7 + d, integer=False)
    S_a = S0.to(dev).contiguous().clone()
    o_a = lla.prefill(q.to(dev).contiguous(), k.to(dev).contiguous(), v.to(dev).contiguous(), S_a, chunk=64)
    S_b = S0.to(dev).contiguous().clone()
    o_b = torch.empty_like(o_a)
    for t in range(T):
        o_b[:, :, t] = lla.decode_step(q[:, :, t].to(dev).contiguous(), k[:, :, t].to(dev).contiguous(),
                                       v[:, :, t].to(dev).contiguous(), S_b)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b)
    assert torch.equal(S_a, S_b)


@pytest.mark.parametrize("T", [1, 3, 16])
@pytest.mark.parametrize("d,dtype", [(128, torch.bfloat16), (64, torch.float32)])
def test_short_prompt_integers_exact(dev, T, d, dtype):
    q, k, v, S0 = _inputs(3, 2, T, d, dtype, seed=100 + T + d, integer=True)
    S = S0.to(dev).contiguous().clone()
    o = lla.prefill(q.to(dev).contiguous(), k.to(dev).contiguous(), v.to(dev).contiguous(), S, chunk=4)
    torch.cuda.synchronize()
    O_ref, S_ref = oracle.recurrence(q, k, v, S0, nthreads=8)
    assert np.array_equal(np64(o), O_ref)
    assert np.array_equal(np64(S), S_ref)


@pytest.mark.parametrize("T", [4, 16, 17])
def test_short_prompt_gaussian_and_chunked_boundary(dev, T):
    """T = 16 takes the fused path, T = 17 the chunked one; both match the oracle."""
    q, k, v, S0 = _inputs(2, 4, T, 128, torch.bfloat16, seed=T, integer=False)
    S = S0.to(dev).contiguous().clone()
    o = lla.prefill(q.to(dev).contiguous(), k.to(dev).contiguous(), v.to(dev).contiguous(), S, chunk=64)
    torch.cuda.synchronize()
    O_ref, S_ref = oracle.recurrence(q, k, v, S0, nthreads=8)
    assert rel_err(np64(o), O_ref) <= TOL
    assert rel_err(np64(S), S_ref) <= TOL


def test_continuation_of_the_decode_workload(dev):
    """4-token continuations of the decode workload's states (256 sequences x 32
    heads, d = 128, after the T = 4096 prefill): sampled heads vs the oracle."""
    cfg = workloads.CONFIGS["decode_B256"]
    B, H, T, C, d = cfg.B, cfg.H, cfg.T, cfg.C, cfg.dk
    S = lla.state_init(B, H, d, d, device=dev)
    slice_b = 32
    qa, ka, va = workloads.config_inputs(cfg, device=dev)
    o_tmp = torch.empty((slice_b, H, T, d), dtype=torch.float32, device=dev)
    for b0 in range(0, B, slice_b):
        lla.prefill(qa[b0:b0 + slice_b], ka[b0:b0 + slice_b], va[b0:b0 + slice_b],
                    S[b0:b0 + slice_b], chunk=C, out=o_tmp)
    del o_tmp
    torch.cuda.synchronize()
    picks = [(0, 0), (255, 31), (17, 5), (128, 16), (201, 30)]
    S_pick = torch.stack([S[b, h] for b, h in picks]).cpu()
    qn, kn, vn = (x.permute(1, 2, 0, 3).contiguous()  # [steps,B,H,d] -> [B,H,steps,d]
                  for x in workloads.decode_inputs(cfg, 4, device=dev))
    o = lla.prefill(qn, kn, vn, S, chunk=C)
    torch.cuda.synchronize()
    # oracle: the picked heads' prefill states continued by the same 4 tokens
    qs, ks, vs = (torch.stack([x[b, h] for b, h in picks]).unsqueeze(0).cpu() for x in (qn, kn, vn))
    O_ref, S_ref = oracle.recurrence(qs, ks, vs, S_pick.unsqueeze(0), nthreads=8)
    got_o = torch.stack([o[b, h] for b, h in picks]).unsqueeze(0)
    got_s = torch.stack([S[b, h] for b, h in picks]).unsqueeze(0)
    assert rel_err(np64(got_o), O_ref) <= TOL
    assert rel_err(np64(got_s), S_ref) <= TOL
