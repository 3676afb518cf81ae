"""GPU parity of the decode step (through the C ABI) against the oracle."""
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


def _decode(q, k, v, S, dev):
    S_gpu = S.to(dev).contiguous().clone()
    o = lla.decode_step(q.to(dev).contiguous(), k.to(dev).contiguous(), v.to(dev).contiguous(), S_gpu)
    torch.cuda.synchronize()
    return o, S_gpu


@pytest.mark.parametrize("B,H,dk,dv,dtype", [
    (4, 8, 128, 128, torch.bfloat16), (2, 3, 64, 64, torch.bfloat16), (3, 2, 5, 7, torch.bfloat16),
    (1, 4, 128, 12, torch.bfloat16), (2, 2, 128, 128, torch.float32), (1, 1, 1, 1, torch.float32),
    (3, 1, 64, 64, torch.float32), (2, 2, 64, 128, torch.bfloat16), (2, 2, 128, 64, torch.bfloat16),
    (1, 2, 32, 32, torch.bfloat16),
])
def test_decode_integers_exact(dev, B, H, dk, dv, dtype):
    g = torch.Generator().manual_seed(B * 100 + dk + dv)
    q = torch.randint(-2, 3, (B, H, dk), generator=g).to(dtype)
    k = torch.randint(-2, 3, (B, H, dk), generator=g).to(dtype)
    v = torch.randint(-2, 3, (B, H, dv), generator=g).to(dtype)
    S = torch.randint(-100, 101, (B, H, dk, dv), generator=g).float()
    o, S_new = _decode(q, k, v, S, dev)
    o_ref, S_ref = oracle.decode_step(q, k, v, S)
    assert np.array_equal(np64(S_new), S_ref)
    assert np.array_equal(np64(o), o_ref)


def test_decode_gaussian(dev):
    g = torch.Generator().manual_seed(3)
    q, k, v = (torch.randn((8, 16, 128), generator=g).mul(128 ** -0.5).bfloat16() for _ in range(3))
    S = torch.randn((8, 16, 128, 128), generator=g) * 4
    o, S_new = _decode(q, k, v, S, dev)
    o_ref, S_ref = oracle.decode_step(q, k, v, S)
    assert rel_err(np64(o), o_ref) <= 1e-5
    assert rel_err(np64(S_new), S_ref) <= 1e-6


def test_decode_after_prefill_config(dev):
    """The decode workload: a T=4096 prefill of 256 x 32 heads (d=128, C=64),
    then 512 decode steps; sampled heads against the oracle over every step
    and the final state."""
    cfg = workloads.CONFIGS["decode_B256"]
    B, H, d = cfg.B, cfg.H, cfg.dk
    steps = cfg.decode_steps
    q, k, v = workloads.config_inputs(cfg, device=dev)
    S = lla.state_init(B, H, d, d, device=dev)
    o_pre = lla.prefill(q, k, v, S, chunk=cfg.C)
    del o_pre
    qd, kd, vd = workloads.decode_inputs(cfg, steps, device=dev)
    rng = np.random.default_rng(50)
    pairs = [(0, 0), (B - 1, H - 1)] + [(int(b), int(h)) for b, h in
                                        zip(rng.integers(0, B, 32), rng.integers(0, H, 32))]
    bi = torch.tensor([p[0] for p in pairs], device=dev)
    hi = torch.tensor([p[1] for p in pairs], device=dev)
    outs = torch.empty((steps, len(pairs), d), dtype=torch.float32, device=dev)
    o = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    for t in range(steps):
        lla.decode_step(qd[t], kd[t], vd[t], S, out=o)
        outs[t] = o[bi, hi]
    torch.cuda.synchronize()
    # oracle: the sampled heads' prefill, then their decode steps
    sel = lambda x: x[bi, hi].cpu()
    _, S_ref = oracle.recurrence(sel(q), sel(k), sel(v), nthreads=16)
    o_ref = np.zeros((steps, len(pairs), d))
    for t in range(steps):
        o_ref[t], S_ref = oracle.decode_step(qd[t][bi, hi].cpu(), kd[t][bi, hi].cpu(),
                                             vd[t][bi, hi].cpu(), S_ref)
    e_o = rel_err(np64(outs), o_ref)
    e_s = rel_err(np64(S[bi, hi]), S_ref)
    print("decode after prefill: rel err o %.3e  S %.3e" % (e_o, e_s))
    assert e_o <= TOL and e_s <= TOL


def test_decode_continues_prefill_on_a_batch_slice_all_heads(dev):
    """Eight sequences drawn like the decode workload (32 heads, d=128): the
    T=4096 prefill followed by the 512 decode steps equals one prefill of all
    4,608 tokens on every head, outputs and final state (GPU against GPU; the
    two sum in different orders, so within the bar)."""
    cfg = workloads.CONFIGS["decode_B256"]
    nb, steps = 8, cfg.decode_steps
    q, k, v = workloads.config_inputs(cfg, device=dev, B=nb)
    qd, kd, vd = workloads.decode_inputs(cfg, steps, device=dev, B=nb)
    S = torch.empty((nb, cfg.H, cfg.dk, cfg.dv), device=dev)
    lla.prefill(q, k, v, S, chunk=cfg.C, zero_state=True)
    o_dec = torch.empty((steps, nb, cfg.H, cfg.dv), device=dev)
    for t in range(steps):
        lla.decode_step(qd[t], kd[t], vd[t], S, out=o_dec[t])
    cat = lambda a, b: torch.cat([a, b.permute(1, 2, 0, 3)], dim=2).contiguous()
    S_all = torch.empty_like(S)
    o_all = lla.prefill(cat(q, qd), cat(k, kd), cat(v, vd), S_all, chunk=cfg.C, zero_state=True)
    torch.cuda.synchronize()
    e_o = rel_err(np64(o_dec.permute(1, 2, 0, 3)), np64(o_all[:, :, cfg.T:]))
    e_s = rel_err(np64(S), np64(S_all))
    print("prefill + 512 decode steps vs one prefill: rel err o %.3e  S %.3e" % (e_o, e_s))
    assert e_o <= TOL and e_s <= TOL
