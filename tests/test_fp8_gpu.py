"""FP8 inputs: Q, K, V (q, k, v) in the OCP E4M3 format, decoded exactly to
bf16 on their way into LDS.  The blog "A 128 000 tokens, l'attention avale
85 % du calcul" reports its attention measurements in FP8.  Checked against
the oracle (which decodes E4M3 from the format's definition): exact on
integer inputs, within the bf16 tolerance on gaussian ones; against the same
call on bf16 copies of the same values (identical bits: only the loads
differ); and at the full benchmark sizes."""
import numpy as np
import pytest
import torch

import decode_lla_prefill_amd as lla
import oracle
import workloads
from gpu_util import TOL, need_gpu, np64, rel_err

pytestmark = pytest.mark.gpu
FP8 = torch.float8_e4m3fn


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def _prefill(q, k, v, S0, C, dev):
    S = S0.to(dev, torch.float32).contiguous().clone()
    o = lla.prefill(q.to(dev).contiguous(), k.to(dev).contiguous(), v.to(dev).contiguous(), S, chunk=C)
    torch.cuda.synchronize()
    return o, S


# B, Hq, Hkv, T, dk, dv, C: the eight-wave d=128 walk (ragged tail, several
# segments), C = 128 (two 64-token sub-chunks), d = 64 four-wave walks, a ragged head dim (element
# path), a short prompt (fused decode steps), grouped heads
FP8_INT = [
    (2, 3, 3, 300, 128, 128, 64),
    (1, 2, 2, 1000, 64, 64, 64),
    (2, 2, 2, 270, 128, 128, 128),
    (1, 3, 3, 77, 40, 72, 16),
    (2, 2, 2, 9, 128, 128, 64),
    (1, 8, 2, 333, 128, 128, 32),
]


@pytest.mark.parametrize("B,Hq,Hkv,T,dk,dv,C", FP8_INT)
def test_fp8_prefill_integers_exact(dev, B, Hq, Hkv, T, dk, dv, C):
    print("fp8 prefill int", B, Hq, Hkv, T, dk, dv, C, flush=True)
    q, k, v = workloads.integers(B, Hq, T, dk, dv, seed=T + dk, dtype=FP8, Hkv=Hkv)
    S0 = torch.randint(-300, 301, (B, Hkv, dk, dv), generator=torch.Generator().manual_seed(T)).float()
    o, S = _prefill(q, k, v, S0, C, dev)
    O_ref, S_ref = oracle.grouped_recurrence(q, k, v, S0, nthreads=8)
    assert np.array_equal(np64(o), O_ref)
    assert np.array_equal(np64(S), S_ref)


@pytest.mark.parametrize("B,Hq,Hkv,T,dk,dv,C", FP8_INT)
def test_fp8_prefill_equals_bf16_of_the_same_values(dev, B, Hq, Hkv, T, dk, dv, C):
    q, k, v = workloads.gaussian(B, Hq, T, dk, dv, seed_base=T, scale=1.0, dtype=FP8, Hkv=Hkv)
    S0 = torch.randn((B, Hkv, dk, dv), generator=torch.Generator().manual_seed(C))
    o8, S8 = _prefill(q, k, v, S0, C, dev)
    ob, Sb = _prefill(q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16), S0, C, dev)
    assert torch.equal(o8, ob)
    assert torch.equal(S8, Sb)


@pytest.mark.parametrize("T,C", [(1000, 64), (700, 128)])
def test_fp8_prefill_gaussian(dev, T, C):
    q, k, v = workloads.gaussian(1, 4, T, 128, 128, seed_base=5 * T, scale=1.0, dtype=FP8)
    S0 = torch.randn((1, 4, 128, 128), generator=torch.Generator().manual_seed(T))
    o, S = _prefill(q, k, v, S0, C, dev)
    O_ref, S_ref = oracle.recurrence(q, k, v, S0, nthreads=8)
    assert rel_err(np64(o), O_ref) <= TOL
    assert rel_err(np64(S), S_ref) <= TOL


def test_fp8_prefill_full_size(dev):
    """The T=8192 workload with FP8 inputs (B=1, H=16, C=64, d=128) in the
    launch configuration the benchmark times, every head against the oracle."""
    cfg = workloads.CONFIGS["prefill_T8192_fp8"]
    q, k, v = workloads.config_inputs(cfg, device=dev)
    S = lla.state_init(cfg.B, cfg.H, cfg.dk, cfg.dv, device=dev)
    call = lla.PreparedPrefill(q, k, v, S, cfg.C)
    call(zero_state=True)
    torch.cuda.synchronize()
    O_ref, S_ref = oracle.recurrence(q.cpu(), k.cpu(), v.cpu(), nthreads=16)
    assert rel_err(np64(call.out), O_ref) <= TOL
    assert rel_err(np64(S), S_ref) <= TOL


def test_fp8_nan_input_reaches_its_outputs(dev):
    """The E4M3 NaN code decodes to NaN: a NaN key poisons the outputs of its
    own and later tokens of that head only."""
    B, H, T, d = 1, 2, 100, 128
    q, k, v = workloads.integers(B, H, T, d, d, seed=3, dtype=FP8)
    kb = k.view(torch.uint8).clone()
    kb[0, 1, 60, 5] = 0x7F  # NaN
    k = kb.view(FP8)
    o, S = _prefill(q, k, v, torch.zeros(B, H, d, d), 64, dev)
    o = o.cpu()
    assert torch.isfinite(o[0, 0]).all() and torch.isfinite(o[0, 1, :60]).all()
    assert torch.isnan(o[0, 1, 60:]).any(dim=-1).all()


# ---- decode ---------------------------------------------------------------------

@pytest.mark.parametrize("B,Hq,Hkv,dk,dv", [(3, 4, 4, 128, 128), (2, 8, 2, 64, 64), (2, 3, 3, 40, 72)])
def test_fp8_decode_integers_exact_and_equal_to_bf16(dev, B, Hq, Hkv, dk, dv):
    gen = torch.Generator().manual_seed(Hq + dk)
    q = torch.randint(-2, 3, (B, Hq, dk), generator=gen).to(FP8)
    k = torch.randint(-2, 3, (B, Hkv, dk), generator=gen).to(FP8)
    v = torch.randint(-2, 3, (B, Hkv, dv), generator=gen).to(FP8)
    S0 = torch.randint(-300, 301, (B, Hkv, dk, dv), generator=gen).float()
    S = S0.to(dev).contiguous()
    o = lla.decode_step(q.to(dev), k.to(dev), v.to(dev), S)
    Sb = S0.to(dev).contiguous()
    ob = lla.decode_step(q.to(torch.bfloat16).to(dev), k.to(torch.bfloat16).to(dev),
                         v.to(torch.bfloat16).to(dev), Sb)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.grouped_decode_step(q, k, v, S0)
    assert np.array_equal(np64(o), o_ref) and np.array_equal(np64(S), S_ref)
    assert torch.equal(o, ob) and torch.equal(S, Sb)


def test_fp8_decode_full_size_sampled(dev):
    """One step of the FP8 decode batch (256 sequences x 32 heads, d=128) as the
    benchmark launches it; sampled sequences against the oracle."""
    cfg = workloads.CONFIGS["decode_B256_fp8"]
    S0 = workloads.random_state(cfg, device=dev)
    qd, kd, vd = workloads.decode_inputs(cfg, 1, device=dev)
    S = S0.clone()
    o = torch.empty((cfg.B, cfg.H, cfg.dv), dtype=torch.float32, device=dev)
    lla.PreparedDecode(qd[0], kd[0], vd[0], S, out=o)()
    torch.cuda.synchronize()
    for b in (0, 131, 255):
        o_ref, S_ref = oracle.decode_step(qd[0, b].cpu(), kd[0, b].cpu(), vd[0, b].cpu(), S0[b].cpu())
        assert rel_err(np64(o[b]), o_ref) <= 1e-4, b
        assert rel_err(np64(S[b]), S_ref) <= 1e-6, b


def test_fp8_short_continuation_equals_decode_steps(dev):
    B, H, T, d = 2, 3, 5, 128
    q, k, v = workloads.gaussian(B, H, T, d, d, seed_base=9, scale=1.0, dtype=FP8, device=dev)
    S0 = torch.randn((B, H, d, d), generator=torch.Generator(device=dev).manual_seed(1), device=dev)
    S_a = S0.clone()
    o_a = lla.prefill(q, k, v, S_a, chunk=64)
    S_b = S0.clone()
    o_b = torch.stack([lla.decode_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                                       v[:, :, t].contiguous(), S_b) for t in range(T)], dim=2)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(S_a, S_b)
