"""The gated (decayed) state on the GPU, through the C ABI, against the oracle.

Reading (the slide deck "Chunking, causality, and parallel prefill" cites the
chunkwise form of gated linear attention, section "Boundary, evidence, and
sources", without a gate): S_t = g_t S_{t-1} + k_t v_t^T, o_t = S_t^T q_t,
one gate per (b,h) and token.  The oracle (oracle.gated_recurrence) is pinned
in tests/test_oracle_gated.py.  Checked here: the chunked prefill within the
floating-point bar on every kernel shape (one and several segments, chunk
tiles of 32, 64 and 128, ragged T and head dims, bf16, fp32 and FP8 inputs);
gates of one on integer inputs exact; the zero-state option; continuation
(prefill, prefill) and (prefill, decode steps); the decode step exact on
integer inputs with dyadic gates and bit-equal to lla_decode_step at g = 1;
gates at the ends of their range; the full T=8192 and decode workloads on
sampled heads."""
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


def _bar(dtype):
    return 1e-5 if dtype == torch.float32 else TOL


CASES = [
    # B, H, T, dk, dv, C, dtype, gate range
    (2, 3, 1000, 64, 64, 64, torch.bfloat16, (0.5, 1.0)),      # several segments
    (1, 2, 2000, 128, 128, 64, torch.bfloat16, (0.9, 1.0)),    # d = 128, two value blocks
    (1, 2, 900, 128, 128, 128, torch.bfloat16, (0.8, 1.0)),    # chunks of 128 (two of 64)
    (2, 2, 333, 32, 32, 32, torch.bfloat16, (0.0, 1.0)),       # chunk tile 32, gates down to 0
    (1, 3, 700, 48, 40, 40, torch.float32, (0.7, 1.0)),        # fp32, ragged dims and chunks
    (1, 2, 1500, 128, 128, 128, torch.float32, (0.9, 1.0)),    # fp32, C > 64: sub-chunks of 64
    (2, 1, 400, 64, 64, 100, torch.float32, (0.5, 1.0)),       # fp32, sub-chunks of 50
    (2, 2, 600, 128, 128, 64, FP8, (0.9, 1.0)),                # FP8 inputs
    (1, 2, 500, 40, 24, 48, torch.bfloat16, (0.6, 1.0)),       # dims not multiples of 16
    (3, 1, 17, 64, 64, 64, torch.bfloat16, (0.5, 1.0)),        # one chunk, ragged
    (1, 1, 5000, 20, 22, 64, torch.bfloat16, (0.95, 1.0)),     # element path, many chunks
]


@pytest.mark.parametrize("B,H,T,dk,dv,C,dtype,grange", CASES)
def test_gated_prefill_within_the_bar(dev, B, H, T, dk, dv, C, dtype, grange):
    print("gated prefill", B, H, T, dk, dv, C, dtype, grange, flush=True)
    scale = 1.0 if dtype == FP8 else dk ** -0.5
    q, k, v = workloads.gaussian(B, H, T, dk, dv, seed_base=T + dk + C, scale=scale, dtype=dtype)
    g = workloads.gates(B, H, T, seed=T + 7, lo=grange[0], hi=grange[1])
    S0 = torch.randn((B, H, dk, dv), generator=torch.Generator().manual_seed(T))
    O_ref, S_ref = oracle.gated_recurrence(q, k, v, g, S0, nthreads=8)
    S = S0.to(dev).contiguous()
    o = lla.prefill_gated(q.to(dev), k.to(dev), v.to(dev), g.to(dev), S, C)
    torch.cuda.synchronize()
    bar = _bar(dtype)
    assert rel_err(np64(o), O_ref) <= bar and rel_err(np64(S), S_ref) <= bar


@pytest.mark.parametrize("B,H,T,d,C", [(1, 2, 1500, 64, 64), (2, 1, 700, 128, 128), (1, 2, 400, 32, 32)])
def test_gates_of_one_on_integers_exact(dev, B, H, T, d, C):
    """g = 1 is the ungated method: integer inputs give exact outputs and S_T."""
    q, k, v = workloads.integers(B, H, T, d, d, seed=T + C)
    S0 = torch.randint(-4, 5, (B, H, d, d), generator=torch.Generator().manual_seed(3)).float()
    O_ref, S_ref = oracle.recurrence(q, k, v, S0, nthreads=8)
    S = S0.to(dev)
    o = lla.prefill_gated(q.to(dev), k.to(dev), v.to(dev), torch.ones(B, H, T, device=dev), S, C)
    torch.cuda.synchronize()
    assert np.array_equal(np64(o), O_ref) and np.array_equal(np64(S), S_ref)


def test_zero_state_option_equals_a_zero_state(dev):
    B, H, T, d, C = 1, 2, 1200, 64, 64
    q, k, v = workloads.gaussian(B, H, T, d, d, seed_base=5, scale=d ** -0.5, device=dev)
    g = workloads.gates(B, H, T, seed=5, device=dev)
    S_a = torch.zeros((B, H, d, d), device=dev)
    o_a = lla.prefill_gated(q, k, v, g, S_a, C)
    S_b = torch.full((B, H, d, d), float("nan"), device=dev)
    o_b = lla.prefill_gated(q, k, v, g, S_b, C, zero_state=True)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(S_a, S_b)


def test_empty_prompt(dev):
    z = torch.zeros((1, 2, 0, 64), dtype=torch.bfloat16, device=dev)
    S = torch.full((1, 2, 64, 64), 3.0, device=dev)
    lla.prefill_gated(z, z, z, torch.zeros((1, 2, 0), device=dev), S, 64)
    torch.cuda.synchronize()
    assert torch.all(S == 3.0)
    lla.prefill_gated(z, z, z, torch.zeros((1, 2, 0), device=dev), S, 64, zero_state=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(S) == 0


def test_prefill_then_prefill_and_then_decode_steps(dev):
    """The decayed state is still the one object handed between calls."""
    B, H, T1, T2, n, d, C = 2, 2, 700, 500, 6, 128, 64
    T = T1 + T2 + n
    q, k, v = workloads.gaussian(B, H, T, d, d, seed_base=11, scale=d ** -0.5)
    g = workloads.gates(B, H, T, seed=11, lo=0.8)
    O_ref, S_ref = oracle.gated_recurrence(q, k, v, g, None, nthreads=8)
    qd, kd, vd, gd = (x.to(dev) for x in (q, k, v, g))
    S = torch.zeros((B, H, d, d), device=dev)
    o1 = lla.prefill_gated(qd[:, :, :T1].contiguous(), kd[:, :, :T1].contiguous(), vd[:, :, :T1].contiguous(),
                           gd[:, :, :T1].contiguous(), S, C)
    o2 = lla.prefill_gated(qd[:, :, T1:T1 + T2].contiguous(), kd[:, :, T1:T1 + T2].contiguous(),
                           vd[:, :, T1:T1 + T2].contiguous(), gd[:, :, T1:T1 + T2].contiguous(), S, C)
    steps = [lla.decode_step_gated(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(),
                                   gd[:, :, t].contiguous(), S) for t in range(T1 + T2, T)]
    torch.cuda.synchronize()
    o = torch.cat([o1, o2, torch.stack(steps, dim=2)], dim=2)
    assert rel_err(np64(o), O_ref) <= TOL and rel_err(np64(S), S_ref) <= TOL


@pytest.mark.parametrize("B,H,dk,dv,dtype", [(4, 8, 128, 128, torch.bfloat16), (3, 5, 64, 64, torch.float32),
                                             (2, 3, 40, 72, torch.bfloat16), (2, 2, 7, 9, FP8)])
def test_decode_step_dyadic_gates_integers_exact(dev, B, H, dk, dv, dtype):
    """Gates 1, 1/2, 1/4 and small integers: every product and sum is exact
    in fp32, so the decode step equals the oracle bit for bit."""
    q, k, v = workloads.integers(B, H, 3, dk, dv, seed=dk + dv, dtype=dtype)
    g = torch.tensor([1.0, 0.5, 0.25])[torch.randint(0, 3, (B, H, 3), generator=torch.Generator().manual_seed(1))]
    S = torch.randint(-8, 9, (B, H, dk, dv), generator=torch.Generator().manual_seed(2)).float()
    Sd = S.to(dev)
    Sr = S.double().numpy()
    for t in range(3):
        o = lla.decode_step_gated(q[:, :, t].contiguous().to(dev), k[:, :, t].contiguous().to(dev),
                                  v[:, :, t].contiguous().to(dev), g[:, :, t].contiguous().to(dev), Sd)
        torch.cuda.synchronize()
        o_ref, Sr = oracle.gated_decode_step(q[:, :, t], k[:, :, t], v[:, :, t], g[:, :, t], Sr)
        assert np.array_equal(np64(o), o_ref), t
    assert np.array_equal(np64(Sd), Sr)


@pytest.mark.parametrize("d", [128, 64, 40])
def test_decode_step_gate_one_is_the_decode_step_bit_for_bit(dev, d):
    B, H = 8, 4
    q, k, v = workloads.gaussian(B, H, 1, d, d, seed_base=d, scale=d ** -0.5, device=dev)
    S0 = torch.randn((B, H, d, d), generator=torch.Generator(device=dev).manual_seed(d), device=dev)
    S_a, S_b = S0.clone(), S0.clone()
    o_a = lla.decode_step_gated(q[:, :, 0].contiguous(), k[:, :, 0].contiguous(), v[:, :, 0].contiguous(),
                                torch.ones(B, H, device=dev), S_a)
    o_b = lla.decode_step(q[:, :, 0].contiguous(), k[:, :, 0].contiguous(), v[:, :, 0].contiguous(), S_b)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(S_a, S_b)


def test_gates_outside_the_range_are_clamped(dev):
    """g > 1 acts as 1, g <= 0 as 2^-126 (about nothing kept): the results
    match the oracle run on the clamped gates."""
    B, H, T, d, C = 1, 2, 400, 64, 64
    q, k, v = workloads.gaussian(B, H, T, d, d, seed_base=13, scale=d ** -0.5)
    g = workloads.gates(B, H, T, seed=13, lo=-0.5, hi=1.5)
    g_used = g.clamp(2.0 ** -126, 1.0)
    S0 = torch.randn((B, H, d, d), generator=torch.Generator().manual_seed(13))
    O_ref, S_ref = oracle.gated_recurrence(q, k, v, g_used, S0, nthreads=8)
    S = S0.to(dev)
    o = lla.prefill_gated(q.to(dev), k.to(dev), v.to(dev), g.to(dev), S, C)
    torch.cuda.synchronize()
    assert rel_err(np64(o), O_ref) <= TOL and rel_err(np64(S), S_ref) <= TOL


def test_gated_prefill_full_size_sampled_heads(dev):
    """The T=8192 workload's shape (B=1, H=16, d=128, C=64) with gates in
    [0.9, 1]: the whole call on the GPU, four heads against the oracle."""
    cfg = workloads.CONFIGS["prefill_T8192"]
    B, H, T, C, d = cfg.B, cfg.H, cfg.T, cfg.C, cfg.dk
    q, k, v = workloads.config_inputs(cfg, device=dev)
    g = workloads.gates(B, H, T, seed=cfg.seed_base + 9, device=dev)
    S = torch.zeros((B, H, d, d), device=dev)
    o = lla.prefill_gated(q, k, v, g, S, C, zero_state=True)
    torch.cuda.synchronize()
    heads = [0, 5, 10, 15]
    O_ref, S_ref = oracle.gated_recurrence(q[:, heads].cpu(), k[:, heads].cpu(), v[:, heads].cpu(),
                                           g[:, heads].cpu(), None, nthreads=4)
    assert rel_err(np64(o[:, heads]), O_ref) <= TOL and rel_err(np64(S[:, heads]), S_ref) <= TOL


def test_gated_decode_full_size_sampled(dev):
    """The decode workload's shape (B=256, H=32, d=128): one gated step, 64
    sampled states against the oracle."""
    cfg = workloads.CONFIGS["decode_B256"]
    B, H, d = cfg.B, cfg.H, cfg.dk
    S0 = workloads.random_state(cfg, device=dev)
    qd, kd, vd = workloads.decode_inputs(cfg, 1, device=dev)
    g = workloads.gates(B, H, 1, seed=4, device=dev)[:, :, 0].contiguous()
    S = S0.clone()
    o = lla.decode_step_gated(qd[0], kd[0], vd[0], g, S)
    torch.cuda.synchronize()
    idx = torch.arange(0, B * H, (B * H) // 64)
    bs, hs = idx // H, idx % H
    o_ref, S_ref = oracle.gated_decode_step(qd[0][bs, hs].cpu(), kd[0][bs, hs].cpu(), vd[0][bs, hs].cpu(),
                                            g[bs, hs].cpu(), S0[bs, hs].cpu())
    assert rel_err(np64(o[bs, hs]), o_ref) <= 1e-5 and rel_err(np64(S[bs, hs]), S_ref) <= 1e-6


# ---- speculative decoding with a decayed state ------------------------------------

@pytest.mark.parametrize("B,H,k,d,C,dtype", [(6, 4, 5, 128, 64, torch.bfloat16), (5, 3, 40, 64, 64, torch.float32),
                                             (4, 2, 300, 128, 128, FP8), (3, 2, 9, 40, 16, torch.bfloat16)])
def test_gated_verify_and_commit_equal_gated_decode_steps(dev, B, H, k, d, C, dtype):
    """A gated verify pass (KEEP_STATE) gives the outputs of the plain gated
    prefill and leaves S as it was; lla_state_commit_gated then advances each
    sequence by its accepted prefix m_b, bit-equal to m_b gated decode steps."""
    print("gated verify + commit", B, H, k, d, C, dtype, flush=True)
    scale = 1.0 if dtype == FP8 else d ** -0.5
    q, kk, v = workloads.gaussian(B, H, k, d, d, seed_base=k + d, scale=scale, dtype=dtype, device=dev)
    g = workloads.gates(B, H, k, seed=k, lo=0.5, hi=1.0, device=dev)
    S0 = torch.randn((B, H, d, d), generator=torch.Generator(device=dev).manual_seed(k), device=dev)
    S = S0.clone()
    o = lla.prefill_gated(q, kk, v, g, S, C, keep_state=True)
    S_plain = S0.clone()
    o_plain = lla.prefill_gated(q, kk, v, g, S_plain, C)
    torch.cuda.synchronize()
    assert torch.equal(o, o_plain)
    assert torch.equal(S, S0)  # the verify pass wrote nothing
    accepted = [(3 * b + 1) % (k + 1) for b in range(B)]
    lla.state_commit_gated(kk, v, g, S, torch.tensor(accepted, dtype=torch.int32, device=dev))
    Sd = S0.clone()
    want = S0.clone()
    for t in range(max(accepted)):
        lla.decode_step_gated(q[:, :, t].contiguous(), kk[:, :, t].contiguous(), v[:, :, t].contiguous(),
                              g[:, :, t].contiguous(), Sd)
        for b in range(B):
            if accepted[b] == t + 1:
                want[b] = Sd[b]
    torch.cuda.synchronize()
    assert torch.equal(S, want)


def test_gated_commit_with_dyadic_gates_exact_against_the_oracle(dev):
    """Gates 1, 1/2, 1/4 on small integers keep every step exact in fp32: the
    commit of m_b tokens equals the oracle's m_b gated decode steps."""
    B, H, k, dk, dv = 4, 3, 7, 24, 7
    q, kk, v = workloads.integers(B, H, k, dk, dv, seed=41, lo=-2, hi=2)
    g = torch.tensor([1.0, 0.5, 0.25])[torch.randint(0, 3, (B, H, k), generator=torch.Generator().manual_seed(3))]
    S0 = torch.randint(-8, 9, (B, H, dk, dv), generator=torch.Generator().manual_seed(4)).float()
    S = S0.to(dev)
    accepted = [7, 0, 3, 100]  # 100 clamps to 7
    lla.state_commit_gated(kk.to(dev), v.to(dev), g.to(dev), S, torch.tensor(accepted, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    for b, m in enumerate(accepted):
        Sr = S0[b:b + 1].double().numpy()
        for t in range(min(m, k)):
            _, Sr = oracle.gated_decode_step(q[b:b + 1, :, t], kk[b:b + 1, :, t], v[b:b + 1, :, t], g[b:b + 1, :, t],
                                             Sr)
        assert np.array_equal(np64(S[b:b + 1]), Sr), b


# ---- shared-state heads with the decayed state -------------------------------------

GQA_CASES = [
    # B, Hq, Hkv, T, dk, dv, C, dtype
    (2, 8, 2, 700, 128, 128, 64, torch.bfloat16),    # eight-wave walk, several segments
    (2, 4, 1, 17, 64, 64, 64, torch.bfloat16),       # one segment: start states staged in the workspace
    (1, 16, 4, 2000, 128, 128, 128, FP8),            # chunks of 128 as two of 64
    (1, 6, 2, 300, 64, 64, 32, torch.float32),       # four-wave walk
    (2, 6, 3, 500, 40, 48, 48, torch.bfloat16),      # dims not multiples of 16
]


@pytest.mark.parametrize("B,Hq,Hkv,T,dk,dv,C,dtype", GQA_CASES)
def test_gated_grouped_prefill_within_the_bar(dev, B, Hq, Hkv, T, dk, dv, C, dtype):
    print("gated grouped prefill", B, Hq, Hkv, T, dk, dv, C, dtype, flush=True)
    scale = 1.0 if dtype == FP8 else dk ** -0.5
    q, k, v = workloads.gaussian(B, Hq, T, dk, dv, seed_base=T + Hq, scale=scale, dtype=dtype, Hkv=Hkv)
    g = workloads.gates(B, Hkv, T, seed=T + 3, lo=0.8, hi=1.0)
    S0 = torch.randn((B, Hkv, dk, dv), generator=torch.Generator().manual_seed(T))
    O_ref, S_ref = oracle.gated_grouped_recurrence(q, k, v, g, S0, nthreads=8)
    for fresh in (False, True):
        S = torch.zeros_like(S0).to(dev) if fresh else S0.to(dev).contiguous()
        o = lla.prefill_gated(q.to(dev), k.to(dev), v.to(dev), g.to(dev), S, C, zero_state=fresh)
        torch.cuda.synchronize()
        if fresh:
            O_ref, S_ref = oracle.gated_grouped_recurrence(q, k, v, g, None, nthreads=8)
        bar = _bar(dtype)
        assert rel_err(np64(o), O_ref) <= bar and rel_err(np64(S), S_ref) <= bar, fresh


@pytest.mark.parametrize("B,Hq,Hkv,T,d,C", [(1, 8, 2, 1500, 128, 64), (2, 6, 2, 400, 64, 64)])
def test_gated_grouped_gates_of_one_on_integers_exact(dev, B, Hq, Hkv, T, d, C):
    q, k, v = workloads.integers(B, Hq, T, d, d, seed=T + d, Hkv=Hkv)
    g = torch.ones((B, Hkv, T))
    S0 = torch.randint(-50, 51, (B, Hkv, d, d), generator=torch.Generator().manual_seed(T)).float()
    S = S0.to(dev)
    o = lla.prefill_gated(q.to(dev), k.to(dev), v.to(dev), g.to(dev), S, C)
    torch.cuda.synchronize()
    O_ref, S_ref = oracle.gated_grouped_recurrence(q, k, v, g, S0, nthreads=8)
    assert np.array_equal(np64(o), O_ref) and np.array_equal(np64(S), S_ref)


@pytest.mark.parametrize("Hq,Hkv,dk,dv,dtype", [(32, 8, 128, 128, torch.bfloat16), (12, 3, 64, 64, torch.float32),
                                                (40, 2, 128, 128, FP8), (6, 2, 40, 7, torch.bfloat16)])
def test_gated_grouped_decode_equals_gated_steps_on_repeated_heads(dev, Hq, Hkv, dk, dv, dtype):
    """Per query head the arithmetic of the gated step (the decay, the
    update, the state read in row order): bit-equal to gated steps on the
    key/value heads, states and gates repeated over each group."""
    B, G = 5, Hq // Hkv
    gen = torch.Generator(device=dev).manual_seed(Hq + dk)
    q = torch.randn((B, Hq, dk), generator=gen, device=dev).to(dtype)
    k = torch.randn((B, Hkv, dk), generator=gen, device=dev).to(dtype)
    v = torch.randn((B, Hkv, dv), generator=gen, device=dev).to(dtype)
    gt = torch.rand((B, Hkv), generator=gen, device=dev) * 0.5 + 0.5
    S0 = torch.randn((B, Hkv, dk, dv), generator=gen, device=dev)
    S_g = S0.clone()
    o_g = lla.decode_step_gated(q, k, v, gt, S_g)
    S_r = S0.repeat_interleave(G, dim=1).contiguous()
    o_r = lla.decode_step_gated(q, k.repeat_interleave(G, dim=1).contiguous(), v.repeat_interleave(G, dim=1).contiguous(),
                                gt.repeat_interleave(G, dim=1).contiguous(), S_r)
    torch.cuda.synchronize()
    assert torch.equal(o_g, o_r)
    assert torch.equal(S_g, S_r[:, ::G])


def test_gated_grouped_decode_dyadic_gates_integers_exact(dev):
    B, Hq, Hkv, dk, dv = 3, 8, 2, 64, 24
    q, k, v = workloads.integers(B, Hq, 3, dk, dv, seed=5, Hkv=Hkv)
    g = torch.tensor([1.0, 0.5, 0.25])[torch.randint(0, 3, (B, Hkv, 3), generator=torch.Generator().manual_seed(6))]
    S = torch.randint(-8, 9, (B, Hkv, dk, dv), generator=torch.Generator().manual_seed(7)).float()
    Sd = S.to(dev)
    Sr = S.double().numpy()
    for t in range(3):
        o = lla.decode_step_gated(q[:, :, t].contiguous().to(dev), k[:, :, t].contiguous().to(dev),
                                  v[:, :, t].contiguous().to(dev), g[:, :, t].contiguous().to(dev), Sd)
        torch.cuda.synchronize()
        o_ref, Sr = oracle.gated_grouped_decode_step(q[:, :, t], k[:, :, t], v[:, :, t], g[:, :, t], Sr)
        assert np.array_equal(np64(o), o_ref), t
    assert np.array_equal(np64(Sd), Sr)


def test_gated_grouped_verify_pass_and_commit(dev):
    """Shared-state heads with a decayed state: the verify pass equals the
    plain gated prefill and leaves S; the commit (on the key/value states)
    equals m_b gated decode steps."""
    B, Hq, Hkv, k, d, C = 4, 8, 2, 12, 128, 64
    q, kk, v = workloads.gaussian(B, Hq, k, d, d, seed_base=31, scale=d ** -0.5, device=dev, Hkv=Hkv)
    g = workloads.gates(B, Hkv, k, seed=32, lo=0.5, hi=1.0, device=dev)
    S0 = torch.randn((B, Hkv, d, d), generator=torch.Generator(device=dev).manual_seed(33), device=dev)
    S = S0.clone()
    o = lla.prefill_gated(q, kk, v, g, S, C, keep_state=True)
    S_plain = S0.clone()
    o_plain = lla.prefill_gated(q, kk, v, g, S_plain, C)
    torch.cuda.synchronize()
    assert torch.equal(o, o_plain) and torch.equal(S, S0)
    accepted = [0, 5, 12, 7]
    lla.state_commit_gated(kk, v, g, S, torch.tensor(accepted, dtype=torch.int32, device=dev))
    Sd, want = S0.clone(), S0.clone()
    for t in range(max(accepted)):
        lla.decode_step_gated(q[:, :, t].contiguous(), kk[:, :, t].contiguous(), v[:, :, t].contiguous(),
                              g[:, :, t].contiguous(), Sd)
        for b in range(B):
            if accepted[b] == t + 1:
                want[b] = Sd[b]
    torch.cuda.synchronize()
    assert torch.equal(S, want)
