"""Shared-state heads: Hq query heads grouped on Hkv key/value heads (blog "A
128 000 tokens, l'attention avale 85 % du calcul", section on sharing heads).
Query head h reads key/value head h // G, G = Hq / Hkv.  The prefill and the
decode step are checked against the oracle (exact on integer inputs, within
the bf16 tolerance on gaussian ones), against the plain call on key/value
heads repeated over their group (the same arithmetic: identical bits), and at
the full benchmark sizes on sampled heads.  Short prompts with groups run on
the matrix cores (bf16, FP8, at least 8 tokens) or as fused grouped decode
steps (fewer tokens, fp32 inputs, verify passes), and are checked
accordingly."""
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


def _run_prefill(q, k, v, S0, C, dev, zero_state=False):
    S = S0.to(dev, torch.float32).contiguous().clone()
    o = lla.prefill(q.to(dev).contiguous(), k.to(dev).contiguous(), v.to(dev).contiguous(), S, chunk=C,
                    zero_state=zero_state)
    torch.cuda.synchronize()
    return o, S


# B, Hq, Hkv, T, dk, dv, C, dtype: the eight-wave bf16 d=128 walk (one and
# several segments, ragged tail), d=64, a short prompt (chunked for groups),
# the fp32 and ragged-dimension paths, the largest group the decode takes,
# chunks of 128
GQA_INT = [
    (2, 8, 2, 300, 128, 128, 64, torch.bfloat16),
    (1, 4, 1, 2100, 128, 128, 64, torch.bfloat16),
    (1, 6, 3, 130, 64, 64, 32, torch.bfloat16),
    (2, 4, 2, 9, 128, 128, 64, torch.bfloat16),
    (2, 6, 3, 77, 40, 72, 16, torch.float32),
    (1, 16, 1, 200, 64, 64, 64, torch.bfloat16),
    (3, 2, 1, 260, 104, 120, 20, torch.bfloat16),
    (1, 6, 2, 700, 128, 128, 128, torch.bfloat16),
]


@pytest.mark.parametrize("B,Hq,Hkv,T,dk,dv,C,dtype", GQA_INT)
def test_gqa_prefill_integers_exact(dev, B, Hq, Hkv, T, dk, dv, C, dtype):
    print("gqa prefill int", B, Hq, Hkv, T, dk, dv, C, dtype, flush=True)
    q, k, v = workloads.integers(B, Hq, T, dk, dv, seed=T + Hq, dtype=dtype, Hkv=Hkv)
    S0 = torch.randint(-300, 301, (B, Hkv, dk, dv), generator=torch.Generator().manual_seed(T)).float()
    o, S = _run_prefill(q, k, v, S0, C, dev)
    O_ref, S_ref = oracle.grouped_recurrence(q, k, v, S0, nthreads=8)
    assert np.array_equal(np64(o), O_ref)
    assert np.array_equal(np64(S), S_ref)


@pytest.mark.parametrize("T,C", [(1000, 64), (517, 32)])
def test_gqa_prefill_gaussian(dev, T, C):
    B, Hq, Hkv, d = 1, 16, 4, 128
    q, k, v = workloads.gaussian(B, Hq, T, d, d, seed_base=T, scale=d ** -0.5, l2norm_k=True, Hkv=Hkv)
    S0 = torch.randn((B, Hkv, d, d), generator=torch.Generator().manual_seed(C))
    o, S = _run_prefill(q, k, v, S0, C, dev)
    O_ref, S_ref = oracle.grouped_recurrence(q, k, v, S0, nthreads=8)
    assert rel_err(np64(o), O_ref) <= TOL
    assert rel_err(np64(S), S_ref) <= TOL


@pytest.mark.parametrize("B,Hq,Hkv,T,d,C", [(2, 8, 2, 300, 128, 64), (1, 12, 4, 1500, 64, 64),
                                            (1, 16, 4, 8192, 128, 64)])
def test_gqa_prefill_equals_repeated_heads(dev, B, Hq, Hkv, T, d, C):
    """Repeating every key/value head (and its state) over its group and making
    the plain call gives the same bits: each query head's walk does the same
    arithmetic on the same data, and the segment plan depends on Hq only."""
    G = Hq // Hkv
    q, k, v = workloads.gaussian(B, Hq, T, d, d, seed_base=7, scale=d ** -0.5, device=dev, Hkv=Hkv)
    S0 = torch.randn((B, Hkv, d, d), generator=torch.Generator(device=dev).manual_seed(3), device=dev)
    S_g = S0.clone()
    o_g = lla.prefill(q, k, v, S_g, chunk=C)
    S_r = S0.repeat_interleave(G, dim=1).contiguous()
    o_r = lla.prefill(q, k.repeat_interleave(G, dim=1).contiguous(),
                      v.repeat_interleave(G, dim=1).contiguous(), S_r, chunk=C)
    torch.cuda.synchronize()
    assert torch.equal(o_g, o_r)
    for g in range(G):
        assert torch.equal(S_g, S_r[:, g::G])


def test_gqa_prefill_full_size_sampled(dev):
    """The grouped T=8192 workload (16 query heads on 4 key/value heads,
    d=128, C=64) in the launch configuration the benchmark times; three query
    heads and every key/value state against the oracle."""
    cfg = workloads.CONFIGS["prefill_T8192_gqa"]
    q, k, v = workloads.config_inputs(cfg, device=dev)
    S = lla.state_init(cfg.B, cfg.kv_heads, cfg.dk, cfg.dv, device=dev)
    call = lla.PreparedPrefill(q, k, v, S, cfg.C)
    call(zero_state=True)
    torch.cuda.synchronize()
    G = cfg.H // cfg.kv_heads
    for h in (0, 6, 15):
        O_ref, _ = oracle.recurrence(q[:, h:h + 1].cpu(), k[:, h // G:h // G + 1].cpu(),
                                     v[:, h // G:h // G + 1].cpu(), nthreads=8)
        assert rel_err(np64(call.out[:, h:h + 1]), O_ref) <= TOL, h
    kc, vc = k.cpu(), v.cpu()
    _, S_ref = oracle.recurrence(kc, kc, vc, nthreads=8)  # the state ignores the queries
    assert rel_err(np64(S), S_ref) <= TOL


# ---- decode ---------------------------------------------------------------------

@pytest.mark.parametrize("B,Hq,Hkv,d,dtype", [(3, 8, 2, 128, torch.bfloat16), (2, 16, 1, 64, torch.float32),
                                              (4, 6, 3, 64, torch.bfloat16), (1, 2, 1, 128, torch.float32)])
def test_gqa_decode_integers_exact(dev, B, Hq, Hkv, d, dtype):
    print("gqa decode int", B, Hq, Hkv, d, dtype, flush=True)
    gen = torch.Generator().manual_seed(Hq * 10 + d)
    q = torch.randint(-2, 3, (B, Hq, d), generator=gen).to(dtype)
    k = torch.randint(-2, 3, (B, Hkv, d), generator=gen).to(dtype)
    v = torch.randint(-2, 3, (B, Hkv, d), generator=gen).to(dtype)
    S0 = torch.randint(-300, 301, (B, Hkv, d, d), generator=gen).float()
    S = S0.to(dev).contiguous()
    o = lla.decode_step(q.to(dev).contiguous(), k.to(dev).contiguous(), v.to(dev).contiguous(), S)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.grouped_decode_step(q, k, v, S0)
    assert np.array_equal(np64(o), o_ref)
    assert np.array_equal(np64(S), S_ref)


# Groups beyond one LDS batch of 16 query rows, and head dims other than
# 64 and 128 (the general kernel: 4 value columns per thread when dv is a
# multiple of 4, else 1)
ANY_SHAPES = [
    # B, Hq, Hkv, dk, dv, dtype
    (2, 40, 2, 128, 128, torch.bfloat16),        # G = 20: two batches
    (1, 64, 1, 64, 64, torch.float32),           # G = 64: four batches
    (3, 8, 2, 96, 80, torch.bfloat16),
    (2, 6, 1, 128, 5, torch.float32),
    (1, 34, 2, 40, 127, torch.float8_e4m3fn),    # G = 17, 64 rows per thread
    (2, 48, 3, 1, 1, torch.bfloat16),
    (1, 36, 2, 33, 128, torch.bfloat16),         # G = 18 on the general kernel
]


@pytest.mark.parametrize("B,Hq,Hkv,dk,dv,dtype", ANY_SHAPES)
def test_gqa_decode_any_shape_integers_exact(dev, B, Hq, Hkv, dk, dv, dtype):
    print("gqa decode any", B, Hq, Hkv, dk, dv, dtype, flush=True)
    gen = torch.Generator().manual_seed(Hq * 7 + dk + dv)
    q = torch.randint(-2, 3, (B, Hq, dk), generator=gen).to(dtype)
    k = torch.randint(-2, 3, (B, Hkv, dk), generator=gen).to(dtype)
    v = torch.randint(-2, 3, (B, Hkv, dv), generator=gen).to(dtype)
    S0 = torch.randint(-300, 301, (B, Hkv, dk, dv), generator=gen).float()
    S = S0.to(dev).contiguous()
    o = lla.decode_step(q.to(dev).contiguous(), k.to(dev).contiguous(), v.to(dev).contiguous(), S)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.grouped_decode_step(q, k, v, S0)
    assert np.array_equal(np64(o), o_ref)
    assert np.array_equal(np64(S), S_ref)


@pytest.mark.parametrize("B,Hq,Hkv,dk,dv,dtype", ANY_SHAPES)
def test_gqa_decode_any_shape_equals_repeated_heads(dev, B, Hq, Hkv, dk, dv, dtype):
    G = Hq // Hkv
    gen = torch.Generator(device=dev).manual_seed(Hq + dk * dv)
    q = torch.randn((B, Hq, dk), generator=gen, device=dev).to(dtype)
    k = torch.randn((B, Hkv, dk), generator=gen, device=dev).to(dtype)
    v = torch.randn((B, Hkv, dv), generator=gen, device=dev).to(dtype)
    S0 = torch.randn((B, Hkv, dk, dv), generator=gen, device=dev)
    S_g = S0.clone()
    o_g = lla.decode_step(q, k, v, S_g)
    S_r = S0.repeat_interleave(G, dim=1).contiguous()
    o_r = lla.decode_step(q, k.repeat_interleave(G, dim=1).contiguous(),
                          v.repeat_interleave(G, dim=1).contiguous(), S_r)
    torch.cuda.synchronize()
    assert torch.equal(o_g, o_r)
    assert torch.equal(S_g, S_r[:, ::G])


@pytest.mark.parametrize("Hq,Hkv,d", [(32, 8, 128), (16, 1, 128), (8, 8, 64), (12, 3, 64)])
def test_gqa_decode_equals_repeated_heads(dev, Hq, Hkv, d):
    B, G = 5, Hq // Hkv
    gen = torch.Generator(device=dev).manual_seed(Hq + d)
    q = torch.randn((B, Hq, d), generator=gen, device=dev).to(torch.bfloat16)
    k = torch.randn((B, Hkv, d), generator=gen, device=dev).to(torch.bfloat16)
    v = torch.randn((B, Hkv, d), generator=gen, device=dev).to(torch.bfloat16)
    S0 = torch.randn((B, Hkv, d, d), generator=gen, device=dev)
    S_g = S0.clone()
    o_g = lla.decode_step(q, k, v, S_g)
    S_r = S0.repeat_interleave(G, dim=1).contiguous()
    o_r = lla.decode_step(q, k.repeat_interleave(G, dim=1).contiguous(),
                          v.repeat_interleave(G, dim=1).contiguous(), S_r)
    torch.cuda.synchronize()
    assert torch.equal(o_g, o_r)
    assert torch.equal(S_g, S_r[:, ::G])


def test_gqa_decode_steps_continue_a_grouped_prefill(dev):
    B, Hq, Hkv, T, d = 2, 8, 2, 150, 128
    q, k, v = workloads.gaussian(B, Hq, T, d, d, seed_base=11, scale=d ** -0.5, Hkv=Hkv)
    S = lla.state_init(B, Hkv, d, d, device=dev)
    o = lla.prefill(q[:, :, :140].to(dev).contiguous(), k[:, :, :140].to(dev).contiguous(),
                    v[:, :, :140].to(dev).contiguous(), S, chunk=64)
    outs = [lla.decode_step(q[:, :, t].to(dev).contiguous(), k[:, :, t].to(dev).contiguous(),
                            v[:, :, t].to(dev).contiguous(), S) for t in range(140, T)]
    torch.cuda.synchronize()
    O_ref, S_ref = oracle.grouped_recurrence(q, k, v, nthreads=8)
    assert rel_err(np64(o), O_ref[:, :, :140]) <= TOL
    assert rel_err(np.stack([np64(x) for x in outs], axis=2), O_ref[:, :, 140:]) <= TOL
    assert rel_err(np64(S), S_ref) <= TOL


def test_gqa_decode_full_size_sampled(dev):
    """One step of the grouped decode batch (256 sequences, 32 query heads on
    8 key/value heads, d=128) as the benchmark launches it; sampled sequences
    against the oracle."""
    cfg = workloads.CONFIGS["decode_B256_gqa"]
    S0 = workloads.random_state(cfg, device=dev)
    qd, kd, vd = workloads.decode_inputs(cfg, 1, device=dev)
    S = S0.clone()
    o = torch.empty((cfg.B, cfg.H, cfg.dv), dtype=torch.float32, device=dev)
    lla.PreparedDecode(qd[0], kd[0], vd[0], S, out=o)()
    torch.cuda.synchronize()
    for b in (0, 97, 255):
        o_ref, S_ref = oracle.grouped_decode_step(qd[0, b:b + 1].cpu(), kd[0, b:b + 1].cpu(),
                                                  vd[0, b:b + 1].cpu(), S0[b:b + 1].cpu())
        assert rel_err(np64(o[b:b + 1]), o_ref) <= 1e-5, b
        assert rel_err(np64(S[b:b + 1]), S_ref) <= 1e-6, b


def test_gqa_continuation_on_matrix_cores_full_size_sampled(dev):
    """The benchmark's 16-token continuation of the grouped decode states
    (256 sequences, 32 query heads on 8 key/value heads, d=128), launched as
    the benchmark launches it (PreparedPrefill: the matrix-core route);
    sampled sequences against the oracle within the bar."""
    cfg = workloads.CONFIGS["decode_B256_gqa"]
    S0 = workloads.random_state(cfg, device=dev)
    qc, kc, vc = (x.permute(1, 2, 0, 3).contiguous() for x in workloads.decode_inputs(cfg, 16, device=dev))
    S = S0.clone()
    o = lla.PreparedPrefill(qc, kc, vc, S, cfg.C)()
    torch.cuda.synchronize()
    for b in (0, 131, 255):
        O_ref, S_ref = oracle.grouped_recurrence(qc[b:b + 1].cpu(), kc[b:b + 1].cpu(), vc[b:b + 1].cpu(),
                                                 S0[b:b + 1].cpu(), nthreads=8)
        assert rel_err(np64(o[b:b + 1]), O_ref) <= TOL, b
        assert rel_err(np64(S[b:b + 1]), S_ref) <= TOL, b


# ---- short continuations with shared-state heads ---------------------------------

@pytest.mark.parametrize("B,Hq,Hkv,T,d,dtype,keep", [
    (2, 8, 2, 5, 128, torch.bfloat16, False), (2, 8, 2, 5, 128, torch.bfloat16, True),
    (1, 16, 1, 4, 128, torch.bfloat16, False), (3, 4, 2, 16, 64, torch.float32, False),
    (3, 4, 2, 16, 64, torch.float32, True), (2, 6, 3, 7, 64, torch.float8_e4m3fn, False),
    (1, 8, 1, 8, 128, torch.bfloat16, True), (2, 4, 1, 1, 128, torch.bfloat16, False),
])
def test_gqa_short_prompt_decode_steps_route_equals_grouped_decode_steps(dev, B, Hq, Hkv, T, d, dtype, keep):
    """T <= 16 tokens with T * G <= 64 that run as fused grouped decode steps
    -- fewer than 8 tokens, fp32 inputs, and every verify pass (the state
    kept) -- give the same bits as T lla_decode_step_gqa calls."""
    print("gqa short prompt, decode-step route", B, Hq, Hkv, T, d, dtype, keep, flush=True)
    q, k, v = workloads.gaussian(B, Hq, T, d, d, seed_base=T * 3 + Hq, scale=d ** -0.5, dtype=dtype,
                                 device=dev, Hkv=Hkv)
    S0 = torch.randn((B, Hkv, d, d), generator=torch.Generator(device=dev).manual_seed(T), device=dev)
    S_a = S0.clone()
    o_a = lla.prefill(q, k, v, S_a, chunk=64, keep_state=keep)
    S_b = S0.clone()
    o_b = torch.stack([lla.decode_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                                       v[:, :, t].contiguous(), S_b) for t in range(T)], dim=2)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b)
    assert torch.equal(S_a, S0 if keep else S_b)


@pytest.mark.parametrize("B,Hq,Hkv,T,d,dtype", [
    (4, 32, 8, 16, 128, torch.bfloat16), (1, 8, 1, 8, 128, torch.bfloat16), (3, 4, 2, 16, 64, torch.bfloat16),
    (2, 6, 2, 9, 128, torch.bfloat16), (2, 8, 2, 10, 64, torch.float8_e4m3fn),
    (1, 6, 1, 8, 128, torch.float8_e4m3fn), (2, 8, 2, 5, 128, torch.bfloat16),
])
def test_gqa_short_prompt_on_matrix_cores_within_the_bar(dev, B, Hq, Hkv, T, d, dtype):
    """With several query heads per state, bf16 and FP8 short prompts of 8 to
    16 tokens run as one chunk on the matrix cores (T G query rows, ragged
    when not a multiple of 16): within the floating-point bar of the oracle,
    from a gaussian state, fresh or continued.  (Shorter ones, last case,
    take the decode-step route, also within the bar.)"""
    print("gqa short prompt, matrix cores", B, Hq, Hkv, T, d, dtype, flush=True)
    scale = 1.0 if dtype == torch.float8_e4m3fn else d ** -0.5
    q, k, v = workloads.gaussian(B, Hq, T, d, d, seed_base=T * 5 + Hq, scale=scale, dtype=dtype, Hkv=Hkv)
    S0 = torch.randn((B, Hkv, d, d), generator=torch.Generator().manual_seed(T + 1))
    for fresh in (False, True):
        o, S = _run_prefill(q, k, v, torch.zeros_like(S0) if fresh else S0, 64, dev, zero_state=fresh)
        O_ref, S_ref = oracle.grouped_recurrence(q, k, v, None if fresh else S0, nthreads=8)
        assert rel_err(np64(o), O_ref) <= TOL and rel_err(np64(S), S_ref) <= TOL, fresh


@pytest.mark.parametrize("Hq,Hkv,T", [(8, 1, 8), (8, 1, 9), (4, 1, 16), (4, 1, 17), (2, 1, 1)])
def test_gqa_short_prompt_integers_exact_at_the_route_boundary(dev, Hq, Hkv, T):
    """T * G = 64 (fused) and 72 (chunked), T = 16 and 17: all exact."""
    B, d = 2, 128
    q, k, v = workloads.integers(B, Hq, T, d, d, seed=T + Hq, Hkv=Hkv)
    S0 = torch.randint(-300, 301, (B, Hkv, d, d), generator=torch.Generator().manual_seed(T)).float()
    o, S = _run_prefill(q, k, v, S0, 64, dev)
    O_ref, S_ref = oracle.grouped_recurrence(q, k, v, S0, nthreads=8)
    assert np.array_equal(np64(o), O_ref)
    assert np.array_equal(np64(S), S_ref)
    S_z = torch.full((B, Hkv, d, d), float("nan"), device=dev)  # fresh prompt: S never read
    o_z = lla.prefill(q.to(dev).contiguous(), k.to(dev).contiguous(), v.to(dev).contiguous(), S_z,
                      chunk=64, zero_state=True)
    torch.cuda.synchronize()
    O_z, S_zr = oracle.grouped_recurrence(q, k, v, nthreads=8)
    assert np.array_equal(np64(o_z), O_z)
    assert np.array_equal(np64(S_z), S_zr)


@pytest.mark.parametrize("B,Hq,Hkv,T,dtype", [(75, 16, 4, 12, torch.bfloat16), (130, 8, 4, 16, torch.float8_e4m3fn),
                                              (3, 16, 2, 8, torch.bfloat16)])
def test_gqa_matrix_core_continuation_walks_several_heads_per_workgroup(dev, B, Hq, Hkv, T, dtype):
    """At d = 128 the matrix-core continuation runs 256 persistent workgroups
    that walk the key/value heads (300 and 520 heads here: two or three per
    workgroup, the next head's loads in flight during the current one; 6
    heads: one each): integers exact against the oracle, from a given state
    and fresh (the state never read)."""
    print("gqa matrix-core continuation, several heads per workgroup", B, Hq, Hkv, T, dtype, flush=True)
    d = 128
    q, k, v = workloads.integers(B, Hq, T, d, d, seed=B + T, Hkv=Hkv, dtype=dtype)
    S0 = torch.randint(-300, 301, (B, Hkv, d, d), generator=torch.Generator().manual_seed(B)).float()
    o, S = _run_prefill(q, k, v, S0, 64, dev)
    O_ref, S_ref = oracle.grouped_recurrence(q, k, v, S0, nthreads=8)
    assert np.array_equal(np64(o), O_ref)
    assert np.array_equal(np64(S), S_ref)
    S_z = torch.full((B, Hkv, d, d), float("nan"), device=dev)  # fresh prompt: S never read
    o_z = lla.prefill(q.to(dev).contiguous(), k.to(dev).contiguous(), v.to(dev).contiguous(), S_z,
                      chunk=64, zero_state=True)
    torch.cuda.synchronize()
    O_z, S_zr = oracle.grouped_recurrence(q, k, v, nthreads=8)
    assert np.array_equal(np64(o_z), O_z)
    assert np.array_equal(np64(S_z), S_zr)
