"""GPU invariants the deck states, and the prefill phases, through the C ABI.

* chunking is exact: every C gives the same result (deck, "Common errors");
* the state is the one object handed between blocks: prefill(T1) then
  prefill(T2) from its state equals prefill(T1 + T2); prefill then decode
  steps equals a longer prefill (deck, "Prefill and decode": two code paths,
  the same numbers);
* the three phases called one by one equal lla_prefill, and the workspace
  holds the state at every segment start;
* repeat runs are bitwise identical; every output element is written.
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


def test_chunk_size_invariance_integers(dev):
    q, k, v = workloads.integers(2, 3, 1500, 128, 128, seed=9)
    ref = None
    for C in (1, 5, 16, 32, 48, 64, 100, 128):
        o, S = gpu_prefill(q, k, v, C=C)
        if ref is None:
            ref = (np64(o), np64(S))
            O_ref, S_ref = oracle.recurrence(q, k, v, nthreads=6)
            assert np.array_equal(ref[0], O_ref) and np.array_equal(ref[1], S_ref)
        else:
            assert np.array_equal(np64(o), ref[0]), C
            assert np.array_equal(np64(S), ref[1]), C


def test_chunk_size_invariance_long_prompt_all_heads(dev):
    """The T=131072 shape at C = 128, 64 and 100: chunks of 128 run as two of
    64 with twice the chunks per segment, which is the plan for C = 64 -- the
    same bits; C = 100 (two of 50) agrees within the tolerance (the oracle
    checks sampled heads in the parity suite)."""
    cfg = workloads.CONFIGS["prefill_T131072"]
    q, k, v = workloads.config_inputs(cfg, device=dev)
    o1, S1 = gpu_prefill(q, k, v, C=128)
    o2, S2 = gpu_prefill(q, k, v, C=64)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    del o2, S2
    o3, S3 = gpu_prefill(q, k, v, C=100)
    e_o = (o1 - o3).abs().max().item() / o1.abs().max().item()
    e_s = (S1 - S3).abs().max().item() / S1.abs().max().item()
    assert e_o <= TOL and e_s <= TOL


def test_continuation_prefill_then_prefill(dev):
    q, k, v = workloads.integers(1, 4, 2500, 64, 64, seed=12)
    o_all, S_all = gpu_prefill(q, k, v, C=64)
    o1, S1 = gpu_prefill(q[:, :, :1111], k[:, :, :1111], v[:, :, :1111], C=64)
    o2, S2 = gpu_prefill(q[:, :, 1111:], k[:, :, 1111:], v[:, :, 1111:], C=64, S0=S1)
    assert torch.equal(torch.cat([o1, o2], 2), o_all) and torch.equal(S2, S_all)


def test_prefill_then_decode_equals_longer_prefill(dev):
    q, k, v = workloads.integers(2, 4, 520, 128, 128, seed=13)
    o_all, S_all = gpu_prefill(q, k, v, C=64)
    o_pre, S = gpu_prefill(q[:, :, :500], k[:, :, :500], v[:, :, :500], C=64)
    for t in range(500, 520):
        o = lla.decode_step(q[:, :, t].contiguous().to(dev), k[:, :, t].contiguous().to(dev),
                            v[:, :, t].contiguous().to(dev), S)
        assert torch.equal(o, o_all[:, :, t]), t
    assert torch.equal(S, S_all)


def test_phases_equal_prefill_and_workspace_holds_segment_states(dev):
    B, H, T, d, C = 1, 2, 64 * 600, 64, 64
    q, k, v = (x.to(dev) for x in workloads.integers(B, H, T, d, d, seed=14))
    G = lla.prefill_segment_chunks(B, H, T, d, d, C)
    n_c = -(-T // C)
    n_seg = -(-n_c // G)
    assert G > 1 and n_seg > 1
    S_a = lla.state_init(B, H, d, d, device=dev)
    o_a = lla.prefill(q, k, v, S_a, chunk=C)
    S_b = lla.state_init(B, H, d, d, device=dev)
    ws = lla.prefill_segment_states(k, v, C, None)
    lla.prefill_state_scan(S_b, T, C, ws)
    o_b = lla.prefill_chunks(q, k, v, S_b, C, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(S_a, S_b)
    slots = np64(ws.view(B, H, n_seg, d, d))
    _, _, ck = oracle.recurrence(q.cpu(), k.cpu(), v.cpu(), ckpt_every=G * C, nthreads=2)
    assert np.array_equal(slots[:, :, 0], np.zeros((B, H, d, d)))
    assert np.array_equal(slots[:, :, 1:], ck[:, :, :n_seg - 1])


def test_repeat_runs_are_bitwise_identical_and_outputs_fully_written(dev):
    cfg = workloads.CONFIGS["prefill_T8192"]
    q, k, v = (x.to(dev) for x in workloads.config_inputs(cfg))
    outs = []
    for _ in range(2):
        S = lla.state_init(cfg.B, cfg.H, cfg.dk, cfg.dv, device=dev)
        o = torch.full((cfg.B, cfg.H, cfg.T, cfg.dv), float("nan"), device=dev)
        lla.prefill(q, k, v, S, chunk=cfg.C, out=o)
        torch.cuda.synchronize()
        assert not torch.isnan(o).any()
        outs.append((o, S))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_empty_prompt_is_a_no_op(dev):
    S = torch.arange(2 * 3 * 8 * 8, dtype=torch.float32, device=dev).view(2, 3, 8, 8)
    S0 = S.clone()
    e = torch.empty((2, 3, 0, 8), dtype=torch.bfloat16, device=dev)
    o = lla.prefill(e, e, e, S, chunk=4)
    torch.cuda.synchronize()
    assert o.shape == (2, 3, 0, 8) and torch.equal(S, S0)


def test_state_init_zeroes(dev):
    S = torch.full((3, 5, 7, 9), 7.0, device=dev)
    lla.state_init(3, 5, 7, 9, out=S)
    torch.cuda.synchronize()
    assert torch.count_nonzero(S).item() == 0


def test_bad_arguments_raise_before_launch(dev):
    q = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16, device=dev)
    S = lla.state_init(1, 1, 64, 64, device=dev)
    with pytest.raises(lla.LlaError):
        lla.prefill(q, q, q, S, chunk=0)
    with pytest.raises(lla.LlaError):
        lla.prefill(q, q, q, S, chunk=129)
    with pytest.raises(TypeError):
        lla.prefill(q.half(), q.half(), q.half(), S, chunk=64)


# B, Hq, Hkv, T, dk, dv, C, dtype: several segments (eight-wave walk), one
# segment and no workspace (the walk reads S itself), d = 64 and fp32
# four-wave walks, a short prompt (fused decode steps), grouped heads, FP8,
# chunks of 128 (run as two of 64; several segments, then one)
ZERO_CASES = [
    (1, 16, 16, 8192, 128, 128, 64, torch.bfloat16),
    (64, 8, 8, 128, 128, 128, 64, torch.bfloat16),
    (4, 8, 8, 1024, 64, 64, 64, torch.bfloat16),
    (64, 8, 8, 128, 64, 64, 64, torch.bfloat16),
    (1, 2, 2, 77, 40, 72, 16, torch.float32),
    (2, 3, 3, 5, 128, 128, 64, torch.bfloat16),
    (1, 8, 2, 333, 128, 128, 32, torch.bfloat16),
    (2, 4, 4, 300, 128, 128, 64, torch.float8_e4m3fn),
    (1, 4, 4, 600, 128, 128, 128, torch.bfloat16),
    (64, 4, 4, 256, 128, 128, 128, torch.bfloat16),
]


@pytest.mark.parametrize("B,Hq,Hkv,T,dk,dv,C,dtype", ZERO_CASES)
def test_zero_state_option_equals_init_then_prefill(dev, B, Hq, Hkv, T, dk, dv, C, dtype):
    """lla_prefill_ex with the zero-state option never reads S (here full of
    NaN) and gives the bits of lla_state_init followed by lla_prefill."""
    print("zero-state", B, Hq, Hkv, T, dk, dv, C, dtype, flush=True)
    q, k, v = workloads.gaussian(B, Hq, T, dk, dv, seed_base=T + B, scale=dk ** -0.5, dtype=dtype,
                                 device=dev, Hkv=Hkv)
    S_a = lla.state_init(B, Hkv, dk, dv, device=dev)
    o_a = lla.prefill(q, k, v, S_a, chunk=C)
    S_b = torch.full((B, Hkv, dk, dv), float("nan"), device=dev)
    o_b = lla.prefill(q, k, v, S_b, chunk=C, zero_state=True)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b)
    assert torch.equal(S_a, S_b)


def test_zero_state_option_on_an_empty_prompt_zeroes_the_state(dev):
    q = torch.zeros((2, 3, 0, 64), dtype=torch.bfloat16, device=dev)
    S = torch.full((2, 3, 64, 64), 7.0, device=dev)
    lla.prefill(q, q, q, S, chunk=64, zero_state=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(S) == 0


def test_prepared_fresh_prompt_repeats(dev):
    """PreparedPrefill(zero_state=True) repeated on the same buffers: the state
    it leaves behind is never read back, so every call gives the same bits."""
    q, k, v = workloads.gaussian(1, 4, 700, 128, 128, seed_base=3, scale=128 ** -0.5, device=dev)
    S = lla.state_init(1, 4, 128, 128, device=dev)
    call = lla.PreparedPrefill(q, k, v, S, 64)
    o1 = call(zero_state=True).clone()
    S1 = S.clone()
    o2 = call(zero_state=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S)
    O_ref, S_ref = oracle.recurrence(q.cpu(), k.cpu(), v.cpu(), nthreads=8)
    assert rel_err(np64(o2), O_ref) <= TOL and rel_err(np64(S), S_ref) <= TOL


# B, Hq, Hkv, T, dk, dv, C, dtype: shapes whose fresh prompts lla_prefill runs
# as one launch (the walks sum the earlier segments themselves): the T=1024
# workload (8 segments of 2 chunks), 32-row tiles with a short last chunk,
# two value blocks (fp32, D = 128), the element path (dk, dv not whole
# vectors), FP8 with chunks of 100 run as two of 50 (16 chunks before the
# last segment, the most this route takes), shared-state heads
ONE_LAUNCH_CASES = [
    (4, 8, 8, 1024, 64, 64, 64, torch.bfloat16),
    (2, 4, 4, 500, 64, 64, 32, torch.bfloat16),
    (1, 2, 2, 77, 40, 72, 16, torch.float32),
    (1, 3, 3, 500, 7, 5, 48, torch.float32),
    (2, 4, 4, 900, 64, 64, 100, torch.float8_e4m3fn),
    (1, 8, 2, 600, 64, 64, 64, torch.bfloat16),
]


def _three_phases(q, k, v, S, C):
    """lla_prefill's three phases called one by one (shared-state heads as
    repeated heads: the same sums per head)."""
    Hq, Hkv = q.shape[1], k.shape[1]
    if Hq != Hkv:
        k, v = (x.repeat_interleave(Hq // Hkv, dim=1).contiguous() for x in (k, v))
        S = S.repeat_interleave(Hq // Hkv, dim=1).contiguous()
    ws = lla.prefill_segment_states(k, v, C, None)
    lla.prefill_state_scan(S, q.shape[2], C, ws)
    o = lla.prefill_chunks(q, k, v, S, C, workspace=ws)
    return o, S[:, ::Hq // Hkv]


@pytest.mark.parametrize("B,Hq,Hkv,T,dk,dv,C,dtype", ONE_LAUNCH_CASES)
def test_one_launch_fresh_prompt_equals_three_phases(dev, B, Hq, Hkv, T, dk, dv, C, dtype):
    """Gaussian inputs, so that any change in the order of the sums shows:
    the one-launch walk gives the bits of the segment pass, the scan and the
    walk, and agrees with the oracle."""
    print("one launch", B, Hq, Hkv, T, dk, dv, C, dtype, flush=True)
    scale = 1.0 if dtype == torch.float8_e4m3fn else dk ** -0.5
    q, k, v = workloads.gaussian(B, Hq, T, dk, dv, seed_base=T + dk, scale=scale, dtype=dtype, device=dev,
                                 Hkv=Hkv)
    G = lla.prefill_segment_chunks(B, Hq, T, dk, dv, C)
    c = (C + 1) // 2 if C > 64 else C
    assert 1 < -(-T // (G * c)) and (-(-T // (G * c)) - 1) * G <= 16  # the one-launch route
    S_a = torch.full((B, Hkv, dk, dv), float("nan"), device=dev)
    o_a = lla.prefill(q, k, v, S_a, chunk=C, zero_state=True)
    o_b, S_b = _three_phases(q, k, v, lla.state_init(B, Hkv, dk, dv, device=dev), C)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(S_a, S_b)
    O_ref, S_ref = oracle.grouped_recurrence(q.cpu(), k.cpu(), v.cpu(), nthreads=8)
    bar = 1e-5 if dtype == torch.float32 else TOL
    assert rel_err(np64(o_a), O_ref) <= bar and rel_err(np64(S_a), S_ref) <= bar


def _published_layout(B, Hkv, T, dk, dv, C):
    """Segments, value blocks and the floats of slots before the flags of the
    one-launch walk's published sums in the workspace: a slot of 64 x D
    floats per (b, key/value head, segment, value block), D the padded head
    dim, blocks of 64 value columns; then one 8-byte flag per slot."""
    G = lla.prefill_segment_chunks(B, Hkv, T, dk, dv, C)
    c = (C + 1) // 2 if C > 64 else C
    n_seg = -(-(-(-T // c)) // G)
    m = max(dk, dv)
    D = 32 if m <= 32 else (64 if m <= 64 else 128)
    n_vb = D // min(D, 64)
    return n_seg, n_vb, B * Hkv * n_seg * n_vb * 64 * D


@pytest.mark.parametrize("B,Hq,Hkv,T,dk,dv,C,dtype", [
    (4, 8, 8, 1024, 64, 64, 64, torch.bfloat16),
    (2, 4, 4, 900, 64, 64, 100, torch.float8_e4m3fn),
    (1, 8, 2, 600, 64, 64, 64, torch.bfloat16),
    (1, 4, 4, 700, 40, 56, 64, torch.bfloat16),
    # one launch only with published sums (more than 16 chunks before the last
    # segment); with the required workspace alone these run the three phases
    (1, 16, 16, 2048, 64, 64, 64, torch.bfloat16),
    (1, 32, 32, 2048, 32, 32, 32, torch.bfloat16),
    (2, 16, 16, 2048, 64, 64, 64, torch.float8_e4m3fn),
])
def test_one_launch_published_sums_equal_summing_in_place(dev, B, Hq, Hkv, T, dk, dv, C, dtype):
    """With room for the published sums, every segment but the last publishes
    its K^T V and the later walks read it; with only the required workspace
    every walk sums the earlier segments itself.  Same bits either way.  The
    flags of the published slots all hold the call's token afterwards (xor
    the id, 0-15, of the XCD that wrote the slot)."""
    print("published sums", B, Hq, Hkv, T, dk, dv, C, dtype, flush=True)
    scale = 1.0 if dtype == torch.float8_e4m3fn else dk ** -0.5
    q, k, v = workloads.gaussian(B, Hq, T, dk, dv, seed_base=3 * T + dv, scale=scale, dtype=dtype, device=dev,
                                 Hkv=Hkv)
    n_seg, n_vb, slot_floats = _published_layout(B, Hkv, T, dk, dv, C)
    required = B * Hkv * n_seg * dk * dv  # floats: one state per segment
    full = lla.prefill_gqa_workspace_size(B, Hq, Hkv, T, dk, dv, C) // 4
    assert full >= slot_floats + 2 * B * Hkv * n_seg * n_vb > required  # (this shape publishes)
    ws_small = torch.empty(required, dtype=torch.float32, device=dev)
    ws_full = torch.full((full,), float("nan"), dtype=torch.float32, device=dev)
    S_a = torch.full((B, Hkv, dk, dv), float("nan"), device=dev)
    S_b = torch.full((B, Hkv, dk, dv), float("nan"), device=dev)
    o_a = lla.prefill(q, k, v, S_a, chunk=C, zero_state=True, workspace=ws_small)
    o_b = lla.prefill(q, k, v, S_b, chunk=C, zero_state=True, workspace=ws_full)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(S_a, S_b)
    flags = ws_full[slot_floats:slot_floats + 2 * B * Hkv * n_seg * n_vb].view(torch.int64)
    published = flags.view(B * Hkv, n_seg, n_vb)[:, :-1].cpu()
    assert (published != 0).all() and ((published >> 4) == (published.flatten()[0] >> 4)).all()


@pytest.mark.parametrize("ticks", [0, 1, 50])
def test_one_launch_short_publish_wait_same_bits(dev, ticks):
    """With the readers' wait for published sums cut to almost nothing, most
    earlier segments are not yet published when a walk looks, so it sums them
    itself, interleaved with the ones it reads: the bits of the three phases
    regardless (the wait is set from the host; every wait still ends)."""
    print("publish wait", ticks, flush=True)
    try:
        lla.set_publish_wait_ticks(ticks)
        for B, H, T, d, C in ((4, 8, 1024, 64, 64), (1, 16, 2048, 64, 64)):
            q, k, v = workloads.gaussian(B, H, T, d, d, seed_base=200 + T, scale=d ** -0.5, device=dev)
            S_a = torch.empty((B, H, d, d), device=dev)
            o_a = lla.prefill(q, k, v, S_a, chunk=C, zero_state=True)
            o_b, S_b = _three_phases(q, k, v, lla.state_init(B, H, d, d, device=dev), C)
            torch.cuda.synchronize()
            assert torch.equal(o_a, o_b) and torch.equal(S_a, S_b), (ticks, B, H, T)
    finally:
        lla.set_publish_wait_ticks(2000)


def test_one_launch_workspace_reused_across_calls(dev):
    """Calls that reuse one workspace, each with new inputs: what an earlier
    call published (slots and flags) never enters a later call's result."""
    B, H, T, d, C = 4, 8, 1024, 64, 64
    ws = torch.empty(lla.prefill_workspace_size(B, H, T, d, d, C) // 4, dtype=torch.float32, device=dev)
    for r in range(4):
        print("reuse", r, flush=True)
        q, k, v = workloads.gaussian(B, H, T, d, d, seed_base=100 + r, scale=d ** -0.5, device=dev)
        S_a = torch.empty((B, H, d, d), device=dev)
        S_b = torch.empty((B, H, d, d), device=dev)
        o_a = lla.prefill(q, k, v, S_a, chunk=C, zero_state=True, workspace=ws)
        o_b, S_ref = _three_phases(q, k, v, lla.state_init(B, H, d, d, device=dev), C)
        torch.cuda.synchronize()
        assert torch.equal(o_a, o_b) and torch.equal(S_a, S_ref), r


def test_one_launch_verify_pass_equals_three_phases(dev):
    """A verify pass (S read, left as it was) from a gaussian state on the
    one-launch route: the outputs of the three phases, S untouched."""
    B, H, T, d, C = 2, 4, 300, 64, 64
    q, k, v = workloads.gaussian(B, H, T, d, d, seed_base=31, scale=d ** -0.5, device=dev)
    S0 = torch.randn((B, H, d, d), generator=torch.Generator().manual_seed(5)).to(dev)
    S_a = S0.clone()
    o_a = lla.prefill(q, k, v, S_a, chunk=C, keep_state=True)
    o_b, _ = _three_phases(q, k, v, S0.clone(), C)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(S_a, S0)
