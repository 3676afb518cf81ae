"""Prepared calls and HIP graphs.

* PreparedPrefill and PreparedDecode hold references to every buffer whose
  address they store, so dropping the caller's references and emptying
  torch's cache cannot free memory the library still reads.
* A fresh-prompt prefill and a decode step captured into a HIP graph (their
  kernels only: no allocation and no memset node is recorded) and replayed
  several times, with new inputs written eagerly and the stream synchronised
  between replays, give the bits of the same calls made eagerly -- plain,
  grouped, FP8 and gated.
"""
import gc

import pytest
import torch

import decode_lla_prefill_amd as lla
import oracle
import workloads
from gpu_util import TOL, need_gpu, np64, rel_err

pytestmark = pytest.mark.gpu


def test_prepared_calls_keep_their_buffers_alive():
    dev = need_gpu()

    def make():
        q, k, v = workloads.gaussian(1, 4, 700, 128, 128, seed_base=5, scale=128 ** -0.5, device=dev)
        S = lla.state_init(1, 4, 128, 128, device=dev)
        return lla.PreparedPrefill(q, k, v, S, 64), tuple(x.cpu() for x in (q, k, v))

    call, (qc, kc, vc) = make()  # the only references to q, k, v, S are inside `call`
    gc.collect()
    torch.cuda.empty_cache()
    junk = torch.full((32 << 20,), float("nan"), device=dev)  # would take freed blocks
    o = call(zero_state=True)
    torch.cuda.synchronize()
    O_ref, S_ref = oracle.recurrence(qc, kc, vc, nthreads=8)
    assert rel_err(np64(o), O_ref) <= TOL
    assert rel_err(np64(call.state), S_ref) <= TOL
    del junk


def _fill(tensors, seed):
    g = torch.Generator(device=tensors[0].device).manual_seed(seed)
    for t in tensors:
        t.copy_(torch.randn(t.shape, generator=g, device=t.device).mul_(t.shape[-1] ** -0.5))


def test_graph_replays_equal_eager_calls():
    dev = need_gpu()
    B, H, T, d, C = 1, 4, 700, 128, 64
    q, k, v = (torch.empty((B, H, T, d), dtype=torch.bfloat16, device=dev) for _ in range(3))
    qd, kd, vd = (torch.empty((B, H, d), dtype=torch.bfloat16, device=dev) for _ in range(3))
    S = lla.state_init(B, H, d, d, device=dev)
    pre = lla.PreparedPrefill(q, k, v, S, C)
    dec = lla.PreparedDecode(qd, kd, vd, S)
    _fill((q, k, v, qd, kd, vd), 0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up on a side stream, as capture does
        pre(zero_state=True)
        dec()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pre(zero_state=True)
        dec()
    torch.cuda.synchronize()
    for r in range(1, 5):
        print("graph replay", r, flush=True)
        _fill((q, k, v, qd, kd, vd), r)
        S_ref = torch.empty_like(S)
        o_ref = lla.prefill(q.clone(), k.clone(), v.clone(), S_ref, chunk=C, zero_state=True)
        od_ref = lla.decode_step(qd.clone(), kd.clone(), vd.clone(), S_ref)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(pre.out, o_ref), r
        assert torch.equal(dec.out, od_ref), r
        assert torch.equal(S, S_ref), r


def test_graph_replays_equal_eager_calls_one_launch():
    """A fresh prompt on the one-launch walk (d = 64, eleven segments): eager
    calls read the earlier segments' published sums, a captured call (whose
    replays could not tell one execution's flags from another's) sums them
    itself; the bits are the same."""
    dev = need_gpu()
    B, H, T, d, C = 1, 4, 700, 64, 64
    q, k, v = (torch.empty((B, H, T, d), dtype=torch.bfloat16, device=dev) for _ in range(3))
    S = lla.state_init(B, H, d, d, device=dev)
    pre = lla.PreparedPrefill(q, k, v, S, C)
    _fill((q, k, v), 0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pre(zero_state=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pre(zero_state=True)
    torch.cuda.synchronize()
    for r in range(1, 5):
        print("one-launch graph replay", r, flush=True)
        _fill((q, k, v), r)
        S_ref = torch.empty_like(S)
        o_ref = lla.prefill(q.clone(), k.clone(), v.clone(), S_ref, chunk=C, zero_state=True)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(pre.out, o_ref), r
        assert torch.equal(S, S_ref), r
        pre(zero_state=True)  # an eager call between the replays, on the same workspace
        torch.cuda.synchronize()
        assert torch.equal(pre.out, o_ref), r


@pytest.mark.parametrize("Hq,Hkv,dtype", [(8, 2, torch.bfloat16), (4, 4, torch.float8_e4m3fn),
                                           (8, 4, torch.float8_e4m3fn)])
def test_graph_replays_equal_eager_calls_grouped_and_fp8(Hq, Hkv, dtype):
    """The same capture with shared-state heads (the walks read their start
    states from the workspace the scan fills) and with FP8 inputs."""
    dev = need_gpu()
    B, T, d, C = 2, 700, 128, 64
    q = torch.empty((B, Hq, T, d), dtype=dtype, device=dev)
    k, v = (torch.empty((B, Hkv, T, d), dtype=dtype, device=dev) for _ in range(2))
    qd = torch.empty((B, Hq, d), dtype=dtype, device=dev)
    kd, vd = (torch.empty((B, Hkv, d), dtype=dtype, device=dev) for _ in range(2))
    S = lla.state_init(B, Hkv, d, d, device=dev)
    pre = lla.PreparedPrefill(q, k, v, S, C)
    dec = lla.PreparedDecode(qd, kd, vd, S)

    def fill(seed):
        g = torch.Generator(device=dev).manual_seed(seed)
        scale = 1.0 if dtype == torch.float8_e4m3fn else d ** -0.5
        for t in (q, k, v, qd, kd, vd):
            t.copy_(torch.randn(t.shape, generator=g, device=dev).mul_(scale).to(dtype))

    fill(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pre(zero_state=True)
        dec()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pre(zero_state=True)
        dec()
    torch.cuda.synchronize()
    for r in range(1, 5):
        print("graph replay", Hq, Hkv, dtype, r, flush=True)
        fill(r)
        S_ref = torch.empty_like(S)
        o_ref = lla.prefill(q.clone(), k.clone(), v.clone(), S_ref, chunk=C, zero_state=True)
        od_ref = lla.decode_step(qd.clone(), kd.clone(), vd.clone(), S_ref)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(pre.out, o_ref), r
        assert torch.equal(dec.out, od_ref), r
        assert torch.equal(S, S_ref), r


@pytest.mark.parametrize("T,d,C", [(700, 128, 64), (500, 64, 32)])
def test_graph_replays_equal_eager_calls_gated(T, d, C):
    """The gated prefill (segment pass, scan with the segment decays, walk)
    and the gated decode step captured and replayed with new inputs and
    gates: the bits of the eager calls."""
    dev = need_gpu()
    B, H = 2, 3
    q, k, v = (torch.empty((B, H, T, d), dtype=torch.bfloat16, device=dev) for _ in range(3))
    qd, kd, vd = (torch.empty((B, H, d), dtype=torch.bfloat16, device=dev) for _ in range(3))
    g, gd = torch.empty((B, H, T), device=dev), torch.empty((B, H), device=dev)
    S = lla.state_init(B, H, d, d, device=dev)
    pre = lla.PreparedGatedPrefill(q, k, v, g, S, C)
    dec = lla.PreparedGatedDecode(qd, kd, vd, gd, S)

    def fill(seed):
        _fill((q, k, v, qd, kd, vd), seed)
        gen = torch.Generator(device=dev).manual_seed(seed + 100)
        g.copy_(torch.rand(g.shape, generator=gen, device=dev) * 0.5 + 0.5)
        gd.copy_(torch.rand(gd.shape, generator=gen, device=dev) * 0.5 + 0.5)

    fill(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pre(zero_state=True)
        dec()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pre(zero_state=True)
        dec()
    torch.cuda.synchronize()
    for r in range(1, 5):
        print("gated graph replay", T, d, C, r, flush=True)
        fill(r)
        S_ref = torch.empty_like(S)
        o_ref = lla.prefill_gated(q.clone(), k.clone(), v.clone(), g.clone(), S_ref, C, zero_state=True)
        od_ref = lla.decode_step_gated(qd.clone(), kd.clone(), vd.clone(), gd.clone(), S_ref)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(pre.out, o_ref), r
        assert torch.equal(dec.out, od_ref), r
        assert torch.equal(S, S_ref), r


def test_graph_replays_equal_eager_calls_grouped_continuation():
    """A captured 16-token continuation of grouped states on the matrix
    cores (the persistent kernel: 320 key/value heads, so workgroups walk
    more than one), replayed from a reset state, equals the eager call."""
    dev = need_gpu()
    B, Hq, Hkv, T, d = 80, 16, 4, 16, 128
    q = torch.empty((B, Hq, T, d), dtype=torch.bfloat16, device=dev)
    k, v = (torch.empty((B, Hkv, T, d), dtype=torch.bfloat16, device=dev) for _ in range(2))
    S0 = torch.empty((B, Hkv, d, d), device=dev)
    S = torch.empty_like(S0)
    cont = lla.PreparedPrefill(q, k, v, S, 64)

    def fill(seed):
        g = torch.Generator(device=dev).manual_seed(seed)
        for t in (q, k, v):
            t.copy_(torch.randn(t.shape, generator=g, device=dev).mul_(d ** -0.5).to(torch.bfloat16))
        S0.copy_(torch.randn(S0.shape, generator=g, device=dev))
        S.copy_(S0)

    fill(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        cont()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cont()
    torch.cuda.synchronize()
    for r in range(1, 5):
        print("graph replay, grouped continuation", r, flush=True)
        fill(r)
        S_ref = S0.clone()
        o_ref = lla.prefill(q.clone(), k.clone(), v.clone(), S_ref, chunk=64)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(cont.out, o_ref), r
        assert torch.equal(S, S_ref), r
