"""Concurrent callers.  The library holds no mutable global state and may be
called from several host threads on different streams: two host threads,
each with its own HIP stream and buffers, run fresh-prompt prefills and a
decode step after each at the same time (different shapes, so different
kernels run side by side).  Every result equals the same calls made one
after another on one stream, bit for bit."""
import threading

import pytest
import torch

import decode_lla_prefill_amd as lla
import workloads
from gpu_util import need_gpu

pytestmark = pytest.mark.gpu

REPS = 6


def _case(seed, B, Hq, Hkv, T, d, C, dev):
    q, k, v = workloads.gaussian(B, Hq, T, d, d, seed_base=seed, scale=d ** -0.5, device=dev, Hkv=Hkv)
    qd, kd, vd = (x[:, :, 0].contiguous() for x in
                  workloads.gaussian(B, Hq, 1, d, d, seed_base=seed + 7, scale=d ** -0.5, device=dev, Hkv=Hkv))
    return dict(q=q, k=k, v=v, qd=qd, kd=kd, vd=vd, C=C, S_shape=(B, Hkv, d, d))


def _run(case, dev):
    """REPS fresh prefills, each followed by one decode step; the outputs."""
    out = []
    S = torch.empty(case["S_shape"], device=dev)
    for _ in range(REPS):
        o = lla.prefill(case["q"], case["k"], case["v"], S, chunk=case["C"], zero_state=True)
        od = lla.decode_step(case["qd"], case["kd"], case["vd"], S)
        out.append((o, od, S.clone()))
    return out


def test_two_threads_on_two_streams_match_sequential_calls():
    dev = need_gpu()
    cases = [_case(11, 1, 8, 8, 3000, 128, 64, dev),   # eight-wave walk, several segments
             _case(23, 2, 8, 2, 777, 128, 32, dev),    # shared-state heads
             ]
    expected = [_run(c, dev) for c in cases]
    torch.cuda.synchronize()

    results, errors = [None] * len(cases), []
    barrier = threading.Barrier(len(cases))

    def worker(i):
        try:
            torch.cuda.set_device(dev)
            stream = torch.cuda.Stream(device=dev)
            with torch.cuda.stream(stream):
                barrier.wait()
                results[i] = _run(cases[i], dev)
            stream.synchronize()
        except Exception as e:  # surfaced in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a caller thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i in range(len(cases)):
        for r in range(REPS):
            for got, ref in zip(results[i][r], expected[i][r]):
                assert torch.equal(got, ref), (i, r)
