"""Where the prefill rounds.  Inside a chunk the masked scores P = tril(Q K^T)
enter the matrix-core product P V in bf16 as a high + low pair (P to about 16
bits: an error of at most 2^-16 |P|), at every chunk size.  Everything else
accumulates in fp32, and the state enters Q S as a bf16 high + low pair.  So
for a prompt of one chunk from a zero state, every output element is within
that factor times (|P| |V|) of the exact result, plus fp32 slack, whatever the
inputs.

With one bf16 value (2^-8 |P|) instead of the pair, an output dominated by one
large score term (few tokens, large q . k) could pass max|err|/max|ref| = 2e-3:
the first case below measured 2.09e-3 at C = 128 that way (unit-scale FP8
inputs, dk = 32, 100 tokens).  With the pair every case stays far inside the
bar."""
import numpy as np
import pytest
import torch

import decode_lla_prefill_amd as lla
import oracle
import workloads
from gpu_util import need_gpu, np64

pytestmark = pytest.mark.gpu
FP8 = torch.float8_e4m3fn


@pytest.mark.parametrize("B,Hq,Hkv,T,dk,dv,C,dtype,scale", [
    (2, 8, 2, 100, 32, 128, 128, FP8, 1.0),
    (1, 2, 2, 120, 128, 128, 128, torch.bfloat16, 1.0),
    (2, 8, 2, 64, 32, 128, 64, FP8, 1.0),
    (2, 8, 2, 9, 32, 128, 16, FP8, 1.0),
    (1, 4, 4, 64, 128, 128, 64, torch.bfloat16, 1.0),
    (2, 2, 2, 37, 64, 64, 64, torch.bfloat16, 0.125),
    (1, 3, 3, 48, 40, 72, 48, torch.bfloat16, 1.0),
])
def test_one_chunk_error_is_bounded_by_the_rounding_of_p(B, Hq, Hkv, T, dk, dv, C, dtype, scale):
    dev = need_gpu()
    assert T <= C
    q, k, v = workloads.gaussian(B, Hq, T, dk, dv, seed_base=T + dk, scale=scale, dtype=dtype, Hkv=Hkv)
    S = torch.empty((B, Hkv, dk, dv), device=dev)
    o = lla.prefill(q.to(dev), k.to(dev), v.to(dev), S, chunk=C, zero_state=True)
    torch.cuda.synchronize()
    O_ref, _ = oracle.grouped_recurrence(q, k, v, np.zeros((B, Hkv, dk, dv)), nthreads=8)
    G = Hq // Hkv
    f64 = lambda t: oracle.decode_e4m3(t.view(torch.uint8).numpy()) if dtype == FP8 else t.double().numpy()
    q64 = f64(q)
    k64 = np.repeat(f64(k), G, axis=1)
    v64 = np.abs(np.repeat(f64(v), G, axis=1))
    kt = k64.transpose(0, 1, 3, 2)
    absP = np.abs(np.tril(q64 @ kt))          # |P| of the one chunk
    absQK = np.tril(np.abs(q64) @ np.abs(kt))  # sum_i |q_i k_i| (fp32 slack of the scores)
    # rounding of P to a bf16 pair (2^-16 |P|), fp32 sums over T terms (P V) and dk
    # terms (Q K^T), each n * 2^-24 of its absolute sum
    u = 2.0 ** -24
    p_round = 2.0 ** -16  # P as a bf16 hi + lo pair
    allowed = ((p_round + (T + 4) * u) * (absP @ v64) * (1 + 2.0 ** -8)
               + 2 * (dk + 4) * u * (absQK @ v64))
    err = np.abs(np.asarray(np64(o)) - O_ref)
    assert (err <= allowed).all(), float((err / np.maximum(allowed, 1e-300)).max())
    # the split keeps even dominated outputs far inside the bar
    assert err.max() / np.abs(O_ref).max() <= 1e-4
