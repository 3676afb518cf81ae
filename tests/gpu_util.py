"""Helpers shared by the GPU tests (test infrastructure)."""
import numpy as np
import pytest
import torch

TOL = 2e-3  # max|err| / max|ref| for bf16 inputs with fp32 accumulation


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_lla_prefill_amd as lla
    lla.library()  # raises if the HIP library is not built: no fallback
    return torch.device("cuda:0")


def np64(t):
    return t.detach().cpu().double().numpy()


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (denom if denom > 0 else 1.0))


def gpu_prefill(q, k, v, C, S0=None, dev="cuda:0"):
    import decode_lla_prefill_amd as lla
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if S0 is None:
        S = lla.state_init(B, H, dk, dv, device=dev)
    else:
        S = S0.to(dev, torch.float32).contiguous().clone()
    o = lla.prefill(q.to(dev).contiguous(), k.to(dev).contiguous(), v.to(dev).contiguous(), S, chunk=C)
    torch.cuda.synchronize()
    return o, S
