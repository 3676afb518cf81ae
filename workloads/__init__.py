"""Seeded synthetic inputs for causal linear attention.

This module only draws and shapes inputs; it holds none of the method's
arithmetic.  Both sides use it: the GPU path (tests, benchmark, smoke check)
and the oracle (which receives the very same tensors upcast to float64).

The workloads follow the shapes of the slide deck "Chunking, causality, and
parallel prefill": its worked case (8 tokens, d = 2, chunk C = 4, q_t = k_t,
"Worked case - full trace"), and larger prefill/decode shapes in the same
notation (B sequences, H heads, T tokens, head dims d_k = d_v, chunk C).

Recipe (also stated in the design notes):
* toy variant 0 is the deck's trace; variants 1..100 draw Q, K, V uniformly
  from {0, 1} (fp32) with ``torch.manual_seed(variant)``;
* gaussian inputs draw Q, K, V ~ N(0, 1) * scale in fp32 with one CPU or
  device generator per tensor (seed = seed_base + {0: q, 1: k, 2: v}),
  optionally L2-normalise every key row in fp32, then round to the storage
  dtype (round-to-nearest-even for bf16);
* integer inputs draw uniformly from {lo..hi}; they are exact in bf16, so
  every product and partial sum of the method is an exact integer.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

# The deck's worked case ("Worked case - full trace"): 8 tokens, d = 2,
# q_t = k_t, keys alternate [1,0],[0,1]; values as printed for chunks 1 and 2.
TRACE_K = [[1, 0], [0, 1], [1, 0], [0, 1], [1, 0], [0, 1], [1, 0], [0, 1]]
TRACE_V = [[2, 3], [5, 1], [1, 1], [0, 4], [0, 1], [2, 2], [1, 0], [0, 0]]


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    H: int
    T: int
    C: int
    dk: int
    dv: int
    dtype: torch.dtype
    scale: float = 1.0
    l2norm_k: bool = False
    seed_base: int = 0
    decode_steps: int = 0
    Hkv: int = 0  # key/value heads (0: one per query head)
    note: str = field(default="", compare=False)

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H


# The deck's toy; three prefill shapes; decode after a T=4096 prefill; the
# T=8192 prefill and the decode batch with four query heads per key/value head
# (shared-state heads, as in grouped-query attention) and with FP8 (E4M3)
# inputs.  Each workload draws from seeds seed_base + {0, 1, 2} (q, k, v),
# + {3, 4, 5} (per-step decode q, k, v) and + 6 (a random state).
CONFIGS = {
    "toy": Config("toy", 1, 1, 8, 4, 2, 2, torch.float32, seed_base=10,
                 note="variant 0 = the deck's trace, variants 1..100 uniform {0,1}"),
    "prefill_B4_T1024": Config("prefill_B4_H8_T1024_C64_d64", 4, 8, 1024, 64, 64, 64, torch.bfloat16,
                 scale=64 ** -0.5, seed_base=20),
    "prefill_T8192": Config("prefill_B1_H16_T8192_C64_d128", 1, 16, 8192, 64, 128, 128,
                 torch.bfloat16, scale=128 ** -0.5, l2norm_k=True, seed_base=30),
    "prefill_T131072": Config("prefill_B1_H32_T131072_C128_d128", 1, 32, 131072, 128, 128, 128,
                 torch.bfloat16, scale=128 ** -0.5, seed_base=40),
    "decode_B256": Config("decode_B256_H32_d128_after_T4096", 256, 32, 4096, 64, 128, 128,
                 torch.bfloat16, scale=128 ** -0.5, seed_base=50, decode_steps=512),
    "prefill_T8192_gqa": Config("prefill_B1_Hq16_Hkv4_T8192_C64_d128", 1, 16, 8192, 64, 128, 128,
                 torch.bfloat16, scale=128 ** -0.5, l2norm_k=True, seed_base=60, Hkv=4),
    "decode_B256_gqa": Config("decode_B256_Hq32_Hkv8_d128", 256, 32, 1, 64, 128, 128,
                 torch.bfloat16, scale=128 ** -0.5, seed_base=70, decode_steps=512, Hkv=8,
                 note="state drawn N(0,1) (seed seed_base + 6), not from a prefill"),
    "prefill_T8192_fp8": Config("prefill_B1_H16_T8192_C64_d128_fp8", 1, 16, 8192, 64, 128, 128,
                 torch.float8_e4m3fn, scale=1.0, seed_base=80,
                 note="N(0,1) rounded to FP8 E4M3 (unit scale uses the format's range)"),
    "decode_B256_fp8": Config("decode_B256_H32_d128_fp8", 256, 32, 1, 64, 128, 128,
                 torch.float8_e4m3fn, scale=1.0, seed_base=90, decode_steps=512,
                 note="state drawn N(0,1) (seed seed_base + 6), not from a prefill"),
}


def toy(variant: int):
    """Toy inputs [1, 1, 8, 2] fp32: variant 0 = the deck's trace."""
    if variant == 0:
        k = torch.tensor(TRACE_K, dtype=torch.float32).view(1, 1, 8, 2)
        v = torch.tensor(TRACE_V, dtype=torch.float32).view(1, 1, 8, 2)
        return k.clone(), k.clone(), v
    g = torch.Generator().manual_seed(int(variant))
    q = torch.randint(0, 2, (1, 1, 8, 2), generator=g).float()
    k = torch.randint(0, 2, (1, 1, 8, 2), generator=g).float()
    v = torch.randint(0, 2, (1, 1, 8, 2), generator=g).float()
    return q, k, v


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def gaussian(B, H, T, dk, dv, seed_base, scale, dtype=torch.bfloat16,
             l2norm_k=False, device="cpu", Hkv=None):
    """Q [B,H,T,dk], K [B,Hkv,T,dk] and V [B,Hkv,T,dv] (Hkv defaults to H):
    N(0,1)*scale in fp32, then cast.

    Generated in slices along B so that large device workloads never hold
    more than one slice of fp32 temporaries.
    """
    out = []
    Hkv = Hkv or H
    for which, d, heads in ((0, dk, H), (1, dk, Hkv), (2, dv, Hkv)):
        g = _gen(device, seed_base + which)
        t = torch.empty((B, heads, T, d), dtype=dtype, device=device)
        for b in range(B):
            x = torch.randn((heads, T, d), generator=g, dtype=torch.float32, device=device)
            x.mul_(scale)
            if which == 1 and l2norm_k:
                x = x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)
            t[b].copy_(x)
            del x
        out.append(t)
    return tuple(out)


def integers(B, H, T, dk, dv, seed, lo=-1, hi=1, dtype=torch.bfloat16, device="cpu", Hkv=None,
             v_range=None):
    """Q [B,H,T,dk], K, V [B,Hkv,T,*] (Hkv defaults to H) with integer values
    uniform in [lo, hi] (V in ``v_range`` = (lo, hi) when given), stored in
    ``dtype``."""
    g = _gen("cpu", seed)
    Hkv = Hkv or H
    v_lo, v_hi = v_range if v_range is not None else (lo, hi)
    q = torch.randint(lo, hi + 1, (B, H, T, dk), generator=g).to(dtype)
    k = torch.randint(lo, hi + 1, (B, Hkv, T, dk), generator=g).to(dtype)
    v = torch.randint(v_lo, v_hi + 1, (B, Hkv, T, dv), generator=g).to(dtype)
    return q.to(device), k.to(device), v.to(device)


def config_inputs(cfg: Config, device="cpu", T=None, B=None):
    """The prefill inputs of a config (optionally truncated in T or B)."""
    return gaussian(B or cfg.B, cfg.H, T or cfg.T, cfg.dk, cfg.dv, cfg.seed_base,
                    cfg.scale, cfg.dtype, cfg.l2norm_k, device, Hkv=cfg.kv_heads)


def decode_inputs(cfg: Config, steps: int, device="cpu", B=None):
    """Per-step decode inputs q [steps,B,H,dk], k [steps,B,Hkv,dk] and
    v [steps,B,Hkv,dv] (bf16).

    Drawn like :func:`gaussian` with seeds seed_base + {3, 4, 5}.
    """
    B = B or cfg.B
    out = []
    for which, d, heads in ((3, cfg.dk, cfg.H), (4, cfg.dk, cfg.kv_heads), (5, cfg.dv, cfg.kv_heads)):
        g = _gen(device, cfg.seed_base + which)
        t = torch.empty((steps, B, heads, d), dtype=cfg.dtype, device=device)
        for s in range(steps):
            x = torch.randn((B, heads, d), generator=g, dtype=torch.float32, device=device)
            t[s].copy_(x.mul_(cfg.scale))
        out.append(t)
    return tuple(out)


def gates(B, H, T, seed, lo=0.9, hi=1.0, device="cpu"):
    """Decay gates [B,H,T] fp32, uniform in [lo, hi] (seeded).  The default
    range is that of forget gates close to one, which keep a long memory;
    lo = 0 reaches gates that forget everything."""
    g = _gen(device, seed)
    return torch.rand((B, H, T), generator=g, dtype=torch.float32, device=device) * (hi - lo) + lo


def random_state(cfg: Config, device="cpu", B=None):
    """A state S [B,Hkv,dk,dv] fp32 drawn N(0,1) with seed seed_base + 6."""
    g = _gen(device, cfg.seed_base + 6)
    return torch.randn((B or cfg.B, cfg.kv_heads, cfg.dk, cfg.dv), generator=g,
                       dtype=torch.float32, device=device)
