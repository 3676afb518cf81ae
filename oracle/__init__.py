"""The CPU oracle for causal linear attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The product path (the HIP
library and its Python binding) never imports, links or runs anything here,
and this package imports nothing from the product.

Two oracles, both in float64 on the host:

* :func:`recurrence` -- the token-by-token recurrence of the slide deck
  "Chunking, causality, and parallel prefill", section "Naive recurrence":
  ``S_t = S_{t-1} + k_t v_t^T`` then ``o_t = S_t^T q_t``.  It runs in plain C
  (``lla_oracle.c``, built with ``-O2 -ffp-contract=off``) so the large
  configurations finish in seconds; this is the oracle every GPU result is
  compared against.
* :func:`chunked` -- the same deck's chunk form ("Split into chunks",
  "Incoming and outgoing state", "Worked case - full trace"): per chunk of C
  tokens ``M = tril(Q_c K_c^T)`` (diagonal kept), ``O_c = M V_c + Q_c S_in``,
  ``S_out = S_in + K_c^T V_c``.  Written step by step in numpy for small
  inputs; it exists to reproduce the deck's chunked trace, its C = 2 transfer
  exercise and its two bugs, and it is pinned against :func:`recurrence`.

Reading of the deck taken here (each also listed in the design notes):
the inter-chunk term is ``Q_c S_in`` (the deck's map prints ``K S_in``, but
its trace uses ``q_t^T S_4`` and has ``q_t = k_t``); the mask keeps the
diagonal; no feature map, normaliser, scale or decay; S is d_k x d_v with the
key dimension as rows; a last chunk shorter than C is the same arithmetic on
fewer rows; decode applies the rank-1 update, then reads the state.

:func:`grouped_recurrence` and :func:`grouped_decode_step` give shared-state
heads (several query heads reading one key/value head's state) by repeating
each key/value head over its group and calling the two functions above.

:func:`gated_recurrence` and :func:`gated_decode_step` give the gated
(decayed) state under the reading ``S_t = g_t S_{t-1} + k_t v_t^T`` with one
scalar gate per stream and token (the pages cite the gated chunkwise form but
state no gate); with ``g = 1`` they are the two functions above.

:func:`decode_e4m3` gives the values of FP8 (E4M3) inputs from the format's
definition, so FP8 tensors enter the oracle exactly as they do the GPU.

Parity of these functions is pinned in ``tests/test_oracle.py`` against values
the deck prints, closed forms and brute force.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lla_oracle.c")
_SO = os.path.join(_HERE, "liblla_oracle.so")
_lock = threading.Lock()
_lib = None

__all__ = ["build", "build_sanitized", "recurrence", "decode_step", "chunked", "causal_mask",
           "incoming_term", "grouped_recurrence", "grouped_decode_step", "decode_e4m3"]


def build(force: bool = True) -> str:
    """Compile ``lla_oracle.c`` into ``liblla_oracle.so`` with gcc."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                        "-pthread", "-o", tmp, _SRC], check=True)
        os.replace(tmp, _SO)
    return _SO


def build_sanitized(out_dir: str) -> str:
    """``lla_oracle.c`` built with the address and undefined-behaviour
    sanitizers (ROCm clang, so that one preloaded runtime serves it and the
    sanitized library; the first finding aborts) into out_dir."""
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, "liblla_oracle.so")
    subprocess.run(["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-ffp-contract=off", "-fPIC", "-shared",
                    "-pthread", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-o", out, _SRC], check=True)
    return out


def _load():
    global _lib
    with _lock:
        if _lib is None:
            # LLA_ORACLE_LIBRARY names another build of lla_oracle.c (the
            # sanitized copy of build_sanitized); by default the in-tree one
            path = os.environ.get("LLA_ORACLE_LIBRARY")
            if not path:
                path = _SO
                if not os.path.exists(_SO):
                    build(force=True)
            lib = ctypes.CDLL(path)
            dp = ctypes.POINTER(ctypes.c_double)
            i64 = ctypes.c_int64
            lib.lla_oracle_recurrence.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64,
                                                  i64, i64, dp, ctypes.c_int]
            lib.lla_oracle_recurrence.restype = ctypes.c_int
            lib.lla_oracle_decode_step.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64]
            lib.lla_oracle_decode_step.restype = ctypes.c_int
            lib.lla_oracle_gated_recurrence.argtypes = [dp, dp, dp, dp, dp, dp, i64, i64, i64, i64,
                                                        ctypes.c_int]
            lib.lla_oracle_gated_recurrence.restype = ctypes.c_int
            lib.lla_oracle_gated_decode_step.argtypes = [dp, dp, dp, dp, dp, dp, i64, i64, i64]
            lib.lla_oracle_gated_decode_step.restype = ctypes.c_int
            _lib = lib
    return _lib


def decode_e4m3(bits) -> np.ndarray:
    """float64 values of OCP FP8 E4M3 codes (uint8 array), from the format's
    definition: sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
    exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there are
    no infinities.  The blog "A 128 000 tokens, l'attention avale 85 % du
    calcul" says its attention figures are measured in FP8; E4M3 is the
    8-bit format taken for inputs here."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((b & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def _f64(a) -> np.ndarray:
    """Exact upcast to a C-contiguous float64 array (accepts numpy or torch;
    torch FP8 E4M3 tensors are decoded with :func:`decode_e4m3`)."""
    if hasattr(a, "detach"):  # torch tensor: upcast exactly on the host
        t = a.detach().cpu()
        if str(t.dtype) == "torch.float8_e4m3fn":
            import torch
            a = decode_e4m3(t.contiguous().view(torch.uint8).numpy())
        else:
            a = t.double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def recurrence(q, k, v, S0=None, ckpt_every: int = 0, nthreads: int = 1):
    """Token-by-token recurrence in float64.

    q, k: [..., T, dk]; v: [..., T, dv]; S0: [..., dk, dv] or None (zeros).
    Returns ``(O, S_T)`` -- or ``(O, S_T, ckpt)`` when ``ckpt_every > 0``,
    where ``ckpt[..., c, :, :]`` is the state after ``(c+1)*ckpt_every``
    tokens.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    lead = q.shape[:-2]
    T, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:-1] != q.shape[:-1]:
        raise ValueError("shape mismatch: q %s k %s v %s" % (q.shape, k.shape, v.shape))
    BH = int(np.prod(lead)) if lead else 1
    S = np.zeros(lead + (dk, dv)) if S0 is None else _f64(S0).copy()
    if S.shape != lead + (dk, dv):
        raise ValueError("S0 shape %s, expected %s" % (S.shape, lead + (dk, dv)))
    O = np.zeros(lead + (T, dv))
    n_ck = T // ckpt_every if ckpt_every > 0 else 0
    ck = np.zeros(lead + (n_ck, dk, dv)) if ckpt_every > 0 else None
    rc = _load().lla_oracle_recurrence(
        _ptr(q), _ptr(k), _ptr(v), _ptr(S), _ptr(O), BH, T, dk, dv,
        int(ckpt_every), _ptr(ck) if ck is not None and ck.size else None,
        int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle recurrence rejected its arguments")
    return (O, S, ck) if ckpt_every > 0 else (O, S)


def decode_step(q, k, v, S):
    """One decode step in float64: ``S += k v^T``, then ``o = S^T q``.

    q, k: [..., dk]; v: [..., dv]; S: [..., dk, dv].  Returns ``(o, S_new)``
    without modifying the caller's S.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    S = _f64(S).copy()
    lead = q.shape[:-1]
    dk, dv = q.shape[-1], v.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    o = np.zeros(lead + (dv,))
    rc = _load().lla_oracle_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(S), _ptr(o),
                                        BH, dk, dv)
    if rc != 0:
        raise RuntimeError("oracle decode step rejected its arguments")
    return o, S


# --- gated (decayed) state, float64 ------------------------------------------
#
# Slide deck "Chunking, causality, and parallel prefill", section "Boundary,
# evidence, and sources": it cites the chunkwise form of gated linear
# attention but states no gate.  Reading taken (a reading, not the pages'
# formula): one scalar gate g_t per (batch, head) stream and token, applied
# to the previous state before the token's update,
#     S_t = g_t S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t.
# With g = 1 it is the recurrence above.


def gated_recurrence(q, k, v, gate, S0=None, nthreads: int = 1):
    """Token-by-token gated recurrence in float64.

    q, k: [..., T, dk]; v: [..., T, dv]; gate: [..., T]; S0: [..., dk, dv] or
    None (zeros).  Returns ``(O, S_T)``."""
    q, k, v, gate = _f64(q), _f64(k), _f64(v), _f64(gate)
    lead = q.shape[:-2]
    T, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:-1] != q.shape[:-1] or gate.shape != q.shape[:-1]:
        raise ValueError("shape mismatch: q %s k %s v %s gate %s" % (q.shape, k.shape, v.shape, gate.shape))
    BH = int(np.prod(lead)) if lead else 1
    S = np.zeros(lead + (dk, dv)) if S0 is None else _f64(S0).copy()
    if S.shape != lead + (dk, dv):
        raise ValueError("S0 shape %s, expected %s" % (S.shape, lead + (dk, dv)))
    O = np.zeros(lead + (T, dv))
    rc = _load().lla_oracle_gated_recurrence(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(S), _ptr(O),
                                             BH, T, dk, dv, int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle gated recurrence rejected its arguments")
    return O, S


def gated_decode_step(q, k, v, gate, S):
    """One gated decode step in float64: ``S = g S + k v^T``, then
    ``o = S^T q``.  q, k: [..., dk]; v: [..., dv]; gate: [...]; S: [..., dk,
    dv].  Returns ``(o, S_new)`` without modifying the caller's S."""
    q, k, v, gate = _f64(q), _f64(k), _f64(v), _f64(gate)
    S = _f64(S).copy()
    lead = q.shape[:-1]
    dk, dv = q.shape[-1], v.shape[-1]
    if gate.shape != lead:
        raise ValueError("gate shape %s, expected %s" % (gate.shape, lead))
    BH = int(np.prod(lead)) if lead else 1
    o = np.zeros(lead + (dv,))
    rc = _load().lla_oracle_gated_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(S), _ptr(o),
                                              BH, dk, dv)
    if rc != 0:
        raise RuntimeError("oracle gated decode step rejected its arguments")
    return o, S


# --- shared-state heads (grouped query heads), float64 ---------------------
#
# Blog "A 128 000 tokens, l'attention avale 85 % du calcul", section "Partager
# les tetes pour alleger la memoire": the group size is how many query heads
# share one key/value head (1: multi-head, Hq: one key/value head for all).
# In linear attention the state is built from keys and values only, so a
# key/value head carries one state and each query head of its group reads it.
# Reading taken: query head h uses key/value head h // G with G = Hq / Hkv
# (consecutive query heads form a group).


def _group(Hq: int, Hkv: int) -> int:
    if Hkv < 1 or Hq < Hkv or Hq % Hkv:
        raise ValueError("Hq = %d query heads cannot be grouped on Hkv = %d heads" % (Hq, Hkv))
    return Hq // Hkv


def grouped_recurrence(q, k, v, S0=None, nthreads: int = 1):
    """Token-by-token recurrence with shared-state heads, float64.

    q: [B, Hq, T, dk]; k: [B, Hkv, T, dk]; v: [B, Hkv, T, dv];
    S0: [B, Hkv, dk, dv] or None.  Every key/value head (and its state) is
    repeated for the G query heads of its group, then :func:`recurrence` runs
    on Hq independent heads.  Returns ``(O [B,Hq,T,dv], S_T [B,Hkv,dk,dv])``;
    the G copies of one state take the same arithmetic, so they are equal and
    the first is returned.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, T, d]")
    G = _group(q.shape[1], k.shape[1])
    S0e = None if S0 is None else np.repeat(_f64(S0), G, axis=1)
    O, S = recurrence(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), S0e, nthreads=nthreads)
    return O, np.ascontiguousarray(S[:, ::G])


def grouped_decode_step(q, k, v, S):
    """One decode step with shared-state heads, float64: q [B,Hq,dk],
    k [B,Hkv,dk], v [B,Hkv,dv], S [B,Hkv,dk,dv].  ``S += k v^T`` once per
    key/value head, then every query head h reads ``o_h = S_{h//G}^T q_h``.
    Returns ``(o [B,Hq,dv], S_new)`` without modifying the caller's S."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3:
        raise ValueError("q, k, v must be [B, H, d]")
    G = _group(q.shape[1], k.shape[1])
    o, S_new = decode_step(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1),
                           np.repeat(_f64(S), G, axis=1))
    return o, np.ascontiguousarray(S_new[:, ::G])


def gated_grouped_recurrence(q, k, v, gate, S0=None, nthreads: int = 1):
    """Gated recurrence with shared-state heads, float64: each key/value
    head's state S_t = g_t S_{t-1} + k_t v_t^T (gate [B, Hkv, T], one per
    state and token) is read by the G query heads of its group, o_t = S_t^T
    q_t.  Every key/value head, its gates and its state are repeated for the
    group, then :func:`gated_recurrence` runs on Hq independent heads.
    Returns ``(O [B,Hq,T,dv], S_T [B,Hkv,dk,dv])`` (the copies are equal; the
    first is returned)."""
    q, k, v, gate = _f64(q), _f64(k), _f64(v), _f64(gate)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4 or gate.ndim != 3:
        raise ValueError("q, k, v must be [B, H, T, d] and gate [B, Hkv, T]")
    G = _group(q.shape[1], k.shape[1])
    S0e = None if S0 is None else np.repeat(_f64(S0), G, axis=1)
    O, S = gated_recurrence(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), np.repeat(gate, G, axis=1),
                            S0e, nthreads=nthreads)
    return O, np.ascontiguousarray(S[:, ::G])


def gated_grouped_decode_step(q, k, v, gate, S):
    """One gated decode step with shared-state heads, float64: q [B,Hq,dk],
    k [B,Hkv,dk], v [B,Hkv,dv], gate [B,Hkv], S [B,Hkv,dk,dv].  ``S = g S +
    k v^T`` once per key/value head, then every query head h reads ``o_h =
    S_{h//G}^T q_h``.  Returns ``(o [B,Hq,dv], S_new)``."""
    q, k, v, gate = _f64(q), _f64(k), _f64(v), _f64(gate)
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3 or gate.ndim != 2:
        raise ValueError("q, k, v must be [B, H, d] and gate [B, Hkv]")
    G = _group(q.shape[1], k.shape[1])
    o, S_new = gated_decode_step(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), np.repeat(gate, G, axis=1),
                                 np.repeat(_f64(S), G, axis=1))
    return o, np.ascontiguousarray(S_new[:, ::G])


# --- the deck's chunk form, step by step (numpy, float64, small inputs) -----

def causal_mask(A: np.ndarray) -> np.ndarray:
    """Lower triangle of a chunk's score matrix, diagonal kept.

    Deck section "Causal triangle": row i (reading token) may read column j
    only when j <= i; cells above the diagonal are forbidden, cells below it
    keep their computed value (zero or not).
    """
    return np.tril(A)


def incoming_term(Qc: np.ndarray, S_in: np.ndarray) -> np.ndarray:
    """What a chunk reads from the past through the state: row t is q_t^T S_in.

    Deck section "Incoming and outgoing state" (o_5 = q_5^T S_4 + local term).
    """
    return Qc @ S_in


def chunked(q, k, v, C: int, S0=None):
    """The chunk form for one stream: q, k [T, dk], v [T, dv], S0 [dk, dv].

    Walks the chunks in order; for each chunk of C tokens (the last one may be
    shorter): the masked score triangle, the output ``M V + Q S_in``, then the
    outgoing state ``S_in + K^T V``.  Returns ``(O, S_T, handoffs, masks)``
    where ``handoffs`` lists the state emitted by every chunk but the last
    (the states handed from one chunk to the next) and ``masks`` the masked
    triangles.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, dk = q.shape
    dv = v.shape[1]
    if C < 1:
        raise ValueError("chunk size must be >= 1")
    S = np.zeros((dk, dv)) if S0 is None else _f64(S0).copy()
    O = np.zeros((T, dv))
    handoffs, masks = [], []
    for start in range(0, T, C):
        Qc, Kc, Vc = q[start:start + C], k[start:start + C], v[start:start + C]
        M = causal_mask(Qc @ Kc.T)
        O[start:start + C] = M @ Vc + incoming_term(Qc, S)
        S = S + Kc.T @ Vc
        masks.append(M)
        if start + C < T:
            handoffs.append(S.copy())
    return O, S, handoffs, masks
