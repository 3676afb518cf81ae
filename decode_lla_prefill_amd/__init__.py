"""decode_lla_prefill_amd -- causal linear attention on AMD Instinct MI355X.

Chunkwise-parallel prefill and the matching decode step of the recurrence
``S_t = S_{t-1} + k_t v_t^T``, ``o_t = S_t^T q_t`` (slide deck "Chunking,
causality, and parallel prefill"), computed by the HIP kernels of
``liblla.so`` (gfx950).  This module only marshals arguments: it checks
tensor shapes/dtypes/devices, allocates outputs and the workspace with
PyTorch, and passes raw device pointers plus the current HIP stream to the
C ABI declared in ``include/lla.h``.  There is no fallback: without the built
library every call raises.

Layouts (all contiguous): q, k [B, H, T, dk]; v [B, H, T, dv] (bf16 or fp32);
o [B, H, T, dv] fp32; state [B, H, dk, dv] fp32 (rows = key dimension).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "LlaError", "library", "library_path", "state_init", "prefill", "decode_step",
    "prefill_workspace_size", "prefill_gqa_workspace_size", "prefill_segment_chunks",
    "prefill_segment_states",
    "prefill_state_scan", "prefill_chunks", "prefill_noalloc", "state_commit", "PreparedPrefill",
    "PreparedDecode", "prefill_gated_workspace_size", "prefill_gated", "decode_step_gated",
    "state_commit_gated", "PreparedGatedPrefill", "PreparedGatedDecode",
    "set_publish_wait_ticks", "EXPORTS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# LLA_LIBRARY names another build of the same library (the host-sanitized
# copy the CPU tests use); by default the in-tree liblla.so.
library_path = os.environ.get("LLA_LIBRARY") or os.path.join(_HERE, "liblla.so")

# Every symbol include/lla.h declares.
EXPORTS = ("lla_status_string", "lla_last_device_error", "lla_state_init",
           "lla_prefill_segment_chunks", "lla_prefill_workspace_size", "lla_prefill",
           "lla_prefill_segment_states", "lla_prefill_state_scan", "lla_prefill_chunks",
           "lla_decode_step", "lla_prefill_gqa_workspace_size", "lla_prefill_gqa",
           "lla_decode_step_gqa", "lla_prefill_ex", "lla_prefill_noalloc", "lla_state_commit",
           "lla_prefill_gated_workspace_size", "lla_prefill_gated", "lla_decode_step_gated",
           "lla_state_commit_gated", "lla_prefill_gated_gqa_workspace_size", "lla_prefill_gated_gqa",
           "lla_decode_step_gated_gqa", "lla_set_publish_wait_ticks")
PREFILL_ZERO_STATE = 1  # lla_prefill_ex: start from S_0 = 0 without reading S
PREFILL_KEEP_STATE = 2  # lla_prefill_ex: read S, do not write it (verify pass of draft tokens)

_BF16, _F32, _FP8 = 0, 1, 2
_lib = None


class LlaError(RuntimeError):
    """A non-OK lla_status from the library."""

    def __init__(self, status: int, what: str):
        self.status = status
        msg = _lib.lla_status_string(status).decode() if _lib is not None else str(status)
        if status == 8 and _lib is not None:  # LLA_ERR_DEVICE
            msg += " (hipError %d)" % _lib.lla_last_device_error()
        super().__init__("%s: %s (status %d)" % (what, msg, status))


def library():
    """Load liblla.so (built by ``python -m decode_lla_prefill_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise ImportError("liblla.so not built: run `python -m decode_lla_prefill_amd.build` "
                              "(looked for %s)" % library_path)
        lib = ctypes.CDLL(library_path)
        vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        st, ci = ctypes.c_int, ctypes.c_int
        lib.lla_status_string.argtypes = [st]
        lib.lla_status_string.restype = ctypes.c_char_p
        lib.lla_last_device_error.argtypes = []
        lib.lla_last_device_error.restype = ci
        lib.lla_state_init.argtypes = [vp, i64, i64, i64, i64, vp]
        lib.lla_state_init.restype = st
        lib.lla_prefill_segment_chunks.argtypes = [i64] * 6
        lib.lla_prefill_segment_chunks.restype = i64
        lib.lla_prefill_workspace_size.argtypes = [i64] * 6
        lib.lla_prefill_workspace_size.restype = sz
        lib.lla_prefill.argtypes = [vp, vp, vp, ci, i64, i64, i64, i64, i64, i64, vp, vp, vp, sz, vp]
        lib.lla_prefill.restype = st
        lib.lla_prefill_chunks.argtypes = lib.lla_prefill.argtypes
        lib.lla_prefill_chunks.restype = st
        lib.lla_prefill_segment_states.argtypes = [vp, vp, ci, i64, i64, i64, i64, i64, i64, vp, sz, vp]
        lib.lla_prefill_segment_states.restype = st
        lib.lla_prefill_state_scan.argtypes = [vp, i64, i64, i64, i64, i64, i64, vp, sz, vp]
        lib.lla_prefill_state_scan.restype = st
        lib.lla_decode_step.argtypes = [vp, vp, vp, ci, i64, i64, i64, i64, vp, vp, vp]
        lib.lla_decode_step.restype = st
        lib.lla_prefill_gqa_workspace_size.argtypes = [i64] * 7
        lib.lla_prefill_gqa_workspace_size.restype = sz
        lib.lla_prefill_gqa.argtypes = [vp, vp, vp, ci, i64, i64, i64, i64, i64, i64, i64, vp, vp, vp,
                                        sz, vp]
        lib.lla_prefill_gqa.restype = st
        lib.lla_decode_step_gqa.argtypes = [vp, vp, vp, ci, i64, i64, i64, i64, i64, vp, vp, vp]
        lib.lla_decode_step_gqa.restype = st
        lib.lla_prefill_ex.argtypes = [vp, vp, vp, ci, i64, i64, i64, i64, i64, i64, i64,
                                       ctypes.c_uint, vp, vp, vp, sz, vp]
        lib.lla_prefill_ex.restype = st
        lib.lla_set_publish_wait_ticks.argtypes = [i64]
        lib.lla_set_publish_wait_ticks.restype = st
        lib.lla_prefill_noalloc.argtypes = [vp, vp, vp, ci, i64, i64, i64, i64, i64, i64, i64,
                                            ctypes.c_uint, vp, vp, vp]
        lib.lla_prefill_noalloc.restype = st
        lib.lla_state_commit.argtypes = [vp, vp, ci, i64, i64, i64, i64, i64, vp, vp, vp]
        lib.lla_state_commit.restype = st
        lib.lla_prefill_gated_workspace_size.argtypes = [i64] * 6
        lib.lla_prefill_gated_workspace_size.restype = sz
        lib.lla_prefill_gated.argtypes = [vp, vp, vp, vp, ci, i64, i64, i64, i64, i64, i64, ctypes.c_uint,
                                          vp, vp, vp, sz, vp]
        lib.lla_prefill_gated.restype = st
        lib.lla_decode_step_gated.argtypes = [vp, vp, vp, vp, ci, i64, i64, i64, i64, vp, vp, vp]
        lib.lla_decode_step_gated.restype = st
        lib.lla_state_commit_gated.argtypes = [vp, vp, vp, ci, i64, i64, i64, i64, i64, vp, vp, vp]
        lib.lla_state_commit_gated.restype = st
        lib.lla_prefill_gated_gqa_workspace_size.argtypes = [i64] * 7
        lib.lla_prefill_gated_gqa_workspace_size.restype = sz
        lib.lla_prefill_gated_gqa.argtypes = [vp, vp, vp, vp, ci, i64, i64, i64, i64, i64, i64, i64,
                                              ctypes.c_uint, vp, vp, vp, sz, vp]
        lib.lla_prefill_gated_gqa.restype = st
        lib.lla_decode_step_gated_gqa.argtypes = [vp, vp, vp, vp, ci, i64, i64, i64, i64, i64, vp, vp, vp]
        lib.lla_decode_step_gated_gqa.restype = st
        _lib = lib
    return _lib


def _check(status: int, what: str):
    if status != 0:
        raise LlaError(status, what)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _BF16
    if t.dtype == torch.float32:
        return _F32
    if t.dtype == torch.float8_e4m3fn:  # OCP FP8 E4M3
        return _FP8
    raise TypeError("inputs must be bfloat16, float32 or float8_e4m3fn, got %s" % t.dtype)


def _ptr(t):
    return None if t is None or t.numel() == 0 else t.data_ptr()


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU (got %s)" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims (got shape %s)" % (name, ndim, tuple(t.shape)))


def _same_device(device, **tensors):
    """Every buffer of a call on the inputs' device (the kernels run there)."""
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError("%s is on %s, the inputs on %s" % (name, t.device, device))


def _qkv_shape(q, k, v):
    """(B, Hq, Hkv, T, dk, dv) of q [B,Hq,T,dk], k [B,Hkv,T,dk], v [B,Hkv,T,dv]."""
    _need(q, "q", ndim=4)
    _need(k, "k", dtype=q.dtype, ndim=4)
    _need(v, "v", dtype=q.dtype, ndim=4)
    B, Hq, T, dk = q.shape
    Hkv = k.shape[1]
    if Hkv < 1 or tuple(k.shape) != (B, Hkv, T, dk) or tuple(v.shape[:3]) != (B, Hkv, T) or Hq % Hkv:
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    _same_device(q.device, k=k, v=v)
    return B, Hq, Hkv, T, dk, v.shape[3]


def _mha_shape(q, k, v):
    B, Hq, Hkv, T, dk, dv = _qkv_shape(q, k, v)
    if Hq != Hkv:
        raise ValueError("the prefill phases take one key/value head per query head")
    return B, Hq, T, dk, dv


def state_init(B: int, H: int, dk: int, dv: int, device=None, out: torch.Tensor = None):
    """A zero state [B, H, dk, dv] fp32 (S_0 of a fresh prompt), via lla_state_init."""
    lib = library()
    if out is None:
        out = torch.empty((B, H, dk, dv), dtype=torch.float32,
                          device=device if device is not None else "cuda")
    _need(out, "state", dtype=torch.float32, ndim=4)
    if tuple(out.shape) != (B, H, dk, dv):
        raise ValueError("state shape %s, expected %s" % (tuple(out.shape), (B, H, dk, dv)))
    _check(lib.lla_state_init(_ptr(out), B, H, dk, dv, _stream(out)), "lla_state_init")
    return out


def prefill_segment_chunks(B, H, T, dk, dv, chunk) -> int:
    """Chunks one workgroup walks (G); segment s covers tokens [s*G*C, (s+1)*G*C)."""
    return int(library().lla_prefill_segment_chunks(B, H, T, dk, dv, chunk))


def set_publish_wait_ticks(ticks: int) -> None:
    """How long (100 MHz GPU real-time ticks) a one-launch walk waits for an
    earlier segment's published sum before summing it itself, for later
    calls (lla_set_publish_wait_ticks; results do not depend on it)."""
    _check(library().lla_set_publish_wait_ticks(int(ticks)), "lla_set_publish_wait_ticks")


def prefill_workspace_size(B, H, T, dk, dv, chunk) -> int:
    return int(library().lla_prefill_workspace_size(B, H, T, dk, dv, chunk))


def prefill_gqa_workspace_size(B, Hq, Hkv, T, dk, dv, chunk) -> int:
    return int(library().lla_prefill_gqa_workspace_size(B, Hq, Hkv, T, dk, dv, chunk))


def _workspace(B, H, T, dk, dv, chunk, device, workspace, Hkv=None):
    need = prefill_gqa_workspace_size(B, H, H if Hkv is None else Hkv, T, dk, dv, chunk)
    if workspace is None:
        if need == 0:
            return None, 0
        workspace = torch.empty(need // 4, dtype=torch.float32, device=device)
    _need(workspace, "workspace")
    return workspace, workspace.numel() * workspace.element_size()


def _state_check(state, B, H, dk, dv):
    _need(state, "state", dtype=torch.float32, ndim=4)
    if tuple(state.shape) != (B, H, dk, dv):
        raise ValueError("state shape %s, expected %s" % (tuple(state.shape), (B, H, dk, dv)))


def _out(out, shape, device):
    if out is None:
        return torch.empty(shape, dtype=torch.float32, device=device)
    _need(out, "out", dtype=torch.float32)
    if tuple(out.shape) != tuple(shape):
        raise ValueError("out shape %s, expected %s" % (tuple(out.shape), tuple(shape)))
    return out


def prefill(q, k, v, state, chunk: int, out=None, workspace=None, zero_state: bool = False,
            keep_state: bool = False):
    """Chunkwise prefill: returns o [B,Hq,T,dv] fp32; ``state`` [B,Hkv,dk,dv] goes
    S_0 -> S_T in place.  k, v with fewer heads than q (Hq a multiple of Hkv)
    select shared-state heads (lla_prefill_gqa).  ``zero_state``: a fresh
    prompt -- start from S_0 = 0 without reading ``state`` (lla_prefill_ex).
    ``keep_state``: a verify pass over draft tokens -- ``state`` is read but
    keeps S_0 (lla_prefill_ex; then :func:`state_commit`)."""
    lib = library()
    B, Hq, Hkv, T, dk, dv = _qkv_shape(q, k, v)
    _state_check(state, B, Hkv, dk, dv)
    out = _out(out, (B, Hq, T, dv), q.device)
    ws, ws_bytes = _workspace(B, Hq, T, dk, dv, chunk, q.device, workspace, Hkv)
    _same_device(q.device, state=state, out=out, workspace=ws)
    if zero_state or keep_state:
        flags = (PREFILL_ZERO_STATE if zero_state else 0) | (PREFILL_KEEP_STATE if keep_state else 0)
        _check(lib.lla_prefill_ex(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, Hq, Hkv, T, dk, dv,
                                  chunk, flags, _ptr(state), _ptr(out), _ptr(ws),
                                  ws_bytes, _stream(q)), "lla_prefill_ex")
    elif Hq == Hkv:
        _check(lib.lla_prefill(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, Hq, T, dk, dv, chunk,
                               _ptr(state), _ptr(out), _ptr(ws), ws_bytes, _stream(q)), "lla_prefill")
    else:
        _check(lib.lla_prefill_gqa(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, Hq, Hkv, T, dk, dv,
                                   chunk, _ptr(state), _ptr(out), _ptr(ws), ws_bytes, _stream(q)),
               "lla_prefill_gqa")
    return out


def prefill_gated_workspace_size(B, H, T, dk, dv, chunk, Hkv=None) -> int:
    """Workspace bytes of a gated prefill (H query heads on Hkv states;
    Hkv defaults to H)."""
    return int(library().lla_prefill_gated_gqa_workspace_size(B, H, Hkv or H, T, dk, dv, chunk))


def _gated_prefill_args(q, k, v, gate, state, chunk, out, workspace):
    """Checks a gated prefill's buffers; returns the head of its argument
    list, its tail and the output."""
    B, Hq, Hkv, T, dk, dv = _qkv_shape(q, k, v)
    _need(gate, "gate", dtype=torch.float32, ndim=3)
    if tuple(gate.shape) != (B, Hkv, T):
        raise ValueError("gate shape %s, expected %s (one gate per state and token)" % (tuple(gate.shape),
                                                                                       (B, Hkv, T)))
    _state_check(state, B, Hkv, dk, dv)
    out = _out(out, (B, Hq, T, dv), q.device)
    need = prefill_gated_workspace_size(B, Hq, T, dk, dv, chunk, Hkv)
    if workspace is None and need:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=q.device)
    if workspace is not None:
        _need(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _same_device(q.device, gate=gate, state=state, out=out, workspace=workspace)
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _dtype_code(q), B, Hq, Hkv, T, dk, dv, chunk)
    tail = (_ptr(state), _ptr(out), _ptr(workspace), ws_bytes)
    return head, tail, out, workspace


def prefill_gated(q, k, v, gate, state, chunk: int, out=None, workspace=None, zero_state: bool = False,
                  keep_state: bool = False):
    """Prefill with a decayed state (lla_prefill_gated_gqa): ``S_t = g_t
    S_{t-1} + k_t v_t^T``, ``o_t = S_t^T q_t``, one gate per state and token.
    q: [B,Hq,T,dk]; k, v: [B,Hkv,T,*] (Hq a multiple of Hkv: shared-state
    heads); ``gate``: fp32 [B,Hkv,T].  Returns o [B,Hq,T,dv] fp32; ``state``
    [B,Hkv,dk,dv] goes S_0 -> S_T in place (``keep_state``: a verify pass,
    ``state`` not written; then :func:`state_commit_gated`)."""
    lib = library()
    head, tail, out, _ = _gated_prefill_args(q, k, v, gate, state, chunk, out, workspace)
    flags = (PREFILL_ZERO_STATE if zero_state else 0) | (PREFILL_KEEP_STATE if keep_state else 0)
    _check(lib.lla_prefill_gated_gqa(*head, flags, *tail, _stream(q)), "lla_prefill_gated_gqa")
    return out


def prefill_noalloc(q, k, v, state, chunk: int, out=None, zero_state: bool = False):
    """:func:`prefill` through lla_prefill_noalloc: the library takes the
    workspace from its static per-device array instead of the caller, so the
    call allocates nothing when ``out`` is given.  Calls that overlap in time
    on one device race on that array."""
    lib = library()
    B, Hq, Hkv, T, dk, dv = _qkv_shape(q, k, v)
    _state_check(state, B, Hkv, dk, dv)
    out = _out(out, (B, Hq, T, dv), q.device)
    _same_device(q.device, state=state, out=out)
    _check(lib.lla_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, Hq, Hkv, T, dk, dv, chunk,
                                   PREFILL_ZERO_STATE if zero_state else 0, _ptr(state), _ptr(out),
                                   _stream(q)), "lla_prefill_noalloc")
    return out


def _commit_args(k, v, state, accepted):
    """Checks the buffers of a commit; returns (B, H, T, dk, dv)."""
    _need(k, "k", ndim=4)
    _need(v, "v", dtype=k.dtype, ndim=4)
    B, H, T, dk = k.shape
    dv = v.shape[3]
    if tuple(v.shape[:3]) != (B, H, T):
        raise ValueError("shape mismatch: k %s v %s" % (tuple(k.shape), tuple(v.shape)))
    _state_check(state, B, H, dk, dv)
    if accepted is not None:
        _need(accepted, "accepted", dtype=torch.int32, ndim=1)
        if accepted.shape[0] != B:
            raise ValueError("accepted has %d entries, expected %d" % (accepted.shape[0], B))
    _same_device(k.device, v=v, state=state, accepted=accepted)
    return B, H, T, dk, dv


def state_commit(k, v, state, accepted=None):
    """After a verify pass (``prefill(..., keep_state=True)``): ``state`` +=
    sum over the first m_b tokens of k_t v_t^T for every sequence b, m_b =
    ``accepted[b]`` (a device int32 tensor [B]; None: all T), with the decode
    step's arithmetic (lla_state_commit).  k, v: [B, Hkv, T, d]."""
    lib = library()
    B, H, T, dk, dv = _commit_args(k, v, state, accepted)
    _check(lib.lla_state_commit(_ptr(k), _ptr(v), _dtype_code(k), B, H, T, dk, dv, _ptr(accepted),
                                _ptr(state), _stream(k)), "lla_state_commit")
    return state


def state_commit_gated(k, v, gate, state, accepted=None):
    """After a gated verify pass (``prefill_gated(..., keep_state=True)``):
    for every sequence b and its first m_b tokens in order, ``state = g_t
    state + k_t v_t^T`` with the gated decode step's arithmetic
    (lla_state_commit_gated).  k, v: [B, H, T, d]; gate: fp32 [B, H, T]."""
    lib = library()
    B, H, T, dk, dv = _commit_args(k, v, state, accepted)
    _need(gate, "gate", dtype=torch.float32, ndim=3)
    if tuple(gate.shape) != (B, H, T):
        raise ValueError("gate shape %s, expected %s" % (tuple(gate.shape), (B, H, T)))
    _same_device(k.device, gate=gate)
    _check(lib.lla_state_commit_gated(_ptr(k), _ptr(v), _ptr(gate), _dtype_code(k), B, H, T, dk, dv,
                                      _ptr(accepted), _ptr(state), _stream(k)), "lla_state_commit_gated")
    return state


def prefill_segment_states(k, v, chunk: int, workspace):
    """Phase 1: K^T V of every segment but the last into workspace slots 1.."""
    lib = library()
    _need(k, "k", ndim=4)
    _need(v, "v", dtype=k.dtype, ndim=4)
    B, H, T, dk = k.shape
    dv = v.shape[3]
    ws, ws_bytes = _workspace(B, H, T, dk, dv, chunk, k.device, workspace)
    _same_device(k.device, v=v, workspace=ws)
    _check(lib.lla_prefill_segment_states(_ptr(k), _ptr(v), _dtype_code(k), B, H, T, dk, dv, chunk,
                                          _ptr(ws), ws_bytes, _stream(k)),
           "lla_prefill_segment_states")
    return ws


def prefill_state_scan(state, T: int, chunk: int, workspace):
    """Phase 2: segment starting states from S_0 (``state``, read only)."""
    lib = library()
    B, H, dk, dv = state.shape
    _state_check(state, B, H, dk, dv)
    ws, ws_bytes = _workspace(B, H, T, dk, dv, chunk, state.device, workspace)
    _same_device(state.device, workspace=ws)
    _check(lib.lla_prefill_state_scan(_ptr(state), B, H, T, dk, dv, chunk, _ptr(ws), ws_bytes,
                                      _stream(state)), "lla_prefill_state_scan")
    return ws


def prefill_chunks(q, k, v, state, chunk: int, workspace=None, out=None):
    """Phase 3: the chunk walk from the segment states; writes o and S_T."""
    lib = library()
    B, H, T, dk, dv = _mha_shape(q, k, v)
    _state_check(state, B, H, dk, dv)
    out = _out(out, (B, H, T, dv), q.device)
    need = prefill_workspace_size(B, H, T, dk, dv, chunk)
    if workspace is not None:
        _need(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if need and workspace is None:
        raise ValueError("this shape needs a %d-byte workspace filled by phases 1 and 2" % need)
    _same_device(q.device, state=state, out=out, workspace=workspace)
    _check(lib.lla_prefill_chunks(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, H, T, dk, dv, chunk,
                                  _ptr(state), _ptr(out), _ptr(workspace), ws_bytes, _stream(q)),
           "lla_prefill_chunks")
    return out


def _step_shape(q, k, v):
    """(B, Hq, Hkv, dk, dv) of q [B,Hq,dk], k [B,Hkv,dk], v [B,Hkv,dv]."""
    _need(q, "q", ndim=3)
    _need(k, "k", dtype=q.dtype, ndim=3)
    _need(v, "v", dtype=q.dtype, ndim=3)
    B, Hq, dk = q.shape
    Hkv, dv = k.shape[1], v.shape[2]
    if Hkv < 1 or tuple(k.shape) != (B, Hkv, dk) or tuple(v.shape[:2]) != (B, Hkv) or Hq % Hkv:
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    _same_device(q.device, k=k, v=v)
    return B, Hq, Hkv, dk, dv


def _step_call(lib, q, k, v, state, out, B, Hq, Hkv, dk, dv):
    """(function, argument tuple) of the decode step for these buffers."""
    if Hq == Hkv:
        return lib.lla_decode_step, (_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, Hq, dk, dv,
                                     _ptr(state), _ptr(out))
    return lib.lla_decode_step_gqa, (_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, Hq, Hkv, dk, dv,
                                     _ptr(state), _ptr(out))


def decode_step(q, k, v, state, out=None):
    """One decode step: ``state += k v^T`` in place; returns o = state^T q [B,Hq,dv]
    fp32.  k, v with fewer heads than q select shared-state heads."""
    lib = library()
    B, Hq, Hkv, dk, dv = _step_shape(q, k, v)
    _state_check(state, B, Hkv, dk, dv)
    out = _out(out, (B, Hq, dv), q.device)
    _same_device(q.device, state=state, out=out)
    fn, args = _step_call(lib, q, k, v, state, out, B, Hq, Hkv, dk, dv)
    _check(fn(*args, _stream(q)), fn.__name__)
    return out


def _gated_step_args(q, k, v, gate, state, out):
    B, Hq, Hkv, dk, dv = _step_shape(q, k, v)
    _need(gate, "gate", dtype=torch.float32, ndim=2)
    if tuple(gate.shape) != (B, Hkv):
        raise ValueError("gate shape %s, expected %s (one gate per state)" % (tuple(gate.shape), (B, Hkv)))
    _state_check(state, B, Hkv, dk, dv)
    out = _out(out, (B, Hq, dv), q.device)
    _same_device(q.device, gate=gate, state=state, out=out)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _dtype_code(q), B, Hq, Hkv, dk, dv, _ptr(state), _ptr(out))
    return args, out


def decode_step_gated(q, k, v, gate, state, out=None):
    """One gated decode step (lla_decode_step_gated_gqa): ``state = g state +
    k v^T`` in place, then o = state^T q for every query head.  q: [B,Hq,dk];
    k, v: [B,Hkv,d*]; gate: fp32 [B,Hkv]."""
    lib = library()
    args, out = _gated_step_args(q, k, v, gate, state, out)
    _check(lib.lla_decode_step_gated_gqa(*args, _stream(q)), "lla_decode_step_gated_gqa")
    return out


class PreparedPrefill:
    """A prefill whose arguments were checked and marshalled once.

    For loops that call the same prefill on the same buffers many times (the
    benchmark, a serving loop): calling the object calls lla_prefill (or, for
    a fresh prompt, lla_prefill_ex with PREFILL_ZERO_STATE) with the stored
    pointers on the current stream.  The object holds references to every
    tensor it was given, so their memory stays allocated while it lives; the
    tensors must keep their shapes.
    """

    def __init__(self, q, k, v, state, chunk, out=None, workspace=None):
        lib = library()
        B, H, Hkv, T, dk, dv = _qkv_shape(q, k, v)
        _state_check(state, B, Hkv, dk, dv)
        self.out = _out(out, (B, H, T, dv), q.device)
        self.workspace, ws_bytes = _workspace(B, H, T, dk, dv, chunk, q.device, workspace, Hkv)
        _same_device(q.device, state=state, out=self.out, workspace=self.workspace)
        self.state = state
        self._lib = lib
        self._init = lib.lla_state_init
        self._grouped = H != Hkv
        dt, ws = _dtype_code(q), _ptr(self.workspace)
        if self._grouped:
            self._fn = lib.lla_prefill_gqa
            self._args = (_ptr(q), _ptr(k), _ptr(v), dt, B, H, Hkv, T, dk, dv, chunk,
                          _ptr(state), _ptr(self.out), ws, ws_bytes)
        else:
            self._fn = lib.lla_prefill
            self._args = (_ptr(q), _ptr(k), _ptr(v), dt, B, H, T, dk, dv, chunk,
                          _ptr(state), _ptr(self.out), ws, ws_bytes)
        self._ex_head = (_ptr(q), _ptr(k), _ptr(v), dt, B, H, Hkv, T, dk, dv, chunk)
        self._ex_tail = (_ptr(state), _ptr(self.out), ws, ws_bytes)
        self._init_args = (_ptr(state), B, Hkv, dk, dv)
        # every tensor whose address is stored above stays alive with this
        # object (the library reads and writes them on each call)
        self._keep = (q, k, v, state, self.out, self.workspace)
        self._seg_args = (_ptr(k), _ptr(v), dt, B, H, T, dk, dv, chunk, ws, ws_bytes)
        self._scan_args = (_ptr(state), B, H, T, dk, dv, chunk, ws, ws_bytes)
        self._device = q.device

    def _stream(self):
        return torch.cuda.current_stream(self._device).cuda_stream

    def __call__(self, zero_state: bool = False, keep_state: bool = False):
        """One prefill; ``zero_state``: a fresh prompt (S_0 = 0, the state is
        not read); ``keep_state``: a verify pass (the state is not written)."""
        st = self._stream()
        if zero_state or keep_state:
            flags = (PREFILL_ZERO_STATE if zero_state else 0) | (PREFILL_KEEP_STATE if keep_state else 0)
            _check(self._lib.lla_prefill_ex(*self._ex_head, flags, *self._ex_tail, st), "lla_prefill_ex")
        else:
            _check(self._fn(*self._args, st), self._fn.__name__)
        return self.out

    # The three phases of the call, one by one (for per-kernel timing; one
    # key/value head per query head only).
    def zero_state(self):
        _check(self._init(*self._init_args, self._stream()), "lla_state_init")

    def segment_states(self):
        self._mha_only()
        _check(self._lib.lla_prefill_segment_states(*self._seg_args, self._stream()),
               "lla_prefill_segment_states")

    def state_scan(self):
        self._mha_only()
        _check(self._lib.lla_prefill_state_scan(*self._scan_args, self._stream()),
               "lla_prefill_state_scan")

    def _mha_only(self):
        if self._grouped:
            raise ValueError("the prefill phases take one key/value head per query head")

    def chunks(self):
        self._mha_only()
        _check(self._lib.lla_prefill_chunks(*self._args, self._stream()), "lla_prefill_chunks")
        return self.out


class PreparedGatedPrefill:
    """A gated prefill (lla_prefill_gated_gqa) over fixed buffers, checked and
    marshalled once (see PreparedPrefill): calling it runs one prefill on the
    current stream, a fresh prompt with ``zero_state``, a verify pass with
    ``keep_state``."""

    def __init__(self, q, k, v, gate, state, chunk, out=None, workspace=None):
        lib = library()
        self._head, self._tail, self.out, self.workspace = _gated_prefill_args(q, k, v, gate, state, chunk, out,
                                                                               workspace)
        self._fn = lib.lla_prefill_gated_gqa
        self._keep = (q, k, v, gate, state, self.out, self.workspace)  # the buffers behind the addresses
        self._device = q.device

    def __call__(self, zero_state: bool = False, keep_state: bool = False):
        st = torch.cuda.current_stream(self._device).cuda_stream
        flags = (PREFILL_ZERO_STATE if zero_state else 0) | (PREFILL_KEEP_STATE if keep_state else 0)
        _check(self._fn(*self._head, flags, *self._tail, st), "lla_prefill_gated_gqa")
        return self.out


class PreparedGatedDecode:
    """A gated decode step (lla_decode_step_gated_gqa) over fixed buffers,
    marshalled once."""

    def __init__(self, q, k, v, gate, state, out=None):
        lib = library()
        self._args, self.out = _gated_step_args(q, k, v, gate, state, out)
        self._fn = lib.lla_decode_step_gated_gqa
        self._keep = (q, k, v, gate, state, self.out)
        self._device = q.device

    def __call__(self):
        _check(self._fn(*self._args, torch.cuda.current_stream(self._device).cuda_stream),
               "lla_decode_step_gated_gqa")
        return self.out


class PreparedDecode:
    """A decode step over fixed buffers, marshalled once (see PreparedPrefill)."""

    def __init__(self, q, k, v, state, out=None):
        lib = library()
        B, Hq, Hkv, dk, dv = _step_shape(q, k, v)
        _state_check(state, B, Hkv, dk, dv)
        self.out = _out(out, (B, Hq, dv), q.device)
        _same_device(q.device, state=state, out=self.out)
        self._fn, self._args = _step_call(lib, q, k, v, state, self.out, B, Hq, Hkv, dk, dv)
        self._keep = (q, k, v, state, self.out)  # the buffers behind the stored addresses
        self._device = q.device

    def __call__(self):
        _check(self._fn(*self._args, torch.cuda.current_stream(self._device).cuda_stream),
               self._fn.__name__)
        return self.out
