"""Host-side checks of the gated calls of the C ABI (no GPU): lla_prefill_gated,
lla_prefill_gated_workspace_size and lla_decode_step_gated reject bad
arguments with the documented status before anything is enqueued.  Pointers
are plain integers; every call here fails validation or is a no-op."""
import ctypes

import pytest
import torch

import decode_lla_prefill_amd as lla

OK, E_NULL, E_SHAPE, E_DTYPE, E_UNSUP, E_ALIGN, E_ALIAS, E_WS = range(8)
BF16, F32 = 0, 1
i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
A = 1 << 32  # a 16-byte aligned fake address; buffers far apart


@pytest.fixture(scope="module")
def lib():
    L = ctypes.CDLL(lla.library_path)
    L.lla_prefill_gated.restype = ctypes.c_int
    L.lla_prefill_gated.argtypes = ([vp, vp, vp, vp, ctypes.c_int] + [i64] * 6 + [ctypes.c_uint] +
                                    [vp, vp, vp, sz, vp])
    L.lla_prefill_gated_workspace_size.restype = sz
    L.lla_prefill_gated_workspace_size.argtypes = [i64] * 6
    L.lla_prefill_workspace_size.restype = sz
    L.lla_prefill_workspace_size.argtypes = [i64] * 6
    L.lla_prefill_segment_chunks.restype = i64
    L.lla_prefill_segment_chunks.argtypes = [i64] * 6
    L.lla_decode_step_gated.restype = ctypes.c_int
    L.lla_decode_step_gated.argtypes = [vp, vp, vp, vp, ctypes.c_int] + [i64] * 4 + [vp, vp, vp]
    L.lla_prefill_gated_gqa.restype = ctypes.c_int
    L.lla_prefill_gated_gqa.argtypes = ([vp, vp, vp, vp, ctypes.c_int] + [i64] * 7 + [ctypes.c_uint] +
                                        [vp, vp, vp, sz, vp])
    L.lla_prefill_gated_gqa_workspace_size.restype = sz
    L.lla_prefill_gated_gqa_workspace_size.argtypes = [i64] * 7
    L.lla_decode_step_gated_gqa.restype = ctypes.c_int
    L.lla_decode_step_gated_gqa.argtypes = [vp, vp, vp, vp, ctypes.c_int] + [i64] * 5 + [vp, vp, vp]
    L.lla_state_commit_gated.restype = ctypes.c_int
    L.lla_state_commit_gated.argtypes = [vp, vp, vp, ctypes.c_int] + [i64] * 5 + [vp, vp, vp]
    return L


def _prefill(lib, **change):
    d = dict(q=A, k=2 * A, v=3 * A, gate=7 * A, dtype=BF16, B=1, H=2, T=100, dk=64, dv=64, C=64, flags=0,
             S=4 * A, O=5 * A, ws=6 * A, ws_bytes=1 << 30)
    d.update(change)
    return lib.lla_prefill_gated(d["q"], d["k"], d["v"], d["gate"], d["dtype"], d["B"], d["H"], d["T"], d["dk"],
                                 d["dv"], d["C"], d["flags"], d["S"], d["O"], d["ws"], d["ws_bytes"], None)


@pytest.mark.parametrize("change,expect", [
    (dict(gate=None), E_NULL), (dict(q=None), E_NULL), (dict(S=None), E_NULL), (dict(O=None), E_NULL),
    (dict(flags=4), E_UNSUP), (dict(flags=7), E_UNSUP), (dict(flags=2, q=None), E_NULL),
    (dict(flags=3, q=None), E_NULL),
    (dict(B=0), E_SHAPE), (dict(dk=129), E_SHAPE), (dict(C=0), E_SHAPE), (dict(C=129), E_SHAPE),
    (dict(dtype=7), E_DTYPE), (dict(dtype=F32, C=128, q=None), E_NULL),
    (dict(gate=7 * A + 2), E_ALIGN), (dict(q=A + 8), E_ALIGN),
    (dict(gate=5 * A + 64), E_ALIAS), (dict(gate=4 * A), E_ALIAS), (dict(O=A + 64), E_ALIAS),
    (dict(T=8192, ws_bytes=16), E_WS), (dict(T=8192, ws=None), E_WS),
    (dict(T=8192, ws=7 * A + 4096), E_ALIAS), (dict(T=8192, ws=6 * A + 8), E_ALIGN),
])
def test_prefill_gated_rejects(lib, change, expect):
    assert _prefill(lib, **change) == expect


def test_prefill_gated_accepts_a_gate_aligned_to_its_elements(lib):
    # a 4-byte aligned gate passes the checks; NULL q/k then fails next
    assert _prefill(lib, gate=7 * A + 4, q=None) == E_NULL


def test_prefill_gated_empty_prompt_is_a_noop(lib):
    assert _prefill(lib, T=0, q=None, k=None, v=None, O=None, gate=None) == OK


@pytest.mark.parametrize("B,H,T,d,C", [(1, 2, 8192, 64, 64), (1, 16, 8192, 128, 64), (4, 8, 1024, 64, 64),
                                       (2, 3, 100, 32, 32), (1, 1, 64, 128, 64)])
def test_gated_workspace_is_the_states_and_one_decay_per_segment(lib, B, H, T, d, C):
    G = lib.lla_prefill_segment_chunks(B, H, T, d, d, C)
    n_seg = -(-(-(-T // C)) // G)
    need = lib.lla_prefill_gated_workspace_size(B, H, T, d, d, C)
    if n_seg == 1:
        assert need == 0
    else:
        assert need == B * H * n_seg * (d * d + 1) * 4
        # (at least the plain prefill's states; that size also covers the
        # one-launch walk's published sums where a shape can take it)
        assert need - B * H * n_seg * 4 <= lib.lla_prefill_workspace_size(B, H, T, d, d, C)


def _decode(lib, **change):
    d = dict(q=A, k=2 * A, v=3 * A, gate=7 * A, dtype=BF16, B=2, H=4, dk=128, dv=128, S=4 * A, o=5 * A)
    d.update(change)
    return lib.lla_decode_step_gated(d["q"], d["k"], d["v"], d["gate"], d["dtype"], d["B"], d["H"], d["dk"],
                                     d["dv"], d["S"], d["o"], None)


@pytest.mark.parametrize("change,expect", [
    (dict(gate=None), E_NULL), (dict(S=None), E_NULL), (dict(B=0), E_SHAPE), (dict(dv=200), E_SHAPE),
    (dict(dtype=5), E_DTYPE), (dict(gate=7 * A + 1), E_ALIGN), (dict(S=4 * A + 8), E_ALIGN),
    (dict(gate=4 * A + 64), E_ALIAS), (dict(gate=5 * A), E_ALIAS), (dict(o=3 * A), E_ALIAS),
])
def test_decode_step_gated_rejects(lib, change, expect):
    assert _decode(lib, **change) == expect


def test_python_binding_checks_gate_shapes_without_the_gpu():
    q = torch.zeros(1, 2, 8, 16, dtype=torch.bfloat16)
    S = torch.zeros(1, 2, 16, 16)
    with pytest.raises((ValueError, TypeError)):
        lla.prefill_gated(q, q, q, torch.ones(1, 2, 8), S, 8)  # host tensors
    with pytest.raises((ValueError, TypeError)):
        lla.decode_step_gated(q[:, :, 0], q[:, :, 0], q[:, :, 0], torch.ones(1, 2), S)


def _commit(lib, **change):
    d = dict(k=A, v=2 * A, gate=3 * A, dtype=BF16, B=2, H=4, T=6, dk=128, dv=128, acc=5 * A, S=4 * A)
    d.update(change)
    return lib.lla_state_commit_gated(d["k"], d["v"], d["gate"], d["dtype"], d["B"], d["H"], d["T"], d["dk"],
                                      d["dv"], d["acc"], d["S"], None)


@pytest.mark.parametrize("change,expect", [
    (dict(gate=None), E_NULL), (dict(k=None), E_NULL), (dict(S=None), E_NULL), (dict(B=0), E_SHAPE),
    (dict(dk=129), E_SHAPE), (dict(dtype=9), E_DTYPE), (dict(gate=3 * A + 2), E_ALIGN),
    (dict(acc=5 * A + 4), E_ALIGN), (dict(S=4 * A + 8), E_ALIGN),
    (dict(gate=4 * A + 64), E_ALIAS), (dict(S=A + 16), E_ALIAS), (dict(acc=4 * A + 4096), E_ALIAS),
])
def test_state_commit_gated_rejects(lib, change, expect):
    assert _commit(lib, **change) == expect


def test_state_commit_gated_of_no_tokens_is_a_noop(lib):
    assert _commit(lib, T=0, k=None, v=None, gate=None) == OK


def _prefill_gqa(lib, **change):
    d = dict(q=A, k=2 * A, v=3 * A, gate=7 * A, dtype=BF16, B=1, Hq=8, Hkv=2, T=100, dk=64, dv=64, C=64, flags=0,
             S=4 * A, O=5 * A, ws=6 * A, ws_bytes=1 << 30)
    d.update(change)
    return lib.lla_prefill_gated_gqa(d["q"], d["k"], d["v"], d["gate"], d["dtype"], d["B"], d["Hq"], d["Hkv"],
                                     d["T"], d["dk"], d["dv"], d["C"], d["flags"], d["S"], d["O"], d["ws"],
                                     d["ws_bytes"], None)


@pytest.mark.parametrize("change,expect", [
    (dict(Hkv=3), E_SHAPE), (dict(Hq=1), E_SHAPE), (dict(Hkv=0), E_SHAPE), (dict(gate=None), E_NULL),
    (dict(dtype=9), E_DTYPE), (dict(flags=4), E_UNSUP),
    # one segment, but grouped heads stage their start states: a workspace is needed
    (dict(ws=None), E_WS), (dict(ws_bytes=16), E_WS),
    # the gate holds one value per state and token: B * Hkv * T = 200 floats
    (dict(gate=4 * A + 64), E_ALIAS), (dict(O=7 * A + 784), E_ALIAS),
])
def test_prefill_gated_gqa_rejects(lib, change, expect):
    assert _prefill_gqa(lib, **change) == expect


def test_gated_gqa_workspace_stages_the_start_states_of_grouped_heads(lib):
    # 50 tokens, one chunk, 2 states: one segment, yet a slot and a decay per state
    assert lib.lla_prefill_gated_gqa_workspace_size(1, 8, 2, 50, 64, 64, 64) == 2 * 1 * (64 * 64 + 1) * 4
    assert lib.lla_prefill_gated_gqa_workspace_size(1, 2, 2, 50, 64, 64, 64) == 0
    # 100 tokens: two chunks, one segment each
    assert lib.lla_prefill_gated_gqa_workspace_size(1, 8, 2, 100, 64, 64, 64) == 2 * 2 * (64 * 64 + 1) * 4
    for args in [(1, 16, 8192, 128, 128, 64), (2, 3, 100, 32, 32, 32)]:
        B, H = args[0], args[1]
        assert lib.lla_prefill_gated_gqa_workspace_size(B, H, H, *args[2:]) == \
            lib.lla_prefill_gated_workspace_size(*args)


def test_decode_step_gated_gqa_rejects(lib):
    args = dict(q=A, k=2 * A, v=3 * A, gate=7 * A, dtype=BF16, B=2, Hq=8, Hkv=2, dk=128, dv=128, S=4 * A, o=5 * A)

    def call(**change):
        d = dict(args, **change)
        return lib.lla_decode_step_gated_gqa(d["q"], d["k"], d["v"], d["gate"], d["dtype"], d["B"], d["Hq"],
                                             d["Hkv"], d["dk"], d["dv"], d["S"], d["o"], None)
    assert call(Hkv=3) == E_SHAPE
    assert call(gate=None) == E_NULL
    assert call(gate=7 * A + 2) == E_ALIGN
    assert call(gate=4 * A + 64) == E_ALIAS  # inside S
