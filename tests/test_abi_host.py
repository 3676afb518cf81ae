"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/lla.h declares, and rejects bad arguments with the
documented status before it enqueues anything.

Every call here fails validation (or is a no-op such as T = 0), so no HIP
call is made and no device memory is touched: pointers are plain integers.
"""
import ctypes
import math
import os
import re

import pytest

import decode_lla_prefill_amd as lla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lla.h")

OK, E_NULL, E_SHAPE, E_DTYPE, E_UNSUP, E_ALIGN, E_ALIAS, E_WS, E_DEV, E_SCRATCH = range(10)
BF16, F32 = 0, 1
i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lla_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    L = ctypes.CDLL(lla.library_path)
    L.lla_status_string.restype = ctypes.c_char_p
    L.lla_status_string.argtypes = [ctypes.c_int]
    L.lla_prefill_segment_chunks.restype = i64
    L.lla_prefill_segment_chunks.argtypes = [i64] * 6
    L.lla_prefill_workspace_size.restype = sz
    L.lla_prefill_workspace_size.argtypes = [i64] * 6
    L.lla_prefill.restype = ctypes.c_int
    L.lla_prefill.argtypes = [vp, vp, vp, ctypes.c_int] + [i64] * 6 + [vp, vp, vp, sz, vp]
    L.lla_prefill_chunks.restype = ctypes.c_int
    L.lla_prefill_chunks.argtypes = L.lla_prefill.argtypes
    L.lla_prefill_segment_states.restype = ctypes.c_int
    L.lla_prefill_segment_states.argtypes = [vp, vp, ctypes.c_int] + [i64] * 6 + [vp, sz, vp]
    L.lla_prefill_state_scan.restype = ctypes.c_int
    L.lla_prefill_state_scan.argtypes = [vp] + [i64] * 6 + [vp, sz, vp]
    L.lla_decode_step.restype = ctypes.c_int
    L.lla_decode_step.argtypes = [vp, vp, vp, ctypes.c_int] + [i64] * 4 + [vp, vp, vp]
    L.lla_state_init.restype = ctypes.c_int
    L.lla_state_init.argtypes = [vp] + [i64] * 4 + [vp]
    L.lla_last_device_error.restype = ctypes.c_int
    L.lla_prefill_gqa_workspace_size.restype = sz
    L.lla_prefill_gqa_workspace_size.argtypes = [i64] * 7
    L.lla_prefill_gqa.restype = ctypes.c_int
    L.lla_prefill_gqa.argtypes = [vp, vp, vp, ctypes.c_int] + [i64] * 7 + [vp, vp, vp, sz, vp]
    L.lla_decode_step_gqa.restype = ctypes.c_int
    L.lla_decode_step_gqa.argtypes = [vp, vp, vp, ctypes.c_int] + [i64] * 5 + [vp, vp, vp]
    L.lla_prefill_noalloc.restype = ctypes.c_int
    L.lla_prefill_noalloc.argtypes = [vp, vp, vp, ctypes.c_int] + [i64] * 7 + [ctypes.c_uint, vp, vp, vp]
    L.lla_state_commit.restype = ctypes.c_int
    L.lla_state_commit.argtypes = [vp, vp, ctypes.c_int] + [i64] * 5 + [vp, vp, vp]
    L.lla_prefill_ex.restype = ctypes.c_int
    L.lla_prefill_ex.argtypes = ([vp, vp, vp, ctypes.c_int] + [i64] * 7 + [ctypes.c_uint] +
                                 [vp, vp, vp, sz, vp])
    return L


def test_header_declares_the_documented_entry_points():
    names = declared_functions()
    for n in ("lla_prefill", "lla_decode_step", "lla_state_init", "lla_prefill_workspace_size",
              "lla_status_string", "lla_last_device_error"):
        assert n in names


def test_library_exports_every_declared_function(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_exports_match_header():
    assert set(lla.EXPORTS) == set(declared_functions())


def test_status_strings(lib):
    seen = set()
    for code in range(10):
        s = lib.lla_status_string(code)
        assert s and s not in seen
        seen.add(s)
    assert lib.lla_status_string(99)  # unknown codes still get a string
    assert lib.lla_last_device_error() == 0


# ---- prefill argument checks ------------------------------------------------------

A = 1 << 32  # a 16-byte aligned fake address; buffers are placed far apart


class Bufs:
    def __init__(self, B=1, H=2, T=100, dk=64, dv=64, C=64, dtype=BF16):
        self.B, self.H, self.T, self.dk, self.dv, self.C, self.dtype = B, H, T, dk, dv, C, dtype
        self.q, self.k, self.v = A, 2 * A, 3 * A
        self.S, self.O, self.ws = 4 * A, 5 * A, 6 * A
        self.ws_bytes = 1 << 30

    def args(self):
        return (self.q, self.k, self.v, self.dtype, self.B, self.H, self.T, self.dk, self.dv,
                self.C, self.S, self.O, self.ws, self.ws_bytes, None)


@pytest.mark.parametrize("fn", ["lla_prefill", "lla_prefill_chunks"])
@pytest.mark.parametrize("change,expect", [
    (dict(q=None), E_NULL), (dict(k=None), E_NULL), (dict(v=None), E_NULL),
    (dict(O=None), E_NULL), (dict(S=None), E_NULL),
    (dict(B=0), E_SHAPE), (dict(H=0), E_SHAPE), (dict(T=-1), E_SHAPE),
    (dict(dk=0), E_SHAPE), (dict(dk=129), E_SHAPE), (dict(dv=129), E_SHAPE),
    (dict(C=0), E_SHAPE), (dict(C=129), E_SHAPE),
    (dict(dtype=7), E_DTYPE),
    (dict(q=A + 8), E_ALIGN), (dict(O=5 * A + 4), E_ALIGN), (dict(S=4 * A + 2), E_ALIGN),
    (dict(O=A + 64), E_ALIAS), (dict(S=3 * A), E_ALIAS), (dict(O=4 * A + 16), E_ALIAS),
    (dict(T=8192, ws_bytes=16), E_WS), (dict(T=8192, ws=None), E_WS),
])
def test_prefill_rejects(lib, fn, change, expect):
    b = Bufs()
    for key, val in change.items():
        setattr(b, key, val)
    assert getattr(lib, fn)(*b.args()) == expect


def test_fp32_chunks_over_64_pass_the_dtype_check_everywhere(lib):
    # chunks of C > 64 run as two sub-chunks for every dtype, so the plan
    # does not depend on it: the one-call and the phase calls take fp32 at
    # C = 128, and the next check (a NULL pointer) decides
    b = Bufs(dtype=F32, C=128)
    b.q = None
    assert lib.lla_prefill(*b.args()) == E_NULL
    assert lib.lla_prefill_chunks(*b.args()) == E_NULL
    assert lib.lla_prefill_segment_states(None, b.v, F32, 1, 2, 100, 64, 64, 128, b.ws, b.ws_bytes,
                                          None) == E_NULL
    b.q = A
    b.O = A + 64
    assert lib.lla_prefill(*b.args()) == E_ALIAS


@pytest.mark.parametrize("B,H,d", [(1, 16, 128), (4, 8, 64), (1, 1, 32), (64, 32, 128), (2, 3, 100)])
def test_fp32_sub_chunk_plan_fits_the_dtype_less_workspace(lib, B, H, d):
    # With exactly lla_prefill_workspace_size bytes, the fp32 plan for C > 64
    # passes the workspace check and stops at the next one (O aliases q).
    for C in (65, 66, 77, 100, 127, 128):
        for T in (1, 17, 64, 65, 129, 200, 1000, 4097, 8192, 65536):
            ws = lib.lla_prefill_workspace_size(B, H, T, d, d, C)
            b = Bufs(B=B, H=H, T=T, dk=d, dv=d, C=C, dtype=F32)
            b.ws, b.ws_bytes = (6 * A, ws) if ws > 0 else (None, 0)
            b.O = A + 64
            assert lib.lla_prefill(*b.args()) == E_ALIAS, (C, T)


def test_prefill_empty_prompt_is_a_noop(lib):
    b = Bufs(T=0)
    b.q = b.k = b.v = b.O = None  # not needed for T = 0
    assert lib.lla_prefill(*b.args()) == OK


def test_prefill_phase_checks(lib):
    b = Bufs(T=8192)
    assert lib.lla_prefill_segment_states(None, b.v, BF16, 1, 2, 8192, 64, 64, 64, b.ws,
                                          b.ws_bytes, None) == E_NULL
    assert lib.lla_prefill_segment_states(b.k, b.v, BF16, 1, 2, 8192, 64, 64, 64, b.ws, 8,
                                          None) == E_WS
    assert lib.lla_prefill_state_scan(None, 1, 2, 8192, 64, 64, 64, b.ws, b.ws_bytes,
                                      None) == E_NULL
    assert lib.lla_prefill_state_scan(b.S, 1, 2, 8192, 64, 200, 64, b.ws, b.ws_bytes,
                                      None) == E_SHAPE


@pytest.mark.parametrize("change,expect", [
    (dict(q=None), E_NULL), (dict(S=None), E_NULL), (dict(o=None), E_NULL),
    (dict(B=0), E_SHAPE), (dict(dk=0), E_SHAPE), (dict(dv=200), E_SHAPE),
    (dict(dtype=5), E_DTYPE), (dict(k=2 * A + 2), E_ALIGN), (dict(S=4 * A + 8), E_ALIGN),
    (dict(o=4 * A + 64), E_ALIAS), (dict(S=A), E_ALIAS), (dict(o=3 * A), E_ALIAS),
])
def test_decode_rejects(lib, change, expect):
    d = dict(q=A, k=2 * A, v=3 * A, dtype=BF16, B=2, H=4, dk=128, dv=128, S=4 * A, o=5 * A)
    d.update(change)
    assert lib.lla_decode_step(d["q"], d["k"], d["v"], d["dtype"], d["B"], d["H"], d["dk"],
                               d["dv"], d["S"], d["o"], None) == expect


def test_state_init_rejects(lib):
    assert lib.lla_state_init(None, 1, 1, 4, 4, None) == E_NULL
    assert lib.lla_state_init(A + 4, 1, 1, 4, 4, None) == E_ALIGN
    assert lib.lla_state_init(A, 0, 1, 4, 4, None) == E_SHAPE
    assert lib.lla_state_init(A, 1, 1, 4, 300, None) == E_SHAPE


# ---- planning: segments and workspace ------------------------------------------------

def _pad(x):
    return 32 if x <= 32 else (64 if x <= 64 else 128)


def _expected_workspace(B, H, n_seg, G, d):
    """One fp32 d x d state per segment per (b,h), nothing for one segment;
    for a shape that can run as one launch -- several segments and at most 16
    chunks before the last, or, with published sums, at most 16 segments of
    at most 8 chunks, 64 chunks before the last and whole heads in each of
    the 8 XCDs' ranges of workgroups -- at least the room for that walk's
    published segment sums: a slot of 64 x D floats per (b,h), segment and
    value block (D = the padded head dim, blocks of 64 columns), and an
    8-byte flag per slot."""
    if n_seg <= 1:
        return 0
    states = B * H * n_seg * d * d * 4
    D = _pad(d)
    n_vb = D // min(D, 64)
    before = (n_seg - 1) * G
    units = B * H * n_seg * n_vb
    wide = n_seg <= 16 and G <= 8 and before <= 64 and units % 8 == 0 and (units // 8) % (n_seg * n_vb) == 0
    if before > 16 and not wide:
        return states
    slots = B * H * n_seg * n_vb
    return max(states, slots * 64 * D * 4 + slots * 8)


def _lines_rule_G(B, H, T, C):
    """Chunks of C per segment by the line rule: the smallest whole number
    that keeps the (sequence, head, segment) lines at most 256."""
    n_c = math.ceil(T / C)
    return min(math.ceil(n_c * B * H / 256), n_c)


@pytest.mark.parametrize("B,H,T,d,C", [
    (1, 1, 8, 2, 4), (1, 1, 7, 2, 4), (4, 8, 1024, 64, 64), (1, 16, 8192, 128, 64),
    (1, 32, 131072, 128, 128), (256, 32, 4096, 128, 64), (3, 5, 1000, 33, 17), (1, 1, 1, 1, 1),
    (2, 3, 1000, 64, 101), (1, 16, 8192, 128, 100), (1, 2, 70, 16, 65), (4, 8, 1024, 64, 128),
    (1, 16, 2048, 64, 64), (1, 16, 4096, 64, 64), (1, 8, 4096, 64, 64), (1, 12, 2048, 64, 64),
])
def test_segments_cover_the_sequence(lib, B, H, T, d, C):
    G = lib.lla_prefill_segment_chunks(B, H, T, d, d, C)
    ws = lib.lla_prefill_workspace_size(B, H, T, d, d, C)
    c = C if C <= 64 else (C + 1) // 2  # the chunk the library runs
    n_c = math.ceil(T / c)
    assert 1 <= G <= n_c
    n_seg = math.ceil(n_c / G)
    assert ws == _expected_workspace(B, H, n_seg, G, d)
    G_C = _lines_rule_G(B, H, T, C)
    n_seg_C = math.ceil(math.ceil(T / C) / G_C)
    if C <= 64:
        assert G == G_C
    else:
        # two sub-chunks per chunk of C, twice as many per segment: never more
        # segments than the plan for C, and for an even C the same tokens
        assert G == min(2 * G_C, n_c)
        assert n_seg <= n_seg_C
        if C % 2 == 0:
            assert n_seg == n_seg_C and (n_seg == 1 or G * c == G_C * C)
    # about one line per compute unit, without one per chunk: more than half
    # of 256 lines (or one per chunk)
    lines = n_seg_C * B * H
    assert lines >= min(math.ceil(T / C) * B * H, 129)


def test_segment_plan_for_the_t8192_workload(lib):
    # 128 chunks x 16 heads = 2048 chunk lines: 256 eight-wave walk workgroups of 8 chunks;
    # chunks of 128 run as two of 64: the same 16 segments, of 8 chunks of 64
    assert lib.lla_prefill_segment_chunks(1, 16, 8192, 128, 128, 128) == 8
    assert lib.lla_prefill_segment_chunks(1, 16, 8192, 128, 128, 64) == 8
    assert lib.lla_prefill_workspace_size(1, 16, 8192, 128, 128, 64) == 16 * 16 * 128 * 128 * 4


def test_size_bounds(lib):
    """B*H <= 2^20 and B*H*T*max(dk,dv) <= 2^58: beyond either, every call
    reports a shape error (and the planners 0) before touching anything."""
    b = Bufs(B=1 << 10, H=1 << 10, T=100)
    assert lib.lla_prefill_segment_chunks(1 << 10, 1 << 10, 100, 64, 64, 64) > 0
    b.H = (1 << 10) + 1
    assert lib.lla_prefill(*b.args()) == E_SHAPE
    assert lib.lla_prefill_segment_chunks(1 << 10, (1 << 10) + 1, 100, 64, 64, 64) == 0
    assert lib.lla_decode_step(A, 2 * A, 3 * A, BF16, 1 << 10, (1 << 10) + 1, 64, 64, 4 * A, 5 * A,
                               None) == E_SHAPE
    assert lib.lla_state_init(A, 1 << 21, 1, 4, 4, None) == E_SHAPE
    # the element bound: 2^58 / (16 heads x 128) tokens is the largest T
    T_max = (1 << 58) // (16 * 128)
    assert lib.lla_prefill_segment_chunks(1, 16, T_max, 128, 128, 64) > 0
    assert lib.lla_prefill_segment_chunks(1, 16, T_max + 1, 128, 128, 64) == 0
    b = Bufs(B=1, H=16, T=T_max + 1, dk=128, dv=128)
    assert lib.lla_prefill(*b.args()) == E_SHAPE


def test_plan_rejects_bad_sizes(lib):
    assert lib.lla_prefill_segment_chunks(1, 1, 8, 2, 2, 0) == 0
    assert lib.lla_prefill_workspace_size(0, 1, 8, 2, 2, 4) == 0


def test_python_binding_raises_without_touching_the_gpu():
    import torch
    q = torch.zeros((1, 1, 8, 2), dtype=torch.bfloat16)
    S = torch.zeros((1, 1, 2, 2), dtype=torch.float32)
    with pytest.raises((lla.LlaError, ValueError, RuntimeError)):
        lla.prefill(q, q, q, S, chunk=4)  # CPU tensors are refused


# ---- shared-state heads (Hq query heads on Hkv key/value heads) --------------------

def _gqa_args(b, Hq, Hkv):
    return (b.q, b.k, b.v, b.dtype, b.B, Hq, Hkv, b.T, b.dk, b.dv, b.C, b.S, b.O, b.ws,
            b.ws_bytes, None)


@pytest.mark.parametrize("Hq,Hkv", [(4, 0), (4, 3), (2, 4), (0, 0), (6, -2)])
def test_prefill_gqa_rejects_head_counts(lib, Hq, Hkv):
    assert lib.lla_prefill_gqa(*_gqa_args(Bufs(), Hq, Hkv)) == E_SHAPE
    assert lib.lla_prefill_gqa_workspace_size(1, Hq, Hkv, 100, 64, 64, 64) == 0


@pytest.mark.parametrize("change,expect", [
    (dict(q=None), E_NULL), (dict(S=None), E_NULL), (dict(dtype=7), E_DTYPE),
    (dict(k=2 * A + 4), E_ALIGN), (dict(T=8192, ws=None), E_WS),
])
def test_prefill_gqa_checks_like_prefill(lib, change, expect):
    b = Bufs()
    for key, val in change.items():
        setattr(b, key, val)
    assert lib.lla_prefill_gqa(*_gqa_args(b, 8, 2)) == expect


def test_prefill_gqa_spans_use_their_own_head_counts(lib):
    # Q and O span Hq heads, K, V and S span Hkv: with 8 query heads on 2
    # key/value heads (T = 100, dk = dv = 64, bf16), K ends at 2*A + 2*100*64*2.
    b = Bufs()
    kv_bytes = 2 * 100 * 64 * 2
    b.O = 2 * A + kv_bytes - 64  # inside K
    assert lib.lla_prefill_gqa(*_gqa_args(b, 8, 2)) == E_ALIAS
    b = Bufs()
    b.S = 3 * A + 2 * 100 * 64 * 2 - 16  # S starts inside V
    assert lib.lla_prefill_gqa(*_gqa_args(b, 8, 2)) == E_ALIAS


def test_prefill_gqa_workspace(lib):
    # a group of one is the plain call
    for args in [(1, 16, 8192, 128, 128, 64), (3, 5, 1000, 33, 33, 17), (2, 4, 10, 64, 64, 64)]:
        B, H = args[0], args[1]
        assert lib.lla_prefill_gqa_workspace_size(B, H, H, *args[2:]) == \
            lib.lla_prefill_workspace_size(*args)
    # groups always stage the start states in the workspace: one state per
    # key/value head per segment, even for a single segment
    assert lib.lla_prefill_gqa_workspace_size(2, 8, 2, 10, 64, 64, 64) == 2 * 2 * 64 * 64 * 4
    ws = lib.lla_prefill_gqa_workspace_size(1, 16, 4, 8192, 128, 128, 64)
    assert ws == 4 * 16 * 128 * 128 * 4  # the T=8192 plan: 16 segments of 8 chunks


@pytest.mark.parametrize("change,expect", [
    (dict(Hkv=0), E_SHAPE), (dict(Hq=6, Hkv=4), E_SHAPE), (dict(Hq=2, Hkv=4), E_SHAPE),
    (dict(Hq=17, Hkv=1, q=None), E_NULL), (dict(dk=96, dv=96, q=None), E_NULL),
    (dict(dk=64, dv=7, q=None), E_NULL), (dict(q=None), E_NULL), (dict(dtype=5), E_DTYPE), (dict(o=2 * A + 256), E_ALIAS),
])
def test_decode_gqa_rejects(lib, change, expect):
    d = dict(q=A, k=2 * A, v=3 * A, dtype=BF16, B=2, Hq=8, Hkv=2, dk=128, dv=128, S=4 * A, o=5 * A)
    d.update(change)
    assert lib.lla_decode_step_gqa(d["q"], d["k"], d["v"], d["dtype"], d["B"], d["Hq"], d["Hkv"],
                                   d["dk"], d["dv"], d["S"], d["o"], None) == expect


def test_python_binding_checks_grouped_shapes():
    import torch
    q = torch.zeros((1, 6, 8, 4), dtype=torch.bfloat16)
    k = torch.zeros((1, 4, 8, 4), dtype=torch.bfloat16)
    S = torch.zeros((1, 4, 4, 4), dtype=torch.float32)
    with pytest.raises(ValueError):
        lla.prefill(q, k, k, S, chunk=4)  # 6 query heads cannot share 4 key/value heads
    with pytest.raises(ValueError):
        lla.decode_step(q[:, :, 0], k[:, :, 0], k[:, :, 0], S)


# ---- lla_prefill_ex -------------------------------------------------------------

ZERO_STATE = 1


def _ex_args(b, Hq, Hkv, flags):
    return (b.q, b.k, b.v, b.dtype, b.B, Hq, Hkv, b.T, b.dk, b.dv, b.C, flags, b.S, b.O, b.ws,
            b.ws_bytes, None)


@pytest.mark.parametrize("flags", [4, 8, 0x80000000, 5])
def test_prefill_ex_rejects_unknown_flags(lib, flags):
    assert lib.lla_prefill_ex(*_ex_args(Bufs(), 2, 2, flags)) == E_UNSUP


KEEP_STATE = 2


@pytest.mark.parametrize("change", [dict(T=17), dict(dk=96, dv=96), dict(dk=64, dv=128), dict(T=16, H=8)])
@pytest.mark.parametrize("flags", [KEEP_STATE, KEEP_STATE | ZERO_STATE])
def test_keep_state_is_checked_like_any_prefill_off_the_fused_route(lib, change, flags):
    # a verify pass off the fused short-prompt route (T > 16, other head
    # dims, T * G > 64) takes the chunked path: the usual checks decide
    # (here a NULL q), nothing refuses the option
    b = Bufs(T=4, dk=128, dv=128)
    Hq, Hkv = (32, 4) if "H" in change else (2, 2)  # T * G = 16 * 8 = 128 > 64
    for key, val in change.items():
        if key != "H":
            setattr(b, key, val)
    b.q = None
    assert lib.lla_prefill_ex(*_ex_args(b, Hq, Hkv, flags)) == E_NULL
    assert lib.lla_prefill_noalloc(*_noalloc_args(b, Hq, Hkv, flags)) == E_NULL


def test_keep_state_with_an_empty_prompt_is_a_noop(lib):
    b = Bufs(T=0)
    b.q = b.k = b.v = b.O = None
    assert lib.lla_prefill_ex(*_ex_args(b, 2, 2, KEEP_STATE | ZERO_STATE)) == OK


@pytest.mark.parametrize("change,expect", [
    (dict(q=None), E_NULL), (dict(S=None), E_NULL), (dict(B=0), E_SHAPE), (dict(dtype=7), E_DTYPE),
    (dict(O=5 * A + 4), E_ALIGN), (dict(O=A + 64), E_ALIAS), (dict(T=8192, ws=None), E_WS),
])
@pytest.mark.parametrize("flags", [0, ZERO_STATE])
def test_prefill_ex_checks_like_prefill(lib, change, expect, flags):
    b = Bufs()
    for key, val in change.items():
        setattr(b, key, val)
    assert lib.lla_prefill_ex(*_ex_args(b, 2, 2, flags)) == expect
    assert lib.lla_prefill(*b.args()) == expect


def test_prefill_ex_head_counts(lib):
    assert lib.lla_prefill_ex(*_ex_args(Bufs(), 4, 3, ZERO_STATE)) == E_SHAPE


# lla_prefill_noalloc: the checks of lla_prefill_ex (no workspace argument),
# then the workspace the shape needs against the library's static array.
def _noalloc_args(b, Hq, Hkv, flags):
    return (b.q, b.k, b.v, b.dtype, b.B, Hq, Hkv, b.T, b.dk, b.dv, b.C, flags, b.S, b.O, None)


def _scratch_bytes():
    text = open(HEADER).read()
    m = re.search(r"#define LLA_NOALLOC_SCRATCH_BYTES \((\d+)u \* 1024u \* 1024u\)", text)
    return int(m.group(1)) << 20


@pytest.mark.parametrize("change,expect", [
    (dict(q=None), E_NULL), (dict(S=None), E_NULL), (dict(B=0), E_SHAPE), (dict(dtype=7), E_DTYPE),
    (dict(O=5 * A + 4), E_ALIGN), (dict(O=A + 64), E_ALIAS), (dict(dtype=F32, C=128, q=None), E_NULL),
])
@pytest.mark.parametrize("flags", [0, ZERO_STATE])
def test_prefill_noalloc_checks_like_prefill_ex(lib, change, expect, flags):
    b = Bufs()
    for key, val in change.items():
        setattr(b, key, val)
    assert lib.lla_prefill_noalloc(*_noalloc_args(b, 2, 2, flags)) == expect
    assert lib.lla_prefill_ex(*_ex_args(b, 2, 2, flags)) == expect


def test_prefill_noalloc_rejects_unknown_flags(lib):
    assert lib.lla_prefill_noalloc(*_noalloc_args(Bufs(), 2, 2, 4)) == E_UNSUP


def test_prefill_noalloc_rejects_a_workspace_beyond_the_static_array(lib):
    # 5 x 128 key/value heads, one 64 KiB state each (grouped heads start from
    # the workspace): 40 MiB, beyond the 32 MiB array; refused before any HIP call
    b = Bufs(B=5, T=64, dk=128, dv=128)
    need = lib.lla_prefill_gqa_workspace_size(5, 256, 128, 64, 128, 128, 64)
    assert need > _scratch_bytes() == 32 << 20
    assert lib.lla_prefill_noalloc(*_noalloc_args(b, 256, 128, 0)) == E_SCRATCH
    assert lib.lla_prefill_noalloc(*_noalloc_args(b, 256, 128, ZERO_STATE)) == E_SCRATCH


def test_every_multi_head_shape_fits_the_static_array(lib):
    """With one query head per key/value head the plan keeps about 512 / n_vb
    segment states in all, so the largest workspace stays below the array: a
    scan over head counts and lengths at d = 128 and d = 64."""
    worst = 0
    for BH in (1, 2, 3, 5, 8, 16, 31, 64, 100, 128, 200, 255, 256, 300, 511, 512, 1000):
        for T in (1, 64, 65, 200, 1000, 4096, 8192, 65536, 131072):
            for d in (64, 128):
                for C in (32, 64, 128):
                    worst = max(worst, lib.lla_prefill_workspace_size(1, BH, T, d, d, C))
    assert 0 < worst <= _scratch_bytes()


# lla_state_commit: the commit after a verify pass
@pytest.mark.parametrize("change,expect", [
    (dict(S=None), E_NULL), (dict(k=None), E_NULL), (dict(v=None), E_NULL),
    (dict(B=0), E_SHAPE), (dict(H=0), E_SHAPE), (dict(T=-1), E_SHAPE), (dict(dk=129), E_SHAPE),
    (dict(dtype=9), E_DTYPE), (dict(S=4 * A + 4), E_ALIGN), (dict(acc=6 * A + 4), E_ALIGN),
    (dict(S=A + 64), E_ALIAS), (dict(acc=4 * A + 64), E_ALIAS),
    (dict(T=0, k=None, v=None), OK),
])
def test_state_commit_rejects(lib, change, expect):
    d = dict(k=A, v=2 * A, dtype=BF16, B=2, H=4, T=4, dk=128, dv=128, acc=6 * A, S=4 * A)
    d.update(change)
    assert lib.lla_state_commit(d["k"], d["v"], d["dtype"], d["B"], d["H"], d["T"], d["dk"], d["dv"],
                                d["acc"], d["S"], None) == expect


def test_missing_library_fails_loudly(tmp_path):
    """No fallback: without the HIP library every entry point raises instead
    of computing anything elsewhere."""
    import subprocess
    import sys
    code = ("import decode_lla_prefill_amd as lla\n"
            "try:\n"
            "    lla.library()\n"
            "except ImportError as e:\n"
            "    print('raised', e)\n"
            "else:\n"
            "    print('loaded')\n")
    env = dict(os.environ, LLA_LIBRARY=str(tmp_path / "absent" / "liblla.so"))
    repo = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=repo, env=env, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.startswith("raised") and "not built" in out.stdout
