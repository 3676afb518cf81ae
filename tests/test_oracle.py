"""Pins for the CPU oracle (no GPU).

Each test ties the oracle to something other than itself:
* values the slide deck "Chunking, causality, and parallel prefill" prints
  (fixtures under tests/golden/, each naming its section);
* closed forms: O = tril(Q K^T) V + Q S_0 and S_T = S_0 + K^T V, evaluated as
  dense float64 matrix products (a different formula from the recurrence);
* brute force on tiny inputs (explicit double sums over every (s <= t) pair);
* invariants the deck states (chunking is exact; prefill and decode agree;
  the state is one fixed-size object handed between blocks).
The planted mistakes (the deck's two bugs) are planted in the oracle, on the
CPU, and must produce the wrong values the deck prints.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _trace():
    g = _golden("trace_c4.json")
    k = np.array(g["k"], dtype=np.float64)
    v = np.array(g["v"], dtype=np.float64)
    return g, k.copy(), k, v  # q_t = k_t in the deck's trace


# --- the deck's printed values ----------------------------------------------

def test_trace_recurrence_matches_printed_values():
    g, q, k, v = _trace()
    O, S8, ck = oracle.recurrence(q, k, v, ckpt_every=4)
    assert np.array_equal(O[:4], np.array(g["o_1_to_4"]))
    assert np.array_equal(O[4:], np.array(g["o_5_to_8"]))
    assert np.array_equal(ck[0], np.array(g["S_4"]))
    assert np.array_equal(S8, np.array(g["S_8"]))


def test_trace_chunked_matches_printed_values():
    g, q, k, v = _trace()
    O, S8, handoffs, masks = oracle.chunked(q, k, v, C=4)
    assert np.array_equal(masks[0], np.array(g["chunk1_masked_scores"]))
    assert np.array_equal(O[:4], np.array(g["o_1_to_4"]))
    assert np.array_equal(O[4:], np.array(g["o_5_to_8"]))
    assert len(handoffs) == 1 and np.array_equal(handoffs[0], np.array(g["S_4"]))
    assert np.array_equal(S8, np.array(g["S_8"]))
    # o_5 = [3,4] (inherited through S_4) + [0,1] (local): the inter-chunk
    # term of tokens 5 and 6 alone.
    inter = oracle.incoming_term(q[4:6], handoffs[0])
    assert np.array_equal(inter, np.array(g["inter_chunk_term_q5_q6"]))


def test_transfer_challenge_c2():
    g = _golden("transfer_c2.json")
    _, q, k, v = _trace()
    O, S8, handoffs, _ = oracle.chunked(q, k, v, C=2)
    assert len(handoffs) == g["handoffs"]
    for got, key in zip(handoffs, ("S_2", "S_4", "S_6")):
        assert np.array_equal(got, np.array(g[key]))
    assert np.array_equal(O[4:], np.array(g["o_5_to_8"]))
    # the recurrence's own states at the same positions
    _, _, ck = oracle.recurrence(q, k, v, ckpt_every=2)
    for c, key in enumerate(("S_2", "S_4", "S_6")):
        assert np.array_equal(ck[c], np.array(g[key]))
    # the chunk-size table: 8/C transitions, C^2 triangle cells
    for C_str, n in g["transitions_by_chunk_size"].items():
        C = int(C_str)
        _, _, h, m = oracle.chunked(q, k, v, C=C)
        assert len(h) + 1 == n
        assert m[0].size == g["triangle_cells_by_chunk_size"][C_str]
        # every chunk hands on a state of the same d x d size
        assert all(s.shape == (2, 2) for s in h)


def test_bug1_dropping_incoming_state(monkeypatch):
    """Deck, 'Worked case', bug 1: without the incoming term o_5 = v_5 = [0,1]."""
    g, q, k, v = _trace()
    monkeypatch.setattr(oracle, "incoming_term", lambda Qc, S: np.zeros((Qc.shape[0], S.shape[1])))
    O, _, _, _ = oracle.chunked(q, k, v, C=4)
    assert np.array_equal(O[4], np.array(g["bug1_drop_incoming_state_o5"]))
    assert not np.array_equal(O[4:], np.array(g["o_5_to_8"]))


def test_bug2_full_mask(monkeypatch):
    """Deck, 'Worked case', bug 2: a full mask lets t5 read t7: o_5 = [4,5]."""
    g, q, k, v = _trace()
    monkeypatch.setattr(oracle, "causal_mask", lambda A: A)
    O, _, _, _ = oracle.chunked(q, k, v, C=4)
    assert np.array_equal(O[4], np.array(g["bug2_full_mask_o5"]))
    assert not np.array_equal(O[4:], np.array(g["o_5_to_8"]))


def test_mask_question_computed_zero_vs_masked_cell():
    """Deck, 'Causal triangle' check: with k3.k4 = 1, cell (4,3) becomes 1
    while cell (3,4) stays masked."""
    _, q, k, v = _trace()
    k = k.copy()
    k[3] = [1, 1]  # k3 = [1,0], so k3.k4 = 1
    q = k.copy()
    _, _, _, masks = oracle.chunked(q, k, v, C=4)
    assert masks[0][3, 2] == 1.0      # row 4, column 3 (1-based)
    assert masks[0][2, 3] == 0.0      # row 3, column 4 stays masked


# --- closed forms and brute force ---------------------------------------------

def _rand(shape, rng):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("BH,T,dk,dv", [(1, 1, 1, 1), (3, 17, 5, 7), (2, 64, 16, 8), (2, 200, 9, 33)])
def test_recurrence_vs_closed_form(BH, T, dk, dv):
    rng = np.random.default_rng(1000 + T)
    q, k, v = _rand((BH, T, dk), rng), _rand((BH, T, dk), rng), _rand((BH, T, dv), rng)
    S0 = _rand((BH, dk, dv), rng)
    O, ST = oracle.recurrence(q, k, v, S0, nthreads=2)
    for b in range(BH):
        O_ref = np.tril(q[b] @ k[b].T) @ v[b] + q[b] @ S0[b]
        S_ref = S0[b] + k[b].T @ v[b]
        scale = np.abs(O_ref).max()
        assert np.abs(O[b] - O_ref).max() <= 1e-12 * max(scale, 1) * T
        assert np.abs(ST[b] - S_ref).max() <= 1e-12 * max(np.abs(S_ref).max(), 1) * T


def test_recurrence_vs_brute_force_sums():
    """o_t[j] = sum_{s<=t} (q_t . k_s) v_s[j] + sum_i q_t[i] S0[i][j], as loops."""
    rng = np.random.default_rng(7)
    T, dk, dv = 6, 3, 4
    q, k, v = _rand((T, dk), rng), _rand((T, dk), rng), _rand((T, dv), rng)
    S0 = _rand((dk, dv), rng)
    O, ST = oracle.recurrence(q, k, v, S0)
    for t in range(T):
        for j in range(dv):
            acc = 0.0
            for s in range(t + 1):
                acc += sum(q[t, i] * k[s, i] for i in range(dk)) * v[s, j]
            acc += sum(q[t, i] * S0[i, j] for i in range(dk))
            assert abs(O[t, j] - acc) <= 1e-12 * (1 + abs(acc))
    for i, j in itertools.product(range(dk), range(dv)):
        ref = S0[i, j] + sum(k[s, i] * v[s, j] for s in range(T))
        assert abs(ST[i, j] - ref) <= 1e-12 * (1 + abs(ref))


def test_integer_inputs_are_exact():
    q, k, v = workloads.integers(2, 3, 150, 12, 10, seed=3)
    O, ST = oracle.recurrence(q, k, v)
    qn, kn, vn = (x.double().numpy() for x in (q, k, v))
    O_ref = np.tril(qn @ np.swapaxes(kn, -1, -2)) @ vn
    S_ref = np.swapaxes(kn, -1, -2) @ vn
    assert np.array_equal(O, O_ref)
    assert np.array_equal(ST, S_ref)


@pytest.mark.parametrize("variant", range(1, 101))
def test_toy_variants_exact(variant):
    q, k, v = workloads.toy(variant)
    O, ST = oracle.recurrence(q, k, v)
    qn, kn, vn = (x.double().numpy()[0, 0] for x in (q, k, v))
    assert np.array_equal(O[0, 0], np.tril(qn @ kn.T) @ vn)
    assert np.array_equal(ST[0, 0], kn.T @ vn)
    Oc, Sc, _, _ = oracle.chunked(qn, kn, vn, C=4)
    assert np.array_equal(Oc, O[0, 0]) and np.array_equal(Sc, ST[0, 0])


# --- invariants -------------------------------------------------------------------

def test_chunking_is_exact_for_every_chunk_size():
    """Deck, 'Common errors': chunking reorders the sums exactly, so the chunk
    size changes only the cost (integer inputs: exact equality for every C)."""
    q, k, v = workloads.integers(1, 1, 37, 6, 5, seed=11)
    qn, kn, vn = (x.double().numpy()[0, 0] for x in (q, k, v))
    O_rec, S_rec = oracle.recurrence(qn, kn, vn)
    for C in list(range(1, 12)) + [16, 36, 37, 64]:
        O, S, h, _ = oracle.chunked(qn, kn, vn, C=C)
        assert np.array_equal(O, O_rec), C
        assert np.array_equal(S, S_rec), C
        assert len(h) == (37 + C - 1) // C - 1


def test_chunk_size_one_is_the_recurrence_and_full_chunk_is_one_triangle():
    rng = np.random.default_rng(5)
    q, k, v = _rand((20, 4), rng), _rand((20, 4), rng), _rand((20, 3), rng)
    O_rec, _ = oracle.recurrence(q, k, v)
    O1, _, _, _ = oracle.chunked(q, k, v, C=1)
    OT, _, h, _ = oracle.chunked(q, k, v, C=20)
    assert np.allclose(O1, O_rec, rtol=0, atol=1e-12)
    assert np.allclose(OT, np.tril(q @ k.T) @ v, rtol=0, atol=1e-12) and h == []


def test_decode_is_one_recurrence_step_and_continues_prefill():
    """Deck, 'Prefill and decode': the two code paths give the same numbers."""
    q, k, v = workloads.integers(2, 2, 30, 8, 6, seed=21)
    O_all, S_all = oracle.recurrence(q, k, v)
    O_pre, S = oracle.recurrence(q[:, :, :25], k[:, :, :25], v[:, :, :25])
    assert np.array_equal(O_pre, O_all[:, :, :25])
    for t in range(25, 30):
        o, S = oracle.decode_step(q[:, :, t], k[:, :, t], v[:, :, t], S)
        assert np.array_equal(o, O_all[:, :, t])
    assert np.array_equal(S, S_all)


def test_continuation_prefill_then_prefill():
    """The state is the one object handed between blocks: prefill(T1) then
    prefill(T2) from its state equals prefill(T1 + T2)."""
    q, k, v = workloads.integers(1, 3, 50, 7, 9, seed=31)
    O_all, S_all = oracle.recurrence(q, k, v)
    O1, S1 = oracle.recurrence(q[:, :, :19], k[:, :, :19], v[:, :, :19])
    O2, S2 = oracle.recurrence(q[:, :, 19:], k[:, :, 19:], v[:, :, 19:], S1)
    assert np.array_equal(np.concatenate([O1, O2], axis=2), O_all)
    assert np.array_equal(S2, S_all)


def test_checkpoints_are_prefix_states_and_threads_do_not_matter():
    q, k, v = workloads.integers(3, 2, 40, 5, 4, seed=41)
    O1, S1, ck = oracle.recurrence(q, k, v, ckpt_every=8, nthreads=1)
    O4, S4, ck4 = oracle.recurrence(q, k, v, ckpt_every=8, nthreads=4)
    assert np.array_equal(O1, O4) and np.array_equal(S1, S4) and np.array_equal(ck, ck4)
    kn, vn = k.double().numpy(), v.double().numpy()
    for c in range(5):
        t = 8 * (c + 1)
        ref = np.swapaxes(kn[:, :, :t], -1, -2) @ vn[:, :, :t]
        assert np.array_equal(ck[:, :, c], ref)


def test_empty_prompt_keeps_state():
    S0 = np.arange(6, dtype=np.float64).reshape(1, 2, 3)
    O, S = oracle.recurrence(np.zeros((1, 0, 2)), np.zeros((1, 0, 2)), np.zeros((1, 0, 3)), S0)
    assert O.shape == (1, 0, 3) and np.array_equal(S, S0)


def test_bf16_inputs_are_upcast_exactly():
    x = torch.tensor([[1.0 + 2 ** -7, -3.0, 2 ** -20]], dtype=torch.bfloat16).view(1, 1, 3)
    q = x
    k = torch.ones(1, 1, 3, dtype=torch.bfloat16)
    v = torch.ones(1, 1, 1, dtype=torch.bfloat16)
    O, _ = oracle.recurrence(q, k, v)
    assert O[0, 0, 0] == (1.0 + 2 ** -7) - 3.0 + 2 ** -20


# --- shared-state heads (grouped query heads) -----------------------------------
# Blog "A 128 000 tokens, l'attention avale 85 % du calcul", section on sharing
# heads: G query heads read one key/value head.  Query head h uses key/value
# head h // G.

def _grouped_brute_force(q, k, v, S0):
    """o[b,h,t,j] = sum_{s<=t} (q_t . k_s) v_s[j] + sum_i q_t[i] S0[i][j] over the
    key/value head h // G, as explicit loops; S_T[b,g] = S0 + sum_s k_s v_s^T."""
    B, Hq, T, dk = q.shape
    Hkv, dv = k.shape[1], v.shape[3]
    G = Hq // Hkv
    O = np.zeros((B, Hq, T, dv))
    for b, h, t, j in itertools.product(range(B), range(Hq), range(T), range(dv)):
        g = h // G
        acc = 0.0
        for s in range(t + 1):
            acc += sum(q[b, h, t, i] * k[b, g, s, i] for i in range(dk)) * v[b, g, s, j]
        acc += sum(q[b, h, t, i] * S0[b, g, i, j] for i in range(dk))
        O[b, h, t, j] = acc
    S = np.zeros((B, Hkv, dk, dv))
    for b, g, i, j in itertools.product(range(B), range(Hkv), range(dk), range(dv)):
        S[b, g, i, j] = S0[b, g, i, j] + sum(k[b, g, s, i] * v[b, g, s, j] for s in range(T))
    return O, S


@pytest.mark.parametrize("Hq,Hkv", [(6, 2), (4, 1), (3, 3), (4, 2)])
def test_grouped_recurrence_vs_brute_force(Hq, Hkv):
    rng = np.random.default_rng(50 + 10 * Hq + Hkv)
    B, T, dk, dv = 2, 5, 3, 2
    q, k, v = _rand((B, Hq, T, dk), rng), _rand((B, Hkv, T, dk), rng), _rand((B, Hkv, T, dv), rng)
    S0 = _rand((B, Hkv, dk, dv), rng)
    O, S = oracle.grouped_recurrence(q, k, v, S0)
    O_ref, S_ref = _grouped_brute_force(q, k, v, S0)
    assert O.shape == (B, Hq, T, dv) and S.shape == (B, Hkv, dk, dv)
    assert np.abs(O - O_ref).max() <= 1e-12 * (1 + np.abs(O_ref).max())
    assert np.abs(S - S_ref).max() <= 1e-12 * (1 + np.abs(S_ref).max())


def test_grouped_recurrence_closed_form_integers():
    """Per query head h: O = tril(Q_h K_g^T) V_g + Q_h S0_g with g = h // G, exact
    on integer inputs (dense products, a different formula from the loop)."""
    B, Hq, Hkv, T, dk, dv = 2, 8, 2, 70, 6, 5
    G = Hq // Hkv
    q, _, _ = workloads.integers(B, Hq, T, dk, dv, seed=61)
    _, k, v = workloads.integers(B, Hkv, T, dk, dv, seed=62)
    S0 = np.random.default_rng(63).integers(-50, 51, (B, Hkv, dk, dv)).astype(np.float64)
    O, S = oracle.grouped_recurrence(q, k, v, S0)
    qn, kn, vn = (x.double().numpy() for x in (q, k, v))
    for b, h in itertools.product(range(B), range(Hq)):
        g = h // G
        assert np.array_equal(O[b, h], np.tril(qn[b, h] @ kn[b, g].T) @ vn[b, g] + qn[b, h] @ S0[b, g])
    assert np.array_equal(S, S0 + np.swapaxes(kn, -1, -2) @ vn)


def test_grouped_mapping_mistake_is_caught(monkeypatch):
    """Planted in the oracle: pairing query head h with key/value head h % Hkv
    (tiling the heads instead of repeating each one) must fail the closed form."""
    B, Hq, Hkv, T, d = 1, 4, 2, 6, 3
    q, _, _ = workloads.integers(B, Hq, T, d, d, seed=71)
    _, k, v = workloads.integers(B, Hkv, T, d, d, seed=72)
    qn, kn, vn = (x.double().numpy() for x in (q, k, v))
    ref = np.stack([np.tril(qn[0, h] @ kn[0, h // 2].T) @ vn[0, h // 2] for h in range(Hq)])
    O, _ = oracle.grouped_recurrence(q, k, v)
    assert np.array_equal(O[0], ref)
    monkeypatch.setattr(oracle.np, "repeat", lambda a, G, axis: np.concatenate([a] * G, axis=axis))
    O_bad, _ = oracle.grouped_recurrence(q, k, v)
    assert not np.array_equal(O_bad[0], ref)


def test_group_of_one_is_the_recurrence_and_state_ignores_queries():
    q, k, v = workloads.integers(2, 3, 40, 7, 5, seed=81)
    S0 = np.random.default_rng(82).integers(-9, 10, (2, 3, 7, 5)).astype(np.float64)
    O1, S1 = oracle.grouped_recurrence(q, k, v, S0)
    O_ref, S_ref = oracle.recurrence(q, k, v, S0)
    assert np.array_equal(O1, O_ref) and np.array_equal(S1, S_ref)
    # with groups of 3 the state is the key/value heads' own recurrence state
    q3, _, _ = workloads.integers(2, 9, 40, 7, 5, seed=83)
    _, S3 = oracle.grouped_recurrence(q3, k, v, S0)
    assert np.array_equal(S3, S_ref)


def test_grouped_decode_continues_grouped_prefill():
    B, Hq, Hkv, T, dk, dv = 2, 6, 2, 24, 8, 4
    q, _, _ = workloads.integers(B, Hq, T, dk, dv, seed=91)
    _, k, v = workloads.integers(B, Hkv, T, dk, dv, seed=92)
    O_all, S_all = oracle.grouped_recurrence(q, k, v)
    O_pre, S = oracle.grouped_recurrence(q[:, :, :20], k[:, :, :20], v[:, :, :20])
    assert np.array_equal(O_pre, O_all[:, :, :20])
    for t in range(20, T):
        o, S = oracle.grouped_decode_step(q[:, :, t], k[:, :, t], v[:, :, t], S)
        assert np.array_equal(o, O_all[:, :, t])
    assert np.array_equal(S, S_all)


def test_grouped_rejects_bad_head_counts():
    z = np.zeros
    with pytest.raises(ValueError):
        oracle.grouped_recurrence(z((1, 5, 2, 3)), z((1, 2, 2, 3)), z((1, 2, 2, 3)))
    with pytest.raises(ValueError):
        oracle.grouped_decode_step(z((1, 2, 3)), z((1, 4, 3)), z((1, 4, 3)), z((1, 4, 3, 3)))


# --- FP8 (E4M3) inputs: the oracle's decoder ---------------------------------------

def test_e4m3_decoder_special_codes():
    """Values the OCP E4M3 definition fixes: 1.0, -2.0, the largest finite value
    448, the smallest normal 2^-6, the smallest subnormal 2^-9, the largest
    subnormal 7/8 * 2^-6, signed zeros and the two NaN codes."""
    d = oracle.decode_e4m3(np.arange(256))
    assert d[0x38] == 1.0 and d[0xC0] == -2.0
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0
    assert d[0x08] == 2.0 ** -6 and d[0x01] == 2.0 ** -9 and d[0x07] == 7 / 8 * 2.0 ** -6
    assert d[0x00] == 0.0 and not np.signbit(d[0x00]) and d[0x80] == 0.0 and np.signbit(d[0x80])
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF]) and np.isnan(d).sum() == 2
    assert np.all(np.diff(d[:0x7F]) > 0)  # positive codes are ordered
    assert np.array_equal(d[0x80:0xFF], -d[:0x7F])


def test_e4m3_decoder_matches_torch_and_fits_bf16():
    """Every code decodes as torch's float8_e4m3fn does, and every finite value
    is exactly a bf16 value (so FP8 inputs may be staged as bf16)."""
    codes = torch.arange(256, dtype=torch.uint8)
    d = oracle.decode_e4m3(codes.numpy())
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(d, ref, equal_nan=True)
    fin = d[np.isfinite(d)]
    assert np.array_equal(torch.tensor(fin).to(torch.bfloat16).double().numpy(), fin)
    # FP8 tensors enter the oracle through the same decoder
    t = torch.randn(2, 3, 7).to(torch.float8_e4m3fn)
    O, _ = oracle.recurrence(t, t, t)
    tb = t.to(torch.bfloat16)
    O_b, _ = oracle.recurrence(tb, tb, tb)
    assert np.array_equal(O, O_b)


def test_e4m3_wrong_bias_is_caught():
    """Planted: an exponent bias of 8 (the other 8-bit E4M3 variant) fails the
    fixed values above."""
    b = np.arange(256)
    e = (b >> 3) & 0xF
    m = b & 7
    wrong = np.where(e == 0, m / 8 * 2.0 ** -7, (1 + m / 8) * np.exp2(e - 8.0))
    assert wrong[0x38] != 1.0 and oracle.decode_e4m3(b)[0x38] == 1.0
