"""Pins for the gated (decayed) oracle (no GPU).

Reading taken (the pages cite the chunkwise form of gated linear attention,
deck "Chunking, causality, and parallel prefill", section "Boundary, evidence,
and sources", but state no gate): one scalar gate g_t per stream and token,

    S_t = g_t S_{t-1} + k_t v_t^T,    o_t = S_t^T q_t.

Each test ties oracle.gated_recurrence / gated_decode_step to something other
than themselves:
* g = 1 reproduces the deck's printed trace ("Worked case - full trace");
* the closed form, evaluated as dense float64 matrix products:
      O   = (tril(Q K^T) * D) V + diag(c) Q S_0,   D[t][s] = prod_{s < l <= t} g_l,
      S_T = c_T S_0 + sum_s D[T][s] k_s v_s^T,      c_t = prod_{l <= t} g_l;
* g = 0 forgets everything before the token: o_t = (q_t . k_t) v_t;
* brute force on tiny inputs (explicit sums over every s <= t);
* a planted mistake -- the gate applied after the update, S_t = g_t (S_{t-1}
  + k_t v_t^T) -- fails the closed form.
With shared-state heads (each key/value head's state and gates read by the
G query heads of its group): brute force with the explicit head mapping,
g = 1 equal to the ungated grouped oracle bit for bit, the decode step as one
token of the recurrence, and a planted h % Hkv mapping that fails.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _closed_form(q, k, v, g, S0):
    """One stream: q, k [T, dk], v [T, dv], g [T], S0 [dk, dv]."""
    T = q.shape[0]
    logc = np.cumsum(np.log(g))                      # log c_t (g > 0 here)
    D = np.exp(logc[:, None] - logc[None, :])        # prod_{s < l <= t} g_l for s <= t
    D = np.tril(D)
    c = np.exp(logc)
    O = (np.tril(q @ k.T) * D) @ v + c[:, None] * (q @ S0)
    S = c[-1] * S0 + (k * D[T - 1][:, None]).T @ v
    return O, S


def _rand(rng, lead, T, dk, dv, lo=0.3):
    q = rng.standard_normal(lead + (T, dk))
    k = rng.standard_normal(lead + (T, dk))
    v = rng.standard_normal(lead + (T, dv))
    g = rng.uniform(lo, 1.0, lead + (T,))
    S0 = rng.standard_normal(lead + (dk, dv))
    return q, k, v, g, S0


def test_gate_one_reproduces_the_printed_trace():
    with open(os.path.join(GOLDEN, "trace_c4.json")) as f:
        gd = json.load(f)
    k = np.array(gd["k"], dtype=np.float64)
    v = np.array(gd["v"], dtype=np.float64)
    O, S8 = oracle.gated_recurrence(k, k, v, np.ones(k.shape[0]))  # q_t = k_t in the trace
    assert np.array_equal(O[:4], np.array(gd["o_1_to_4"]))
    assert np.array_equal(O[4:], np.array(gd["o_5_to_8"]))
    assert np.array_equal(S8, np.array(gd["S_8"]))


def test_gate_one_is_the_ungated_recurrence_bit_for_bit():
    rng = np.random.default_rng(1)
    q, k, v, _, S0 = _rand(rng, (3,), 40, 7, 5)
    O1, S1 = oracle.gated_recurrence(q, k, v, np.ones((3, 40)), S0)
    O0, S0_ = oracle.recurrence(q, k, v, S0)
    assert np.array_equal(O1, O0) and np.array_equal(S1, S0_)


@pytest.mark.parametrize("T,dk,dv,lo", [(1, 3, 2, 0.5), (9, 4, 6, 0.3), (64, 16, 8, 0.05), (200, 8, 8, 0.9)])
def test_closed_form(T, dk, dv, lo):
    rng = np.random.default_rng(T + dk)
    q, k, v, g, S0 = _rand(rng, (2,), T, dk, dv, lo)
    O, S = oracle.gated_recurrence(q, k, v, g, S0, nthreads=2)
    for b in range(2):
        O_ref, S_ref = _closed_form(q[b], k[b], v[b], g[b], S0[b])
        assert np.allclose(O[b], O_ref, rtol=1e-10, atol=1e-10)
        assert np.allclose(S[b], S_ref, rtol=1e-10, atol=1e-10)


def test_brute_force_tiny():
    rng = np.random.default_rng(7)
    T, dk, dv = 5, 3, 2
    q, k, v, g, S0 = _rand(rng, (), T, dk, dv)
    O, S = oracle.gated_recurrence(q, k, v, g, S0)
    for t in range(T):
        o = np.zeros(dv)
        for s in range(t + 1):
            w = 1.0
            for l in range(s + 1, t + 1):
                w *= g[l]
            for i in range(dk):
                for j in range(dv):
                    o[j] += w * q[t, i] * k[s, i] * v[s, j]
        c = 1.0
        for l in range(t + 1):
            c *= g[l]
        for i in range(dk):
            for j in range(dv):
                o[j] += c * q[t, i] * S0[i, j]
        assert np.allclose(O[t], o, rtol=1e-12, atol=1e-12), t


def test_gate_zero_forgets_everything_before_the_token():
    rng = np.random.default_rng(3)
    q, k, v, _, S0 = _rand(rng, (), 6, 4, 3)
    O, S = oracle.gated_recurrence(q, k, v, np.zeros(6), S0)
    assert np.allclose(O, (q * k).sum(1)[:, None] * v, rtol=0, atol=1e-12)
    assert np.allclose(S, np.outer(k[-1], v[-1]), rtol=0, atol=1e-12)


def test_decay_after_the_update_is_caught():
    """A planted mistake: the gate applied after the token's update."""
    rng = np.random.default_rng(5)
    q, k, v, g, S0 = _rand(rng, (), 12, 4, 3)

    def wrong(q, k, v, g, S0):
        S = S0.copy()
        O = np.zeros((q.shape[0], v.shape[1]))
        for t in range(q.shape[0]):
            S = g[t] * (S + np.outer(k[t], v[t]))
            O[t] = S.T @ q[t]
        return O, S

    O_ref, _ = _closed_form(q, k, v, g, S0)
    O_w, _ = wrong(q, k, v, g, S0)
    O, _ = oracle.gated_recurrence(q, k, v, g, S0)
    assert np.allclose(O, O_ref, rtol=1e-10, atol=1e-10)
    assert not np.allclose(O_w, O_ref, rtol=1e-3, atol=1e-3)


def test_decode_step_is_one_token_of_the_recurrence():
    rng = np.random.default_rng(9)
    q, k, v, g, S0 = _rand(rng, (4,), 3, 5, 6)
    O, S = oracle.gated_recurrence(q, k, v, g, S0)
    Sd = S0.copy()
    for t in range(3):
        o, Sd = oracle.gated_decode_step(q[:, t], k[:, t], v[:, t], g[:, t], Sd)
        assert np.array_equal(o, O[:, t])
    assert np.array_equal(Sd, S)


def test_prefill_then_prefill_equals_one_prefill():
    """The gated state is still the one object handed between blocks."""
    rng = np.random.default_rng(11)
    q, k, v, g, S0 = _rand(rng, (2,), 30, 4, 4)
    O, S = oracle.gated_recurrence(q, k, v, g, S0)
    Oa, Sa = oracle.gated_recurrence(q[:, :13], k[:, :13], v[:, :13], g[:, :13], S0)
    Ob, Sb = oracle.gated_recurrence(q[:, 13:], k[:, 13:], v[:, 13:], g[:, 13:], Sa)
    assert np.array_equal(np.concatenate([Oa, Ob], 1), O) and np.array_equal(Sb, S)


# ---- shared-state heads with the decayed state ------------------------------------

def _gated_grouped_brute_force(q, k, v, g, S0):
    """Explicit sums: query head h of a group of G reads key/value head h // G,
    whose state decays by that head's gates."""
    B, Hq, T, dk = q.shape
    Hkv, dv = k.shape[1], v.shape[3]
    G = Hq // Hkv
    O = np.zeros((B, Hq, T, dv))
    S = np.zeros((B, Hkv, dk, dv))
    for b in range(B):
        for hk in range(Hkv):
            for t in range(T):
                c = 1.0
                for l in range(t + 1):
                    c *= g[b, hk, l]
                St = c * S0[b, hk]
                for s in range(t + 1):
                    w = 1.0
                    for l in range(s + 1, t + 1):
                        w *= g[b, hk, l]
                    St = St + w * np.outer(k[b, hk, s], v[b, hk, s])
                for j in range(G):
                    O[b, hk * G + j, t] = St.T @ q[b, hk * G + j, t]
                if t == T - 1:
                    S[b, hk] = St
    return O, S


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (6, 1), (3, 3)])
def test_gated_grouped_recurrence_vs_brute_force(Hq, Hkv):
    rng = np.random.default_rng(Hq * 10 + Hkv)
    B, T, dk, dv = 2, 6, 3, 4
    q = rng.standard_normal((B, Hq, T, dk))
    k = rng.standard_normal((B, Hkv, T, dk))
    v = rng.standard_normal((B, Hkv, T, dv))
    g = rng.uniform(0.2, 1.0, (B, Hkv, T))
    S0 = rng.standard_normal((B, Hkv, dk, dv))
    O, S = oracle.gated_grouped_recurrence(q, k, v, g, S0)
    O_ref, S_ref = _gated_grouped_brute_force(q, k, v, g, S0)
    assert np.allclose(O, O_ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(S, S_ref, rtol=1e-12, atol=1e-12)


def test_gated_grouped_gate_one_is_the_grouped_recurrence_bit_for_bit():
    rng = np.random.default_rng(21)
    q = rng.standard_normal((2, 6, 20, 5))
    k = rng.standard_normal((2, 2, 20, 5))
    v = rng.standard_normal((2, 2, 20, 3))
    S0 = rng.standard_normal((2, 2, 5, 3))
    O1, S1 = oracle.gated_grouped_recurrence(q, k, v, np.ones((2, 2, 20)), S0)
    O0, S0_ = oracle.grouped_recurrence(q, k, v, S0)
    assert np.array_equal(O1, O0) and np.array_equal(S1, S0_)


def test_gated_grouped_decode_step_is_one_token_of_the_recurrence():
    rng = np.random.default_rng(23)
    q = rng.standard_normal((3, 8, 4, 6))
    k = rng.standard_normal((3, 2, 4, 6))
    v = rng.standard_normal((3, 2, 4, 5))
    g = rng.uniform(0.3, 1.0, (3, 2, 4))
    S0 = rng.standard_normal((3, 2, 6, 5))
    O, S = oracle.gated_grouped_recurrence(q, k, v, g, S0)
    Sd = S0.copy()
    for t in range(4):
        o, Sd = oracle.gated_grouped_decode_step(q[:, :, t], k[:, :, t], v[:, :, t], g[:, :, t], Sd)
        assert np.array_equal(o, O[:, :, t])
    assert np.array_equal(Sd, S)


def test_gated_grouped_mapping_mistake_is_caught():
    """A planted mistake -- query head h reading key/value head h % Hkv
    instead of h // G -- disagrees with the brute force."""
    rng = np.random.default_rng(25)
    B, Hq, Hkv, T, d = 1, 4, 2, 5, 3
    q = rng.standard_normal((B, Hq, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    g = rng.uniform(0.3, 1.0, (B, Hkv, T))
    O_ref, _ = _gated_grouped_brute_force(q, k, v, g, np.zeros((B, Hkv, d, d)))
    idx = np.arange(Hq) % Hkv
    O_bad, _ = oracle.gated_recurrence(q, k[:, idx], v[:, idx], g[:, idx])
    O, _ = oracle.gated_grouped_recurrence(q, k, v, g)
    assert np.allclose(O, O_ref, rtol=1e-12, atol=1e-12)
    assert not np.allclose(O_bad, O_ref, rtol=1e-3, atol=1e-3)
