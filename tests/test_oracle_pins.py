"""Pins of the fp64 oracle against things other than itself.

Each test fixes part of the oracle by a value or property that the method or the
mathematics determines independently of the oracle's own code:
  * hand-worked fixtures (tests/golden/),
  * brute force with explicit dense transition matrices
    S_t = (I - beta k k^T) diag(alpha) S_{t-1} + beta k v^T  (a different form of the
    update than the oracle's step-by-step loop),
  * exact rational arithmetic (fractions) for g = 0,
  * closed forms (beta = 0 pure decay, one-hot key overwrite, scalar case),
  * invariants (beta = 0 and g = 0 leave S unchanged; beta = 1 with a unit key gives
    S^T k = v),
  * structure (linearity in (S0, V), split-carry, chunk form = recurrence,
    replay = recomputation).
A plausible slip in the oracle (decay after the delta step, output from the old
state, a wrong sign or transposed state, a dropped beta) fails at least one.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import kda_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(rng, T, H, dk, dv, gate_scale=0.1):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    g = -gate_scale * np.log1p(np.exp(rng.standard_normal((T, H, dk))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, g, beta


def brute_force(q, k, v, g, beta, h0, scale, use_l2=True, eps=O.EPS):
    """Dense-matrix form of one sequence: S <- (I - b k k^T) diag(a) S + b k v^T."""
    T, H, dk = q.shape
    dv = v.shape[2]
    o = np.zeros((T, H, dv))
    S = h0.copy()
    I = np.eye(dk)
    for t in range(T):
        for h in range(H):
            qv, kv = q[t, h], k[t, h]
            if use_l2:
                qv = qv / np.sqrt(np.dot(qv, qv) + eps)
                kv = kv / np.sqrt(np.dot(kv, kv) + eps)
            M = (I - beta[t, h] * np.outer(kv, kv)) @ np.diag(np.exp(g[t, h]))
            S[h] = M @ S[h] + beta[t, h] * np.outer(kv, v[t, h])
            o[t, h] = scale * (S[h].T @ qv)
    return o, S


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


@pytest.mark.parametrize("name", ["hand_dk2_T2.json", "hand_l2norm.json"])
def test_golden_hand_worked(name):
    fx = json.load(open(os.path.join(GOLDEN, name)))
    toks = fx["tokens"]
    q = np.array([[t["q"]] for t in toks])
    k = np.array([[t["k"]] for t in toks])
    v = np.array([[t["v"]] for t in toks])
    g = np.array([[t["g"]] for t in toks])
    beta = np.array([[t["beta"]] for t in toks])
    h0 = np.array(fx["h0"])[None, None]
    s = fx["settings"]
    o, ht, _ = O.recurrent(q, k, v, g, beta, [0, len(toks)], h0=h0, scale=s["scale"],
                           use_qk_l2norm=s["use_qk_l2norm"], eps=s.get("eps", O.EPS))
    tol = fx["tolerance_abs"]
    np.testing.assert_allclose(o[:, 0], np.array(fx["expected"]["o"]), rtol=0, atol=tol)
    np.testing.assert_allclose(ht[0, 0], np.array(fx["expected"]["ht"]), rtol=0, atol=tol)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("use_l2", [True, False])
def test_brute_force_dense_transition(seed, use_l2):
    rng = np.random.default_rng(seed)
    T, H, dk, dv = 7, 2, 5, 4
    q, k, v, g, beta = rand_inputs(rng, T, H, dk, dv, gate_scale=0.5)
    h0 = rng.standard_normal((H, dk, dv))
    scale = dk ** -0.5
    o_ref, S_ref = brute_force(q, k, v, g, beta, h0, scale, use_l2)
    o, ht, _ = O.recurrent(q, k, v, g, beta, [0, T], h0=h0[None], scale=scale,
                           use_qk_l2norm=use_l2)
    assert rel(o, o_ref) < 1e-13
    assert rel(ht[0], S_ref) < 1e-13


def _frac_recurrence(q, k, v, beta, S):
    """Exact rational recurrence with g = 0 (alpha = 1), no L2 norm, scale = 1."""
    dk, dv = len(S), len(S[0])
    outs = []
    for qt, kt, vt, bt in zip(q, k, v, beta):
        p = [sum(S[c][j] * kt[c] for c in range(dk)) for j in range(dv)]
        u = [bt * (vt[j] - p[j]) for j in range(dv)]
        S = [[S[c][j] + kt[c] * u[j] for j in range(dv)] for c in range(dk)]
        outs.append([sum(S[c][j] * qt[c] for c in range(dk)) for j in range(dv)])
    return outs, S


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_exact_rationals_dyadic(seed):
    """Small dyadic inputs keep every fp64 operation exact, so the oracle must equal
    the exact rational result bit for bit."""
    rng = np.random.default_rng(100 + seed)
    T, dk, dv = 3, 3, 2
    vals = [Fraction(n, 4) for n in range(-4, 5)]
    pick = lambda *s: rng.integers(0, len(vals), size=s)
    q = [[vals[i] for i in row] for row in pick(T, dk)]
    k = [[vals[i] for i in row] for row in pick(T, dk)]
    v = [[vals[i] for i in row] for row in pick(T, dv)]
    beta = [Fraction(1, 2), Fraction(1, 4), Fraction(1, 1)][:T]
    S0 = [[vals[i] for i in row] for row in pick(dk, dv)]
    o_ex, S_ex = _frac_recurrence(q, k, v, beta, S0)
    f = lambda a: np.array(a, dtype=np.float64)
    o, ht, _ = O.recurrent(f(q)[:, None], f(k)[:, None], f(v)[:, None], np.zeros((T, 1, dk)),
                           f(beta)[:, None], [0, T], h0=f(S0)[None, None], scale=1.0,
                           use_qk_l2norm=False)
    assert np.array_equal(o[:, 0], f([[float(x) for x in r] for r in o_ex]))
    assert np.array_equal(ht[0, 0], f([[float(x) for x in r] for r in S_ex]))


def test_invariant_beta0_g0_state_unchanged():
    rng = np.random.default_rng(5)
    T, H, dk, dv = 6, 3, 8, 5
    q, k, v, _, _ = rand_inputs(rng, T, H, dk, dv)
    h0 = rng.standard_normal((1, H, dk, dv))
    o, ht, _ = O.recurrent(q, k, v, np.zeros((T, H, dk)), np.zeros((T, H)), [0, T], h0=h0)
    assert np.array_equal(ht, h0)
    # and the output is the read-out of the unchanged state
    qh = q / np.sqrt((q * q).sum(-1, keepdims=True) + O.EPS)
    ref = dk ** -0.5 * np.einsum("thc,hcj->thj", qh, h0[0])
    assert rel(o, ref) < 1e-14


@pytest.mark.parametrize("use_l2", [False, True])
def test_invariant_beta1_unit_key_stores_value(use_l2):
    """beta = 1 with a unit key: after the update S^T k = v, whatever the gate."""
    rng = np.random.default_rng(6)
    H, dk, dv = 4, 16, 8
    for _ in range(5):
        q = rng.standard_normal((1, H, dk))
        k = rng.standard_normal((1, H, dk))
        if use_l2:
            k *= 1e4  # eps = 1e-6 is then negligible: |kh| = 1 - O(1e-14)
        else:
            k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.standard_normal((1, H, dv))
        g = -np.abs(rng.standard_normal((1, H, dk)))
        h0 = rng.standard_normal((1, H, dk, dv))
        _, ht, _ = O.recurrent(q, k, v, g, np.ones((1, H)), [0, 1], h0=h0, use_qk_l2norm=use_l2)
        kh = k[0] / np.linalg.norm(k[0], axis=-1, keepdims=True)
        got = np.einsum("hcj,hc->hj", ht[0], kh)
        np.testing.assert_allclose(got, v[0], rtol=0, atol=1e-12)


def test_closed_form_pure_decay():
    """beta = 0: S_t = diag(exp(G_t)) S0 and o_t = scale (exp(G_t) * qh)^T S0."""
    rng = np.random.default_rng(7)
    T, H, dk, dv = 9, 2, 6, 3
    q, k, v, g, _ = rand_inputs(rng, T, H, dk, dv, gate_scale=0.7)
    h0 = rng.standard_normal((1, H, dk, dv))
    o, ht, _ = O.recurrent(q, k, v, g, np.zeros((T, H)), [0, T], h0=h0, scale=0.3)
    G = np.cumsum(g, axis=0)
    qh = q / np.sqrt((q * q).sum(-1, keepdims=True) + O.EPS)
    o_ref = 0.3 * np.einsum("thc,hcj->thj", np.exp(G) * qh, h0[0])
    S_ref = np.exp(G[-1])[:, :, None] * h0[0]
    assert rel(o, o_ref) < 1e-13
    assert rel(ht[0], S_ref) < 1e-13


def test_closed_form_one_hot_overwrite():
    """One-hot keys, beta = 1, g = 0: row i_t of S is overwritten by v_t."""
    rng = np.random.default_rng(8)
    T, dk, dv = 10, 5, 4
    idx = rng.integers(0, dk, size=T)
    k = np.zeros((T, 1, dk))
    k[np.arange(T), 0, idx] = 1.0
    q = rng.standard_normal((T, 1, dk))
    v = rng.standard_normal((T, 1, dv))
    h0 = rng.standard_normal((1, 1, dk, dv))
    o, ht, _ = O.recurrent(q, k, v, np.zeros((T, 1, dk)), np.ones((T, 1)), [0, T], h0=h0,
                           scale=1.0, use_qk_l2norm=False)
    S = h0[0, 0].copy()
    for t in range(T):
        S[idx[t]] = v[t, 0]
        np.testing.assert_allclose(o[t, 0], S.T @ q[t, 0], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(ht[0, 0], S, rtol=0, atol=1e-15)


def test_closed_form_scalar():
    """dk = dv = 1, no norm: s <- alpha s (1 - beta k^2) + beta k v, o = scale q s."""
    rng = np.random.default_rng(9)
    T = 20
    q, k, v = (rng.standard_normal((T, 1, 1)) for _ in range(3))
    g = -np.abs(rng.standard_normal((T, 1, 1)))
    beta = rng.uniform(size=(T, 1))
    o, ht, _ = O.recurrent(q, k, v, g, beta, [0, T], h0=np.full((1, 1, 1, 1), 0.7), scale=2.0,
                           use_qk_l2norm=False)
    s = 0.7
    for t in range(T):
        a, kk, b = np.exp(g[t, 0, 0]), k[t, 0, 0], beta[t, 0]
        s = a * s * (1 - b * kk * kk) + b * kk * v[t, 0, 0]
        assert abs(o[t, 0, 0] - 2.0 * q[t, 0, 0] * s) <= 1e-13 * max(1.0, abs(s))
    assert abs(ht[0, 0, 0, 0] - s) <= 1e-13 * max(1.0, abs(s))


def test_linearity_in_state_and_values():
    rng = np.random.default_rng(10)
    T, H, dk, dv = 12, 2, 6, 5
    q, k, v, g, beta = rand_inputs(rng, T, H, dk, dv)
    h0 = rng.standard_normal((1, H, dk, dv))
    o_full, h_full, _ = O.recurrent(q, k, v, g, beta, [0, T], h0=h0)
    o_s, h_s, _ = O.recurrent(q, k, np.zeros_like(v), g, beta, [0, T], h0=h0)
    o_v, h_v, _ = O.recurrent(q, k, v, g, beta, [0, T], h0=None)
    assert rel(o_s + o_v, o_full) < 1e-13
    assert rel(h_s + h_v, h_full) < 1e-13


def test_split_carry_equals_one_call():
    rng = np.random.default_rng(11)
    T, H, dk, dv = 40, 2, 8, 8
    q, k, v, g, beta = rand_inputs(rng, T, H, dk, dv)
    h0 = rng.standard_normal((1, H, dk, dv))
    o, ht, _ = O.recurrent(q, k, v, g, beta, [0, T], h0=h0)
    a = 17
    o1, h1, _ = O.recurrent(q[:a], k[:a], v[:a], g[:a], beta[:a], [0, a], h0=h0)
    o2, h2, _ = O.recurrent(q[a:], k[a:], v[a:], g[a:], beta[a:], [0, T - a], h0=h1)
    assert rel(np.concatenate([o1, o2]), o) < 1e-14
    assert rel(h2, ht) < 1e-14


def test_varlen_sequences_are_independent():
    rng = np.random.default_rng(12)
    lens = [5, 0, 11, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, dk, dv = int(cu[-1]), 2, 4, 3
    q, k, v, g, beta = rand_inputs(rng, T, H, dk, dv)
    h0 = rng.standard_normal((len(lens), H, dk, dv))
    o, ht, _ = O.recurrent(q, k, v, g, beta, cu, h0=h0)
    for i in range(len(lens)):
        s, e = cu[i], cu[i + 1]
        oi, hi, _ = O.recurrent(q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e], [0, e - s],
                                h0=h0[i:i + 1])
        assert np.array_equal(o[s:e], oi)
        assert np.array_equal(ht[i], hi[0])
    assert np.array_equal(ht[1], h0[1])  # empty sequence: state passes through


@pytest.mark.parametrize("chunk", [1, 4, 16, 64])
def test_chunk_form_equals_recurrence(chunk):
    rng = np.random.default_rng(13)
    lens = [150, 64, 1, 37]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, dk, dv = int(cu[-1]), 2, 16, 12
    q, k, v, g, beta = rand_inputs(rng, T, H, dk, dv, gate_scale=0.3)
    h0 = rng.standard_normal((len(lens), H, dk, dv))
    o1, h1, _ = O.recurrent(q, k, v, g, beta, cu, h0=h0)
    o2, h2 = O.chunked(q, k, v, g, beta, cu, h0=h0, chunk=chunk)
    assert rel(o2, o1) < 1e-12
    assert rel(h2, h1) < 1e-12


@settings(max_examples=25, deadline=None)
@given(lens=st.lists(st.integers(0, 90), min_size=1, max_size=3),
       dk=st.sampled_from([1, 3, 8]), dv=st.sampled_from([1, 5, 8]),
       seed=st.integers(0, 10_000), use_l2=st.booleans())
def test_chunk_form_property(lens, dk, dv, seed, use_l2):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H = int(cu[-1]), 2
    q, k, v, g, beta = rand_inputs(rng, T, H, dk, dv, gate_scale=0.3)
    h0 = rng.standard_normal((len(lens), H, dk, dv))
    o1, h1, _ = O.recurrent(q, k, v, g, beta, cu, h0=h0, use_qk_l2norm=use_l2)
    o2, h2 = O.chunked(q, k, v, g, beta, cu, h0=h0, chunk=64, use_qk_l2norm=use_l2)
    if T:
        assert rel(o2, o1) < 1e-11
    assert rel(h2, h1) < 1e-11


def test_records_hold_normalised_key_gate_and_update():
    rng = np.random.default_rng(14)
    N, T, H, dk, dv = 2, 3, 2, 6, 4
    q = rng.standard_normal((N, T, H, dk))
    k = rng.standard_normal((N, T, H, dk))
    v = rng.standard_normal((N, T, H, dv))
    g = -np.abs(rng.standard_normal((N, T, H, dk)))
    beta = rng.uniform(size=(N, T, H))
    h0 = rng.standard_normal((N, H, dk, dv))
    _, _, rec = O.decode(q, k, v, g, beta, h0, want_records=True)
    kh = k / np.sqrt((k * k).sum(-1, keepdims=True) + O.EPS)
    np.testing.assert_allclose(rec[..., :dk], kh, rtol=1e-15, atol=0)
    np.testing.assert_allclose(rec[..., dk:2 * dk], np.exp(g), rtol=1e-15, atol=0)
    # u_t = beta_t (v_t - S'^T kh_t) with S' the decayed state before token t
    S = h0.copy()
    for t in range(T):
        Sd = np.exp(g[:, t])[..., None] * S
        u = beta[:, t, :, None] * (v[:, t] - np.einsum("nhcj,nhc->nhj", Sd, kh[:, t]))
        np.testing.assert_allclose(rec[:, t, :, 2 * dk:], u, rtol=1e-12, atol=1e-13)
        S = Sd + np.einsum("nhc,nhj->nhcj", kh[:, t], u)


@pytest.mark.parametrize("seed", [0, 1])
def test_replay_equals_recompute(seed):
    """ReplaySSM: replaying accepted records from the committed state equals running the
    recurrence over the accepted tokens only."""
    rng = np.random.default_rng(20 + seed)
    N, T, H, dk, dv = 5, 8, 2, 8, 6
    q = rng.standard_normal((N, T, H, dk))
    k = rng.standard_normal((N, T, H, dk))
    v = rng.standard_normal((N, T, H, dv))
    g = -0.1 * np.log1p(np.exp(rng.standard_normal((N, T, H, dk))))
    beta = 1 / (1 + np.exp(-rng.standard_normal((N, T, H))))
    h0 = rng.standard_normal((N, H, dk, dv))
    acc = np.array([0, 1, 4, 7, 8])
    o_ver, _, rec = O.decode(q, k, v, g, beta, h0, want_records=True)
    S = O.replay(h0, rec, acc)
    for n in range(N):
        a = acc[n]
        if a == 0:
            assert np.array_equal(S[n], h0[n])
            continue
        o_n, h_n, _ = O.decode(q[n:n + 1, :a], k[n:n + 1, :a], v[n:n + 1, :a], g[n:n + 1, :a],
                               beta[n:n + 1, :a], h0[n:n + 1])
        assert rel(S[n], h_n[0]) < 1e-13
        assert rel(o_ver[n, :a], o_n[0]) < 1e-14  # verify outputs of accepted tokens


def test_oracle_rejects_bad_arguments():
    rng = np.random.default_rng(0)
    q, k, v, g, beta = rand_inputs(rng, 4, 1, 2, 2)
    with pytest.raises(ValueError):
        O.recurrent(q, k, v, g, beta, [0, 3])
    with pytest.raises(ValueError):
        O.recurrent(q, k, v, g, beta, [1, 4])
    with pytest.raises(RuntimeError):
        O.replay(np.zeros((1, 1, 2, 2)), np.zeros((1, 2, 1, 6)), [3])
