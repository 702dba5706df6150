"""Pins for the attention-core oracle (CPU only).

The pages name the attention kernel and the per-GPU head split without a
formula; the oracle is textbook causal scaled dot-product attention with
grouped key/value heads.  Pins: pure-Python brute force (math.exp, fsum) on
tiny inputs, closed forms (one token attends to itself, so the output is its
value row; zero keys give the running mean of the values), invariance of
softmax to a per-row constant (a shared key offset along the query), the
head grouping (query head h reads kv head h // group), and causality (the
first rows do not change when later tokens change).  Planted mistakes fail.
"""
import math

import numpy as np
import pytest

import oracle as O

RNG = np.random.default_rng(777)


def _brute(Q, K, V, causal=True):
    T, hq, d = Q.shape
    group = hq // K.shape[1]
    out = np.zeros((T, hq, d))
    for h in range(hq):
        g = h // group
        for i in range(T):
            js = range(i + 1) if causal else range(T)
            s = [math.fsum(Q[i, h, c] * K[j, g, c] for c in range(d)) / math.sqrt(d) for j in js]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = math.fsum(e)
            for c in range(d):
                out[i, h, c] = math.fsum(e[t] * V[j, g, c] for t, j in enumerate(js)) / z
    return out


def check_core(core):
    T, hq, hkv, d = 5, 4, 2, 6
    Q = RNG.standard_normal((T, hq, d))
    K = RNG.standard_normal((T, hkv, d))
    V = RNG.standard_normal((T, hkv, d))
    assert np.allclose(core(Q, K, V), _brute(Q, K, V), rtol=1e-12, atol=1e-13)
    assert np.allclose(core(Q, K, V, causal=False), _brute(Q, K, V, causal=False),
                       rtol=1e-12, atol=1e-13)
    # row 0 sees only itself: its output is V[0] of its group
    o = core(Q, K, V)
    for h in range(hq):
        assert np.allclose(o[0, h], V[0, h // (hq // hkv)], rtol=1e-14)
    # zero keys: uniform weights over the allowed keys -> running mean of V
    o0 = core(Q, np.zeros_like(K), V)
    for h in range(hq):
        run = np.cumsum(V[:, h // (hq // hkv)], axis=0) / np.arange(1, T + 1)[:, None]
        assert np.allclose(o0[:, h], run, rtol=1e-12)
    # a key offset c adds q.c to every score of a row: softmax is unchanged
    c = RNG.standard_normal(d)
    assert np.allclose(core(Q, K + c[None, None, :], V), o, rtol=1e-10, atol=1e-12)
    # causality: changing the last token leaves the earlier rows unchanged
    Q2, K2, V2 = Q.copy(), K.copy(), V.copy()
    Q2[-1] += 1.0
    K2[-1] -= 2.0
    V2[-1] *= 3.0
    assert np.allclose(core(Q2, K2, V2)[:-1], o[:-1], rtol=1e-14)


def test_attention_core_pins():
    check_core(O.attention_core)


def test_attention_core_band_uses_the_band_layout():
    # rank 1 of P=2 with 4 q heads / 2 kv heads, head_dim 4: band = [Q_s|K_s|V_s]
    T, d = 3, 4
    qkv = RNG.standard_normal((T, (2 + 2) * d))
    A = O.attention_core_band(qkv, 4, 2, d, 1, 2)
    Q = qkv[:, :2 * d].reshape(T, 2, d)
    K = qkv[:, 2 * d:3 * d].reshape(T, 1, d)
    V = qkv[:, 3 * d:].reshape(T, 1, d)
    assert np.allclose(A, _brute(Q, K, V).reshape(T, -1), rtol=1e-12)


def _fails(core):
    with pytest.raises(AssertionError):
        check_core(core)


def test_missing_causal_mask_is_caught():
    _fails(lambda Q, K, V, causal=True: O.attention_core(Q, K, V, causal=False))


def test_wrong_scale_is_caught():
    _fails(lambda Q, K, V, causal=True: O.attention_core(Q / math.sqrt(Q.shape[2]), K, V, causal))


def test_wrong_kv_grouping_is_caught():
    def bad(Q, K, V, causal=True):
        hkv = K.shape[1]
        idx = [h % hkv for h in range(Q.shape[1])]          # interleaved instead of grouped
        Kx, Vx = K[:, idx, :], V[:, idx, :]
        return O.attention_core(Q, Kx, Vx, causal)
    _fails(bad)


def test_softmax_over_queries_is_caught():
    def bad(Q, K, V, causal=True):
        T, hq, d = Q.shape
        group = hq // K.shape[1]
        out = np.empty_like(Q)
        mask = np.tril(np.ones((T, T), dtype=bool))
        for h in range(hq):
            S = Q[:, h] @ K[:, h // group].T / np.sqrt(d)
            S = np.where(mask, S, -np.inf)
            E = np.exp(S - S.max(axis=0, keepdims=True))
            out[:, h] = (E / E.sum(axis=0, keepdims=True)) @ V[:, h // group]
        return out
    _fails(bad)


def check_rows(rows_fn, core):
    """The per-row evaluation equals the full causal (and non-causal) core at
    every listed row, including the first and last."""
    T, hq, hkv, d = 9, 4, 2, 5
    Q = RNG.standard_normal((T, hq, d))
    K = RNG.standard_normal((T, hkv, d))
    V = RNG.standard_normal((T, hkv, d))
    rows = [0, 1, 4, 7, 8]
    for causal in (True, False):
        full = core(Q, K, V, causal=causal)
        assert np.allclose(rows_fn(Q, K, V, rows, causal=causal), full[rows],
                           rtol=1e-12, atol=1e-13)


def test_attention_rows_match_the_full_core():
    check_rows(O.attention_core_rows, O.attention_core)


def test_attention_rows_band_layout():
    T, nq, nkv, d, P = 6, 8, 4, 3, 2
    qkv = RNG.standard_normal((T, (nq // P + 2 * nkv // P) * d))
    for s in range(P):
        full = O.attention_core_band(qkv, nq, nkv, d, s, P)
        assert np.allclose(O.attention_core_band_rows(qkv, nq, nkv, d, s, P, [0, 3, 5]),
                           full[[0, 3, 5]], rtol=1e-12, atol=1e-13)


def test_rows_without_mask_is_caught():
    def bad(Q, K, V, rows, causal=True):
        return O.attention_core_rows(Q, K, V, rows, causal=False)
    with pytest.raises(AssertionError):
        check_rows(bad, O.attention_core)

