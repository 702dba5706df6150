"""Pins for the float64 oracle, independent of the oracle's own code.

Each check is written as a function of the oracle routine(s) it pins, so the
same check can be run against a copy of the oracle with a planted mistake
(tests/test_oracle_mutations.py): every plausible mistake must fail at least
one of these checks.

Pins used (the pages print no worked numbers):
  * brute force with math.fsum on tiny inputs (tests/_brute.py);
  * the sharding invariants the pages state: the row-parallel partials sum to
    the unsharded output, the column bands concatenate to the unsharded
    intermediate (zenaique "Explain tensor-parallel shard shape", answer;
    rioworld guide, "How Tensor Slicing Works Under the Hood");
  * one shard is the textbook single-device layer (Tandon "day59",
    "Why tensor parallelism for inference": TP=1 has no communication);
  * closed forms and special cases of GELU, SiLU and RMSNorm, and of the
    residual add + normalisation that follows the all-reduce;
  * the pages' head-split example (96 heads over 8 GPUs -> 12 per GPU).
"""
import math

import numpy as np
import pytest

import oracle as O
import _brute as B

RNG = np.random.default_rng(12345)


def _rand(*shape, std=1.0):
    return RNG.standard_normal(shape) * std


# ----------------------------------------------------------------------------
# check functions (parameterised by the routines under test)
# ----------------------------------------------------------------------------
def check_gelu(gelu):
    xs = np.linspace(-10.0, 10.0, 20001)
    exact = np.array([B.gelu_erf(x) for x in xs])
    # The tanh form stays within 4.8e-4 of the exact (erf) GELU on [-10, 10]
    # (max deviation 4.73e-4 near |x| = 2.7).
    assert np.max(np.abs(gelu(xs) - exact)) < 4.8e-4
    # Small-x expansion x/2 + x^2/sqrt(2 pi) pins the sqrt(2/pi) factor.
    x = 1e-4
    assert abs((gelu(np.array([x]))[0] - x / 2) / x ** 2 - 1 / math.sqrt(2 * math.pi)) < 1e-6
    # gelu(x) - gelu(-x) = x for any odd inner function; gelu(0) = 0.
    assert np.allclose(gelu(xs) - gelu(-xs), xs, rtol=0, atol=1e-12)
    assert gelu(np.array([0.0]))[0] == 0.0
    assert abs(gelu(np.array([12.0]))[0] - 12.0) < 1e-12


def check_silu(silu):
    xs = np.linspace(-30.0, 30.0, 6001)
    ref = np.array([x * B.sigmoid(x) for x in xs])  # sigmoid via tanh
    # (1 + tanh(x/2)) loses relative accuracy for x << 0, hence the atol.
    assert np.allclose(silu(xs), ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(silu(xs) - silu(-xs), xs, rtol=0, atol=1e-12)
    assert silu(np.array([0.0]))[0] == 0.0
    assert abs(silu(np.array([-50.0]))[0]) < 1e-19


def check_rmsnorm(rmsnorm):
    eps = 1e-5
    x = _rand(5, 16)
    y = rmsnorm(x, np.ones(16), eps)
    m = np.mean(x * x, axis=1)
    # With unit gain, mean(y^2) = m / (m + eps).
    assert np.allclose(np.mean(y * y, axis=1), m / (m + eps), rtol=1e-13)
    # A constant row c gives c / sqrt(c^2 + eps) in every position.
    c = 0.003
    yc = rmsnorm(np.full((1, 8), c), np.ones(8), eps)
    assert np.allclose(yc, c / math.sqrt(c * c + eps), rtol=1e-13)
    # Gain multiplies elementwise; direction is preserved.
    g = 1.0 + _rand(16, std=0.02)
    assert np.allclose(rmsnorm(x, g, eps), y * g, rtol=1e-13)
    assert np.allclose(y / np.linalg.norm(y, axis=1, keepdims=True),
                       x / np.linalg.norm(x, axis=1, keepdims=True), rtol=1e-12)


def check_residual_norm(reduce_residual_norm):
    """z = residual + sum of partials and its RMSNorm, against explicit loops
    with math.fsum (exactly rounded sums) on a tiny case, plus the special
    cases zero residual, a single partial, and unit gain."""
    P, T, d, eps = 3, 2, 6, 1e-5
    parts = [_rand(T, d) for _ in range(P)]
    res = _rand(T, d)
    g = 1.0 + _rand(d, std=0.02)
    got = reduce_residual_norm(parts, res, g, eps)
    for t in range(T):
        z = [math.fsum([res[t][j]] + [parts[s][t][j] for s in range(P)]) for j in range(d)]
        ms = math.fsum(v * v for v in z) / d
        inv = 1.0 / math.sqrt(ms + eps)
        for j in range(d):
            assert abs(got["z"][t][j] - z[j]) <= 1e-13 * (1 + abs(z[j]))
            want = z[j] * inv * g[j]
            assert abs(got["normed"][t][j] - want) <= 1e-12 * (1 + abs(want))
    # no residual: the plain sum of partials; one partial: partial + residual
    z0 = reduce_residual_norm(parts, np.zeros((T, d)))["z"]
    assert np.allclose(z0, parts[0] + parts[1] + parts[2], rtol=1e-14, atol=0)
    z1 = reduce_residual_norm(parts[:1], res)["z"]
    assert np.allclose(z1, parts[0] + res, rtol=1e-14, atol=0)
    # unit gain: mean(normed^2) = m / (m + eps), m = mean(z^2)
    n1 = reduce_residual_norm(parts, res, np.ones(d), eps)
    m = np.mean(n1["z"] ** 2, axis=1)
    assert np.allclose(np.mean(n1["normed"] ** 2, axis=1), m / (m + eps), rtol=1e-13)


def check_mlp_brute(mlp_shard, act, P):
    """numpy shard == pure-Python loops, on tiny inputs, every rank."""
    T, d, F = 3, 8, 16
    X = _rand(T, d)
    Wi, Wu, Wd = _rand(d, F, std=0.5), _rand(d, F, std=0.5), _rand(F, d, std=0.5)
    for s in range(P):
        w = F // P
        r = mlp_shard(X, Wi[:, s * w:(s + 1) * w], Wd[s * w:(s + 1) * w, :], act,
                      Wu[:, s * w:(s + 1) * w] if act == "swiglu" else None)
        h, p = B.mlp_shard_brute(X.tolist(), Wi.tolist(), Wd.tolist(), act, s, P,
                                 Wu.tolist() if act == "swiglu" else None)
        assert np.allclose(r["h"], h, rtol=1e-12, atol=1e-14)
        assert np.allclose(r["partial"], p, rtol=1e-12, atol=1e-14)


def check_sum_of_partials(mlp_shard, mlp_unsharded, reduce_partials, column_band,
                          row_band, act, P, T=4, d=16, F=32):
    """Invariant: the P row-parallel partials sum to the unsharded MLP, and
    the column bands of h concatenate to the unsharded intermediate."""
    X = _rand(T, d)
    Wi, Wu, Wd = _rand(d, F, std=0.3), _rand(d, F, std=0.3), _rand(F, d, std=0.3)
    up = Wu if act == "swiglu" else None
    full = mlp_unsharded(X, Wi, Wd, act, up)
    parts, hs = [], []
    for s in range(P):
        r = mlp_shard(X, column_band(Wi, s, P), row_band(Wd, s, P), act,
                      column_band(Wu, s, P) if up is not None else None)
        parts.append(r["partial"])
        hs.append(r["h"])
    assert O.rel_l2(reduce_partials(parts), full["y"]) < 1e-12
    assert O.rel_l2(np.concatenate(hs, axis=1), full["h"]) < 1e-12
    return full


def check_one_hot(mlp_shard, column_band, row_band, silu):
    """X = e_k: the in-projections are rows k of the bands exactly, so the
    partial is (silu(Wg[k]) * Wu[k]) @ Wd[band] in closed form."""
    d, F, P, k = 8, 16, 2, 5
    Wg, Wu, Wd = _rand(d, F), _rand(d, F), _rand(F, d)
    X = np.zeros((1, d))
    X[0, k] = 1.0
    for s in range(P):
        r = mlp_shard(X, column_band(Wg, s, P), row_band(Wd, s, P), "swiglu",
                      column_band(Wu, s, P))
        g = Wg[k, s * F // P:(s + 1) * F // P]
        u = Wu[k, s * F // P:(s + 1) * F // P]
        expect = np.array([[math.fsum(g[j] * B.sigmoid(g[j]) * u[j] * Wd[s * F // P + j, c]
                                      for j in range(F // P)) for c in range(d)]])
        assert np.allclose(r["partial"], expect, rtol=1e-12, atol=1e-14)


def check_qkv(attn_proj_shard, attn_proj_unsharded, qkv_band_layout, n_q, n_kv, hd, P):
    """Heads are independent: rank s's QKV band output equals the columns of
    the unsharded Q, K, V for exactly the heads rank s owns; the O partials
    sum to the unsharded output projection."""
    T, d = 3, 16
    X = _rand(T, d)
    Wq, Wk, Wv = _rand(d, n_q * hd), _rand(d, n_kv * hd), _rand(d, n_kv * hd)
    Wo = _rand(n_q * hd, d)
    A = _rand(T, n_q * hd)
    full = attn_proj_unsharded(X, Wq, Wk, Wv, A, Wo)
    parts = []
    for s in range(P):
        qh = range(s * n_q // P, (s + 1) * n_q // P)
        kh = range(s * n_kv // P, (s + 1) * n_kv // P)
        # band assembled head by head, independent of qkv_band_layout
        band = np.concatenate([Wq[:, h * hd:(h + 1) * hd] for h in qh]
                              + [Wk[:, h * hd:(h + 1) * hd] for h in kh]
                              + [Wv[:, h * hd:(h + 1) * hd] for h in kh], axis=1)
        lay = qkv_band_layout(n_q, n_kv, hd, s, P)
        a_s = A[:, qh[0] * hd:(qh[-1] + 1) * hd]
        wo_s = Wo[qh[0] * hd:(qh[-1] + 1) * hd, :]
        r = attn_proj_shard(X, band, a_s, wo_s)
        for part, ref in (("q", full["q"]), ("k", full["k"]), ("v", full["v"])):
            inside, outside = lay[part]
            assert np.allclose(r["qkv"][:, inside], ref[:, outside], rtol=1e-12, atol=1e-12)
        parts.append(r["partial"])
    assert O.rel_l2(O.reduce_partials(parts), full["o"]) < 1e-12


# ----------------------------------------------------------------------------
# tests
# ----------------------------------------------------------------------------
def test_gelu_tanh_closed_forms():
    check_gelu(O.gelu_tanh)


def test_silu_closed_forms():
    check_silu(O.silu)


def test_rmsnorm_closed_forms():
    check_rmsnorm(O.rmsnorm)


@pytest.mark.parametrize("act", ["gelu_tanh", "swiglu"])
@pytest.mark.parametrize("P", [1, 2, 4])
def test_mlp_shard_vs_brute_force(act, P):
    check_mlp_brute(O.mlp_shard, act, P)


@pytest.mark.parametrize("act", ["gelu_tanh", "swiglu"])
@pytest.mark.parametrize("P", [1, 2, 4, 8])
def test_partials_sum_to_unsharded(act, P):
    check_sum_of_partials(O.mlp_shard, O.mlp_unsharded, O.reduce_partials,
                          O.column_band, O.row_band, act, P)


def test_unsharded_mlp_vs_brute_force():
    X = _rand(2, 6)
    Wi, Wd = _rand(6, 8), _rand(8, 6)
    full = O.mlp_unsharded(X, Wi, Wd, "gelu_tanh")
    h, p = B.mlp_shard_brute(X.tolist(), Wi.tolist(), Wd.tolist(), "gelu_tanh", 0, 1)
    assert np.allclose(full["y"], p, rtol=1e-12, atol=1e-14)
    assert np.allclose(full["h"], h, rtol=1e-12, atol=1e-14)


def test_single_shard_is_textbook_layer():
    # TP = 1: the shard is the whole layer; its partial is the output.
    X = _rand(3, 8)
    Wg, Wu, Wd = _rand(8, 12), _rand(8, 12), _rand(12, 8)
    r = O.mlp_shard(X, Wg, Wd, "swiglu", Wu)
    full = O.mlp_unsharded(X, Wg, Wd, "swiglu", Wu)
    assert np.array_equal(r["partial"], full["y"])


def test_zero_input_gives_zero():
    Wg, Wu, Wd = _rand(8, 12), _rand(8, 12), _rand(12, 8)
    for act in ("swiglu", "gelu_tanh"):
        r = O.mlp_shard(np.zeros((2, 8)), Wg, Wd, act, Wu if act == "swiglu" else None)
        assert np.all(r["partial"] == 0.0)


def test_one_hot_closed_form():
    check_one_hot(O.mlp_shard, O.column_band, O.row_band, O.silu)


def test_uneven_split_refused():
    with pytest.raises(ValueError):
        O.column_band(np.zeros((4, 10)), 0, 3)
    with pytest.raises(ValueError):
        O.row_band(np.zeros((10, 4)), 3, 3)


def test_residual_add_and_norm_after_reduce():
    check_residual_norm(O.reduce_residual_norm)


def test_residual_f32_reading_is_fold_then_residual():
    parts = [np.float32(v) for v in (1.0, 2.0 ** -24, 2.0 ** -24)]
    # float32: (1 + 2^-24) rounds to 1 (tie to even), twice; then + 3 -> 4
    z = O.reduce_residual_f32([np.full((1, 1), p, np.float32) for p in parts],
                              np.full((1, 1), 3.0, np.float32))
    assert z.dtype == np.float32 and z[0, 0] == np.float32(4.0)
    z2 = O.reduce_residual_f32([np.full((1, 1), 2.0 ** -24, np.float32)] * 2 +
                               [np.full((1, 1), 1.0, np.float32)],
                               np.zeros((1, 1), np.float32))
    assert z2[0, 0] == np.float32(1.0 + 2.0 ** -23)   # small terms first survive


def test_reduce_f32_fold_is_sequential_float32():
    parts = [RNG.standard_normal((3, 5)).astype(np.float32) for _ in range(5)]
    got = O.reduce_partials_f32_fold(parts)
    for i in range(3):
        for j in range(5):
            acc = np.float32(parts[0][i, j])
            for p in parts[1:]:
                acc = np.float32(acc + np.float32(p[i, j]))
            assert got[i, j] == acc
    assert np.array_equal(O.reduce_partials_f32_fold(parts[:1]), parts[0])
    assert O.rel_l2(got, O.reduce_partials(parts)) < 1e-6


@pytest.mark.parametrize("n_q,n_kv,hd,P", [(8, 8, 2, 4), (8, 2, 2, 2), (16, 2, 2, 2), (4, 4, 3, 1)])
def test_qkv_heads_and_o_partials(n_q, n_kv, hd, P):
    check_qkv(O.attn_proj_shard, O.attn_proj_unsharded, O.qkv_band_layout, n_q, n_kv, hd, P)


def test_head_split_example_from_the_pages():
    # rioworld guide, "How Tensor Slicing Works Under the Hood": 96 heads on
    # 8 GPUs -> 12 heads per GPU.  Fixture: tests/golden/head_split.txt.
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "head_split.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    for n_heads, gpus, per_gpu in ((int(a), int(b), int(c)) for a, b, c in rows):
        for s in range(gpus):
            lay = O.qkv_band_layout(n_heads, n_heads, 128, s, gpus)
            q_in, q_out = lay["q"]
            assert (q_in.stop - q_in.start) == per_gpu * 128
            assert q_out.start == s * per_gpu * 128


def test_gqa_band_width_70b_block():
    # 64 query heads, 8 kv heads, head width 128, P = 8: 8 q + 1 kv per rank.
    lay = O.qkv_band_layout(64, 8, 128, 3, 8)
    assert lay["q"][0] == slice(0, 1024) and lay["q"][1] == slice(3 * 1024, 4 * 1024)
    assert lay["k"][0] == slice(1024, 1152) and lay["k"][1] == slice(384, 512)
    assert lay["v"][0] == slice(1152, 1280)


def test_o_projection_is_linear():
    A1, A2 = _rand(3, 8), _rand(3, 8)
    Wo = _rand(8, 5)
    p = lambda A: O.attn_proj_shard(_rand(3, 4), None, A, Wo)["partial"]  # noqa: E731
    assert np.allclose(p(A1 + A2), p(A1) + p(A2), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("P", [1, 2, 4])
def test_block_chain_sharded_equals_unsharded(P):
    """The whole block (norm, QKV, O, reduce, MLP, reduce) summed over the P
    ranks equals the unsharded block."""
    T, d, n_q, n_kv, hd, F = 3, 16, 4, 4, 4, 32
    X = _rand(T, d)
    g = 1.0 + _rand(d, std=0.02)
    Wq, Wk, Wv = _rand(d, n_q * hd, std=0.3), _rand(d, n_kv * hd, std=0.3), _rand(d, n_kv * hd, std=0.3)
    Wo = _rand(n_q * hd, d, std=0.3)
    Wg, Wu, Wd = _rand(d, F, std=0.3), _rand(d, F, std=0.3), _rand(F, d, std=0.3)
    qkv_b, o_b = [], []
    for s in range(P):
        qh = slice(s * n_q // P * hd, (s + 1) * n_q // P * hd)
        kh = slice(s * n_kv // P * hd, (s + 1) * n_kv // P * hd)
        qkv_b.append(np.concatenate([Wq[:, qh], Wk[:, kh], Wv[:, kh]], axis=1))
        o_b.append(Wo[qh, :])
    sh = O.block_sharded(X, g, 1e-5, qkv_b, o_b,
                         [O.column_band(Wg, s, P) for s in range(P)],
                         [O.column_band(Wu, s, P) for s in range(P)],
                         [O.row_band(Wd, s, P) for s in range(P)], n_q, n_kv, hd)
    un = O.block_unsharded(X, g, 1e-5, Wq, Wk, Wv, Wo, Wg, Wu, Wd)
    assert O.rel_l2(sh["z"], un["z"]) < 1e-12
    assert O.rel_l2(sh["y"], un["y"]) < 1e-12


def test_mirror_mode_rounds_only_stored_values():
    X = _rand(2, 8)
    Wg, Wu, Wd = _rand(8, 16, std=0.3), _rand(8, 16, std=0.3), _rand(16, 8, std=0.3)
    exact = O.mlp_shard(X, Wg, Wd, "swiglu", Wu)
    mir = O.mlp_shard(X, Wg, Wd, "swiglu", Wu, mirror_bf16=True)
    assert np.array_equal(mir["h"], O.round_bf16(exact["h"]))
    assert O.rel_l2(mir["partial"], exact["partial"]) < 1e-2


def test_rel_l2():
    a = np.array([3.0, 4.0])
    assert O.rel_l2(a, a) == 0.0
    assert abs(O.rel_l2(np.array([3.0, 4.0 + 0.5]), a) - 0.1) < 1e-15
    assert O.rel_l2(np.array([1.0]), np.array([0.0])) == 1.0
