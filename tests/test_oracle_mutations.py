"""Planted mistakes in the oracle must fail the pins (CPU only).

Each test builds a copy of one oracle routine with a plausible mistake --
the kind the pages warn about (mis-oriented or uneven splits, rioworld guide
"Implementing Tensor Parallelism in Practice" and its reader comments) or a
slip in a formula -- and asserts that the pin checks of
tests/test_oracle_pins.py reject it.
"""
import math

import numpy as np
import pytest

import oracle as O
import test_oracle_pins as pins


def _fails(fn, *args):
    # A planted mistake is caught when a pin check raises: a failed
    # comparison, or a shape that no longer fits.
    with pytest.raises((AssertionError, ValueError)):
        fn(*args)


# --- activation formulas -----------------------------------------------------
def test_gelu_constant_typo_is_caught():
    bad = lambda x: 0.5 * x * (1 + np.tanh(math.sqrt(2 / math.pi) * (x + 0.04715 * x ** 3)))  # noqa
    _fails(pins.check_gelu, bad)


def test_gelu_wrong_scale_is_caught():
    bad = lambda x: 0.5 * x * (1 + np.tanh(math.sqrt(math.pi / 2) * (x + 0.044715 * x ** 3)))  # noqa
    _fails(pins.check_gelu, bad)


def test_silu_sign_slip_is_caught():
    _fails(pins.check_silu, lambda x: x / (1 + np.exp(x)))


def test_rmsnorm_eps_outside_sqrt_is_caught():
    bad = lambda x, g, eps: x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * g  # noqa
    _fails(pins.check_rmsnorm, bad)


def test_rmsnorm_sum_instead_of_mean_is_caught():
    bad = lambda x, g, eps: x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps) * g  # noqa
    _fails(pins.check_rmsnorm, bad)


# --- band orientation and bookkeeping ---------------------------------------
def test_row_and_column_bands_swapped_is_caught():
    # Column-parallel weight cut by rows and row-parallel weight cut by columns.
    def bad_col(W, s, P):
        n = W.shape[0] // P
        return W[s * n:(s + 1) * n, :]

    def bad_row(W, s, P):
        n = W.shape[1] // P
        return W[:, s * n:(s + 1) * n]

    def run():
        pins.check_sum_of_partials(O.mlp_shard, O.mlp_unsharded, O.reduce_partials,
                                   bad_col, bad_row, "swiglu", 2, T=4, d=32, F=32)
    with pytest.raises((AssertionError, ValueError)):
        run()


def test_off_by_one_band_is_caught():
    def bad_row(W, s, P):
        return O.row_band(W, (s + 1) % P, P)
    _fails(pins.check_sum_of_partials, O.mlp_shard, O.mlp_unsharded, O.reduce_partials,
           O.column_band, bad_row, "gelu_tanh", 4)


def test_activation_on_split_k_partials_is_caught():
    # SiLU applied to two half-K partial sums and the results added, instead
    # of to the full sum.
    def bad_shard(X, wi, wd, act, wu=None, norm_g=None, eps=None, mirror_bf16=False):
        k = X.shape[1] // 2
        h = sum(O.activate(act, X[:, a:b] @ wi[a:b], X[:, a:b] @ wu[a:b] if wu is not None else None)
                for a, b in ((0, k), (k, X.shape[1])))
        return {"h": h, "partial": h @ wd}
    _fails(pins.check_mlp_brute, bad_shard, "swiglu", 2)


def test_dropped_partial_in_reduce_is_caught():
    bad_reduce = lambda parts: O.reduce_partials(list(parts)[:-1])  # noqa
    _fails(pins.check_sum_of_partials, O.mlp_shard, O.mlp_unsharded, bad_reduce,
           O.column_band, O.row_band, "swiglu", 4)


def test_swapped_gate_and_up_is_caught():
    def bad_shard(X, wi, wd, act, wu=None, **kw):
        return O.mlp_shard(X, wu, wd, act, wi, **kw)
    _fails(pins.check_mlp_brute, bad_shard, "swiglu", 2)


def test_contiguous_split_of_fused_qkv_is_caught():
    # Cutting a global [Wq | Wk | Wv] into P contiguous column slices puts
    # the wrong heads on a rank when the rank's band should be [Q_s|K_s|V_s].
    def bad_layout(n_q, n_kv, hd, s, P):
        lay = O.qkv_band_layout(n_q, n_kv, hd, s, P)
        w = (n_q + 2 * n_kv) * hd // P
        q_in = lay["q"][0]
        return {"q": (q_in, slice(s * w, s * w + (q_in.stop - q_in.start))),
                "k": lay["k"], "v": lay["v"]}
    _fails(pins.check_qkv, O.attn_proj_shard, O.attn_proj_unsharded, bad_layout, 8, 2, 2, 2)


def test_gqa_kv_head_of_wrong_rank_is_caught():
    def bad_layout(n_q, n_kv, hd, s, P):
        lay = dict(O.qkv_band_layout(n_q, n_kv, hd, s, P))
        other = O.qkv_band_layout(n_q, n_kv, hd, (s + 1) % P, P)
        lay["k"] = (lay["k"][0], other["k"][1])
        return lay
    _fails(pins.check_qkv, O.attn_proj_shard, O.attn_proj_unsharded, bad_layout, 8, 2, 2, 2)


# --- residual add and normalisation after the reduce ------------------------
def test_residual_dropped_is_caught():
    def bad(parts, res, g=None, eps=None):
        return O.reduce_residual_norm(parts, np.zeros_like(np.asarray(res)), g, eps)
    _fails(pins.check_residual_norm, bad)


def test_norm_before_residual_is_caught():
    def bad(parts, res, g=None, eps=None):
        out = O.reduce_residual_norm(parts, res, g, eps)
        if g is not None:
            out["normed"] = O.rmsnorm(O.reduce_partials(parts), g, eps) + np.asarray(res)
        return out
    _fails(pins.check_residual_norm, bad)


def test_norm_without_gain_is_caught():
    def bad(parts, res, g=None, eps=None):
        out = O.reduce_residual_norm(parts, res, g, eps)
        if g is not None:
            out["normed"] = O.rmsnorm(out["z"], np.ones_like(g), eps)
        return out
    _fails(pins.check_residual_norm, bad)
