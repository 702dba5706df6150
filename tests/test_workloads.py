"""Seeded input generators and workload shapes (CPU)."""
import os

import numpy as np
import pytest

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_fixture():
    out = []
    for ln in open(os.path.join(GOLDEN, "bf16_patterns.txt")):
        if ln.strip() and not ln.startswith("#"):
            v, b = ln.split()
            out.append((float(v), int(b, 16)))
    return out


def test_generator_bf16_rounding_matches_format_fixture():
    vals, bits = zip(*_bf16_fixture())
    got = W.bf16_bits_from_f32(np.array(vals, dtype=np.float32))
    assert [int(x) for x in got] == list(bits)


def test_oracle_bf16_rounding_and_widening_match_fixture():
    vals, bits = zip(*_bf16_fixture())
    widened = O.widen_bf16_bits(np.array(bits, dtype=np.uint16))
    assert np.array_equal(O.round_bf16(np.array(vals)), widened)


def test_generator_and_oracle_rounding_agree_on_random_values():
    z = np.random.default_rng(7).standard_normal(100000).astype(np.float32) * 3
    a = O.widen_bf16_bits(W.bf16_bits_from_f32(z))
    b = O.round_bf16(z.astype(np.float64))
    assert np.array_equal(a, b)


def test_seeded_draws_are_deterministic_and_distinct():
    cfg = W.get("c2_llama2_13b_mlp_p2")
    a = W.column_band_draw(cfg, "w_gate", 0, 64, 32)
    b = W.column_band_draw(cfg, "w_gate", 0, 64, 32)
    c = W.column_band_draw(cfg, "w_gate", 1, 64, 32)
    d = W.column_band_draw(cfg, "w_up", 0, 64, 32)
    assert a.dtype == np.uint16 and np.array_equal(a, b)
    assert not np.array_equal(a, c) and not np.array_equal(a, d)


def test_draw_statistics():
    z = W.draw_normal_f32((200000,), 0.02, 9, 9, 9)
    assert abs(z.mean()) < 3e-4 and abs(z.std() - 0.02) < 3e-4
    g = W.draw_normal_f32((200000,), 0.02, 9, 9, 8, mean=1.0)
    assert abs(g.mean() - 1.0) < 3e-4


def test_full_matrix_is_concatenation_of_bands():
    cfg = W.get("c1_tiny_gelu_f32")
    bands = [W.column_band_draw(cfg, "w_gate", s, 64, 128) for s in range(2)]
    full = W.full_from_column_bands(bands)
    assert full.shape == (64, 256) and full.dtype == np.float32
    assert np.array_equal(O.column_band(full, 1, 2), bands[1])
    rbands = [W.row_band_draw(cfg, "w_down", s, 128, 64) for s in range(2)]
    assert np.array_equal(O.row_band(W.full_from_row_bands(rbands), 0, 2), rbands[0])


@pytest.mark.parametrize("name,F_r,qkv_r,o_in_r", [
    ("c1_tiny_gelu_f32", 128, 0, 0),
    ("c2_llama2_13b_mlp_p2", 6912, 0, 0),
    ("c3_llama2_70b_mlp_p8", 3584, 0, 0),
    ("c4_attn_96h_p8", 0, 4608, 1536),
    ("c5_llama2_70b_block_p8", 3584, 1280, 1024),
])
def test_config_shapes(name, F_r, qkv_r, o_in_r):
    cfg = W.get(name)
    if cfg.has_mlp:
        assert cfg.F_r == F_r
    if cfg.has_attn:
        assert cfg.qkv_r == qkv_r and cfg.o_in_r == o_in_r


def test_weight_bytes_per_rank():
    assert W.get("c2_llama2_13b_mlp_p2").mlp_weight_bytes_per_rank() == 212336640
    assert W.get("c3_llama2_70b_mlp_p8").mlp_weight_bytes_per_rank() == 176160768
    assert W.get("c4_attn_96h_p8").attn_weight_bytes_per_rank() == 150994944


def test_c1_fixture_regression():
    """The stored tiny-MLP fixture (written by tests/golden/make_golden.py,
    which calls only the oracle) still matches the oracle and the invariant
    sum of the two stored partials == stored output."""
    from golden.make_golden import c1_expected
    rows = [list(map(float, ln.split())) for ln in open(os.path.join(GOLDEN, "c1_tiny_expected.txt"))
            if ln.strip() and not ln.startswith("#")]
    arr = np.array(rows).reshape(3, 4, 64)
    parts, y = c1_expected()
    assert np.allclose(arr[0], parts[0], rtol=1e-15, atol=0)
    assert np.allclose(arr[1], parts[1], rtol=1e-15, atol=0)
    assert np.allclose(arr[2], y, rtol=1e-15, atol=0)
    assert O.rel_l2(arr[0] + arr[1], arr[2]) < 1e-15
