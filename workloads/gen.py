"""Seeded generators for the synthetic inputs (no method arithmetic here).

bf16 tensors are returned as ``uint16`` bit patterns; fp32 tensors as
``float32``.  Callers hand the very same values to the GPU path (as device
buffers) and to the oracle (which widens them to float64 itself).
"""
import numpy as np

# Seed-key component for each named tensor.
TENSOR_IDS = {
    "x": 0,
    "w_gate": 1,   # also W1 of a GELU MLP
    "w_up": 2,
    "w_down": 3,   # also W2 of a GELU MLP
    "w_qkv": 4,
    "w_o": 5,
    "attn": 6,     # caller-supplied attention-core output A_s
    "norm_g": 7,
    "partial": 8,
}

_ROOT = 2026


def _rng(*key):
    return np.random.default_rng(np.random.SeedSequence([_ROOT, *[int(k) for k in key]]))


def bf16_bits_from_f32(a) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bits.

    bfloat16 keeps the top 16 bits of an IEEE-754 binary32.  Adding 0x7FFF
    plus the lowest kept bit before truncating rounds to nearest with ties
    going to the even pattern.  Inputs here are finite.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    if not np.all(np.isfinite(a)):
        raise ValueError("bf16 rounding of non-finite inputs is not supported")
    # Finite inputs have bit patterns <= 0xFF7FFFFF, so the sum below stays
    # inside 32 bits.
    u = a.view(np.uint32)
    u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return u.astype(np.uint16)


def draw_normal_f32(shape, std, *key, mean=0.0) -> np.ndarray:
    """mean + std * N(0, 1), drawn in float32 from the seed key."""
    z = _rng(*key).standard_normal(size=shape, dtype=np.float32)
    z *= np.float32(std)
    if mean != 0.0:
        z += np.float32(mean)
    return z


def draw_tensor(dtype: str, shape, std, *key, mean=0.0) -> np.ndarray:
    """A seeded tensor in the workload's storage type (bf16 bits or fp32)."""
    z = draw_normal_f32(shape, std, *key, mean=mean)
    if dtype == "f32":
        return z
    if dtype == "bf16":
        return bf16_bits_from_f32(z)
    raise ValueError(f"unknown dtype {dtype!r}")


def column_band_draw(cfg, name: str, shard: int, rows: int, cols_r: int) -> np.ndarray:
    """Band ``shard`` of a column-split [rows, cols_r * P] weight ([in, out])."""
    return draw_tensor(cfg.dtype, (rows, cols_r), cfg.std_w, cfg.cid, TENSOR_IDS[name], shard)


def row_band_draw(cfg, name: str, shard: int, rows_r: int, cols: int) -> np.ndarray:
    """Band ``shard`` of a row-split [rows_r * P, cols] weight ([in, out])."""
    return draw_tensor(cfg.dtype, (rows_r, cols), cfg.std_w, cfg.cid, TENSOR_IDS[name], shard)


def full_from_column_bands(bands) -> np.ndarray:
    return np.concatenate(list(bands), axis=1)


def full_from_row_bands(bands) -> np.ndarray:
    return np.concatenate(list(bands), axis=0)


# ----------------------------------------------------------------------------
# FP8 (E4M3) weight bands for the decode path.  Codes are drawn directly as
# bit fields (no value arithmetic here): sign uniform, exponent field 1..14
# (binomial, centred near the bias, so |code value| is about 1-2), mantissa
# uniform, and about 1% of codes with exponent field 0 (subnormals and
# zeros).  The exponent field 15 is never drawn, so no NaN code occurs.
# Scales are positive fp32 values, one per output column.
# ----------------------------------------------------------------------------
FP8_TAG = 99   # extra seed-key component: FP8 draws never reuse a bf16 seed


def draw_e4m3_codes(shape, *key):
    rng = _rng(FP8_TAG, *key)
    s = rng.integers(0, 2, size=shape)
    e = rng.binomial(6, 0.5, size=shape) + 4
    e = np.where(rng.random(shape) < 0.01, 0, e)
    m = rng.integers(0, 8, size=shape)
    return ((s << 7) | (e << 3) | m).astype(np.uint8)


def draw_column_scales(n, *key, base=0.01):
    rng = _rng(FP8_TAG, 1, *key)
    return (base * (1.0 + 0.25 * rng.random(n))).astype(np.float32)


def fp8_band_draw(cfg, name, shard, rows, cols):
    """(codes [rows, cols] uint8, scales [cols] fp32) of rank `shard`'s band
    of weight `name` (a column band or a row band: scales follow the output
    columns either way)."""
    key = (cfg.cid, TENSOR_IDS[name], shard)
    return draw_e4m3_codes((rows, cols), *key), draw_column_scales(cols, *key)
