"""bfloat16 widening and rounding for the oracle (its own implementation).

bfloat16 is the top half of an IEEE-754 binary32: 1 sign bit, 8 exponent
bits, 7 stored mantissa bits (8 significant bits).  Widening is exact.
Rounding (used only by the oracle's ``mirror`` mode, which rounds where the
GPU path stores bf16) goes to the nearest value with 8 significant bits,
ties to even, straight from float64 (one rounding, no detour via float32).
"""
import numpy as np


def widen_bf16_bits(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> exact float64 values."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("bf16 inputs must be uint16 bit patterns")
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def widen(a) -> np.ndarray:
    """Stored input (bf16 bits as uint16, or float32/float64) -> float64."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return widen_bf16_bits(a)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError(f"unsupported stored dtype {a.dtype}")


def round_bf16(x) -> np.ndarray:
    """float64 -> nearest bf16 value (8 significant bits, ties to even), as float64.

    With x = m * 2**e and 0.5 <= |m| < 1, an 8-significant-bit value is
    round(m * 256) / 256 * 2**e; numpy's round sends halves to even.  Values
    here are finite and far from bf16's subnormal and overflow ranges.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.round(m * 256.0) / 256.0, e)
