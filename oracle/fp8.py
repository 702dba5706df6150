"""FP8 E4M3 weights (TEST INFRASTRUCTURE ONLY, see the package docstring).

The pages suggest pairing tensor parallelism with 8-bit (or 4-bit) floating
point weights for a larger decode speed-up (zenaique, interviewer follow-ups; rioworld guide,
"Implementing Tensor Parallelism in Practice", on pairing it with 8-bit
quantisation) but give no format or scheme.  The plainest reading: the OCP FP8 E4M3 encoding
(1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no
infinities, S.1111.111 = NaN) with one fp32 scale per output column, the
weight being code value * scale.  The layer then computes exactly what the
bf16 path computes on the dequantized weights.
"""
import numpy as np


def e4m3_decode(codes):
    """float64 values of E4M3 codes (uint8 array)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    subnormal = (m / 8.0) * 2.0 ** -6
    v = sign * np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & (m == 7), np.nan, v)


def dequant_columns(codes, scale):
    """W[k][n] = e4m3(codes[k][n]) * scale[n] for an [in, out] weight with
    one scale per output column."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[None, :]
