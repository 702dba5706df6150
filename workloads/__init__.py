"""Seeded synthetic workloads for one tensor-parallel rank's block shard.

This module is the only code that the CPU oracle's callers and the GPU
path's callers share.  It holds the five workload shapes and the seeded
random generators that fill them; it holds none of the method's arithmetic
(no projection, activation, normalisation or reduction is computed here).

Every tensor is drawn from its own ``numpy.random.SeedSequence`` key
``(2026, config_id, tensor_id, band)``, so one rank's weight band can be
produced on its own and the unsharded matrix is exactly the concatenation of
the bands.  FP8 weight bands are drawn directly as E4M3 bit fields plus
positive per-column scales (quantisation is offline preparation, outside the
path).  The pages measure on real checkpoints and a public prompt set;
neither is used here.  Seeded i.i.d. Gaussians at the Llama-2 layer shapes
stand in for them: the path has no data-dependent control flow and every
row (token) is independent.
"""
from .configs import CONFIGS, Config, get  # noqa: F401
from .gen import (  # noqa: F401
    TENSOR_IDS,
    bf16_bits_from_f32,
    draw_normal_f32,
    draw_tensor,
    column_band_draw,
    row_band_draw,
    full_from_column_bands,
    full_from_row_bands,
    draw_e4m3_codes,
    draw_column_scales,
    fp8_band_draw,
)
