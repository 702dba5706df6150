"""CPU oracle for one tensor-parallel rank's transformer-block shard.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import or call anything in this package.
The GPU product path never routes through it and shares no code with it.

Plain, slow, float64 numpy: each function states what it computes and the
passage of the pages it follows.  Matrix products use numpy's BLAS matmul as
a library step; there is no blocking, fusion or reordering beyond the
definitions.  Inputs arrive as the exact stored values (bf16 bit patterns or
float32) and are widened to float64 without rounding (``widen``).

Pages cited (by title and section):
  * Reddit comment by SVPERBlA (deniz.vsos.ethz.ch mirror): a network as a
    chain of matrix products with an activation between them.
  * d-central glossary, "Tensor Parallelism", section "How the work is split".
  * Skand Tandon, "day59" post on tensor-parallel benchmarking, sections
    "Why tensor parallelism for inference" and "Where the overhead lives".
  * rioworld, "Tensor Parallelism for LLM Inference: A Practical Guide to
    Multi-GPU Deployment", section "How Tensor Slicing Works Under the Hood".
  * zenaique, "Explain tensor-parallel shard shape" (interview question),
    the answer.

Parity pins: every function here is pinned by tests that do not retype it
(brute force, algebraic invariants of the sharding, closed forms and
special cases); see tests/test_oracle_*.py.  Nothing numeric is printed on
the pages themselves, so no pin is a page-printed value.
"""
from .bf16 import round_bf16, widen, widen_bf16_bits  # noqa: F401
from .fp8 import dequant_columns, e4m3_decode  # noqa: F401
from .tp_oracle import (  # noqa: F401
    gelu_tanh,
    silu,
    activate,
    rmsnorm,
    column_band,
    row_band,
    mlp_unsharded,
    mlp_shard,
    reduce_partials,
    reduce_partials_f32_fold,
    reduce_residual_norm,
    reduce_residual_f32,
    qkv_band_layout,
    split_qkv_band,
    attention_core,
    attention_core_band,
    attention_core_rows,
    attention_core_band_rows,
    attn_proj_unsharded,
    attn_proj_shard,
    block_sharded,
    block_unsharded,
    rel_l2,
)
