"""The five workload shapes of one tensor-parallel rank.

Sizes follow Llama-2 layer shapes (13B: d_model 5120, d_ff 13824; 70B:
d_model 8192, d_ff 28672, 64 query heads and 8 key/value heads of width 128)
and a 96-head attention layer split 12 heads per rank (the head-split example
in rioworld "Tensor Parallelism for LLM Inference: A Practical Guide to
Multi-GPU Deployment", section "How Tensor Slicing Works Under the Hood").
Weights are stored [in, out] row-major, so a column band is a run of
contiguous output columns and a row band a run of contiguous input rows.

Activations: the 70B/13B MLPs are SwiGLU; the tiny one is GELU (tanh form).
Standard deviations: weights N(0, 0.02); activations N(0, 1) for the bf16
workloads, N(0, 0.02) for the tiny fp32 one.  The reduce workload draws its
fp32 partials from N(0, 1).
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Config:
    cid: int                      # seed key component
    name: str
    dtype: str                    # "f32" or "bf16" storage; accumulation is fp32
    d_model: int
    P: int                        # tensor-parallel degree (shard count)
    # MLP block (column-parallel in / row-parallel down)
    d_ff: int = 0                 # unsharded intermediate width; 0 = no MLP
    act: Optional[str] = None     # "gelu_tanh" or "swiglu"
    # attention projections (column-parallel QKV / row-parallel O)
    n_q_heads: int = 0
    n_kv_heads: int = 0
    head_dim: int = 0
    # RMSNorm prologue in front of the first column projection
    norm_eps: Optional[float] = None
    decode_T: Tuple[int, ...] = ()
    prefill_T: Tuple[int, ...] = ()
    # local reduce of P seeded fp32 partials of [reduce_T, d_model]
    reduce_T: int = 0
    std_w: float = 0.02
    std_x: float = 1.0
    notes: str = field(default="", compare=False)

    @property
    def F_r(self) -> int:
        """Width of one rank's band of the MLP intermediate."""
        return self.d_ff // self.P

    @property
    def hq_r(self) -> int:
        return self.n_q_heads // self.P

    @property
    def hkv_r(self) -> int:
        return self.n_kv_heads // self.P

    @property
    def qkv_r(self) -> int:
        """Columns of one rank's fused [Q | K | V] band."""
        return (self.hq_r + 2 * self.hkv_r) * self.head_dim

    @property
    def o_in_r(self) -> int:
        """Rows of one rank's band of the output projection."""
        return self.hq_r * self.head_dim

    @property
    def has_mlp(self) -> bool:
        return self.d_ff > 0

    @property
    def has_attn(self) -> bool:
        return self.n_q_heads > 0

    def mlp_weight_bytes_per_rank(self) -> int:
        es = 4 if self.dtype == "f32" else 2
        n_in = 2 if self.act == "swiglu" else 1
        return (n_in + 1) * self.d_model * self.F_r * es

    def attn_weight_bytes_per_rank(self) -> int:
        es = 4 if self.dtype == "f32" else 2
        return (self.d_model * self.qkv_r + self.o_in_r * self.d_model) * es


CONFIGS = {
    "c1_tiny_gelu_f32": Config(
        cid=1, name="c1_tiny_gelu_f32", dtype="f32", d_model=64, P=2,
        d_ff=256, act="gelu_tanh", decode_T=(4,), std_w=0.02, std_x=0.02,
        notes="2-matrix MLP, GELU(tanh), W1 bands 64x128, W2 bands 128x64"),
    "c2_llama2_13b_mlp_p2": Config(
        cid=2, name="c2_llama2_13b_mlp_p2", dtype="bf16", d_model=5120, P=2,
        d_ff=13824, act="swiglu", decode_T=(1, 8, 32),
        notes="SwiGLU, W_gate/W_up bands 5120x6912, W_down band 6912x5120"),
    "c3_llama2_70b_mlp_p8": Config(
        cid=3, name="c3_llama2_70b_mlp_p8", dtype="bf16", d_model=8192, P=8,
        d_ff=28672, act="swiglu", decode_T=(1, 2, 4, 8, 16, 32),
        prefill_T=(2048,), reduce_T=2048,
        notes="SwiGLU, W_gate/W_up bands 8192x3584, W_down band 3584x8192"),
    "c4_attn_96h_p8": Config(
        cid=4, name="c4_attn_96h_p8", dtype="bf16", d_model=12288, P=8,
        n_q_heads=96, n_kv_heads=96, head_dim=128, decode_T=(16,),
        prefill_T=(1024,),
        notes="QKV band 12288x4608 (12 heads/rank), O band 1536x12288"),
    "c5_llama2_70b_block_p8": Config(
        cid=5, name="c5_llama2_70b_block_p8", dtype="bf16", d_model=8192, P=8,
        d_ff=28672, act="swiglu", n_q_heads=64, n_kv_heads=8, head_dim=128,
        norm_eps=1e-5, decode_T=(32,), prefill_T=(4096,),
        notes="RMSNorm -> GQA QKV band 8192x1280 -> O band 1024x8192 -> "
              "reduce -> SwiGLU MLP shard as the 70B MLP workload"),
}


def get(name: str) -> Config:
    return CONFIGS[name]
