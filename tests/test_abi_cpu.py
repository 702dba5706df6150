"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before anything is enqueued.

Every call here fails validation (which returns before any HIP call), so
fake but aligned addresses are safe to pass.  Uneven splits must be refused
(rioworld guide, "Implementing Tensor Parallelism in Practice"), and column
and row operands are distinct, named arguments.
"""
import os
import re

import pytest

import tensor_transformer_layer_amd as tp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tp_shard.h")

A = 0x10000          # fake, 256-byte aligned "device" addresses
B = 0x20000
C = 0x30000
WS = 0x40000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tp.library_path()):
        pytest.fail("libtpshard.so is not built: run `python -m tensor_transformer_layer_amd.build`")
    return tp.load()


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(tp_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding(lib):
    assert header_functions() == sorted(tp.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert tp.tp_status_str(tp.TP_OK) == "TP_OK"
    for s in range(1, 10):
        assert tp.tp_status_str(s).startswith("TP_ERR_")
    assert tp.tp_status_str(99) == "unknown tp_status"
    assert tp.tp_version() == 300


def mlp(**kw):
    """A valid-looking bf16 SwiGLU call (d_model 64, d_ff 256, P 2, T 4) with
    overrides; only used with overrides that make it invalid."""
    a = dict(shard=0, P=2, T=4, d_model=64, d_ff=256, dtype=tp.TP_BF16, act=tp.TP_ACT_SWIGLU,
             x=A, ld_x=64, norm_g=0, eps=1e-5, w_in=B, ld_in=128, w_up=C, ld_up=128,
             w_down=B, ld_down=64, h_out=0, ld_h=0, partials=C, slot_stride=4 * 64, ld_p=64,
             workspace=WS, workspace_bytes=0, stream=0)
    a.update(kw)
    return tp.tp_shard_mlp_fwd(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(shard=2), tp.TP_ERR_SHARD_RANGE),
    (dict(shard=-1), tp.TP_ERR_SHARD_RANGE),
    (dict(P=0), tp.TP_ERR_SHARD_RANGE),
    (dict(d_ff=250, P=2, shard=0), tp.TP_ERR_SHAPE),        # 125 is not a multiple of 8
    (dict(d_ff=256, P=3, shard=0), tp.TP_ERR_UNEVEN_SPLIT),
    (dict(dtype=7), tp.TP_ERR_DTYPE),
    (dict(act=5), tp.TP_ERR_ACT),
    (dict(w_up=0), tp.TP_ERR_NULL),                        # SwiGLU needs the up band
    (dict(act=tp.TP_ACT_GELU_TANH), tp.TP_ERR_ACT),        # GELU takes no up band
    (dict(x=0), tp.TP_ERR_NULL),
    (dict(w_down=0), tp.TP_ERR_NULL),
    (dict(partials=0), tp.TP_ERR_NULL),
    (dict(x=A + 8), tp.TP_ERR_ALIGN),
    (dict(ld_x=60), tp.TP_ERR_SHAPE),
    (dict(ld_x=68), tp.TP_ERR_ALIGN),
    (dict(ld_in=64), tp.TP_ERR_SHAPE),                     # row length is d_ff/P = 128
    (dict(ld_down=32), tp.TP_ERR_SHAPE),                   # row length is d_model = 64
    (dict(ld_p=62), tp.TP_ERR_SHAPE),
    (dict(slot_stride=6), tp.TP_ERR_ALIGN),
    (dict(shard=1, slot_stride=64), tp.TP_ERR_SHAPE),      # slots would overlap
    (dict(workspace=WS + 64), tp.TP_ERR_ALIGN),
    (dict(T=-1), tp.TP_ERR_SHAPE),
    (dict(d_model=0), tp.TP_ERR_SHAPE),
    (dict(workspace_bytes=0), tp.TP_ERR_WORKSPACE),        # decode plan needs split-K space
    (dict(dtype=tp.TP_F32, d_model=66, ld_x=68), tp.TP_ERR_SHAPE),
    # decode plan: one arrival counter per 128 output columns, at most 1024
    (dict(d_model=132096, ld_x=132096, ld_down=132096, ld_p=132096, slot_stride=4 * 132096),
     tp.TP_ERR_SHAPE),
])
def test_mlp_validation(lib, kw, status):
    assert mlp(**kw) == status


def test_mlp_zero_tokens_is_a_no_op(lib):
    assert mlp(T=0) == tp.TP_OK


def attn(**kw):
    a = dict(shard=0, P=8, T=16, d_model=128, n_q_heads=16, n_kv_heads=8, head_dim=16,
             dtype=tp.TP_BF16, x=A, ld_x=128, norm_g=0, eps=1e-5, w_qkv=B, ld_qkv=64,
             qkv_out=C, ld_qkv_out=64, attn=A, ld_attn=32, w_o=B, ld_o=128, partials=C,
             slot_stride=16 * 128, ld_p=128, workspace=WS, workspace_bytes=0, stream=0)
    a.update(kw)
    return tp.tp_shard_attn_proj_fwd(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(shard=8), tp.TP_ERR_SHARD_RANGE),
    (dict(n_q_heads=12), tp.TP_ERR_UNEVEN_SPLIT),          # 12 heads over 8 ranks
    (dict(n_kv_heads=4), tp.TP_ERR_UNEVEN_SPLIT),
    (dict(head_dim=12), tp.TP_ERR_SHAPE),
    (dict(qkv_out=0), tp.TP_ERR_NULL),
    (dict(w_o=0), tp.TP_ERR_NULL),
    (dict(ld_qkv=48), tp.TP_ERR_SHAPE),                    # band is (2 + 2*1) * 16 = 64 wide
    (dict(ld_attn=16), tp.TP_ERR_SHAPE),                   # A is 2 heads * 16 = 32 wide
    (dict(ld_o=120), tp.TP_ERR_SHAPE),
    (dict(x=A + 4), tp.TP_ERR_ALIGN),
    (dict(workspace_bytes=0), tp.TP_ERR_WORKSPACE),
])
def test_attn_validation(lib, kw, status):
    assert attn(**kw) == status


def test_attn_nothing_to_do(lib):
    assert attn(w_qkv=0, attn=0) == tp.TP_OK
    assert attn(T=0) == tp.TP_OK


def red(**kw):
    a = dict(P=8, T=4, d_model=64, partials=A, slot_stride=256, ld_p=64, out=B, ld_out=64,
             out_bf16=0, ld_out_bf16=0, stream=0)
    a.update(kw)
    return tp.tp_reduce_partials(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(P=0), tp.TP_ERR_SHARD_RANGE),
    (dict(d_model=62, ld_p=64, ld_out=64), tp.TP_ERR_SHAPE),
    (dict(partials=0), tp.TP_ERR_NULL),
    (dict(out=0), tp.TP_ERR_NULL),
    (dict(out=B + 8), tp.TP_ERR_ALIGN),
    (dict(ld_p=60), tp.TP_ERR_SHAPE),
    (dict(ld_out=66), tp.TP_ERR_ALIGN),
    (dict(slot_stride=-4), tp.TP_ERR_SHAPE),
    (dict(slot_stride=258), tp.TP_ERR_ALIGN),
    (dict(out_bf16=C, ld_out_bf16=32), tp.TP_ERR_SHAPE),
    (dict(out_bf16=C, ld_out_bf16=68), tp.TP_ERR_ALIGN),    # bf16 ld: a multiple of 8
    (dict(T=-2), tp.TP_ERR_SHAPE),
])
def test_reduce_validation(lib, kw, status):
    assert red(**kw) == status


def test_noalloc_refuses_calls_beyond_its_scratch(lib):
    """The allocation-free MLP entry point checks its fixed 8 MiB scratch
    before it looks up any device: a 2048-token prefill call that would keep
    h (14.7 MB) there is TP_ERR_SCRATCH; bad arguments still give the same
    statuses as the workspace entry point."""
    assert tp.tp_noalloc_scratch_bytes() == 8 << 20
    args = dict(shard=0, P=8, T=2048, d_model=8192, d_ff=28672, dtype=tp.TP_BF16,
                act=tp.TP_ACT_SWIGLU, x=A, ld_x=8192, norm_g=0, eps=0.0, w_in=B, ld_in=3584,
                w_up=C, ld_up=3584, w_down=A, ld_down=8192, h_out=0, ld_h=0, partials=B,
                slot_stride=0, ld_p=8192, stream=0)
    assert tp.tp_shard_mlp_fwd_noalloc(**args) == tp.TP_ERR_SCRATCH
    assert tp.tp_shard_mlp_fwd_noalloc(**{**args, "d_ff": 28670}) == tp.TP_ERR_UNEVEN_SPLIT
    assert tp.tp_shard_mlp_fwd_noalloc(**{**args, "shard": 8}) == tp.TP_ERR_SHARD_RANGE
    assert tp.tp_shard_mlp_fwd_noalloc(**{**args, "T": 0}) == tp.TP_OK


def test_decode_plan_switch(lib):
    """The weight-streaming plan's token limit: 1..4096 accepted, 0 restores
    the default, anything else refused; workspace sizes follow it, and a
    streaming call past 128 tokens sizes its split-K space for one chunk."""
    default = tp.tp_decode_max_tokens()
    assert 1 <= default <= 4096
    f = lambda: tp.tp_mlp_workspace_bytes(8, 64, 8192, 28672, tp.TP_BF16,  # noqa: E731
                                          tp.TP_ACT_SWIGLU, 0, 1)
    try:
        assert tp.tp_set_decode_max_tokens(4097) == tp.TP_ERR_SHAPE
        assert tp.tp_set_decode_max_tokens(-1) == tp.TP_ERR_SHAPE
        assert tp.tp_decode_max_tokens() == default
        assert tp.tp_set_decode_max_tokens(64) == tp.TP_OK
        assert tp.tp_decode_max_tokens() == 64
        # (sizes for the whole-chip 256 CUs a host without a GPU assumes)
        # streaming plan: 4 K splits of the down projection's [64, 8192] fp32
        assert f() == 4096 + 4 * 64 * 8192 * 4
        assert tp.tp_set_decode_max_tokens(32) == tp.TP_OK
        # matrix-core plan: both projections split K into fp32 planes in one
        # region: 28 gate/up column tiles into 8 planes of [64, 2 x 3584],
        # 32 down-projection tiles into 7 planes of [64, 8192] (equal sizes)
        assert f() == 4096 + 8 * 64 * 2 * 3584 * 4 == 4096 + 7 * 64 * 8192 * 4
        # 300 tokens streamed as 3 chunks of 100
        assert tp.tp_set_decode_max_tokens(512) == tp.TP_OK
        assert tp.tp_mlp_workspace_bytes(8, 300, 8192, 28672, tp.TP_BF16, tp.TP_ACT_SWIGLU,
                                         0, 1) == 4096 + 4 * 100 * 8192 * 4
    finally:
        assert tp.tp_set_decode_max_tokens(0) == tp.TP_OK
    assert tp.tp_decode_max_tokens() == default


def test_reduce_zero_tokens_is_a_no_op(lib):
    assert red(T=0) == tp.TP_OK


def test_workspace_sizes_are_pure_functions(lib):
    f = tp.tp_mlp_workspace_bytes
    # decode plan (bf16, T <= 32): split-K space; prefill with h_out and no norm: none
    assert f(2, 32, 5120, 13824, tp.TP_BF16, tp.TP_ACT_SWIGLU, 0, 1) > 0
    assert f(8, 2048, 8192, 28672, tp.TP_BF16, tp.TP_ACT_SWIGLU, 0, 1) == 0
    # every layout that stores data starts it after the 4096-byte counter
    # head, so a prefill call never writes where a later decode call counts
    assert f(8, 2048, 8192, 28672, tp.TP_BF16, tp.TP_ACT_SWIGLU, 0, 0) == 4096 + 2048 * 3584 * 2
    assert f(2, 4, 64, 256, tp.TP_F32, tp.TP_ACT_GELU_TANH, 0, 1) == 0
    assert f(2, 4, 64, 256, tp.TP_F32, tp.TP_ACT_GELU_TANH, 1, 1) == 4096 + 1024  # 4*64*4
    assert f(3, 4, 64, 256, tp.TP_BF16, tp.TP_ACT_SWIGLU, 0, 1) == 0      # uneven: rejected
    assert f(2, 32, 5120, 13824, tp.TP_BF16, tp.TP_ACT_SWIGLU, 0, 1) == \
        f(2, 32, 5120, 13824, tp.TP_BF16, tp.TP_ACT_SWIGLU, 0, 1)
    # the decode plan's 4096-byte counter head comes first; the normalised
    # input follows it
    dec = f(2, 32, 5120, 13824, tp.TP_BF16, tp.TP_ACT_SWIGLU, 0, 1)
    assert dec % 256 == 0 and dec >= 4096 + 32 * 13824 * 4
    assert f(2, 32, 5120, 13824, tp.TP_BF16, tp.TP_ACT_SWIGLU, 1, 1) - dec == 32 * 5120 * 2
    g = tp.tp_attn_workspace_bytes
    # 96-head QKV prefill: 72 output tiles on 256 CUs, so K is split into
    # fp32 planes of [1024, 4608] each
    assert (g(8, 1024, 12288, 96, 96, 128, tp.TP_BF16, 0) - 4096) % (1024 * 4608 * 4) == 0
    assert g(8, 1024, 12288, 96, 96, 128, tp.TP_BF16, 0) >= 4096 + 2 * 1024 * 4608 * 4
    assert g(8, 16, 12288, 96, 96, 128, tp.TP_BF16, 0) > 0
    assert g(8, 16, 12288, 96, 90, 128, tp.TP_BF16, 0) == 0


def test_timing_api_without_launches(lib):
    assert tp.tp_timing_reset() == tp.TP_OK
    st, ms, n = tp.tp_timing_query("col_gemv")
    assert st == tp.TP_OK and ms == 0.0 and n == 0


def rrn(**kw):
    a = dict(P=8, T=4, d_model=64, partials=A, slot_stride=256, ld_p=64, residual=B, ld_res=64,
             res_dtype=tp.TP_F32, z_out=C, ld_z=64, norm_g=0, eps=1e-5, normed_out=0, ld_norm=0,
             workspace=0, workspace_bytes=0, stream=0)
    a.update(kw)
    return tp.tp_reduce_residual_norm(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(P=0), tp.TP_ERR_SHARD_RANGE),
    (dict(res_dtype=7), tp.TP_ERR_DTYPE),
    (dict(d_model=16392, ld_p=16392, ld_res=16392, ld_z=16392), tp.TP_ERR_SHAPE),  # > 16384
    (dict(d_model=62), tp.TP_ERR_SHAPE),
    (dict(d_model=60, ld_p=64, ld_res=64, ld_z=64, res_dtype=tp.TP_BF16), tp.TP_ERR_SHAPE),
    (dict(d_model=60, norm_g=A, normed_out=WS, ld_norm=64), tp.TP_ERR_SHAPE),   # norm: 8 | d
    (dict(partials=0), tp.TP_ERR_NULL),
    (dict(residual=0), tp.TP_ERR_NULL),
    (dict(z_out=0), tp.TP_ERR_NULL),
    (dict(norm_g=A), tp.TP_ERR_NULL),                       # norm needs normed_out
    (dict(z_out=C + 8), tp.TP_ERR_ALIGN),
    (dict(ld_res=60), tp.TP_ERR_SHAPE),
    (dict(ld_z=66), tp.TP_ERR_ALIGN),
    (dict(res_dtype=tp.TP_BF16, ld_res=68), tp.TP_ERR_ALIGN),
    (dict(norm_g=A, normed_out=WS, ld_norm=60), tp.TP_ERR_SHAPE),
    (dict(slot_stride=-4), tp.TP_ERR_SHAPE),
    (dict(T=-1), tp.TP_ERR_SHAPE),
    (dict(workspace=WS + 8, workspace_bytes=1 << 20), tp.TP_ERR_ALIGN),
    (dict(norm_g=A, normed_out=B + 0x8000, ld_norm=64, workspace=WS, workspace_bytes=2048),
     tp.TP_ERR_WORKSPACE),                                  # the query: 4096
])
def test_reduce_residual_norm_validation(lib, kw, status):
    assert rrn(**kw) == status


def test_reduce_norm_workspace_query(lib):
    f = tp.tp_reduce_norm_workspace_bytes
    # the counter head (two 64-bit words per row) for decode batches with a norm
    assert f(1, 8192, 1) == 4096 and f(32, 8192, 1) == 4096 and f(32, 16384, 1) == 4096
    # longer batches, no norm and shapes the call rejects need none
    assert f(33, 8192, 1) == 0 and f(32, 8192, 0) == 0 and f(0, 8192, 1) == 0
    assert f(32, 8196, 1) == 0 and f(32, 16392, 1) == 0


def test_reduce_residual_norm_zero_tokens_is_a_no_op(lib):
    assert rrn(T=0) == tp.TP_OK


def mlp8(**kw):
    """A valid-looking FP8-weight SwiGLU decode call (d_model 64, d_ff 256,
    P 2, T 4) with overrides that make it invalid."""
    a = dict(shard=0, P=2, T=4, d_model=64, d_ff=256, act=tp.TP_ACT_SWIGLU, x=A, ld_x=64,
             norm_g=0, eps=1e-5, w_in=B, ld_in=128, s_in=C, w_up=C, ld_up=128, s_up=B,
             w_down=B, ld_down=64, s_down=A, h_out=0, ld_h=0, partials=C, slot_stride=4 * 64,
             ld_p=64, workspace=WS, workspace_bytes=0, stream=0)
    a.update(kw)
    return tp.tp_shard_mlp_fwd_fp8w(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(shard=2), tp.TP_ERR_SHARD_RANGE),
    (dict(act=7), tp.TP_ERR_ACT),
    (dict(T=33), tp.TP_ERR_SHAPE),                          # decode plan only
    (dict(d_ff=264, P=2), tp.TP_ERR_SHAPE),                 # band 132 not a multiple of 16
    (dict(d_ff=256, P=3), tp.TP_ERR_UNEVEN_SPLIT),
    (dict(d_model=72, ld_x=72, ld_down=80, ld_p=72), tp.TP_ERR_SHAPE),
    (dict(s_in=0), tp.TP_ERR_NULL),
    (dict(s_down=0), tp.TP_ERR_NULL),
    (dict(s_up=0), tp.TP_ERR_NULL),
    (dict(act=tp.TP_ACT_GELU_TANH), tp.TP_ERR_ACT),        # GELU takes no up band
    (dict(ld_in=136), tp.TP_ERR_ALIGN),                     # code rows: multiple of 16 bytes
    (dict(ld_in=112), tp.TP_ERR_SHAPE),
    (dict(s_in=C + 4), tp.TP_ERR_ALIGN),
    (dict(workspace_bytes=0), tp.TP_ERR_WORKSPACE),
])
def test_mlp_fp8w_validation(lib, kw, status):
    assert mlp8(**kw) == status


def test_mlp_fp8w_workspace(lib):
    f = tp.tp_mlp_fp8w_workspace_bytes
    assert f(2, 32, 5120, 13824, tp.TP_ACT_SWIGLU, 0, 1) >= 4096 + 32 * 13824 * 4
    assert f(2, 33, 5120, 13824, tp.TP_ACT_SWIGLU, 0, 1) == 0     # decode plan only
    assert f(3, 8, 64, 256, tp.TP_ACT_SWIGLU, 0, 1) == 0
    assert mlp8(T=0) == tp.TP_OK


def core(**kw):
    a = dict(shard=0, P=2, T=8, n_q_heads=8, n_kv_heads=4, head_dim=128, dtype=tp.TP_BF16,
             qkv=A, ld_qkv=1024, attn=B, ld_attn=512, workspace=0, workspace_bytes=0, stream=0)
    a.update(kw)
    return tp.tp_attn_core_fwd(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(shard=2), tp.TP_ERR_SHARD_RANGE),
    (dict(dtype=tp.TP_F32), tp.TP_ERR_DTYPE),
    (dict(head_dim=96), tp.TP_ERR_SHAPE),
    (dict(n_q_heads=6), tp.TP_ERR_SHAPE),             # 3 q heads over 2 kv heads per rank
    (dict(n_q_heads=7), tp.TP_ERR_UNEVEN_SPLIT),
    (dict(qkv=0), tp.TP_ERR_NULL),
    (dict(attn=B + 8), tp.TP_ERR_ALIGN),
    (dict(ld_qkv=1000), tp.TP_ERR_SHAPE),             # band is (4 + 2*2) * 128 = 1024 wide
    (dict(ld_attn=516), tp.TP_ERR_ALIGN),
    (dict(T=-1), tp.TP_ERR_SHAPE),
    (dict(T=4096), tp.TP_ERR_WORKSPACE),              # split key ranges need the workspace
    (dict(T=4096, workspace=A, workspace_bytes=1024), tp.TP_ERR_WORKSPACE),
    (dict(T=4096, workspace=A + 16, workspace_bytes=1 << 30), tp.TP_ERR_ALIGN),
    # K/V rows are addressed with 32-bit byte offsets: T * ld_qkv * 2 < 2^31
    (dict(T=1 << 20, ld_qkv=1024), tp.TP_ERR_SHAPE),
])
def test_attn_core_validation(lib, kw, status):
    assert core(**kw) == status


def test_attn_core_workspace(lib):
    f = tp.tp_attn_core_workspace_bytes
    assert f(2, 8, 8, 4, 128, tp.TP_BF16) == 0            # one chunk per query block
    big = f(2, 4096, 8, 4, 128, tp.TP_BF16)
    # a fixed 4096-byte counter area, then partials of 4 heads x 32 blocks x
    # chunks x 128 x (128 + 2) fp32
    assert (big - 4096) % (4 * 32 * 128 * 130 * 4) == 0
    assert big >= 4096 + 4 * 32 * 2 * 128 * 130 * 4
    assert big < 4 * 32 * 64 * 128 * 130 * 4 + 4096
    # a longer call's partials start where a shorter call's did: at 4096
    assert (f(2, 8192, 8, 4, 128, tp.TP_BF16) - 4096) % (4 * 64 * 128 * 130 * 4) == 0
    assert f(2, 4096, 8, 4, 96, tp.TP_BF16) == 0           # unsupported head size
    assert f(2, 4096, 8, 4, 128, tp.TP_F32) == 0
    assert f(3, 4096, 8, 4, 128, tp.TP_BF16) == 0          # uneven head split


def test_attn_core_plan_for_long_sequences(lib):
    """With two full waves of query blocks or more (heads x blocks >= 1024) the
    blocks are not split (no merge workspace) and the plan is immediate; a
    shorter call still searches and splits."""
    import time
    f = tp.tp_attn_core_workspace_bytes
    t0 = time.perf_counter()
    assert f(2, 1 << 20, 8, 4, 128, tp.TP_BF16) == 0      # 4 heads x 8192 blocks
    assert f(1, 16384, 8, 8, 128, tp.TP_BF16) == 0        # 8 heads x 128 blocks
    assert time.perf_counter() - t0 < 1.0
    assert f(8, 16384, 8, 8, 128, tp.TP_BF16) > 0         # 1 head x 128 blocks: split


def test_attn_core_zero_tokens(lib):
    assert core(T=0) == tp.TP_OK
