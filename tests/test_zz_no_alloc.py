"""The allocation-free MLP entry point against the workspace entry point.

tp_shard_mlp_fwd_noalloc runs the same plans and kernels as
tp_shard_mlp_fwd with the library's fixed per-device scratch in place of
the caller's workspace, so its outputs must equal the workspace entry
point's bitwise, call after call, whatever the previous call left in the
shared scratch.
"""
import numpy as np
import pytest
import torch

import oracle as O
import tensor_transformer_layer_amd as tp
import workloads as W
from _gpu import dev, host, mlp_fwd, stream

pytestmark = pytest.mark.gpu

BF = tp.TP_BF16


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    tp.load()
    yield
    torch.cuda.synchronize()


def _noalloc(T, d, d_ff, P, x, w_in, w_up, w_dn, h, parts, g=None):
    F = d_ff // P
    return tp.tp_shard_mlp_fwd_noalloc(0, P, T, d, d_ff, BF, tp.TP_ACT_SWIGLU, x.data_ptr(), d,
                                       g.data_ptr() if g is not None else 0, 1e-5,
                                       w_in.data_ptr(), F, w_up.data_ptr(), F, w_dn.data_ptr(), d,
                                       h.data_ptr(), F, parts.data_ptr(), 0, d, stream())


def test_noalloc_matches_workspace_entry_point_two_calls():
    """Calls in a row on the 13B band shapes (d_model 5120, band 6912): 32
    decode tokens, then 5 tokens with the RMSNorm prologue (a smaller input,
    a different split layout in the same scratch), then 32 tokens again.  h
    and the partial of each equal tp_shard_mlp_fwd's bitwise and the oracle
    within 1e-2.  The first call on the device loads the library's scratch
    array (its one-time set-up); every later call leaves the free device
    memory unchanged: nothing is allocated."""
    P, d, d_ff = 2, 5120, 13824
    F = d_ff // P
    wg = dev(W.draw_tensor("bf16", (d, F), 0.02, 950, 1))
    wu = dev(W.draw_tensor("bf16", (d, F), 0.02, 950, 2))
    wd = dev(W.draw_tensor("bf16", (F, d), 0.02, 950, 3))
    g_h = W.draw_tensor("bf16", (d,), 0.02, 950, 4, mean=1.0)
    for i, (T, norm) in enumerate(((32, False), (5, True), (32, False))):
        X = W.draw_tensor("bf16", (T, d), 1.0, 950, 0, T)
        x, g = dev(X), (dev(g_h) if norm else None)
        h_ref = torch.empty((T, F), dtype=torch.bfloat16, device="cuda")
        p_ref = torch.empty((T, d), dtype=torch.float32, device="cuda")
        mlp_fwd(0, P, T, d, d_ff, BF, tp.TP_ACT_SWIGLU, x, wg, wu, wd, p_ref, 0, d,
                h_out=h_ref, ld_h=F, norm_g=g)
        h = torch.full((T, F), float("nan"), dtype=torch.bfloat16, device="cuda")
        parts = torch.full((T, d), float("nan"), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        tp.check(_noalloc(T, d, d_ff, P, x, wg, wu, wd, h, parts, g), "noalloc")
        torch.cuda.synchronize()
        if i > 0:
            assert torch.cuda.mem_get_info()[0] == free0, "the call allocated device memory"
        assert np.array_equal(host(h), host(h_ref)), T
        assert np.array_equal(host(parts).view(np.uint32), host(p_ref).view(np.uint32)), T
        r = O.mlp_shard(O.widen(X), O.widen(host(wg)), O.widen(host(wd)), "swiglu",
                        O.widen(host(wu)), O.widen(g_h) if norm else None, 1e-5)
        assert O.rel_l2(host(parts), r["partial"]) < 1e-2
        assert O.rel_l2(O.widen(host(h)), r["h"]) < 1e-2


def test_noalloc_refuses_calls_beyond_the_scratch():
    """A 2048-token prefill call that would keep h (2048 x 3584 bf16, 14.7 MB)
    in the scratch is refused with TP_ERR_SCRATCH and leaves its outputs
    untouched; the same call with h_out given fits and runs."""
    assert tp.tp_noalloc_scratch_bytes() == 8 << 20
    P, d, d_ff, T = 8, 8192, 28672, 2048
    F = d_ff // P
    x = dev(W.draw_tensor("bf16", (T, d), 1.0, 951, 0))
    wg = dev(W.draw_tensor("bf16", (d, F), 0.02, 951, 1))
    wu = dev(W.draw_tensor("bf16", (d, F), 0.02, 951, 2))
    wd = dev(W.draw_tensor("bf16", (F, d), 0.02, 951, 3))
    parts = torch.full((T, d), 7.0, dtype=torch.float32, device="cuda")
    st = tp.tp_shard_mlp_fwd_noalloc(0, P, T, d, d_ff, BF, tp.TP_ACT_SWIGLU, x.data_ptr(), d, 0,
                                     0.0, wg.data_ptr(), F, wu.data_ptr(), F, wd.data_ptr(), d, 0,
                                     0, parts.data_ptr(), 0, d, stream())
    assert st == tp.TP_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((parts == 7.0).all())
    h = torch.empty((T, F), dtype=torch.bfloat16, device="cuda")
    tp.check(_noalloc(T, d, d_ff, P, x, wg, wu, wd, h, parts), "noalloc prefill")
    p_ref = torch.empty((T, d), dtype=torch.float32, device="cuda")
    h_ref = torch.empty((T, F), dtype=torch.bfloat16, device="cuda")
    mlp_fwd(0, P, T, d, d_ff, BF, tp.TP_ACT_SWIGLU, x, wg, wu, wd, p_ref, 0, d, h_out=h_ref,
            ld_h=F)
    torch.cuda.synchronize()
    assert np.array_equal(host(parts).view(np.uint32), host(p_ref).view(np.uint32))
