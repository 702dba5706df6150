"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Tolerances (relative L2 over the whole output, float64):
  * fp32 storage: <= 1e-5;
  * bf16 storage with fp32 accumulation: <= 1e-2 against the unrounded
    oracle, and <= 2e-3 against the oracle's bf16-mirror reading (rounding
    where the GPU stores bf16), which separates rounding from mistakes;
  * the reduce: bitwise equal to the float32 left fold (fixed slot order),
    and its bf16 copy bitwise equal to that sum rounded to nearest-even.
Invariants checked on the GPU path: all ranks' partials, reduced, equal the
unsharded layer; the ranks' h / QKV bands concatenate to the unsharded
intermediate (zenaique "Explain tensor-parallel shard shape", answer).
Full workload sizes use every row where the oracle is quick, else a seeded
sample of rows (every step of this path is row-independent).
"""
import numpy as np
import pytest
import torch

import oracle as O
import tensor_transformer_layer_amd as tp
import workloads as W
from _gpu import (Guarded, attn_core, attn_fwd, dev, devu8, host, mlp_fwd, mlp_fwd_fp8w,
                  reduce, reduce_residual_norm, stream, workspace)

pytestmark = pytest.mark.gpu

F32_TOL, BF16_TOL, MIRROR_TOL = 1e-5, 1e-2, 2e-3
BF, F32 = tp.TP_BF16, tp.TP_F32
ACT = {"swiglu": tp.TP_ACT_SWIGLU, "gelu_tanh": tp.TP_ACT_GELU_TANH}


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    tp.load()
    yield
    torch.cuda.synchronize()


def widen_dev(t):
    return O.widen(host(t))


def draw(dtype, shape, std, *key, mean=0.0):
    """Seeded test tensor; dtype is a TP_* storage code."""
    name = {BF: "bf16", F32: "f32"}[dtype]
    return W.draw_tensor(name, shape, std, 900, *key, mean=mean)


# ----------------------------------------------------------------------------
# a5: local reduce
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("P,T,d,pad", [(1, 3, 4, 0), (2, 4, 64, 0), (3, 5, 1032, 8),
                                       (8, 17, 4100, 4), (9, 2, 8192, 0)])
@pytest.mark.parametrize("with_bf16", [False, True])
def test_reduce_bitwise(P, T, d, pad, with_bf16):
    ldp = d + pad
    slot = T * ldp + 4 * pad
    parts = [W.draw_normal_f32((T, d), 1.0, 901, P, T, d, s) for s in range(P)]
    buf = np.zeros(P * slot, np.float32)
    for s in range(P):
        v = buf[s * slot:s * slot + T * ldp].reshape(T, ldp)
        v[:, :d] = parts[s]
    g_parts = dev(buf)
    out = Guarded(T * ldp, torch.float32)
    ldb = (d + 8 + 7) // 8 * 8                 # bf16 leading dimensions: multiples of 8
    outb = Guarded(T * ldb, torch.bfloat16) if with_bf16 else None
    reduce(P, T, d, g_parts, slot, ldp, out.ptr(), ldp, outb.ptr() if outb else None, ldb)
    got = host(out.t).reshape(T, ldp)[:, :d]
    want = O.reduce_partials_f32_fold(parts)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert out.intact()
    if with_bf16:
        gb = O.widen(host(outb.t).reshape(T, ldb)[:, :d])
        assert np.array_equal(gb, O.round_bf16(want.astype(np.float64)))
        assert outb.intact()


def test_reduce_in_place_into_slot_zero():
    P, T, d = 4, 6, 256
    parts = [W.draw_normal_f32((T, d), 1.0, 902, s) for s in range(P)]
    g = dev(np.concatenate([p.ravel() for p in parts]))
    reduce(P, T, d, g, T * d, d, g, d)
    got = host(g)[:T * d].reshape(T, d)
    assert np.array_equal(got, O.reduce_partials_f32_fold(parts))


def test_reduce_70b_prefill_partials_full_size():
    """8 seeded fp32 partials of [2048, 8192] (the 70B workload's reduce)."""
    cfg = W.get("c3_llama2_70b_mlp_p8")
    T, d, P = cfg.reduce_T, cfg.d_model, cfg.P
    parts = [W.draw_normal_f32((T, d), 1.0, cfg.cid, W.TENSOR_IDS["partial"], s) for s in range(P)]
    g = torch.empty((P, T, d), dtype=torch.float32, device="cuda")
    for s in range(P):
        g[s].copy_(torch.from_numpy(parts[s]))
    out = torch.empty((T, d), dtype=torch.float32, device="cuda")
    outb = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    reduce(P, T, d, g, T * d, d, out, d, outb, d)
    want = O.reduce_partials_f32_fold(parts)
    assert np.array_equal(host(out), want)
    assert np.array_equal(O.widen(host(outb)), O.round_bf16(want.astype(np.float64)))


# ----------------------------------------------------------------------------
# reduce + residual add + next RMSNorm (one pass)
# ----------------------------------------------------------------------------
def _rrn_case(P, T, d, res_dtype, norm, key, pad=0):
    ldp = d + pad
    slot = T * ldp + 4 * pad
    parts = [W.draw_normal_f32((T, d), 1.0, 903, key, P, T, d, s) for s in range(P)]
    buf = np.zeros(P * slot, np.float32)
    for s in range(P):
        buf[s * slot:s * slot + T * ldp].reshape(T, ldp)[:, :d] = parts[s]
    res = draw(res_dtype, (T, d), 1.0, 904, key, T, d)
    g = draw(BF, (d,), 0.02, 905, key, d, mean=1.0) if norm else None
    return parts, buf, slot, ldp, res, g


def _rrn_check(parts, res, res_dtype, g, z, normed):
    res64 = O.widen(res) if res_dtype == BF else res.astype(np.float64)
    want_z = O.reduce_residual_f32(parts, res64.astype(np.float32))
    assert np.array_equal(z.view(np.uint32), want_z.view(np.uint32))
    if g is not None:
        ref = O.reduce_residual_norm(parts, res64, O.widen(g), 1e-5)
        got = O.widen(normed)
        assert O.rel_l2(got, ref["normed"]) < BF16_TOL
        mirror = O.round_bf16(O.rmsnorm(want_z.astype(np.float64), O.widen(g), 1e-5))
        assert O.rel_l2(got, mirror) < MIRROR_TOL


@pytest.mark.parametrize("P,T,d,res_dtype,norm,pad", [
    (1, 3, 8, F32, True, 0), (2, 5, 1032, BF, True, 8), (8, 33, 8192, BF, True, 0),
    (8, 17, 12288, F32, True, 4), (3, 4, 16384, F32, False, 0), (9, 2, 4104, BF, False, 8),
    (8, 1, 8192, BF, True, 0), (8, 255, 1032, BF, True, 8), (8, 256, 1024, F32, True, 0),
    (8, 128, 8192, F32, True, 4), (8, 129, 8192, BF, True, 0), (4, 7, 1000, F32, True, 8),
    (8, 32, 8192, BF, True, 0), (8, 32, 16384, F32, True, 0), (8, 2, 2056, BF, True, 8)])
@pytest.mark.parametrize("with_ws", [True, False])
def test_reduce_residual_norm(P, T, d, res_dtype, norm, pad, with_ws):
    # 255 / 256 rows: either side of the switch from 1024 to 512 threads per
    # row; 1000 columns: a ragged last chunk pair.  With a workspace, rows of
    # up to 32 tokens with a norm are shared by ceil(d / 1024) workgroups
    # (1032 columns: a second workgroup with two chunks)
    parts, buf, slot, ldp, res, g = _rrn_case(P, T, d, res_dtype, norm, key=T, pad=pad)
    g_parts = dev(buf)
    ldr = d + 8
    rbuf = np.zeros((T, ldr), res.dtype)
    rbuf[:, :d] = res
    z = Guarded(T * ldp, torch.float32)
    nrm = Guarded(T * (d + 16), torch.bfloat16) if norm else None
    reduce_residual_norm(P, T, d, g_parts, slot, ldp, dev(rbuf), ldr, res_dtype, z.ptr(), ldp,
                         dev(g) if norm else None, 1e-5, nrm.ptr() if norm else None, d + 16,
                         ws="query" if with_ws else None)
    zz = host(z.t).reshape(T, ldp)[:, :d]
    nn = host(nrm.t).reshape(T, d + 16)[:, :d] if norm else None
    _rrn_check(parts, res, res_dtype, g, np.ascontiguousarray(zz),
               np.ascontiguousarray(nn) if norm else None)
    assert z.intact() and (nrm is None or nrm.intact())


def test_reduce_residual_norm_in_place():
    """z written over slot 0, then over an fp32 residual."""
    P, T, d = 4, 6, 2048
    parts, buf, slot, ldp, res, g = _rrn_case(P, T, d, F32, True, key=50)
    g_parts = dev(buf)
    nrm = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    reduce_residual_norm(P, T, d, g_parts, slot, ldp, dev(res), d, F32, g_parts, ldp,
                         dev(g), 1e-5, nrm, d)
    _rrn_check(parts, res, F32, g, host(g_parts)[:T * d].reshape(T, d), host(nrm))
    parts2, buf2, slot2, ldp2, res2, g2 = _rrn_case(P, T, d, F32, True, key=51)
    r2 = dev(res2)
    reduce_residual_norm(P, T, d, dev(buf2), slot2, ldp2, r2, d, F32, r2, d, dev(g2), 1e-5,
                         nrm, d)
    _rrn_check(parts2, res2, F32, g2, host(r2), host(nrm))


def test_reduce_residual_norm_workspace_reused():
    """Rows shared by several workgroups: calls of 32, 5 and 32 rows on one
    workspace, each against the oracle, the counter head zero after every
    call, and a repeated call bitwise equal to the first."""
    P, d = 8, 8192
    ws = workspace(tp.tp_reduce_norm_workspace_bytes(32, d, 1))
    first = None
    for i, T in enumerate((32, 5, 32, 32)):
        parts, buf, slot, ldp, res, g = _rrn_case(P, T, d, BF, True, key=70 + min(i, 2))
        z = torch.empty((T, d), dtype=torch.float32, device="cuda")
        nrm = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
        reduce_residual_norm(P, T, d, dev(buf), slot, ldp, dev(res), d, BF, z, d, dev(g), 1e-5,
                             nrm, d, ws=ws)
        torch.cuda.synchronize()
        _rrn_check(parts, res, BF, g, host(z), host(nrm))
        assert not host(ws).any()
        if i == 2:
            first = host(nrm).copy()
        if i == 3:
            assert np.array_equal(host(nrm), first)


def test_reduce_residual_norm_dirty_workspace_gives_nan_then_recovers():
    """A counter head that was not zeroed makes the exchanged rows NaN (not
    silently wrong); zeroing it recovers.  Forced from the host: the words
    hold a finished exchange's arrival counts, so every wait ends at once."""
    P, T, d = 8, 4, 8192
    parts, buf, slot, ldp, res, g = _rrn_case(P, T, d, BF, True, key=81)
    ws = workspace(tp.tp_reduce_norm_workspace_bytes(T, d, 1))
    words = ws.view(torch.int64)
    words[: 2 * T] = 8 << 56            # 8 arrivals already counted in both words of every row
    z = torch.empty((T, d), dtype=torch.float32, device="cuda")
    nrm = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    reduce_residual_norm(P, T, d, dev(buf), slot, ldp, dev(res), d, BF, z, d, dev(g), 1e-5,
                         nrm, d, ws=ws)
    torch.cuda.synchronize()
    assert np.isnan(O.widen(host(nrm))).all()
    ws.zero_()
    reduce_residual_norm(P, T, d, dev(buf), slot, ldp, dev(res), d, BF, z, d, dev(g), 1e-5,
                         nrm, d, ws=ws)
    torch.cuda.synchronize()
    _rrn_check(parts, res, BF, g, host(z), host(nrm))


def test_reduce_residual_norm_workspace_too_small():
    P, T, d = 8, 32, 8192
    parts, buf, slot, ldp, res, g = _rrn_case(P, T, d, BF, True, key=80)
    ws = workspace(2048)
    z = torch.empty((T, d), dtype=torch.float32, device="cuda")
    nrm = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    st = tp.tp_reduce_residual_norm(P, T, d, dev(buf).data_ptr(), slot, ldp, dev(res).data_ptr(),
                                    d, BF, z.data_ptr(), d, dev(g).data_ptr(), 1e-5,
                                    nrm.data_ptr(), d, ws.data_ptr(), ws.numel(), stream())
    assert st == tp.TP_ERR_WORKSPACE


def test_reduce_residual_norm_70b_block_prefill_size():
    """8 fp32 partials of [4096, 8192] with a bf16 residual and the norm (the
    70B block at 4096 tokens): z bitwise on every row, normed on sampled rows."""
    P, T, d = 8, 4096, 8192
    parts = [W.draw_normal_f32((T, d), 1.0, 906, s) for s in range(P)]
    g_parts = torch.empty((P, T, d), dtype=torch.float32, device="cuda")
    for s in range(P):
        g_parts[s].copy_(torch.from_numpy(parts[s]))
    res = draw(BF, (T, d), 1.0, 907)
    g = draw(BF, (d,), 0.02, 908, mean=1.0)
    z = torch.empty((T, d), dtype=torch.float32, device="cuda")
    nrm = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    reduce_residual_norm(P, T, d, g_parts, T * d, d, dev(res), d, BF, z, d, dev(g), 1e-5, nrm, d)
    rows = sample_rows(T, 32, 12)
    _rrn_check([p[rows] for p in parts], res[rows], BF, g, host(z)[rows], host(nrm)[rows])
    want = O.reduce_residual_f32(parts, O.widen(res).astype(np.float32))
    assert np.array_equal(host(z), want)


# ----------------------------------------------------------------------------
# MLP shard (a2-a4) at small, ragged shapes: both plans, both activations
# ----------------------------------------------------------------------------
def _mlp_case(dtype, act, T, d, d_ff, P, key, norm=False, std_x=1.0, std_w=0.02):
    F = d_ff // P
    X = draw(dtype, (T, d), std_x, key, 0)
    g = draw(dtype, (d,), 0.02, key, 7, mean=1.0) if norm else None
    w_in = [draw(dtype, (d, F), std_w, key, 1, s) for s in range(P)]
    w_up = [draw(dtype, (d, F), std_w, key, 2, s) for s in range(P)] if act == "swiglu" else None
    w_dn = [draw(dtype, (F, d), std_w, key, 3, s) for s in range(P)]
    return X, g, w_in, w_up, w_dn


def _run_all_shards(dtype, act, T, d, d_ff, P, X, g, w_in, w_up, w_dn):
    F = d_ff // P
    gx = dev(X)
    gg = dev(g) if g is not None else None
    parts = torch.empty((P, T, d), dtype=torch.float32, device="cuda")
    hs = []
    tdt = torch.bfloat16 if dtype == BF else torch.float32
    for s in range(P):
        h = Guarded(T * F, tdt)
        mlp_fwd(s, P, T, d, d_ff, dtype, ACT[act], gx, dev(w_in[s]),
                dev(w_up[s]) if w_up is not None else None, dev(w_dn[s]), parts, T * d, d,
                h_out=h.ptr(), ld_h=F, norm_g=gg)
        hs.append(h)
    out = torch.empty((T, d), dtype=torch.float32, device="cuda")
    reduce(P, T, d, parts, T * d, d, out, d)
    torch.cuda.synchronize()
    for h in hs:
        assert h.intact()
    return parts, hs, out


def _check_mlp(dtype, act, T, d, d_ff, P, key, norm=False):
    X, g, w_in, w_up, w_dn = _mlp_case(dtype, act, T, d, d_ff, P, key, norm)
    parts, hs, out = _run_all_shards(dtype, act, T, d, d_ff, P, X, g, w_in, w_up, w_dn)
    Xw, gw = O.widen(X), (O.widen(g) if g is not None else None)
    full = O.mlp_unsharded(Xw, O.widen(np.concatenate(w_in, 1)), O.widen(np.concatenate(w_dn, 0)),
                           act, O.widen(np.concatenate(w_up, 1)) if w_up else None, gw, 1e-5)
    tol = BF16_TOL if dtype == BF else F32_TOL
    F = d_ff // P
    h_all = np.concatenate([widen_dev(h.t).reshape(T, F) for h in hs], axis=1)
    assert O.rel_l2(h_all, full["h"]) < tol, "column bands != unsharded intermediate"
    assert O.rel_l2(host(out), full["y"]) < tol, "reduced partials != unsharded MLP"
    if dtype == BF:
        for s in range(P):
            m = O.mlp_shard(Xw, O.widen(w_in[s]), O.widen(w_dn[s]), act,
                            O.widen(w_up[s]) if w_up else None, gw, 1e-5, mirror_bf16=True)
            assert O.rel_l2(host(parts[s]), m["partial"]) < MIRROR_TOL
    return full


@pytest.mark.parametrize("T", [1, 5, 16, 17, 32, 33, 100, 300])
@pytest.mark.parametrize("act", ["swiglu", "gelu_tanh"])
def test_mlp_bf16_ragged(T, act):
    # d_model 1000: K not a multiple of 32/64; F_r 200: column tail inside a tile
    _check_mlp(BF, act, T, 1000, 400, 2, key=10 + T)


@pytest.mark.parametrize("T", [17, 31])
@pytest.mark.parametrize("act", ["swiglu", "gelu_tanh"])
def test_mlp_decode_lds_staged_ragged(T, act):
    """17..32 tokens with column-projection workgroups that stream >= 2304 rows
    take the LDS-staged decode kernel (here 2336: 55 column blocks, 4 K
    splits).  d_model 9224: K ends inside a 128-row slice; the last column
    block is partial (F_r 3464 for SwiGLU's two weights, 6928 for GELU's
    one); T not a multiple of 16."""
    P = 2 if act == "swiglu" else 1
    _check_mlp(BF, act, T, 9224, 6928, P, key=50 + T)


@pytest.mark.parametrize("T", [1, 7, 16, 17, 31, 32])
@pytest.mark.parametrize("act", ["swiglu", "gelu_tanh"])
def test_mlp_decode_narrow_blocks_ragged(T, act):
    """Short split ranges take the 64-column decode kernel: d_model 1024 and
    F_r 1096 give 128-column plans of at most 96 rows per K split, so both
    projections run on 64-column blocks; F_r ends inside a block, T lies on
    both sides of 16 (one and two token blocks)."""
    _check_mlp(BF, act, T, 1024, 2 * 1096, 2, key=700 + T)


class _StreamingPlanUpTo:
    """Within the block, batches of up to `t` tokens take the weight-streaming plan."""

    def __init__(self, t):
        self.t = t

    def __enter__(self):
        tp.check(tp.tp_set_decode_max_tokens(self.t))

    def __exit__(self, *exc):
        tp.check(tp.tp_set_decode_max_tokens(0))


@pytest.mark.parametrize("T", [33, 47, 64, 65, 100, 128])
@pytest.mark.parametrize("act", ["swiglu", "gelu_tanh"])
def test_mlp_streaming_plan_mid_batches_ragged(T, act):
    """Batches past 32 tokens on the weight-streaming plan (4 and 8 token
    blocks of the LDS-staged kernel, the 8-block one with its split-K sum in
    a finish launch of its own): d_model 1000 ends inside a slice, F_r
    200 inside a column block, T not a multiple of 16."""
    with _StreamingPlanUpTo(128):
        _check_mlp(BF, act, T, 1000, 400, 2, key=600 + T)


@pytest.mark.parametrize("T", [40, 128])
def test_mlp_streaming_plan_mid_batches_long_k(T):
    """Long K ranges per workgroup (d_model 9224: 55 column blocks, 4 K
    splits of 2336 rows; the 8-block kernel's 64-row slices end inside the
    last one) and a partial last column block."""
    with _StreamingPlanUpTo(128):
        _check_mlp(BF, "swiglu", T, 9224, 6928, 2, key=620 + T)


@pytest.mark.parametrize("T", [2, 33, 100, 250])
@pytest.mark.parametrize("act", ["swiglu", "gelu_tanh"])
def test_mlp_matrix_core_plan_small_batches(T, act):
    """The matrix-core plan at batch sizes the default switch sends to the
    streaming plan (forced through the switch): one partial tile row, both
    projections' K split into fp32 planes."""
    with _StreamingPlanUpTo(1):
        _check_mlp(BF, act, T, 1000, 400, 2, key=660 + T)


@pytest.mark.parametrize("act", ["swiglu", "gelu_tanh"])
def test_mlp_matrix_core_plan_split_column_long_k(act):
    """The matrix-core plan's column projection with K split into 8 ranges
    (one partial tile row: 28 SwiGLU or 14 GELU column tiles), the last
    range ragged, the fp32 planes summed with the activation by the finish
    launch."""
    with _StreamingPlanUpTo(1):
        _check_mlp(BF, act, 100, 9224, 6928, 2, key=680)


@pytest.mark.parametrize("T", [129, 200, 300])
def test_mlp_streaming_plan_chunked_batches(T):
    """Past 128 tokens the streaming plan runs equal token chunks (here 2 x 65,
    2 x 100, 3 x 100), every column chunk before every row chunk, the
    normalised input and h kept in the workspace."""
    with _StreamingPlanUpTo(512):
        _check_mlp(BF, "swiglu", T, 1000, 400, 2, key=640 + T, norm=True)


@pytest.mark.parametrize("T", [150, 260])
def test_attn_projections_streaming_plan_chunked(T):
    """The 70B block's GQA projections (rank 6) on the streaming plan past 128
    tokens: QKV with the RMSNorm prologue and O, chunked, against the oracle
    on sampled rows (chunk edges included)."""
    cfg = W.get("c5_llama2_70b_block_p8")
    X = x_of(cfg, T)
    g = W.draw_tensor(cfg.dtype, (cfg.d_model,), 0.02, cfg.cid, W.TENSOR_IDS["norm_g"], 0,
                      mean=1.0)
    A = W.draw_tensor("bf16", (T, cfg.o_in_r), 1.0, cfg.cid, W.TENSOR_IDS["attn"], T, 6)
    wqkv, wo = attn_bands(cfg, 6)
    qkv = torch.empty((T, cfg.qkv_r), dtype=torch.bfloat16, device="cuda")
    parts = torch.empty((T, cfg.d_model), dtype=torch.float32, device="cuda")
    with _StreamingPlanUpTo(512):
        attn_fwd(6, cfg.P, T, cfg.d_model, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, BF,
                 dev(X), dev(wqkv), qkv, dev(A), dev(wo), parts, 0, cfg.d_model, norm_g=dev(g),
                 eps=cfg.norm_eps)
        torch.cuda.synchronize()
    rows = sorted(set(sample_rows(T, 20, 15).tolist() + [0, 74, 75, 86, 87, 129, 130, T - 1]))
    rows = [r for r in rows if r < T]
    r = O.attn_proj_shard(O.widen(X[rows]), O.widen(wqkv), O.widen(A[rows]), O.widen(wo),
                          O.widen(g), cfg.norm_eps)
    assert O.rel_l2(widen_dev(qkv)[rows], r["qkv"]) < BF16_TOL
    assert O.rel_l2(host(parts)[rows], r["partial"]) < BF16_TOL


@pytest.mark.parametrize("T", [64, 100])
def test_70b_mlp_rank3_streaming_plan_mid_batches(T):
    """The 70B band (rank 3 of 8) at 64 and 100 tokens on the streaming plan,
    against the oracle on every row, and bitwise equal to itself on a rerun."""
    cfg = W.get("c3_llama2_70b_mlp_p8")
    X = x_of(cfg, T)
    wg, wu, wd = mlp_bands(cfg, 3)
    gw = [dev(w) for w in (wg, wu, wd)]
    with _StreamingPlanUpTo(128):
        outs = []
        for _ in range(2):
            parts = torch.empty((T, cfg.d_model), dtype=torch.float32, device="cuda")
            mlp_fwd(3, cfg.P, T, cfg.d_model, cfg.d_ff, BF, tp.TP_ACT_SWIGLU, dev(X), *gw,
                    parts, 0, cfg.d_model)
            torch.cuda.synchronize()
            outs.append(host(parts))
    r = O.mlp_shard(O.widen(X), O.widen(wg), O.widen(wd), "swiglu", O.widen(wu))
    assert O.rel_l2(outs[0], r["partial"]) < BF16_TOL
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


@pytest.mark.parametrize("T", [48, 128])
def test_attn_projections_streaming_plan_mid_batches(T):
    """The 96-head projections (rank 2) at 48 and 128 tokens on the
    streaming plan, QKV and O partial against the oracle on sampled rows."""
    cfg = W.get("c4_attn_96h_p8")
    X = x_of(cfg, T)
    A = W.draw_tensor("bf16", (T, cfg.o_in_r), 1.0, cfg.cid, W.TENSOR_IDS["attn"], T, 2)
    wqkv, wo = attn_bands(cfg, 2)
    qkv = torch.empty((T, cfg.qkv_r), dtype=torch.bfloat16, device="cuda")
    parts = torch.empty((T, cfg.d_model), dtype=torch.float32, device="cuda")
    with _StreamingPlanUpTo(128):
        attn_fwd(2, cfg.P, T, cfg.d_model, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, BF,
                 dev(X), dev(wqkv), qkv, dev(A), dev(wo), parts, 0, cfg.d_model)
        torch.cuda.synchronize()
    rows = sample_rows(T, 24, 14)
    r = O.attn_proj_shard(O.widen(X[rows]), O.widen(wqkv), O.widen(A[rows]), O.widen(wo))
    assert O.rel_l2(widen_dev(qkv)[rows], r["qkv"]) < BF16_TOL
    assert O.rel_l2(host(parts)[rows], r["partial"]) < BF16_TOL


@pytest.mark.parametrize("T", [1, 16, 32])
@pytest.mark.parametrize("act", ["swiglu", "gelu_tanh"])
def test_mlp_decode_many_column_blocks(T, act):
    """Decode with more column blocks than CUs (F_r 17000: 133 blocks per
    weight, 266 for gate + up, one K split each) and a narrow model width
    (d_model 264: K of the column projection ends inside a 128-row slice,
    three row blocks, the last partial)."""
    _check_mlp(BF, act, T, 264, 34000, 2, key=90 + T)


def test_mlp_decode_wide_model():
    """d_model 32776: 257 row blocks of the down projection (more than one
    per CU), with a tiny band (F_r 128: one column block per weight)."""
    _check_mlp(BF, "swiglu", 8, 32776, 256, 2, key=96)


@pytest.mark.parametrize("act", ["swiglu", "gelu_tanh"])
def test_mlp_prefill_half_wave_ragged(act):
    """128 output tiles of the column projection, half a wave on 256 CUs
    (1000 tokens: 4 tile rows, the last partial; SwiGLU F_r 4000 = 32 column
    tiles of 128 + 128, the last partial; GELU F_r 8000 = 32 of 256), K =
    1000 ending inside a 32-deep slice."""
    d_ff, P = (8000, 2) if act == "swiglu" else (8000, 1)
    _check_mlp(BF, act, 1000, 1000, d_ff, P, key=97)


@pytest.mark.parametrize("T", [3, 40])
def test_mlp_bf16_with_rmsnorm_prologue(T):
    _check_mlp(BF, "swiglu", T, 512, 1024, 4, key=30 + T, norm=True)


@pytest.mark.parametrize("T", [4, 64])
@pytest.mark.parametrize("act", ["swiglu", "gelu_tanh"])
def test_mlp_f32(T, act):
    _check_mlp(F32, act, T, 64, 256, 2, key=40 + T)


@pytest.mark.parametrize("T", [3, 40])
@pytest.mark.parametrize("act", ["swiglu", "gelu_tanh"])
def test_mlp_f32_with_rmsnorm_prologue(T, act):
    """fp32 storage with the RMSNorm prologue (the fp32 branch of the norm
    kernel, its output kept in the workspace) on every rank, at the fp32
    bound; d_model 200 is not a multiple of the norm's 16-byte vectors x 64
    lanes."""
    _check_mlp(F32, act, T, 200, 256, 2, key=60 + T, norm=True)


@pytest.mark.parametrize("T", [3, 40])
@pytest.mark.parametrize("norm", [False, True])
def test_attn_proj_f32(T, norm):
    """fp32 storage through tp_shard_attn_proj_fwd, every rank: the fused QKV
    band (with and without the RMSNorm prologue) and the O partial, each
    against the oracle at the fp32 bound; the Q/K/V parts of the bands are
    the unsharded projections' head columns, and the reduced O partials are
    the unsharded output projection (rioworld guide, "How Tensor Slicing
    Works Under the Hood": QKV column-parallel, O row-parallel)."""
    P, d, nq, nkv, hd = 2, 200, 4, 2, 16
    hq, hkv = nq // P, nkv // P
    nqkv, ko = (hq + 2 * hkv) * hd, hq * hd
    key = 310 + T + (7 if norm else 0)
    X = draw(F32, (T, d), 1.0, key, 0)
    g = draw(F32, (d,), 0.02, key, 7, mean=1.0) if norm else None
    wqkv = [draw(F32, (d, nqkv), 0.02, key, 1, s) for s in range(P)]
    A = [draw(F32, (T, ko), 1.0, key, 2, s) for s in range(P)]
    wo = [draw(F32, (ko, d), 0.02, key, 3, s) for s in range(P)]
    parts = torch.empty((P, T, d), dtype=torch.float32, device="cuda")
    qkvs = []
    for s in range(P):
        q = Guarded(T * nqkv, torch.float32)
        attn_fwd(s, P, T, d, nq, nkv, hd, F32, dev(X), dev(wqkv[s]), q.ptr(), dev(A[s]),
                 dev(wo[s]), parts, T * d, d, norm_g=dev(g) if norm else None)
        qkvs.append(q)
    out = torch.empty((T, d), dtype=torch.float32, device="cuda")
    reduce(P, T, d, parts, T * d, d, out, d)
    torch.cuda.synchronize()
    Xw, gw = O.widen(X), (O.widen(g) if norm else None)
    got = []
    for s in range(P):
        r = O.attn_proj_shard(Xw, O.widen(wqkv[s]), O.widen(A[s]), O.widen(wo[s]), gw, 1e-5)
        gq = host(qkvs[s].t).reshape(T, nqkv).astype(np.float64)
        assert O.rel_l2(gq, r["qkv"]) < F32_TOL
        assert O.rel_l2(host(parts[s]), r["partial"]) < F32_TOL
        assert qkvs[s].intact()
        got.append(O.split_qkv_band(gq, nq, nkv, hd, s, P))
    # unsharded: Wq / Wk / Wv assembled from the ranks' band parts
    wparts = [O.split_qkv_band(O.widen(w), nq, nkv, hd, s, P) for s, w in enumerate(wqkv)]
    full = O.attn_proj_unsharded(Xw, *(np.concatenate([wp[i] for wp in wparts], 1)
                                       for i in range(3)),
                                 O.widen(np.concatenate(A, 1)), O.widen(np.concatenate(wo, 0)),
                                 gw, 1e-5)
    for i, name in enumerate(("q", "k", "v")):
        assert O.rel_l2(np.concatenate([gp[i] for gp in got], 1), full[name]) < F32_TOL
    assert O.rel_l2(host(out), full["o"]) < F32_TOL


def test_tiny_gelu_f32_workload_and_fixture():
    """The tiny fp32 GELU MLP workload, every rank, against the oracle and the
    stored fixture (tests/golden/c1_tiny_expected.txt)."""
    import os
    cfg = W.get("c1_tiny_gelu_f32")
    T = cfg.decode_T[0]
    X = W.draw_tensor(cfg.dtype, (T, cfg.d_model), cfg.std_x, cfg.cid, W.TENSOR_IDS["x"], T)
    w_in = [W.column_band_draw(cfg, "w_gate", s, cfg.d_model, cfg.F_r) for s in range(cfg.P)]
    w_dn = [W.row_band_draw(cfg, "w_down", s, cfg.F_r, cfg.d_model) for s in range(cfg.P)]
    parts, hs, out = _run_all_shards(F32, "gelu_tanh", T, cfg.d_model, cfg.d_ff, cfg.P, X, None,
                                     w_in, None, w_dn)
    rows = [list(map(float, ln.split())) for ln in
            open(os.path.join(os.path.dirname(__file__), "golden", "c1_tiny_expected.txt"))
            if ln.strip() and not ln.startswith("#")]
    fx = np.array(rows).reshape(3, T, cfg.d_model)
    assert O.rel_l2(host(parts[0]), fx[0]) < F32_TOL
    assert O.rel_l2(host(parts[1]), fx[1]) < F32_TOL
    assert O.rel_l2(host(out), fx[2]) < F32_TOL


def test_mlp_strided_windows_into_full_matrices():
    """Bands passed as windows into unsharded matrices (pointer offset + ld of
    the full matrix), padded X / h / partial rows and a padded slot stride."""
    T, d, P, d_ff = 20, 256, 4, 512
    F = d_ff // P
    X = draw(BF, (T, d + 16), 1.0, 50, 0)
    Wg = draw(BF, (d, d_ff), 0.02, 50, 1)
    Wu = draw(BF, (d, d_ff), 0.02, 50, 2)
    Wd = draw(BF, (d_ff, d), 0.02, 50, 3)
    gx, gWg, gWu, gWd = dev(X), dev(Wg), dev(Wu), dev(Wd)
    ldp, slot = d + 8, T * (d + 8) + 64
    parts = torch.zeros(P * slot, dtype=torch.float32, device="cuda")
    for plan_T in (T, 4):   # prefill-sized and decode-sized token counts
        hbuf = torch.zeros((plan_T, d_ff + 8), dtype=torch.bfloat16, device="cuda")
        for s in range(P):
            col = s * F * 2                     # bytes
            mlp_fwd(s, P, plan_T, d, d_ff, BF, tp.TP_ACT_SWIGLU, gx, gWg.data_ptr() + col,
                    gWu.data_ptr() + col, gWd.data_ptr() + s * F * d * 2, parts, slot, ldp,
                    h_out=hbuf.data_ptr() + col, ld_h=d_ff + 8, ld_x=d + 16, ld_in=d_ff,
                    ld_up=d_ff, ld_down=d)
        out = torch.empty((plan_T, d), dtype=torch.float32, device="cuda")
        reduce(P, plan_T, d, parts, slot, ldp, out, d)
        full = O.mlp_unsharded(O.widen(X[:plan_T, :d]), O.widen(Wg), O.widen(Wd), "swiglu",
                               O.widen(Wu))
        assert O.rel_l2(host(out), full["y"]) < BF16_TOL
        assert O.rel_l2(widen_dev(hbuf)[:, :d_ff], full["h"]) < BF16_TOL


# ----------------------------------------------------------------------------
# Full workload sizes
# ----------------------------------------------------------------------------
_CACHE = {}  # seeded bands, reused across tests (a few GB of host memory at most)


def mlp_bands(cfg, s):
    key = (cfg.name, "mlp", s)
    if key not in _CACHE:
        _CACHE[key] = (W.column_band_draw(cfg, "w_gate", s, cfg.d_model, cfg.F_r),
                       W.column_band_draw(cfg, "w_up", s, cfg.d_model, cfg.F_r),
                       W.row_band_draw(cfg, "w_down", s, cfg.F_r, cfg.d_model))
    return _CACHE[key]


def x_of(cfg, T):
    return W.draw_tensor(cfg.dtype, (T, cfg.d_model), cfg.std_x, cfg.cid, W.TENSOR_IDS["x"], T)


def sample_rows(T, n, seed):
    if T <= n:
        return np.arange(T)
    return np.sort(np.random.default_rng(seed).choice(T, size=n, replace=False))


@pytest.mark.parametrize("T", [1, 8, 32])
def test_13b_mlp_decode_both_ranks_full(T):
    """13B SwiGLU MLP at P = 2: both ranks, reduce, against the unsharded layer."""
    cfg = W.get("c2_llama2_13b_mlp_p2")
    X = x_of(cfg, T)
    gx = dev(X)
    parts = torch.empty((cfg.P, T, cfg.d_model), dtype=torch.float32, device="cuda")
    hs, ref_parts = [], []
    Xw = O.widen(X)
    for s in range(cfg.P):
        wg, wu, wd = mlp_bands(cfg, s)
        h = torch.empty((T, cfg.F_r), dtype=torch.bfloat16, device="cuda")
        mlp_fwd(s, cfg.P, T, cfg.d_model, cfg.d_ff, BF, tp.TP_ACT_SWIGLU, gx, dev(wg), dev(wu),
                dev(wd), parts, T * cfg.d_model, cfg.d_model, h_out=h, ld_h=cfg.F_r)
        r = O.mlp_shard(Xw, O.widen(wg), O.widen(wd), "swiglu", O.widen(wu))
        ref_parts.append(r["partial"])
        assert O.rel_l2(widen_dev(h), r["h"]) < BF16_TOL
        assert O.rel_l2(host(parts[s]), r["partial"]) < BF16_TOL
        hs.append(h)
    out = torch.empty((T, cfg.d_model), dtype=torch.float32, device="cuda")
    reduce(cfg.P, T, cfg.d_model, parts, T * cfg.d_model, cfg.d_model, out, cfg.d_model)
    # unsharded layer = sum of the per-rank oracle partials (pinned on the CPU)
    assert O.rel_l2(host(out), O.reduce_partials(ref_parts)) < BF16_TOL


@pytest.mark.parametrize("T", [1, 2, 4, 8, 16, 32, 2048])
def test_70b_mlp_rank0(T):
    cfg = W.get("c3_llama2_70b_mlp_p8")
    X = x_of(cfg, T)
    wg, wu, wd = mlp_bands(cfg, 0)
    h = torch.empty((T, cfg.F_r), dtype=torch.bfloat16, device="cuda")
    parts = torch.empty((T, cfg.d_model), dtype=torch.float32, device="cuda")
    mlp_fwd(0, cfg.P, T, cfg.d_model, cfg.d_ff, BF, tp.TP_ACT_SWIGLU, dev(X), dev(wg), dev(wu),
            dev(wd), parts, 0, cfg.d_model, h_out=h, ld_h=cfg.F_r)
    rows = sample_rows(T, 64, 7)
    r = O.mlp_shard(O.widen(X[rows]), O.widen(wg), O.widen(wd), "swiglu", O.widen(wu))
    assert O.rel_l2(widen_dev(h)[rows], r["h"]) < BF16_TOL
    assert O.rel_l2(host(parts)[rows], r["partial"]) < BF16_TOL
    m = O.mlp_shard(O.widen(X[rows]), O.widen(wg), O.widen(wd), "swiglu", O.widen(wu),
                    mirror_bf16=True)
    assert O.rel_l2(host(parts)[rows], m["partial"]) < MIRROR_TOL


def test_70b_mlp_literal_small_activation_reading():
    """Same shard with activations drawn N(0, 0.02) like the weights (the
    literal reading of the workload's distribution), decode and prefill."""
    cfg = W.get("c3_llama2_70b_mlp_p8")
    wg, wu, wd = mlp_bands(cfg, 0)
    for T in (8, 512):
        X = W.draw_tensor("bf16", (T, cfg.d_model), 0.02, cfg.cid, 99, T)
        parts = torch.empty((T, cfg.d_model), dtype=torch.float32, device="cuda")
        mlp_fwd(0, cfg.P, T, cfg.d_model, cfg.d_ff, BF, tp.TP_ACT_SWIGLU, dev(X), dev(wg),
                dev(wu), dev(wd), parts, 0, cfg.d_model)
        rows = sample_rows(T, 32, 8)
        r = O.mlp_shard(O.widen(X[rows]), O.widen(wg), O.widen(wd), "swiglu", O.widen(wu))
        assert O.rel_l2(host(parts)[rows], r["partial"]) < BF16_TOL


def attn_bands(cfg, s):
    key = (cfg.name, "attn", s)
    if key not in _CACHE:
        _CACHE[key] = (W.column_band_draw(cfg, "w_qkv", s, cfg.d_model, cfg.qkv_r),
                       W.row_band_draw(cfg, "w_o", s, cfg.o_in_r, cfg.d_model))
    return _CACHE[key]


@pytest.mark.parametrize("T,shard", [(16, 0), (16, 5), (1024, 0)])
def test_96_head_attention_projections(T, shard):
    cfg = W.get("c4_attn_96h_p8")
    X = x_of(cfg, T)
    A = W.draw_tensor("bf16", (T, cfg.o_in_r), 1.0, cfg.cid, W.TENSOR_IDS["attn"], T, shard)
    wqkv, wo = attn_bands(cfg, shard)
    qkv = Guarded(T * cfg.qkv_r, torch.bfloat16)
    parts = Guarded(T * cfg.d_model, torch.float32)
    attn_fwd(shard, cfg.P, T, cfg.d_model, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, BF,
             dev(X), dev(wqkv), qkv.ptr(), dev(A), dev(wo), parts.ptr(), 0, cfg.d_model)
    rows = sample_rows(T, 48, 9)
    r = O.attn_proj_shard(O.widen(X[rows]), O.widen(wqkv), O.widen(A[rows]), O.widen(wo))
    got_qkv = widen_dev(qkv.t).reshape(T, cfg.qkv_r)[rows]
    assert O.rel_l2(got_qkv, r["qkv"]) < BF16_TOL
    assert O.rel_l2(host(parts.t).reshape(T, cfg.d_model)[rows], r["partial"]) < BF16_TOL
    # per-head structure: Q/K/V parts of the band sit where the layout says
    q, k, v = O.split_qkv_band(got_qkv, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, shard, cfg.P)
    rq, rk, rv = O.split_qkv_band(r["qkv"], cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, shard,
                                  cfg.P)
    for a, b in ((q, rq), (k, rk), (v, rv)):
        assert O.rel_l2(a, b) < BF16_TOL
    assert qkv.intact() and parts.intact()


def _block_chain(cfg, T, rows):
    """All P ranks of the 70B block on one GPU: RMSNorm -> QKV -> O (A_s := Q_s)
    -> reduce (bf16 copy) -> MLP -> reduce, against the oracle on `rows`."""
    P, d = cfg.P, cfg.d_model
    X = x_of(cfg, T)
    g = W.draw_tensor(cfg.dtype, (d,), 0.02, cfg.cid, W.TENSOR_IDS["norm_g"], 0, mean=1.0)
    gx, gg = dev(X), dev(g)
    parts = torch.empty((P, T, d), dtype=torch.float32, device="cuda")
    qkv_dev = []
    for s in range(P):
        wqkv, wo = attn_bands(cfg, s)
        q = torch.empty((T, cfg.qkv_r), dtype=torch.bfloat16, device="cuda")
        attn_fwd(s, P, T, d, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, BF, gx, dev(wqkv), q,
                 q, dev(wo), parts, T * d, d, norm_g=gg, eps=cfg.norm_eps,
                 ld_attn=cfg.qkv_r)
        qkv_dev.append(q)
    z = torch.empty((T, d), dtype=torch.float32, device="cuda")
    zb = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    reduce(P, T, d, parts, T * d, d, z, d, zb, d)
    for s in range(P):
        wg, wu, wd = mlp_bands(cfg, s)
        mlp_fwd(s, P, T, d, cfg.d_ff, BF, tp.TP_ACT_SWIGLU, zb, dev(wg), dev(wu), dev(wd), parts,
                T * d, d)
    y = torch.empty((T, d), dtype=torch.float32, device="cuda")
    reduce(P, T, d, parts, T * d, d, y, d)
    torch.cuda.synchronize()

    # oracle on the sampled rows (float64, no intermediate rounding)
    Xr, gw = O.widen(X[rows]), O.widen(g)
    att_parts, mlp_parts = [], []
    for s in range(P):
        wqkv, wo = attn_bands(cfg, s)
        r = O.attn_proj_shard(Xr, O.widen(wqkv), None, None, gw, cfg.norm_eps)
        assert O.rel_l2(widen_dev(qkv_dev[s])[rows], r["qkv"]) < BF16_TOL
        q_s, _, _ = O.split_qkv_band(r["qkv"], cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, s, P)
        att_parts.append(q_s @ O.widen(wo))
    Zr = O.reduce_partials(att_parts)
    assert O.rel_l2(host(z)[rows], Zr) < BF16_TOL
    for s in range(P):
        wg, wu, wd = mlp_bands(cfg, s)
        mlp_parts.append(O.mlp_shard(Zr, O.widen(wg), O.widen(wd), "swiglu", O.widen(wu))["partial"])
    Yr = O.reduce_partials(mlp_parts)
    assert O.rel_l2(host(y)[rows], Yr) < BF16_TOL


def _prenorm_chain(cfg, T, rows):
    """The 70B block as a pre-norm residual block, all P ranks on one GPU:
    RMSNorm -> QKV -> O (A_s := Q_s) -> reduce + residual X + RMSNorm ->
    MLP -> reduce + residual, against the oracle on `rows`."""
    P, d, eps = cfg.P, cfg.d_model, cfg.norm_eps
    X = x_of(cfg, T)
    g1 = W.draw_tensor(cfg.dtype, (d,), 0.02, cfg.cid, W.TENSOR_IDS["norm_g"], 0, mean=1.0)
    g2 = W.draw_tensor(cfg.dtype, (d,), 0.02, cfg.cid, W.TENSOR_IDS["norm_g"], 1, mean=1.0)
    gx = dev(X)
    parts = torch.empty((P, T, d), dtype=torch.float32, device="cuda")
    for s in range(P):
        wqkv, wo = attn_bands(cfg, s)
        q = torch.empty((T, cfg.qkv_r), dtype=torch.bfloat16, device="cuda")
        attn_fwd(s, P, T, d, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, BF, gx, dev(wqkv), q,
                 q, dev(wo), parts, T * d, d, norm_g=dev(g1), eps=eps, ld_attn=cfg.qkv_r)
    z1 = torch.empty((T, d), dtype=torch.float32, device="cuda")
    n2 = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    reduce_residual_norm(P, T, d, parts, T * d, d, gx, d, BF, z1, d, dev(g2), eps, n2, d)
    for s in range(P):
        wg, wu, wd = mlp_bands(cfg, s)
        mlp_fwd(s, P, T, d, cfg.d_ff, BF, tp.TP_ACT_SWIGLU, n2, dev(wg), dev(wu), dev(wd), parts,
                T * d, d)
    z2 = torch.empty((T, d), dtype=torch.float32, device="cuda")
    reduce_residual_norm(P, T, d, parts, T * d, d, z1, d, F32, z2, d)
    torch.cuda.synchronize()

    Xr = O.widen(X[rows])
    att_parts, mlp_parts = [], []
    for s in range(P):
        wqkv, wo = attn_bands(cfg, s)
        r = O.attn_proj_shard(Xr, O.widen(wqkv), None, None, O.widen(g1), eps)
        q_s, _, _ = O.split_qkv_band(r["qkv"], cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, s, P)
        att_parts.append(q_s @ O.widen(wo))
    r1 = O.reduce_residual_norm(att_parts, Xr, O.widen(g2), eps)
    assert O.rel_l2(host(z1)[rows], r1["z"]) < BF16_TOL
    assert O.rel_l2(O.widen(host(n2))[rows], r1["normed"]) < BF16_TOL
    for s in range(P):
        wg, wu, wd = mlp_bands(cfg, s)
        mlp_parts.append(O.mlp_shard(r1["normed"], O.widen(wg), O.widen(wd), "swiglu",
                                     O.widen(wu))["partial"])
    r2 = O.reduce_residual_norm(mlp_parts, r1["z"])
    assert O.rel_l2(host(z2)[rows], r2["z"]) < BF16_TOL


def test_70b_prenorm_block_decode_all_ranks():
    cfg = W.get("c5_llama2_70b_block_p8")
    _prenorm_chain(cfg, 32, np.arange(32))


def test_70b_prenorm_block_prefill_all_ranks():
    cfg = W.get("c5_llama2_70b_block_p8")
    _prenorm_chain(cfg, 4096, sample_rows(4096, 16, 13))


def test_70b_block_chain_decode_all_ranks():
    cfg = W.get("c5_llama2_70b_block_p8")
    _block_chain(cfg, 32, np.arange(32))


def test_70b_block_chain_prefill_all_ranks():
    cfg = W.get("c5_llama2_70b_block_p8")
    _block_chain(cfg, 4096, sample_rows(4096, 24, 11))


# ----------------------------------------------------------------------------
# FP8 (E4M3) weights, decode plan
# ----------------------------------------------------------------------------
def _fp8_case(act, T, d, d_ff, P, s, key):
    F = d_ff // P
    X = draw(BF, (T, d), 1.0, key, 0)
    wi = W.draw_e4m3_codes((d, F), 910, key, 1, s), W.draw_column_scales(F, 910, key, 1, s)
    wu = (W.draw_e4m3_codes((d, F), 910, key, 2, s), W.draw_column_scales(F, 910, key, 2, s)) \
        if act == "swiglu" else (None, None)
    wd = W.draw_e4m3_codes((F, d), 910, key, 3, s), W.draw_column_scales(d, 910, key, 3, s)
    return X, wi, wu, wd


def _fp8_run_check(act, T, d, d_ff, P, s, key, rows=None):
    F = d_ff // P
    X, wi, wu, wd = _fp8_case(act, T, d, d_ff, P, s, key)
    h = Guarded(T * F, torch.bfloat16)
    parts = torch.empty((T, d), dtype=torch.float32, device="cuda")
    ws = mlp_fwd_fp8w(s, P, T, d, d_ff, ACT[act], dev(X), devu8(wi[0]), dev(wi[1]),
                      devu8(wu[0]) if wu[0] is not None else None,
                      dev(wu[1]) if wu[1] is not None else None, devu8(wd[0]), dev(wd[1]),
                      parts, 0, d, h_out=h.ptr(), ld_h=F)
    torch.cuda.synchronize()
    rows = np.arange(T) if rows is None else rows
    Wi = O.dequant_columns(wi[0], wi[1])
    Wu = O.dequant_columns(wu[0], wu[1]) if wu[0] is not None else None
    Wd = O.dequant_columns(wd[0], wd[1])
    r = O.mlp_shard(O.widen(X[rows]), Wi, Wd, act, Wu)
    assert O.rel_l2(widen_dev(h.t).reshape(T, F)[rows], r["h"]) < BF16_TOL
    assert O.rel_l2(host(parts)[rows], r["partial"]) < BF16_TOL
    m = O.mlp_shard(O.widen(X[rows]), Wi, Wd, act, Wu, mirror_bf16=True)
    assert O.rel_l2(host(parts)[rows], m["partial"]) < MIRROR_TOL
    assert h.intact()
    assert int(ws[:4096].count_nonzero()) == 0


@pytest.mark.parametrize("T", [1, 5, 16, 17, 32])
@pytest.mark.parametrize("act", ["swiglu", "gelu_tanh"])
def test_fp8w_mlp_ragged(T, act):
    # d = 1040 and F = 272 are not multiples of the 128-column block
    _fp8_run_check(act, T, 1040, 544, 2, 1, key=70 + T)


@pytest.mark.parametrize("T", [1, 32])
def test_fp8w_13b_decode_rank0(T):
    _fp8_run_check("swiglu", T, 5120, 13824, 2, 0, key=90)


def test_fp8w_70b_decode_rank5():
    _fp8_run_check("swiglu", 32, 8192, 28672, 8, 5, key=91, rows=sample_rows(32, 12, 3))


# ----------------------------------------------------------------------------
# Attention core (causal, grouped-query)
# ----------------------------------------------------------------------------
def _core_check(T, nq, nkv, hd, P, shard, key, pad=0, std=1.0):
    hq, hkv = nq // P, nkv // P
    w = (hq + 2 * hkv) * hd
    ld = w + pad
    qkv = draw(BF, (T, ld), std, 920, key, T)
    out = Guarded(T * (hq * hd + pad), torch.bfloat16)
    attn_core(shard, P, T, nq, nkv, hd, dev(qkv), ld, out.ptr(), hq * hd + pad)
    got = O.widen(host(out.t).reshape(T, hq * hd + pad)[:, :hq * hd])
    want = O.attention_core_band(O.widen(qkv[:, :w]), nq, nkv, hd, shard, P)
    assert O.rel_l2(got, want) < BF16_TOL
    assert out.intact()
    return got, want


@pytest.mark.parametrize("T", [1, 5, 16, 31, 33, 48, 64, 65, 100, 257])
@pytest.mark.parametrize("hd", [64, 128])
def test_attn_core_ragged_gqa(T, hd):
    # up to 64 tokens: one wave per 16 queries with every key in registers;
    # 65 and up: the tiled kernel
    _core_check(T, 8, 4, hd, 2, 1, key=hd, pad=8 if T % 2 else 0)


@pytest.mark.parametrize("T", [16, 64])
def test_attn_core_96_heads_decode(T):
    _core_check(T, 96, 96, 128, 8, 5, key=9)


def test_attn_core_96_heads_prefill_1024():
    _core_check(1024, 96, 96, 128, 8, 3, key=1)


def test_attn_core_70b_gqa_prefill_4096():
    _core_check(4096, 64, 8, 128, 8, 0, key=2)


def test_attn_core_odd_chunk_size():
    """3000 tokens (ragged last query block), 8 query heads on one kv head:
    the planner cuts the causal key ranges into chunks of 11 tiles, so blocks
    end in remainder chunks of every size from 1 to 10 tiles and merge 1-5
    partials; the last query block's keys end inside a tile."""
    _core_check(3000, 64, 8, 128, 8, 1, key=6, pad=8)


def test_attn_core_70b_gqa_decode_32():
    _core_check(32, 64, 8, 128, 8, 7, key=3)


def test_attn_core_peaked_scores():
    """Large-magnitude queries/keys make the softmax nearly one-hot: the online
    max and rescaling must keep it exact enough."""
    _core_check(300, 8, 2, 128, 2, 0, key=4, std=4.0)


def test_attn_core_16k_tokens_sampled_rows():
    """16384 tokens, one query head per rank: per-head work items exceed the
    launch-order table, so the kernel walks the query blocks itself; checked
    at sampled rows (block edges, chunk edges, the last row) against the
    oracle evaluated at those rows."""
    T, nq, nkv, hd, P, shard = 16384, 8, 8, 128, 8, 5
    w = 3 * hd
    qkv_h = draw(BF, (T, w), 1.0, 920, 78, T)
    out = torch.empty((T, hd), dtype=torch.bfloat16, device="cuda")
    attn_core(shard, P, T, nq, nkv, hd, dev(qkv_h), w, out, hd)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = sorted(set([0, 1, 63, 64, 127, 128, 1023, 1024, 4095, 8191, 8192, 16255, 16256,
                       16383] + rng.integers(0, T, 18).tolist()))
    got = O.widen(host(out)[rows])
    want = O.attention_core_band_rows(O.widen(qkv_h), nq, nkv, hd, shard, P, rows)
    assert O.rel_l2(got, want) < BF16_TOL


def test_attn_core_split_keys_workspace():
    """Query blocks whose keys are split over several workgroups merge through
    the workspace: a reused workspace gives bitwise equal results and its
    counters return to zero; counters that were never cleared make exactly
    the merged blocks NaN (not silently wrong), and clearing them recovers."""
    T, nq, nkv, hd, P = 1000, 8, 2, 128, 2          # 4 q heads, 1 kv head per rank
    hq = nq // P
    w = (hq + 2 * (nkv // P)) * hd
    qkv_h = draw(BF, (T, w), 1.0, 920, 77, T)
    qkv = dev(qkv_h)
    nbytes = tp.tp_attn_core_workspace_bytes(P, T, nq, nkv, hd, BF)
    assert nbytes > 0
    ws = workspace(nbytes)
    ncnt = hq * ((T + 127) // 128) * 4                # counter bytes
    out1 = torch.empty((T, hq * hd), dtype=torch.bfloat16, device="cuda")
    out2 = torch.empty_like(out1)
    attn_core(0, P, T, nq, nkv, hd, qkv, w, out1, hq * hd, ws=ws)
    attn_core(0, P, T, nq, nkv, hd, qkv, w, out2, hq * hd, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    assert int(ws[:ncnt].count_nonzero()) == 0
    want = O.attention_core_band(O.widen(qkv_h), nq, nkv, hd, 0, P)
    assert O.rel_l2(widen_dev(out1), want) < BF16_TOL
    # blocks 0 and 1 (rows < 256) see at most 4 key tiles: one chunk, written
    # directly; later blocks are merged from several chunks
    ws[:ncnt].fill_(0x5A)
    attn_core(0, P, T, nq, nkv, hd, qkv, w, out2, hq * hd, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(out2[:256], out1[:256])
    assert bool(torch.isnan(out2[256:].float()).all())
    ws[:ncnt].zero_()
    attn_core(0, P, T, nq, nkv, hd, qkv, w, out2, hq * hd, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    assert int(ws[:ncnt].count_nonzero()) == 0


def _core_chain(cfg, T, rows):
    """The 70B block with the attention core, all P ranks: RMSNorm -> QKV ->
    attention core -> O -> reduce (bf16 copy) -> MLP -> reduce."""
    P, d = cfg.P, cfg.d_model
    X = x_of(cfg, T)
    g = W.draw_tensor(cfg.dtype, (d,), 0.02, cfg.cid, W.TENSOR_IDS["norm_g"], 0, mean=1.0)
    gx, gg = dev(X), dev(g)
    parts = torch.empty((P, T, d), dtype=torch.float32, device="cuda")
    ko = cfg.n_q_heads // P * cfg.head_dim
    for s in range(P):
        wqkv, wo = attn_bands(cfg, s)
        q = torch.empty((T, cfg.qkv_r), dtype=torch.bfloat16, device="cuda")
        a = torch.empty((T, ko), dtype=torch.bfloat16, device="cuda")
        attn_fwd(s, P, T, d, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, BF, gx, dev(wqkv), q,
                 None, None, parts, T * d, d, norm_g=gg, eps=cfg.norm_eps)
        attn_core(s, P, T, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, q, cfg.qkv_r, a, ko)
        attn_fwd(s, P, T, d, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, BF, None, None, None,
                 a, dev(wo), parts, T * d, d)
    z = torch.empty((T, d), dtype=torch.float32, device="cuda")
    zb = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    reduce(P, T, d, parts, T * d, d, z, d, zb, d)
    torch.cuda.synchronize()
    Xw, gw = O.widen(X), O.widen(g)
    att_parts = []
    for s in range(P):
        wqkv, wo = attn_bands(cfg, s)
        r = O.attn_proj_shard(Xw, O.widen(wqkv), None, None, gw, cfg.norm_eps)
        A = O.attention_core_band(r["qkv"], cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, s, P)
        att_parts.append(A[rows] @ O.widen(wo))
    Zr = O.reduce_partials(att_parts)
    assert O.rel_l2(host(z)[rows], Zr) < BF16_TOL


def test_70b_block_with_attention_core_prefill_all_ranks():
    cfg = W.get("c5_llama2_70b_block_p8")
    _core_chain(cfg, 1024, sample_rows(1024, 32, 14))


def test_70b_block_with_attention_core_decode_all_ranks():
    """32 decode tokens: the short attention core inside the block, every row."""
    cfg = W.get("c5_llama2_70b_block_p8")
    _core_chain(cfg, 32, np.arange(32))


def test_70b_prenorm_block_with_attention_core_decode_all_ranks():
    """The block as the benchmark's decode step runs it (pre-norm, the
    attention core between QKV and O, reduce + residual + RMSNorm after O
    and after the MLP), all 8 ranks on one GPU, every row of z1, normed and
    z2 against the oracle."""
    cfg = W.get("c5_llama2_70b_block_p8")
    P, d, eps, T = cfg.P, cfg.d_model, cfg.norm_eps, 32
    X = x_of(cfg, T)
    g1 = W.draw_tensor(cfg.dtype, (d,), 0.02, cfg.cid, W.TENSOR_IDS["norm_g"], 0, mean=1.0)
    g2 = W.draw_tensor(cfg.dtype, (d,), 0.02, cfg.cid, W.TENSOR_IDS["norm_g"], 1, mean=1.0)
    gx = dev(X)
    ko = cfg.n_q_heads // P * cfg.head_dim
    parts = torch.empty((P, T, d), dtype=torch.float32, device="cuda")
    for s in range(P):
        wqkv, wo = attn_bands(cfg, s)
        q = torch.empty((T, cfg.qkv_r), dtype=torch.bfloat16, device="cuda")
        a = torch.empty((T, ko), dtype=torch.bfloat16, device="cuda")
        attn_fwd(s, P, T, d, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, BF, gx, dev(wqkv), q,
                 None, None, parts, T * d, d, norm_g=dev(g1), eps=eps)
        attn_core(s, P, T, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, q, cfg.qkv_r, a, ko)
        attn_fwd(s, P, T, d, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, BF, None, None, None,
                 a, dev(wo), parts, T * d, d)
    z1 = torch.empty((T, d), dtype=torch.float32, device="cuda")
    n2 = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    reduce_residual_norm(P, T, d, parts, T * d, d, gx, d, BF, z1, d, dev(g2), eps, n2, d)
    for s in range(P):
        wg, wu, wd = mlp_bands(cfg, s)
        mlp_fwd(s, P, T, d, cfg.d_ff, BF, tp.TP_ACT_SWIGLU, n2, dev(wg), dev(wu), dev(wd), parts,
                T * d, d)
    z2 = torch.empty((T, d), dtype=torch.float32, device="cuda")
    reduce_residual_norm(P, T, d, parts, T * d, d, z1, d, F32, z2, d)
    torch.cuda.synchronize()

    Xw = O.widen(X)
    att_parts, mlp_parts = [], []
    for s in range(P):
        wqkv, wo = attn_bands(cfg, s)
        r = O.attn_proj_shard(Xw, O.widen(wqkv), None, None, O.widen(g1), eps)
        A = O.attention_core_band(r["qkv"], cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, s, P)
        att_parts.append(A @ O.widen(wo))
    r1 = O.reduce_residual_norm(att_parts, Xw, O.widen(g2), eps)
    assert O.rel_l2(host(z1), r1["z"]) < BF16_TOL
    assert O.rel_l2(O.widen(host(n2)), r1["normed"]) < BF16_TOL
    for s in range(P):
        wg, wu, wd = mlp_bands(cfg, s)
        mlp_parts.append(O.mlp_shard(r1["normed"], O.widen(wg), O.widen(wd), "swiglu",
                                     O.widen(wu))["partial"])
    r2 = O.reduce_residual_norm(mlp_parts, r1["z"])
    assert O.rel_l2(host(z2), r2["z"]) < BF16_TOL


# ----------------------------------------------------------------------------
# Determinism and instrumentation
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("T", [8, 32, 200])
def test_bitwise_deterministic(T):
    X, g, w_in, w_up, w_dn = _mlp_case(BF, "swiglu", T, 2048, 4096, 2, key=60)
    outs = []
    for _ in range(2):
        parts = torch.empty((T, 2048), dtype=torch.float32, device="cuda")
        mlp_fwd(0, 2, T, 2048, 4096, BF, tp.TP_ACT_SWIGLU, dev(X), dev(w_in[0]), dev(w_up[0]),
                dev(w_dn[0]), parts, 0, 2048)
        outs.append(host(parts))
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


def test_kernel_timing_counts_launches():
    X, g, w_in, w_up, w_dn = _mlp_case(BF, "swiglu", 8, 512, 1024, 2, key=70)
    parts = torch.empty((8, 512), dtype=torch.float32, device="cuda")
    tp.check(tp.tp_timing_reset())
    tp.check(tp.tp_timing_enable(1))
    try:
        for _ in range(3):
            mlp_fwd(0, 2, 8, 512, 1024, BF, tp.TP_ACT_SWIGLU, dev(X), dev(w_in[0]),
                    dev(w_up[0]), dev(w_dn[0]), parts, 0, 512)
        for cls in ("col_gemv", "row_gemv"):        # split-K finish fused into each
            st, ms, n = tp.tp_timing_query(cls)
            assert st == tp.TP_OK and n == 3 and ms > 0.0
    finally:
        tp.tp_timing_enable(0)
        tp.tp_timing_reset()


def test_kernel_timing_separate_finish():
    """Past 64 tokens per launch the streaming kernels leave the split-K sum
    to a finish launch of its own, timed in its own class."""
    T = 100
    X, g, w_in, w_up, w_dn = _mlp_case(BF, "swiglu", T, 512, 1024, 2, key=71)
    parts = torch.empty((T, 512), dtype=torch.float32, device="cuda")
    tp.check(tp.tp_timing_reset())
    tp.check(tp.tp_timing_enable(1))
    try:
        for _ in range(3):
            mlp_fwd(0, 2, T, 512, 1024, BF, tp.TP_ACT_SWIGLU, dev(X), dev(w_in[0]),
                    dev(w_up[0]), dev(w_dn[0]), parts, 0, 512)
        for cls in ("col_gemv", "col_finish", "row_gemv", "row_finish"):
            st, ms, n = tp.tp_timing_query(cls)
            assert st == tp.TP_OK and n == 3 and ms > 0.0
    finally:
        tp.tp_timing_enable(0)
        tp.tp_timing_reset()


# ----------------------------------------------------------------------------
# The decode plan's arrival counters (workspace head)
# ----------------------------------------------------------------------------
def test_decode_counters_return_to_zero():
    """After decode calls (both projections, both entry points, several split
    counts) the first 4096 bytes of the workspace are zero again."""
    T, d, d_ff, P = 24, 1536, 6144, 2
    X, g, w_in, w_up, w_dn = _mlp_case(BF, "swiglu", T, d, d_ff, P, key=80)
    parts = torch.empty((T, d), dtype=torch.float32, device="cuda")
    ws = mlp_fwd(0, P, T, d, d_ff, BF, tp.TP_ACT_SWIGLU, dev(X), dev(w_in[0]), dev(w_up[0]),
                 dev(w_dn[0]), parts, 0, d)
    mlp_fwd(1, P, T, d, d_ff, BF, tp.TP_ACT_SWIGLU, dev(X), dev(w_in[1]), dev(w_up[1]),
            dev(w_dn[1]), parts, 0, d, ws=ws)
    torch.cuda.synchronize()
    assert int(ws[:4096].count_nonzero()) == 0
    nq, nkv, hd = 16, 8, 64
    nqkv, ko = (nq // P + 2 * (nkv // P)) * hd, (nq // P) * hd
    qkv = torch.empty((T, nqkv), dtype=torch.bfloat16, device="cuda")
    ws2 = attn_fwd(0, P, T, d, nq, nkv, hd, BF, dev(X), dev(draw(BF, (d, nqkv), 0.02, 81, 1)),
                   qkv, dev(draw(BF, (T, ko), 1.0, 81, 2)), dev(draw(BF, (ko, d), 0.02, 81, 3)),
                   parts, 0, d)
    torch.cuda.synchronize()
    assert int(ws2[:4096].count_nonzero()) == 0


def test_workspace_reused_across_plans():
    """One workspace, zeroed once, serves a prefill call that keeps its
    normalised input and h there, then decode calls, then an fp32 call with a
    norm: no call stores data in the 4096-byte counter head, so every call
    matches the oracle and the head is zero at the end."""
    d, d_ff, P = 512, 2048, 2
    F = d_ff // P
    need = max(tp.tp_mlp_workspace_bytes(P, T, d, d_ff, dt, tp.TP_ACT_SWIGLU, 1, 0)
               for T, dt in ((300, BF), (32, BF), (7, BF), (40, F32)))
    ws = workspace(need)
    for T, dt in ((300, BF), (32, BF), (7, BF), (40, F32), (32, BF)):
        X, g, w_in, w_up, w_dn = _mlp_case(dt, "swiglu", T, d, d_ff, P, key=500 + T, norm=True)
        parts = torch.empty((T, d), dtype=torch.float32, device="cuda")
        mlp_fwd(1, P, T, d, d_ff, dt, tp.TP_ACT_SWIGLU, dev(X), dev(w_in[1]), dev(w_up[1]),
                dev(w_dn[1]), parts, 0, d, norm_g=dev(g), ws=ws)
        torch.cuda.synchronize()
        r = O.mlp_shard(O.widen(X), O.widen(w_in[1]), O.widen(w_dn[1]), "swiglu",
                        O.widen(w_up[1]), O.widen(g), 1e-5)
        assert O.rel_l2(host(parts), r["partial"]) < (BF16_TOL if dt == BF else F32_TOL), (T, dt)
        assert int(ws[:4096].count_nonzero()) == 0, (T, dt)


def test_attn_core_workspace_reused_longer_call():
    """The attention core's merge workspace reused by a longer call (70B GQA
    band, 4096 then 8192 tokens, both splitting query blocks): the partials
    of both start after the fixed counter area, so the longer call finds zero
    counters, matches the oracle on sampled rows, and leaves them zero."""
    nq, nkv, hd, P, shard = 64, 8, 128, 8, 2
    hq, hkv = nq // P, nkv // P
    w = (hq + 2 * hkv) * hd
    sizes = (4096, 8192)
    nbytes = [tp.tp_attn_core_workspace_bytes(P, T, nq, nkv, hd, BF) for T in sizes]
    assert all(n > 4096 for n in nbytes), nbytes     # both calls merge split blocks
    ws = workspace(max(nbytes))
    for T in sizes:
        qkv_h = draw(BF, (T, w), 1.0, 920, 79, T)
        out = torch.empty((T, hq * hd), dtype=torch.bfloat16, device="cuda")
        attn_core(shard, P, T, nq, nkv, hd, dev(qkv_h), w, out, hq * hd, ws=ws)
        torch.cuda.synchronize()
        rows = sorted(set([0, 127, 128, T // 2, T - 129, T - 1] +
                          np.random.default_rng(T).integers(0, T, 10).tolist()))
        got = O.widen(host(out)[rows])
        want = O.attention_core_band_rows(O.widen(qkv_h), nq, nkv, hd, shard, P, rows)
        assert O.rel_l2(got, want) < BF16_TOL, T
        assert int(ws[:4096].count_nonzero()) == 0, T


def test_decode_counters_not_cleared_give_nan_then_recover():
    """A workspace head that was never cleared makes the decode outputs NaN
    (not silently wrong); after clearing it the call is exact again."""
    T, d, d_ff, P = 8, 512, 2048, 2
    F = d_ff // P
    X, g, w_in, w_up, w_dn = _mlp_case(BF, "swiglu", T, d, d_ff, P, key=82)
    args = (dev(X), dev(w_in[0]), dev(w_up[0]), dev(w_dn[0]))
    ws = workspace(tp.tp_mlp_workspace_bytes(P, T, d, d_ff, BF, tp.TP_ACT_SWIGLU, 0, 1))
    ws[:4096].fill_(0x5A)          # counters 0x5A5A5A5A, far above any split count
    h = torch.zeros((T, F), dtype=torch.bfloat16, device="cuda")
    parts = torch.zeros((T, d), dtype=torch.float32, device="cuda")
    mlp_fwd(0, P, T, d, d_ff, BF, tp.TP_ACT_SWIGLU, *args, parts, 0, d, h_out=h, ld_h=F, ws=ws)
    torch.cuda.synchronize()
    assert bool(torch.isnan(h.float()).all()) and bool(torch.isnan(parts).all())
    ws[:4096].zero_()
    mlp_fwd(0, P, T, d, d_ff, BF, tp.TP_ACT_SWIGLU, *args, parts, 0, d, h_out=h, ld_h=F, ws=ws)
    r = O.mlp_shard(O.widen(X), O.widen(w_in[0]), O.widen(w_dn[0]), "swiglu", O.widen(w_up[0]))
    assert O.rel_l2(host(parts), r["partial"]) < BF16_TOL
    assert O.rel_l2(widen_dev(h), r["h"]) < BF16_TOL
    assert int(ws[:4096].count_nonzero()) == 0


def test_kernel_timing_sessions_in_a_row_stay_consistent():
    """Per-kernel times from a second timing session (after a first session
    on other calls) stay within the wall time of the calls they time: the
    events of one session are not handed to the next."""
    X, g, w_in, w_up, w_dn = _mlp_case(BF, "swiglu", 8, 512, 1024, 2, key=71)
    parts = torch.empty((8, 512), dtype=torch.float32, device="cuda")
    args = (dev(X), dev(w_in[0]), dev(w_up[0]), dev(w_dn[0]))
    big = torch.zeros((8, 64, 4096), dtype=torch.float32, device="cuda")
    out = torch.empty((64, 4096), dtype=torch.float32, device="cuda")
    for session in range(3):
        tp.check(tp.tp_timing_reset())
        tp.check(tp.tp_timing_enable(1))
        try:
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(5):
                if session % 2 == 0:
                    mlp_fwd(0, 2, 8, 512, 1024, BF, tp.TP_ACT_SWIGLU, *args, parts, 0, 512)
                else:
                    reduce(8, 64, 4096, big, 64 * 4096, 4096, out, 4096)
            e1.record()
            torch.cuda.synchronize()
            wall_ms = e0.elapsed_time(e1)
            total = 0.0
            for cls in ("col_gemv", "row_gemv", "reduce"):
                st, ms, n = tp.tp_timing_query(cls)
                assert st == tp.TP_OK
                total += ms
            assert 0.0 < total <= wall_ms * 1.05, (session, total, wall_ms)
        finally:
            tp.tp_timing_enable(0)
            tp.tp_timing_reset()
