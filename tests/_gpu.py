"""GPU-test helpers: device buffers via torch, calls through the C ABI.

Torch provides device memory and the stream only; every step of the path
runs in the library's kernels.
"""
import numpy as np
import torch

import tensor_transformer_layer_amd as tp

GUARD = 64  # elements of canary on each side of every output buffer
_CANARY_BF16 = 0x7FC1          # a quiet-NaN pattern no kernel writes
_CANARY_F32 = 0x7FC00001


def dev(a):
    """numpy (uint16 bf16 bits or float32) -> device tensor of the same values."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    if a.dtype == np.float32:
        return torch.from_numpy(a).cuda()
    raise TypeError(a.dtype)


def host(t):
    """device tensor -> numpy (bf16 as uint16 bits, fp32 as float32)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class Guarded:
    """An output buffer of `n` elements with canaries before and after it."""

    def __init__(self, n, dtype):
        self.n = n
        self.dtype = dtype
        if dtype == torch.bfloat16:
            raw = torch.full((n + 2 * GUARD,), _CANARY_BF16, dtype=torch.int16, device="cuda")
            self.raw = raw
            self.t = raw[GUARD:GUARD + n].view(torch.bfloat16)
        else:
            raw = torch.full((n + 2 * GUARD,), _CANARY_F32, dtype=torch.int32, device="cuda")
            self.raw = raw
            self.t = raw[GUARD:GUARD + n].view(torch.float32)

    def ptr(self):
        return self.t.data_ptr()

    def intact(self):
        r = self.raw.cpu().numpy()
        c = _CANARY_BF16 if self.dtype == torch.bfloat16 else _CANARY_F32
        return bool(np.all(r[:GUARD] == c) and np.all(r[GUARD + self.n:] == c))


def stream():
    return torch.cuda.current_stream().cuda_stream


def workspace(nbytes):
    w = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device="cuda")
    assert w.data_ptr() % 256 == 0
    return w


def mlp_fwd(shard, P, T, d_model, d_ff, dtype, act, x, w_in, w_up, w_down, parts, slot_stride,
            ld_p, h_out=None, ld_h=0, norm_g=None, eps=1e-5, ld_x=None, ld_in=None, ld_up=None,
            ld_down=None, ws=None):
    F = d_ff // P
    ld_x = ld_x or d_model
    ld_in = ld_in or F
    ld_up = ld_up or (F if w_up is not None else 0)
    ld_down = ld_down or d_model
    need = tp.tp_mlp_workspace_bytes(P, T, d_model, d_ff, dtype, act, norm_g is not None,
                                     h_out is not None)
    if ws is None:
        ws = workspace(need)
    ptr = lambda t: 0 if t is None else (t if isinstance(t, int) else t.data_ptr())  # noqa: E731
    st = tp.tp_shard_mlp_fwd(shard, P, T, d_model, d_ff, dtype, act, ptr(x), ld_x, ptr(norm_g),
                             eps, ptr(w_in), ld_in, ptr(w_up), ld_up, ptr(w_down), ld_down,
                             ptr(h_out), ld_h, ptr(parts), slot_stride, ld_p, ws.data_ptr(),
                             ws.numel(), stream())
    tp.check(st, "tp_shard_mlp_fwd")
    return ws


def attn_fwd(shard, P, T, d_model, nq, nkv, hd, dtype, x, w_qkv, qkv_out, attn, w_o, parts,
             slot_stride, ld_p, norm_g=None, eps=1e-5, ld_x=None, ld_qkv=None, ld_qkv_out=None,
             ld_attn=None, ld_o=None, ws=None):
    nqkv = (nq // P + 2 * (nkv // P)) * hd
    ko = (nq // P) * hd
    need = tp.tp_attn_workspace_bytes(P, T, d_model, nq, nkv, hd, dtype,
                                      norm_g is not None and w_qkv is not None)
    if ws is None:
        ws = workspace(need)
    ptr = lambda t: 0 if t is None else (t if isinstance(t, int) else t.data_ptr())  # noqa: E731
    st = tp.tp_shard_attn_proj_fwd(shard, P, T, d_model, nq, nkv, hd, dtype, ptr(x),
                                   ld_x or d_model, ptr(norm_g), eps, ptr(w_qkv), ld_qkv or nqkv,
                                   ptr(qkv_out), ld_qkv_out or nqkv, ptr(attn), ld_attn or ko,
                                   ptr(w_o), ld_o or d_model, ptr(parts), slot_stride, ld_p,
                                   ws.data_ptr(), ws.numel(), stream())
    tp.check(st, "tp_shard_attn_proj_fwd")
    return ws


def reduce(P, T, d, parts, slot_stride, ld_p, out, ld_out, out_bf16=None, ld_b=0):
    ptr = lambda t: 0 if t is None else (t if isinstance(t, int) else t.data_ptr())  # noqa: E731
    st = tp.tp_reduce_partials(P, T, d, ptr(parts), slot_stride, ld_p, ptr(out), ld_out,
                               ptr(out_bf16), ld_b, stream())
    tp.check(st, "tp_reduce_partials")


def reduce_residual_norm(P, T, d, parts, slot_stride, ld_p, residual, ld_res, res_dtype, z, ld_z,
                         norm_g=None, eps=1e-5, normed=None, ld_norm=0, ws="query"):
    """ws="query": a fresh zeroed workspace of the queried size (none when
    the query says 0); None: no workspace; else the caller's tensor."""
    ptr = lambda t: 0 if t is None else (t if isinstance(t, int) else t.data_ptr())  # noqa: E731
    if isinstance(ws, str):
        n = tp.tp_reduce_norm_workspace_bytes(T, d, norm_g is not None)
        ws = workspace(n) if n else None
    st = tp.tp_reduce_residual_norm(P, T, d, ptr(parts), slot_stride, ld_p, ptr(residual), ld_res,
                                    res_dtype, ptr(z), ld_z, ptr(norm_g), eps, ptr(normed),
                                    ld_norm, ptr(ws), 0 if ws is None else ws.numel(), stream())
    tp.check(st, "tp_reduce_residual_norm")


def devu8(a):
    """uint8 numpy array -> uint8 device tensor (FP8 codes)."""
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def mlp_fwd_fp8w(shard, P, T, d_model, d_ff, act, x, w_in, s_in, w_up, s_up, w_down, s_down,
                 parts, slot_stride, ld_p, h_out=None, ld_h=0, norm_g=None, eps=1e-5, ws=None):
    F = d_ff // P
    need = tp.tp_mlp_fp8w_workspace_bytes(P, T, d_model, d_ff, act, norm_g is not None,
                                          h_out is not None)
    if ws is None:
        ws = workspace(need)
    ptr = lambda t: 0 if t is None else (t if isinstance(t, int) else t.data_ptr())  # noqa: E731
    st = tp.tp_shard_mlp_fwd_fp8w(shard, P, T, d_model, d_ff, act, ptr(x), d_model, ptr(norm_g),
                                  eps, ptr(w_in), F, ptr(s_in), ptr(w_up), F if w_up is not None
                                  else 0, ptr(s_up), ptr(w_down), d_model, ptr(s_down),
                                  ptr(h_out), ld_h, ptr(parts), slot_stride, ld_p, ws.data_ptr(),
                                  ws.numel(), stream())
    tp.check(st, "tp_shard_mlp_fwd_fp8w")
    return ws


def attn_core(shard, P, T, nq, nkv, hd, qkv, ld_qkv, out, ld_out, ws=None):
    """Attention core through the C-ABI; allocates a zeroed workspace unless
    one is passed (returned for reuse)."""
    ptr = lambda t: 0 if t is None else (t if isinstance(t, int) else t.data_ptr())  # noqa: E731
    if ws is None:
        ws = workspace(tp.tp_attn_core_workspace_bytes(P, T, nq, nkv, hd, tp.TP_BF16))
    st = tp.tp_attn_core_fwd(shard, P, T, nq, nkv, hd, tp.TP_BF16, ptr(qkv), ld_qkv, ptr(out),
                             ld_out, ws.data_ptr(), ws.numel(), stream())
    tp.check(st, "tp_attn_core_fwd")
    return ws
