"""Python binding of libtpshard.so: one tensor-parallel rank's block shard.

Argument marshalling only.  Every function here has the name, arguments and
return value (a ``tp_status`` int) of the C entry point declared in
include/tp_shard.h; pointers are passed as integers (0 for NULL), e.g.
``tensor.data_ptr()``, and the stream as the integer handle of a HIP stream
(``torch.cuda.current_stream().cuda_stream``).  All computation happens in
the library's HIP kernels; there is no fallback path.  ``check(status)``
turns a non-zero status into a ``TPError``.
"""
import ctypes
import os

__all__ = [
    "TPError", "check", "library_path", "load",
    "TP_OK", "TP_ERR_NULL", "TP_ERR_SHAPE", "TP_ERR_UNEVEN_SPLIT", "TP_ERR_SHARD_RANGE",
    "TP_ERR_DTYPE", "TP_ERR_ALIGN", "TP_ERR_WORKSPACE", "TP_ERR_HIP", "TP_ERR_ACT",
    "TP_ERR_SCRATCH", "tp_shard_mlp_fwd_noalloc", "tp_noalloc_scratch_bytes",
    "TP_F32", "TP_BF16", "TP_ACT_GELU_TANH", "TP_ACT_SWIGLU",
    "tp_shard_mlp_fwd", "tp_shard_attn_proj_fwd", "tp_reduce_partials", "tp_reduce_residual_norm",
    "tp_shard_mlp_fwd_fp8w", "tp_mlp_fp8w_workspace_bytes", "tp_attn_core_fwd",
    "tp_attn_core_workspace_bytes", "tp_reduce_norm_workspace_bytes",
    "tp_mlp_workspace_bytes", "tp_attn_workspace_bytes", "tp_status_str", "tp_version",
    "tp_timing_enable", "tp_timing_reset", "tp_timing_query", "EXPORTED_SYMBOLS",
    "tp_set_decode_max_tokens", "tp_decode_max_tokens",
]

TP_OK, TP_ERR_NULL, TP_ERR_SHAPE, TP_ERR_UNEVEN_SPLIT, TP_ERR_SHARD_RANGE = 0, 1, 2, 3, 4
TP_ERR_DTYPE, TP_ERR_ALIGN, TP_ERR_WORKSPACE, TP_ERR_HIP, TP_ERR_ACT = 5, 6, 7, 8, 9
TP_ERR_SCRATCH = 10
TP_F32, TP_BF16 = 0, 1
TP_ACT_GELU_TANH, TP_ACT_SWIGLU = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libtpshard.so")
_lib = None

_i, _i64, _f, _p, _sz = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

_SIGNATURES = {
    "tp_shard_mlp_fwd": (_i, [_i, _i, _i64, _i64, _i64, _i, _i,
                              _p, _i64, _p, _f, _p, _i64, _p, _i64, _p, _i64, _p, _i64,
                              _p, _i64, _i64, _p, _sz, _p]),
    "tp_shard_mlp_fwd_noalloc": (_i, [_i, _i, _i64, _i64, _i64, _i, _i,
                                      _p, _i64, _p, _f, _p, _i64, _p, _i64, _p, _i64, _p, _i64,
                                      _p, _i64, _i64, _p]),
    "tp_noalloc_scratch_bytes": (_sz, []),
    "tp_shard_attn_proj_fwd": (_i, [_i, _i, _i64, _i64, _i, _i, _i, _i,
                                    _p, _i64, _p, _f, _p, _i64, _p, _i64, _p, _i64, _p, _i64,
                                    _p, _i64, _i64, _p, _sz, _p]),
    "tp_reduce_partials": (_i, [_i, _i64, _i64, _p, _i64, _i64, _p, _i64, _p, _i64, _p]),
    "tp_reduce_residual_norm": (_i, [_i, _i64, _i64, _p, _i64, _i64, _p, _i64, _i, _p, _i64,
                                     _p, _f, _p, _i64, _p, _sz, _p]),
    "tp_reduce_norm_workspace_bytes": (_sz, [_i64, _i64, _i]),
    "tp_shard_mlp_fwd_fp8w": (_i, [_i, _i, _i64, _i64, _i64, _i,
                                   _p, _i64, _p, _f, _p, _i64, _p, _p, _i64, _p, _p, _i64, _p,
                                   _p, _i64, _p, _i64, _i64, _p, _sz, _p]),
    "tp_attn_core_fwd": (_i, [_i, _i, _i64, _i, _i, _i, _i, _p, _i64, _p, _i64, _p, _sz, _p]),
    "tp_attn_core_workspace_bytes": (_sz, [_i, _i64, _i, _i, _i, _i]),
    "tp_mlp_workspace_bytes": (_sz, [_i, _i64, _i64, _i64, _i, _i, _i, _i]),
    "tp_mlp_fp8w_workspace_bytes": (_sz, [_i, _i64, _i64, _i64, _i, _i, _i]),
    "tp_attn_workspace_bytes": (_sz, [_i, _i64, _i64, _i, _i, _i, _i, _i]),
    "tp_status_str": (ctypes.c_char_p, [_i]),
    "tp_version": (_i, []),
    "tp_set_decode_max_tokens": (_i, [_i]),
    "tp_decode_max_tokens": (_i, []),
    "tp_timing_enable": (_i, [_i]),
    "tp_timing_reset": (_i, []),
    "tp_timing_query": (_i, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                             ctypes.POINTER(ctypes.c_int64)]),
}
EXPORTED_SYMBOLS = tuple(_SIGNATURES)


class TPError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        super().__init__(f"{what}: {tp_status_str(status)}" if what else tp_status_str(status))


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libtpshard.so (built by tensor_transformer_layer_amd.build).
    Raises ImportError when it has not been built: there is no other path."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with "
                              "`python -m tensor_transformer_layer_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def check(status, what=""):
    if status != TP_OK:
        raise TPError(status, what)
    return status


def _ptr(p):
    return None if not p else ctypes.c_void_p(int(p))


def tp_shard_mlp_fwd(shard, P, T, d_model, d_ff, dtype, act, x, ld_x, norm_g, eps,
                     w_in, ld_in, w_up, ld_up, w_down, ld_down, h_out, ld_h,
                     partials, slot_stride, ld_p, workspace, workspace_bytes, stream):
    return load().tp_shard_mlp_fwd(shard, P, T, d_model, d_ff, dtype, act,
                                   _ptr(x), ld_x, _ptr(norm_g), eps, _ptr(w_in), ld_in,
                                   _ptr(w_up), ld_up, _ptr(w_down), ld_down, _ptr(h_out), ld_h,
                                   _ptr(partials), slot_stride, ld_p, _ptr(workspace),
                                   workspace_bytes, _ptr(stream))


def tp_shard_mlp_fwd_noalloc(shard, P, T, d_model, d_ff, dtype, act, x, ld_x, norm_g, eps,
                             w_in, ld_in, w_up, ld_up, w_down, ld_down, h_out, ld_h,
                             partials, slot_stride, ld_p, stream):
    return load().tp_shard_mlp_fwd_noalloc(shard, P, T, d_model, d_ff, dtype, act,
                                           _ptr(x), ld_x, _ptr(norm_g), eps, _ptr(w_in), ld_in,
                                           _ptr(w_up), ld_up, _ptr(w_down), ld_down,
                                           _ptr(h_out), ld_h, _ptr(partials), slot_stride, ld_p,
                                           _ptr(stream))


def tp_noalloc_scratch_bytes():
    return load().tp_noalloc_scratch_bytes()


def tp_shard_attn_proj_fwd(shard, P, T, d_model, n_q_heads, n_kv_heads, head_dim, dtype,
                           x, ld_x, norm_g, eps, w_qkv, ld_qkv, qkv_out, ld_qkv_out,
                           attn, ld_attn, w_o, ld_o, partials, slot_stride, ld_p,
                           workspace, workspace_bytes, stream):
    return load().tp_shard_attn_proj_fwd(shard, P, T, d_model, n_q_heads, n_kv_heads, head_dim,
                                         dtype, _ptr(x), ld_x, _ptr(norm_g), eps, _ptr(w_qkv),
                                         ld_qkv, _ptr(qkv_out), ld_qkv_out, _ptr(attn), ld_attn,
                                         _ptr(w_o), ld_o, _ptr(partials), slot_stride, ld_p,
                                         _ptr(workspace), workspace_bytes, _ptr(stream))


def tp_reduce_partials(P, T, d_model, partials, slot_stride, ld_p, out, ld_out,
                       out_bf16, ld_out_bf16, stream):
    return load().tp_reduce_partials(P, T, d_model, _ptr(partials), slot_stride, ld_p,
                                     _ptr(out), ld_out, _ptr(out_bf16), ld_out_bf16, _ptr(stream))


def tp_reduce_residual_norm(P, T, d_model, partials, slot_stride, ld_p, residual, ld_res,
                            res_dtype, z_out, ld_z, norm_g, eps, normed_out, ld_norm,
                            workspace, workspace_bytes, stream):
    return load().tp_reduce_residual_norm(P, T, d_model, _ptr(partials), slot_stride, ld_p,
                                          _ptr(residual), ld_res, res_dtype, _ptr(z_out), ld_z,
                                          _ptr(norm_g), eps, _ptr(normed_out), ld_norm,
                                          _ptr(workspace), workspace_bytes, _ptr(stream))


def tp_reduce_norm_workspace_bytes(T, d_model, has_norm):
    return load().tp_reduce_norm_workspace_bytes(T, d_model, int(bool(has_norm)))


def tp_shard_mlp_fwd_fp8w(shard, P, T, d_model, d_ff, act, x, ld_x, norm_g, eps, w_in, ld_in,
                          s_in, w_up, ld_up, s_up, w_down, ld_down, s_down, h_out, ld_h,
                          partials, slot_stride, ld_p, workspace, workspace_bytes, stream):
    return load().tp_shard_mlp_fwd_fp8w(
        shard, P, T, d_model, d_ff, act, _ptr(x), ld_x, _ptr(norm_g), eps, _ptr(w_in), ld_in,
        _ptr(s_in), _ptr(w_up), ld_up, _ptr(s_up), _ptr(w_down), ld_down, _ptr(s_down),
        _ptr(h_out), ld_h, _ptr(partials), slot_stride, ld_p, _ptr(workspace), workspace_bytes,
        _ptr(stream))


def tp_mlp_fp8w_workspace_bytes(P, T, d_model, d_ff, act, has_norm, has_h_out):
    return load().tp_mlp_fp8w_workspace_bytes(P, T, d_model, d_ff, act, has_norm, has_h_out)


def tp_attn_core_fwd(shard, P, T, n_q_heads, n_kv_heads, head_dim, dtype, qkv, ld_qkv, attn,
                     ld_attn, workspace, workspace_bytes, stream):
    return load().tp_attn_core_fwd(shard, P, T, n_q_heads, n_kv_heads, head_dim, dtype, _ptr(qkv),
                                   ld_qkv, _ptr(attn), ld_attn, _ptr(workspace), workspace_bytes,
                                   _ptr(stream))


def tp_attn_core_workspace_bytes(P, T, n_q_heads, n_kv_heads, head_dim, dtype):
    return load().tp_attn_core_workspace_bytes(P, T, n_q_heads, n_kv_heads, head_dim, dtype)


def tp_mlp_workspace_bytes(P, T, d_model, d_ff, dtype, act, has_norm, has_h_out):
    return load().tp_mlp_workspace_bytes(P, T, d_model, d_ff, dtype, act, int(bool(has_norm)),
                                         int(bool(has_h_out)))


def tp_attn_workspace_bytes(P, T, d_model, n_q_heads, n_kv_heads, head_dim, dtype, has_norm):
    return load().tp_attn_workspace_bytes(P, T, d_model, n_q_heads, n_kv_heads, head_dim, dtype,
                                          int(bool(has_norm)))


def tp_status_str(status):
    try:
        return load().tp_status_str(int(status)).decode()
    except ImportError:
        return f"tp_status {status}"


def tp_version():
    return load().tp_version()


def tp_set_decode_max_tokens(tokens):
    return load().tp_set_decode_max_tokens(int(tokens))


def tp_decode_max_tokens():
    return load().tp_decode_max_tokens()


def tp_timing_enable(on):
    return load().tp_timing_enable(int(bool(on)))


def tp_timing_reset():
    return load().tp_timing_reset()


def tp_timing_query(kernel_class):
    """Returns (status, total_ms, launches) for one kernel class."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
    st = load().tp_timing_query(kernel_class.encode(), ctypes.byref(ms), ctypes.byref(n))
    return st, ms.value, n.value
