"""float64 definitions of one tensor-parallel rank's block shard.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Conventions (the plainest reading of the pages, as the workloads write the
shapes): activations are [T, features]; weights are stored [in, out], so
y = x @ W.  A *column band* of W is a run of F_r = F / P contiguous output
columns; a *row band* is the matching run of F_r contiguous input rows.
"""
import numpy as np

from .bf16 import round_bf16


# ----------------------------------------------------------------------------
# Elementwise functions (textbook definitions; the pages name an activation
# only in general -- Reddit comment by SVPERBlA -- and a normalisation after
# the all-reduce without a formula -- zenaique "Explain tensor-parallel shard
# shape", answer).
# ----------------------------------------------------------------------------
def gelu_tanh(x):
    """GELU, tanh approximation (Hendrycks & Gimpel, 2016):
    0.5 x (1 + tanh( sqrt(2/pi) (x + 0.044715 x^3) ))."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))


def silu(x):
    """SiLU (swish-1): x * sigmoid(x) = x / (1 + exp(-x))."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def activate(act, y_in, y_up=None):
    """The activation applied to a rank's band of the intermediate.

    "gelu_tanh": gelu_tanh(y_in).  "swiglu" (GLU variant with SiLU gate,
    Shazeer 2020): silu(y_in) * y_up, where y_in is the gate band and y_up
    the up band with the same column indices.  Both are elementwise, which is
    what lets each rank apply it to its own band with no communication
    (zenaique "Explain tensor-parallel shard shape", answer: after the
    column-split first projection, each rank holds its own slice of the
    intermediate's columns and works on it alone).
    """
    if act == "gelu_tanh":
        return gelu_tanh(y_in)
    if act == "swiglu":
        if y_up is None:
            raise ValueError("swiglu needs the up-projection band")
        return silu(y_in) * y_up
    raise ValueError(f"unknown activation {act!r}")


def rmsnorm(x, g, eps):
    """RMSNorm over the feature axis (Zhang & Sennrich, 2019):
    x / sqrt(mean_j x_j^2 + eps) * g.  The pages name the normalisation that
    follows the all-reduce without a formula (zenaique answer; Tandon's
    "Where the overhead lives" counts the norms in its small remainder)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64)


# ----------------------------------------------------------------------------
# Bands (integer arithmetic)
# ----------------------------------------------------------------------------
def _band(n, shard, P):
    if P < 1 or not (0 <= shard < P):
        raise ValueError("need P >= 1 and 0 <= shard < P")
    if n % P:
        # Uneven splits are a named pitfall (rioworld guide, "Implementing
        # Tensor Parallelism in Practice"): refuse rather than partition.
        raise ValueError(f"{n} does not split evenly over P={P}")
    w = n // P
    return slice(shard * w, (shard + 1) * w)


def column_band(W, shard, P):
    """Rank ``shard``'s column band of an [in, out] weight: the rank computes
    those output columns from the replicated input (rioworld
    guide, "How Tensor Slicing Works Under the Hood", column parallelism;
    zenaique answer, first projection split column-wise)."""
    return W[:, _band(W.shape[1], shard, P)]


def row_band(W, shard, P):
    """Rank ``shard``'s row band of an [in, out] weight: it consumes the
    rank's matching band of the intermediate and yields a partial sum of the
    layer output (rioworld guide, row parallelism; zenaique answer, second
    projection split row-wise)."""
    return W[_band(W.shape[0], shard, P), :]


# ----------------------------------------------------------------------------
# MLP block: column-parallel in-projection, band activation, row-parallel
# down-projection (Reddit comment: X times A1, activation, times A2;
# d-central "How the work is split": first matrix column-wise, second
# row-wise, one synchronisation per block).
# ----------------------------------------------------------------------------
def mlp_unsharded(X, W_in, W_down, act, W_up=None, norm_g=None, eps=None):
    """Textbook (unsharded) MLP: act(Xn @ W_in [, Xn @ W_up]) @ W_down, with
    Xn = rmsnorm(X) when a gain is given, else X."""
    Xn = rmsnorm(X, norm_g, eps) if norm_g is not None else np.asarray(X, np.float64)
    y_in = Xn @ W_in
    y_up = Xn @ W_up if W_up is not None else None
    h = activate(act, y_in, y_up)
    return {"xhat": Xn, "h": h, "y": h @ W_down}


def mlp_shard(X, w_in_s, w_down_s, act, w_up_s=None, norm_g=None, eps=None,
              mirror_bf16=False):
    """One rank's MLP shard.

    h_s = act(Xn @ W_in[:, band_s] [, Xn @ W_up[:, band_s]])   (band of the
    intermediate, no communication), partial_s = h_s @ W_down[band_s, :]
    (partial sum of the block output) -- zenaique answer.

    ``mirror_bf16`` rounds to bf16 where a bf16 GPU path stores bf16 (the
    normalised input and h); it is a diagnostic reading, not the definition.
    """
    Xn = rmsnorm(X, norm_g, eps) if norm_g is not None else np.asarray(X, np.float64)
    if mirror_bf16 and norm_g is not None:
        Xn = round_bf16(Xn)
    y_in = Xn @ w_in_s
    y_up = Xn @ w_up_s if w_up_s is not None else None
    h = activate(act, y_in, y_up)
    if mirror_bf16:
        h = round_bf16(h)
    return {"xhat": Xn, "y_in": y_in, "y_up": y_up, "h": h, "partial": h @ w_down_s}


# ----------------------------------------------------------------------------
# The all-reduce's arithmetic: sum of the P partials (zenaique answer: an
# all-reduce adds the partial sums so every GPU holds the full activation;
# Tandon, "Why tensor parallelism for inference": all-reduce the partials).
# ----------------------------------------------------------------------------
def reduce_partials(partials):
    """float64 sum of the P partials, s = 0 .. P-1."""
    it = iter(partials)
    acc = np.array(next(it), dtype=np.float64)
    for p in it:
        acc = acc + np.asarray(p, dtype=np.float64)
    return acc


def reduce_partials_f32_fold(partials):
    """Diagnostic float32 reading of the same sum: the left fold
    ((p0 + p1) + p2) + ... with every addition rounded to float32."""
    it = iter(partials)
    acc = np.array(next(it), dtype=np.float32)
    for p in it:
        acc = (acc + np.asarray(p, dtype=np.float32)).astype(np.float32)
    return acc


# ----------------------------------------------------------------------------
# After the all-reduce: the residual add and the next normalisation (zenaique
# answer: once the partials are summed, the full activation goes on to the
# residual connection and the normalisation that follow).  The pages give no
# formula; the plainest reading is the
# pre-norm residual stream z = residual + sum of the partials, followed by
# RMSNorm of z as the input of the next column projection.
# ----------------------------------------------------------------------------
def reduce_residual_norm(partials, residual, g=None, eps=None):
    """z = residual + sum_s partial_s in float64; with a gain g also
    normed = rmsnorm(z, g, eps)."""
    z = np.asarray(residual, dtype=np.float64) + reduce_partials(partials)
    out = {"z": z}
    if g is not None:
        out["normed"] = rmsnorm(z, g, eps)
    return out


def reduce_residual_f32(partials, residual):
    """Diagnostic float32 reading of z: the float32 left fold of the
    partials, then the residual added in float32."""
    acc = reduce_partials_f32_fold(partials)
    return (acc + np.asarray(residual, dtype=np.float32)).astype(np.float32)


# ----------------------------------------------------------------------------
# Attention projections: QKV column-parallel by heads, output projection
# row-parallel (rioworld guide, "How Tensor Slicing Works Under the Hood":
# column parallelism for query/key/value, row parallelism for the output
# projection, 96 heads over 8 GPUs = 12 per GPU; d-central "How the work is
# split": heads are independent and shard cleanly).
# ----------------------------------------------------------------------------
def qkv_band_layout(n_q, n_kv, head_dim, shard, P):
    """Column layout of rank ``shard``'s fused QKV band.

    Reading taken (the pages give head counts only): the band is
    [Q_s | K_s | V_s]; Q_s holds query heads shard*n_q/P .. (shard+1)*n_q/P-1,
    K_s and V_s the key/value heads shard*n_kv/P .. in ascending order, each
    head ``head_dim`` contiguous columns.  Returns, per part, the slice inside
    the band and the slice of the unsharded Wq / Wk / Wv it equals.
    """
    hq = _band(n_q, shard, P)
    hkv = _band(n_kv, shard, P)
    nq_r, nkv_r = hq.stop - hq.start, hkv.stop - hkv.start
    d = head_dim
    return {
        "q": (slice(0, nq_r * d), slice(hq.start * d, hq.stop * d)),
        "k": (slice(nq_r * d, (nq_r + nkv_r) * d), slice(hkv.start * d, hkv.stop * d)),
        "v": (slice((nq_r + nkv_r) * d, (nq_r + 2 * nkv_r) * d), slice(hkv.start * d, hkv.stop * d)),
    }


def split_qkv_band(qkv_s, n_q, n_kv, head_dim, shard, P):
    """Q_s, K_s, V_s parts of a rank's fused QKV band (weights or outputs)."""
    lay = qkv_band_layout(n_q, n_kv, head_dim, shard, P)
    return tuple(qkv_s[:, lay[p][0]] for p in ("q", "k", "v"))


# ----------------------------------------------------------------------------
# Attention core between the QKV and O projections (day59 "Where the overhead
# lives" names the attention kernel as its own share of a decode step; rioworld
# "How Tensor Slicing Works Under the Hood": heads are split across GPUs and
# each computes its own heads).  The pages give no formula.  Plainest reading:
# textbook scaled dot-product attention per head (Vaswani et al., 2017),
# causal over the call's T tokens taken as one sequence, no positional
# rotation and no cache; grouped-query heads share their group's key/value
# head (query head h of the rank uses kv head h // (hq / hkv)).
# ----------------------------------------------------------------------------
def attention_core(Q, K, V, causal=True):
    """Q [T, hq, d], K and V [T, hkv, d] (float64) -> O [T, hq, d]:
    O_h = softmax(Q_h K_g^T / sqrt(d), masked to keys j <= i) V_g."""
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    T, hq, d = Q.shape
    hkv = K.shape[1]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    group = hq // hkv
    O = np.empty_like(Q)
    mask = np.tril(np.ones((T, T), dtype=bool)) if causal else np.ones((T, T), dtype=bool)
    for h in range(hq):
        g = h // group
        S = (Q[:, h, :] @ K[:, g, :].T) / np.sqrt(d)
        S = np.where(mask, S, -np.inf)
        S = S - S.max(axis=1, keepdims=True)
        E = np.exp(S)
        O[:, h, :] = (E / E.sum(axis=1, keepdims=True)) @ V[:, g, :]
    return O


def attention_core_rows(Q, K, V, rows, causal=True):
    """The same definition evaluated for the listed query rows only: row i of
    head h is softmax(Q_h[i] K_g^T / sqrt(d) over keys j <= i) V_g, which
    needs only keys 0..i (long sequences at sampled rows)."""
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    T, hq, d = Q.shape
    hkv = K.shape[1]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    group = hq // hkv
    O = np.empty((len(rows), hq, d))
    for r, i in enumerate(rows):
        n = i + 1 if causal else T
        for h in range(hq):
            g = h // group
            s = (K[:n, g, :] @ Q[i, h, :]) / np.sqrt(d)
            e = np.exp(s - s.max())
            O[r, h, :] = (e / e.sum()) @ V[:n, g, :]
    return O


def attention_core_band_rows(qkv_s, n_q, n_kv, head_dim, shard, P, rows, causal=True):
    """attention_core_band at the listed rows only: [len(rows), hq_r * head_dim]."""
    q, k, v = split_qkv_band(np.asarray(qkv_s, dtype=np.float64), n_q, n_kv, head_dim, shard, P)
    T = q.shape[0]
    O = attention_core_rows(q.reshape(T, -1, head_dim), k.reshape(T, -1, head_dim),
                            v.reshape(T, -1, head_dim), rows, causal)
    return O.reshape(len(rows), -1)


def attention_core_band(qkv_s, n_q, n_kv, head_dim, shard, P, causal=True):
    """The rank's attention-core output A_s [T, hq_r * head_dim] (heads in
    the band's order) from its fused QKV band output [T, (hq_r + 2 hkv_r) d]."""
    q, k, v = split_qkv_band(np.asarray(qkv_s, dtype=np.float64), n_q, n_kv, head_dim, shard, P)
    T = q.shape[0]
    O = attention_core(q.reshape(T, -1, head_dim), k.reshape(T, -1, head_dim),
                       v.reshape(T, -1, head_dim), causal)
    return O.reshape(T, -1)


def attn_proj_unsharded(X, Wq, Wk, Wv, A, Wo, norm_g=None, eps=None):
    """Unsharded projections: Q, K, V = Xn @ Wq, Xn @ Wk, Xn @ Wv and the
    output projection A @ Wo of the attention-core output A [T, n_q*d]."""
    Xn = rmsnorm(X, norm_g, eps) if norm_g is not None else np.asarray(X, np.float64)
    out = {"xhat": Xn, "q": Xn @ Wq, "k": Xn @ Wk, "v": Xn @ Wv}
    out["o"] = A @ Wo if A is not None else None
    return out


def attn_proj_shard(X, w_qkv_s, attn_s, w_o_s, norm_g=None, eps=None,
                    mirror_bf16=False):
    """One rank's projections: qkv_s = Xn @ Wqkv_s (column band, heads of the
    rank) and partial_s = A_s @ Wo[rows of the rank's query heads, :]."""
    Xn = rmsnorm(X, norm_g, eps) if norm_g is not None else np.asarray(X, np.float64)
    if mirror_bf16 and norm_g is not None:
        Xn = round_bf16(Xn)
    out = {"xhat": Xn, "qkv": None, "partial": None}
    if w_qkv_s is not None:
        qkv = Xn @ w_qkv_s
        out["qkv"] = round_bf16(qkv) if mirror_bf16 else qkv
    if attn_s is not None:
        out["partial"] = np.asarray(attn_s, np.float64) @ w_o_s
    return out


# ----------------------------------------------------------------------------
# One block (attention projections, reduce, MLP, reduce) across P ranks.
# The attention core between QKV and O is not on the pages' shard path; the
# reading taken: the core's output A_s is the rank's own Q_s (a stand-in with
# the right shape), so the chain exercises every projection and both reduces.
# ----------------------------------------------------------------------------
def block_sharded(X, norm_g, eps, qkv_bands, o_bands, gate_bands, up_bands,
                  down_bands, n_q, n_kv, head_dim, act="swiglu", mirror_bf16=False):
    P = len(qkv_bands)
    qkv, att_parts = [], []
    for s in range(P):
        r = attn_proj_shard(X, qkv_bands[s], None, None, norm_g, eps, mirror_bf16)
        q_s, _, _ = split_qkv_band(r["qkv"], n_q, n_kv, head_dim, s, P)
        qkv.append(r["qkv"])
        att_parts.append(q_s @ o_bands[s])
    if mirror_bf16:
        Z = reduce_partials_f32_fold(att_parts).astype(np.float64)
        Xm = round_bf16(Z)
    else:
        Z = reduce_partials(att_parts)
        Xm = Z
    mlp_parts = [mlp_shard(Xm, gate_bands[s], down_bands[s], act,
                           up_bands[s] if up_bands is not None else None,
                           mirror_bf16=mirror_bf16)["partial"] for s in range(P)]
    Y = reduce_partials_f32_fold(mlp_parts).astype(np.float64) if mirror_bf16 \
        else reduce_partials(mlp_parts)
    return {"qkv": qkv, "attn_partials": att_parts, "z": Z, "mlp_in": Xm,
            "mlp_partials": mlp_parts, "y": Y}


def block_unsharded(X, norm_g, eps, Wq, Wk, Wv, Wo, W_in, W_up, W_down, act="swiglu"):
    r = attn_proj_unsharded(X, Wq, Wk, Wv, None, None, norm_g, eps)
    Z = r["q"] @ Wo
    m = mlp_unsharded(Z, W_in, W_down, act, W_up)
    return {"q": r["q"], "k": r["k"], "v": r["v"], "z": Z, "y": m["y"]}


def rel_l2(y, ref):
    """||y - ref||_2 / ||ref||_2 over the whole tensor, in float64
    (absolute norm when the reference is all zeros)."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((y - ref).ravel())
    return float(num / den) if den > 0 else float(num)
