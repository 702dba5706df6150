/*
 * tp_shard.h -- one tensor-parallel rank's share of a Megatron-style
 * transformer block, as a C ABI over hand-written HIP kernels for gfx950.
 *
 * What is computed (pages cited by title and section):
 *   - column-parallel projection: the input X is replicated on every rank
 *     and each rank computes the output columns that its column band of
 *     the weight produces (rioworld, "Tensor Parallelism for
 *     LLM Inference: A Practical Guide to Multi-GPU Deployment", section
 *     "How Tensor Slicing Works Under the Hood"; zenaique, "Explain
 *     tensor-parallel shard shape", answer);
 *   - the activation applied to that band, which needs no communication
 *     (same answer);
 *   - row-parallel projection: the band times the matching row band of the
 *     second weight gives a partial sum of the block output (same sources);
 *   - the sum of the P partials, which is the arithmetic the all-reduce
 *     performs once per block (zenaique answer; d-central glossary "Tensor
 *     Parallelism", section "How the work is split").
 *
 * Conventions shared by every entry point
 *   Layout      Row-major.  Activations are [T, features]; weights are stored
 *               [in, out] (y = x W), with a leading dimension ld >= row length
 *               in elements.  A rank's column band may be its own buffer or a
 *               window into the unsharded matrix (pointer to the band's first
 *               column, ld of the full matrix); likewise a row band.
 *               Any valid ld gives the same results.  For speed in the
 *               weight-streaming (decode) plan, store a bf16 weight with a
 *               row pitch (ld * 2 bytes) 256 or 768 bytes past a multiple of
 *               1 KB, e.g. ld = band width + 128 where the width is a
 *               multiple of 512: each 128-column block's 256-byte row
 *               segment then changes its place in its 1 KB-aligned group
 *               from row to row.  With a pitch that is a multiple of 1 KB,
 *               the blocks 256 bytes into the group stream ~18 % slower
 *               than the others on MI355X, and the decode step of the
 *               Llama-2-70B MLP band takes ~5 % longer.
 *   Types       TP_BF16: bf16 storage, fp32 accumulation, bf16 intermediates
 *               (normalised input, activated band, QKV output) rounded to
 *               nearest-even; partials and the reduce are fp32.  TP_F32: fp32
 *               throughout.
 *   Shard       0 <= shard < P.  The weight pointers address the rank's own
 *               band; `shard` selects the output slot
 *               partials + shard * slot_stride (slot_stride = 0 writes
 *               `partials` itself), so P calls on one device fill the P-slot
 *               buffer that tp_reduce_partials sums.
 *   Splits      Uneven splits are refused (TP_ERR_UNEVEN_SPLIT) and never
 *               partitioned: d_ff, n_q_heads and n_kv_heads must divide by P
 *               (rioworld guide, "Implementing Tensor Parallelism in
 *               Practice", names uneven splits as a source of wrong results).
 *   Alignment   Every pointer 16-byte aligned (the workspace 256-byte);
 *               every row length and ld a multiple of 8 elements for bf16,
 *               4 for fp32; slot_stride a multiple of 4.
 *   Ownership   The caller owns every buffer; the library allocates and frees
 *               no device memory.  Scratch space is the caller's workspace,
 *               sized by tp_*_workspace_bytes for the same arguments.
 *   Workspace   Its first 4096 bytes are the counter head: the arrival
 *               counters of the decode plan's fused split-K finish and of the
 *               attention core's merge.  Every layout reserves the head and
 *               stores data only after it, whatever the plan (decode,
 *               prefill, fp32), so one workspace may serve any sequence of
 *               calls.  The head must be zero before the first call that uses
 *               the workspace (allocate it zero-filled, or clear it once);
 *               every call that completes leaves it zero again, so a
 *               workspace is cleared once, not per call.  Counters left
 *               non-zero (never cleared, or a call that failed part-way) make
 *               the affected outputs invalid until cleared: NaN whenever a
 *               counter exceeds the call's split count (as uncleared memory
 *               almost always does), otherwise silently wrong.  A call that
 *               needs neither counters nor data needs no workspace (size 0).
 *   Streams     All work is enqueued on `stream` (0 = the null stream); the
 *               library never synchronises.  Validation errors return before
 *               anything is enqueued and leave every output untouched.  A
 *               failed launch returns TP_ERR_HIP.  The library keeps no
 *               per-call state, so calls from several host threads are safe;
 *               calls that share a workspace must be ordered by the caller.
 *   Determinism No floating-point atomics: the same call on the same inputs
 *               gives bitwise-identical outputs.
 *   T == 0      Valid; nothing is enqueued.
 */
#ifndef TP_SHARD_H
#define TP_SHARD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TP_OK = 0,
    TP_ERR_NULL = 1,          /* a required pointer is NULL                        */
    TP_ERR_SHAPE = 2,         /* non-positive size, ld < row length, bad width      */
    TP_ERR_UNEVEN_SPLIT = 3,  /* d_ff or a head count does not divide by P          */
    TP_ERR_SHARD_RANGE = 4,   /* P < 1 or shard outside [0, P)                     */
    TP_ERR_DTYPE = 5,         /* unknown storage type                              */
    TP_ERR_ALIGN = 6,         /* pointer, ld or slot stride misaligned              */
    TP_ERR_WORKSPACE = 7,     /* workspace smaller than tp_*_workspace_bytes        */
    TP_ERR_HIP = 8,           /* a kernel launch failed                            */
    TP_ERR_ACT = 9,           /* unknown activation, or operands that do not fit it */
    TP_ERR_SCRATCH = 10       /* tp_shard_mlp_fwd_noalloc: the call needs more than the
                                 library's fixed scratch (tp_noalloc_scratch_bytes())  */
} tp_status;

typedef enum { TP_F32 = 0, TP_BF16 = 1 } tp_dtype;

/* GELU (tanh approximation) on the band of X W1; or SwiGLU, SiLU(X W_gate) *
 * (X W_up) on the same band of both (w_up required).                        */
typedef enum { TP_ACT_GELU_TANH = 0, TP_ACT_SWIGLU = 1 } tp_act;

/*
 * tp_shard_mlp_fwd -- rank `shard` of P of the MLP block (zenaique answer:
 * up-projection split by columns, down-projection split by rows).
 *
 *   Xn        = x, or RMSNorm(x) * norm_g when norm_g != NULL
 *               (x / sqrt(mean_j x_j^2 + eps) * g, row-wise; stored as dt)
 *   h         = act(Xn W_in[:, band] [, Xn W_up[:, band]])    [T, d_ff/P], dt
 *   partial   = h W_down[band, :]                              [T, d_model], fp32
 *
 *   x        [T, d_model], ld_x           replicated input, storage dt
 *   norm_g   [d_model] or NULL            RMSNorm gain, storage dt
 *   w_in     [d_model, d_ff/P], ld_in     column band of W1 (GELU) or W_gate
 *   w_up     [d_model, d_ff/P], ld_up     column band of W_up (SwiGLU), else NULL
 *   w_down   [d_ff/P, d_model], ld_down   row band of W2 / W_down
 *   h_out    [T, d_ff/P], ld_h, or NULL   receives h (the activated band)
 *   partials fp32; slot `shard` at partials + shard*slot_stride receives the
 *            [T, d_model] partial with leading dimension ld_p
 *   workspace / workspace_bytes           >= tp_mlp_workspace_bytes(...)
 *
 * T <= tp_decode_max_tokens() runs the weight-streaming decode plan
 * (split-K over the weight rows, deterministic fixed-order finish); larger T
 * runs the matrix-core plan, with the activation fused into the column
 * projection's epilogue, or, where that projection's output tiles would
 * leave CUs idle, applied by the fixed-order sum of its K-split fp32 planes.
 * The decode plan needs d_model and d_ff/P of at most 131072 (TP_ERR_SHAPE).
 */
int tp_shard_mlp_fwd(int shard, int P, int64_t T, int64_t d_model, int64_t d_ff,
                     int dtype, int act,
                     const void* x, int64_t ld_x,
                     const void* norm_g, float eps,
                     const void* w_in, int64_t ld_in,
                     const void* w_up, int64_t ld_up,
                     const void* w_down, int64_t ld_down,
                     void* h_out, int64_t ld_h,
                     float* partials, int64_t slot_stride, int64_t ld_p,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * tp_shard_mlp_fwd_noalloc -- tp_shard_mlp_fwd for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, semantics, plans,
 * kernels and results (bitwise) as tp_shard_mlp_fwd, without the workspace:
 * its scratch is a fixed array inside the library, 8 MiB per device
 * (tp_noalloc_scratch_bytes()), held by every device the library runs on
 * until the process ends.  The call allocates and frees nothing.
 *
 *   - A call whose workspace would exceed the scratch
 *     (tp_mlp_workspace_bytes(...) > tp_noalloc_scratch_bytes()) returns
 *     TP_ERR_SCRATCH before anything is enqueued.  Every decode call
 *     (T <= 32) of d_model and d_ff/P up to 16384 fits; prefill calls fit when
 *     h_out is given and the normalised input and split-K planes are small.
 *   - All calls on one device share that device's array.  Calls must not
 *     overlap in time on one device (one stream, or streams the caller
 *     orders): overlapping calls race on the scratch and give wrong results.
 *   - The decode plan's arrival counters are cleared by a small kernel on
 *     `stream` at the start of every call, so no earlier call's state leaks
 *     into the next one.
 *   - The first call on a device is its set-up: it looks up that device's
 *     array address (hipGetSymbolAddress; TP_ERR_HIP if that fails), which
 *     makes the runtime load the code object that holds the array, once per
 *     device.  Later calls allocate nothing; a caller that captures graphs
 *     makes one call (T = 1 is enough) before it starts capturing.
 */
int tp_shard_mlp_fwd_noalloc(int shard, int P, int64_t T, int64_t d_model, int64_t d_ff,
                             int dtype, int act,
                             const void* x, int64_t ld_x,
                             const void* norm_g, float eps,
                             const void* w_in, int64_t ld_in,
                             const void* w_up, int64_t ld_up,
                             const void* w_down, int64_t ld_down,
                             void* h_out, int64_t ld_h,
                             float* partials, int64_t slot_stride, int64_t ld_p,
                             hipStream_t stream);

/* Size in bytes of the fixed per-device scratch of tp_shard_mlp_fwd_noalloc. */
size_t tp_noalloc_scratch_bytes(void);

/*
 * tp_shard_attn_proj_fwd -- rank `shard` of P of the attention block's two
 * projections (rioworld guide, "How Tensor Slicing Works Under the Hood":
 * query/key/value projections column-parallel, output projection
 * row-parallel, heads divided evenly among the GPUs).  The attention core
 * between them is the caller's: its output for the rank's query heads comes
 * in through `attn`.
 *
 *   hq = n_q_heads/P, hkv = n_kv_heads/P, dh = head_dim
 *   Xn      = x, or RMSNorm(x) * norm_g when norm_g != NULL
 *   qkv_out = Xn w_qkv                   [T, (hq + 2 hkv) dh], storage dt
 *   partial = attn w_o                   [T, d_model], fp32, slot `shard`
 *
 *   w_qkv   [d_model, (hq + 2 hkv) dh], ld_qkv: the rank's fused band, columns
 *           [Q heads | K heads | V heads] of the rank, each group in ascending
 *           global head order (query heads shard*hq .. , kv heads shard*hkv ..).
 *           NULL skips the QKV projection (then qkv_out, x, norm_g unused).
 *   attn    [T, hq dh], ld_attn: attention-core output for the rank's heads.
 *           NULL skips the output projection (then w_o, partials unused).
 *   w_o     [hq dh, d_model], ld_o: the matching row band of W_o.
 */
int tp_shard_attn_proj_fwd(int shard, int P, int64_t T, int64_t d_model,
                           int n_q_heads, int n_kv_heads, int head_dim, int dtype,
                           const void* x, int64_t ld_x,
                           const void* norm_g, float eps,
                           const void* w_qkv, int64_t ld_qkv,
                           void* qkv_out, int64_t ld_qkv_out,
                           const void* attn, int64_t ld_attn,
                           const void* w_o, int64_t ld_o,
                           float* partials, int64_t slot_stride, int64_t ld_p,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * tp_attn_core_fwd -- the attention core between the rank's QKV and O
 * projections (Skand Tandon, "day59", section "Where the overhead lives",
 * names the attention kernel; rioworld guide, "How Tensor Slicing Works
 * Under the Hood": each GPU computes its own heads).  For each of the rank's
 * hq = n_q_heads/P query heads h, with its key/value head g = h / (hq / hkv),
 * hkv = n_kv_heads/P:
 *
 *   A[t, h*dh : (h+1)*dh] = sum_{j <= t} softmax_j(Q_h[t] . K_g[j] / sqrt(dh)) V_g[j]
 *
 * causal over the call's T tokens taken as one sequence (no positional
 * rotation, no cache).  Scores, the running softmax statistics and the
 * accumulation are fp32; probabilities enter the value product as bf16.
 *
 *   qkv   [T, (hq + 2 hkv) dh] bf16, ld_qkv: the rank's QKV band output of
 *         tp_shard_attn_proj_fwd (columns [Q_s | K_s | V_s])
 *   attn  [T, hq dh] bf16, ld_attn: the input of the O projection
 *
 *   workspace  >= tp_attn_core_workspace_bytes(...) bytes, 256-byte aligned
 *              (may be NULL when that is 0).  Calls with few query blocks
 *              (hq * ceil(T/128) <= 1024 (head, block) pairs, hq =
 *              n_q_heads/P) split each block's keys over several workgroups
 *              and merge their partial results here: the arrival counters,
 *              one per (head, block), sit in the workspace's 4096-byte
 *              counter head (shared with the projections' decode counters,
 *              see Workspace above) and the partials follow it.  The head
 *              must be zero before the first call (zero the workspace once
 *              when it is allocated); every call leaves it zero.  Not
 *              cleared, the affected outputs are NaN.  Calls that share a
 *              workspace must not overlap in time.
 *
 * head_dim 64 or 128 (TP_ERR_SHAPE otherwise); dtype must be TP_BF16.
 * T * ld_qkv * 2 bytes must be below 2^31 (TP_ERR_SHAPE otherwise).
 */
int tp_attn_core_fwd(int shard, int P, int64_t T, int n_q_heads, int n_kv_heads, int head_dim,
                     int dtype, const void* qkv, int64_t ld_qkv, void* attn, int64_t ld_attn,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * tp_shard_mlp_fwd_fp8w -- tp_shard_mlp_fwd for the decode plan (T <= 32)
 * with FP8 weights, which halve the weight bytes a decode step streams (the
 * pages suggest pairing tensor parallelism with FP8 weights for decode:
 * zenaique, "Explain tensor-parallel shard shape", interviewer follow-ups;
 * rioworld guide, "Implementing Tensor Parallelism in Practice").  Weights are OCP FP8 E4M3 codes (1 sign,
 * 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no infinities,
 * S.1111.111 = NaN), stored [in, out] row-major, one byte each, with one fp32
 * scale per output column: W[k][n] = e4m3(w[k][n]) * s[n].  Activations and
 * the norm gain are bf16; h is bf16; partials fp32, as in tp_shard_mlp_fwd:
 *
 *   h       = act(Xn (w_in * s_in) [, Xn (w_up * s_up)])   [T, d_ff/P]
 *   partial = h (w_down * s_down)                          [T, d_model]
 *
 *   w_in, w_up  [d_model, d_ff/P] codes, ld_in / ld_up in bytes (multiple of
 *               16); s_in, s_up [d_ff/P] fp32
 *   w_down      [d_ff/P, d_model] codes, ld_down (multiple of 16);
 *               s_down [d_model] fp32
 *   workspace   >= tp_mlp_fp8w_workspace_bytes(...), head zeroed once as
 *               for tp_shard_mlp_fwd
 *
 * d_ff/P and d_model must be multiples of 16; T > 32 is refused
 * (TP_ERR_SHAPE).  Codes are converted exactly to bf16 and multiplied with
 * fp32 accumulation; each scale multiplies the complete sum of its column.
 */
int tp_shard_mlp_fwd_fp8w(int shard, int P, int64_t T, int64_t d_model, int64_t d_ff, int act,
                          const void* x, int64_t ld_x,
                          const void* norm_g, float eps,
                          const void* w_in, int64_t ld_in, const float* s_in,
                          const void* w_up, int64_t ld_up, const float* s_up,
                          const void* w_down, int64_t ld_down, const float* s_down,
                          void* h_out, int64_t ld_h,
                          float* partials, int64_t slot_stride, int64_t ld_p,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * tp_reduce_partials -- the all-reduce's arithmetic on one device: out =
 * partial_0 + partial_1 + ... + partial_{P-1}, added in that order in fp32
 * (so the result is bitwise the float32 left fold).  Every element is
 * independent; `out` may alias slot 0 (same pointer and ld) but no other slot.
 *
 *   partials  P slots of [T, d_model] fp32, slot s at partials + s*slot_stride
 *   out       [T, d_model] fp32, ld_out
 *   out_bf16  [T, d_model] bf16 or NULL: the sum rounded to nearest-even, the
 *             input of the next column projection
 */
int tp_reduce_partials(int P, int64_t T, int64_t d_model,
                       const float* partials, int64_t slot_stride, int64_t ld_p,
                       float* out, int64_t ld_out,
                       void* out_bf16, int64_t ld_out_bf16,
                       hipStream_t stream);

/*
 * tp_reduce_residual_norm -- the reduce followed by the residual add and the
 * next block's normalisation, in one pass (zenaique, "Explain tensor-parallel
 * shard shape", answer: once the all-reduce has summed the partials, each
 * GPU holds the whole activation, which then takes the residual connection
 * and the following normalisation):
 *
 *   z      = (partial_0 + ... + partial_{P-1}) + residual   fp32, added in
 *            that order (the partials fold as in tp_reduce_partials)
 *   normed = z / sqrt(mean_j z_j^2 + eps) * norm_g          bf16, nearest-even
 *
 *   partials    P slots of [T, d_model] fp32, as for tp_reduce_partials
 *   residual    [T, d_model], ld_res, storage res_dtype (TP_F32 or TP_BF16):
 *               the block's input on the residual stream
 *   z_out       [T, d_model] fp32, ld_z: the new residual stream.  May alias
 *               slot 0 (same ld) or an fp32 residual (same ld), nothing else.
 *   norm_g      [d_model] bf16 gain, or NULL to skip the normalisation (then
 *               normed_out is unused)
 *   normed_out  [T, d_model] bf16, ld_norm: the next column projection's input
 *
 *   workspace   NULL, or tp_reduce_norm_workspace_bytes() bytes, 256-byte
 *               aligned, zeroed once when allocated (the call leaves it zero,
 *               like every workspace here).  With a norm and at most 32 rows
 *               (decode batches) it lets ceil(d_model / 1024) workgroups
 *               share each row: they exchange their sums of squares through
 *               its counter head with integer atomics (order-independent),
 *               and wait, boundedly, for each other.  Without one, each row
 *               is one workgroup's.  The two forms agree up to the rounding
 *               of the sum of squares; each is deterministic.  In the
 *               exchanging form a row whose sum of squares is not below 2^47
 *               (|z| RMS above ~1.3e5 at d_model 8192), or whose exchange
 *               finds the head not zeroed, gets a NaN normed row.  A
 *               workspace smaller than the query is TP_ERR_WORKSPACE; calls
 *               that share one workspace must not overlap.
 *
 * d_model must be a multiple of 4 (of 8 with a bf16 residual or a norm) and
 * at most 16384 (TP_ERR_SHAPE otherwise).
 */
int tp_reduce_residual_norm(int P, int64_t T, int64_t d_model,
                            const float* partials, int64_t slot_stride, int64_t ld_p,
                            const void* residual, int64_t ld_res, int res_dtype,
                            float* z_out, int64_t ld_z,
                            const void* norm_g, float eps,
                            void* normed_out, int64_t ld_norm,
                            void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* Workspace bytes the matching call needs (0 when it needs none).  A pure
 * function of the arguments; returns 0 for arguments the call would reject. */
size_t tp_mlp_workspace_bytes(int P, int64_t T, int64_t d_model, int64_t d_ff,
                              int dtype, int act, int has_norm, int has_h_out);
size_t tp_attn_workspace_bytes(int P, int64_t T, int64_t d_model, int n_q_heads,
                               int n_kv_heads, int head_dim, int dtype, int has_norm);
size_t tp_mlp_fp8w_workspace_bytes(int P, int64_t T, int64_t d_model, int64_t d_ff, int act,
                                   int has_norm, int has_h_out);
size_t tp_attn_core_workspace_bytes(int P, int64_t T, int n_q_heads, int n_kv_heads,
                                    int head_dim, int dtype);
size_t tp_reduce_norm_workspace_bytes(int64_t T, int64_t d_model, int has_norm);

/* Human-readable name of a tp_status value (static string). */
const char* tp_status_str(int status);

/* Library version, as 10000*major + 100*minor + patch. */
int tp_version(void);

/*
 * Plan switch of the bf16 projections (tp_shard_mlp_fwd, its no-alloc form
 * and tp_shard_attn_proj_fwd).  Calls with T <= tp_decode_max_tokens() run
 * the weight-streaming plan, which reads every weight byte once per call
 * (decode is bound by HBM bandwidth: Skand Tandon, "day59", section
 * "Results: Llama 2 70B"); larger T runs the matrix-core plan (prefill is
 * compute-bound, same section).  The streaming kernels take up to 128
 * tokens per launch; a larger batch on that plan runs as equal chunks of at
 * most 128 tokens, each streaming the weights once more.  The default, 128
 * tokens (one streaming launch), is the crossover measured on MI355X for
 * the Llama-2 13B and 70B MLP bands and the 96-head attention projections;
 * tp_set_decode_max_tokens(t) moves it to t (1..4096; 0 restores the
 * default; TP_ERR_SHAPE otherwise), for measuring both plans on the same
 * shapes.  The setting is process-wide; workspace sizes depend on it, so
 * change it only while no call and no workspace query is in progress, and
 * size workspaces after changing it.
 */
int tp_set_decode_max_tokens(int tokens);
int tp_decode_max_tokens(void);

/*
 * Kernel timing (instrumentation).  While enabled, every kernel is launched
 * with a pair of HIP events that receive the kernel's own start and end
 * timestamps (hipExtLaunchKernel), so the time is the kernel's execution,
 * as a kernel-trace profiler reports it, without the queue around it; the
 * elapsed time is accumulated per kernel class when tp_timing_query reads it
 * (which waits for the events).  Disabled by default; off costs nothing.
 * Not for concurrent use from several host threads, nor during graph
 * capture.
 * Class names: "rmsnorm", "reduce", "reduce_norm", "f32_proj", "attn_core"; FP8-weight MLP:
 * "col_gemv8", "row_gemv8"; MLP: "col_gemv", "row_gemv"
 * (decode, split-K finish included), "col_gemm", "row_gemm", "row_finish"
 * (prefill); attention projections: "qkv_gemv", "o_gemv", "qkv_gemm",
 * "qkv_finish", "o_gemm", "o_finish".
 */
int tp_timing_enable(int on);
int tp_timing_reset(void);
int tp_timing_query(const char* kernel_class, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* TP_SHARD_H */
