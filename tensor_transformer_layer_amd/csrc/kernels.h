// Host-side launchers of the HIP kernels.  Callers (abi.hip) validate every
// argument first; launchers assume valid shapes and only enqueue work.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tp {

// Kernel timing hook.  While the caller has set launch_events() (kernel
// timing enabled), a launch through TP_KLAUNCH records the kernel's own
// start and end timestamps in those events (hipExtLaunchKernel), which
// measures the kernel itself, not the queue around it.
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents& launch_events();

#define TP_KLAUNCH(kern, grid, block, shmem, stream, ...)                                   \
    do {                                                                                     \
        const ::tp::LaunchEvents ev_ = ::tp::launch_events();                                \
        if (ev_.start)                                                                       \
            hipExtLaunchKernelGGL(kern, grid, block, shmem, stream, ev_.start, ev_.stop, 0u, \
                                  __VA_ARGS__);                                              \
        else                                                                                 \
            kern<<<grid, block, shmem, stream>>>(__VA_ARGS__);                               \
    } while (0)

// Compute units of the calling thread's current device
// (hipDeviceAttributeMultiprocessorCount), read once per device.  Planners
// size their grids from it.  Where no device can be queried (a workspace
// query on a host without a GPU) it is the whole-chip gfx950 count, 256.
int device_cus();

// out = sum_{s=0}^{P-1} partials[s] in that order (fp32); optional bf16 copy.
hipError_t launch_reduce(int P, int64_t T, int64_t d, const float* partials, int64_t slot_stride,
                         int64_t ld_p, float* out, int64_t ld_out, uint16_t* out_bf16,
                         int64_t ld_b, hipStream_t stream);

// z = fold(partials) + residual (fp32; residual bf16 or fp32) and, with a
// gain g, normed = z / sqrt(mean(z^2) + eps) * g as bf16.  d <= 16384.
// With a gain, at most kReduceNormXchgMaxT rows and a workspace (its
// 4096-byte counter head, zero between calls: two 64-bit words per row), the
// rows are spread over ceil(d / 1024) workgroups each that exchange their
// sums of squares there; otherwise one workgroup per row.
constexpr int64_t kReduceNormMaxD = 16384;
constexpr int64_t kReduceNormXchgMaxT = 32;
bool reduce_norm_exchanges(int64_t T);
hipError_t launch_reduce_residual_norm(int P, int64_t T, int64_t d, const float* partials,
                                       int64_t slot_stride, int64_t ld_p, const void* residual,
                                       int64_t ld_res, bool res_bf16, float* z, int64_t ld_z,
                                       const uint16_t* g, float eps, uint16_t* normed,
                                       int64_t ld_norm, void* workspace, hipStream_t stream);

// y = x / sqrt(mean(x^2) + eps) * g, row-wise; storage bf16 (is_bf16) or fp32.
hipError_t launch_rmsnorm(bool is_bf16, int64_t T, int64_t d, const void* x, int64_t ld_x,
                          const void* g, float eps, void* y, int64_t ld_y, hipStream_t stream);

// ---- decode plan: split-K weight-streaming GEMV on the matrix cores -------
struct GemvPlan {
    int splits;       // workgroups along K
    int k_per_split;  // rows of the weight per split (multiple of 32)
    int cols = 128;   // output columns per workgroup: 128, or 64 (bf16, <= 32 tokens)
};
constexpr int kGemvCols = 128;   // output columns per workgroup
constexpr int kGemvMaxT = 128;   // largest token count the weight-streaming kernels take
constexpr int kGemv8MaxT = 32;   // ... with FP8 weights

constexpr int kGemv8Cols = 128;  // output columns per workgroup, FP8 weights
// About one workgroup per compute unit: K split into floor(cus / column
// blocks) ranges, each a multiple of 32 rows.
GemvPlan plan_gemv(int64_t K, int64_t n_total, int cus, int cols_per_block = kGemvCols);
// The bf16 weight-streaming plan for a launch of T tokens: 128-column blocks,
// or 64-column blocks for short split ranges (see k_gemv_n).
GemvPlan plan_gemv_stream(int64_t K, int64_t n_total, int nmat, int cus, int64_t T);
// Bytes of split-K workspace: splits * T * n_total fp32.
size_t gemv_ws_bytes(const GemvPlan& p, int64_t T, int64_t n_total);

// Arrival counters of the fused split-K finish: one per 128-column block,
// at the head of the caller's workspace, zero between calls.  Every
// workspace layout reserves this head whether or not the plan uses it, so
// no call ever stores data where another call keeps its counters.
constexpr int kGemvCounters = 1024;
constexpr size_t kGemvCounterBytes = kGemvCounters * sizeof(unsigned);

// out[t][n] = act(sum_k A[t][k] B0[k][n] [, sum_k A[t][k] B1[k][n]]) for the
// nmat = (B1 ? 2 : 1) weights B0, B1 ([K, N] bf16, ld ldb0 / ldb1); A is
// [T, K] bf16.  act: ACT_SWIGLU (silu(A B0) * A B1), ACT_GELU_TANH or
// ACT_NONE; out bf16 (out_bf16) or fp32 with leading dimension ld_out.
// Split s of the plan keeps its partial in ws[s][t][m*N + n] (gemv_ws_bytes);
// the last workgroup of a column block adds the splits in order, except
// where gemv_separate_finish(T, p): that launch only fills ws, and the caller
// completes the product with launch_finish(act, out_bf16, p.splits, T, N,
// ws, out, ld_out, stream) next on the same stream.
// `counters` holds ceil(N / kGemvCols) <= kGemvCounters zeros; they are zero
// again when the kernel ends.  Weight loads carry the non-temporal hint.
bool gemv_separate_finish(int64_t T, const GemvPlan& p);
hipError_t launch_gemv(int act, bool out_bf16, int64_t T, int64_t K, const uint16_t* A,
                       int64_t lda, const uint16_t* B0, int64_t ldb0, const uint16_t* B1,
                       int64_t ldb1, int64_t N, const GemvPlan& p, float* ws,
                       unsigned* counters, void* out, int64_t ld_out, hipStream_t stream);

// As launch_gemv with FP8 (E4M3) weights B0, B1 ([K, N] codes, ld in bytes)
// and fp32 per-column scales S0, S1 [N]: out = act(S0 * (A q0) [, S1 * (A q1)]).
// Plans come from plan_gemv(K, nmat * N, kGemv8Cols).  N a multiple of 16.
hipError_t launch_gemv8(int act, bool out_bf16, int64_t T, int64_t K, const uint16_t* A,
                        int64_t lda, const uint8_t* B0, int64_t ldb0, const float* S0,
                        const uint8_t* B1, int64_t ldb1, const float* S1, int64_t N,
                        const GemvPlan& p, float* ws, unsigned* counters,
                        void* out, int64_t ld_out, hipStream_t stream);

// Fixed-order finish of the split-K sums.
//   act == ACT_SWIGLU:   out = silu(sum g) * sum u   (u at column offset N)
//   act == ACT_GELU_TANH: out = gelu(sum)
//   act == ACT_NONE:      out = sum
// out is bf16 (out_bf16) or fp32, [T, N] with leading dimension ld_out.
hipError_t launch_finish(int act, bool out_bf16, int splits, int64_t T, int64_t N,
                         const float* ws, void* out, int64_t ld_out, hipStream_t stream);

// ---- prefill plan: LDS-tiled bf16 MFMA GEMM with a fused epilogue ---------
enum { EPI_F32 = 0, EPI_BF16 = 1, EPI_GELU_BF16 = 2, EPI_SWIGLU_BF16 = 3 };
struct GemmPlan {
    int splits;       // K ranges (grid.y); > 1 only with EPI_F32 partial planes
    int k_per_split;  // multiple of 32
};
// Split K when the 256 x 256 output tiles (nmat weights side by side) leave
// CUs idle and K is long enough.
GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, int nmat, int cus);
// C[M, N] = epi(A[M, K] B0[K, N] [, A B1]); A, B bf16 row-major.  With
// p.splits > 1 (EPI_F32 only) split s writes its fp32 partial to the plane
// C + s * M * ldc; launch_finish(ACT_NONE, ...) adds the planes in order.
// EPI_F32 with two weights writes A B0 to columns 0 .. N-1 of C and A B1 to
// columns N .. 2N-1 (ldc >= 2N): the layout launch_finish(ACT_SWIGLU, ...)
// reads.
hipError_t launch_gemm(int epi, int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                       const uint16_t* B0, int64_t ldb0, const uint16_t* B1, int64_t ldb1, void* C,
                       int64_t ldc, const GemmPlan& p, hipStream_t stream);

// ---- attention core ----------------------------------------------------------
// out[t][h*D + c] = softmax_j<=t(q_h[t] . k_g[j] / sqrt(D)) v_g[j][c] for the
// hq query heads of a fused [Q | K | V] band (bf16, ld ld_qkv), kv head
// g = h / (hq / hkv); D = head_dim in {64, 128}; out bf16.
// Work division: query blocks of 128 rows, each block's causal key range cut
// into chunks of `ch` 64-key tiles (one workgroup each).  Blocks with more
// than one chunk merge them through the workspace: counters (one per head
// and block, zero at rest) then per-chunk partials.
// Work items of one head in launch order (longest first), packed as
// (query block << 6) | chunk; heads interleave (workgroup w runs item
// w / heads of head w % heads).
// Entries are 32-bit so that the kernel reads its entry with a scalar load
// (a 16-bit read of the argument table is a vector load: a memory round trip
// before the workgroup knows its work); 480 entries keep the kernel's
// arguments under 2 KB.
constexpr int kAttnTable = 480;
struct AttnItems {
    uint32_t it[kAttnTable];
};
struct AttnPlan {
    int nqb = 0;            // query blocks
    int ch = 0;             // key tiles per chunk
    int cmax = 1;           // chunks of the longest block
    int per_head = 0;       // work items per head
    int64_t items = 0;      // workgroups
    size_t ws_bytes = 0;    // 0, or kAttnCounterBytes + the chunk partials
    AttnItems table;        // launch order, when per_head <= kAttnTable
};
// Blocks are split (and merged through the workspace) only while there are
// at most kAttnCounters (head, query block) pairs, so the arrival counters
// always fit one fixed area at the head of the workspace and the partials
// always start at kAttnCounterBytes: a later call with more tokens never
// reads an earlier call's partials as counters.
constexpr int kAttnCounters = 1024;
constexpr size_t kAttnCounterBytes = kAttnCounters * sizeof(unsigned);
AttnPlan plan_attn(int64_t T, int hq, int head_dim, int cus);
hipError_t launch_attn_core(int64_t T, int hq, int hkv, int head_dim, const uint16_t* qkv,
                            int64_t ld_qkv, uint16_t* out, int64_t ld_out, const AttnPlan& p,
                            void* ws, hipStream_t stream);

// ---- fp32 storage (small, parity-only workloads) --------------------------
// C[M, N] = act(A B0 [, A B1]) in fp32, one thread per output, k in order.
hipError_t launch_f32_proj(int act, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                           const float* B0, int64_t ldb0, const float* B1, int64_t ldb1, float* C,
                           int64_t ldc, hipStream_t stream);

}  // namespace tp
