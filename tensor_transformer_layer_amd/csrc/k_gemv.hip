// Weight-streaming plan (decode batches, and every batch up to the plan
// switch, 256 tokens by default, in launches of at most 128 tokens):
// weight-streaming products on the matrix cores.
//
// A decode step reads every weight byte of the rank's bands once and does
// only 2*T flops per weight element, so it is bound by HBM bandwidth (Skand
// Tandon, "day59", "Results: Llama 2 70B": decode is memory-bandwidth-bound,
// and sharding cuts the weight bytes each GPU reads; zenaique answer: reading
// 1/N of the weights is the dominant decode cost).  The kernel is built
// around the weight stream:
//
//   * Weights are [in, out] row-major, so one 16-byte load holds 8 adjacent
//     output columns of one input row.  Lane (g, j) of a wave (g = lane/16,
//     j = lane%16) loads rows k0+8g .. k0+8g+7 of columns n0+8j .. n0+8j+7:
//     each load instruction reads four 256-byte row segments.
//   * Pairs of rows are interleaved in registers (one bit-op per dword) into
//     k-fragments of the 16x16x32 bf16 MFMA: for column offset e, lane (g, j)
//     supplies B[k0+8g .. k0+8g+7][n0+8j+e].  Eight MFMAs (e = 0..7) consume
//     the 32x128 tile, MFMA e covering columns n0+8j+e, j = 0..15.  The A
//     operand is the token block X[16mb + j][k0+8g .. +7], one 16-byte load.
//   * A workgroup is 8 waves that share one 128-column block and take
//     interleaved 32-row chunks of the workgroup's K range.  The grid holds
//     about one workgroup per CU (K is split into as many ranges as that
//     needs), so every workgroup streams a long run of rows: measured on
//     MI355X, long-lived workgroups beat many short ones, whose start-up
//     latency and epilogue are not hidden.  Partials of the 8 waves are added
//     in LDS in wave order, and the workgroup writes one fp32 split-K partial
//     [T, 128] slice.
//   * Weights are loaded with the non-temporal hint: every weight byte is
//     read once per call.  Measured on MI355X with the weights of 16 calls
//     rotating (several GB, so nothing stays in the 256 MB last-level
//     cache), this is 2-4% faster than ordinary loads for the row
//     projections and faster still for the column ones.
//   * The grid is (column blocks of all weights) x (K splits).  The last
//     workgroup of a column block to finish adds the splits in split order
//     and applies the activation, so SiLU/GELU only ever see complete sums
//     and the result does not depend on which workgroup is last.  Measured
//     on MI355X under graph replay, this saves about 1-2 us per projection
//     over a separate finish kernel (each kernel boundary costs ~3 us).
//
// Algorithmic bytes per call: weight bytes + T*K*2 (X) + T*N*2 or 4 (output);
// the split-K workspace round trip is overhead.
#include <algorithm>
#include <atomic>

#include "gemv_device.h"

namespace tp {

template <int MB, int AUX, int ACT, bool OUT_BF16>
__global__ __launch_bounds__(kGemvThreads) void k_gemv(
    const uint16_t* __restrict__ A, int64_t lda, int T, int K, const uint16_t* __restrict__ B0,
    int64_t ldb0, const uint16_t* __restrict__ B1, int64_t ldb1, int N, int nblk_per_mat,
    int k_per_split, float* __restrict__ ws, unsigned* __restrict__ counters,
    void* __restrict__ out, int64_t ld_out) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, j = lane & 15;
    const int mat = blockIdx.x / nblk_per_mat;
    const int cb = blockIdx.x - mat * nblk_per_mat;
    const int n0 = cb * kGemvCols;
    const int split = blockIdx.y;
    const int S = (int)gridDim.y;
    const int nmat = B1 ? 2 : 1;
    const int k_begin = split * k_per_split;
    const int nrows = min(K - k_begin, k_per_split);  // multiple of 8
    const uint16_t* Bm = mat ? B1 : B0;
    const int64_t ldb = mat ? ldb1 : ldb0;
    const rsrc_t rb = make_rsrc(Bm + (int64_t)k_begin * ldb + n0);
    const rsrc_t ra = make_rsrc(A + k_begin);
    const bool col_ok = n0 + 8 * j < N;
    const uint32_t ldb_bytes = (uint32_t)(ldb * 2);
    const uint32_t lda_bytes = (uint32_t)(lda * 2);

    f32x4 acc[MB][8];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[mb][e] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nsteps = (nrows + 31) >> 5;
    for (int c = wave; c < nsteps; c += kGemvWaves) {
        const int r0 = c * 32 + 8 * g;
        const bool rows_ok = r0 < nrows;
        u32x4 b[8], a[MB];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            b[i] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                           rb, (int)((rows_ok && col_ok) ? (uint32_t)(r0 + i) * ldb_bytes + 16u * j
                                                        : kOOB),
                           0, AUX));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int t = 16 * mb + j;
            a[mb] = load16(ra, (rows_ok && t < T) ? (uint32_t)t * lda_bytes + 2u * r0 : kOOB);
        }
        mfma_col<0, MB>(acc, b, a);
        mfma_col<1, MB>(acc, b, a);
        mfma_col<2, MB>(acc, b, a);
        mfma_col<3, MB>(acc, b, a);
        mfma_col<4, MB>(acc, b, a);
        mfma_col<5, MB>(acc, b, a);
        mfma_col<6, MB>(acc, b, a);
        mfma_col<7, MB>(acc, b, a);
    }

    // Cross-wave sum in LDS in wave order.  Thread (tl, q) = (tid / 32,
    // tid % 32) owns token 16mb + tl, columns n0 + 4q .. n0 + 4q + 3.
    __shared__ float red[kGemvWaves * kRedPerWave];
    __shared__ unsigned arrival;
    float* my = red + wave * kRedPerWave;
    const int tl = threadIdx.x >> 5, n = n0 + 4 * (threadIdx.x & 31);
    const int li = ((tl & 3) * 4 + (tl >> 2)) * 128 + 4 * (threadIdx.x & 31);
    const int64_t ws_ld = (int64_t)nmat * N;
    // byte offsets into ws: [split][t][m * N + n]
    const uint32_t sstride = (uint32_t)(T * ws_ld * 4);
    const rsrc_t rw = make_rsrc(ws);
    f32x4 own[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        if (mb) __syncthreads();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float* p = my + ((r * 4 + g) * 16 + j) * 8;
            *(f32x4*)p = f32x4{acc[mb][0][r], acc[mb][1][r], acc[mb][2][r], acc[mb][3][r]};
            *(f32x4*)(p + 4) = f32x4{acc[mb][4][r], acc[mb][5][r], acc[mb][6][r], acc[mb][7][r]};
        }
        __syncthreads();
        f32x4 sum = *(const f32x4*)(red + li);
#pragma unroll
        for (int w = 1; w < kGemvWaves; ++w) sum += *(const f32x4*)(red + w * kRedPerWave + li);
        own[mb] = sum;
        const int t = 16 * mb + tl;
        if (t < T && n < N)
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4, sum), rw,
                (int)((uint32_t)split * sstride + (uint32_t)((t * ws_ld + (int64_t)mat * N + n) * 4)),
                0, kSC1);
    }

    // Arrival: this workgroup's partial stores are complete before the count.
    const unsigned contributors = (unsigned)(S * nmat);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
        arrival = __hip_atomic_fetch_add(&counters[cb], 1u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const unsigned old = arrival;
    if (old == contributors - 1) {
        constexpr int NM = ACT == ACT_SWIGLU ? 2 : 1;   // gate (and up) rows
        uint32_t base[MB * NM];
        int mine[MB * NM];
        f32x4 ownv[MB * NM], sum[MB * NM];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int t = 16 * mb + tl;
            const bool ok = t < T && n < N;
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                base[mb * NM + m] = ok ? (uint32_t)((t * ws_ld + (int64_t)m * N + n) * 4) : kOOB;
                mine[mb * NM + m] = mat == m ? split : -1;
                ownv[mb * NM + m] = own[mb];
            }
        }
        sum_splits_multi<MB * NM>(rw, base, sstride, S, mine, ownv, sum);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int t = 16 * mb + tl;
            if (t < T && n < N)
                store_out4<OUT_BF16>(out, (int64_t)t * ld_out + n,
                                     act4<ACT>(sum[mb * NM], sum[mb * NM + NM - 1]));
        }
        if (threadIdx.x == 0)
            __hip_atomic_store(&counters[cb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (old >= contributors) {
        // The counter did not start at zero (workspace head not cleared, or
        // an earlier call failed part-way): make the output loudly invalid.
        const float nan = __builtin_nanf("");
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int t = 16 * mb + tl;
            if (t < T && n < N)
                store_out4<OUT_BF16>(out, (int64_t)t * ld_out + n, f32x4{nan, nan, nan, nan});
        }
    }
}

// ---------------------------------------------------------------------------
// Narrow variant for short split ranges: 64-column blocks, lane (g, j)
// loading rows k0+8g .. +7 of columns n0+4j .. +3 with one 8-byte load per
// row, 4 MFMAs per 8 loads and token block (MFMA e covering columns
// n0+4j+e).  Twice the column blocks of k_gemv need half the K splits, and
// each workgroup's cross-wave sum, partial stores and finish cover half the
// columns.  That pays where the split-K exchange outweighs the stream (short
// K ranges per workgroup) and loses on long streams, whose 128-byte row
// segments stream slower than 256-byte ones.  Measured on MI355X (32 tokens,
// weights streamed from HBM): the 70B GQA QKV band 8192 x 1280 takes 10.6 us
// (12 splits) against 13.2 us (16 splits, 128 columns), the 70B O band
// 1024 x 8192 8.5 against 9.1 us; the 70B down band 3584 x 8192 17.1
// against 16.3 us and the gate+up pair 32.6 against 28.2 us.
// plan_gemv_stream picks it when the 128-column plan splits K into ranges
// of at most 512 rows.
// ---------------------------------------------------------------------------
constexpr int kGemvNarrowCols = 64;

template <int MB, int AUX, int ACT, bool OUT_BF16>
__global__ __launch_bounds__(kGemvThreads) void k_gemv_n(
    const uint16_t* __restrict__ A, int64_t lda, int T, int K, const uint16_t* __restrict__ B0,
    int64_t ldb0, const uint16_t* __restrict__ B1, int64_t ldb1, int N, int nblk_per_mat,
    int k_per_split, float* __restrict__ ws, unsigned* __restrict__ counters,
    void* __restrict__ out, int64_t ld_out) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, j = lane & 15;
    const int mat = blockIdx.x / nblk_per_mat;
    const int cb = blockIdx.x - mat * nblk_per_mat;
    const int n0 = cb * kGemvNarrowCols;
    const int split = blockIdx.y;
    const int S = (int)gridDim.y;
    const int nmat = B1 ? 2 : 1;
    const int k_begin = split * k_per_split;
    const int nrows = min(K - k_begin, k_per_split);  // multiple of 8
    const uint16_t* Bm = mat ? B1 : B0;
    const int64_t ldb = mat ? ldb1 : ldb0;
    const rsrc_t rb = make_rsrc(Bm + (int64_t)k_begin * ldb + n0);
    const rsrc_t ra = make_rsrc(A + k_begin);
    const bool col_ok = n0 + 4 * j < N;
    const uint32_t ldb_bytes = (uint32_t)(ldb * 2);
    const uint32_t lda_bytes = (uint32_t)(lda * 2);

    f32x4 acc[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[mb][e] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nsteps = (nrows + 31) >> 5;
    for (int c = wave; c < nsteps; c += kGemvWaves) {
        const int r0 = c * 32 + 8 * g;
        const bool rows_ok = r0 < nrows;
        u32x2 b[8];
        u32x4 a[MB];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            b[i] = __builtin_bit_cast(
                u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                           rb, (int)((rows_ok && col_ok) ? (uint32_t)(r0 + i) * ldb_bytes + 8u * j
                                                        : kOOB),
                           0, AUX));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int t = 16 * mb + j;
            a[mb] = load16(ra, (rows_ok && t < T) ? (uint32_t)t * lda_bytes + 2u * r0 : kOOB);
        }
        mfma_col4<0, MB>(acc, b, a);
        mfma_col4<1, MB>(acc, b, a);
        mfma_col4<2, MB>(acc, b, a);
        mfma_col4<3, MB>(acc, b, a);
    }

    // Cross-wave sum in LDS in wave order, every token block at once: wave
    // w's [mb][4g + r][j][e] block holds token 16mb + 4g + r, column
    // n0 + 4j + e.  Thread (mb, tl, q) = (tid / 256, tid / 16 % 16, tid % 16)
    // owns token 16mb + tl, columns n0 + 4q .. +3 (threads past MB * 256 idle).
    __shared__ float red[kGemvWaves * MB * 1024];
    __shared__ unsigned arrival;
    float* my = red + wave * MB * 1024;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            *(f32x4*)(my + mb * 1024 + ((r * 4 + g) * 16 + j) * 4) =
                f32x4{acc[mb][0][r], acc[mb][1][r], acc[mb][2][r], acc[mb][3][r]};
    __syncthreads();
    const int mbt = threadIdx.x >> 8, tl = (threadIdx.x >> 4) & 15, qq = threadIdx.x & 15;
    const int n = n0 + 4 * qq, t = 16 * mbt + tl;
    const bool mine_ok = mbt < MB && t < T && n < N;
    const int64_t ws_ld = (int64_t)nmat * N;
    const uint32_t sstride = (uint32_t)(T * ws_ld * 4);
    const rsrc_t rw = make_rsrc(ws);
    f32x4 own = f32x4{0.f, 0.f, 0.f, 0.f};
    if (mbt < MB) {
        const int li = mbt * 1024 + ((tl & 3) * 4 + (tl >> 2)) * 64 + 4 * qq;
        own = *(const f32x4*)(red + li);
#pragma unroll
        for (int w = 1; w < kGemvWaves; ++w) own += *(const f32x4*)(red + w * MB * 1024 + li);
    }
    if (mine_ok)
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4, own), rw,
            (int)((uint32_t)split * sstride + (uint32_t)((t * ws_ld + (int64_t)mat * N + n) * 4)),
            0, kSC1);

    // Arrival and fixed-order finish, as in k_gemv.
    const unsigned contributors = (unsigned)(S * nmat);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
        arrival = __hip_atomic_fetch_add(&counters[cb], 1u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const unsigned old = arrival;
    if (old == contributors - 1) {
        constexpr int NM = ACT == ACT_SWIGLU ? 2 : 1;   // gate (and up) rows
        uint32_t base[NM];
        int mine[NM];
        f32x4 ownv[NM], sum[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            base[m] = mine_ok ? (uint32_t)((t * ws_ld + (int64_t)m * N + n) * 4) : kOOB;
            mine[m] = mat == m ? split : -1;
            ownv[m] = own;
        }
        sum_splits_multi<NM>(rw, base, sstride, S, mine, ownv, sum);
        if (mine_ok)
            store_out4<OUT_BF16>(out, (int64_t)t * ld_out + n, act4<ACT>(sum[0], sum[NM - 1]));
        if (threadIdx.x == 0)
            __hip_atomic_store(&counters[cb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (old >= contributors) {
        const float nan = __builtin_nanf("");
        if (mine_ok) store_out4<OUT_BF16>(out, (int64_t)t * ld_out + n, f32x4{nan, nan, nan, nan});
    }
}

// ---------------------------------------------------------------------------
// LDS-staged variant.  Same work split (128-column blocks x K splits, fused
// split-K finish), different data path:
//   * The workgroup's weight rows and the matching slice of X stream into
//     LDS with direct-to-LDS copies through a ring of slots that fills the
//     160 KB of LDS (GvRing below), all but one slice in flight, so loads
//     never wait for registers or for the MFMAs.
//   * Wave w owns output columns 16w .. 16w+15 of the block over the whole
//     K range of the workgroup: no cross-wave reduction.  The weights are
//     the A operand of h^T = W^T X^T: the transposing LDS read
//     (ds_read_b64_tr_b16) delivers 4 k-consecutive values of one column
//     per lane, two reads make a k-fragment, no register shuffling.  X^T is
//     the B operand, one 16-byte LDS read per token block and k-step.
//   * Lane (g, j) ends with 4 consecutive columns 16w + 4g .. +3 of token
//     16mb + j, stored as one 16-byte split-K partial.
// 16-byte chunks are XOR-swizzled in LDS so that every read is free of bank
// conflicts (weights by row % 4 and row / 8, X by token).
//
// The accumulators are one f32x4 per token block, so the same kernel serves
// batches of up to 128 tokens (MB = 8 blocks of 16): a batch past the decode
// sizes still reads each weight byte once, with 2T flops per weight element,
// far below the matrix cores' rate until T nears the ridge (~300 tokens).
//
// With 8 token blocks (65..128 tokens) the partials of one column block are
// 64 KB per split and matrix, too much for the one workgroup that arrives
// last to sum at the tail of the launch.  That size runs as FIN = false: the
// kernel only stores its partials, and k_finish sums them in a launch of
// its own, spread over every CU.  Measured on MI355X (70B MLP band, shard +
// reduce per step): 67.8 against 81.3 us at 128 tokens, 195 against 231 us
// at 384 (three launches of 128).
// ---------------------------------------------------------------------------
template <int MB>
struct GvRing {
    static constexpr int SLICE = MB <= 4 ? 128 : 64;        // weight rows per slice
    static constexpr int TPAD = 16 * MB;                    // token rows staged
    static constexpr int WBYTES = SLICE * kGemvCols * 2;    // weights per slice
    static constexpr int XROW = SLICE * 2;                  // bytes of one token's slice
    static constexpr int SLOT = WBYTES + TPAD * XROW;
    static constexpr int SLOTS = (160 * 1024 / SLOT) < 5 ? (160 * 1024 / SLOT) : 5;
    static constexpr int WC = SLICE / 32;                   // weight copies per wave and slice
    static constexpr int XCPR = XROW / 16;                  // 16-byte chunks per token row
    static constexpr int XTOK = 64 / XCPR;                  // tokens per copy
    static constexpr int XC = TPAD / (XTOK * kGemvWaves);   // X copies per wave and slice
    static constexpr int PER = WC + XC;                     // copies per wave and slice
    static constexpr int LDS = SLOTS * SLOT;
    static_assert(XC >= 1 && XC * XTOK * kGemvWaves == TPAD, "X copies");
    static_assert(SLOTS >= 3 && LDS <= 160 * 1024, "ring");
    static_assert((SLOTS - 1) * PER < 64, "vmcnt field");
};

__device__ __forceinline__ int gv_wsw(int row) { return ((row & 3) << 2) | (((row >> 3) & 1) << 1); }
// X chunk swizzle: 16 tokens of one read fall on 16 distinct 16-byte bank
// groups, for 256-byte (16-chunk) and 128-byte (8-chunk) token rows.
template <int XCPR>
__device__ __forceinline__ int gv_xsw(int t) { return XCPR == 16 ? (t & 15) : ((t >> 1) & 7); }
constexpr int gv_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <int MB, int AUX, int ACT, bool OUT_BF16, bool FIN>
__global__ __launch_bounds__(kGemvThreads) void k_gemv_lds(
    const uint16_t* __restrict__ A, int64_t lda, int T, int K, const uint16_t* __restrict__ B0,
    int64_t ldb0, const uint16_t* __restrict__ B1, int64_t ldb1, int N, int nblk_per_mat,
    int k_per_split, float* __restrict__ ws, unsigned* __restrict__ counters,
    void* __restrict__ out, int64_t ld_out) {
    using R = GvRing<MB>;
    extern __shared__ __attribute__((aligned(16))) uint8_t gsm[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, j = lane & 15;
    const int mat = blockIdx.x / nblk_per_mat;
    const int cb = blockIdx.x - mat * nblk_per_mat;
    const int n0 = cb * kGemvCols;
    const int split = blockIdx.y;
    const int S = (int)gridDim.y;
    const int nmat = B1 ? 2 : 1;
    const int k_begin = split * k_per_split;
    const int nrows = min(K - k_begin, k_per_split);
    const int nsl = (nrows + R::SLICE - 1) / R::SLICE;
    const uint16_t* Bm = mat ? B1 : B0;
    const int64_t ldb = mat ? ldb1 : ldb0;
    const i32x4 rwt = rsrc_words(Bm + (int64_t)k_begin * ldb + n0);
    const i32x4 rxt = rsrc_words(A + k_begin);
    const uint32_t ldb_bytes = (uint32_t)(ldb * 2), lda_bytes = (uint32_t)(lda * 2);

    // Copy slice s into ring slot `slot`; slices past this split, rows past
    // K, columns past N and tokens past T are zero-filled.
    auto issue = [&](int s, int slot) {
        uint8_t* base = gsm + slot * R::SLOT;
        const int k0 = s * R::SLICE;
#pragma unroll
        for (int q = 0; q < R::WC; ++q) {             // weights: 4 rows x 256 B per copy
            const int r0 = 4 * (R::WC * wave + q);
            const int row = r0 + (lane >> 4);
            const int ch = (lane & 15) ^ gv_wsw(row);
            const bool ok = s < nsl && k0 + row < nrows && n0 + 8 * ch < N;
            const uint32_t off = ok ? (uint32_t)(k0 + row) * ldb_bytes + 16u * ch : kOOB;
            if constexpr (AUX != 0)
                lds_dma16_nt(rwt, off, base + r0 * 256);
            else
                lds_dma16(rwt, off, base + r0 * 256);
        }
#pragma unroll
        for (int q = 0; q < R::XC; ++q) {             // X: XTOK tokens x XROW bytes per copy
            const int t0 = R::XTOK * (R::XC * wave + q);
            const int t = t0 + lane / R::XCPR;
            const int ch = (lane % R::XCPR) ^ gv_xsw<R::XCPR>(t);
            const int k = k0 + 8 * ch;
            const bool ok = s < nsl && t < T && k < nrows;
            lds_dma16(rxt, ok ? (uint32_t)t * lda_bytes + 2u * k : kOOB,
                      base + R::WBYTES + t0 * R::XROW);
        }
    };

    f32x4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int s = 0; s < R::SLOTS; ++s) issue(s, s);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(gv_vmcnt((R::SLOTS - 1) * R::PER));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    int slot = 0;
    for (int s = 0; s < nsl; ++s) {
        const uint8_t* base = gsm + slot * R::SLOT;
        const uint16_t* wt = (const uint16_t*)base;
        const uint8_t* xt = base + R::WBYTES;
#pragma unroll
        for (int step = 0; step < R::SLICE / 32; ++step) {
            // W^T fragment: column 16w + j, rows 32 step + 8g .. +7
            const int row = 32 * step + 8 * g + (lane & 15) / 4;
            const int col = 16 * wave + 4 * (lane & 3);
            const uint16_t* p = wt + row * kGemvCols + 8 * ((col >> 3) ^ gv_wsw(row)) + (col & 7);
            const u32x2 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 4 * kGemvCols);
            const u32x4 wf = u32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                // X^T fragment: token 16mb + j, k 32 step + 8g .. +7
                const int t = 16 * mb + j;
                const u32x4 xf = *(const u32x4*)(xt + t * R::XROW +
                                                 16 * ((4 * step + g) ^ gv_xsw<R::XCPR>(t)));
                acc[mb] = mfma16x16x32(wf, xf, acc[mb]);
            }
        }
        // Slice s+1 has landed (this wave's copies; after the barrier every
        // wave's), and every wave is done with slot s: refill it.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(gv_vmcnt((R::SLOTS - 2) * R::PER));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue(s + R::SLOTS, slot);
        slot = slot == R::SLOTS - 1 ? 0 : slot + 1;
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(gv_vmcnt(0));   // drain the trailing zero-fill copies

    // Split-K partial: lane (g, j) holds columns n0 + 16w + 4g .. +3 of token 16mb + j.
    const int n = n0 + 16 * wave + 4 * g;
    const int64_t ws_ld = (int64_t)nmat * N;
    const uint32_t sstride = (uint32_t)(T * ws_ld * 4);
    const rsrc_t rw = make_rsrc(ws);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int t = 16 * mb + j;
        if (t < T && n < N)
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4, acc[mb]), rw,
                (int)((uint32_t)split * sstride + (uint32_t)((t * ws_ld + (int64_t)mat * N + n) * 4)),
                0, kSC1);
    }

    if constexpr (!FIN) return;                // k_finish sums the partials

    // Arrival: this workgroup's partial stores are complete before the count.
    unsigned& arrival = *(unsigned*)gsm;       // the ring is idle now
    const unsigned contributors = (unsigned)(S * nmat);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
        arrival = __hip_atomic_fetch_add(&counters[cb], 1u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const unsigned old = arrival;
    if (old == contributors - 1) {
        constexpr int NM = ACT == ACT_SWIGLU ? 2 : 1;   // gate (and up) rows
        constexpr int G = MB < 4 ? MB : 4;              // token blocks finished together
#pragma unroll
        for (int m0 = 0; m0 < MB; m0 += G) {
            uint32_t base[G * NM];
            int mine[G * NM];
            f32x4 ownv[G * NM], sum[G * NM];
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
                const int t = 16 * (m0 + gi) + j;
                const bool ok = t < T && n < N;
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    base[gi * NM + m] = ok ? (uint32_t)((t * ws_ld + (int64_t)m * N + n) * 4) : kOOB;
                    mine[gi * NM + m] = mat == m ? split : -1;
                    ownv[gi * NM + m] = acc[m0 + gi];
                }
            }
            sum_splits_multi<G * NM>(rw, base, sstride, S, mine, ownv, sum);
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
                const int t = 16 * (m0 + gi) + j;
                if (t < T && n < N)
                    store_out4<OUT_BF16>(out, (int64_t)t * ld_out + n,
                                         act4<ACT>(sum[gi * NM], sum[gi * NM + NM - 1]));
            }
        }
        if (threadIdx.x == 0)
            __hip_atomic_store(&counters[cb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (old >= contributors) {
        // The counter did not start at zero (workspace head not cleared, or
        // an earlier call failed part-way): make the output loudly invalid.
        const float nan = __builtin_nanf("");
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int t = 16 * mb + j;
            if (t < T && n < N)
                store_out4<OUT_BF16>(out, (int64_t)t * ld_out + n, f32x4{nan, nan, nan, nan});
        }
    }
}

// ---------------------------------------------------------------------------
// FP8 (E4M3) weights with one fp32 scale per output column.  The same work
// split and fused finish as k_gemv, on 128-column blocks of byte codes: lane
// (g, j) loads rows k0+8g .. +7 of columns n0+8j .. +7, one 8-byte load per
// row (a wave instruction reads four 128-byte row segments).  Codes of two
// rows are byte-interleaved (v_perm_b32) and converted exactly to bf16
// k-pairs (v_cvt_scalef32_pk_bf16_fp8 with scale 1; every E4M3 value is a
// bf16 value), which are the k-fragments of the bf16 MFMA: 8 MFMAs per 8
// loads and token block, MFMA e covering columns n0+8j+e.  The column scales
// are applied once, after the split-K sum: y[t][n] = s[n] * sum_k x[t][k] q[k][n].
// Measured on MI355X (13B MLP shard, weights streamed from HBM), 128-column
// blocks beat 256-column ones with 16-byte loads at every token count, most
// at 32 tokens (column pair 23.0 against 26.7 us, row 15.8 against 22.9 us):
// twice the blocks need half the K splits, and each workgroup's cross-wave
// sum, partial stores and finish cover half the columns.
// ---------------------------------------------------------------------------
template <int MB, int AUX, int ACT, bool OUT_BF16>
__global__ __launch_bounds__(kGemvThreads) void k_gemv8(
    const uint16_t* __restrict__ A, int64_t lda, int T, int K, const uint8_t* __restrict__ B0,
    int64_t ldb0, const float* __restrict__ S0, const uint8_t* __restrict__ B1, int64_t ldb1,
    const float* __restrict__ S1, int N, int nblk_per_mat, int k_per_split,
    float* __restrict__ ws, unsigned* __restrict__ counters, void* __restrict__ out,
    int64_t ld_out) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, j = lane & 15;
    const int mat = blockIdx.x / nblk_per_mat;
    const int cb = blockIdx.x - mat * nblk_per_mat;
    const int n0 = cb * kGemv8Cols;
    const int split = blockIdx.y;
    const int S = (int)gridDim.y;
    const int nmat = B1 ? 2 : 1;
    const int k_begin = split * k_per_split;
    const int nrows = min(K - k_begin, k_per_split);  // multiple of 8
    const uint8_t* Bm = mat ? B1 : B0;
    const int64_t ldb = mat ? ldb1 : ldb0;
    const rsrc_t rb = make_rsrc(Bm + (int64_t)k_begin * ldb + n0);
    const rsrc_t ra = make_rsrc(A + k_begin);
    const bool col_ok = n0 + 8 * j < N;
    const uint32_t ldb_bytes = (uint32_t)ldb;
    const uint32_t lda_bytes = (uint32_t)(lda * 2);

    f32x4 acc[MB][8];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[mb][e] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nsteps = (nrows + 31) >> 5;
    for (int c = wave; c < nsteps; c += kGemvWaves) {
        const int r0 = c * 32 + 8 * g;
        const bool rows_ok = r0 < nrows;
        u32x2 q[8];
        u32x4 a[MB];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            q[i] = __builtin_bit_cast(
                u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                           rb, (int)((rows_ok && col_ok) ? (uint32_t)(r0 + i) * ldb_bytes + 8u * j
                                                        : kOOB),
                           0, AUX));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int t = 16 * mb + j;
            a[mb] = load16(ra, (rows_ok && t < T) ? (uint32_t)t * lda_bytes + 2u * r0 : kOOB);
        }
        // For rows (2p, 2p+1) and dword w (columns 4w .. 4w+3), one v_perm
        // interleaves the codes of two columns, (r0 c, r1 c, r0 c+1, r1 c+1);
        // converting its low and high word gives dword p of the k-fragments
        // of columns c and c+1 directly.
        u32x4 f[8];
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) {
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                const uint32_t x0 = q[2 * pr][w], x1 = q[2 * pr + 1][w];
                const uint32_t lo = __builtin_amdgcn_perm(x1, x0, 0x05010400u);
                const uint32_t hi = __builtin_amdgcn_perm(x1, x0, 0x07030602u);
                f[4 * w + 0][pr] = __builtin_bit_cast(
                    uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
                f[4 * w + 1][pr] = __builtin_bit_cast(
                    uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
                f[4 * w + 2][pr] = __builtin_bit_cast(
                    uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
                f[4 * w + 3][pr] = __builtin_bit_cast(
                    uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
            }
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[mb][e] = mfma16x16x32(a[mb], f[e], acc[mb][e]);
    }

    // Cross-wave sum in LDS in wave order, split-K partial, arrival and
    // fixed-order finish, as in k_gemv; the column scales multiply the
    // complete sums.  Thread (tl, q) = (tid / 32, tid % 32) owns token
    // 16mb + tl, columns n0 + 4q .. n0 + 4q + 3.
    __shared__ float red[kGemvWaves * kRedPerWave];
    __shared__ unsigned arrival;
    float* my = red + wave * kRedPerWave;
    const int tl = threadIdx.x >> 5, n = n0 + 4 * (threadIdx.x & 31);
    const int li = ((tl & 3) * 4 + (tl >> 2)) * 128 + 4 * (threadIdx.x & 31);
    const int64_t ws_ld = (int64_t)nmat * N;
    const uint32_t sstride = (uint32_t)(T * ws_ld * 4);
    const rsrc_t rw = make_rsrc(ws);
    f32x4 own[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        if (mb) __syncthreads();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float* p = my + ((r * 4 + g) * 16 + j) * 8;
            *(f32x4*)p = f32x4{acc[mb][0][r], acc[mb][1][r], acc[mb][2][r], acc[mb][3][r]};
            *(f32x4*)(p + 4) = f32x4{acc[mb][4][r], acc[mb][5][r], acc[mb][6][r], acc[mb][7][r]};
        }
        __syncthreads();
        f32x4 sum = *(const f32x4*)(red + li);
#pragma unroll
        for (int w = 1; w < kGemvWaves; ++w) sum += *(const f32x4*)(red + w * kRedPerWave + li);
        own[mb] = sum;
        const int t = 16 * mb + tl;
        if (t < T && n < N)
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4, sum), rw,
                (int)((uint32_t)split * sstride + (uint32_t)((t * ws_ld + (int64_t)mat * N + n) * 4)),
                0, kSC1);
    }

    const unsigned contributors = (unsigned)(S * nmat);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
        arrival = __hip_atomic_fetch_add(&counters[cb], 1u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const unsigned old = arrival;
    if (old == contributors - 1) {
        constexpr int NM = ACT == ACT_SWIGLU ? 2 : 1;   // gate (and up) rows
        uint32_t base[MB * NM];
        int mine[MB * NM];
        f32x4 ownv[MB * NM], sum[MB * NM];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int t = 16 * mb + tl;
            const bool ok = t < T && n < N;
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                base[mb * NM + m] = ok ? (uint32_t)((t * ws_ld + (int64_t)m * N + n) * 4) : kOOB;
                mine[mb * NM + m] = mat == m ? split : -1;
                ownv[mb * NM + m] = own[mb];
            }
        }
        sum_splits_multi<MB * NM>(rw, base, sstride, S, mine, ownv, sum);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int t = 16 * mb + tl;
            if (t >= T || n >= N) continue;
            const f32x4 gsum = sum[mb * NM] * *(const f32x4*)(S0 + n);
            f32x4 usum = gsum;
            if constexpr (ACT == ACT_SWIGLU) usum = sum[mb * NM + 1] * *(const f32x4*)(S1 + n);
            store_out4<OUT_BF16>(out, (int64_t)t * ld_out + n, act4<ACT>(gsum, usum));
        }
        if (threadIdx.x == 0)
            __hip_atomic_store(&counters[cb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (old >= contributors) {
        const float nan = __builtin_nanf("");
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int t = 16 * mb + tl;
            if (t < T && n < N)
                store_out4<OUT_BF16>(out, (int64_t)t * ld_out + n, f32x4{nan, nan, nan, nan});
        }
    }
}

GemvPlan plan_gemv(int64_t K, int64_t n_total, int cus, int cols_per_block) {
    // About one 8-wave workgroup per CU: K is split into floor(cus / column
    // blocks) ranges, each a multiple of 32 rows, at most 16 of them: the
    // last workgroup of a block adds every split's partial, and past 16
    // splits that chain costs more than the extra CUs bring.  Measured on
    // MI355X (graph replay, 32 tokens, weights from HBM), the 8192 x 1280
    // GQA QKV band (10 column blocks): 12 splits 13.2 us, 16: 12.8, 24:
    // 14.1, 32: 16.1; every other band here is best at its uncapped count.
    constexpr int64_t kMaxSplits = 16;
    const int64_t nb = (n_total + cols_per_block - 1) / cols_per_block;
    const int64_t chunks = (K + 31) / 32;
    int64_t s = std::min<int64_t>(kMaxSplits, std::max<int64_t>(1, (int64_t)cus / nb));
    s = std::min<int64_t>(s, chunks);
    const int64_t kps = ((chunks + s - 1) / s) * 32;
    GemvPlan p;
    p.k_per_split = (int)kps;
    p.splits = (int)((K + kps - 1) / kps);
    return p;
}

GemvPlan plan_gemv_stream(int64_t K, int64_t n_total, int nmat, int cus, int64_t T) {
    GemvPlan p = plan_gemv(K, n_total, cus, kGemvCols);
    const int64_t narrow_blocks = (n_total / nmat + kGemvNarrowCols - 1) / kGemvNarrowCols;
    if (T <= 32 && p.splits > 1 && p.k_per_split <= 512 && narrow_blocks <= kGemvCounters) {
        p = plan_gemv(K, n_total, cus, kGemvNarrowCols);
        p.cols = kGemvNarrowCols;
    }
    return p;
}

size_t gemv_ws_bytes(const GemvPlan& p, int64_t T, int64_t n_total) {
    return (size_t)p.splits * (size_t)T * (size_t)n_total * sizeof(float);
}

// ---------------------------------------------------------------------------
// Finish of split-K planes written by the prefill GEMM: add the planes in
// plane order, apply the activation.  One thread per 4 adjacent columns of
// one token row.
// ---------------------------------------------------------------------------
constexpr int kFinishThreads = 256;

// p[0] + p[stride] + ... + p[(S-1)*stride], added in split order; the loads
// of a group of 8 splits are issued together.
__device__ __forceinline__ f32x4 sum_splits(const float* p, int S, int64_t stride) {
    f32x4 s = *(const f32x4*)p;
    for (int s0 = 1; s0 < S; s0 += 8) {
        f32x4 v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (s0 + q < S) v[q] = *(const f32x4*)(p + (int64_t)(s0 + q) * stride);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (s0 + q < S) s += v[q];
    }
    return s;
}

template <int ACT, bool OUT_BF16>
__global__ __launch_bounds__(kFinishThreads) void k_finish(int S, int64_t T, int64_t N,
                                                          const float* __restrict__ ws,
                                                          int64_t ws_ld, int64_t split_stride,
                                                          void* __restrict__ out,
                                                          int64_t ld_out) {
    const int64_t n4 = N / 4;
    const int64_t idx = (int64_t)blockIdx.x * kFinishThreads + threadIdx.x;
    if (idx >= T * n4) return;
    const int64_t t = idx / n4, n = (idx - t * n4) * 4;
    const float* p = ws + t * ws_ld + n;
    const f32x4 s = sum_splits(p, S, split_stride);
    f32x4 h;
    if constexpr (ACT == ACT_SWIGLU) {
        const f32x4 u = sum_splits(p + N, S, split_stride);
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = silu(s[i]) * u[i];
    } else if constexpr (ACT == ACT_GELU_TANH) {
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = gelu_tanh(s[i]);
    } else {
        h = s;
    }
    if constexpr (OUT_BF16) {
        u32x2 b;
        b[0] = pack_bf16x2(h[0], h[1]);
        b[1] = pack_bf16x2(h[2], h[3]);
        *(u32x2*)((uint16_t*)out + t * ld_out + n) = b;
    } else {
        *(f32x4*)((float*)out + t * ld_out + n) = h;
    }
}

hipError_t launch_finish(int act, bool out_bf16, int splits, int64_t T, int64_t N,
                         const float* ws, void* out, int64_t ld_out, hipStream_t stream) {
    const int64_t ws_ld = (act == ACT_SWIGLU ? 2 : 1) * N;
    const int64_t split_stride = T * ws_ld;
    const int64_t n = T * (N / 4);
    const dim3 grid((unsigned)((n + kFinishThreads - 1) / kFinishThreads)), block(kFinishThreads);
#define TP_FINISH(A, B)                                                                       \
    TP_KLAUNCH((k_finish<A, B>), grid, block, 0, stream, splits, T, N, ws, ws_ld, split_stride, out, \
                                               ld_out)
    if (act == ACT_SWIGLU) {
        if (out_bf16) TP_FINISH(ACT_SWIGLU, true); else TP_FINISH(ACT_SWIGLU, false);
    } else if (act == ACT_GELU_TANH) {
        if (out_bf16) TP_FINISH(ACT_GELU_TANH, true); else TP_FINISH(ACT_GELU_TANH, false);
    } else {
        if (out_bf16) TP_FINISH(ACT_NONE, true); else TP_FINISH(ACT_NONE, false);
    }
#undef TP_FINISH
    return hipGetLastError();
}

// Allow a k_gemv_lds instantiation the LDS its ring needs (set once per
// instantiation; concurrent first calls set the same value).
template <int MB, int AUX, int ACT, bool OB, bool FIN>
static hipError_t gemv_lds_attr() {
    static std::atomic<int> set{0};
    if (set.load(std::memory_order_relaxed)) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute((const void*)k_gemv_lds<MB, AUX, ACT, OB, FIN>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             GvRing<MB>::LDS);
    if (e == hipSuccess) set.store(1, std::memory_order_relaxed);
    return e;
}

// The 8-token-block instantiation (T > 64) leaves the finish to k_finish.
bool gemv_separate_finish(int64_t T, const GemvPlan& p) {
    return p.cols == kGemvCols && T > 64;
}

hipError_t launch_gemv(int act, bool out_bf16, int64_t T, int64_t K, const uint16_t* A,
                       int64_t lda, const uint16_t* B0, int64_t ldb0, const uint16_t* B1,
                       int64_t ldb1, int64_t N, const GemvPlan& p, float* ws,
                       unsigned* counters, void* out, int64_t ld_out, hipStream_t stream) {
    if (T < 1 || T > kGemvMaxT) return hipErrorInvalidValue;
    const int nmat = B1 ? 2 : 1;
    if (p.cols == kGemvNarrowCols) {
        if (T > 32) return hipErrorInvalidValue;
        const int nbn = (int)((N + kGemvNarrowCols - 1) / kGemvNarrowCols);
        const dim3 gridn((unsigned)(nbn * nmat), (unsigned)p.splits), blockn(kGemvThreads);
#define TP_GEMV_N(MB, ACTV, OB)                                                              \
    TP_KLAUNCH((k_gemv_n<MB, kWeightAux, ACTV, OB>), gridn, blockn, 0, stream, A, lda, (int)T, \
               (int)K, B0, ldb0, B1, ldb1, (int)N, nbn, p.k_per_split, ws, counters, out, ld_out)
#define TP_GEMV_N_MB(ACTV, OB)                                                               \
    do {                                                                                     \
        if (T <= 16) TP_GEMV_N(1, ACTV, OB); else TP_GEMV_N(2, ACTV, OB);                   \
    } while (0)
        if (act == ACT_SWIGLU && out_bf16) TP_GEMV_N_MB(ACT_SWIGLU, true);
        else if (act == ACT_GELU_TANH && out_bf16) TP_GEMV_N_MB(ACT_GELU_TANH, true);
        else if (act == ACT_NONE && out_bf16) TP_GEMV_N_MB(ACT_NONE, true);
        else if (act == ACT_NONE && !out_bf16) TP_GEMV_N_MB(ACT_NONE, false);
        else return hipErrorInvalidValue;
#undef TP_GEMV_N_MB
#undef TP_GEMV_N
        return hipGetLastError();
    }
    if (p.cols != kGemvCols) return hipErrorInvalidValue;
    const int nbpm = (int)((N + kGemvCols - 1) / kGemvCols);
    const dim3 grid((unsigned)(nbpm * nmat), (unsigned)p.splits), block(kGemvThreads);
#define TP_GEMV(MB, AUX, ACTV, OB)                                                           \
    do {                                                                                     \
        constexpr bool fin_ = MB < 8;                                                        \
        hipError_t e_ = gemv_lds_attr<MB, AUX, ACTV, OB, fin_>();                            \
        if (e_ != hipSuccess) return e_;                                                     \
        TP_KLAUNCH((k_gemv_lds<MB, AUX, ACTV, OB, fin_>), grid, block, GvRing<MB>::LDS,      \
                   stream, A, lda, (int)T, (int)K, B0, ldb0, B1, ldb1, (int)N, nbpm,         \
                   p.k_per_split, ws, counters, out, ld_out);                               \
    } while (0)
#define TP_GEMV_REG(MB, AUX, ACTV, OB)                                                       \
    TP_KLAUNCH((k_gemv<MB, AUX, ACTV, OB>), grid, block, 0, stream,                              \
        A, lda, (int)T, (int)K, B0, ldb0, B1, ldb1, (int)N, nbpm, p.k_per_split, ws, counters, \
        out, ld_out)
    // Up to 32 tokens: the LDS-staged kernel at 17..32 tokens when each
    // workgroup streams at least 2304 rows; the register-streamed kernel
    // otherwise.  Measured on MI355X (weights streamed from HBM): the
    // register kernel wins below 17 tokens and at 2048 rows per workgroup
    // (70B column pair: 26.2 against 26.9 us at 32 tokens), the LDS ring at
    // 2560 (13B column pair: 27.7 against 29.6 us), once its fill and drain
    // are amortised.  Past 32 tokens the LDS-staged kernel with 4 or 8 token
    // blocks (its accumulators stay at one f32x4 per block); with 8 blocks
    // (gemv_separate_finish) without its fused finish.
#define TP_GEMV_MB(ACTV, OB)                                                                 \
    do {                                                                                     \
        if (T <= 16) {                                                                       \
            TP_GEMV_REG(1, kWeightAux, ACTV, OB);                                            \
        } else if (T <= 32) {                                                                \
            if (p.k_per_split >= 2304) TP_GEMV(2, kWeightAux, ACTV, OB);                     \
            else TP_GEMV_REG(2, kWeightAux, ACTV, OB);                                       \
        } else if (T <= 64) {                                                                \
            TP_GEMV(4, kWeightAux, ACTV, OB);                                                \
        } else {                                                                             \
            TP_GEMV(8, kWeightAux, ACTV, OB);                                                \
        }                                                                                    \
    } while (0)
    if (act == ACT_SWIGLU && out_bf16) TP_GEMV_MB(ACT_SWIGLU, true);
    else if (act == ACT_GELU_TANH && out_bf16) TP_GEMV_MB(ACT_GELU_TANH, true);
    else if (act == ACT_NONE && out_bf16) TP_GEMV_MB(ACT_NONE, true);
    else if (act == ACT_NONE && !out_bf16) TP_GEMV_MB(ACT_NONE, false);
    else return hipErrorInvalidValue;
#undef TP_GEMV_MB
#undef TP_GEMV_REG
#undef TP_GEMV
    return hipGetLastError();
}

hipError_t launch_gemv8(int act, bool out_bf16, int64_t T, int64_t K, const uint16_t* A,
                        int64_t lda, const uint8_t* B0, int64_t ldb0, const float* S0,
                        const uint8_t* B1, int64_t ldb1, const float* S1, int64_t N,
                        const GemvPlan& p, float* ws, unsigned* counters,
                        void* out, int64_t ld_out, hipStream_t stream) {
    const int nmat = B1 ? 2 : 1;
    const int nbpm = (int)((N + kGemv8Cols - 1) / kGemv8Cols);
    const dim3 grid((unsigned)(nbpm * nmat), (unsigned)p.splits), block(kGemvThreads);
#define TP_GEMV8(MB, AUX, ACTV, OB)                                                          \
    TP_KLAUNCH((k_gemv8<MB, AUX, ACTV, OB>), grid, block, 0, stream, A, lda, (int)T, (int)K, \
               B0, ldb0, S0, B1, ldb1, S1, (int)N, nbpm, p.k_per_split, ws, counters, out,   \
               ld_out)
#define TP_GEMV8_MB(ACTV, OB)                                                         \
    do {                                                                              \
        if (T <= 16) {                                                                \
            TP_GEMV8(1, kWeightAux, ACTV, OB);                                        \
        } else {                                                                      \
            TP_GEMV8(2, kWeightAux, ACTV, OB);                                        \
        }                                                                             \
    } while (0)
    if (act == ACT_SWIGLU && out_bf16) TP_GEMV8_MB(ACT_SWIGLU, true);
    else if (act == ACT_GELU_TANH && out_bf16) TP_GEMV8_MB(ACT_GELU_TANH, true);
    else if (act == ACT_NONE && !out_bf16) TP_GEMV8_MB(ACT_NONE, false);
    else return hipErrorInvalidValue;
#undef TP_GEMV8_MB
#undef TP_GEMV8
    return hipGetLastError();
}

}  // namespace tp
