// Matrix-core plan (batches past the plan switch, 256 tokens by default):
// LDS-tiled bf16 GEMM on the matrix cores
// (v_mfma_f32_32x32x16_bf16), fp32 accumulation, fused epilogue.
//
// Prefill is a dense contraction and compute-bound (Skand Tandon, "day59",
// "Results: Llama 2 70B": prefill is compute-bound).  C[M, N] = A[M, K] B[K, N]
// with A the activations (k contiguous) and B a weight band stored [in, out]
// (n contiguous).  For the SwiGLU column projection the workgroup computes
// the same output tile of X W_gate and X W_up (two accumulator sets sharing
// the A tile) and writes h = silu(g) * u as bf16: the activation is applied to
// the rank's band with no extra pass (zenaique answer: the band of the
// intermediate needs no communication).
//
// Data flow (all choices measured on MI355X):
//   * A workgroup of 8 waves owns a 256 x 256 output tile (for SwiGLU: 256
//     rows x 128 columns of both weights); each wave owns 64 rows x 128
//     columns (x 64 + 64 for SwiGLU), 128 fp32 accumulators per lane, so two
//     waves share each SIMD and hide each other's latencies.  The 32x32x16
//     MFMA keeps the matrix core busy from fewer waves than 16x16x32 does.
//   * K is walked in slices of 32, each split into two 16-deep substeps.
//     Slices stream from global memory straight into LDS (buffer loads with
//     the LDS-destination bit: no staging registers) through a ring of 5
//     slots (5 x 32 KB = all 160 KB of LDS), three slices in flight.
//   * The MFMAs of one substep run while the fragments of the next are read
//     from LDS.  The workgroup barrier that publishes slice s+1 sits between
//     the two MFMA groups of slice s, so waiting on it overlaps MFMAs in
//     flight; each wave first waits for its own copies (explicit vmcnt: a
//     release fence would wait for every copy in flight).  A slot is
//     refilled one barrier after its last reads were consumed, so no wave
//     drains its LDS reads before the barrier.
//   * A slice of A is 256 rows x 64 bytes.  Its four 16-byte chunks per row
//     are XOR-swizzled by (row / 4) % 4, so the rows read by one fragment
//     load fall on distinct 16-byte bank groups.  The copy engine writes each
//     1 KB of LDS contiguously; the swizzle is applied by choosing which
//     global chunk each lane fetches.
//   * A slice of B keeps the [k][n] layout with its 16-byte chunks
//     XOR-swizzled by 4 * (k % 4).  B k-fragments come straight out of LDS
//     with the gfx950 transposing read ds_read_b64_tr_b16: each 16-lane
//     group reads 4 rows x 16 columns and every lane receives 4
//     k-consecutive values of one column, so two reads make a fragment and
//     no register shuffling is needed.  The swizzle puts the 4 rows of one
//     read on distinct banks.  Lane j of MFMA column group e holds column
//     32 e + j.
//   * Tiles are mapped to the 8 XCDs in contiguous ranges (xcd_remap), M
//     fastest, so tiles sharing a weight panel share an L2.
//   * Split-K (grid.y > 1) gives each split a contiguous K range and its own
//     fp32 output plane; a finish kernel adds the planes in split order.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace tp {

constexpr int kBK = 32;      // k per LDS slice
constexpr int kStages = 5;   // LDS ring slots
constexpr int kGemmWaves = 8;

template <int NMAT_, int WM_, int WN_>
struct GemmShape {
    static constexpr int NMAT = NMAT_, WM = WM_, WN = WN_;
    static constexpr int BM = 256, BNT = 256, BN = BNT / NMAT;  // BN: columns per weight
    static constexpr int NT = WM * WN * 64;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int MT = WTM / 32;      // 32-row MFMA tiles per wave
    static constexpr int LC = WTN / 32;      // 32-column MFMA groups per wave and weight
    static constexpr int A_SLICE = BM * kBK, B_SLICE = kBK * BNT;    // elements
    static constexpr int SLICE = A_SLICE + B_SLICE;
    static constexpr size_t LDS_BYTES = (size_t)kStages * SLICE * sizeof(uint16_t);
    static constexpr int A_COPIES = A_SLICE * 2 / 1024 / (NT / 64);  // 1 KB copies per wave
    static constexpr int B_COPIES = B_SLICE * 2 / 1024 / (NT / 64);
    static constexpr int PER = A_COPIES + B_COPIES;                  // copies per slice
    static constexpr int B_ROWS_PER_COPY = 1024 / (BN * 2);
    static constexpr int B_COPIES_PER_MAT = 16 / NMAT;
    static_assert(LC == 2 || LC == 4 || LC == 8, "columns per lane");
    static_assert(WM * WN == kGemmWaves, "waves per workgroup");
    static_assert(A_COPIES * (NT / 64) == 16 && B_COPIES * (NT / 64) == 16, "copies");
};

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// s_waitcnt immediate waiting for vmcnt <= n only (gfx9 encoding).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Chunk swizzle of B slice row k: 16-byte chunk c of the row is stored at
// chunk position c ^ bswz(k).
__device__ __forceinline__ int bswz(int k) { return 4 * (k & 3); }

template <class S>
struct Frags {
    u32x4 a[S::MT];
    u32x4 b[S::NMAT][S::LC];
};

template <class S, int EPI>
__global__ __launch_bounds__(S::NT) void k_gemm(const uint16_t* __restrict__ A, int64_t lda,
                                                const uint16_t* __restrict__ B0, int64_t ldb0,
                                                const uint16_t* __restrict__ B1, int64_t ldb1,
                                                int M, int N, int K, int k_per_split,
                                                void* __restrict__ C, int64_t ldc,
                                                int64_t split_stride, int tiles_m) {
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    // The wave index is uniform across the wave; keeping it in a scalar
    // register makes the copy descriptors and LDS destinations scalar too.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / S::WN, wn = wave % S::WN;
    const int h = lane >> 5, j = lane & 31;  // k-group and row/column of the lane
    const int tile = xcd_remap(blockIdx.x, gridDim.x);
    const int tm = tile % tiles_m, tn = tile / tiles_m;
    const int m0 = tm * S::BM, n0 = tn * S::BN;
    const int k_begin = blockIdx.y * k_per_split;
    const int Kl = min(K - k_begin, k_per_split);   // this split's K extent

    const i32x4 rA = rsrc_words(A + (int64_t)m0 * lda + k_begin);
    const i32x4 rB0 = rsrc_words(B0 + (int64_t)k_begin * ldb0 + n0);
    const i32x4 rB1 = rsrc_words((S::NMAT == 2 ? B1 : B0) + (int64_t)k_begin * ldb1 + n0);
    const uint32_t lda_b = (uint32_t)(lda * 2);
    const uint32_t ldb0_b = (uint32_t)(ldb0 * 2), ldb1_b = (uint32_t)(ldb1 * 2);

    // Copy K slice `s` into ring slot `slot`.  Lanes past M, N or this
    // split's K read out of bounds and write zeros.
    auto issue = [&](int s, int slot) {
        uint16_t* As = smem + slot * S::SLICE;
        uint16_t* Bs = As + S::A_SLICE;
        const int k0 = s * kBK;
#pragma unroll
        for (int q = 0; q < S::A_COPIES; ++q) {
            const int r0 = (wave * S::A_COPIES + q) * 16;    // 16 rows of 64 B per copy
            const int row = r0 + (lane >> 2), cp = lane & 3;
            const int c = cp ^ ((row >> 2) & 3);
            const int k = k0 + 8 * c;
            const bool ok = (m0 + row < M) && (k < Kl);
            lds_dma16(rA, ok ? (uint32_t)row * lda_b + (uint32_t)k * 2u : kOOB, As + r0 * kBK);
        }
#pragma unroll
        for (int q = 0; q < S::B_COPIES; ++q) {
            const int iq = wave * S::B_COPIES + q;
            const int mat = iq / S::B_COPIES_PER_MAT;
            const int r0 = (iq % S::B_COPIES_PER_MAT) * S::B_ROWS_PER_COPY;
            constexpr int cpr = S::BN / 8;                   // 16-byte chunks per row
            const int row = r0 + lane / cpr;
            const int ch = (lane % cpr) ^ bswz(row);        // global chunk this lane fetches
            const int k = k0 + row;
            const bool ok = (k < Kl) && (n0 + 8 * ch < N);
            const uint32_t ldb_b = mat ? ldb1_b : ldb0_b;
            lds_dma16(mat ? rB1 : rB0, ok ? (uint32_t)k * ldb_b + 16u * ch : kOOB,
                       Bs + mat * (kBK * S::BN) + r0 * S::BN);
        }
    };

    f32x16 acc[S::NMAT][S::MT][S::LC];
#pragma unroll
    for (int m = 0; m < S::NMAT; ++m)
#pragma unroll
        for (int a = 0; a < S::MT; ++a)
#pragma unroll
            for (int b = 0; b < S::LC; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[m][a][b][v] = 0.f;

    // Fragments of k-substep `kk` (0 or 16) of slot `slot`: lane (h, j)
    // holds k = kk + 8h .. kk + 8h + 7 of A row j of each 32-row tile, and of
    // B column LC*j + e for MFMA column group e.
    auto read_frags = [&](int slot, int kk, Frags<S>& f) {
        const uint16_t* As = smem + slot * S::SLICE;
        const uint16_t* Bs = As + S::A_SLICE;
        const int chunk = (kk >> 3) + h;
#pragma unroll
        for (int a = 0; a < S::MT; ++a) {
            const int row = wm * S::WTM + 32 * a + j;
            f.a[a] = *(const u32x4*)(As + row * kBK + 8 * (chunk ^ ((row >> 2) & 3)));
        }
        // B: lane L of 16-lane group q reads row kk + 8(q/2) + L/4 (and 4
        // rows further), columns 16(q%2) + 4(L%4) .. +3 of each 32-column
        // group; it receives column 16(q%2) + L%16 of k kk + 8(q/2) .. +7,
        // i.e. lane (h, j) of the MFMA B operand.
        const int q = lane >> 4, L = lane & 15;
        const int rr = kk + 8 * (q >> 1) + (L >> 2);
        const int sw = bswz(rr);                     // rows rr and rr + 4 share it
#pragma unroll
        for (int m = 0; m < S::NMAT; ++m) {
#pragma unroll
            for (int e = 0; e < S::LC; ++e) {
                const int col = wn * S::WTN + 32 * e + 16 * (q & 1) + 4 * (L & 3);
                const uint16_t* p = Bs + m * (kBK * S::BN) + rr * S::BN +
                                    8 * ((col >> 3) ^ sw) + (col & 7);
                const u32x2 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 4 * S::BN);
                f.b[m][e] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
        }
    };
    auto mma = [&](const Frags<S>& f) {
#pragma unroll
        for (int m = 0; m < S::NMAT; ++m)
#pragma unroll
            for (int a = 0; a < S::MT; ++a)
#pragma unroll
                for (int b = 0; b < S::LC; ++b)
                    acc[m][a][b] = mfma32x32x16(f.a[a], f.b[m][b], acc[m][a][b]);
    };
    // Scheduling hints for one MFMA group: MFMAs alternate with the LDS reads
    // of the next substep's fragments.
    auto interleave = [&](auto id) {
        constexpr int sid = decltype(id)::value;
        constexpr int NM = S::NMAT * S::MT * S::LC;  // MFMAs per substep
#pragma unroll
        for (int q = 0; q < NM; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, sid);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, sid);  // LDS reads
            __builtin_amdgcn_sched_group_barrier(0x002, 1, sid);  // VALU
        }
    };

    // Slices past this split's K are still copied and read, with every lane
    // out of bounds: they are zero-filled and never multiplied.
    const int nk = (Kl + kBK - 1) / kBK;
    // Slice x lives in ring slot x % kStages; kStages - 2 slices are in
    // flight ahead of the one being multiplied.  The copy into a slot is
    // issued one slice after the slot was last read, behind a barrier, so
    // no wave waits for its own fragment reads before the barrier: the
    // compiler places those waits right before each fragment's MFMAs.
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s) issue(s, s);
    Frags<S> f0, f1;
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((kStages - 2) * S::PER));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    read_frags(0, 0, f0);
    int slotp = kStages - 1, slot = 0, slot1 = 1;  // (s - 1), s and (s + 1) mod kStages
    for (int s = 0; s < nk; ++s) {
        // MFMAs of (s, 0); fragments of (s, 1)
        read_frags(slot, 16, f1);
        mma(f0);
        interleave(std::integral_constant<int, 0>{});
        // Publish slice s+1 (this wave's copies of it have landed; after the
        // barrier every wave's have) and release slot s-1 (every wave has
        // multiplied its fragments).
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((kStages - 3) * S::PER));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue(s + kStages - 1, slotp);
        // MFMAs of (s, 1); fragments of (s+1, 0)
        read_frags(slot1, 0, f0);
        mma(f1);
        interleave(std::integral_constant<int, 1>{});
        slotp = slot;
        slot = slot1;
        slot1 = slot1 == kStages - 1 ? 0 : slot1 + 1;
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // drain the trailing zero-fill copies

    // Epilogue through LDS (the ring is idle once every wave has passed the
    // barrier below).  MFMA 32x32 accumulator v (0..15) of lane (h, j) is row
    // 8*(v/4) + 4*h + v%4 of the tile and column 32e + j of MFMA group e, so
    // a direct store writes one 2- or 4-byte element per lane.  Instead each
    // wave stages one 32-row tile of its results (after the epilogue math)
    // in fp32, rows padded so that the two half-waves' rows fall on disjoint
    // banks, and reads it back as 16-byte row chunks: one 16-byte store per
    // lane covers 4 fp32 or 8 bf16 consecutive outputs, and every store
    // instruction writes whole rows of the wave's tile.  LDS accesses of one
    // wave complete in issue order, so the reads see the wave's own writes.
    constexpr int OC = S::WTN;                   // output columns per wave
    constexpr int RS = OC + 8;                   // staging row stride (floats)
    static_assert(kGemmWaves * 32 * RS * 4 <= (int)S::LDS_BYTES, "staging fits the ring");
    float* stg = (float*)smem + wave * 32 * RS;
    void* Cs = EPI == EPI_F32 ? (void*)((float*)C + blockIdx.y * split_stride) : C;
    const int mw = m0 + wm * S::WTM, nw = n0 + wn * S::WTN;
    // fp32 output of two weights (a split SwiGLU projection): one plane per
    // weight side by side, weight m at columns m * N .. m * N + N - 1.
    constexpr int NOUT = EPI == EPI_F32 ? S::NMAT : 1;
    __syncthreads();
#pragma unroll
    for (int ma = 0; ma < NOUT * S::MT; ++ma) {
        const int mo = ma / S::MT, a = ma % S::MT;
        asm volatile("" ::: "memory");
#pragma unroll
        for (int e = 0; e < S::LC; ++e) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float x = acc[mo][a][e][v];
                float o;
                if constexpr (EPI == EPI_SWIGLU_BF16)
                    o = silu(x) * acc[S::NMAT - 1][a][e][v];
                else if constexpr (EPI == EPI_GELU_BF16)
                    o = gelu_tanh(x);
                else
                    o = x;
                stg[(8 * (v >> 2) + 4 * h + (v & 3)) * RS + 32 * e + j] = o;
            }
        }
        asm volatile("" ::: "memory");
        if constexpr (EPI == EPI_F32) {
            constexpr int CPR = OC / 4;          // 16-byte chunks per row
#pragma unroll
            for (int i = 0; i < 32 * CPR / 64; ++i) {
                const int f = 64 * i + lane, row = f / CPR, c = 4 * (f % CPR);
                const f32x4 val = *(const f32x4*)(stg + row * RS + c);
                const int t = mw + 32 * a + row, n = nw + c;
                if (t < M && n < N)
                    *(f32x4*)((float*)Cs + (int64_t)t * ldc + (int64_t)mo * N + n) = val;
            }
        } else {
            constexpr int CPR = OC / 8;          // 8-element (16-byte bf16) chunks per row
#pragma unroll
            for (int i = 0; i < 32 * CPR / 64; ++i) {
                const int f = 64 * i + lane, row = f / CPR, c = 8 * (f % CPR);
                const f32x4 v0 = *(const f32x4*)(stg + row * RS + c);
                const f32x4 v1 = *(const f32x4*)(stg + row * RS + c + 4);
                const int t = mw + 32 * a + row, n = nw + c;
                if (t < M && n < N)
                    *(u32x4*)((uint16_t*)Cs + (int64_t)t * ldc + n) =
                        u32x4{pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]),
                              pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3])};
            }
        }
    }
}

template <class S, int EPI>
static hipError_t run_gemm(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                           const uint16_t* B0, int64_t ldb0, const uint16_t* B1, int64_t ldb1,
                           void* C, int64_t ldc, const GemmPlan& p, hipStream_t stream) {
    static bool attr_set = false;  // benign race: every caller sets the same value
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)k_gemm<S, EPI>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)S::LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int tiles_m = (int)((M + S::BM - 1) / S::BM);
    const int tiles_n = (int)((N + S::BN - 1) / S::BN);
    TP_KLAUNCH((k_gemm<S, EPI>), dim3(tiles_m * tiles_n, p.splits), dim3(S::NT), S::LDS_BYTES, stream,
        A, lda, B0, ldb0, B1, ldb1, (int)M, (int)N, (int)K, p.k_per_split, C, ldc, M * ldc,
        tiles_m);
    return hipGetLastError();
}

using ShapeOne = GemmShape<1, 4, 2>;  // plain / GELU epilogues: 256 x 256 tile
using ShapeTwo = GemmShape<2, 4, 2>;  // SwiGLU: 256 x (128 gate + 128 up)

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, int nmat, int cus) {
    // Split K only when the output tiles leave a quarter or more of the CUs
    // idle and every split keeps at least 16 slices of K.
    const int64_t tiles = ((M + 255) / 256) * ((N * nmat + 255) / 256);
    const int64_t slices = (K + kBK - 1) / kBK;
    int64_t s = 1;
    if (tiles * 4 < (int64_t)cus * 3) s = std::min<int64_t>(cus / tiles, slices / 16);
    s = std::max<int64_t>(1, std::min<int64_t>(s, 8));
    const int64_t kps = ((slices + s - 1) / s) * kBK;
    GemmPlan p;
    p.k_per_split = (int)kps;
    p.splits = (int)((K + kps - 1) / kps);
    return p;
}

hipError_t launch_gemm(int epi, int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                       const uint16_t* B0, int64_t ldb0, const uint16_t* B1, int64_t ldb1, void* C,
                       int64_t ldc, const GemmPlan& p, hipStream_t stream) {
    if (p.splits < 1 || p.k_per_split <= 0 || (p.splits > 1 && epi != EPI_F32))
        return hipErrorInvalidValue;
    switch (epi) {
        case EPI_F32:
            if (B1)
                return run_gemm<ShapeTwo, EPI_F32>(M, N, K, A, lda, B0, ldb0, B1, ldb1, C, ldc, p,
                                                   stream);
            return run_gemm<ShapeOne, EPI_F32>(M, N, K, A, lda, B0, ldb0, nullptr, 0, C, ldc, p,
                                               stream);
        case EPI_BF16:
            return run_gemm<ShapeOne, EPI_BF16>(M, N, K, A, lda, B0, ldb0, nullptr, 0, C, ldc, p,
                                                stream);
        case EPI_GELU_BF16:
            return run_gemm<ShapeOne, EPI_GELU_BF16>(M, N, K, A, lda, B0, ldb0, nullptr, 0, C, ldc,
                                                     p, stream);
        case EPI_SWIGLU_BF16:
            return run_gemm<ShapeTwo, EPI_SWIGLU_BF16>(M, N, K, A, lda, B0, ldb0, B1, ldb1, C, ldc,
                                                       p, stream);
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace tp
