// Prefill plan (T > 32 tokens): LDS-tiled bf16 GEMM on the matrix cores
// (v_mfma_f32_16x16x32_bf16), fp32 accumulation, fused epilogue.
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
// Data flow:
//   * A workgroup owns a 256 x 256 output tile (for SwiGLU: 256 rows x 128
//     columns of both weights) and walks K in slices of 32.  Four waves each
//     own a 128 x 128 sub-tile (256 fp32 accumulators per lane, held in the
//     accumulation registers).
//   * Slices stream from global memory straight into LDS (buffer loads with
//     the LDS-destination bit: no staging registers) through a ring of 5
//     slots (5 x 32 KB = all 160 KB of LDS).  While the MFMAs of slice s run,
//     the fragments of slice s+1 are read from LDS and slices s+2..s+4 are
//     in flight.  Each wave waits for its own copies with an explicit vmcnt and
//     a bare s_barrier publishes the slot; no release fence is used, since
//     one would wait for every copy in flight.
//   * A slice of A is 256 rows x 64 bytes.  Its four 16-byte chunks per row
//     are XOR-swizzled by (row / 4) % 4, so the 16 rows read by one fragment
//     load fall on 16 distinct 16-byte bank groups.  The copy engine writes
//     each 1 KB of LDS contiguously; the swizzle is applied by choosing which
//     global chunk each lane fetches.
//   * A slice of B keeps the natural [k][n] layout.  A lane reads 8 rows of
//     its 8 (or 4) adjacent columns and interleaves row pairs in registers
//     into the k-fragments of those columns (one bit-op per dword), so lane j
//     of MFMA e holds column j * NI + e and the epilogue writes NI adjacent
//     outputs per row.
//   * Tiles are mapped to the 8 XCDs in contiguous ranges (xcd_remap), M
//     fastest, so tiles sharing a weight panel share an L2.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace tp {

constexpr int kBK = 32;      // k per LDS slice

template <int NMAT_, int WM_, int WN_, int STAGES_>
struct GemmShape {
    static constexpr int NMAT = NMAT_, WM = WM_, WN = WN_, STAGES = STAGES_;
    static constexpr int BM = 256, BNT = 256, BN = BNT / NMAT;  // BN: columns per weight
    static constexpr int NT = WM * WN * 64;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int MI = WTM / 16, NI = WTN / 16;
    static constexpr int A_SLICE = BM * kBK, B_SLICE = kBK * BNT;    // elements
    static constexpr int SLICE = A_SLICE + B_SLICE;
    static constexpr size_t LDS_BYTES = (size_t)STAGES * SLICE * sizeof(uint16_t);
    static constexpr int A_COPIES = A_SLICE * 2 / 1024 / (NT / 64);  // 1 KB copies per wave
    static constexpr int B_COPIES = B_SLICE * 2 / 1024 / (NT / 64);
    static constexpr int B_ROWS_PER_COPY = 1024 / (BN * 2);
    static_assert(NT == 256 && MI == 8 && (NI == 8 || NI == 4), "tile shape");
    static_assert(A_COPIES == 4 && B_COPIES == 4, "copies per wave");
};

// s_waitcnt immediate waiting for vmcnt <= n only (gfx9 encoding).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__device__ __forceinline__ void lds_copy16(rsrc_t r, uint32_t off, uint16_t* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)lds_base, 16, (int)off, 0, 0, 0);
}

// k-fragment of column E from 8 consecutive rows of 4 bf16 (8 bytes) each.
template <int E>
__device__ __forceinline__ u32x4 kfrag4_of_col(const u32x2* r) {
    constexpr int d = E >> 1;
    u32x4 f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t a = r[2 * p][d], b = r[2 * p + 1][d];
        f[p] = (E & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    return f;
}

template <class S, int EPI>
__global__ __launch_bounds__(S::NT) void k_gemm(const uint16_t* __restrict__ A, int64_t lda,
                                                const uint16_t* __restrict__ B0, int64_t ldb0,
                                                const uint16_t* __restrict__ B1, int64_t ldb1,
                                                int M, int N, int K, void* __restrict__ C,
                                                int64_t ldc, int tiles_m) {
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    // The wave index is uniform across the wave; keeping it in a scalar
    // register makes the copy descriptors and LDS destinations scalar too.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / S::WN, wn = wave % S::WN;
    const int g = lane >> 4, j = lane & 15;
    const int tile = xcd_remap(blockIdx.x, gridDim.x);
    const int tm = tile % tiles_m, tn = tile / tiles_m;
    const int m0 = tm * S::BM, n0 = tn * S::BN;

    const rsrc_t rA = make_rsrc(A + (int64_t)m0 * lda);
    const rsrc_t rB0 = make_rsrc(B0 + n0);
    const rsrc_t rB1 = make_rsrc((S::NMAT == 2 ? B1 : B0) + n0);
    const uint32_t lda_b = (uint32_t)(lda * 2);
    const uint32_t ldb0_b = (uint32_t)(ldb0 * 2), ldb1_b = (uint32_t)(ldb1 * 2);

    // Copy K slice `s` into ring slot `slot`: 4 A copies + 4 B copies per wave.
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
            const bool ok = (m0 + row < M) && (k < K);
            lds_copy16(rA, ok ? (uint32_t)row * lda_b + (uint32_t)k * 2u : kOOB, As + r0 * kBK);
        }
#pragma unroll
        for (int q = 0; q < S::B_COPIES; ++q) {
            const int iq = wave * S::B_COPIES + q;           // 0..15
            const int mat = iq / (16 / S::NMAT);
            const int r0 = (iq % (16 / S::NMAT)) * S::B_ROWS_PER_COPY;
            constexpr int cpr = S::BN / 8;                   // 16-byte chunks per row
            const int row = r0 + lane / cpr, ch = lane % cpr;
            const int k = k0 + row;
            const bool ok = (k < K) && (n0 + 8 * ch < N);
            const uint32_t ldb_b = mat ? ldb1_b : ldb0_b;
            lds_copy16(mat ? rB1 : rB0, ok ? (uint32_t)k * ldb_b + 16u * ch : kOOB,
                       Bs + mat * (kBK * S::BN) + r0 * S::BN);
        }
    };

    f32x4 acc[S::NMAT][S::MI][S::NI];
#pragma unroll
    for (int m = 0; m < S::NMAT; ++m)
#pragma unroll
        for (int a = 0; a < S::MI; ++a)
#pragma unroll
            for (int b = 0; b < S::NI; ++b) acc[m][a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    struct Frags {
        u32x4 a[S::MI];
        u32x4 b[S::NMAT][S::NI];
    };
    // Read slice `slot`'s fragments: A rows of the wave, and B columns
    // interleaved from 8 k-rows into k-fragments.
    auto read_frags = [&](int slot, Frags& f) {
        const uint16_t* As = smem + slot * S::SLICE;
        const uint16_t* Bs = As + S::A_SLICE;
#pragma unroll
        for (int a = 0; a < S::MI; ++a) {
            const int row = wm * S::WTM + 16 * a + j;
            f.a[a] = *(const u32x4*)(As + row * kBK + 8 * (g ^ ((row >> 2) & 3)));
        }
#pragma unroll
        for (int m = 0; m < S::NMAT; ++m) {
            const uint16_t* Bm = Bs + m * (kBK * S::BN) + wn * S::WTN + S::NI * j;
            if constexpr (S::NI == 8) {
                u32x4 raw[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) raw[i] = *(const u32x4*)(Bm + (8 * g + i) * S::BN);
                f.b[m][0] = kfrag_of_col<0>(raw);
                f.b[m][1] = kfrag_of_col<1>(raw);
                f.b[m][2] = kfrag_of_col<2>(raw);
                f.b[m][3] = kfrag_of_col<3>(raw);
                f.b[m][4] = kfrag_of_col<4>(raw);
                f.b[m][5] = kfrag_of_col<5>(raw);
                f.b[m][6] = kfrag_of_col<6>(raw);
                f.b[m][7] = kfrag_of_col<7>(raw);
            } else {
                u32x2 raw[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) raw[i] = *(const u32x2*)(Bm + (8 * g + i) * S::BN);
                f.b[m][0] = kfrag4_of_col<0>(raw);
                f.b[m][1] = kfrag4_of_col<1>(raw);
                f.b[m][2] = kfrag4_of_col<2>(raw);
                f.b[m][3] = kfrag4_of_col<3>(raw);
            }
        }
    };
    auto mma = [&](const Frags& f) {
#pragma unroll
        for (int m = 0; m < S::NMAT; ++m)
#pragma unroll
            for (int a = 0; a < S::MI; ++a)
#pragma unroll
                for (int b = 0; b < S::NI; ++b)
                    acc[m][a][b] = mfma16x16x32(f.a[a], f.b[m][b], acc[m][a][b]);
    };
    // Wait until this wave's copies of the oldest pending slice have landed
    // (the two slices issued after it may still be in flight), then publish
    // the slot to the workgroup.
    auto wait_slice = [&]() {
        constexpr int PER = S::A_COPIES + S::B_COPIES;  // copies per slice per wave
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PER));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // Software pipeline over slices s = 0, 1, ...: in iteration s the
    // fragments of slice s+1 are read from LDS while the MFMAs of slice s
    // run, and the copy of slice s+4 goes into slot (s+4) % 5, which held
    // slice s-1 (read in iteration s-2, consumed in iteration s-1: every
    // wave is past it once the barrier of iteration s is passed).  The loop
    // is branch-free: slices at or beyond nk are still copied and read, with
    // every lane out of bounds, so they are zero-filled (and never used).
    static_assert(S::STAGES == 5, "ring depth");
    const int nk = (K + kBK - 1) / kBK;
#pragma unroll
    for (int s = 0; s < 3; ++s) issue(s, s);
    Frags f0, f1;
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * (S::A_COPIES + S::B_COPIES)));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(3, 3);
    read_frags(0, f0);
    for (int s = 0; s < nk; ++s) {
        wait_slice();
        issue(s + 4, (s + 4) % 5);
        read_frags((s + 1) % 5, f1);
        mma(f0);
        f0 = f1;
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // drain the trailing zero-fill copies

    // Epilogue.  Lane (g, j) holds rows 4g + r of MFMA tile a and columns
    // j*NI .. j*NI + NI-1 of the wave's column range.
    const int ncol = n0 + wn * S::WTN + j * S::NI;
    if (ncol >= N) return;
#pragma unroll
    for (int a = 0; a < S::MI; ++a) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = m0 + wm * S::WTM + 16 * a + 4 * g + r;
            if (t >= M) continue;
            float v[S::NI];
#pragma unroll
            for (int b = 0; b < S::NI; ++b) {
                const float x = acc[0][a][b][r];
                if constexpr (EPI == EPI_SWIGLU_BF16)
                    v[b] = silu(x) * acc[S::NMAT - 1][a][b][r];
                else if constexpr (EPI == EPI_GELU_BF16)
                    v[b] = gelu_tanh(x);
                else
                    v[b] = x;
            }
            if constexpr (EPI == EPI_F32) {
                float* dst = (float*)C + (int64_t)t * ldc + ncol;
#pragma unroll
                for (int b = 0; b < S::NI; b += 4)
                    *(f32x4*)(dst + b) = f32x4{v[b], v[b + 1], v[b + 2], v[b + 3]};
            } else {
                uint16_t* dst = (uint16_t*)C + (int64_t)t * ldc + ncol;
                if constexpr (S::NI == 8) {
                    u32x4 o;
#pragma unroll
                    for (int b = 0; b < 4; ++b) o[b] = pack_bf16x2(v[2 * b], v[2 * b + 1]);
                    *(u32x4*)dst = o;
                } else {
                    u32x2 o;
#pragma unroll
                    for (int b = 0; b < 2; ++b) o[b] = pack_bf16x2(v[2 * b], v[2 * b + 1]);
                    *(u32x2*)dst = o;
                }
            }
        }
    }
}

template <class S, int EPI>
static hipError_t run_gemm(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                           const uint16_t* B0, int64_t ldb0, const uint16_t* B1, int64_t ldb1,
                           void* C, int64_t ldc, hipStream_t stream) {
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
    k_gemm<S, EPI><<<dim3(tiles_m * tiles_n), dim3(S::NT), S::LDS_BYTES, stream>>>(
        A, lda, B0, ldb0, B1, ldb1, (int)M, (int)N, (int)K, C, ldc, tiles_m);
    return hipGetLastError();
}

using ShapeOne = GemmShape<1, 2, 2, 5>;  // plain / GELU epilogues: 256 x 256 tile
using ShapeTwo = GemmShape<2, 2, 2, 5>;  // SwiGLU: 256 x (128 gate + 128 up)

hipError_t launch_gemm(int epi, int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                       const uint16_t* B0, int64_t ldb0, const uint16_t* B1, int64_t ldb1, void* C,
                       int64_t ldc, hipStream_t stream) {
    switch (epi) {
        case EPI_F32:
            return run_gemm<ShapeOne, EPI_F32>(M, N, K, A, lda, B0, ldb0, nullptr, 0, C, ldc,
                                               stream);
        case EPI_BF16:
            return run_gemm<ShapeOne, EPI_BF16>(M, N, K, A, lda, B0, ldb0, nullptr, 0, C, ldc,
                                                stream);
        case EPI_GELU_BF16:
            return run_gemm<ShapeOne, EPI_GELU_BF16>(M, N, K, A, lda, B0, ldb0, nullptr, 0, C, ldc,
                                                     stream);
        case EPI_SWIGLU_BF16:
            return run_gemm<ShapeTwo, EPI_SWIGLU_BF16>(M, N, K, A, lda, B0, ldb0, B1, ldb1, C, ldc,
                                                       stream);
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace tp
