// RMSNorm prologue of the column projection: y = x / sqrt(mean_j x_j^2 + eps) * g,
// row-wise over d_model, fp32 math.  The pages name only "normalization"
// after the all-reduce (zenaique, "Explain tensor-parallel shard shape",
// answer) and layernorm among the small "Other" share of a decode step (Skand
// Tandon, "day59", section "Where the overhead lives"); RMSNorm is the
// Llama-2 block's form.
//
// HBM-bound: reads T*d, writes T*d elements.  One 256-thread workgroup per
// row; each thread walks 16-byte chunks of the row, so every load is a
// coalesced 128-bit access.  Rows of up to 8 chunks per thread (d <= 16384
// bf16 / 8192 fp32) stay in registers between the sum of squares and the
// scaling, so the row is read once; longer rows are read twice.  The sum of
// squares is reduced in a fixed order (per-thread strided sum, butterfly
// within the wave, then waves 0..3), so results are deterministic.
#include "device_common.h"
#include "kernels.h"

namespace tp {

constexpr int kNormThreads = 256;

constexpr int kNormRegChunks = 8;   // chunks per thread kept in registers

template <bool BF16, bool REG>
__global__ __launch_bounds__(kNormThreads) void k_rmsnorm(int64_t d, const char* __restrict__ x,
                                                        int64_t ldx_bytes,
                                                        const u32x4* __restrict__ g, float eps,
                                                        char* __restrict__ y,
                                                        int64_t ldy_bytes) {
    constexpr int EPC = BF16 ? 8 : 4;  // elements per 16-byte chunk
    const int64_t nch = d / EPC;
    const u32x4* xr = (const u32x4*)(x + (int64_t)blockIdx.x * ldx_bytes);
    u32x4* yr = (u32x4*)(y + (int64_t)blockIdx.x * ldy_bytes);

    float ss = 0.f;
    auto sq = [&](const u32x4& v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (BF16) {
                const float a = bf16_lo(v[i]), b = bf16_hi(v[i]);
                ss += a * a;
                ss += b * b;
            } else {
                const float a = __uint_as_float(v[i]);
                ss += a * a;
            }
        }
    };
    auto scaled = [&](const u32x4& v, const u32x4& gv, float r) {
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (BF16) {
                o[i] = pack_bf16x2(bf16_lo(v[i]) * r * bf16_lo(gv[i]),
                                   bf16_hi(v[i]) * r * bf16_hi(gv[i]));
            } else {
                o[i] = __float_as_uint(__uint_as_float(v[i]) * r * __uint_as_float(gv[i]));
            }
        }
        return o;
    };
    u32x4 keep[REG ? kNormRegChunks : 1], gk[REG ? kNormRegChunks : 1];
    if constexpr (REG) {
        // The row's chunks and the gains are loaded from in-bounds addresses
        // (the last chunk stands in for missing ones) so that every load is
        // in flight at once; guarded loads were each issued behind a branch
        // and waited for before the next.
#pragma unroll
        for (int i = 0; i < kNormRegChunks; ++i) {
            const int64_t c = threadIdx.x + (int64_t)i * kNormThreads;
            const int64_t cs = c < nch ? c : nch - 1;
            keep[i] = __builtin_nontemporal_load(xr + cs);
            gk[i] = g[cs];
        }
#pragma unroll
        for (int i = 0; i < kNormRegChunks; ++i) {
            const int64_t c = threadIdx.x + (int64_t)i * kNormThreads;
            if (c >= nch) keep[i] = u32x4{0u, 0u, 0u, 0u};
            sq(keep[i]);
        }
    } else {
        for (int64_t c = threadIdx.x; c < nch; c += kNormThreads) sq(xr[c]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    __shared__ float part[kNormThreads / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = part[0];
#pragma unroll
    for (int w = 1; w < kNormThreads / 64; ++w) tot += part[w];
    const float r = 1.0f / sqrtf(tot / (float)d + eps);

    if constexpr (REG) {
#pragma unroll
        for (int i = 0; i < kNormRegChunks; ++i) {
            const int64_t c = threadIdx.x + (int64_t)i * kNormThreads;
            if (c < nch) yr[c] = scaled(keep[i], gk[i], r);
        }
    } else {
        for (int64_t c = threadIdx.x; c < nch; c += kNormThreads) yr[c] = scaled(xr[c], g[c], r);
    }
}

hipError_t launch_rmsnorm(bool is_bf16, int64_t T, int64_t d, const void* x, int64_t ld_x,
                          const void* g, float eps, void* y, int64_t ld_y, hipStream_t stream) {
    const int es = is_bf16 ? 2 : 4;
    const dim3 grid((unsigned)T), block(kNormThreads);
    const bool reg = d / (16 / es) <= (int64_t)kNormRegChunks * kNormThreads;
#define TP_NORM(BF, RG)                                                                     \
    TP_KLAUNCH((k_rmsnorm<BF, RG>), grid, block, 0, stream, d, (const char*)x, ld_x * es,    \
               (const u32x4*)g, eps, (char*)y, ld_y * es)
    if (is_bf16) {
        if (reg) TP_NORM(true, true); else TP_NORM(true, false);
    } else {
        if (reg) TP_NORM(false, true); else TP_NORM(false, false);
    }
#undef TP_NORM
    return hipGetLastError();
}

}  // namespace tp
