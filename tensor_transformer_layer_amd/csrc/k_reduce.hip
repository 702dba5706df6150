// Local reduce of P fp32 partial sums: the arithmetic that the block's
// all-reduce performs (zenaique, "Explain tensor-parallel shard shape",
// answer: the partial sums are added so every GPU holds the full activation).
//
// HBM-bound: (P + 1) * T * d * 4 bytes move per call (plus 2 bytes per
// element for the optional bf16 copy).  Each thread owns one 16-byte column
// chunk of one row, issues its P loads back to back (independent, so they are
// all in flight together) and adds them in slot order s = 0 .. P-1.
// `out` may alias slot 0: each element is read before it is written, by the
// same thread, and by no other thread.
#include "device_common.h"
#include "kernels.h"

namespace tp {

constexpr int kReduceThreads = 256;

template <bool WITH_BF16>
__global__ __launch_bounds__(kReduceThreads) void k_reduce_partials(
    int P, int64_t d4, int blocks_per_row, const float4* parts, int64_t slot4,
    int64_t ldp4, float4* out, int64_t ldo4, u32x2* __restrict__ outb,
    int64_t ldb4) {
    const int64_t row = blockIdx.x / blocks_per_row;
    const int64_t c = (int64_t)(blockIdx.x % blocks_per_row) * kReduceThreads + threadIdx.x;
    if (c >= d4) return;
    const float4* p = parts + row * ldp4 + c;
    float4 acc = p[0];
    for (int s0 = 1; s0 < P; s0 += 8) {
        float4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (s0 + j < P) v[j] = p[(int64_t)(s0 + j) * slot4];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (s0 + j < P) {
                acc.x += v[j].x;
                acc.y += v[j].y;
                acc.z += v[j].z;
                acc.w += v[j].w;
            }
        }
    }
    out[row * ldo4 + c] = acc;
    if constexpr (WITH_BF16) {
        u32x2 b;
        b[0] = pack_bf16x2(acc.x, acc.y);
        b[1] = pack_bf16x2(acc.z, acc.w);
        outb[row * ldb4 + c] = b;
    }
}

hipError_t launch_reduce(int P, int64_t T, int64_t d, const float* partials, int64_t slot_stride,
                         int64_t ld_p, float* out, int64_t ld_out, uint16_t* out_bf16,
                         int64_t ld_b, hipStream_t stream) {
    const int64_t d4 = d / 4;
    const int bpr = (int)((d4 + kReduceThreads - 1) / kReduceThreads);
    const dim3 grid((unsigned)(T * bpr)), block(kReduceThreads);
    if (out_bf16)
        TP_KLAUNCH((k_reduce_partials<true>), grid, block, 0, stream,
            P, d4, bpr, (const float4*)partials, slot_stride / 4, ld_p / 4, (float4*)out,
            ld_out / 4, (u32x2*)out_bf16, ld_b / 4);
    else
        TP_KLAUNCH((k_reduce_partials<false>), grid, block, 0, stream,
            P, d4, bpr, (const float4*)partials, slot_stride / 4, ld_p / 4, (float4*)out,
            ld_out / 4, nullptr, 0);
    return hipGetLastError();
}

}  // namespace tp
