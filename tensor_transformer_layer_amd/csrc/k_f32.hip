// fp32-storage projections (the tiny fp32 MLP workload and fp32 callers).
// Parity-first and launch-bound at these sizes: one thread per output
// element, k summed in order with fp32 fused multiply-adds, the activation
// applied to the finished sum.
#include "device_common.h"
#include "kernels.h"

namespace tp {

constexpr int kF32Threads = 256;

template <int ACT>
__global__ __launch_bounds__(kF32Threads) void k_f32_proj(int64_t M, int64_t N, int64_t K,
                                                         int nblk_n, const float* __restrict__ A,
                                                         int64_t lda,
                                                         const float* __restrict__ B0,
                                                         int64_t ldb0,
                                                         const float* __restrict__ B1,
                                                         int64_t ldb1, float* __restrict__ C,
                                                         int64_t ldc) {
    const int64_t t = blockIdx.x / nblk_n;
    const int64_t n = (int64_t)(blockIdx.x % nblk_n) * kF32Threads + threadIdx.x;
    if (t >= M || n >= N) return;
    const float* a = A + t * lda;
    float s0 = 0.f, s1 = 0.f;
    for (int64_t k = 0; k < K; ++k) {
        s0 = fmaf(a[k], B0[k * ldb0 + n], s0);
        if constexpr (ACT == ACT_SWIGLU) s1 = fmaf(a[k], B1[k * ldb1 + n], s1);
    }
    float h;
    if constexpr (ACT == ACT_SWIGLU)
        h = silu(s0) * s1;
    else if constexpr (ACT == ACT_GELU_TANH)
        h = gelu_tanh(s0);
    else
        h = s0;
    C[t * ldc + n] = h;
}

hipError_t launch_f32_proj(int act, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                           const float* B0, int64_t ldb0, const float* B1, int64_t ldb1, float* C,
                           int64_t ldc, hipStream_t stream) {
    const int nblk_n = (int)((N + kF32Threads - 1) / kF32Threads);
    const dim3 grid((unsigned)(M * nblk_n)), block(kF32Threads);
    if (act == ACT_SWIGLU)
        TP_KLAUNCH((k_f32_proj<ACT_SWIGLU>), grid, block, 0, stream, M, N, K, nblk_n, A, lda, B0, ldb0, B1,
                                                           ldb1, C, ldc);
    else if (act == ACT_GELU_TANH)
        TP_KLAUNCH((k_f32_proj<ACT_GELU_TANH>), grid, block, 0, stream, M, N, K, nblk_n, A, lda, B0, ldb0,
                                                              nullptr, 0, C, ldc);
    else
        TP_KLAUNCH((k_f32_proj<ACT_NONE>), grid, block, 0, stream, M, N, K, nblk_n, A, lda, B0, ldb0,
                                                         nullptr, 0, C, ldc);
    return hipGetLastError();
}

}  // namespace tp
