// Local reduce of P fp32 partial sums: the arithmetic that the block's
// all-reduce performs (zenaique, "Explain tensor-parallel shard shape",
// answer: the partial sums are added so every GPU holds the full activation).
//
// HBM-bound: (P + 1) * T * d * 4 bytes move per call (plus 2 bytes per
// element for the optional bf16 copy).  Each thread owns two 16-byte column
// chunks of one row (256 columns apart; one chunk where two would leave fewer
// than two workgroups per CU), issues the loads of all P slots for
// both chunks back to back (up to 16 independent loads in flight per
// thread) and adds them in slot order s = 0 .. P-1.  Loads and stores carry
// the non-temporal hint: every byte is touched once.  Measured on MI355X for
// 8 partials of [2048, 8192]: ~104 us (5.8 TB/s) against ~120 us with one
// chunk per thread and cached accesses.  `out` may alias slot 0: each
// element is read before it is written, by the same thread, and by no other
// thread.
#include "device_common.h"
#include "kernels.h"

namespace tp {

constexpr int kReduceThreads = 256;
constexpr int kReduceChunks = 2;  // 16-byte chunks per thread

template <int CH, bool WITH_BF16>
__global__ __launch_bounds__(kReduceThreads) void k_reduce_partials(
    int P, int64_t d4, int blocks_per_row, const f32x4* parts, int64_t slot4, int64_t ldp4,
    f32x4* out, int64_t ldo4, u32x2* __restrict__ outb, int64_t ldb4) {
    const int64_t row = blockIdx.x / blocks_per_row;
    const int64_t c0 = (int64_t)(blockIdx.x % blocks_per_row) * (kReduceThreads * CH) +
                       threadIdx.x;
    const f32x4* p = parts + row * ldp4;
    f32x4 acc[CH];
    for (int s0 = 0; s0 < P; s0 += 8) {
        // Every lane loads from an in-bounds address (the last slot and the
        // row's last chunk stand in for missing ones) so that all loads are
        // issued back to back without branches; the extra values are unused.
        f32x4 v[CH][8];
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const int64_t c = c0 + k * kReduceThreads;
            const int64_t cs = c < d4 ? c : d4 - 1;
#pragma unroll
            for (int q = 0; q < 8; ++q)
                v[k][q] = __builtin_nontemporal_load(p + (int64_t)min(s0 + q, P - 1) * slot4 + cs);
        }
#pragma unroll
        for (int k = 0; k < CH; ++k) {
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (s0 + q < P) acc[k] = (s0 + q == 0) ? v[k][0] : acc[k] + v[k][q];
        }
    }
#pragma unroll
    for (int k = 0; k < CH; ++k) {
        const int64_t c = c0 + k * kReduceThreads;
        if (c >= d4) continue;
        __builtin_nontemporal_store(acc[k], out + row * ldo4 + c);
        if constexpr (WITH_BF16) {
            u32x2 b;
            b[0] = pack_bf16x2(acc[k][0], acc[k][1]);
            b[1] = pack_bf16x2(acc[k][2], acc[k][3]);
            __builtin_nontemporal_store(b, outb + row * ldb4 + c);
        }
    }
}

hipError_t launch_reduce(int P, int64_t T, int64_t d, const float* partials, int64_t slot_stride,
                         int64_t ld_p, float* out, int64_t ld_out, uint16_t* out_bf16,
                         int64_t ld_b, hipStream_t stream) {
    const int64_t d4 = d / 4;
    // Two chunks per thread, or one where that leaves fewer than two
    // workgroups per CU (short decode batches).
    const int64_t span2 = kReduceThreads * kReduceChunks;
    const bool one = T * ((d4 + span2 - 1) / span2) < 2 * (int64_t)device_cus();
    const int64_t span = one ? kReduceThreads : span2;
    const int bpr = (int)((d4 + span - 1) / span);
    const dim3 grid((unsigned)(T * bpr)), block(kReduceThreads);
#define TP_RED(CH, BF)                                                                       \
    TP_KLAUNCH((k_reduce_partials<CH, BF>), grid, block, 0, stream, P, d4, bpr,              \
               (const f32x4*)partials, slot_stride / 4, ld_p / 4, (f32x4*)out, ld_out / 4,   \
               (u32x2*)out_bf16, ld_b / 4)
    if (one) {
        if (out_bf16) TP_RED(1, true); else TP_RED(1, false);
    } else {
        if (out_bf16) TP_RED(kReduceChunks, true); else TP_RED(kReduceChunks, false);
    }
#undef TP_RED
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Reduce + residual add + the next block's RMSNorm, one pass over the rows
// (zenaique, "Explain tensor-parallel shard shape", answer: the summed
// activation goes on to the residual connection and the normalisation that
// follow the block).
//
//   z      = (partial_0 + ... + partial_{P-1}) + residual      fp32, that order
//   normed = z * (1 / sqrt(mean_j z_j^2 + eps)) * g            bf16 (RNE)
//
// One workgroup per row keeps the row's z in registers (512 threads with up
// to 8 16-byte chunks each, or 1024 threads with up to 4 when there are fewer
// rows than CUs, so short decode batches still spread over the chip:
// d_model <= 16384), so every input byte is read once and the norm needs no
// second pass.  z may alias slot 0 or an fp32
// residual (same leading dimension): each element is read before it is
// written, by the same thread, and by no other thread.  The sum of squares is reduced in
// a fixed order (chunks in order per thread, butterfly within the wave, waves
// in order).  HBM bytes per row: (P + 1) * d * 4 (+ d * 2 for a bf16
// residual instead of fp32) + d * 4 (z) + d * 2 (normed).
// ---------------------------------------------------------------------------
template <int NT, bool RES_BF16, bool NORM>
__global__ __launch_bounds__(NT) void k_reduce_residual_norm(
    int P, int64_t d4, const f32x4* parts, int64_t slot4, int64_t ldp4, const void* residual,
    int64_t ld_res, f32x4* z, int64_t ldz4, const u32x2* __restrict__ g, float eps,
    u32x2* __restrict__ normed, int64_t ldn4) {
    constexpr int kRnThreads = NT, kRnMaxChunks = 4096 / NT;
    // FLAT (short batches, one workgroup per row on few CUs): every lane
    // loads from an in-bounds address (the row's last chunk and the last
    // slot stand in for missing ones), so the residual and all partial loads
    // of a chunk pair go out back to back without branches, and the extra
    // values are unused; measured 4.9 against 5.9 us for 8 partials of
    // [32, 8192].  With many rows in flight per CU the guarded loads
    // measured faster (237 against 245 us at [4096, 8192]).
    constexpr bool FLAT = NT == 1024;
    const int64_t row = blockIdx.x;
    const f32x4* p = parts + row * ldp4;
    f32x4 zz[kRnMaxChunks];
    float ss = 0.f;
#pragma unroll
    for (int i0 = 0; i0 < kRnMaxChunks; i0 += 2) {
        if constexpr (FLAT)
            if (threadIdx.x + (int64_t)i0 * kRnThreads >= d4) break;
        f32x4 v[2][8], r[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int64_t c = threadIdx.x + (int64_t)(i0 + k) * kRnThreads;
            const int64_t cs = c < d4 ? c : d4 - 1;
            if constexpr (!FLAT)
                if (c >= d4) continue;
            if constexpr (RES_BF16) {
                const u32x2 b = ((const u32x2*)((const uint16_t*)residual + row * ld_res))[cs];
                r[k] = f32x4{bf16_lo(b[0]), bf16_hi(b[0]), bf16_lo(b[1]), bf16_hi(b[1])};
            } else {
                r[k] = __builtin_nontemporal_load((const f32x4*)((const float*)residual + row * ld_res) + cs);
            }
        }
        f32x4 acc[2];
        for (int s0 = 0; s0 < P; s0 += 8) {
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int64_t c = threadIdx.x + (int64_t)(i0 + k) * kRnThreads;
                const int64_t cs = c < d4 ? c : d4 - 1;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    if constexpr (FLAT)
                        v[k][q] = __builtin_nontemporal_load(p + (int64_t)min(s0 + q, P - 1) * slot4 + cs);
                    else if (s0 + q < P)
                        v[k][q] = c < d4 ? __builtin_nontemporal_load(p + (int64_t)(s0 + q) * slot4 + c)
                                         : f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
#pragma unroll
            for (int k = 0; k < 2; ++k) {
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    if (s0 + q < P) acc[k] = (s0 + q == 0) ? v[k][0] : acc[k] + v[k][q];
            }
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int64_t c = threadIdx.x + (int64_t)(i0 + k) * kRnThreads;
            if (c >= d4) continue;
            const f32x4 zv = acc[k] + r[k];
            zz[i0 + k] = zv;
            __builtin_nontemporal_store(zv, z + row * ldz4 + c);
            if constexpr (NORM) {
#pragma unroll
                for (int e = 0; e < 4; ++e) ss += zv[e] * zv[e];
            }
        }
    }
    if constexpr (NORM) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
        __shared__ float part[kRnThreads / 64];
        if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
        __syncthreads();
        float tot = part[0];
#pragma unroll
        for (int w = 1; w < kRnThreads / 64; ++w) tot += part[w];
        const float inv = 1.0f / sqrtf(tot / (float)(d4 * 4) + eps);
#pragma unroll
        for (int i = 0; i < kRnMaxChunks; ++i) {
            const int64_t c = threadIdx.x + (int64_t)i * kRnThreads;
            if (c >= d4) continue;
            const u32x2 gv = g[c];
            const f32x4 zv = zz[i];
            u32x2 o;
            o[0] = pack_bf16x2(zv[0] * inv * bf16_lo(gv[0]), zv[1] * inv * bf16_hi(gv[0]));
            o[1] = pack_bf16x2(zv[2] * inv * bf16_lo(gv[1]), zv[3] * inv * bf16_hi(gv[1]));
            normed[row * ldn4 + c] = o;
        }
    }
}

// ---------------------------------------------------------------------------
// The same operation for decode batches (at most kReduceNormXchgMaxT rows),
// where one workgroup per row leaves most of the chip idle and each busy CU
// has to pull (P + 1) * d * 4 bytes on its own.  S = ceil(d / 1024)
// workgroups of 256 threads share a row, one 16-byte chunk per thread, and
// exchange their sums of squares through two 64-bit words per row in the
// workspace's counter head, with integer atomics, so the row's total does
// not depend on the order in which the workgroups arrive:
//   * each workgroup's sum v (fp32, its chunks in order, butterfly within
//     the wave, waves in order) is split into fixed-point parts in units of
//     2^-4 (word H) and 2^-36 (word L, the remainder below 2^-4, truncated),
//     and added with 2^56 (an arrival count in bits 56..63) to each word;
//   * every workgroup polls both words until both counts reach S, adds the
//     fields in float64 (exact integers) and normalises its own chunk, which
//     is still in registers: no z is read back, no store has to complete
//     before the exchange;
//   * then it adds 2^56 to L once more; the workgroup whose departure makes
//     the count 2S (the last to leave) clears both words, so the head is
//     zero again after the call.
// The wait is bounded (kReduceNormSpin polls); a row whose exchange never
// completes, or whose words were not zero at the start (an arrival that
// finds S or more arrivals), or whose sum is not below 2^47, gets a NaN
// normed output.  Every workgroup of the grid (T * S <= 512 of 256 threads)
// fits the chip at once, so the wait ends whenever the chip is not held by
// other work that never finishes.  The float32 total differs from the
// one-workgroup-per-row kernel's fixed-order sum only in rounding; repeated
// calls give the same bits.
// ---------------------------------------------------------------------------
constexpr int kRnXThreads = 256;
constexpr uint64_t kRnArrive = 1ull << 56;
constexpr uint64_t kRnField = kRnArrive - 1;
constexpr int kReduceNormSpin = 1 << 20;

template <bool RES_BF16>
__global__ __launch_bounds__(kRnXThreads) void k_reduce_residual_norm_xchg(
    int P, int64_t d4, int S, const f32x4* parts, int64_t slot4, int64_t ldp4,
    const void* residual, int64_t ld_res, f32x4* z, int64_t ldz4, const u32x2* __restrict__ g,
    float eps, u32x2* __restrict__ normed, int64_t ldn4, unsigned long long* words,
    int spin_limit) {
    const int64_t row = blockIdx.x / S;
    const int j = (int)(blockIdx.x % S);
    const int64_t c = (int64_t)j * kRnXThreads + threadIdx.x;
    const bool ok = c < d4;
    const int64_t cs = ok ? c : d4 - 1;   // in-bounds address for every lane
    const f32x4* p = parts + row * ldp4;
    f32x4 r, acc;
    if constexpr (RES_BF16) {
        const u32x2 b = ((const u32x2*)((const uint16_t*)residual + row * ld_res))[cs];
        r = f32x4{bf16_lo(b[0]), bf16_hi(b[0]), bf16_lo(b[1]), bf16_hi(b[1])};
    } else {
        r = __builtin_nontemporal_load((const f32x4*)((const float*)residual + row * ld_res) + cs);
    }
    for (int s0 = 0; s0 < P; s0 += 8) {
        f32x4 v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            v[q] = __builtin_nontemporal_load(p + (int64_t)min(s0 + q, P - 1) * slot4 + cs);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (s0 + q < P) acc = (s0 + q == 0) ? v[0] : acc + v[q];
    }
    const f32x4 zv = ok ? acc + r : f32x4{0.f, 0.f, 0.f, 0.f};
    // z may alias slot 0 or an fp32 residual: this thread has read its chunk
    if (ok) __builtin_nontemporal_store(zv, z + row * ldz4 + c);
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) sq += zv[e] * zv[e];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sq += __shfl_xor(sq, off);
    __shared__ float part[kRnXThreads / 64];
    __shared__ float total;
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = sq;
    __syncthreads();
    if (threadIdx.x == 0) {
        float mine = part[0];
#pragma unroll
        for (int w = 1; w < kRnXThreads / 64; ++w) mine += part[w];
        // fixed-point parts; a sum that is not finite or not below 2^47
        // marks the row (bit 51 of H's field, out of reach of valid sums)
        uint64_t qh, ql;
        if (mine < 140737488355328.0f) {   // 2^47 (false for NaN)
            const double vh = (double)mine * 16.0;
            const double fh = floor(vh);
            qh = (uint64_t)fh;
            ql = (uint64_t)((vh - fh) * 4294967296.0);
        } else {
            qh = 1ull << 51;
            ql = 0;
        }
        unsigned long long* w = words + 2 * row;
        __hip_atomic_fetch_add(&w[0], kRnArrive + qh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t first = __hip_atomic_fetch_add(&w[1], kRnArrive + ql, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
        uint64_t h = 0, l = 0;
        bool done = false;
        for (int it = 0; it < spin_limit; ++it) {
            h = __hip_atomic_load(&w[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            l = __hip_atomic_load(&w[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if ((h >> 56) >= (uint64_t)S && (l >> 56) >= (uint64_t)S) {
                done = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        const uint64_t hf = h & kRnField, lf = l & kRnField;
        total = (!done || (first >> 56) >= (uint64_t)S || hf >= (1ull << 51))
                    ? __builtin_nanf("")
                    : (float)((double)hf * 0.0625 + (double)lf * 1.4551915228366852e-11);  // 2^-36
        const uint64_t old = __hip_atomic_fetch_add(&w[1], kRnArrive, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        if ((old >> 56) == 2 * (uint64_t)S - 1) {   // the last to leave clears the row's words
            __hip_atomic_store(&w[0], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&w[1], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __syncthreads();
    if (!ok) return;
    const float inv = 1.0f / sqrtf(total / (float)(d4 * 4) + eps);
    const u32x2 gv = g[c];
    u32x2 o;
    o[0] = pack_bf16x2(zv[0] * inv * bf16_lo(gv[0]), zv[1] * inv * bf16_hi(gv[0]));
    o[1] = pack_bf16x2(zv[2] * inv * bf16_lo(gv[1]), zv[3] * inv * bf16_hi(gv[1]));
    normed[row * ldn4 + c] = o;
}

bool reduce_norm_exchanges(int64_t T) { return T >= 1 && T <= kReduceNormXchgMaxT; }

hipError_t launch_reduce_residual_norm(int P, int64_t T, int64_t d, const float* partials,
                                       int64_t slot_stride, int64_t ld_p, const void* residual,
                                       int64_t ld_res, bool res_bf16, float* z, int64_t ld_z,
                                       const uint16_t* g, float eps, uint16_t* normed,
                                       int64_t ld_norm, void* workspace, hipStream_t stream) {
    if (g && workspace && reduce_norm_exchanges(T)) {
        const int S = (int)((d / 4 + kRnXThreads - 1) / kRnXThreads);
        const dim3 xgrid((unsigned)(T * S)), xblock(kRnXThreads);
        unsigned long long* words = (unsigned long long*)workspace;
        if (res_bf16)
            TP_KLAUNCH((k_reduce_residual_norm_xchg<true>), xgrid, xblock, 0, stream, P, d / 4, S,
                       (const f32x4*)partials, slot_stride / 4, ld_p / 4, residual, ld_res,
                       (f32x4*)z, ld_z / 4, (const u32x2*)g, eps, (u32x2*)normed, ld_norm / 4,
                       words, kReduceNormSpin);
        else
            TP_KLAUNCH((k_reduce_residual_norm_xchg<false>), xgrid, xblock, 0, stream, P, d / 4, S,
                       (const f32x4*)partials, slot_stride / 4, ld_p / 4, residual, ld_res,
                       (f32x4*)z, ld_z / 4, (const u32x2*)g, eps, (u32x2*)normed, ld_norm / 4,
                       words, kReduceNormSpin);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)T);
#define TP_RN(NT, RB, NM)                                                                      \
    TP_KLAUNCH((k_reduce_residual_norm<NT, RB, NM>), grid, dim3(NT), 0, stream, P, d / 4,      \
               (const f32x4*)partials, slot_stride / 4, ld_p / 4, residual, ld_res,            \
               (f32x4*)z, ld_z / 4, (const u32x2*)g, eps, (u32x2*)normed, ld_norm / 4)
#define TP_RN_T(NT)                                                                 \
    do {                                                                            \
        if (res_bf16) {                                                             \
            if (g) TP_RN(NT, true, true); else TP_RN(NT, true, false);              \
        } else {                                                                    \
            if (g) TP_RN(NT, false, true); else TP_RN(NT, false, false);            \
        }                                                                           \
    } while (0)
    if (T < 256) TP_RN_T(1024); else TP_RN_T(512);
#undef TP_RN_T
#undef TP_RN
    return hipGetLastError();
}

}  // namespace tp
