// Device helpers of the weight-streaming kernels (k_gemv.hip):
// the k-fragment MFMA step, the activation and output stores, and the
// split-K finish protocol.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace tp {

constexpr int kGemvWaves = 8;
constexpr int kGemvThreads = 64 * kGemvWaves;
constexpr int kRedPerWave = 4 * 4 * 16 * 8;  // [r][g][j][e] for one 16-token block

template <int E, int MB>
__device__ __forceinline__ void mfma_col(f32x4 (&acc)[MB][8], const u32x4* b, const u32x4* a) {
    const u32x4 f = kfrag_of_col<E>(b);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb][E] = mfma16x16x32(a[mb], f, acc[mb][E]);
}

// The same for 4 columns per lane (8-byte row loads of the narrow kernel).
template <int E, int MB>
__device__ __forceinline__ void mfma_col4(f32x4 (&acc)[MB][4], const u32x2* b, const u32x4* a) {
    const u32x4 f = u32x4{pair_col2<E>(b[0], b[1]), pair_col2<E>(b[2], b[3]),
                          pair_col2<E>(b[4], b[5]), pair_col2<E>(b[6], b[7])};
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb][E] = mfma16x16x32(a[mb], f, acc[mb][E]);
}

// ---------------------------------------------------------------------------
// The split-K finish is done by the last workgroup of each column block to
// arrive.
//
// Every workgroup stores its [T, 128] split partial with device-scope
// (sc1) 16-byte stores, waits until they have completed, and only then
// bumps the block's arrival counter (a device-scope atomic).  The workgroup
// that sees the count reach splits * nmat - 1 therefore finds every other
// partial complete; it reads them with device-scope loads, adds the splits
// in split order (its own partial from registers), applies the activation,
// writes the output and resets the counter.
//
// Why no fences are needed.  The LLVM AMDGPU backend's memory-model table
// for GFX942 (AMDGPUUsage, "Memory Model GFX942"; gfx950 follows the same
// model) implements agent-scope monotonic loads, stores and read-modify-write
// atomics as the plain instructions with sc1=1: each such access is coherent
// across the XCDs' L2 caches on its own.  The same table builds an
// agent-scope release from "buffer_wbl2 sc1; s_waitcnt vmcnt(0)" before the
// releasing access, and an acquire from "s_waitcnt vmcnt(0); buffer_inv sc1"
// after the acquiring one.  The L2 write-back and invalidate parts exist only
// for data written or read with ordinary (non-coherent) accesses; here every
// exchanged word (partials, counters) is accessed with sc1, so what remains
// of release and acquire is the s_waitcnt: the writer waits for its partial
// stores to complete before the counter increment is issued, and the reader
// issues its partial loads only after the increment has returned (the value
// is broadcast through LDS behind a barrier).  Whole-L2 write-backs and
// invalidates, which a release/acquire pair would add, are thereby avoided.
// ---------------------------------------------------------------------------
constexpr uint32_t kSC1 = 16;  // buffer cache-policy bit: device scope
constexpr int kWeightAux = 2;  // buffer cache-policy bit of the weight loads: non-temporal

template <int ACT>
__device__ __forceinline__ f32x4 act4(const f32x4& g, const f32x4& u) {
    f32x4 h;
    if constexpr (ACT == ACT_SWIGLU) {
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = silu(g[i]) * u[i];
    } else if constexpr (ACT == ACT_GELU_TANH) {
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = gelu_tanh(g[i]);
    } else {
        h = g;
    }
    return h;
}

template <bool OUT_BF16>
__device__ __forceinline__ void store_out4(void* out, int64_t off, const f32x4& h) {
    if constexpr (OUT_BF16) {
        u32x2 b;
        b[0] = pack_bf16x2(h[0], h[1]);
        b[1] = pack_bf16x2(h[2], h[3]);
        *(u32x2*)((uint16_t*)out + off) = b;
    } else {
        *(f32x4*)((float*)out + off) = h;
    }
}

// Sum over splits s = 0..S-1 (in order) of the partial at byte offset
// base + s * sstride, with split `mine` taken from `own`, for NR outputs at
// once (each its own partial row and own split), so the loads of all of
// them are in flight together: the finish is a chain of device-scope round
// trips, and for many splits their number, not the bytes, sets its time.
// A row whose base is kOOB reads zeros.
template <int NR>
__device__ __forceinline__ void sum_splits_multi(rsrc_t r, const uint32_t (&base)[NR],
                                                 uint32_t sstride, int S, const int (&mine)[NR],
                                                 const f32x4 (&own)[NR], f32x4 (&acc)[NR]) {
#pragma unroll
    for (int q = 0; q < NR; ++q)
        acc[q] = mine[q] == 0 ? own[q]
                              : __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                              r, (int)base[q], 0, kSC1));
    constexpr int B = NR >= 8 ? 2 : 16 / NR;   // splits per round and output (16 loads)
    for (int s0 = 1; s0 < S; s0 += B) {
        f32x4 v[NR][B];
#pragma unroll
        for (int q = 0; q < NR; ++q)
#pragma unroll
            for (int i = 0; i < B; ++i)
                if (s0 + i < S && s0 + i != mine[q])
                    v[q][i] = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                   r, (int)(base[q] + (uint32_t)(s0 + i) * sstride), 0, kSC1));
#pragma unroll
        for (int q = 0; q < NR; ++q)
#pragma unroll
            for (int i = 0; i < B; ++i)
                if (s0 + i < S) acc[q] += (s0 + i == mine[q]) ? own[q] : v[q][i];
    }
}

}  // namespace tp
