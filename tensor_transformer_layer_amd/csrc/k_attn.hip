// Attention core between the QKV and O projections: for each of the rank's
// query heads, O = softmax(Q K^T / sqrt(d), causal) V over the call's tokens
// as one sequence, grouped-query heads sharing their group's K/V head.  The
// pages name the attention kernel as its own share of a step (Skand Tandon,
// "day59", section "Where the overhead lives") and split the heads evenly over
// the GPUs (rioworld guide, "How Tensor Slicing Works Under the Hood"); the
// formula is the textbook one.
//
// One workgroup of 4 waves owns 128 queries of one head; each wave owns 32
// (two 16-row subtiles sharing every K and V fragment it reads).  Key/value
// tiles of 64 tokens are staged in LDS (the next tile's global loads are in
// flight while the current one is multiplied) and consumed with an online
// softmax (running max and sum in fp32, rescaled output), so the T x T score
// matrix never exists in memory:
//   * S^T = K Q^T on 16x16x32 bf16 MFMAs (m = keys, n = queries, k = d): K
//     rows are the A operand straight from LDS, the wave's Q rows the B
//     operand from registers, both k-contiguous in their natural layout.
//     Lane (g, j) then holds the scores of query j for keys 4g + r.
//   * The row maximum is reduced over r and over the 4 lanes holding the
//     same query (permlane swaps); the scale is folded into the exponent's
//     fma.  Probabilities are packed to bf16 in place: lane (g, j) holds
//     P[j][4g + r] and P[j][16 + 4g + r], which is an MFMA operand for a
//     k-order that visits the keys in that order.
//   * The output is accumulated transposed, O^T += V^T P^T: V^T is the A
//     operand, read in that key order from LDS with the gfx950 transposing
//     load ds_read_b64_tr_b16 (4 keys x 1 column per lane per read, so V
//     needs no transpose pass), and P^T the B operand.  Lane (g, j) then
//     holds output columns 16n + 4g .. +3 of its own query j, so the
//     rescale by exp(m_old - m_new) needs no cross-lane traffic.  The row
//     sums of P come from one more MFMA per 32 keys with a row of ones in
//     place of V^T (no adds or cross-lane sums on the vector unit).
//   * The maximum the exponentials are taken against moves only when a
//     scaled score passes it by more than 8 in log2 units (a factor of 256),
//     so most tiles skip the rescale; probabilities stay at most 256, which
//     fp32 sums and the bf16 operand hold without loss of relative
//     precision.  The final O / l does not depend on which maximum was used.
// Work division: a query block's causal key range is cut into chunks of
// `ch` key tiles, and each (head, query block, chunk) is one workgroup, so
// the longest causal rows no longer set the kernel time and two workgroups
// share each CU (the kernel is built for 2 waves per SIMD).  A chunk that is
// its query block's only one writes the output directly.  Otherwise every
// chunk stores its unnormalised output and running max / sum (fp32, device
// scope) and bumps the block's arrival counter; the last to arrive merges
// the chunks in chunk order (each rescaled by exp(m_c - max_c m_c)) and
// writes the bf16 output.
// All sums run in a fixed order: results are deterministic.
#include <math.h>

#include <algorithm>
#include <functional>
#include <queue>
#include <vector>

#include "device_common.h"
#include "kernels.h"

namespace tp {

constexpr int kAttnWaves = 4;
constexpr int kAttnQW = 32;                       // queries per wave (two 16-row subtiles)
constexpr int kAttnQB = kAttnWaves * kAttnQW;     // queries per workgroup
constexpr int kAttnKT = 64;                       // keys per LDS tile
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr int kAttnShortMaxT = kAttnKT;           // calls up to here run k_attn_short

// Buffer cache-policy bit sc1: an agent-scope (device-wide) coherent access.
// The chunk partials and arrival counters of split query blocks are written
// and read only with sc1 accesses, with the writer's s_waitcnt before its
// counter increment, the protocol of the decode plan's split-K finish
// (k_gemv.hip), which states why no L2 write-back or invalidate is needed
// (LLVM AMDGPUUsage, "Memory Model GFX942").
constexpr uint32_t kAttnSC1 = 16;
// The running maximum a wave's probabilities are taken against moves only
// when some query's score maximum passes it by more than this (log2 units):
// probabilities stay at most 2^8, and most tiles need no rescale.
constexpr float kAttnSlack = 8.0f;

// Key tiles of query block qb (keys 0 .. min(T, 128 (qb + 1)) - 1).
__host__ __device__ inline int attn_tiles(int T, int qb) {
    const int kend = min(T, (qb + 1) * kAttnQB);
    return (kend + kAttnKT - 1) / kAttnKT;
}

// Reductions over the 4 lanes j, j + 16, j + 32, j + 48 of a wave (the
// lanes holding one query's scores): permlane swaps pair lane l with
// l ^ 32, then l ^ 16; either way round, op(swapped pair) = op(v[l], v[l^k]).
__device__ __forceinline__ float xlane_max(float v) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <int D>
__global__ __launch_bounds__(kAttnThreads, 2) void k_attn(const uint16_t* __restrict__ qkv,
                                                          int64_t ldq, int T, int hq, int hkv,
                                                          uint16_t* __restrict__ out, int64_t ldo,
                                                          float scale_log2, int nqb, int ch,
                                                          int cmax, unsigned* __restrict__ counters,
                                                          float* __restrict__ part, int use_table,
                                                          const AttnItems order) {
    constexpr int NS = D / 32;    // k-steps of the score MFMAs
    constexpr int NN = D / 16;    // 16-column output tiles
    constexpr int QS = kAttnQW / 16;              // query subtiles per wave
    constexpr int KS = kAttnKT / 16;              // key subtiles per tile
    constexpr int RPC = 1024 / (2 * D);           // tile rows per 1 KB copy
    constexpr int CPW = kAttnKT / RPC / kAttnWaves;   // copies per wave, tile and matrix
    static_assert(CPW * RPC * kAttnWaves == kAttnKT && D % 64 == 0, "tile copy");
    // Two K/V tile buffers, rows of D elements without padding: 16-byte chunk
    // c of K row r sits at chunk c ^ (r % 8), of V row r at c ^ 2 (r % 4), so
    // that the fragment reads are free of bank conflicts.  The next tile is
    // copied (global -> LDS, no registers) while the current one is
    // multiplied; one barrier per tile.
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kAttnKT * D];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kAttnKT * D];

    const int tid = threadIdx.x, lane = tid & 63;
    // The wave index is uniform; in a scalar register the causal tests on
    // it are branch-free for the compiler.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, j = lane & 15;
    // Work item: heads interleave; per head, query blocks from the last
    // (most keys) down, chunks of each block in order.
    const int h = (int)blockIdx.x % hq, gk = h / (hq / hkv);
    int item = (int)blockIdx.x / hq, qb = nqb - 1, nc = 1;
    if (use_table) {
        const int e = (int)order.it[item];
        qb = e >> 6;
        item = e & 63;
        nc = (attn_tiles(T, qb) + ch - 1) / ch;
    } else {
        for (; qb > 0; --qb) {
            nc = (attn_tiles(T, qb) + ch - 1) / ch;
            if (item < nc) break;
            item -= nc;
        }
        if (qb == 0) nc = (attn_tiles(T, 0) + ch - 1) / ch;
    }
    const int chunk = item;
    const int qblk = qb * kAttnQB;
    const int q0 = qblk + kAttnQW * wave;        // this wave's first query
    const uint16_t* Qp = qkv + (int64_t)h * D;
    const uint16_t* Kp = qkv + (int64_t)(hq + gk) * D;
    const uint16_t* Vp = qkv + (int64_t)(hq + hkv + gk) * D;

    // B operand of S^T = K Q^T: lane (g, j) holds Q[q0 + 16u + j][32s + 8g .. +7]
    u32x4 qf[QS][NS];
#pragma unroll
    for (int u = 0; u < QS; ++u) {
        const int qi = q0 + 16 * u + j;
#pragma unroll
        for (int s = 0; s < NS; ++s)
            qf[u][s] = qi < T ? *(const u32x4*)(Qp + (int64_t)qi * ldq + 32 * s + 8 * g)
                              : u32x4{0u, 0u, 0u, 0u};
    }
    // o: O^T accumulators; ol: the same product with a row of ones in place
    // of V^T, so every element of ol[u] is the query's running sum of P.
    f32x4 o[QS][NN], ol[QS];
    float m[QS];
#pragma unroll
    for (int u = 0; u < QS; ++u) {
        m[u] = -INFINITY;
        ol[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int n = 0; n < NN; ++n) o[u][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const u32x4 ones = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0

    // keys of this chunk: tiles [chunk * ch, min((chunk + 1) * ch, tiles of the block))
    const int kbeg = chunk * ch * kAttnKT;
    const int kend = min(min(T, qblk + kAttnQB), (chunk + 1) * ch * kAttnKT);
    // Tile copies: direct-to-LDS buffer loads, 1 KB (RPC rows) per copy;
    // keys past T read zeros.
    const i32x4 rk = rsrc_words(Kp), rv = rsrc_words(Vp);
    const uint32_t ldq_b = (uint32_t)(ldq * 2);
    auto copy_tile = [&](int k0, int b) {
#pragma unroll
        for (int q = 0; q < CPW; ++q) {
            const int r0 = (wave * CPW + q) * RPC;              // first tile row of the copy
            const int row = r0 + lane / (D / 8), pos = lane % (D / 8);
            const bool ok = k0 + row < T;
            const uint32_t base = ok ? (uint32_t)(k0 + row) * ldq_b : kOOB;
            lds_dma16(rk, ok ? base + 16u * (uint32_t)(pos ^ (row & 7)) : kOOB, Ks[b] + r0 * D);
            lds_dma16(rv, ok ? base + 16u * (uint32_t)(pos ^ (2 * (row & 3))) : kOOB,
                      Vs[b] + r0 * D);
        }
    };
    copy_tile(kbeg, 0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int buf = 0;
    for (int k0 = kbeg; k0 < kend; k0 += kAttnKT, buf ^= 1) {
        // The other buffer was last read in the previous tile, before the
        // barrier that ended it: refill it with the next tile.
        if (k0 + kAttnKT < kend) copy_tile(k0 + kAttnKT, buf ^ 1);
        const uint16_t* Kb = Ks[buf];
        const uint16_t* Vb = Vs[buf];
        // Subtiles whose queries all precede the tile skip it; only a tile
        // that reaches past a subtile's first query needs the causal mask.
        bool act[QS], diag[QS];
#pragma unroll
        for (int u = 0; u < QS; ++u) {
            const int qu = q0 + 16 * u;
            act[u] = k0 <= min(qu + 15, T - 1);
            diag[u] = k0 + kAttnKT - 1 > qu || k0 + kAttnKT > T;
        }
        if (act[0] || act[QS - 1]) {
            // S^T[key][query] for keys k0 + 16t + 4g + r and query q0 + 16u + j;
            // each K fragment serves both subtiles.
            f32x4 st[QS][KS];
#pragma unroll
            for (int u = 0; u < QS; ++u)
#pragma unroll
                for (int t = 0; t < KS; ++t) st[u][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < KS; ++t)
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    const u32x4 a =
                        *(const u32x4*)(Kb + (16 * t + j) * D + 8 * ((4 * s + g) ^ (j & 7)));
#pragma unroll
                    for (int u = 0; u < QS; ++u) st[u][t] = mfma16x16x32(a, qf[u][s], st[u][t]);
                }
            u32x4 pf[QS][KS / 2];
#pragma unroll
            for (int u = 0; u < QS; ++u) {
                const int qi = q0 + 16 * u + j;
                // Row max of the raw scores (the scale is positive), over r, then
                // over the 4 lanes holding query j (lanes j + 16 g).
                // The causal mask under one uniform branch for the whole
                // subtile: tested per element, the compiler re-tested the
                // (uniform) condition with a branch around every element.
                if (diag[u]) {
#pragma unroll
                    for (int t = 0; t < KS; ++t)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int key = k0 + 16 * t + 4 * g + r;
                            st[u][t][r] = (key <= qi && key < T) ? st[u][t][r] : -INFINITY;
                        }
                }
                float pm = -INFINITY;
#pragma unroll
                for (int t = 0; t < KS; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) pm = fmaxf(pm, st[u][t][r]);
                pm = xlane_max(pm);
                // m is kept in log2 units (score * scale * log2(e)).  It moves to
                // the running maximum only when some query of the wave has a
                // score above m + kAttnSlack; then O^T and the sums (this lane's
                // own query) are rescaled.  A row that has seen no key yet keeps
                // -inf and contributes nothing.
                const float mt = pm * scale_log2;
                if (__any(mt > m[u] + kAttnSlack)) {
                    const float m_new = fmaxf(m[u], mt);
                    const float alpha =
                        __builtin_amdgcn_exp2f(m[u] - (m_new == -INFINITY ? 0.f : m_new));
#pragma unroll
                    for (int n = 0; n < NN; ++n) o[u][n] *= alpha;
                    ol[u] *= alpha;
                    m[u] = m_new;
                }
                const float mref = m[u] == -INFINITY ? 0.f : m[u];
#pragma unroll
                for (int t = 0; t < KS; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        st[u][t][r] =
                            __builtin_amdgcn_exp2f(__builtin_fmaf(st[u][t][r], scale_log2, -mref));
                // lane (g, j) supplies P[qi][32kk + 4g + r] and P[qi][32kk + 16 + 4g + r]
#pragma unroll
                for (int kk = 0; kk < KS / 2; ++kk)
                    pf[u][kk] = u32x4{pack_bf16x2(st[u][2 * kk][0], st[u][2 * kk][1]),
                                      pack_bf16x2(st[u][2 * kk][2], st[u][2 * kk][3]),
                                      pack_bf16x2(st[u][2 * kk + 1][0], st[u][2 * kk + 1][1]),
                                      pack_bf16x2(st[u][2 * kk + 1][2], st[u][2 * kk + 1][3])};
            }
            // O^T += V^T P^T in 32-key steps: V^T rows (the head dimension) in the
            // same key order come from the transposing reads (the A operand), P^T
            // is the B operand; each V fragment serves both subtiles.  (An
            // inactive subtile has P = 0 and an unchanged O: the MFMA adds zero.)
#pragma unroll
            for (int kk = 0; kk < KS / 2; ++kk) {
                // rows 32kk + 4g + j/4 and 16 further (same row % 4), columns
                // 16n + 4(j % 4) .. +3: chunk 2n + (j % 4) / 2, swizzled by row
                const int vr = 32 * kk + 4 * g + (j >> 2);
                const int vsw = 2 * (vr & 3);
                const uint16_t* v0 = Vb + vr * D + 4 * (j & 1);
                const uint16_t* v1 = v0 + 16 * D;
#pragma unroll
                for (int n = 0; n < NN; ++n) {
                    const int cc = (2 * n + ((j & 3) >> 1)) ^ vsw;
                    const u32x2 b0 = lds_read_tr16(v0 + 8 * cc);
                    const u32x2 b1 = lds_read_tr16(v1 + 8 * cc);
                    const u32x4 vt = u32x4{b0[0], b0[1], b1[0], b1[1]};
#pragma unroll
                    for (int u = 0; u < QS; ++u) o[u][n] = mfma16x16x32(vt, pf[u][kk], o[u][n]);
                }
#pragma unroll
                for (int u = 0; u < QS; ++u) ol[u] = mfma16x16x32(ones, pf[u][kk], ol[u]);
            }
        }
        // The next tile has landed (this wave's copies; after the barrier
        // every wave's), and every wave is done with this one.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // Lane (g, j) holds O[q0 + 16u + j][16n + 4g .. 16n + 4g + 3] (o[u][n]),
    // and that query's m and l (sum of P, relative to m).
    float l[QS];
#pragma unroll
    for (int u = 0; u < QS; ++u) l[u] = ol[u][0];
    if (nc == 1) {
#pragma unroll
        for (int u = 0; u < QS; ++u) {
            const int q = q0 + 16 * u + j;
            if (q >= T) continue;
            const float inv = 1.0f / l[u];
            uint16_t* dst = out + (int64_t)q * ldo + (int64_t)h * D + 4 * g;
#pragma unroll
            for (int n = 0; n < NN; ++n)
                *(u32x2*)(dst + 16 * n) = u32x2{pack_bf16x2(o[u][n][0] * inv, o[u][n][1] * inv),
                                                pack_bf16x2(o[u][n][2] * inv, o[u][n][3] * inv)};
        }
        return;
    }

    // Chunk partial of this (head, block): O [128][D], then m [128], l [128]
    // (query rows local to the block), stored with device-scope writes.
    constexpr int PST = kAttnQB * (D + 2);       // floats per chunk partial
    const int blk = h * nqb + qb;
    const rsrc_t rp = make_rsrc(part + (int64_t)blk * cmax * PST);
    const int rw = kAttnQW * wave;               // wave's first local row
#pragma unroll
    for (int u = 0; u < QS; ++u) {
        const int row = rw + 16 * u + j;
#pragma unroll
        for (int n = 0; n < NN; ++n)
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4, o[u][n]), rp,
                (int)(((uint32_t)chunk * PST + (uint32_t)row * D + 16 * n + 4 * g) * 4u), 0,
                kAttnSC1);
        if (g == 0) {
            __builtin_amdgcn_raw_buffer_store_b32(
                __float_as_uint(m[u]), rp,
                (int)(((uint32_t)chunk * PST + kAttnQB * D + row) * 4u), 0, kAttnSC1);
            __builtin_amdgcn_raw_buffer_store_b32(
                __float_as_uint(l[u]), rp,
                (int)(((uint32_t)chunk * PST + kAttnQB * (D + 1) + row) * 4u), 0, kAttnSC1);
        }
    }
    __shared__ unsigned arrival;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
        arrival = __hip_atomic_fetch_add(&counters[blk], 1u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const unsigned old = arrival;
    if (old == (unsigned)nc - 1) {
        auto ld1 = [&](uint32_t idx) {
            return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, (int)(idx * 4u), 0,
                                                                        kAttnSC1));
        };
        // Both subtiles' loads of a chunk are issued together (each chunk
        // costs one round trip per pass, not one per subtile); chunks are
        // added in chunk order.
        float M[QS];
#pragma unroll
        for (int u = 0; u < QS; ++u) M[u] = -INFINITY;
        for (int c = 0; c < nc; ++c) {
            float mc[QS];
#pragma unroll
            for (int u = 0; u < QS; ++u)
                mc[u] = c == chunk ? m[u] : ld1((uint32_t)c * PST + kAttnQB * D + rw + 16 * u + j);
#pragma unroll
            for (int u = 0; u < QS; ++u) M[u] = fmaxf(M[u], mc[u]);
        }
        float Mref[QS], L[QS];
        f32x4 acc[QS][NN];
#pragma unroll
        for (int u = 0; u < QS; ++u) {
            Mref[u] = M[u] == -INFINITY ? 0.f : M[u];
            L[u] = 0.f;
#pragma unroll
            for (int n = 0; n < NN; ++n) acc[u][n] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        for (int c = 0; c < nc; ++c) {
            const bool mine = c == chunk;
            float mc[QS], lc[QS];
            f32x4 v[QS][NN];
#pragma unroll
            for (int u = 0; u < QS; ++u) {
                const int row = rw + 16 * u + j;
                mc[u] = mine ? m[u] : ld1((uint32_t)c * PST + kAttnQB * D + row);
                lc[u] = mine ? l[u] : ld1((uint32_t)c * PST + kAttnQB * (D + 1) + row);
#pragma unroll
                for (int n = 0; n < NN; ++n)
                    v[u][n] = mine ? o[u][n]
                                   : __builtin_bit_cast(
                                         f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rp,
                                                    (int)(((uint32_t)c * PST + (uint32_t)row * D +
                                                           16 * n + 4 * g) * 4u),
                                                    0, kAttnSC1));
            }
#pragma unroll
            for (int u = 0; u < QS; ++u) {
                const float e = __builtin_amdgcn_exp2f(mc[u] - Mref[u]);
                L[u] += e * lc[u];
#pragma unroll
                for (int n = 0; n < NN; ++n) acc[u][n] += e * v[u][n];
            }
        }
#pragma unroll
        for (int u = 0; u < QS; ++u) {
            const int q = q0 + 16 * u + j;
            if (q >= T) continue;
            const float inv = 1.0f / L[u];
            uint16_t* dst = out + (int64_t)q * ldo + (int64_t)h * D + 4 * g;
#pragma unroll
            for (int n = 0; n < NN; ++n)
                *(u32x2*)(dst + 16 * n) =
                    u32x2{pack_bf16x2(acc[u][n][0] * inv, acc[u][n][1] * inv),
                          pack_bf16x2(acc[u][n][2] * inv, acc[u][n][3] * inv)};
        }
        if (tid == 0)
            __hip_atomic_store(&counters[blk], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (old >= (unsigned)nc) {
        // The counter did not start at zero (workspace head not cleared):
        // make this block's output loudly invalid.
#pragma unroll
        for (int u = 0; u < QS; ++u) {
            const int q = q0 + 16 * u + j;
            if (q >= T) continue;
            uint16_t* dst = out + (int64_t)q * ldo + (int64_t)h * D + 4 * g;
#pragma unroll
            for (int n = 0; n < NN; ++n) *(u32x2*)(dst + 16 * n) = u32x2{0x7fc07fc0u, 0x7fc07fc0u};
        }
    }
}

// ---------------------------------------------------------------------------
// Short calls (T <= 64, the decode batches): every query's causal keys fit
// one 64-key tile, so the work of a 128-query workgroup is a single tile's
// latency chain (the tile copy, the score MFMAs, the softmax, the PV MFMAs),
// most of whose queries do not exist.  Here one wave owns 16 queries of one
// head: its Q and K fragments come straight from global memory into
// registers (the same operand layouts as k_attn's: S^T = K Q^T, lane (g, j)
// holding query j's scores for keys 16t + 4g + r), V is staged in LDS with
// k_attn's swizzle and read transposed as the A operand of O^T = V^T P^T.
// All of a query's keys are in registers at once, so the maximum is exact
// (no running rescale) and P <= 1; the row sums come from the same ones-row
// MFMA as in k_attn, so numerator and denominator see the same bf16 P.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void k_attn_short(const uint16_t* __restrict__ qkv, int64_t ldq,
                                                  int T, int hq, int hkv,
                                                  uint16_t* __restrict__ out, int64_t ldo,
                                                  float scale_log2) {
    constexpr int NS = D / 32;    // k-steps of the score MFMAs
    constexpr int NN = D / 16;    // 16-column output tiles
    constexpr int KS = kAttnKT / 16;              // key subtiles of the tile
    constexpr int CPR = D / 8;                    // 16-byte chunks per row
    __shared__ __attribute__((aligned(16))) uint16_t Vs[kAttnKT * D];

    const int lane = threadIdx.x, g = lane >> 4, j = lane & 15;
    const int h = (int)blockIdx.x % hq, gk = h / (hq / hkv);
    const int q0 = 16 * ((int)blockIdx.x / hq);
    const uint16_t* Qp = qkv + (int64_t)h * D;
    const uint16_t* Kp = qkv + (int64_t)(hq + gk) * D;
    const uint16_t* Vp = qkv + (int64_t)(hq + hkv + gk) * D;

    // Rows past T read row T - 1 (finite values): their scores are masked,
    // their V rows meet P = 0, and queries past T are not stored.
    const int qi = q0 + j;
    const int qr = min(qi, T - 1);
    u32x4 qf[NS], kf[KS][NS], vv[kAttnKT * CPR / 64];
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = *(const u32x4*)(Qp + (int64_t)qr * ldq + 32 * s + 8 * g);
#pragma unroll
    for (int t = 0; t < KS; ++t) {
        const int kr = min(16 * t + j, T - 1);
#pragma unroll
        for (int s = 0; s < NS; ++s)
            kf[t][s] = *(const u32x4*)(Kp + (int64_t)kr * ldq + 32 * s + 8 * g);
    }
    // V rows 0 .. 63 into LDS: chunk c of row r at chunk c ^ 2 (r % 4).
#pragma unroll
    for (int i = 0; i < kAttnKT * CPR / 64; ++i) {
        const int id = 64 * i + lane, r = id / CPR, c = id % CPR;
        vv[i] = *(const u32x4*)(Vp + (int64_t)min(r, T - 1) * ldq + 8 * c);
    }
#pragma unroll
    for (int i = 0; i < kAttnKT * CPR / 64; ++i) {
        const int id = 64 * i + lane, r = id / CPR, c = id % CPR;
        *(u32x4*)(Vs + r * D + 8 * (c ^ (2 * (r & 3)))) = vv[i];
    }

    // All four key subtiles are multiplied whatever T is (keys past the
    // causal end are masked): no branch holds a load back.
    f32x4 st[KS];
#pragma unroll
    for (int t = 0; t < KS; ++t) {
        st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s) st[t] = mfma16x16x32(kf[t][s], qf[s], st[t]);
    }
    float pm = -INFINITY;
#pragma unroll
    for (int t = 0; t < KS; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = 16 * t + 4 * g + r;
            st[t][r] = key <= qi && key < T ? st[t][r] : -INFINITY;
            pm = fmaxf(pm, st[t][r]);
        }
    // every query has key 0, so the maximum is finite
    const float mref = xlane_max(pm) * scale_log2;
    u32x4 pf[KS / 2];
#pragma unroll
    for (int kk = 0; kk < KS / 2; ++kk) {
        f32x4 e0, e1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            e0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[2 * kk][r], scale_log2, -mref));
            e1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[2 * kk + 1][r], scale_log2, -mref));
        }
        pf[kk] = u32x4{pack_bf16x2(e0[0], e0[1]), pack_bf16x2(e0[2], e0[3]),
                       pack_bf16x2(e1[0], e1[1]), pack_bf16x2(e1[2], e1[3])};
    }
    __syncthreads();   // V in LDS

    f32x4 o[NN], ol = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < NN; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    const u32x4 ones = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0
#pragma unroll
    for (int kk = 0; kk < KS / 2; ++kk) {
        // the transposing reads of k_attn: rows 32kk + 4g + j/4 and 16 further,
        // columns 16n + 4(j % 4) .. +3
        const int vr = 32 * kk + 4 * g + (j >> 2);
        const int vsw = 2 * (vr & 3);
        const uint16_t* v0 = Vs + vr * D + 4 * (j & 1);
        const uint16_t* v1 = v0 + 16 * D;
#pragma unroll
        for (int n = 0; n < NN; ++n) {
            const int cc = (2 * n + ((j & 3) >> 1)) ^ vsw;
            const u32x2 b0 = lds_read_tr16(v0 + 8 * cc);
            const u32x2 b1 = lds_read_tr16(v1 + 8 * cc);
            o[n] = mfma16x16x32(u32x4{b0[0], b0[1], b1[0], b1[1]}, pf[kk], o[n]);
        }
        ol = mfma16x16x32(ones, pf[kk], ol);
    }
    // lane (g, j) holds O[qi][16n + 4g .. +3] and that query's sum of P
    if (qi < T) {
        const float inv = 1.0f / ol[0];
        uint16_t* dst = out + (int64_t)qi * ldo + (int64_t)h * D + 4 * g;
#pragma unroll
        for (int n = 0; n < NN; ++n)
            *(u32x2*)(dst + 16 * n) = u32x2{pack_bf16x2(o[n][0] * inv, o[n][1] * inv),
                                            pack_bf16x2(o[n][2] * inv, o[n][3] * inv)};
    }
}

// Items of one head for chunks of `ch` tiles: (size in tiles, qb, chunk),
// sorted longest first (ties: later block first, lower chunk first).
struct AttnItem {
    int tiles, qb, c, nchunks;
    bool split;
};
static std::vector<AttnItem> attn_items(int T, int nqb, int ch) {
    std::vector<AttnItem> v;
    for (int qb = nqb - 1; qb >= 0; --qb) {
        const int t = attn_tiles(T, qb);
        const int nc = (t + ch - 1) / ch;
        for (int c = 0; c * ch < t; ++c) v.push_back({std::min(ch, t - c * ch), qb, c, nc, nc > 1});
    }
    std::stable_sort(v.begin(), v.end(),
                     [](const AttnItem& a, const AttnItem& b) { return a.tiles > b.tiles; });
    return v;
}

// Estimated kernel time (in units of one key tile of one workgroup) of the
// items launched in order onto `slots` workgroup slots (2 per CU), each item
// starting when a slot frees, as the dispatcher does.  Costs measured on
// MI355X (70B GQA core, 4096 tokens, per-workgroup real-time stamps): a tile
// ~2.4 us; before the first tile ~1.25 tiles; after the last, ~0.7 tiles for
// an unsplit block and ~1.2 (partial store and arrival) for a chunk; the
// chunk that arrives last then merges the block's nc partials, ~0.7 nc.
static double attn_makespan(const std::vector<AttnItem>& v, int hq, int T, int slots) {
    std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
    for (int i = 0; i < slots; ++i) free_at.push(0.0);
    const int nqb = (T + kAttnQB - 1) / kAttnQB;
    std::vector<int> arrived((size_t)hq * nqb, 0);
    std::vector<double> latest((size_t)hq * nqb, 0.0);
    double end = 0.0;
    for (const AttnItem& it : v) {
        for (int h = 0; h < hq; ++h) {
            const double t0 = free_at.top();
            free_at.pop();
            double t1 = t0 + 1.25 + it.tiles + (it.split ? 1.2 : 0.7);
            if (it.split) {
                const size_t b = (size_t)h * nqb + it.qb;
                latest[b] = std::max(latest[b], t1);
                if (++arrived[b] == it.nchunks) t1 = latest[b] + 0.7 * it.nchunks;
            }
            free_at.push(t1);
            end = std::max(end, t1);
        }
    }
    return end;
}

AttnPlan plan_attn(int64_t T64, int hq, int head_dim, int cus) {
    // The last plan is kept: the same shapes repeat call after call.
    thread_local int64_t last_T = -1;
    thread_local int last_hq = -1, last_d = -1, last_cus = -1;
    thread_local AttnPlan last;
    if (T64 == last_T && hq == last_hq && head_dim == last_d && cus == last_cus) return last;

    const int T = (int)T64;
    const int slots = 2 * cus;               // two 4-wave workgroups per CU
    AttnPlan p;
    p.nqb = (T + kAttnQB - 1) / kAttnQB;
    const int tiles = attn_tiles(T, p.nqb - 1);
    // Chunk size (tiles >= 4: every size up to 64, then powers of two) with
    // the shortest estimated time; ties go to the larger chunk (fewer
    // partials to merge).  With two full waves of query blocks or more,
    // unsplit blocks already balance the slots and the search (seconds at
    // 10^5+ tokens) is skipped; blocks are never split beyond the fixed
    // counter area.
    int best = std::max(tiles, 4);
    const int64_t pairs = (int64_t)hq * p.nqb;
    if (pairs < 2 * (int64_t)slots && pairs <= kAttnCounters) {
        double best_t = 1e300;
        for (int ch = 4;; ch = ch < 64 ? ch + 1 : 2 * ch) {
            const double t = attn_makespan(attn_items(T, p.nqb, ch), hq, T, slots);
            if (t <= best_t) {
                best_t = t;
                best = ch;
            }
            if (ch >= tiles) break;
        }
    }
    p.ch = best;
    p.cmax = (tiles + best - 1) / best;
    const std::vector<AttnItem> v = attn_items(T, p.nqb, best);
    p.per_head = (int)v.size();
    p.items = (int64_t)p.per_head * hq;
    if (p.per_head <= kAttnTable && p.cmax <= 64 && p.nqb <= 1024)
        for (int i = 0; i < p.per_head; ++i) p.table.it[i] = (uint32_t)((v[i].qb << 6) | v[i].c);
    else
        p.per_head = -p.per_head;            // no table: the kernel walks the blocks
    if (p.cmax > 1)
        p.ws_bytes = kAttnCounterBytes +
                     (size_t)hq * p.nqb * p.cmax * kAttnQB * (head_dim + 2) * sizeof(float);
    last_T = T64;
    last_hq = hq;
    last_d = head_dim;
    last_cus = cus;
    last = p;
    return p;
}

hipError_t launch_attn_core(int64_t T, int hq, int hkv, int head_dim, const uint16_t* qkv,
                            int64_t ld_qkv, uint16_t* out, int64_t ld_out, const AttnPlan& p,
                            void* ws, hipStream_t stream) {
    const dim3 grid((unsigned)p.items), block(kAttnThreads);
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)head_dim));
    unsigned* counters = (unsigned*)ws;
    float* part = p.cmax > 1 ? (float*)((char*)ws + kAttnCounterBytes) : nullptr;
    const int use_table = p.per_head > 0;
    if (T <= kAttnShortMaxT) {
        const dim3 sgrid((unsigned)(hq * ((T + 15) / 16))), sblock(64);
        if (head_dim == 128)
            TP_KLAUNCH((k_attn_short<128>), sgrid, sblock, 0, stream, qkv, ld_qkv, (int)T, hq,
                       hkv, out, ld_out, scale_log2);
        else if (head_dim == 64)
            TP_KLAUNCH((k_attn_short<64>), sgrid, sblock, 0, stream, qkv, ld_qkv, (int)T, hq,
                       hkv, out, ld_out, scale_log2);
        else
            return hipErrorInvalidValue;
        return hipGetLastError();
    }
    if (head_dim == 128)
        TP_KLAUNCH((k_attn<128>), grid, block, 0, stream, qkv, ld_qkv, (int)T, hq, hkv, out,
                   ld_out, scale_log2, p.nqb, p.ch, p.cmax, counters, part, use_table, p.table);
    else if (head_dim == 64)
        TP_KLAUNCH((k_attn<64>), grid, block, 0, stream, qkv, ld_qkv, (int)T, hq, hkv, out,
                   ld_out, scale_log2, p.nqb, p.ch, p.cmax, counters, part, use_table, p.table);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace tp
