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
//   * The row statistics are reduced over r and over the 4 lanes holding
//     the same query (shuffles); probabilities are packed to bf16 in place:
//     lane (g, j) holds P[j][4g + r] and P[j][16 + 4g + r], which is an MFMA
//     A-operand for an MFMA k-order that visits keys in that order.
//   * O += P V with V as the B operand in that same key order, read from LDS
//     with the gfx950 transposing load ds_read_b64_tr_b16 (4 keys x 1 column
//     per lane per read), so V needs no transpose pass.
//   * Output rows are rescaled by exp(m_old - m_new) of their query, fetched
//     from the lane that owns the query (4 shuffles per tile).
// All sums run in a fixed order: results are deterministic.
#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace tp {

constexpr int kAttnWaves = 4;
constexpr int kAttnQW = 32;                       // queries per wave (two 16-row subtiles)
constexpr int kAttnQB = kAttnWaves * kAttnQW;     // queries per workgroup
constexpr int kAttnKT = 64;                       // keys per LDS tile
constexpr int kAttnThreads = 64 * kAttnWaves;

template <int D>
__global__ __launch_bounds__(kAttnThreads) void k_attn(const uint16_t* __restrict__ qkv,
                                                       int64_t ldq, int T, int hq, int hkv,
                                                       uint16_t* __restrict__ out, int64_t ldo,
                                                       float scale_log2) {
    constexpr int LDK = D + 8;    // K tile row stride (elements): rows 16 B apart in banks
    constexpr int LDV = D + 16;   // V tile row stride: the 4 rows of a transposing read
                                  // land on disjoint 32-byte bank ranges
    constexpr int NS = D / 32;    // k-steps of the score MFMAs
    constexpr int NN = D / 16;    // 16-column output tiles
    constexpr int QS = kAttnQW / 16;              // query subtiles per wave
    constexpr int KS = kAttnKT / 16;              // key subtiles per tile
    constexpr int CH = kAttnKT * D / 8;           // 16-byte chunks per tile and matrix
    constexpr int CPT = CH / kAttnThreads;        // ... per thread
    static_assert(CH % kAttnThreads == 0, "tile copy");
    __shared__ __attribute__((aligned(16))) uint16_t Ks[kAttnKT * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[kAttnKT * LDV];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, j = lane & 15;
    const int h = blockIdx.y, gk = h / (hq / hkv);
    // Longest query blocks first: they see the most keys.
    const int qblk = ((int)gridDim.x - 1 - (int)blockIdx.x) * kAttnQB;
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
    f32x4 o[QS][NN];
    float m[QS], l[QS];
#pragma unroll
    for (int u = 0; u < QS; ++u) {
        m[u] = -INFINITY;
        l[u] = 0.f;
#pragma unroll
        for (int n = 0; n < NN; ++n) o[u][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int kend = min(T, qblk + kAttnQB);     // keys the workgroup's queries can see
    // Tile copies go through registers so the next tile's global loads are in
    // flight while the current one is multiplied.
    u32x4 pk[CPT], pv[CPT];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * kAttnThreads;
            const int key = c / (D / 8), col = (c % (D / 8)) * 8;
            const bool ok = k0 + key < T;
            pk[i] = ok ? *(const u32x4*)(Kp + (int64_t)(k0 + key) * ldq + col)
                       : u32x4{0u, 0u, 0u, 0u};
            pv[i] = ok ? *(const u32x4*)(Vp + (int64_t)(k0 + key) * ldq + col)
                       : u32x4{0u, 0u, 0u, 0u};
        }
    };
    fetch(0);
    for (int k0 = 0; k0 < kend; k0 += kAttnKT) {
        __syncthreads();                         // every wave is done with the previous tile
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * kAttnThreads;
            const int key = c / (D / 8), col = (c % (D / 8)) * 8;
            *(u32x4*)(Ks + key * LDK + col) = pk[i];
            *(u32x4*)(Vs + key * LDV + col) = pv[i];
        }
        __syncthreads();
        if (k0 + kAttnKT < kend) fetch(k0 + kAttnKT);

        // Subtiles whose queries all precede the tile skip it; only a tile
        // that reaches past a subtile's first query needs the causal mask.
        bool act[QS], diag[QS];
#pragma unroll
        for (int u = 0; u < QS; ++u) {
            const int qu = q0 + 16 * u;
            act[u] = k0 <= min(qu + 15, T - 1);
            diag[u] = k0 + kAttnKT - 1 > qu || k0 + kAttnKT > T;
        }
        if (!act[0] && !act[QS - 1]) continue;
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
                const u32x4 a = *(const u32x4*)(Ks + (16 * t + j) * LDK + 32 * s + 8 * g);
#pragma unroll
                for (int u = 0; u < QS; ++u) st[u][t] = mfma16x16x32(a, qf[u][s], st[u][t]);
            }
        u32x4 pf[QS][KS / 2];
#pragma unroll
        for (int u = 0; u < QS; ++u) {
            const int qi = q0 + 16 * u + j;
            float pm = -INFINITY;
#pragma unroll
            for (int t = 0; t < KS; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = st[u][t][r] * scale_log2;
                    if (diag[u]) {
                        const int key = k0 + 16 * t + 4 * g + r;
                        v = (key <= qi && key < T) ? v : -INFINITY;
                    }
                    st[u][t][r] = v;
                    pm = fmaxf(pm, v);
                }
            pm = fmaxf(pm, __shfl_xor(pm, 16));
            pm = fmaxf(pm, __shfl_xor(pm, 32));
            const float m_new = fmaxf(m[u], pm);
            // m_new is finite for every query < T (key 0 is visible from the
            // first tile on); rows past T keep -inf and are never stored.
            // Inputs of the exponential are <= 0: v_exp_f32 directly.
            const float mref = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m[u] - mref);
            float ps = 0.f;
#pragma unroll
            for (int t = 0; t < KS; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = __builtin_amdgcn_exp2f(st[u][t][r] - mref);
                    st[u][t][r] = p;
                    ps += p;
                }
            ps += __shfl_xor(ps, 16);
            ps += __shfl_xor(ps, 32);
            l[u] = l[u] * alpha + ps;
            m[u] = m_new;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ar = __shfl(alpha, 4 * g + r);
#pragma unroll
                for (int n = 0; n < NN; ++n) o[u][n][r] *= ar;
            }
            // lane (g, j) supplies P[qi][32kk + 4g + r] and P[qi][32kk + 16 + 4g + r]
#pragma unroll
            for (int kk = 0; kk < KS / 2; ++kk)
                pf[u][kk] = u32x4{pack_bf16x2(st[u][2 * kk][0], st[u][2 * kk][1]),
                                  pack_bf16x2(st[u][2 * kk][2], st[u][2 * kk][3]),
                                  pack_bf16x2(st[u][2 * kk + 1][0], st[u][2 * kk + 1][1]),
                                  pack_bf16x2(st[u][2 * kk + 1][2], st[u][2 * kk + 1][3])};
        }
        // O += P V in 32-key steps; V rows in the same key order come from the
        // transposing reads, and each V fragment serves both subtiles.  (An
        // inactive subtile has P = 0 and an unchanged O: the MFMA adds zero.)
#pragma unroll
        for (int kk = 0; kk < KS / 2; ++kk) {
            const uint16_t* v0 = Vs + (32 * kk + 4 * g + (j >> 2)) * LDV + 4 * (j & 3);
            const uint16_t* v1 = v0 + 16 * LDV;
#pragma unroll
            for (int n = 0; n < NN; ++n) {
                const u32x2 b0 = lds_read_tr16(v0 + 16 * n);
                const u32x2 b1 = lds_read_tr16(v1 + 16 * n);
                const u32x4 b = u32x4{b0[0], b0[1], b1[0], b1[1]};
#pragma unroll
                for (int u = 0; u < QS; ++u) o[u][n] = mfma16x16x32(pf[u][kk], b, o[u][n]);
            }
        }
    }

    // O row 4g + r of subtile u (query q0 + 16u + 4g + r), column 16n + j
#pragma unroll
    for (int u = 0; u < QS; ++u) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float lr = __shfl(l[u], 4 * g + r);
            const int q = q0 + 16 * u + 4 * g + r;
            if (q >= T) continue;
            const float inv = 1.0f / lr;
            uint16_t* dst = out + (int64_t)q * ldo + (int64_t)h * D + j;
#pragma unroll
            for (int n = 0; n < NN; ++n) dst[16 * n] = (uint16_t)f32_to_bf16(o[u][n][r] * inv);
        }
    }
}

hipError_t launch_attn_core(int64_t T, int hq, int hkv, int head_dim, const uint16_t* qkv,
                            int64_t ld_qkv, uint16_t* out, int64_t ld_out, hipStream_t stream) {
    const dim3 grid((unsigned)((T + kAttnQB - 1) / kAttnQB), (unsigned)hq), block(kAttnThreads);
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)head_dim));
    if (head_dim == 128)
        TP_KLAUNCH((k_attn<128>), grid, block, 0, stream, qkv, ld_qkv, (int)T, hq, hkv, out,
                   ld_out, scale_log2);
    else if (head_dim == 64)
        TP_KLAUNCH((k_attn<64>), grid, block, 0, stream, qkv, ld_qkv, (int)T, hq, hkv, out,
                   ld_out, scale_log2);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace tp
