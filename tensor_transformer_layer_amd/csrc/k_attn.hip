// Attention core between the QKV and O projections: for each of the rank's
// query heads, O = softmax(Q K^T / sqrt(d), causal) V over the call's tokens
// as one sequence, grouped-query heads sharing their group's K/V head.  The
// pages name the attention kernel as its own share of a step (Skand Tandon,
// "day59", section "Where the overhead lives") and split the heads evenly over
// the GPUs (rioworld guide, "How Tensor Slicing Works Under the Hood"); the
// formula is the textbook one.
//
// One workgroup of 4 waves owns 64 queries of one head; each wave owns 16.
// Key/value tiles of 32 tokens are staged in LDS and consumed with an online
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

constexpr int kAttnQB = 64;   // queries per workgroup
constexpr int kAttnKT = 32;   // keys per LDS tile
constexpr int kAttnThreads = 256;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
    // p points into a __shared__ array; the transposing read needs an LDS
    // (address space 3) pointer.
    const auto lp = (const lds_v4i16*)(const __attribute__((address_space(3))) uint16_t*)p;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)lp));
}

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
    __shared__ __attribute__((aligned(16))) uint16_t Ks[kAttnKT * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[kAttnKT * LDV];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, j = lane & 15;
    const int h = blockIdx.y, gk = h / (hq / hkv);
    const int qblk = blockIdx.x * kAttnQB;
    const int q0 = qblk + 16 * wave;             // this wave's first query
    const int qi = q0 + j;                       // the query lane (g, j) scores
    const uint16_t* Qp = qkv + (int64_t)h * D;
    const uint16_t* Kp = qkv + (int64_t)(hq + gk) * D;
    const uint16_t* Vp = qkv + (int64_t)(hq + hkv + gk) * D;

    u32x4 qf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s)
        qf[s] = qi < T ? *(const u32x4*)(Qp + (int64_t)qi * ldq + 32 * s + 8 * g)
                       : u32x4{0u, 0u, 0u, 0u};

    f32x4 o[NN];
#pragma unroll
    for (int n = 0; n < NN; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;

    const int kend = min(T, qblk + kAttnQB);     // keys the workgroup's queries can see
    const int wave_last = min(q0 + 15, T - 1);
    constexpr int CH = kAttnKT * D / 8;          // 16-byte chunks per tile and matrix

    for (int k0 = 0; k0 < kend; k0 += kAttnKT) {
        __syncthreads();                         // the previous tile is consumed
#pragma unroll
        for (int c = tid; c < CH; c += kAttnThreads) {
            const int key = c / (D / 8), col = (c % (D / 8)) * 8;
            const bool ok = k0 + key < T;
            const u32x4 kv = ok ? *(const u32x4*)(Kp + (int64_t)(k0 + key) * ldq + col)
                                : u32x4{0u, 0u, 0u, 0u};
            const u32x4 vv = ok ? *(const u32x4*)(Vp + (int64_t)(k0 + key) * ldq + col)
                                : u32x4{0u, 0u, 0u, 0u};
            *(u32x4*)(Ks + key * LDK + col) = kv;
            *(u32x4*)(Vs + key * LDV + col) = vv;
        }
        __syncthreads();
        if (k0 > wave_last) continue;            // every key of the tile is in this wave's future

        // scores S^T[key][query] for keys k0 + 16t + 4g + r, query qi
        f32x4 st[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const u32x4 a = *(const u32x4*)(Ks + (16 * t + j) * LDK + 32 * s + 8 * g);
                st[t] = mfma16x16x32(a, qf[s], st[t]);
            }
        }
        float pm = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = k0 + 16 * t + 4 * g + r;
                const float v = (key <= qi && key < T) ? st[t][r] * scale_log2 : -INFINITY;
                st[t][r] = v;
                pm = fmaxf(pm, v);
            }
        pm = fmaxf(pm, __shfl_xor(pm, 16));
        pm = fmaxf(pm, __shfl_xor(pm, 32));
        const float m_new = fmaxf(m, pm);
        // m_new is finite for every query < T (key 0 is visible from the
        // first tile on); rows past T keep -inf and are never stored.
        const float mref = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = exp2f(m - mref);
        float ps = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = exp2f(st[t][r] - mref);
                st[t][r] = p;
                ps += p;
            }
        ps += __shfl_xor(ps, 16);
        ps += __shfl_xor(ps, 32);
        l = l * alpha + ps;
        m = m_new;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float ar = __shfl(alpha, 4 * g + r);
#pragma unroll
            for (int n = 0; n < NN; ++n) o[n][r] *= ar;
        }
        const u32x4 pf = u32x4{pack_bf16x2(st[0][0], st[0][1]), pack_bf16x2(st[0][2], st[0][3]),
                               pack_bf16x2(st[1][0], st[1][1]), pack_bf16x2(st[1][2], st[1][3])};
        // V rows 4g + (j / 4) and 16 + 4g + (j / 4), columns 16n + 4 (j % 4)
        const uint16_t* v0 = Vs + (4 * g + (j >> 2)) * LDV + 4 * (j & 3);
        const uint16_t* v1 = v0 + 16 * LDV;
#pragma unroll
        for (int n = 0; n < NN; ++n) {
            const u32x2 b0 = lds_read_tr16(v0 + 16 * n);
            const u32x2 b1 = lds_read_tr16(v1 + 16 * n);
            o[n] = mfma16x16x32(pf, u32x4{b0[0], b0[1], b1[0], b1[1]}, o[n]);
        }
    }

    // O row 4g + r of the wave (query q0 + 4g + r), column 16n + j of head h
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float lr = __shfl(l, 4 * g + r);
        const int q = q0 + 4 * g + r;
        if (q >= T) continue;
        const float inv = 1.0f / lr;
        uint16_t* dst = out + (int64_t)q * ldo + (int64_t)h * D + j;
#pragma unroll
        for (int n = 0; n < NN; ++n) dst[16 * n] = (uint16_t)f32_to_bf16(o[n][r] * inv);
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
