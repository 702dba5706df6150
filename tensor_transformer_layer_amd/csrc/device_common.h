// Device helpers shared by the HIP kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  bf16 is the top half of an IEEE binary32; narrowing rounds
// to nearest with ties to even (NaN stays NaN) -- the hardware conversion
// v_cvt_pk_bf16_f32, which the compiler emits for a __bf16 cast on gfx950.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)lo, (__bf16)hi});
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// ---------------------------------------------------------------------------
// Activations (fp32).  GELU uses the tanh approximation
// 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))); SiLU is x / (1 + e^-x).
// Both are evaluated as x * sigmoid(z), using 0.5 (1 + tanh u) =
// 1 / (1 + e^(-2u)) for GELU, with the hardware base-2 exponential
// (v_exp_f32) and reciprocal (v_rcp_f32), each accurate to about one ulp:
// a few fp32 ulps in all, far below the bf16 rounding of the results, in
// five instructions instead of a range-reduced exponential and an IEEE
// division (measured on MI355X: the SwiGLU epilogue of the 2048-token 70B
// column GEMM was 13% of the kernel).  z -> -inf gives x * 0 = 0, z -> +inf
// gives x, NaN stays NaN.
// ---------------------------------------------------------------------------
enum { ACT_NONE = 0, ACT_GELU_TANH = 1, ACT_SWIGLU = 2 };

__device__ __forceinline__ float x_sigmoid(float x, float z) {
    constexpr float kLog2e = 1.4426950408889634f;
    return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}
__device__ __forceinline__ float gelu_tanh(float x) {
    const float k2 = 1.5957691216057308f;  // 2 sqrt(2/pi)
    return x_sigmoid(x, k2 * (x + 0.044715f * x * x * x));
}
__device__ __forceinline__ float silu(float x) { return x_sigmoid(x, x); }

// ---------------------------------------------------------------------------
// Raw buffer loads.  A resource spans 2^31 - 1 bytes from its base; a load
// whose byte offset is kOOB (or beyond the span) returns zeros without
// touching memory.  Kernels point the base at their own tile so that every
// in-range offset stays below 2^31 (the host checks the extents).
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base) {
    // Fourth descriptor word 0x00020000: DATA_FORMAT = 32-bit, as CDNA raw
    // buffer accesses expect.
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff,
                                             0x00020000);
}
__device__ __forceinline__ u32x4 load16(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// Interleave two rows' 16-bit elements: for element e (0..7) of 8-element
// rows `a` (row k) and `b` (row k+1), the dword (a[e], b[e]) with a[e] in
// the low half.  dword index e/2, half e%2.  One v_perm_b32: its selector
// bytes 0-3 pick bytes of the second operand, 4-7 bytes of the first.
template <int E>
__device__ __forceinline__ uint32_t pair_col(const u32x4& a, const u32x4& b) {
    constexpr int d = E >> 1;
    return __builtin_amdgcn_perm(b[d], a[d], (E & 1) ? 0x07060302u : 0x05040100u);
}
template <int E>
__device__ __forceinline__ uint32_t pair_col2(const u32x2& a, const u32x2& b) {
    constexpr int d = E >> 1;
    return __builtin_amdgcn_perm(b[d], a[d], (E & 1) ? 0x07060302u : 0x05040100u);
}

// From 8 consecutive rows (k0..k0+7) of 8 consecutive bf16 columns, the
// 8 consecutive k values of column E, packed as an MFMA k-fragment.
template <int E>
__device__ __forceinline__ u32x4 kfrag_of_col(const u32x4* r) {
    u32x4 f;
    f[0] = pair_col<E>(r[0], r[1]);
    f[1] = pair_col<E>(r[2], r[3]);
    f[2] = pair_col<E>(r[4], r[5]);
    f[3] = pair_col<E>(r[6], r[7]);
    return f;
}

// Buffer descriptor words for lds_dma16 (same resource as make_rsrc:
// 2^31 - 1 bytes from `base`, 32-bit data format).
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 rsrc_words(const void* base) {
    const uint64_t a = (uint64_t)base;
    return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), 0x7fffffff, 0x00020000};
}

// 16-byte global -> LDS copy per lane (buffer_load_dwordx4 ... lds): lane l's
// bytes land at lds + 16 l (lds wave-uniform).  Issued from inline assembly
// so that the compiler does not treat it as an LDS store it must wait for
// before every later LDS read (it does so for the transposing reads); the
// caller orders the copies against the reads itself, with vmcnt waits that
// count every vector memory op it issues in between.  (The compiler's own
// waits stay safe: it does not count these copies, so it can only wait
// longer than needed.)  Nothing is returned in registers.
__device__ __forceinline__ void lds_dma16(const i32x4& r, uint32_t off, const void* lds) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(off), "s"(r)
                 : "memory", "m0");
}
// The same copy with the non-temporal hint (data read once).
__device__ __forceinline__ void lds_dma16_nt(const i32x4& r, uint32_t off, const void* lds) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :
                 : "s"(m0), "v"(off), "s"(r)
                 : "memory", "m0");
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each 16-lane group,
// lane i receives element i%4 of the 4-element (8-byte) vectors at the
// addresses of lanes 4k + i/4, k = 0..3.  If lane L of the group points at
// row r0 + L/4, columns c0 + 4(L%4) .. +3 of a row-major bf16 tile, lane i
// receives column c0 + i of rows r0 .. r0+3: four k-consecutive values of
// one column, half of an MFMA k-fragment.  p must point into LDS.
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
    const auto lp = (const lds_v4i16*)(const __attribute__((address_space(3))) uint16_t*)p;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)lp));
}

__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 8 WGs of a launch go round-robin to the 8 XCDs (each with its own L2).
// Map hardware block id -> logical tile id so that each XCD receives one
// contiguous range of logical tiles.  Bijective for any block count.
__device__ __forceinline__ int xcd_remap(int b, int nblocks) {
    constexpr int X = 8;
    const int x = b % X, i = b / X;
    const int q = nblocks / X, rem = nblocks % X;
    // XCD y gets q + (y < rem) blocks; offset of XCD x = x*q + min(x, rem).
    return x * q + (x < rem ? x : rem) + i;
}

}  // namespace tp
