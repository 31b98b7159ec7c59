// Device helpers shared by the chunked GDN kernels: bf16 / fp32 MFMA wrappers, LDS transpose
// reads, the wave prefix sum of the gate cumsum, buffer resources and the workgroup barrier
// used for LDS hand-offs.
#pragma once

#include "internal.h"

namespace tr {
namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;                 // tokens per chunk
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16k32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// 16x16 products in two operand layouts: X in row layout (lane (m, g = l / 16) holds
// X[m][4g .. 4g+3]) and Y in accumulator layout (lane (n, g) holds Y[4g .. 4g+3][n]); X Y + C
// comes out in the accumulator layout.  With the operands swapped (Y's registers as X, X's as
// Y) the same call gives the product transposed, i.e. in row layout.
// The product is formed from bf16 hi / lo splits of both operands on 16x16x16 bf16 MFMA (the
// A and B operand layouts of that instruction are the row and accumulator layouts):
// X Y ~ Xhi Yhi + Xhi Ylo + Xlo Yhi, leaving out Xlo Ylo (about 2^-16 of |X| |Y| per term),
// small terms first.  Three 16x16x16 products instead of four fp32 16x16x4 ones.
// x ~ hi + lo for two values: hi = bf16(x), lo = bf16(x - hi).  x - hi is exact in fp32 (the
// rounding error of a rounding to fewer bits), so v_dot2_f32_bf16 of the packed hi pair with
// (-1, -0) or (-0, -1), accumulated onto x, forms it in one instruction instead of widening
// hi back to fp32 and subtracting; the result is the same bits.  The zero of each selector is
// -0 so that neither pair matches an inline constant: the compiler encodes (-1, +0) as the
// inline constant -1.0, which the hardware does not read as that bf16 pair (measured: every
// lane wrong), while literal selectors give x - hi exactly.
__device__ __forceinline__ void split2(float x0, float x1, bf16x2& hi, bf16x2& lo) {
    hi = bf16x2{(bf16)x0, (bf16)x1};
    const float r0 = __builtin_amdgcn_fdot2_f32_bf16(hi, bf16x2{(bf16)-1.f, (bf16)-0.f}, x0, false);
    const float r1 = __builtin_amdgcn_fdot2_f32_bf16(hi, bf16x2{(bf16)-0.f, (bf16)-1.f}, x1, false);
    lo = bf16x2{(bf16)r0, (bf16)r1};
}
__device__ __forceinline__ void split_bf4(const f32x4& x, bf16x4& hi, bf16x4& lo) {
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
        bf16x2 h, l;
        split2(x[i], x[i + 1], h, l);
        hi[i] = h[0]; hi[i + 1] = h[1];
        lo[i] = l[0]; lo[i + 1] = l[1];
    }
}
__device__ __forceinline__ f32x4 mm16x3(const f32x4& xrow, const f32x4& yacc, f32x4 c) {
    bf16x4 xh, xl, yh, yl;
    split_bf4(xrow, xh, xl);
    split_bf4(yacc, yh, yl);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xl, yh, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xh, yl, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xh, yh, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Within each 16-lane group, lane
// a + 4p supplies the address of row R_p, columns [X_a, X_a + 4) of a row-major tile
// (X_a may differ per a); lane 4a + b then receives column X_a + b at rows R_0..R_3.
__device__ __forceinline__ bf16x4 lds_tr4(const bf16* p) {
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p));
    return __builtin_bit_cast(bf16x4, r);
}
__device__ __forceinline__ bf16x8 cat(const bf16x4& lo, const bf16x4& hi) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) { r[i] = lo[i]; r[4 + i] = hi[i]; }
    return r;
}
__device__ __forceinline__ bf16x4 to_bf4(const f32x4& x, float sign) {
    bf16x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (bf16)(sign * x[i]);
    return r;
}

// Workgroup barrier for LDS hand-offs only.  __syncthreads() would also wait for every
// outstanding global load, including the next chunk's prefetch issued just before it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts, then row broadcasts).
__device__ __forceinline__ float wave_prefix_sum(float x) {
    float y;
    y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xf, 0xf, false));
    x += y;   // row_shr:1
    y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xf, 0xf, false));
    x += y;   // row_shr:2
    y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xf, 0xf, false));
    x += y;   // row_shr:4
    y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xf, 0xf, false));
    x += y;   // row_shr:8
    y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x142, 0xa, 0xf, false));
    x += y;   // row_bcast:15 into rows 1 and 3
    y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x143, 0xc, 0xf, false));
    x += y;   // row_bcast:31 into rows 2 and 3
    return x;
}

// Four consecutive table entries starting at a multiple of 4.
__device__ __forceinline__ f32x4 tab4(const float* t, int i) { return *reinterpret_cast<const f32x4*>(t + i); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Sequence at longest-first rank `rank`: the order travels as the kernel's first argument and
// is read through the kernel-argument segment (indexing the by-value argument with a variable
// would copy it to scratch memory).
__device__ __forceinline__ int seq_at(int rank) {
    typedef const __attribute__((address_space(4))) uint16_t kshort;
    return ((kshort*)__builtin_amdgcn_kernarg_segment_ptr())[rank];
}

}  // namespace gdn
}  // namespace tr
