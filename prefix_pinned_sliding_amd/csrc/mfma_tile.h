// Register and LDS helpers shared by the MFMA attention kernels (prefill and training).
//
// Layout of v_mfma_f32_16x16x32_bf16 on a wave of 64 lanes, l16 = lane % 16, lg = lane / 16:
// operand A (16 x 32): lane holds row l16, k = 8 lg .. 8 lg + 7;
// operand B (32 x 16): lane holds column l16, k = 8 lg .. 8 lg + 7;
// result (16 x 16): lane holds rows 4 lg .. 4 lg + 3 of column l16.
// The k order inside one instruction is free as long as A and B use the same one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace psa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNeg = -1.0e30f;        // initial running max (finite: -inf - kNeg = -inf)
__device__ constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& w) {
    return __builtin_bit_cast(bf16x8, w);
}

// Max over lanes l, l^16, l^32, l^48 (the four lane groups holding one row).
__device__ __forceinline__ float row_max4(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}
__device__ __forceinline__ float row_sum4(float x) {
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

// Column of a transposed tile for the first of 4 consecutive rows 4kq .. 4kq + 3. An
// accumulator block pair (rows 0..15 and 16..31 of a 32-row group) gives lane group g the
// rows 4g .. 4g + 3 and 16 + 4g .. 16 + 4g + 3; storing those 8 rows side by side at
// columns 8g .. 8g + 7 makes the matching operand one aligned 16-byte LDS read.
__device__ __forceinline__ int vt_col(int kq) {
    const int q = kq & 7;
    return 32 * (kq >> 3) + (q < 4 ? 8 * q : 8 * (q - 4) + 4);
}

// Store 4 rows x 8 columns (rows 4kq .. 4kq + 3, 16-byte chunk dc of each) transposed:
// 8 LDS rows (one per column) of 4 elements at vt_col(kq).
template <int VSTR>
__device__ __forceinline__ void store_transposed4(uint16_t* vt_s, int kq, int dc,
                                                  const u32x4* r) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const uint32_t a0 = r[0][x], a1 = r[1][x], a2 = r[2][x], a3 = r[3][x];
        u32x2 lo, hi;   // columns 2x (low halves) and 2x + 1 (high halves)
        lo[0] = __builtin_amdgcn_perm(a1, a0, 0x05040100u);
        lo[1] = __builtin_amdgcn_perm(a3, a2, 0x05040100u);
        hi[0] = __builtin_amdgcn_perm(a1, a0, 0x07060302u);
        hi[1] = __builtin_amdgcn_perm(a3, a2, 0x07060302u);
        const int d0 = dc * 8 + 2 * x;
        const int col = vt_col(kq);
        *reinterpret_cast<u32x2*>(vt_s + d0 * VSTR + col) = lo;
        *reinterpret_cast<u32x2*>(vt_s + (d0 + 1) * VSTR + col) = hi;
    }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposed MFMA operand from a row-major bf16 tile in LDS (ds_read_b64_tr_b16, gfx950).
// Within each 16-lane group the instruction takes the 16 lanes' 4-element reads as a 16 x 4
// tile T and hands lane i the elements T[i / 4 + 4 j][i % 4], j = 0..3. So if lane k of a
// group reads row r0 + k / 4 at column c0 + 4 (k % 4), lane i receives column c0 + i of
// rows r0 .. r0 + 3. Two reads (rows r0 .. r0 + 3 and r1 .. r1 + 3) fill the 8 k-values of
// one operand. `p0`, `p1`: this lane's addresses for the two reads (8-byte aligned).
__device__ __forceinline__ bf16x8 lds_read_tr2(const uint16_t* p0, const uint16_t* p1) {
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
    const s16x8 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, ab);
}

// Two bf16 values packed into one 32-bit word (first in the low half).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

}  // namespace
}  // namespace psa
