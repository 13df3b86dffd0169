// Rotary helpers. Stored keys: the float64 rotation at an absolute position and the single
// rounding to the storage type; the append kernel and the prefill staging kernel both use
// these, so a chunk's keys attended by prefill are byte-identical to the keys the cache
// then holds. Queries (never stored): a float32 rotation of a float64-reduced angle, used
// by the decode and prefill attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace psa {

__device__ __forceinline__ double bf16_bits_to_f64(uint16_t b) {
    return (double)__uint_as_float((uint32_t)b << 16);
}

// float64 -> bfloat16 bits, one rounding to nearest, ties to even, on the float64 bit
// fields: results below 2^-126 become bfloat16 subnormals, a carry out of the fraction
// bumps the exponent, overflow gives infinity, NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f64_to_bf16_bits(double x) {
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
    const int e = (int)((u >> 52) & 0x7FF);
    const uint64_t frac = u & ((1ull << 52) - 1);
    if (e == 0x7FF) return sign | (frac ? 0x7FC0 : 0x7F80);
    if (e == 0) return sign;                       // float64 zero or subnormal
    const int E = e - 1023;
    if (E >= -126) {
        uint64_t body = ((uint64_t)(E + 127) << 7) | (frac >> 45);
        const uint64_t rem = frac & ((1ull << 45) - 1);
        const uint64_t half = 1ull << 44;
        if (rem > half || (rem == half && (body & 1ull))) ++body;
        if (body >= 0x7F80ull) body = 0x7F80ull;
        return sign | (uint16_t)body;
    }
    const int sh = -E - 81;                        // leaves units of 2^-133
    if (sh >= 64) return sign;
    const uint64_t full = frac | (1ull << 52);
    uint64_t kept = full >> sh;
    const uint64_t rem = full & ((1ull << sh) - 1);
    const uint64_t half = 1ull << (sh - 1);
    if (rem > half || (rem == half && (kept & 1ull))) ++kept;
    return sign | (uint16_t)kept;
}

// sin and cos of the angle p * theta, the angle rounded once in float64.
__device__ __forceinline__ void angle_sincos(int p, double theta, double* sn, double* cs) {
#pragma clang fp contract(off)
    const double phi = (double)p * theta;
    sincos(phi, sn, cs);
}

// Rotate the pair (x, y) by an angle with sine sn and cosine cs in float64:
// (x c - y s, x s + y c), each product and each sum rounded on its own (no fused
// multiply-add).
__device__ __forceinline__ void rotate_with(double x, double y, double sn, double cs, double* xr,
                                            double* yr) {
#pragma clang fp contract(off)
    const double a = x * cs;
    const double b = y * sn;
    const double c = x * sn;
    const double d = y * cs;
    *xr = a - b;
    *yr = c + d;
}

// Rotated, scaled query pair for position p (fp32 result). The angle p * theta_i is formed
// and reduced modulo 2*pi in float64, then sin/cos are taken in float32: queries are never
// stored, so float32 accuracy (~1e-7 relative) is all the logits need.
__device__ __forceinline__ void rotate_query(float x, float y, int p, double theta, float sc,
                                             float* xr, float* yr) {
    const double phi = (double)p * theta;
    const double two_pi = 6.283185307179586;
    const double r = phi - two_pi * rint(phi * (1.0 / two_pi));
    float sn, cs;
    sincosf((float)r, &sn, &cs);
    *xr = (x * cs - y * sn) * sc;
    *yr = (x * sn + y * cs) * sc;
}

// The same rotation for queries that are rounded to bf16 afterwards (prefill): the angle is
// reduced to a fraction of a turn in [-1/2, 1/2] in float64 and sin/cos come from the
// hardware's sin(2 pi x) and cos(2 pi x) (absolute error of order 1e-6, far below the
// bf16 rounding that follows).
__device__ __forceinline__ void rotate_query_bf16(float x, float y, int p, double theta, float sc,
                                                  float* xr, float* yr) {
    const double turns = (double)p * theta * 0.15915494309189535;   // 1 / (2 pi)
    const float fr = (float)(turns - rint(turns));
    const float sn = __builtin_amdgcn_sinf(fr), cs = __builtin_amdgcn_cosf(fr);
    *xr = (x * cs - y * sn) * sc;
    *yr = (x * sn + y * cs) * sc;
}

}  // namespace psa
