// Device-side element conversions used by the kernels of libgqa.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

// bf16 is the upper half of an IEEE binary32: widening is a shift.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// binary32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// OCP E4M3FN -> binary32, exact. Layout s.eeee.mmm, exponent bias 7; exponent field 0
// holds subnormals m * 2^-9; s.1111.111 is NaN; there are no infinities.
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t c) {
    const uint32_t sign = (c & 0x80u) << 24;
    const uint32_t e = (c >> 3) & 0xFu;
    const uint32_t m = c & 0x7u;
    if (e == 0xFu && m == 0x7u) return __uint_as_float(0x7fc00000u | sign);
    if (e == 0u) {
        const float mag = (float)m * 0.001953125f;  // m * 2^-9
        return sign ? -mag : mag;
    }
    return __uint_as_float(sign | ((e + 120u) << 23) | (m << 20));  // rebias 7 -> 127
}

// Two INT4 fields in one byte (low four bits: the even element); field u stands for u - 8.
struct I4x2 {
    uint8_t b;
};

template <int KVT> struct KvElem;
template <> struct KvElem<0> { using T = float; };
template <> struct KvElem<1> { using T = uint16_t; };
template <> struct KvElem<2> { using T = uint8_t; };
template <> struct KvElem<3> { using T = I4x2; };

// Cache append for fp8 slabs with a fixed scale: the E4M3FN code of the fp32 quotient x / scale,
// magnitudes beyond the largest code (448) saturated, NaN to the NaN code 0x7F; the hardware
// conversion rounds to nearest, ties to even (it gives 0xFF for every NaN, so those bytes are
// replaced). Packs four codes (byte i = code of x[i]).
__device__ __forceinline__ uint32_t quant_e4m3fn_x4(float x0, float x1, float x2, float x3, float scale) {
    const float q0 = x0 / scale, q1 = x1 / scale, q2 = x2 / scale, q3 = x3 / scale;
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(q0, -448.f), 448.f), fminf(fmaxf(q1, -448.f), 448.f),
                                                   0, false);  // bytes 0, 1
    const uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(q2, -448.f), 448.f),
                                                                 fminf(fmaxf(q3, -448.f), 448.f), lo, true);  // bytes 2, 3
    const uint32_t nan = (q0 != q0 ? 0xFFu : 0u) | (q1 != q1 ? 0xFF00u : 0u) | (q2 != q2 ? 0xFF0000u : 0u) |
                         (q3 != q3 ? 0xFF000000u : 0u);
    return (c & ~nan) | (0x7F7F7F7Fu & nan);
}

__device__ __forceinline__ float load_f32(const float *p, long i) { return p[i]; }
__device__ __forceinline__ float load_f32(const uint16_t *p, long i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float load_f32(const uint8_t *p, long i) { return e4m3fn_to_f32(p[i]); }
// Element i of a packed INT4 array (in units of its scale).
__device__ __forceinline__ float load_f32(const I4x2 *p, long i) {
    const uint32_t byte = p[i >> 1].b;
    return (float)((int)((i & 1) ? byte >> 4 : byte & 15u) - 8);
}

// INT4 field of the fp32 quotient x / scale: nearest integer, ties to even (the default
// rounding of rintf), clamped to -8 .. 7, plus 8; NaN stores the field of 0.
__device__ __forceinline__ uint32_t quant_int4(float x, float scale) {
    const float q = x / scale;
    if (q != q) return 8u;
    return (uint32_t)((int)fminf(fmaxf(rintf(q), -8.f), 7.f) + 8);
}

__device__ __forceinline__ void store_f32(float *p, long i, float x) { p[i] = x; }
__device__ __forceinline__ void store_f32(uint16_t *p, long i, float x) { p[i] = f32_to_bf16(x); }

}  // namespace gqa
