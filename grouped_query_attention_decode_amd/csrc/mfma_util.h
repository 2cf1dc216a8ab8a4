// gfx950 matrix-core and LDS helpers shared by the decode and prefill kernels.
//
// Lane layouts (wave64), as the hardware defines them:
//  v_mfma_f32_16x16x32_bf16  A (16x32): lane l holds A[l%16][8*(l/16) .. +7]
//                            B (32x16): lane l holds B[8*(l/16) .. +7][l%16]
//                            C (16x16): lane l holds C[4*(l/16) + i][l%16], i = 0..3
//  ds_read_b64_tr_b16        per 16-lane group, lane j supplies the address of a row of
//                            four 16-bit values M[j][0..3]; lane i receives
//                            M[4k + i/4][i%4] for k = 0..3.
//  ds_read_b64_tr_b8         same with eight 8-bit values: lane i receives
//                            M[2k + i/8][i%8] for k = 0..7.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4_t;

#define GQA_LDS(T, p) ((__attribute__((address_space(3))) T *)(p))

__device__ __forceinline__ f32x4_t mfma16x16x32(const i32x4_t &a, const i32x4_t &b, const f32x4_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// Two transposed 4 x b16 reads make one 8 x bf16 MFMA operand.
__device__ __forceinline__ i32x2_t lds_read_tr16(const void *p) {
    return __builtin_bit_cast(i32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(GQA_LDS(i16x4_t, p)));
}

__device__ __forceinline__ i32x2_t lds_read_tr8(const void *p) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32(GQA_LDS(i32x2_t, p));
}

// Eight E4M3FN codes (byte k of the pair of dwords = element k) -> eight exact bf16, two per
// v_cvt_scalef32_pk_bf16_fp8 with scale 1 (every E4M3FN value, subnormals included, is a bf16
// value; checked bit for bit against the fp32 conversion for all 256 codes in every byte
// position).
__device__ __forceinline__ i32x4_t e4m3x8_to_bf16x8(i32x2_t c) {
    i32x4_t r;
    r[0] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], 1.0f, false));
    r[1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], 1.0f, true));
    r[2] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], 1.0f, false));
    r[3] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], 1.0f, true));
    return r;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2v_t __attribute__((ext_vector_type(2)));

// Round-to-nearest-even packing of two binary32 values into a bf16 pair
// (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ int pack_bf16_rne(float lo, float hi) {
    const f32x2v_t v = {lo, hi};
    return __builtin_bit_cast(int, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over lane pairs (l, l ^ 16) and (l, l ^ 32), result in every lane. One
// v_permlane16_swap / v_permlane32_swap called with the same value in both operands leaves x
// of the partner lane in one of its two outputs and x of the lane itself in the other, so
// combining the two outputs is the pair reduction: a VALU operation instead of an LDS lane
// shuffle on the softmax's dependency chain.
__device__ __forceinline__ float max_xor16(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// DPP lane move (a VALU operand modifier, no LDS round trip): quad_perm within groups of four
// lanes (0xB1: lane ^ 1, 0x4E: lane ^ 2) and row_ror within rows of 16 (0x124: by 4, 0x128: by 8).
template <int CTRL> __device__ __forceinline__ int dpp_move(int x) {
    return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}

}  // namespace gqa
