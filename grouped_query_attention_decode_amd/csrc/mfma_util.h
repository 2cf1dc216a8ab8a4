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

// Upper halves of two binary32 values as one packed bf16 pair (exact when the low 16
// bits are zero, as for every value widened from E4M3FN).
__device__ __forceinline__ int pack_hi16(float lo, float hi) {
    return (int)__builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Eight E4M3FN codes (byte k of the pair of dwords = element k) -> eight exact bf16.
__device__ __forceinline__ i32x4_t e4m3x8_to_bf16x8(i32x2_t c) {
    const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(c[0], false);
    const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8(c[0], true);
    const f32x2_t d = __builtin_amdgcn_cvt_pk_f32_fp8(c[1], false);
    const f32x2_t e = __builtin_amdgcn_cvt_pk_f32_fp8(c[1], true);
    i32x4_t r;
    r[0] = pack_hi16(a[0], a[1]);
    r[1] = pack_hi16(b[0], b[1]);
    r[2] = pack_hi16(d[0], d[1]);
    r[3] = pack_hi16(e[0], e[1]);
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

}  // namespace gqa
