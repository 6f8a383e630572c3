// MXFP8 block codec on the device: E8M0 block scales and E4M3 elements.
//
// [NVIDIA CuTe DSL fusion-kernel page, problem and core-idea sections: BF16
// activations become MXFP8 plus a transposed copy; Transformer Engine page,
// three-components section: group-aware MXFP8 quantization.] The pages give
// no encoding rule; the OCP Microscaling (MX) v1.0 formats are used with the
// scale rounded up (as the Transformer Engine MXFP8 recipe does): a block of
// 32 elements shares the smallest exponent e with amax <= 448 * 2^e, clamped
// to [-127, 127], stored as E8M0 (e + 127); an all-zero block takes code 0.
// Elements are v / 2^e in E4M3 (1-4-3, bias 7, no infinities), rounded to
// nearest-even (saturation to +-448 is kept as a guard); the sign of zero is
// kept.
#pragma once

#include "common.hpp"

namespace moe {

// Block exponent from the bf16 bit pattern of the block's largest magnitude.
// amax = (1 + M/128) * 2^(E-127): e = E - 127 - 8, plus one when the
// significand exceeds 1.75 (M > 96), since 448 = 1.75 * 2^8.
__device__ __forceinline__ int mx_block_exp(uint32_t amax_bits) {
    const int E = (int)(amax_bits >> 7) & 0xff;
    if (E == 0) return -127;  // zero or subnormal maximum: the clamp bound
    const int e = E - 127 - 8 + ((amax_bits & 0x7fu) > 96u ? 1 : 0);
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^-e as an fp32 value, e in [-127, 120] (the range mx_block_exp yields for
// finite bf16 input).
__device__ __forceinline__ float mx_inv_scale(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// E4M3 code of y (round to nearest-even, saturating to 448, sign kept).
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    const int ex = (int)(a >> 23) - 127;
    if (ex < -10) return sign;  // |y| < 2^-10 rounds to zero
    const uint32_t m = (a & 0x7fffffu) | 0x800000u;  // 24-bit significand
    if (ex >= -6) {                                     // E4M3 normal range
        uint32_t q = m >> 20;
        const uint32_t rem = m & 0xfffffu;
        if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;
        int e2 = ex;
        if (q == 16u) {
            q = 8u;
            ++e2;
        }
        if (e2 > 8 || (e2 == 8 && q > 14u)) return sign | 0x7eu;
        return sign | ((uint32_t)(e2 + 7) << 3) | (q & 7u);
    }
    const int s = 14 - ex;  // subnormal spacing 2^-9: shift 21..24
    uint32_t q = m >> s;
    const uint32_t rem = m & ((1u << s) - 1u), half = 1u << (s - 1);
    if (rem > half || (rem == half && (q & 1u))) ++q;
    return sign | q;  // q == 8 is the smallest normal, code 0x08
}

// The kernels encode with gfx950's packed conversion instruction instead:
// it rounds to nearest-even and gives e4m3_rne's code for every finite
// |y| <= 448, which the block scale guarantees (checked exhaustively over
// bf16 inputs); e4m3_rne stays as the written-out definition.

// four fp32 values -> four E4M3 codes, first value in the low byte
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    int u = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    u = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, u, true);
    return (uint32_t)u;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// one fp32 value -> its E4M3 code
__device__ __forceinline__ uint32_t e4m3_hw(float y) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.f, 0, false) & 0xffu;
}

}  // namespace moe
