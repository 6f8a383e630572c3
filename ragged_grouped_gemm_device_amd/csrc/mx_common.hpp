// MXFP8 block codec on the device: E8M0 block scales and E4M3 elements.
//
// [NVIDIA CuTe DSL fusion-kernel page, problem and core-idea sections: BF16
// activations become MXFP8 plus a transposed copy; Transformer Engine page,
// three-components section: group-aware MXFP8 quantization.] The pages give
// no encoding rule; the OCP Microscaling (MX) v1.0 formats are used with the
// scale rounded up, so that no element of a block is clipped (the floor rule
// clips block maxima with a significand above 1.75 by up to 12.5%, more than
// the MXFP8 path's 6e-2 error budget): a block of
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

// two bf16 magnitudes (or other 16-bit fields) per register
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a),
                                                                  __builtin_bit_cast(u16x2_t, b)));
}

// The value of lane l ^ M inside each 32-lane half (M = 1, 2, 4, 8, 16): DPP
// quad permutes for 1 and 2, a rotation of the 16-lane row by 8 for 8, and a
// bit-mask ds_swizzle (and 0x1f, xor M) for 4 and 16.
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
    if constexpr (M == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
    else if constexpr (M == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);
    else if constexpr (M == 8) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, true);
    else return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (M << 10));
}

// Column-wise MXFP8 blocks of one 32 x 32 block held the MFMA way: lane l has
// row l & 31 and, in 16-bit slot j of pk[j / 2] (bf16 bits), column
// 8 (j / 4) + 4 h + j % 4 with h = l / 32. The 32-row maxima come from a
// transposing butterfly inside each half: every exchange pairs lanes whose
// rows differ in one bit and halves the slots a lane carries (it keeps the
// half its partner sends), so after the exchanges across row bits 4..1 lane
// pair (2i, 2i + 1) carries slot i, and one more exchange finishes its
// maximum (9 exchanges for 16 columns instead of 5 per column). The E8M0
// codes travel back the same way. Codes go to q[c * ldq + row], the scale of
// column c to sc[c * lds] (each lane of a pair stores the same byte).
template <class Sink>
__device__ __forceinline__ void mx_colq32_impl(const uint32_t pk[8], int lane, uint8_t* sc, int64_t lds,
                                               Sink sink) {
    const bool b4 = lane & 16, b3 = lane & 8, b2 = lane & 4, b1 = lane & 2;
    const int h = (lane >> 5) & 1;
    uint32_t t1[4], t2[2];
#pragma unroll
    for (int p = 0; p < 4; ++p) {  // rows r, r ^ 16: slots 2p, 2p + 1 (+ 8 b4)
        const uint32_t lo = pk[p] & 0x7fff7fffu, hi = pk[p + 4] & 0x7fff7fffu;
        t1[p] = max_u16x2(b4 ? hi : lo, xor_lane<16>(b4 ? lo : hi));
    }
#pragma unroll
    for (int p = 0; p < 2; ++p)  // slots 2p, 2p + 1 (+ 4 b3 + 8 b4)
        t2[p] = max_u16x2(b3 ? t1[p + 2] : t1[p], xor_lane<8>(b3 ? t1[p] : t1[p + 2]));
    // slots 0, 1 (+ 2 b2 + 4 b3 + 8 b4)
    const uint32_t t3 = max_u16x2(b2 ? t2[1] : t2[0], xor_lane<4>(b2 ? t2[0] : t2[1]));
    // slot i = b1 + 2 b2 + 4 b3 + 8 b4
    uint32_t t4 = max(b1 ? t3 >> 16 : t3 & 0xffffu, xor_lane<2>(b1 ? t3 & 0xffffu : t3 >> 16));
    t4 = max(t4, xor_lane<1>(t4));
    const uint32_t ec = (uint32_t)(mx_block_exp(t4) + 127);
    const int i = (lane >> 1) & 15;
    sc[(int64_t)(8 * (i >> 2) + 4 * h + (i & 3)) * lds] = (uint8_t)ec;
    // codes back to every slot: w0[p] holds slots 2p, 2p + 1
    uint32_t o = xor_lane<2>(ec);
    const uint32_t w3 = b1 ? (o | (ec << 16)) : (ec | (o << 16));
    o = xor_lane<4>(w3);
    const uint32_t w2[2] = {b2 ? o : w3, b2 ? w3 : o};
    uint32_t w1[4], w0[8];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        o = xor_lane<8>(w2[p]);
        w1[p] = b3 ? o : w2[p];
        w1[p + 2] = b3 ? w2[p] : o;
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        o = xor_lane<16>(w1[p]);
        w0[p] = b4 ? o : w1[p];
        w0[p + 4] = b4 ? w1[p] : o;
    }
    // Codes: the 4 slots 4Q + s of a lane become one word, and a 4 x 4 byte
    // transpose across the lanes of a row quad (two exchanges, each followed
    // by a byte permute) leaves lane t of the quad with slot 4Q + t for the
    // quad's 4 rows: one 4-byte store per column and quad instead of four
    // 1-byte stores.
    const int row = lane & 31, t = row & 3;
    const uint32_t sel1 = (t & 1) ? 0x03070105u : 0x06020400u;  // bytes 0-3: own word, 4-7: partner's
    const uint32_t sel2 = (t & 2) ? 0x03020706u : 0x05040100u;
#pragma unroll
    for (int Q = 0; Q < 4; ++Q) {
        float y[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int j = 4 * Q + s;
            const uint32_t ecj = (w0[j >> 1] >> (16 * (j & 1))) & 0xffffu;
            const float inv = __uint_as_float((254u - ecj) << 23);  // 2^-(ecj - 127)
            y[s] = ((j & 1) ? bf16_hi(pk[j >> 1]) : bf16_lo(pk[j >> 1])) * inv;
        }
        uint32_t w = e4m3x4(y[0], y[1], y[2], y[3]);
        w = __builtin_amdgcn_perm(xor_lane<1>(w), w, sel1);  // 16-bit pairs: rows (2i, 2i + 1)
        w = __builtin_amdgcn_perm(xor_lane<2>(w), w, sel2);  // words: rows 4i .. 4i + 3
        sink(Q, w);  // column 8 Q + 4 h + t, rows (row & ~3) .. (row & ~3) + 3
    }
}

// Codes to q[c * ldq + row] directly.
__device__ __forceinline__ void mx_colq32(const uint32_t pk[8], int lane, uint8_t* q, int64_t ldq,
                                          uint8_t* sc, int64_t lds) {
    const int row = lane & 31, t = row & 3, h = (lane >> 5) & 1;
    uint8_t* qr = q + (row & ~3);
    mx_colq32_impl(pk, lane, sc, lds,
                   [&](int Q, uint32_t w) { *(uint32_t*)(qr + (int64_t)(8 * Q + 4 * h + t) * ldq) = w; });
}

// Codes to an LDS stage of 32 columns x 128 rows (block I holds rows 32 I ..
// 32 I + 31), 128 bytes per column whose 16-byte row segments are XOR-swizzled
// by the column (segment g of column c at (g ^ (c & 7)) * 16): the quads' word
// writes then hit distinct banks, and mx_stage_flush sends each column out as
// whole 16-byte pieces (one 128-byte line per column and band) instead of the
// 32-byte pieces the direct stores leave scattered over 16 columns.
__device__ __forceinline__ void mx_colq32_stage(const uint32_t pk[8], int lane, uint8_t* stage, int I,
                                                uint8_t* sc, int64_t lds) {
    const int row = lane & 31, t = row & 3, h = (lane >> 5) & 1;
    const int r = 32 * I + (row & ~3);
    mx_colq32_impl(pk, lane, sc, lds, [&](int Q, uint32_t w) {
        const int c = 8 * Q + 4 * h + t;
        *(uint32_t*)(stage + c * 128 + (((r >> 4) ^ (c & 7)) << 4) + (r & 15)) = w;
    });
}

// The stage's columns to q[c * ldq + row], rows [0, rows) of the band only
// (rows is a multiple of 16), 16 bytes per lane and piece.
__device__ __forceinline__ void mx_stage_flush(const uint8_t* stage, int lane, uint8_t* q, int64_t ldq,
                                               int rows) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int idx = it * 64 + lane;
        const int c = idx >> 3, g = idx & 7;
        if (g * 16 < rows)
            *(uint4*)(q + (int64_t)c * ldq + g * 16) = *(const uint4*)(stage + c * 128 + ((g ^ (c & 7)) << 4));
    }
}

// The 32 codes of a row-wise block, held as four words per lane (word Q: codes
// 8 Q + 4 h .. 8 Q + 4 h + 3 of the row, h the lane half), leave as one 16-byte
// store per lane: half 0 writes codes 0-15 and half 1 codes 16-31, after each
// trades two words with lane l ^ 32 (v_permlane32_swap, which needs every lane
// of the wavefront active). q: the row's first code of the block.
__device__ __forceinline__ void mx_store_row32(const uint32_t w[4], int lane, uint8_t* q) {
    const int h = (lane >> 5) & 1;
    const uint32_t g0 = h ? w[0] : w[2], g1 = h ? w[1] : w[3];
    const auto s0 = __builtin_amdgcn_permlane32_swap(g0, g0, false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(g1, g1, false, false);
    const uint32_t r0 = h ? s0[0] : s0[1], r1 = h ? s1[0] : s1[1];
    *(uint4*)(q + 16 * h) = h ? make_uint4(r0, w[2], r1, w[3]) : make_uint4(w[0], r0, w[1], r1);
}

// Row-wise MXFP8 block of one row of a 32 x 32 block held the MFMA way: this
// lane has 16 of the row's 32 bf16 values (pk[j / 2], 16-bit slot j: column
// 8 (j / 4) + 4 h + j % 4, h = lane / 32), the lane l ^ 32 the other 16. The
// block maximum is one lane exchange away; the codes go to q (the row's first
// column of the block) as one 16-byte piece per lane (mx_store_row32), the
// E8M0 scale to *sc (the same byte from both lanes).
__device__ __forceinline__ void mx_rowq32(const uint32_t pk[8], int lane, uint8_t* q, uint8_t* sc) {
    uint32_t am = 0;
#pragma unroll
    for (int r = 0; r < 8; ++r) am = max_u16x2(am, pk[r] & 0x7fff7fffu);
    uint32_t amax = max(am & 0xffffu, am >> 16);
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 32, 64));
    const int e = mx_block_exp(amax);
    const float inv = mx_inv_scale(e);
    uint32_t w[4];
#pragma unroll
    for (int Q = 0; Q < 4; ++Q)
        w[Q] = e4m3x4(bf16_lo(pk[2 * Q]) * inv, bf16_hi(pk[2 * Q]) * inv, bf16_lo(pk[2 * Q + 1]) * inv,
                      bf16_hi(pk[2 * Q + 1]) * inv);
    mx_store_row32(w, lane, q);
    *sc = (uint8_t)(e + 127);
}

}  // namespace moe
