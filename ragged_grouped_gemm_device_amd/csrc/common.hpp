// Device-side helpers shared by the gfx950 kernels of libmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

#define LDS_AS __attribute__((address_space(3)))

namespace moe {

// Compile-time loop: f(std::integral_constant<int, i>) for i in [0, N).
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN): gfx950 converts
// in hardware (v_cvt_pk_bf16_f32), two values per instruction.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

// Logistic sigmoid 1 / (1 + e^-x) with the hardware exp and reciprocal
// (about 1 ulp each); saturates to 0 / 1 for large |x|.
__device__ __forceinline__ float sigmoid_f(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

// GLU gate activations. ACT 0: SiLU (SwiGLU), x * sigmoid(x). ACT 1: GELU in
// its exact form (GeGLU), x * Phi(x) with Phi(x) = (1 + erf(x / sqrt 2)) / 2.
template <int ACT>
__device__ __forceinline__ float glu_gate(float x) {
    if constexpr (ACT == 0) return x * sigmoid_f(x);
    else return 0.5f * x * (1.f + erff(x * 0.70710678118654752f));
}

// The gate activation f(x) and its derivative f'(x):
// SiLU' = s (1 + x (1 - s)), s = sigmoid(x); GELU' = Phi(x) + x phi(x).
template <int ACT>
__device__ __forceinline__ void glu_gate_grad(float x, float& f, float& df) {
    if constexpr (ACT == 0) {
        const float s = sigmoid_f(x);
        f = x * s;
        df = s * (1.f + x * (1.f - s));
    } else {
        const float cdf = 0.5f * (1.f + erff(x * 0.70710678118654752f));
        f = x * cdf;
        df = cdf + x * (0.39894228040143268f * __expf(-0.5f * x * x));
    }
}

// Non-gated activation (ACT == 2: squared ReLU, relu(x)^2) and its derivative 2 relu(x).
template <int ACT>
__device__ __forceinline__ void plain_act_grad(float x, float& f, float& df) {
    static_assert(ACT == 2, "squared ReLU only");
    const float r = fmaxf(x, 0.f);
    f = r * r;
    df = 2.f * r;
}

// Unpack 4 bf16 held in a uint2 into floats.
__device__ __forceinline__ void unpack_bf16x4(uint2 v, float* f) {
    f[0] = __uint_as_float(v.x << 16);
    f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16);
    f[3] = __uint_as_float(v.y & 0xffff0000u);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Order this wavefront's LDS writes before its later reads of other lanes' data.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Streaming (non-temporal) stores for the GEMM outputs: the weight gradients,
// the H saved for the backward pass, and the bf16 outputs (Y, dX_perm, dH, A')
// that the next kernels read once, at these sizes mostly from HBM anyway.
// They do not take last-level cache lines from the operands being multiplied
// (measured 0.2-2% faster per kernel; 8-byte pieces, partial cache lines,
// measured slower and keep normal stores).
typedef uint32_t u32x4_nt_t __attribute__((ext_vector_type(4)));
template <class T>
__device__ __forceinline__ void st_nt16(void* p, T v) {
    static_assert(sizeof(T) == 16, "16-byte store");
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_nt_t, v), (u32x4_nt_t*)p);
}

// Butterfly sum over the 64 lanes of a wavefront.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

}  // namespace moe
