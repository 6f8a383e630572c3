// Memory-bound gather (permute) and weighted un-permute (combine) kernels.
//
// [SonicMoE로 보는 GPU 커널 최적화, SonicMoE section: the gather, scatter and
// expert-aggregation sub-kernels move 2TKd bytes without compute.]
// [Dropless MoE 학습과 NVIDIA Transformer Engine 소개, EP section: dispatch
// permutes tokens expert-major; combine restores token order and accumulates.]
//
// Both kernels move 16-byte vectors: each thread owns a fixed (row, 16-byte
// column chunk) and keeps several independent loads in flight, so the HBM
// traffic is fully coalesced along rows.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kUnroll = 4;

// x_perm[r] = x[src_of[r] / k] for r < offsets[E]; padding rows are zero.
__global__ void __launch_bounds__(256) permute_kernel(const uint4* __restrict__ x,
                                                      const int32_t* __restrict__ src_of,
                                                      const int32_t* __restrict__ offsets, int k,
                                                      int E, int cpr, int64_t total,
                                                      uint4* __restrict__ x_perm) {
    const int64_t rows = offsets[E];
    const int64_t limit = min(total, rows * cpr);
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i0 = (int64_t)blockIdx.x * 256 * kUnroll + threadIdx.x; i0 < limit;
         i0 += stride * kUnroll) {
        uint4 v[kUnroll];
        int64_t dst[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = i0 + (int64_t)u * 256;
            dst[u] = -1;
            v[u] = make_uint4(0, 0, 0, 0);
            if (i < limit) {
                const int64_t r = i / cpr;
                const int c = (int)(i - r * cpr);
                const int32_t src = src_of[r];
                dst[u] = i;
                if (src >= 0) v[u] = x[(int64_t)(src / k) * cpr + c];
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (dst[u] >= 0) x_perm[dst[u]] = v[u];
    }
}

// out[t] = sum_j w[t, j] * y[row_of[t*k + j]] in ascending j (fp32), bf16 once.
__global__ void __launch_bounds__(256) combine_kernel(const uint4* __restrict__ y,
                                                      const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ w, int k, int cpr,
                                                      int64_t total, uint4* __restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
        const int64_t t = i / cpr;
        const int c = (int)(i - t * cpr);
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = 0.f;
        for (int j = 0; j < k; ++j) {
            const int64_t r = row_of[t * k + j];
            const float wj = w ? w[t * k + j] : 1.f;
            const uint4 v = y[r * cpr + c];
            float f[8];
            unpack_bf16x4(make_uint2(v.x, v.y), f);
            unpack_bf16x4(make_uint2(v.z, v.w), f + 4);
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[q] = fmaf(wj, f[q], acc[q]);
        }
        uint4 o;
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        o.z = pack_bf16x2(acc[4], acc[5]);
        o.w = pack_bf16x2(acc[6], acc[7]);
        out[i] = o;
    }
}

static int grid_for(int64_t work, int per_block) {
    int64_t g = (work + per_block - 1) / per_block;
    const int64_t cap = 256 * 32;  // 32 workgroups per CU on 256 CUs: enough in flight
    if (g > cap) g = cap;
    return (int)(g < 1 ? 1 : g);
}

int launch_permute(const uint16_t* x, const int32_t* src_of, const int32_t* offsets, int k, int E,
                   int d, int64_t M_cap, uint16_t* x_perm, hipStream_t s) {
    const int cpr = d / 8;
    const int64_t total = M_cap * cpr;
    permute_kernel<<<grid_for(total, 256 * kUnroll), 256, 0, s>>>(
        (const uint4*)x, src_of, offsets, k, E, cpr, total, (uint4*)x_perm);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_combine(const uint16_t* y, const int32_t* row_of, const float* w, int T, int k, int d,
                   uint16_t* out, hipStream_t s) {
    const int cpr = d / 8;
    const int64_t total = (int64_t)T * cpr;
    combine_kernel<<<grid_for(total, 256), 256, 0, s>>>((const uint4*)y, row_of, w, k, cpr, total,
                                                        (uint4*)out);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace moe
