// Memory-bound gather (permute) and weighted un-permute (combine) kernels.
//
// [SonicMoE로 보는 GPU 커널 최적화, SonicMoE section: the gather, scatter and
// expert-aggregation sub-kernels move 2TKd bytes without compute.]
// [Dropless MoE 학습과 NVIDIA Transformer Engine 소개, EP section: dispatch
// permutes tokens expert-major; combine restores token order and accumulates.]
//
// Both kernels move 16-byte vectors: each thread owns (row, 16-byte column
// chunk) pairs and keeps several independent loads in flight, so the HBM
// traffic is fully coalesced along rows.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kUnroll = 4;
// Streaming (non-temporal) 16-byte accesses: data touched once and larger than
// the last-level cache bypasses it instead of evicting what the next kernel reads.
typedef uint32_t nt_u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load((const nt_u32x4_t*)p));
}
__device__ __forceinline__ void st_stream(uint4* p, uint4 v) {
    __builtin_nontemporal_store(__builtin_bit_cast(nt_u32x4_t, v), (nt_u32x4_t*)p);
}
// bytes one launch moves above which it streams (twice the 256 MB last-level cache)
constexpr int64_t kStreamBytes = 512ll << 20;


// x_perm[row_of[t*k + j]] = x[t]; padding rows of every expert region are
// zero. Token-major: each token row is read from HBM once and written to its
// k rows (a destination-major gather would read it k times). The workgroups
// past main_blocks clear the padding, which sits in the last 127 rows of a
// region (regions are 128-row multiples and start with their real rows).
template <bool NT_STORE>
__global__ void __launch_bounds__(256) permute_kernel(const uint4* __restrict__ x,
                                                      const int32_t* __restrict__ row_of,
                                                      const int32_t* __restrict__ src_of,
                                                      const int32_t* __restrict__ offsets, int T,
                                                      int k, int E, int cpr, int64_t M_cap,
                                                      int main_blocks, uint4* __restrict__ x_perm) {
    if ((int)blockIdx.x < main_blocks) {
        const int64_t total = (int64_t)T * cpr;
        const int64_t stride = (int64_t)main_blocks * 256;
        for (int64_t i0 = (int64_t)blockIdx.x * 256 * kUnroll + threadIdx.x; i0 < total;
             i0 += stride * kUnroll) {
            uint4 v[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t i = i0 + (int64_t)u * 256;
                if (i < total) v[u] = ld_stream(x + i);
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t i = i0 + (int64_t)u * 256;
                if (i < total) {
                    const int64_t t = i / cpr;
                    const int c = (int)(i - t * cpr);
                    const int32_t* ro = row_of + t * k;
                    for (int j = 0; j < k; ++j) {
                        const int64_t r = ro[j];
                        if ((uint64_t)r < (uint64_t)M_cap) {  // guard only
                            if constexpr (NT_STORE) st_stream(x_perm + r * cpr + c, v[u]);
                            else x_perm[r * cpr + c] = v[u];
                        }
                    }
                }
            }
        }
    } else {
        // one candidate row per wavefront: a uniform test, then 64 lanes clear it
        const int wave = (int)((blockIdx.x - main_blocks) * 4 + (threadIdx.x >> 6));
        const int lane = threadIdx.x & 63;
        const int nwaves = (int)(gridDim.x - main_blocks) * 4;
        for (int q = wave; q < E * 127; q += nwaves) {
            const int e = q / 127, rr = q - e * 127;
            const int64_t r = (int64_t)offsets[e + 1] - 127 + rr;
            if (r >= offsets[e] && src_of[r] < 0)
                for (int c = lane; c < cpr; c += 64) x_perm[r * cpr + c] = make_uint4(0, 0, 0, 0);
        }
    }
}

// out[t] = sum_j w[t, j] * y[row_of[t*k+j]] in ascending j (fp32), bf16 once.
template <bool NT>
__global__ void __launch_bounds__(256) combine_kernel(const uint4* __restrict__ y,
                                                      const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ w, int k, int cpr,
                                                      int64_t total, uint4* __restrict__ out) {
    constexpr int U = 2;  // chunks per thread and iteration: independent loads in flight
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i0 = (int64_t)blockIdx.x * 256 * U + threadIdx.x; i0 < total; i0 += stride * U) {
        float acc[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[u][q] = 0.f;
        for (int j = 0; j < k; ++j) {
            uint4 v[U];
            float wj[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = i0 + (int64_t)u * 256;
                v[u] = make_uint4(0, 0, 0, 0);
                wj[u] = 0.f;
                if (i < total) {
                    const int64_t t = i / cpr;
                    const int c = (int)(i - t * cpr);
                    const int64_t r = row_of[t * k + j];
                    wj[u] = w ? w[t * k + j] : 1.f;
                    v[u] = NT ? ld_stream(y + r * cpr + c) : y[r * cpr + c];
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float f[8];
                unpack_bf16x4(make_uint2(v[u].x, v[u].y), f);
                unpack_bf16x4(make_uint2(v[u].z, v[u].w), f + 4);
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[u][q] = fmaf(wj[u], f[q], acc[u][q]);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = i0 + (int64_t)u * 256;
            if (i < total) {
                uint4 o;
                o.x = pack_bf16x2(acc[u][0], acc[u][1]);
                o.y = pack_bf16x2(acc[u][2], acc[u][3]);
                o.z = pack_bf16x2(acc[u][4], acc[u][5]);
                o.w = pack_bf16x2(acc[u][6], acc[u][7]);
                if constexpr (NT) st_stream(out + i, o);
                else out[i] = o;
            }
        }
    }
}

static int grid_for(int64_t work, int per_block) {
    int64_t g = (work + per_block - 1) / per_block;
    const int64_t cap = 256 * 32;  // 32 workgroups per CU on 256 CUs: enough in flight
    if (g > cap) g = cap;
    return (int)(g < 1 ? 1 : g);
}

int launch_permute(const uint16_t* x, const int32_t* row_of, const int32_t* src_of,
                   const int32_t* offsets, int T, int k, int E, int d, int64_t M_cap, uint16_t* x_perm,
                   hipStream_t s) {
    const int cpr = d / 8;
    const int main_blocks = grid_for((int64_t)T * cpr, 256 * kUnroll);
    const int pad_blocks = std::min(256, (E * 127 + 3) / 4);
    // x is read once: streaming loads. The permuted copy streams too when it is
    // one plain copy (k = 1) too large for the last-level cache; with k > 1, or
    // smaller, the normal stores measured faster over the whole step.
    const bool nt_store = k == 1 && (int64_t)T * d * 2 >= kStreamBytes;
    if (nt_store)
        permute_kernel<true><<<main_blocks + pad_blocks, 256, 0, s>>>((const uint4*)x, row_of, src_of, offsets, T, k,
                                                                    E, cpr, M_cap, main_blocks, (uint4*)x_perm);
    else
        permute_kernel<false><<<main_blocks + pad_blocks, 256, 0, s>>>((const uint4*)x, row_of, src_of, offsets, T, k,
                                                                     E, cpr, M_cap, main_blocks, (uint4*)x_perm);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_combine(const uint16_t* y, const int32_t* row_of, const float* w, int T, int k, int d,
                   uint16_t* out, hipStream_t s) {
    const int cpr = d / 8;
    const int64_t total = (int64_t)T * cpr;
    const bool nt = (int64_t)T * k * d * 2 >= kStreamBytes;  // the Y rows read
    if (nt)
        combine_kernel<true><<<grid_for(total, 512), 256, 0, s>>>((const uint4*)y, row_of, w, k, cpr, total, (uint4*)out);
    else
        combine_kernel<false><<<grid_for(total, 512), 256, 0, s>>>((const uint4*)y, row_of, w, k, cpr, total, (uint4*)out);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace moe
