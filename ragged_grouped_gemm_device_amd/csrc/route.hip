// Routing and ragged layout kernels (gfx950).
//
// route_topk_kernel: softmax over E + top-k per token, one group of lanes per
//   token (8, 16, 32 or 64 lanes, the smallest that holds E, 64 beyond 32).
//   [Dropless MoE 학습과 NVIDIA Transformer Engine 소개, section on ragged
//   tensors: a learned router activates each token's top-K experts.]
// route_bwd_kernel: the router's softmax backward from dS (one wavefront per
//   token; route_bwd_group_kernel: one group of 8, 16 or 32 lanes when E <= 32).
// layout kernels: per-expert counts, 128-aligned offsets and the two row maps,
//   computed on the device with no host readback, deterministically (a stable
//   counting sort: per-chunk histograms, an exclusive scan over chunks, then
//   in-order ranks from wavefront ballots; no atomics decide an order).
//   [NVIDIA CuTe DSL fusion-kernel page, core-idea section: per-expert token
//   counts live in GPU memory; Transformer Engine page, grouped-GEMM section:
//   expert regions aligned to 128 tokens; dropless-boundary section: one slot
//   per (token, expert) pair, regions padded to the alignment unit.]
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kMaxPerLane = MOE_MAX_E / 64;   // logits per lane of a full wavefront (E <= 1024)

// One group of G lanes per token (G = 8, 16 or 32 when E <= G, one logit per
// lane; G = 64 otherwise, up to MOE_MAX_E / 64 logits per lane), so small
// expert counts do not leave most of a wavefront idle. Reductions are lane
// exchanges inside the group.
template <int G, int PER>
__global__ void __launch_bounds__(256) route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int renorm,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w,
                                                         int32_t* __restrict__ err_word) {
    const int lane = lane_id();
    const int gl = lane % G;  // lane inside the token's group
    const int t = (int)(((int64_t)blockIdx.x * 256 + threadIdx.x) / G);
    const bool active = t < T;
    const float* row = logits + (int64_t)t * E;
    float v[PER];
    bool bad = false;
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = gl + G * i;
        float x = -INFINITY;
        if (active && e < E) {
            x = row[e];
            if (!isfinite(x)) {
                bad = true;
                x = -INFINITY;  // a non-finite logit is never preferred
            }
        }
        v[i] = x;
        mx = fmaxf(mx, x);
    }
    if (__ballot(bad) != 0ull && lane == 0 && err_word) atomicOr(err_word, MOE_ERRBIT_NONFINITE_LOGIT);
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i)
        if (gl + G * i < E && v[i] > -INFINITY) s += expf(v[i] - mx);
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if (!(mx > -INFINITY)) s = 1.f;  // every logit non-finite: weights become 0

    uint32_t taken = 0;  // bit i: v[i] already selected
    float chosen_w[8];
    float wsum = 0.f;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = gl + G * i;
            if (e < E && !((taken >> i) & 1u) && (v[i] > bv || bi == 0x7fffffff)) {
                bv = v[i];
                bi = e;
            }
        }
#pragma unroll
        for (int o = G / 2; o > 0; o >>= 1) {
            const float ov = __shfl_xor(bv, o, 64);
            const int oi = __shfl_xor(bi, o, 64);
            if (ov > bv || (ov == bv && oi < bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi % G) == gl) taken |= 1u << (bi / G);
        const float p = (bv > -INFINITY) ? expf(bv - mx) / s : 0.f;
        wsum += p;
        if (j < 8) chosen_w[j] = p;
        if (active && gl == 0) {
            topk_idx[(int64_t)t * k + j] = bi;
            if (!renorm) topk_w[(int64_t)t * k + j] = p;
        }
    }
    if (renorm && active && gl == 0) {
        const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
        for (int j = 0; j < k; ++j) {
            float p;
            if (j < 8) {
                p = chosen_w[j];
            } else {
                // k > 8: recompute from the logit; a non-finite one weighs 0, as
                // in the selection above
                const float x = row[topk_idx[(int64_t)t * k + j]];
                p = isfinite(x) ? expf(x - mx) / s : 0.f;
            }
            topk_w[(int64_t)t * k + j] = p * inv;
        }
    }
}

// Lanes of this wavefront whose value of e (0 <= e < 2^nbits) equals ours.
__device__ __forceinline__ uint64_t match_lanes(int e, bool valid, int nbits) {
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
    }
    return valid ? m : 0ull;
}

// Per-chunk histograms (chunk = kChunkPairs consecutive pairs, one wavefront)
// and the -1 fill of src_of.
__global__ void __launch_bounds__(256) layout_hist_kernel(const int32_t* __restrict__ topk_idx,
                                                          int64_t P, int E, int nchunks,
                                                          int32_t* __restrict__ hist,
                                                          int32_t* __restrict__ src_of,
                                                          int64_t M_cap) {
    extern __shared__ int32_t s_cnt[];  // [4][E]
    const int wave = threadIdx.x >> 6, lane = lane_id();
    int32_t* cnt = s_cnt + wave * E;
    for (int e = lane; e < E; e += 64) cnt[e] = 0;
    // fill src_of with -1 (grid-stride)
    for (int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x; r < M_cap; r += (int64_t)gridDim.x * 256)
        src_of[r] = -1;
    const int chunk = blockIdx.x * 4 + wave;
    __syncthreads();
    if (chunk < nchunks) {
        const int64_t base = (int64_t)chunk * kChunkPairs;
        for (int s = 0; s < kChunkPairs; s += 64) {
            const int64_t p = base + s + lane;
            if (p < P) atomicAdd(&cnt[topk_idx[p]], 1);  // integer sum: order-free
        }
    }
    __syncthreads();
    if (chunk < nchunks)
        for (int e = lane; e < E; e += 64) hist[(int64_t)chunk * E + e] = cnt[e];
}

// Exclusive scan of the histograms over chunks (per expert), counts, and the
// 128-aligned offsets. One workgroup.
__global__ void __launch_bounds__(1024) layout_scan_kernel(const int32_t* __restrict__ hist,
                                                           int nchunks, int E,
                                                           int32_t* __restrict__ base,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets) {
    __shared__ int32_t s_pad[MOE_MAX_E];
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int32_t run = 0;
        for (int c = 0; c < nchunks; ++c) {
            base[(int64_t)c * E + e] = run;
            run += hist[(int64_t)c * E + e];
        }
        counts[e] = run;
        s_pad[e] = (run + MOE_ALIGN_ROWS - 1) / MOE_ALIGN_ROWS * MOE_ALIGN_ROWS;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t o = 0;
        offsets[0] = 0;
        for (int e = 0; e < E; ++e) {
            o += s_pad[e];
            offsets[e + 1] = o;
        }
    }
}

// In-order ranks: each wavefront walks its chunk 64 pairs at a time.
__global__ void __launch_bounds__(256) layout_scatter_kernel(const int32_t* __restrict__ topk_idx,
                                                             int64_t P, int E, int nbits,
                                                             int nchunks,
                                                             const int32_t* __restrict__ base,
                                                             const int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ row_of,
                                                             int32_t* __restrict__ src_of) {
    extern __shared__ int32_t s_cnt[];  // [4][E]
    const int wave = threadIdx.x >> 6, lane = lane_id();
    int32_t* cnt = s_cnt + wave * E;
    const int chunk = blockIdx.x * 4 + wave;
    if (chunk >= nchunks) return;  // wave-private LDS: no block barrier below
    for (int e = lane; e < E; e += 64) cnt[e] = base[(int64_t)chunk * E + e] + offsets[e];
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int64_t b0 = (int64_t)chunk * kChunkPairs;
    for (int s = 0; s < kChunkPairs; s += 64) {
        const int64_t p = b0 + s + lane;
        const bool valid = p < P;
        const int e = valid ? topk_idx[p] : 0;
        const uint64_t m = match_lanes(e, valid, nbits);
        int32_t row = 0;
        if (valid) row = cnt[e] + __popcll(m & lt);
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
        if (valid && (m & lt) == 0ull) cnt[e] = row + __popcll(m);  // group leader advances
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
        if (valid) {
            row_of[p] = row;
            src_of[row] = (int32_t)p;
        }
    }
}

// Router backward, one wavefront per token: dlogits from dS = dL/dw for the
// experts the forward chose. Without renormalisation w_j = p_{e_j} (softmax
// over all E) and dl_e = p_e (g_e - sum_j p_{e_j} dS_j) with g_e = dS_j for
// e = e_j, else 0; with renormalisation w is the softmax over the chosen
// logits and dl_{e_j} = w_j (dS_j - sum_i w_i dS_i), 0 elsewhere. The chosen
// slots are scattered through a per-wavefront LDS row. Non-finite logits
// count as -inf (probability 0), as in the forward.
// [SonicMoE로 보는 GPU 커널 최적화, backward-rewrite section: dS is the
// router-score gradient; it continues through the router's softmax.]
__global__ void __launch_bounds__(256) route_bwd_kernel(const float* __restrict__ logits, int T, int E,
                                                        int k, int renorm,
                                                        const int32_t* __restrict__ topk_idx,
                                                        const float* __restrict__ ds,
                                                        float* __restrict__ dlogits) {
    __shared__ float s_g[4][MOE_MAX_E];
    const int lane = lane_id();
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    const bool live = t < T;  // no early exit: the block barrier below needs every wave
    float* g = s_g[threadIdx.x >> 6];
    const float* row = logits + (int64_t)(live ? t : 0) * E;
    float v[kMaxPerLane];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + 64 * i;
        float x = -INFINITY;
        if (live && e < E) {
            x = row[e];
            if (!isfinite(x)) x = -INFINITY;
            g[e] = 0.f;
        }
        v[i] = x;
        mx = fmaxf(mx, x);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i)
        if (lane + 64 * i < E && v[i] > -INFINITY) s += expf(v[i] - mx);
    s = wave_sum(s);
    if (!(mx > -INFINITY)) s = 1.f;
    const float inv_s = 1.f / s;
    // chosen slots: probability p_j of e_j; P = sum of the chosen probabilities
    float pj_sum = 0.f, c = 0.f;
    for (int j0 = 0; j0 < k; j0 += 64) {
        const int j = j0 + lane;
        float pj = 0.f, dj = 0.f;
        if (live && j < k) {
            const float x = row[topk_idx[(int64_t)t * k + j]];
            pj = isfinite(x) ? expf(x - mx) * inv_s : 0.f;
            dj = ds[(int64_t)t * k + j];
        }
        pj_sum += pj;
        c += pj * dj;
    }
    pj_sum = wave_sum(pj_sum);
    c = wave_sum(c);  // sum_j p_j dS_j
    if (renorm) c = pj_sum > 0.f ? c / pj_sum : 0.f;  // sum_j w_j dS_j
    __syncthreads();  // g rows cleared
    for (int j0 = 0; j0 < k; j0 += 64) {
        const int j = j0 + lane;
        if (live && j < k) {
            const int e = topk_idx[(int64_t)t * k + j];
            const float dj = ds[(int64_t)t * k + j];
            if (renorm) {
                const float x = row[e];
                const float pj = isfinite(x) ? expf(x - mx) * inv_s : 0.f;
                const float wj = pj_sum > 0.f ? pj / pj_sum : 0.f;
                g[e] = wj * (dj - c);
            } else {
                g[e] = dj;
            }
        }
    }
    __syncthreads();  // chosen slots scattered
    if (!live) return;
    float* out = dlogits + (int64_t)t * E;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + 64 * i;
        if (e < E) {
            const float pe = v[i] > -INFINITY ? expf(v[i] - mx) * inv_s : 0.f;
            out[e] = renorm ? g[e] : pe * (g[e] - c);
        }
    }
}

// The same for E <= G = 8, 16 or 32: one group of G lanes per token, lane gl
// holding logit gl, so small expert counts do not leave most of a wavefront
// idle. The chosen slots' probabilities come from the lanes holding their
// logits (a lane exchange inside the group), in slot order.
template <int G>
__global__ void __launch_bounds__(256) route_bwd_group_kernel(const float* __restrict__ logits, int T, int E,
                                                              int k, int renorm,
                                                              const int32_t* __restrict__ topk_idx,
                                                              const float* __restrict__ ds,
                                                              float* __restrict__ dlogits) {
    const int lane = lane_id();
    const int gl = lane % G, gbase = lane - gl;
    const int t = (int)(((int64_t)blockIdx.x * 256 + threadIdx.x) / G);
    const bool live = t < T;
    const bool own = live && gl < E;
    float x = -INFINITY;
    if (own) {
        x = logits[(int64_t)t * E + gl];
        if (!isfinite(x)) x = -INFINITY;
    }
    float mx = x;
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    float s = x > -INFINITY ? expf(x - mx) : 0.f;
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if (!(mx > -INFINITY)) s = 1.f;
    const float inv_s = 1.f / s;
    // P = sum of the chosen probabilities, c = sum_j p_j dS_j; and this lane's
    // slot (its dS and probability) if its expert was chosen
    float pj_sum = 0.f, c = 0.f, dsel = 0.f, psel = 0.f;
    bool chosen = false;
    for (int j = 0; j < k; ++j) {
        const int ej = live ? topk_idx[(int64_t)t * k + j] : 0;
        const float dj = live ? ds[(int64_t)t * k + j] : 0.f;
        const float xj = __shfl(x, gbase + (ej & (G - 1)), 64);
        const float pj = xj > -INFINITY ? expf(xj - mx) * inv_s : 0.f;
        pj_sum += pj;
        c += pj * dj;
        if (ej == gl) {
            chosen = true;
            dsel = dj;
            psel = pj;
        }
    }
    if (renorm) c = pj_sum > 0.f ? c / pj_sum : 0.f;  // sum_j w_j dS_j
    if (!own) return;
    float out;
    if (renorm) {
        const float wj = pj_sum > 0.f ? psel / pj_sum : 0.f;
        out = chosen ? wj * (dsel - c) : 0.f;
    } else {
        const float pe = x > -INFINITY ? expf(x - mx) * inv_s : 0.f;
        out = pe * ((chosen ? dsel : 0.f) - c);
    }
    dlogits[(int64_t)t * E + gl] = out;
}

int launch_route_bwd(const float* logits, int T, int E, int k, int renorm, const int32_t* topk_idx,
                     const float* ds, float* dlogits, hipStream_t s) {
    auto grouped = [&](auto kern, int g) {
        const int64_t blocks = ((int64_t)T * g + 255) / 256;
        kern<<<(unsigned)blocks, 256, 0, s>>>(logits, T, E, k, renorm, topk_idx, ds, dlogits);
    };
    if (E <= 8)
        grouped(route_bwd_group_kernel<8>, 8);
    else if (E <= 16)
        grouped(route_bwd_group_kernel<16>, 16);
    else if (E <= 32)
        grouped(route_bwd_group_kernel<32>, 32);
    else
        route_bwd_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, T, E, k, renorm, topk_idx, ds, dlogits);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_route(const float* logits, int T, int E, int k, int renorm, int32_t* topk_idx,
                 float* topk_w, int32_t* counts, int32_t* offsets, int32_t* row_of,
                 int32_t* src_of, int64_t M_cap, int32_t* err_word, void* ws, hipStream_t s) {
    const int64_t P = (int64_t)T * k;
    const int nchunks = (int)((P + kChunkPairs - 1) / kChunkPairs);
    int32_t* hist = (int32_t*)ws;
    int32_t* base = hist + (int64_t)nchunks * E;
    auto topk = [&](auto kern, int g) {
        const int64_t blocks = ((int64_t)T * g + 255) / 256;
        kern<<<(unsigned)blocks, 256, 0, s>>>(logits, T, E, k, renorm, topk_idx, topk_w, err_word);
    };
    if (E <= 8)
        topk(route_topk_kernel<8, 1>, 8);
    else if (E <= 16)
        topk(route_topk_kernel<16, 1>, 16);
    else if (E <= 32)
        topk(route_topk_kernel<32, 1>, 32);
    else
        topk(route_topk_kernel<64, MOE_MAX_E / 64>, 64);
    const int nblk = (nchunks + 3) / 4;
    const size_t lds = 4 * (size_t)E * sizeof(int32_t);
    layout_hist_kernel<<<nblk, 256, lds, s>>>(topk_idx, P, E, nchunks, hist, src_of, M_cap);
    layout_scan_kernel<<<1, 1024, 0, s>>>(hist, nchunks, E, base, counts, offsets);
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    layout_scatter_kernel<<<nblk, 256, lds, s>>>(topk_idx, P, E, nbits, nchunks, base, offsets,
                                                 row_of, src_of);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

size_t route_workspace_bytes(int T, int k, int E) {
    const int64_t P = (int64_t)T * k;
    const int64_t nchunks = (P + kChunkPairs - 1) / kChunkPairs;
    return (size_t)(2 * nchunks * E) * sizeof(int32_t);
}

// Scratch of the allocation-free routing entry point: the per-chunk
// histograms and scan bases of the layout, in device memory the library
// reserves statically (kRouteStaticScratch bytes per GPU, held until the
// process ends). Nothing in it has to start at zero: the histogram kernel
// writes every chunk's counts and the scan every base before they are read.
// In host code `scratch` names a host-side stand-in; the kernels get the
// device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[kRouteStaticScratch];

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr if the lookup fails.
static void* route_scratch_ptr() {
    static std::mutex mu;
    static void* ptr[kMaxDevices];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        ptr[dev] = p;
    }
    return ptr[dev];
}

int launch_route_noalloc(const float* logits, int T, int E, int k, int renorm, int32_t* topk_idx,
                         float* topk_w, int32_t* counts, int32_t* offsets, int32_t* row_of,
                         int32_t* src_of, int64_t M_cap, int32_t* err_word, hipStream_t s) {
    if (route_workspace_bytes(T, k, E) > kRouteStaticScratch) return -3;
    void* ws = route_scratch_ptr();
    if (!ws) return -4;
    return launch_route(logits, T, E, k, renorm, topk_idx, topk_w, counts, offsets, row_of, src_of, M_cap,
                        err_word, ws, s);
}

}  // namespace moe
