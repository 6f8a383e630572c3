// Routing and ragged layout kernels (gfx950).
//
// route_topk_kernel: softmax over E + top-k per token, one group of lanes per
//   token (8, 16, 32 or 64 lanes, the smallest that holds E, 64 beyond 32).
//   [Dropless MoE 학습과 NVIDIA Transformer Engine 소개, section on ragged
//   tensors: a learned router activates each token's top-K experts.]
// route_bwd_kernel: the router's softmax backward from dS (one wavefront per
//   token; route_bwd_group_kernel: one group of 8, 16 or 32 lanes when E <= 32).
// layout: per-expert counts, 128-aligned offsets and the two row maps,
//   computed on the device with no host readback, deterministically (a stable
//   counting sort: per-chunk histograms, an exclusive scan over chunks, then
//   in-order ranks from wavefront ballots; no atomics decide an order).
//   Fused path, two kernels: route_chunk_kernel routes a chunk of tokens and
//   counts its experts in LDS; layout_chunk_kernel scans the chunk counts in
//   parallel (each workgroup its own prefix) and ranks its chunk. General path
//   for many chunks x experts: top-k, chunk histograms, a scan per expert, ranks.
//   [NVIDIA CuTe DSL fusion-kernel page, core-idea section: per-expert token
//   counts live in GPU memory; Transformer Engine page, grouped-GEMM section:
//   expert regions aligned to 128 tokens; dropless-boundary section: one slot
//   per (token, expert) pair, regions padded to the alignment unit.]
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kMaxPerLane = MOE_MAX_E / 64;   // logits per lane of a full wavefront (E <= 1024)
constexpr int kRouteBlock = 1024;             // threads of a fused-routing workgroup

// Softmax top-k of token t by the G lanes of its group (taken for E > 32: a
// whole wavefront, PER >= E / 64 logits per lane): k rounds of a group-wide
// arg-max (larger logit first, the smaller index on ties) by lane exchanges.
// With cnt != nullptr the group's first lane also counts the token's k experts
// into the LDS histogram cnt (integer atomics: the sums do not depend on their
// order).
template <int G, int PER>
__device__ __forceinline__ void route_token(const float* __restrict__ logits, int T, int E, int k,
                                            int renorm, int t, int32_t* __restrict__ topk_idx,
                                            float* __restrict__ topk_w, int32_t* __restrict__ err_word,
                                            int32_t* cnt) {
    const int lane = lane_id();
    const int gl = lane % G;  // lane inside the token's group
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
            if (cnt) atomicAdd(&cnt[bi], 1);
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

// The same for E <= G <= 32 (one logit per lane), by ranks instead of k
// rounds of group-wide arg-max exchanges: the group's logits go through the
// wavefront's LDS row wrow[0..64), every lane reads its group's G slots
// (broadcast reads) and counts the logits ahead of its own (larger, or equal
// with a smaller index: the order the arg-max rounds take), and the logit of
// rank j < k fills slot j. The softmax denominator and the renormalising sum
// are sums in expert and in slot order over LDS (wrow[64..128) and
// wrow[0..64)), so every lane of a group gets the same value. Counting ranks
// costs E compares per lane: with more experts the arg-max rounds are cheaper.
template <int G>
__device__ __forceinline__ void route_token_ranked(const float* __restrict__ logits, int T, int E, int k,
                                                   int renorm, int t, int32_t* __restrict__ topk_idx,
                                                   float* __restrict__ topk_w, int32_t* __restrict__ err_word,
                                                   int32_t* cnt, float* wrow) {
    static_assert(G == 8 || G == 16 || G == 32, "ranked top-k group");
    const int lane = lane_id();
    const int gl = lane % G, gb = lane - gl;  // the group's logits sit at wrow[gb + e]
    const bool mine = t < T && gl < E;
    float x = -INFINITY;
    bool bad = false;
    if (mine) {
        x = logits[(int64_t)t * E + gl];
        if (!isfinite(x)) {
            bad = true;
            x = -INFINITY;  // a non-finite logit is never preferred
        }
    }
    if (__ballot(bad) != 0ull && lane == 0 && err_word) atomicOr(err_word, MOE_ERRBIT_NONFINITE_LOGIT);
    wrow[lane] = x;
    wave_lds_sync();
    // slots e >= E hold -inf (and 0 below): they change no rank, max or sum,
    // so every read is unconditional (16-byte reads, no branch between them)
    int rank = 0;
    float mx = -INFINITY;
    const float4* row4 = (const float4*)(wrow + gb);
#pragma unroll
    for (int j4 = 0; j4 < G / 4; ++j4) {
        const float4 y4 = row4[j4];
        const float ys[4] = {y4.x, y4.y, y4.z, y4.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            mx = fmaxf(mx, ys[u]);
            rank += (ys[u] > x || (ys[u] == x && 4 * j4 + u < gl)) ? 1 : 0;
        }
    }
    const float ex = x > -INFINITY ? expf(x - mx) : 0.f;
    wrow[64 + lane] = ex;
    wave_lds_sync();
    float s = 0.f;
    const float4* ex4 = (const float4*)(wrow + 64 + gb);
#pragma unroll
    for (int j4 = 0; j4 < G / 4; ++j4) {
        const float4 v4 = ex4[j4];
        s += v4.x;
        s += v4.y;
        s += v4.z;
        s += v4.w;
    }
    if (!(mx > -INFINITY)) s = 1.f;  // every logit non-finite: weights become 0
    const float p = x > -INFINITY ? ex / s : 0.f;
    const bool sel = mine && rank < k;
    if (sel) {
        topk_idx[(int64_t)t * k + rank] = gl;
        if (!renorm) topk_w[(int64_t)t * k + rank] = p;
        if (cnt) atomicAdd(&cnt[gl], 1);
    }
    if (renorm) {
        if (sel) wrow[gb + rank] = p;  // the first row is read no more: slot j's probability
        wave_lds_sync();
        float wsum = 0.f;
#pragma unroll
        for (int j4 = 0; j4 < G / 4; ++j4) {
            const float4 v4 = row4[j4];
            const float vs[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) wsum += 4 * j4 + u < k ? vs[u] : 0.f;
        }
        const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
        if (sel) topk_w[(int64_t)t * k + rank] = p * inv;
    }
    wave_lds_sync();  // the next token may overwrite wrow
}

template <int G, int PER>
__device__ __forceinline__ void route_token_any(const float* __restrict__ logits, int T, int E, int k, int renorm,
                                                int t, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                                                int32_t* __restrict__ err_word, int32_t* cnt, float* wrow) {
    if constexpr (G <= 32)
        route_token_ranked<G>(logits, T, E, k, renorm, t, topk_idx, topk_w, err_word, cnt, wrow);
    else
        route_token<G, PER>(logits, T, E, k, renorm, t, topk_idx, topk_w, err_word, cnt);
}

// LDS floats per wavefront for route_token_any.
template <int G>
constexpr int kTokenRow = G <= 32 ? 128 : 1;

template <int G, int PER>
__global__ void __launch_bounds__(256) route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int renorm,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w,
                                                         int32_t* __restrict__ err_word) {
    __shared__ __align__(16) float s_x[4][kTokenRow<G>];
    const int t = (int)(((int64_t)blockIdx.x * 256 + threadIdx.x) / G);
    route_token_any<G, PER>(logits, T, E, k, renorm, t, topk_idx, topk_w, err_word, nullptr,
                            s_x[threadIdx.x >> 6]);
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


// Inclusive prefix sum of v over the 256 threads of a workgroup (part: 256
// ints of LDS); *total receives the sum of all. Begins and ends with a barrier.
__device__ __forceinline__ int32_t block_scan256(int32_t v, int32_t* part, int32_t* total) {
    const int tid = threadIdx.x;
    __syncthreads();
    part[tid] = v;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        const int32_t add = tid >= o ? part[tid - o] : 0;
        __syncthreads();
        part[tid] += add;
        __syncthreads();
    }
    const int32_t r = part[tid];
    *total = part[255];
    __syncthreads();
    return r;
}

// Region starts off[0..E] (LDS) from the expert totals tot[0..E) (LDS): the
// exclusive prefix sum of the totals rounded up to MOE_ALIGN_ROWS, four
// experts per thread of a 256-thread workgroup.
__device__ __forceinline__ void aligned_offsets(const int32_t* tot, int E, int32_t* off, int32_t* part) {
    const int tid = threadIdx.x;
    int32_t v[4], run = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = 4 * tid + i;
        v[i] = e < E ? (tot[e] + MOE_ALIGN_ROWS - 1) / MOE_ALIGN_ROWS * MOE_ALIGN_ROWS : 0;
        run += v[i];
    }
    int32_t all;
    int32_t ex = block_scan256(run, part, &all) - run;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = 4 * tid + i;
        if (e < E) off[e] = ex;
        ex += v[i];
    }
    if (tid == 0) off[E] = all;
    __syncthreads();
}

// In-order ranks of the pairs [q0, q1) by one wavefront, 64 at a time: pair p
// with expert e gets row cnt[e] + (earlier lanes with the same e), and the
// group's first lane advances cnt[e] (cnt: the wavefront's own LDS row).
__device__ __forceinline__ void rank_pairs(const int32_t* __restrict__ topk_idx, int64_t q0, int64_t q1,
                                           int nbits, int32_t* cnt, int32_t* __restrict__ row_of,
                                           int32_t* __restrict__ src_of) {
    const int lane = lane_id();
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int64_t sb = q0; sb < q1; sb += 64) {
        const int64_t p = sb + lane;
        const bool valid = p < q1;
        const int e = valid ? topk_idx[p] : 0;
        const uint64_t m = match_lanes(e, valid, nbits);
        int32_t row = 0;
        if (valid) row = cnt[e] + __popcll(m & lt);
        wave_lds_sync();
        if (valid && (m & lt) == 0ull) cnt[e] = row + __popcll(m);  // group leader advances
        wave_lds_sync();
        if (valid) {
            row_of[p] = row;
            src_of[row] = (int32_t)p;
        }
    }
}

// ---- Fused path (two kernels) ----------------------------------------------

// First half: workgroup c routes the tokens [c CT, (c + 1) CT) (kRouteBlock /
// G tokens per pass) and writes that chunk's expert histogram hist[c][0..E);
// every workgroup also fills its share of src_of with -1 (the real rows are
// written by the second half).
template <int G, int PER>
__global__ void __launch_bounds__(kRouteBlock) route_chunk_kernel(const float* __restrict__ logits, int T,
                                                                  int E, int k, int renorm, int CT,
                                                                  int32_t* __restrict__ topk_idx,
                                                                  float* __restrict__ topk_w,
                                                                  int32_t* __restrict__ err_word,
                                                                  int32_t* __restrict__ hist,
                                                                  int32_t* __restrict__ src_of,
                                                                  int64_t M_cap) {
    __shared__ int32_t s_cnt[MOE_MAX_E];
    __shared__ __align__(16) float s_x[kRouteBlock / 64][kTokenRow<G>];
    for (int e = threadIdx.x; e < E; e += kRouteBlock) s_cnt[e] = 0;
    for (int64_t r = (int64_t)blockIdx.x * kRouteBlock + threadIdx.x; r < M_cap;
         r += (int64_t)gridDim.x * kRouteBlock)
        src_of[r] = -1;
    __syncthreads();
    const int t0 = blockIdx.x * CT, t1 = min(T, t0 + CT);
    // every lane of a group runs the token loop equally often (the group's lane
    // exchanges need all of them); a token at or past t1 is inactive
    for (int tb = t0; tb < t1; tb += kRouteBlock / G) {
        const int t = tb + (int)threadIdx.x / G;
        route_token_any<G, PER>(logits, t < t1 ? T : 0, E, k, renorm, t < t1 ? t : 0, topk_idx, topk_w,
                                err_word, s_cnt, s_x[threadIdx.x >> 6]);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kRouteBlock) hist[(int64_t)blockIdx.x * E + e] = s_cnt[e];
}

// Second half: workgroup c sums all chunk histograms (the expert totals) and
// those of the chunks before c (its chunk's first rank per expert), forms the
// region starts (workgroup 0 writes counts and offsets), then ranks its
// chunk's pairs in order: four quarter-chunks, one per wavefront, each
// starting after the quarters before it. Integer sums only: the layout does
// not depend on the order they are taken in.
__global__ void __launch_bounds__(256) layout_chunk_kernel(const int32_t* __restrict__ topk_idx, int T, int k,
                                                           int E, int nbits, int CT, int nchunks,
                                                           const int32_t* __restrict__ hist,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ row_of,
                                                           int32_t* __restrict__ src_of) {
    __shared__ int32_t s_tot[MOE_MAX_E], s_base[MOE_MAX_E], s_off[MOE_MAX_E + 1];
    __shared__ int32_t s_q[4][MOE_MAX_E];  // quarter-chunk histograms, then their first rows
    __shared__ int32_t s_part[256];
    const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
    const int c = blockIdx.x;
    for (int e = tid; e < E; e += 256) {
        s_tot[e] = 0;
        s_base[e] = 0;
        for (int w = 0; w < 4; ++w) s_q[w][e] = 0;
    }
    __syncthreads();
    // thread (e, part) sums the chunks part, part + parts, ... of expert e
    {
        const int width = min(E, 256), parts = 256 / width;
        const int part = tid / width;
        for (int e0 = 0; e0 < E; e0 += 256) {
            const int e = e0 + tid % width;
            if (e < E && part < parts) {
                int32_t tot = 0, base = 0;
                // 8 loads in flight per thread
                for (int cb = part; cb < nchunks; cb += 8 * parts) {
                    int32_t h[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int cc = cb + u * parts;
                        h[u] = cc < nchunks ? hist[(int64_t)cc * E + e] : 0;
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        tot += h[u];
                        base += cb + u * parts < c ? h[u] : 0;
                    }
                }
                atomicAdd(&s_tot[e], tot);
                atomicAdd(&s_base[e], base);
            }
        }
    }
    // quarter-chunk histograms
    const int64_t p0 = (int64_t)c * CT * k, p1 = min((int64_t)T * k, p0 + (int64_t)CT * k);
    const int64_t qlen = (p1 - p0 + 3) / 4;
    const int64_t q0 = min(p1, p0 + wave * qlen), q1 = min(p1, q0 + qlen);
    for (int64_t p = q0 + lane; p < q1; p += 64) atomicAdd(&s_q[wave][topk_idx[p]], 1);
    __syncthreads();
    aligned_offsets(s_tot, E, s_off, s_part);
    if (c == 0) {
        for (int e = tid; e < E; e += 256) {
            counts[e] = s_tot[e];
            offsets[e] = s_off[e];
        }
        if (tid == 0) offsets[E] = s_off[E];
    }
    for (int e = tid; e < E; e += 256) {
        int32_t run = s_off[e] + s_base[e];
        for (int w = 0; w < 4; ++w) {
            const int32_t h = s_q[w][e];
            s_q[w][e] = run;
            run += h;
        }
    }
    __syncthreads();
    rank_pairs(topk_idx, q0, q1, nbits, s_q[wave], row_of, src_of);
}

// ---- General path (four kernels; any number of chunks) ---------------------

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

// Exclusive scan of the histograms over chunks, one workgroup per expert (each
// thread a run of consecutive chunks), and the expert's count.
__global__ void __launch_bounds__(256) layout_scan_kernel(const int32_t* __restrict__ hist, int nchunks, int E,
                                                          int32_t* __restrict__ base,
                                                          int32_t* __restrict__ counts) {
    __shared__ int32_t s_part[256];
    const int e = blockIdx.x, tid = threadIdx.x;
    const int per = (nchunks + 255) / 256;
    const int c0 = min(nchunks, tid * per), c1 = min(nchunks, c0 + per);
    int32_t run = 0;
    for (int c = c0; c < c1; ++c) run += hist[(int64_t)c * E + e];
    int32_t all;
    int32_t ex = block_scan256(run, s_part, &all) - run;
    for (int c = c0; c < c1; ++c) {
        base[(int64_t)c * E + e] = ex;
        ex += hist[(int64_t)c * E + e];
    }
    if (tid == 0) counts[e] = all;
}

// Region starts from the counts (every workgroup; workgroup 0 writes them),
// then in-order ranks: each wavefront walks its chunk 64 pairs at a time.
__global__ void __launch_bounds__(256) layout_scatter_kernel(const int32_t* __restrict__ topk_idx,
                                                             int64_t P, int E, int nbits,
                                                             int nchunks,
                                                             const int32_t* __restrict__ base,
                                                             const int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ row_of,
                                                             int32_t* __restrict__ src_of) {
    __shared__ int32_t s_tot[MOE_MAX_E], s_off[MOE_MAX_E + 1], s_part[256];
    extern __shared__ int32_t s_cnt[];  // [4][E]
    const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
    for (int e = tid; e < E; e += 256) s_tot[e] = counts[e];
    __syncthreads();
    aligned_offsets(s_tot, E, s_off, s_part);
    if (blockIdx.x == 0)
        for (int e = tid; e <= E; e += 256) offsets[e] = s_off[e];
    const int chunk = blockIdx.x * 4 + wave;
    if (chunk >= nchunks) return;  // wave-private LDS from here on: no block barrier below
    int32_t* cnt = s_cnt + wave * E;
#pragma unroll 4
    for (int e = lane; e < E; e += 64) cnt[e] = base[(int64_t)chunk * E + e] + s_off[e];
    wave_lds_sync();
    const int64_t b0 = (int64_t)chunk * kChunkPairs;
    rank_pairs(topk_idx, b0, min(P, b0 + kChunkPairs), nbits, cnt, row_of, src_of);
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

// How a routing call runs: the fused pair when every second-half workgroup can
// afford to read all chunk histograms (at most kFusedHist entries, and
// kFusedHistReads entries read over the whole grid) with at most
// kFusedPasses token passes per first-half workgroup; else the general path.
struct RoutePlan {
    int G;        // lanes per token
    bool fused;
    int nchunks;  // chunks of the layout sort
    int CT;       // tokens per chunk (fused path)
};
constexpr int64_t kFusedHist = 65536, kFusedHistReads = (int64_t)8 << 20;
constexpr int kFusedPasses = 2;

static RoutePlan route_plan(int T, int k, int E) {
    RoutePlan pl{};
    pl.G = E <= 8 ? 8 : E <= 16 ? 16 : E <= 32 ? 32 : 64;
    for (int passes = 1; passes <= kFusedPasses; passes *= 2) {
        const int64_t ct = (int64_t)(kRouteBlock / pl.G) * passes;
        const int64_t nc = ((int64_t)T + ct - 1) / ct;
        if (nc * E <= kFusedHist && nc * nc * E <= kFusedHistReads) {
            pl.fused = true;
            pl.nchunks = (int)nc;
            pl.CT = (int)ct;
            return pl;
        }
    }
    pl.fused = false;
    pl.nchunks = (int)(((int64_t)T * k + kChunkPairs - 1) / kChunkPairs);
    return pl;
}

int launch_route(const float* logits, int T, int E, int k, int renorm, int32_t* topk_idx,
                 float* topk_w, int32_t* counts, int32_t* offsets, int32_t* row_of,
                 int32_t* src_of, int64_t M_cap, int32_t* err_word, void* ws, hipStream_t s) {
    const RoutePlan pl = route_plan(T, k, E);
    const int64_t P = (int64_t)T * k;
    int32_t* hist = (int32_t*)ws;
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    if (pl.fused) {
        auto first = [&](auto kern) {
            kern<<<pl.nchunks, kRouteBlock, 0, s>>>(logits, T, E, k, renorm, pl.CT, topk_idx, topk_w, err_word,
                                                    hist, src_of, M_cap);
        };
        if (pl.G == 8)
            first(route_chunk_kernel<8, 1>);
        else if (pl.G == 16)
            first(route_chunk_kernel<16, 1>);
        else if (pl.G == 32)
            first(route_chunk_kernel<32, 1>);
        else if (E <= 128)
            first(route_chunk_kernel<64, 2>);
        else if (E <= 256)
            first(route_chunk_kernel<64, 4>);
        else if (E <= 512)
            first(route_chunk_kernel<64, 8>);
        else
            first(route_chunk_kernel<64, MOE_MAX_E / 64>);
        layout_chunk_kernel<<<pl.nchunks, 256, 0, s>>>(topk_idx, T, k, E, nbits, pl.CT, pl.nchunks, hist,
                                                       counts, offsets, row_of, src_of);
        return hipGetLastError() == hipSuccess ? 0 : -4;
    }
    int32_t* base = hist + (int64_t)pl.nchunks * E;
    auto topk = [&](auto kern) {
        const int64_t blocks = ((int64_t)T * pl.G + 255) / 256;
        kern<<<(unsigned)blocks, 256, 0, s>>>(logits, T, E, k, renorm, topk_idx, topk_w, err_word);
    };
    if (pl.G == 8)
        topk(route_topk_kernel<8, 1>);
    else if (pl.G == 16)
        topk(route_topk_kernel<16, 1>);
    else if (pl.G == 32)
        topk(route_topk_kernel<32, 1>);
    else if (E <= 128)
        topk(route_topk_kernel<64, 2>);
    else if (E <= 256)
        topk(route_topk_kernel<64, 4>);
    else if (E <= 512)
        topk(route_topk_kernel<64, 8>);
    else
        topk(route_topk_kernel<64, MOE_MAX_E / 64>);
    const int nblk = (pl.nchunks + 3) / 4;
    const size_t lds = 4 * (size_t)E * sizeof(int32_t);
    layout_hist_kernel<<<nblk, 256, lds, s>>>(topk_idx, P, E, pl.nchunks, hist, src_of, M_cap);
    layout_scan_kernel<<<E, 256, 0, s>>>(hist, pl.nchunks, E, base, counts);
    layout_scatter_kernel<<<nblk, 256, lds, s>>>(topk_idx, P, E, nbits, pl.nchunks, base, counts, offsets,
                                                 row_of, src_of);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

size_t route_workspace_bytes(int T, int k, int E) {
    const RoutePlan pl = route_plan(T, k, E);
    const int64_t words = (pl.fused ? 1 : 2) * (int64_t)pl.nchunks * E;
    return (size_t)words * sizeof(int32_t);
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
