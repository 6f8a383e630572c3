// Grouped GEMMs of the expert MLP on gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
// One kernel template covers every GEMM of the path:
//   ragged-M (rows of the expert-major buffer are the M dimension; the expert
//   of a tile is found from the device offsets):
//     FC1 + SwiGLU epilogue, FC2, FC2 dgrad + dSwiGLU epilogue, FC1 dgrad;
//   ragged-K (the expert's rows are the reduction dimension): both wgrads.
// [Dropless MoE 학습과 NVIDIA Transformer Engine 소개, grouped-GEMM section:
// one call for all experts over their real token counts, empty groups pass
// through; NVIDIA CuTe DSL fusion-kernel page, core-idea section: the GLU is
// applied in the GEMM epilogue over gate/up-interleaved weights and the work
// is built from device-side counts; SonicMoE page, backward-rewrite and GEMM-
// overlapping sections: the dH kernel reloads H in its epilogue and stores
// dH, dS and A'; kernel structure prologue/mainloop/epilogue and software
// pipelining from its GPU-kernel primer and IO-hiding sections.]
//
// Workgroup tile 256 x 256 x 64, 4 wavefronts in a 2 x 2 grid, each owning a
// 128 x 128 sub-tile as 4 x 4 MFMA 32x32 tiles (fp32 accumulators). Operands
// are staged global -> registers -> LDS (two LDS buffers: the next K slab is
// fetched while the current one is multiplied). An operand whose K index is
// contiguous in memory is kept K-major in LDS and read with ds_read_b128; an
// operand whose M/N index is contiguous is kept MN-major and read with the
// gfx950 transpose load ds_read_b64_tr_b16, so no operand is transposed in
// memory. The MFMA is issued with the B fragment as its first operand, which
// leaves each lane holding one output row and 4-column runs: the epilogues
// read/write 8-byte vectors per lane and reduce rows mostly in registers.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 256;

enum Epi { EPI_BF16 = 0, EPI_SWIGLU = 1, EPI_DSWIGLU = 2, EPI_F32 = 3 };

struct GemmArgs {
    const uint16_t* A;  // activations (token rows)
    int64_t lda;
    const uint16_t* B;  // weights (ragged-M) or gradients (ragged-K)
    int64_t ldb;
    int64_t b_estride;  // per-expert stride of B (ragged-M)
    const int32_t* offsets;
    int E;
    int M;  // ragged-K: rows of the output (features of A)
    int N;  // output columns
    int K;  // ragged-M: reduction length
    uint16_t* out0;  // bf16 C / H / dH
    int64_t ld0;
    uint16_t* out1;  // A (SwiGLU) / A' (dSwiGLU)
    int64_t ld1;
    float* outf;  // fp32 C (wgrad) / dS partials
    int64_t ldf;
    int64_t f_estride;
    const uint16_t* aux;  // H for the dSwiGLU epilogue
    int64_t ld_aux;
    const float* topk_w;
    const int32_t* src_of;
    int n_part;  // dS partial columns per row
};

// LDS layouts (offsets in bf16 elements). 16-byte chunks are XOR-swizzled
// with the low bits of the row so that the fragment reads of a wavefront
// spread over the LDS banks.
__device__ __forceinline__ int kmaj_off(int r, int chunk) {  // [256 rows][64 k]
    return r * BK + ((chunk ^ (r & 7)) << 3);
}
__device__ __forceinline__ int mnmaj_off(int k, int chunk) {  // [64 k][256 mn]
    return k * 256 + ((chunk ^ ((k & 7) << 2)) << 3);
}

// Workgroup order -> tile order: consecutive workgroups land on different
// XCDs (round robin over 8); give each XCD a contiguous range of tiles so
// tiles that share operands share an L2.
__device__ __forceinline__ int xcd_remap(int b, int total) {
    const int x = b & 7, i = b >> 3;
    const int q = total >> 3, r = total & 7;
    return x * q + min(x, r) + i;
}

template <bool KMAJ>
struct Stage {
    // Global -> register staging of one 256 x 64 operand slab (8 x 16 B per thread).
    uint4 v[8];
};

template <bool RAGGED_K, bool A_KMAJ, bool B_KMAJ, int EPI>
__global__ void __launch_bounds__(kThreads, 1) grouped_gemm_kernel(GemmArgs p) {
    __shared__ __attribute__((aligned(16))) uint16_t s_a[2][BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t s_b[2][BN * BK];
    __shared__ int s_tiles[MOE_MAX_E + 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int ntn = (p.N + BN - 1) / BN;

    // ---------------------------------------------------------- tile decode
    int e, row0, row_end, n0, m0 = 0, k_begin, k_end;
    if constexpr (!RAGGED_K) {
        // prefix sum of per-expert M tiles (exclusive), E <= 1024
        for (int i = tid; i < p.E; i += kThreads) {
            const int rows = p.offsets[i + 1] - p.offsets[i];
            s_tiles[i + 1] = (rows + BM - 1) / BM;
        }
        if (tid == 0) s_tiles[0] = 0;
        __syncthreads();
        if (tid < 64) {
            int carry = 0;
            for (int base = 0; base < p.E; base += 64) {
                const int i = base + lane;
                int v = (i < p.E) ? s_tiles[i + 1] : 0;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int u = __shfl_up(v, o, 64);
                    if (lane >= o) v += u;
                }
                if (i < p.E) s_tiles[i + 1] = v + carry;
                carry += __shfl(v, 63, 64);
            }
        }
        __syncthreads();
        const int mtiles = s_tiles[p.E];
        const int total = mtiles * ntn;
        if ((int)blockIdx.x >= total) return;
        const int t = xcd_remap(blockIdx.x, total);
        // bands of 8 M tiles, N-tiles inner: neighbours share B column slabs
        constexpr int G = 8;
        const int band = t / (G * ntn);
        const int within = t - band * G * ntn;
        const int bm = min(G, mtiles - band * G);
        const int mt = band * G + within % bm;
        const int nt = within / bm;
        int lo = 0, hi = p.E;  // last expert with s_tiles[e] <= mt
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_tiles[mid] <= mt) lo = mid; else hi = mid;
        }
        e = lo;
        row0 = p.offsets[e] + (mt - s_tiles[e]) * BM;
        row_end = p.offsets[e + 1];
        n0 = nt * BN;
        k_begin = 0;
        k_end = p.K;
    } else {
        const int ntm = (p.M + BM - 1) / BM;
        const int total = gridDim.x;
        const int t = xcd_remap(blockIdx.x, total);
        e = t / (ntm * ntn);
        const int r = t - e * ntm * ntn;
        const int mt = r / ntn, nt = r - (r / ntn) * ntn;
        m0 = mt * BM;
        n0 = nt * BN;
        row0 = 0;
        row_end = 0;
        k_begin = p.offsets[e];
        k_end = p.offsets[e + 1];
    }

    const uint16_t* Bp = RAGGED_K ? p.B : p.B + (int64_t)e * p.b_estride;

    // ---------------------------------------------------------- global loads
    auto load_a = [&](uint4* v, int k0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int id = i * kThreads + tid;
            if constexpr (A_KMAJ) {
                const int r = id >> 3, c = id & 7;
                const int row = row0 + r;
                v[i] = (row < row_end) ? *(const uint4*)(p.A + (int64_t)row * p.lda + k0 + c * 8)
                                       : make_uint4(0, 0, 0, 0);
            } else {
                const int kr = id >> 5, c = id & 31;
                const int col = m0 + c * 8;
                v[i] = (col < p.M) ? *(const uint4*)(p.A + (int64_t)(k0 + kr) * p.lda + col)
                                   : make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto load_b = [&](uint4* v, int k0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int id = i * kThreads + tid;
            if constexpr (B_KMAJ) {
                const int r = id >> 3, c = id & 7;
                const int n = n0 + r;
                v[i] = (n < p.N) ? *(const uint4*)(Bp + (int64_t)n * p.ldb + k0 + c * 8)
                                 : make_uint4(0, 0, 0, 0);
            } else {
                const int kr = id >> 5, c = id & 31;
                const int col = n0 + c * 8;
                v[i] = (col < p.N) ? *(const uint4*)(Bp + (int64_t)(k0 + kr) * p.ldb + col)
                                   : make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto store_a = [&](const uint4* v, uint16_t* s) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int id = i * kThreads + tid;
            const int off = A_KMAJ ? kmaj_off(id >> 3, id & 7) : mnmaj_off(id >> 5, id & 31);
            *(uint4*)(s + off) = v[i];
        }
    };
    auto store_b = [&](const uint4* v, uint16_t* s) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int id = i * kThreads + tid;
            const int off = B_KMAJ ? kmaj_off(id >> 3, id & 7) : mnmaj_off(id >> 5, id & 31);
            *(uint4*)(s + off) = v[i];
        }
    };

    // ---------------------------------------------------------- fragments
    // Fragment of a 32-row (or 32-column) MFMA operand tile at K step ks:
    // lane l holds index (l & 31) and k = 16 ks + 8 (l >> 5) + [0, 8).
    auto frag = [&](const uint16_t* s, bool kmaj, int base, int ks) -> bf16x8_t {
        if (kmaj) {
            const int r = base + (lane & 31);
            const uint4 v = *(const uint4*)(s + kmaj_off(r, 2 * ks + (lane >> 5)));
            return __builtin_bit_cast(bf16x8_t, v);
        } else {
            const int lg = lane & 15;
            const int c = base + 16 * ((lane >> 4) & 1) + 4 * (lg & 3);
            const int k0 = 16 * ks + 8 * (lane >> 5) + (lg >> 2);
            const int o0 = mnmaj_off(k0, c >> 3) + (c & 7);
            const int o1 = mnmaj_off(k0 + 4, c >> 3) + (c & 7);
            const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_t*)(s + o0));
            const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_t*)(s + o1));
            return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16_t){};

    // ---------------------------------------------------------- main loop
    const int nk = (k_end - k_begin) / BK;
    if (nk > 0) {
        uint4 ra[8], rb[8];
        load_a(ra, k_begin);
        load_b(rb, k_begin);
        store_a(ra, s_a[0]);
        store_b(rb, s_b[0]);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            const bool more = kt + 1 < nk;
            if (more) {
                load_a(ra, k_begin + (kt + 1) * BK);
                load_b(rb, k_begin + (kt + 1) * BK);
            }
            const uint16_t* sa = s_a[cur];
            const uint16_t* sb = s_b[cur];
#pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks) {
                bf16x8_t fa[4], fb[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) fa[i] = frag(sa, A_KMAJ, wm * 128 + 32 * i, ks);
#pragma unroll
                for (int j = 0; j < 4; ++j) fb[j] = frag(sb, B_KMAJ, wn * 128 + 32 * j, ks);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
            }
            if (more) {
                store_a(ra, s_a[cur ^ 1]);
                store_b(rb, s_b[cur ^ 1]);
            }
            __syncthreads();
        }
    }

    // ---------------------------------------------------------- epilogue
    // lane holds row (l & 31) of each 32 x 32 tile and, in register 4q + s,
    // column 8q + 4h + s with h = l >> 5.
    const int h = lane >> 5;
    const int rbase = (RAGGED_K ? m0 : row0) + wm * 128 + (lane & 31);
    const int cbase = n0 + wn * 128 + 4 * h;

    if constexpr (EPI == EPI_F32) {
        float* out = p.outf + (int64_t)e * p.f_estride;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = rbase + 32 * i;
            if (m >= p.M) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (n0 + wn * 128 + 32 * j >= p.N) continue;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = cbase + 32 * j + 8 * q;
                    float4 v = make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                           acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                    *(float4*)(out + (int64_t)m * p.ldf + c) = v;
                }
            }
        }
    } else if constexpr (EPI == EPI_BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = rbase + 32 * i;
            if (m >= row_end) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (n0 + wn * 128 + 32 * j >= p.N) continue;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = cbase + 32 * j + 8 * q;
                    uint2 v;
                    v.x = pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
                    v.y = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                    *(uint2*)(p.out0 + (int64_t)m * p.ld0 + c) = v;
                }
            }
        }
    } else if constexpr (EPI == EPI_SWIGLU) {
        // columns come in (gate 32, up 32) pairs: tiles j = 2u (gate), 2u+1 (up)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = rbase + 32 * i;
            if (m >= row_end) continue;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int hc = n0 + wn * 128 + 64 * u;  // first gate column of the pair
                if (hc >= p.N) continue;
                const int ac = hc / 2 + 4 * h;          // output column base
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float av[4];
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const float g = acc[i][2 * u][4 * q + s];
                        const float up = acc[i][2 * u + 1][4 * q + s];
                        av[s] = g / (1.f + __expf(-g)) * up;
                    }
                    uint2 v;
                    v.x = pack_bf16x2(av[0], av[1]);
                    v.y = pack_bf16x2(av[2], av[3]);
                    *(uint2*)(p.out1 + (int64_t)m * p.ld1 + ac + 8 * q) = v;
                    if (p.out0) {
                        uint2 g2, u2;
                        g2.x = pack_bf16x2(acc[i][2 * u][4 * q], acc[i][2 * u][4 * q + 1]);
                        g2.y = pack_bf16x2(acc[i][2 * u][4 * q + 2], acc[i][2 * u][4 * q + 3]);
                        u2.x = pack_bf16x2(acc[i][2 * u + 1][4 * q], acc[i][2 * u + 1][4 * q + 1]);
                        u2.y = pack_bf16x2(acc[i][2 * u + 1][4 * q + 2], acc[i][2 * u + 1][4 * q + 3]);
                        const int64_t rowp = (int64_t)m * p.ld0;
                        *(uint2*)(p.out0 + rowp + hc + 4 * h + 8 * q) = g2;
                        *(uint2*)(p.out0 + rowp + hc + 32 + 4 * h + 8 * q) = u2;
                    }
                }
            }
        }
    } else if constexpr (EPI == EPI_DSWIGLU) {
        // acc = dA' over activation columns c; H holds (gate, up) interleaved.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = rbase + 32 * i;
            const bool row_ok = m < row_end;
            float w = 0.f;
            if (row_ok) {
                const int src = p.src_of[m];
                w = src >= 0 ? p.topk_w[src] : 0.f;
            }
            float dsum = 0.f;
            if (row_ok) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int ct = n0 + wn * 128 + 32 * j;  // first column of the tile
                    if (ct >= p.N) continue;
                    const int gcol = 2 * ct;                 // gate block of this 32-column tile
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int cc = 8 * q + 4 * h;        // column within the tile
                        const int64_t hrow = (int64_t)m * p.ld_aux;
                        float g[4], uu[4];
                        unpack_bf16x4(*(const uint2*)(p.aux + hrow + gcol + cc), g);
                        unpack_bf16x4(*(const uint2*)(p.aux + hrow + gcol + 32 + cc), uu);
                        float dg[4], du[4], aw[4];
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            const float sg = 1.f / (1.f + __expf(-g[s]));
                            const float sl = g[s] * sg;
                            const float a = sl * uu[s];
                            const float dap = acc[i][j][4 * q + s];
                            dsum = fmaf(dap, a, dsum);
                            const float da = w * dap;
                            dg[s] = da * uu[s] * sg * (1.f + g[s] * (1.f - sg));
                            du[s] = da * sl;
                            aw[s] = w * a;
                        }
                        const int64_t drow = (int64_t)m * p.ld0;
                        uint2 v;
                        v.x = pack_bf16x2(dg[0], dg[1]);
                        v.y = pack_bf16x2(dg[2], dg[3]);
                        *(uint2*)(p.out0 + drow + gcol + cc) = v;
                        v.x = pack_bf16x2(du[0], du[1]);
                        v.y = pack_bf16x2(du[2], du[3]);
                        *(uint2*)(p.out0 + drow + gcol + 32 + cc) = v;
                        v.x = pack_bf16x2(aw[0], aw[1]);
                        v.y = pack_bf16x2(aw[2], aw[3]);
                        *(uint2*)(p.out1 + (int64_t)m * p.ld1 + ct + cc) = v;
                    }
                }
            }
            dsum += __shfl_xor(dsum, 32, 64);  // the partner lane holds the other half
            if (row_ok && h == 0) p.outf[(int64_t)m * p.n_part + (n0 / BN) * 2 + wn] = dsum;
        }
    }
}

// dS[t, j] = sum of the partials of row row_of[t*k+j] in ascending order.
__global__ void __launch_bounds__(256) ds_reduce_kernel(const float* __restrict__ part,
                                                        const int32_t* __restrict__ row_of,
                                                        int64_t P, int n_part,
                                                        float* __restrict__ ds) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= P) return;
    const float* r = part + (int64_t)row_of[i] * n_part;
    float s = 0.f;
    for (int c = 0; c < n_part; ++c) s += r[c];
    ds[i] = s;
}

// ------------------------------------------------------------------ launchers
static int ragged_m_grid(int64_t M_cap, int E, int N) {
    // upper bound on M tiles: every expert region is 128-row aligned, so
    // sum_e ceil(rows_e / 256) <= M_cap / 256 + E
    const int64_t mt = M_cap / BM + E + 1;
    int64_t g = mt * ((N + BN - 1) / BN);
    return (int)g;
}

template <bool RAGGED_K, bool A_KMAJ, bool B_KMAJ, int EPI>
static int run(const GemmArgs& a, int grid, hipStream_t s) {
    if (grid <= 0) return 0;
    grouped_gemm_kernel<RAGGED_K, A_KMAJ, B_KMAJ, EPI><<<grid, kThreads, 0, s>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

static GemmArgs zero_args() {
    GemmArgs a;
    __builtin_memset(&a, 0, sizeof(a));
    return a;
}

int ds_partials_per_row(int n) { return 2 * ((n + BN - 1) / BN); }

int launch_fc1_swiglu(const uint16_t* x_perm, const uint16_t* w1, const int32_t* offsets, int E,
                      int d, int n, int64_t M_cap, uint16_t* h, uint16_t* a, hipStream_t s) {
    GemmArgs g = zero_args();
    g.A = x_perm; g.lda = d;
    g.B = w1; g.ldb = 2 * n; g.b_estride = (int64_t)d * 2 * n;
    g.offsets = offsets; g.E = E; g.N = 2 * n; g.K = d;
    g.out0 = h; g.ld0 = 2 * n;
    g.out1 = a; g.ld1 = n;
    return run<false, true, false, EPI_SWIGLU>(g, ragged_m_grid(M_cap, E, 2 * n), s);
}

int launch_fc2(const uint16_t* a, const uint16_t* w2, const int32_t* offsets, int E, int d, int n,
               int64_t M_cap, uint16_t* y, hipStream_t s) {
    GemmArgs g = zero_args();
    g.A = a; g.lda = n;
    g.B = w2; g.ldb = d; g.b_estride = (int64_t)n * d;
    g.offsets = offsets; g.E = E; g.N = d; g.K = n;
    g.out0 = y; g.ld0 = d;
    return run<false, true, false, EPI_BF16>(g, ragged_m_grid(M_cap, E, d), s);
}

int launch_dgrad2_dswiglu(const uint16_t* dy_u, const uint16_t* w2, const uint16_t* h,
                          const float* topk_w, const int32_t* src_of, const int32_t* offsets,
                          int E, int d, int n, int64_t M_cap, uint16_t* dh, uint16_t* a_w,
                          float* ds_part, hipStream_t s) {
    GemmArgs g = zero_args();
    g.A = dy_u; g.lda = d;
    g.B = w2; g.ldb = d; g.b_estride = (int64_t)n * d;  // row c of W2_e is column c of W2_e^T
    g.offsets = offsets; g.E = E; g.N = n; g.K = d;
    g.out0 = dh; g.ld0 = 2 * n;
    g.out1 = a_w; g.ld1 = n;
    g.outf = ds_part; g.n_part = ds_partials_per_row(n);
    g.aux = h; g.ld_aux = 2 * n;
    g.topk_w = topk_w; g.src_of = src_of;
    return run<false, true, true, EPI_DSWIGLU>(g, ragged_m_grid(M_cap, E, n), s);
}

int launch_ds_reduce(const float* ds_part, const int32_t* row_of, int T, int k, int n,
                     float* ds, hipStream_t s) {
    const int64_t P = (int64_t)T * k;
    ds_reduce_kernel<<<(int)((P + 255) / 256), 256, 0, s>>>(ds_part, row_of, P,
                                                           ds_partials_per_row(n), ds);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_dgrad1(const uint16_t* dh, const uint16_t* w1, const int32_t* offsets, int E, int d,
                  int n, int64_t M_cap, uint16_t* dx_perm, hipStream_t s) {
    GemmArgs g = zero_args();
    g.A = dh; g.lda = 2 * n;
    g.B = w1; g.ldb = 2 * n; g.b_estride = (int64_t)d * 2 * n;  // row r of W1_e = column r of W1_e^T
    g.offsets = offsets; g.E = E; g.N = d; g.K = 2 * n;
    g.out0 = dx_perm; g.ld0 = d;
    return run<false, true, true, EPI_BF16>(g, ragged_m_grid(M_cap, E, d), s);
}

int launch_wgrad(const uint16_t* act, int Ma, const uint16_t* grad, int Nb, const int32_t* offsets,
                 int E, float* dw, hipStream_t s) {
    GemmArgs g = zero_args();
    g.A = act; g.lda = Ma;
    g.B = grad; g.ldb = Nb;
    g.offsets = offsets; g.E = E; g.M = Ma; g.N = Nb;
    g.outf = dw; g.ldf = Nb; g.f_estride = (int64_t)Ma * Nb;
    const int grid = E * ((Ma + BM - 1) / BM) * ((Nb + BN - 1) / BN);
    return run<true, false, false, EPI_F32>(g, grid, s);
}

}  // namespace moe
