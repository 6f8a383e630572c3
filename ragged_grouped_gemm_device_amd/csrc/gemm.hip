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
// Workgroup tile 256 x 256 x 64, 8 wavefronts (two per SIMD) in a 2 x 4 grid,
// each owning a 128 x 64 sub-tile as 4 x 2 MFMA 32x32 tiles (fp32
// accumulators); a wavefront raises its issue priority while it runs MFMAs so
// its sibling's memory instructions fill the gaps. Operands move global -> LDS
// with direct buffer loads (two LDS buffers: the next K slab streams in while
// the current one is multiplied); reads past an expert's rows or past N come
// back as zeros from the buffer bounds. An operand whose K index is
// contiguous in memory is kept K-major in LDS and read with ds_read_b128; an
// operand whose M/N index is contiguous is kept MN-major and read with the
// gfx950 transpose load ds_read_b64_tr_b16, so no operand is transposed in
// memory. The MFMA is issued with the B fragment as its first operand, which
// leaves each lane holding one output row and 4-column runs: the epilogues
// read/write 8-byte vectors per lane and reduce rows mostly in registers.
#include "gemm_common.hpp"
#include "mx_common.hpp"

namespace moe {

constexpr int BK = 64;                    // K elements per LDS slab
constexpr int kLoads = BM * BK * 2 / (kThreads * 16);  // 16-byte copies per thread per slab

enum Epi { EPI_BF16 = 0, EPI_SWIGLU = 1, EPI_DSWIGLU = 2, EPI_F32 = 3, EPI_SWIGLU_MX = 4 };

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
    uint8_t* q_row;  // MXFP8 copy of A: codes [M_cap, n], scales [M_cap, n/32]
    uint8_t* s_row;
    uint8_t* q_col;  // transposed: codes [n, M_cap], scales [n, M_cap/32] (nullable)
    uint8_t* s_col;
    int64_t M_cap;
};

// Element offsets (bf16) inside the LDS slabs.
__device__ __forceinline__ int kmaj_off(int r, int chunk) { return kmaj_byte(r, chunk) >> 1; }
__device__ __forceinline__ int mnmaj_off(int k, int chunk) { return mnmaj_byte(k, chunk) >> 1; }

template <bool RAGGED_K, bool A_KMAJ, bool B_KMAJ, int EPI>
__global__ void __launch_bounds__(kThreads, 1) grouped_gemm_kernel(GemmArgs p) {
    // per stage: the A slab (BM x BK) then the B slab (BN x BK), 64 KiB
    __shared__ __attribute__((aligned(1024))) uint16_t s_ab[2][(BM + BN) * BK];
    __shared__ int s_tiles[MOE_MAX_E + 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int ntn = (p.N + BN - 1) / BN;

    // ---------------------------------------------------------- tile decode
    int e, row0, row_end, n0, m0 = 0, k_begin, k_end;
    if constexpr (!RAGGED_K) {
        RaggedTile tile;
        if (!ragged_m_tile(p.offsets, p.E, ntn, s_tiles, tile)) return;
        e = tile.e;
        row0 = tile.row0;
        row_end = tile.row_end;
        n0 = tile.n0;
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

    // ---------------------------------------------------------- operand sources
    // Buffer resources bound the readable bytes: rows past the expert's region
    // (ragged M) or past N read as zero; masked lanes use an offset past the end.
    const uint16_t* a_base;
    uint32_t a_bytes, a_step;
    if constexpr (!RAGGED_K) {
        a_base = p.A + (int64_t)row0 * p.lda;
        a_bytes = (uint32_t)((int64_t)(row_end - row0) * p.lda * 2);
        a_step = BK * 2;
    } else {
        a_base = p.A + (int64_t)k_begin * p.lda;
        a_bytes = (uint32_t)((int64_t)(k_end - k_begin) * p.lda * 2);
        a_step = (uint32_t)(BK * p.lda * 2);
    }
    const uint16_t* b_base;
    uint32_t b_bytes, b_step;
    if constexpr (RAGGED_K) {
        b_base = p.B + (int64_t)k_begin * p.ldb;
        b_bytes = (uint32_t)((int64_t)(k_end - k_begin) * p.ldb * 2);
        b_step = (uint32_t)(BK * p.ldb * 2);
    } else if constexpr (B_KMAJ) {
        b_base = p.B + (int64_t)e * p.b_estride + (int64_t)n0 * p.ldb;
        b_bytes = (uint32_t)((int64_t)(p.N - n0) * p.ldb * 2);
        b_step = BK * 2;
    } else {
        b_base = p.B + (int64_t)e * p.b_estride;
        b_bytes = (uint32_t)((int64_t)p.K * p.ldb * 2);
        b_step = (uint32_t)(BK * p.ldb * 2);
    }
    const __amdgpu_buffer_rsrc_t rsrc_a = make_rsrc(a_base, a_bytes);
    const __amdgpu_buffer_rsrc_t rsrc_b = make_rsrc(b_base, b_bytes);

    // Lane byte offsets of the 8 x 16 B chunks this thread moves per slab.
    // Instruction i of wavefront w fills LDS block i*4 + w (1 KiB); lane l
    // writes chunk l of it, so the lane loads whichever global chunk the
    // swizzled layout puts there.
    uint32_t a_off[kLoads], b_off[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int q = (i * kWaves + wave) * 64 + lane;
        if constexpr (A_KMAJ) {
            const int r = q >> 3, c = (q & 7) ^ kmaj_swz(r);
            a_off[i] = (uint32_t)((r * p.lda + c * 8) * 2);
        } else {
            const int kr = q >> 5, c = (q & 31) ^ ((kr & 7) << 2);
            const int col = m0 + c * 8;
            a_off[i] = col < p.M ? (uint32_t)((kr * p.lda + col) * 2) : kMasked;
        }
        if constexpr (B_KMAJ) {
            const int r = q >> 3, c = (q & 7) ^ kmaj_swz(r);
            b_off[i] = (uint32_t)((r * p.ldb + c * 8) * 2);
        } else {
            const int kr = q >> 5, c = (q & 31) ^ ((kr & 7) << 2);
            const int col = n0 + c * 8;
            b_off[i] = col < p.N ? (uint32_t)((kr * p.ldb + col) * 2) : kMasked;
        }
    }

    // Enqueue the direct global -> LDS copies of K slab `ks_idx` into buffer `buf`.
    auto issue = [&](int ks_idx, int buf) {
        const uint32_t da = (uint32_t)ks_idx * a_step, db = (uint32_t)ks_idx * b_step;
        LDS_AS char* lds = (LDS_AS char*)(&s_ab[buf][0]);
#pragma unroll
        for (int i = 0; i < kLoads; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_a, (LDS_AS void*)(lds + (i * kWaves + wave) * 1024),
                                                     16, a_off[i] + da, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < kLoads; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_b, (LDS_AS void*)(lds + BM * BK * 2 + (i * kWaves + wave) * 1024), 16,
                b_off[i] + db, 0, 0, 0);
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

    f32x16_t acc[4][TNW];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < TNW; ++j) acc[i][j] = (f32x16_t){};

    // ---------------------------------------------------------- main loop
    // Slab kt+1 streams into the other LDS buffer while slab kt is multiplied;
    // the fragments of K step ks+1 are read while the MFMAs of ks run.
    const int nk = (k_end - k_begin) / BK;
    if (nk > 0) {
        bf16x8_t fa[2][4], fb[2][TNW];
        issue(0, 0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        {
            const uint16_t* sa = s_ab[0];
            const uint16_t* sb = s_ab[0] + BM * BK;
#pragma unroll
            for (int i = 0; i < 4; ++i) fa[0][i] = frag(sa, A_KMAJ, wm * 128 + 32 * i, 0);
#pragma unroll
            for (int j = 0; j < TNW; ++j) fb[0][j] = frag(sb, B_KMAJ, wn * WN + 32 * j, 0);
        }
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < nk) issue(kt + 1, cur ^ 1);
            const uint16_t* sa = s_ab[cur];
            const uint16_t* sb = s_ab[cur] + BM * BK;
            static_for<BK / 16>([&](auto KS) {
                constexpr int ks = KS;
                constexpr int c = ks & 1;
                if constexpr (ks + 1 < BK / 16) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) fa[c ^ 1][i] = frag(sa, A_KMAJ, wm * 128 + 32 * i, ks + 1);
#pragma unroll
                    for (int j = 0; j < TNW; ++j) fb[c ^ 1][j] = frag(sb, B_KMAJ, wn * WN + 32 * j, ks + 1);
                }
                __builtin_amdgcn_s_setprio(1);  // the MFMA phase wins issue over the sibling wavefront
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < TNW; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[c][j], fa[c][i], acc[i][j], 0, 0, 0);
                __builtin_amdgcn_s_setprio(0);
            });
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (kt + 1 < nk) {
                const uint16_t* na = s_ab[cur ^ 1];
                const uint16_t* nb = s_ab[cur ^ 1] + BM * BK;
#pragma unroll
                for (int i = 0; i < 4; ++i) fa[0][i] = frag(na, A_KMAJ, wm * 128 + 32 * i, 0);
#pragma unroll
                for (int j = 0; j < TNW; ++j) fb[0][j] = frag(nb, B_KMAJ, wn * WN + 32 * j, 0);
            }
        }
    }

    // ---------------------------------------------------------- epilogue
    // lane holds row (l & 31) of each 32 x 32 tile and, in register 4q + s,
    // column 8q + 4h + s with h = l >> 5.
    const int h = lane >> 5;
    const int rbase = (RAGGED_K ? m0 : row0) + wm * 128 + (lane & 31);
    const int cbase = n0 + wn * WN + 4 * h;

    if constexpr (EPI == EPI_F32) {
        float* out = p.outf + (int64_t)e * p.f_estride;
        static_for<4>([&](auto I) {
            const int m = rbase + 32 * I;
            if (m < p.M) {
                static_for<TNW>([&](auto J) {
                    if (n0 + wn * WN + 32 * J < p.N) {
                        static_for<4>([&](auto Q) {
                            const int c = cbase + 32 * J + 8 * Q;
                            const float4 v = make_float4(acc[I][J][4 * Q], acc[I][J][4 * Q + 1],
                                                         acc[I][J][4 * Q + 2], acc[I][J][4 * Q + 3]);
                            *(float4*)(out + (int64_t)m * p.ldf + c) = v;
                        });
                    }
                });
            }
        });
    } else if constexpr (EPI == EPI_BF16) {
        static_for<4>([&](auto I) {
            const int m = rbase + 32 * I;
            if (m < row_end) {
                static_for<TNW>([&](auto J) {
                    if (n0 + wn * WN + 32 * J < p.N) {
                        static_for<4>([&](auto Q) {
                            const int c = cbase + 32 * J + 8 * Q;
                            uint2 v;
                            v.x = pack_bf16x2(acc[I][J][4 * Q], acc[I][J][4 * Q + 1]);
                            v.y = pack_bf16x2(acc[I][J][4 * Q + 2], acc[I][J][4 * Q + 3]);
                            *(uint2*)(p.out0 + (int64_t)m * p.ld0 + c) = v;
                        });
                    }
                });
            }
        });
    } else if constexpr (EPI == EPI_SWIGLU_MX) {
        // SwiGLU as below, then the MXFP8 copies of the bf16-rounded A: row-wise
        // blocks (32 columns of a row: 16 in this lane, 16 in lane l ^ 32) and
        // column-wise blocks (32 rows of a column: one per lane of a half-wave).
        // 32-row blocks never straddle experts (regions are 128-row aligned).
        const int n = p.N / 2;
        static_for<4>([&](auto I) {
            const int m = rbase + 32 * I;
            const int mb = row0 + wm * 128 + 32 * I;  // first row of this 32-row block
            if (mb < row_end) {
                static_for<TNW / 2>([&](auto U) {
                    const int hc = n0 + wn * WN + 64 * U;
                    if (hc < p.N) {
                        const int ac = hc / 2;  // first A column of the 32-column block
                        const f32x16_t& G = acc[I][2 * U];
                        const f32x16_t& Up = acc[I][2 * U + 1];
                        uint32_t ab[16];
                        uint32_t amax = 0;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const float g = G[r];
                            ab[r] = f32_to_bf16(g / (1.f + __expf(-g)) * Up[r]);
                            amax = max(amax, ab[r] & 0x7fffu);
                        }
                        static_for<4>([&](auto Q) {
                            uint2 v;
                            v.x = ab[4 * Q] | (ab[4 * Q + 1] << 16);
                            v.y = ab[4 * Q + 2] | (ab[4 * Q + 3] << 16);
                            *(uint2*)(p.out1 + (int64_t)m * p.ld1 + ac + 4 * h + 8 * Q) = v;
                            if (p.out0) {
                                uint2 g2, u2;
                                g2.x = pack_bf16x2(G[4 * Q], G[4 * Q + 1]);
                                g2.y = pack_bf16x2(G[4 * Q + 2], G[4 * Q + 3]);
                                u2.x = pack_bf16x2(Up[4 * Q], Up[4 * Q + 1]);
                                u2.y = pack_bf16x2(Up[4 * Q + 2], Up[4 * Q + 3]);
                                const int64_t rowp = (int64_t)m * p.ld0;
                                *(uint2*)(p.out0 + rowp + hc + 4 * h + 8 * Q) = g2;
                                *(uint2*)(p.out0 + rowp + hc + 32 + 4 * h + 8 * Q) = u2;
                            }
                        });
                        // row-wise block
                        amax = max(amax, (uint32_t)__shfl_xor((int)amax, 32, 64));
                        const int er = mx_block_exp(amax);
                        const float invr = mx_inv_scale(er);
                        static_for<4>([&](auto Q) {
                            const uint32_t w = e4m3_rne(bf16_to_f32(ab[4 * Q]) * invr) |
                                               (e4m3_rne(bf16_to_f32(ab[4 * Q + 1]) * invr) << 8) |
                                               (e4m3_rne(bf16_to_f32(ab[4 * Q + 2]) * invr) << 16) |
                                               (e4m3_rne(bf16_to_f32(ab[4 * Q + 3]) * invr) << 24);
                            *(uint32_t*)(p.q_row + (int64_t)m * n + ac + 4 * h + 8 * Q) = w;
                        });
                        if (h == 0) p.s_row[(int64_t)m * (n / 32) + ac / 32] = (uint8_t)(er + 127);
                        // column-wise blocks, stored transposed
                        if (p.q_col) {
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                uint32_t cm = ab[r] & 0x7fffu;
#pragma unroll
                                for (int o = 1; o < 32; o <<= 1) cm = max(cm, (uint32_t)__shfl_xor((int)cm, o, 64));
                                const int ec = mx_block_exp(cm);
                                const int c = ac + 8 * (r >> 2) + 4 * h + (r & 3);
                                p.q_col[(int64_t)c * p.M_cap + m] = (uint8_t)e4m3_rne(bf16_to_f32(ab[r]) * mx_inv_scale(ec));
                                if ((lane & 31) == 0) p.s_col[(int64_t)c * (p.M_cap / 32) + mb / 32] = (uint8_t)(ec + 127);
                            }
                        }
                    }
                });
            }
        });
    } else if constexpr (EPI == EPI_SWIGLU) {
        // columns come in (gate 32, up 32) pairs: tiles j = 2u (gate), 2u+1 (up)
        static_for<4>([&](auto I) {
            const int m = rbase + 32 * I;
            if (m < row_end) {
                static_for<TNW / 2>([&](auto U) {
                    const int hc = n0 + wn * WN + 64 * U;  // first gate column of the pair
                    if (hc < p.N) {
                        const int ac = hc / 2 + 4 * h;      // output column base
                        static_for<4>([&](auto Q) {
                            const f32x16_t& G = acc[I][2 * U];
                            const f32x16_t& Up = acc[I][2 * U + 1];
                            float av[4];
#pragma unroll
                            for (int s = 0; s < 4; ++s) {
                                const float g = G[4 * Q + s];
                                av[s] = g / (1.f + __expf(-g)) * Up[4 * Q + s];
                            }
                            uint2 v;
                            v.x = pack_bf16x2(av[0], av[1]);
                            v.y = pack_bf16x2(av[2], av[3]);
                            *(uint2*)(p.out1 + (int64_t)m * p.ld1 + ac + 8 * Q) = v;
                            if (p.out0) {
                                uint2 g2, u2;
                                g2.x = pack_bf16x2(G[4 * Q], G[4 * Q + 1]);
                                g2.y = pack_bf16x2(G[4 * Q + 2], G[4 * Q + 3]);
                                u2.x = pack_bf16x2(Up[4 * Q], Up[4 * Q + 1]);
                                u2.y = pack_bf16x2(Up[4 * Q + 2], Up[4 * Q + 3]);
                                const int64_t rowp = (int64_t)m * p.ld0;
                                *(uint2*)(p.out0 + rowp + hc + 4 * h + 8 * Q) = g2;
                                *(uint2*)(p.out0 + rowp + hc + 32 + 4 * h + 8 * Q) = u2;
                            }
                        });
                    }
                });
            }
        });
    } else if constexpr (EPI == EPI_DSWIGLU) {
        // acc = dA' over activation columns c; H holds (gate, up) interleaved.
        static_for<4>([&](auto I) {
            const int m = rbase + 32 * I;
            const bool row_ok = m < row_end;
            float w = 0.f;
            if (row_ok) {
                const int src = p.src_of[m];
                w = src >= 0 ? p.topk_w[src] : 0.f;
            }
            float dsum = 0.f;
            if (row_ok) {
                const int64_t hrow = (int64_t)m * p.ld_aux;
                const int64_t drow = (int64_t)m * p.ld0;
                static_for<TNW>([&](auto J) {
                    const int ct = n0 + wn * WN + 32 * J;  // first column of the tile
                    if (ct < p.N) {
                        const int gcol = 2 * ct;             // gate block of this 32-column tile
                        static_for<4>([&](auto Q) {
                            const int cc = 8 * Q + 4 * h;    // column within the tile
                            float g[4], uu[4];
                            unpack_bf16x4(*(const uint2*)(p.aux + hrow + gcol + cc), g);
                            unpack_bf16x4(*(const uint2*)(p.aux + hrow + gcol + 32 + cc), uu);
                            float dg[4], du[4], aw[4];
#pragma unroll
                            for (int s = 0; s < 4; ++s) {
                                const float sg = 1.f / (1.f + __expf(-g[s]));
                                const float sl = g[s] * sg;
                                const float a = sl * uu[s];
                                const float dap = acc[I][J][4 * Q + s];
                                dsum = fmaf(dap, a, dsum);
                                const float da = w * dap;
                                dg[s] = da * uu[s] * sg * (1.f + g[s] * (1.f - sg));
                                du[s] = da * sl;
                                aw[s] = w * a;
                            }
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
                        });
                    }
                });
            }
            dsum += __shfl_xor(dsum, 32, 64);  // the partner lane holds the other half
            if (row_ok && h == 0) p.outf[(int64_t)m * p.n_part + (n0 / BN) * (BN / WN) + wn] = dsum;
        });
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

int ds_partials_per_row(int n) { return (BN / WN) * ((n + BN - 1) / BN); }

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

int launch_fc1_swiglu_mx(const uint16_t* x_perm, const uint16_t* w1, const int32_t* offsets, int E,
                         int d, int n, int64_t M_cap, uint16_t* h, uint16_t* a, uint8_t* a_q,
                         uint8_t* a_s, uint8_t* at_q, uint8_t* at_s, hipStream_t s) {
    GemmArgs g = zero_args();
    g.A = x_perm; g.lda = d;
    g.B = w1; g.ldb = 2 * n; g.b_estride = (int64_t)d * 2 * n;
    g.offsets = offsets; g.E = E; g.N = 2 * n; g.K = d;
    g.out0 = h; g.ld0 = 2 * n;
    g.out1 = a; g.ld1 = n;
    g.q_row = a_q; g.s_row = a_s; g.q_col = at_q; g.s_col = at_s; g.M_cap = M_cap;
    return run<false, true, false, EPI_SWIGLU_MX>(g, ragged_m_grid(M_cap, E, 2 * n), s);
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
