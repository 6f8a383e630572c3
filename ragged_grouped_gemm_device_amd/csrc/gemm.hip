// Grouped GEMMs of the expert MLP on gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
// One kernel template covers every GEMM of the path:
//   ragged-M (rows of the expert-major buffer are the M dimension; the expert
//   of a tile is found from the device offsets):
//     FC1 + GLU epilogue (SwiGLU or GeGLU), FC2, FC2 dgrad + dGLU epilogue,
//     FC1 dgrad;
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
// accumulators); in the bf16 modes a wavefront raises its issue priority while
// it runs MFMAs so its sibling's memory instructions fill the gaps. Operands
// move global -> LDS with direct buffer loads (two LDS buffers: the next K slab
// streams in while the current one is multiplied); reads past an expert's rows
// or past N come back as zeros from the buffer bounds. An operand whose K index
// is contiguous in memory is kept K-major in LDS and read with ds_read_b128; an
// operand whose M/N index is contiguous is kept MN-major and read with the
// gfx950 transpose load ds_read_b64_tr_b16, so no operand is transposed in
// memory. The MFMA is issued with the B fragment as its first operand, which
// leaves each lane holding one output row and 4-column runs: the epilogues
// read/write 8-byte vectors per lane and reduce rows mostly in registers.
//
// The kernel is persistent: one workgroup per compute unit walks a static
// tile order, and the first K slab of its next tile is fetched during the
// last slab of the current one, so that load runs under the final MFMAs and
// the epilogue stores. Ragged-K tiles are ordered by their expert's row count,
// longest first, so the short tiles fill the tail of the schedule.
#include <algorithm>

#include "gemm_common.hpp"
#include "mx_common.hpp"

namespace moe {

constexpr int BK = 64;                    // K elements per LDS slab
constexpr int kLoads = BM * BK * 2 / (kThreads * 16);  // 16-byte copies per thread per slab

enum Epi {
    EPI_BF16 = 0, EPI_GLU = 1, EPI_DGLU = 2, EPI_F32 = 3, EPI_GLU_MX = 4, EPI_DGLU_MX = 5,
    EPI_ACT = 6,   // non-gated activation (sReLU): H and A = f(H), same columns
    EPI_DACT = 7,  // its backward: dH = w dA' f'(H), A' = w f(H), dS partials
    EPI_BF16_MX = 8,  // bf16 C (optional) and its row-wise MXFP8 copy (GroupGemm + Quantize)
};

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
    uint16_t* out1;  // A (GLU) / A' (dGLU)
    int64_t ld1;
    float* outf;  // fp32 C (wgrad) / dS partials
    int64_t ldf;
    int64_t f_estride;
    const uint16_t* aux;  // H for the dGLU epilogue
    int64_t ld_aux;
    const float* topk_w;
    const int32_t* src_of;  // expert-major row -> pair index t*k + j (-1: padding)
    int gk;                 // top-k of the routing (gathered operands)
    uint64_t gk_magic;      // ceil(2^64 / gk) for gk > 1: token = src * magic >> 64
    int64_t g_rows;         // rows of the un-permuted tensor a gathered operand reads
    int n_part;  // dS partial columns per row
    uint8_t* q_row;  // MXFP8 copy of A: codes [M_cap, n], scales [M_cap, n/32]
    uint8_t* s_row;
    uint8_t* q_col;  // transposed: codes [n, M_cap], scales [n, M_cap/32] (nullable)
    uint8_t* s_col;
    uint8_t* q2_col;  // dGLU MX: A' transposed codes [n, M_cap], scales [n, M_cap/32]
    uint8_t* s2_col;
    int64_t M_cap;
    // MXFP8 operands (MX kernels): A and B hold E4M3 codes, addressed as pairs
    // of bytes (lda, ldb, b_estride and K count 2-byte units); as and bs hold
    // their block scales, kb bytes per row: A [M_cap, kb], B [E, N, kb]
    const uint8_t* as;
    const uint8_t* bs;
    int kb;
};

// Token of a pair index src = t*k + j without an integer division: with
// magic = ceil(2^64 / k), floor(src * magic / 2^64) = floor(src / k) for every
// 32-bit src when k <= 2^32 (the rounding excess stays below 1/k).
__device__ __forceinline__ int token_of(int src, int k, uint64_t magic) {
    return k == 1 ? src : (int)__umul64hi((uint64_t)(uint32_t)src, magic);
}

// Element offsets (bf16) inside the LDS slabs.
__device__ __forceinline__ int kmaj_off(int r, int chunk) { return kmaj_byte(r, chunk) >> 1; }
__device__ __forceinline__ int mnmaj_off(int k, int chunk) { return mnmaj_byte(k, chunk) >> 1; }

// Where one operand slab comes from: base and readable size from it (the
// buffer resource of slab ks is rebuilt at each issue from base + ks * step,
// a few scalar ops), the byte step per K slab and per copy index, and this
// lane's offset for copy 0 (relative to the slab's own base).
struct SlabSrc {
    const uint16_t* a_base;
    const uint16_t* b_base;
    int64_t a_bytes, b_bytes;
    uint32_t a_step, b_step;
    uint32_t a_istep, b_istep;
    uint32_t a_off, b_off;
    uint32_t g_off[kLoads];  // gathered operand: this lane's offset for copy i (slab 0)
    int g_col0;              // ragged-K gathered operand: first column of the tile
};

// MX: block scales of a tile's A rows and B rows
struct ScaleSrc {
    const uint8_t* as_base;
    const uint8_t* bs_base;
    int64_t as_bytes, bs_bytes;
};

// Enqueue the direct global -> LDS copies of K slab `ks` (A slab then B slab)
// into the LDS stage at `lds`. Copy i of wavefront w fills LDS block i * 8 + w
// (1 KiB); lane l writes chunk l of it. The resource of slab ks starts at the
// slab (base + ks * step, in 64 bits), so lane offsets span one slab's rows:
// below 2^31 for any operand size. A masked lane's offset (kMasked plus less
// than a slab) stays past the resource's end without wrapping.
template <int GATHER>
// part: 0 = the A slab's copies only, 1 = the B slab's only, 2 = both.
__device__ __forceinline__ void issue_slab(const SlabSrc& sr, int ks, LDS_AS char* lds, int wave, int part = 2) {
    const i32x4_t ra = rsrc_from(sr.a_base, sr.a_bytes, (int64_t)ks * sr.a_step);
    const i32x4_t rb = rsrc_from(sr.b_base, sr.b_bytes, (int64_t)ks * sr.b_step);
    const uint32_t l0 = (uint32_t)(uintptr_t)lds + wave * 1024;
    if (part != 1) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
        lds_copy16(ra, l0 + i * kWaves * 1024, GATHER == 1 ? sr.g_off[i] : sr.a_off + i * sr.a_istep);
    }
    if (part != 0) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
        lds_copy16(rb, l0 + BM * BK * 2 + i * kWaves * 1024, GATHER == 2 ? sr.g_off[i] : sr.b_off + i * sr.b_istep);
    }
}

// GATHER: 0, or the operand (1 = A, 2 = B) whose rows are read from an
// un-permuted tensor through src_of (row -> token (src_of / k), -1 -> zeros)
// instead of from an expert-major copy. Ragged M gathers the K-major A rows
// of a tile once per tile; ragged K gathers the K rows of every slab, with
// the token indices of the next slab loaded one copy-issue ahead.
template <bool RAGGED_K, bool A_KMAJ, bool B_KMAJ, int EPI, int ACT, int GATHER, bool MX>
__global__ void __launch_bounds__(kThreads, 1) grouped_gemm_kernel(GemmArgs p) {
    // MX: both operands are K-major E4M3 codes on v_mfma_scale_f32_32x32x64_f8f6f4;
    // a 128-byte slab then holds 128 K values (2 MFMA steps of 64)
    static_assert(!MX || (A_KMAJ && B_KMAJ && !RAGGED_K && GATHER == 0), "MX: K-major, ragged M");
    // per stage: the A slab (BM x BK) then the B slab (BN x BK), 64 KiB
    __shared__ __attribute__((aligned(1024))) uint16_t s_ab[2][(BM + BN) * BK];
    __shared__ int s_tiles[MOE_MAX_E + 1];  // ragged M: tile prefix; ragged K: experts by work
    // MX: block scales of 4 consecutive slabs (a group), 16 bytes for each of the
    // BM A rows then the BN B rows, double-buffered by group
    __shared__ __attribute__((aligned(1024))) uint8_t s_sc[MX ? 2 : 1][MX ? (BM + BN) * 16 : 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / (kWaves / 2), wn = wave % (kWaves / 2);  // 2 x (kWaves / 2) wavefront grid
    const int ntn = (p.N + BN - 1) / BN;
    const int ntm = RAGGED_K ? (p.M + BM - 1) / BM : 0;

    // ---------------------------------------------------------- schedule
    // Persistent workgroups walk a logical tile order. Ragged M: bands of 4 M
    // tiles (8 in the MX mode) with M tiles inner, and each XCD (workgroups are dealt to the 8
    // XCDs round robin) takes a contiguous run of 1/8 of every round. Ragged
    // K: experts by descending row count (longest tiles first), so the tail
    // of the schedule holds the short tiles.
    int total;
    if constexpr (!RAGGED_K) {
        total = ragged_m_prefix(p.offsets, p.E, s_tiles) * ntn;
    } else {
        // sort keys in the operand stage, which no copy has touched yet
        experts_by_rows<kThreads>(p.offsets, p.E, (uint64_t*)&s_ab[0][0], s_tiles);
        total = p.E * ntm * ntn;
    }
    // Round r covers tiles [r nb, (r + 1) nb); within it, XCD x (workgroups
    // b with b % 8 == x) takes the contiguous run starting at x nb / 8, so the
    // tiles live on one XCD at a time are neighbours that share operands in
    // its L2.
    const int nb = gridDim.x;  // a multiple of 8
    auto logical = [&](int round) -> int {
        const int b = blockIdx.x;
        return round * nb + (b & 7) * (nb >> 3) + (b >> 3);
    };

    struct Tile {
        int e, row0, row_end, n0, m0, k_begin, k_end;
    };
    auto get_tile = [&](int t) -> Tile {
        Tile tl;
        if constexpr (!RAGGED_K) {
            const RaggedTile r = ragged_m_decode<MX ? 8 : 4>(p.offsets, p.E, ntn, total / ntn, s_tiles, t);
            tl.e = __builtin_amdgcn_readfirstlane(r.e);
            tl.row0 = __builtin_amdgcn_readfirstlane(r.row0);
            tl.row_end = __builtin_amdgcn_readfirstlane(r.row_end);
            tl.n0 = __builtin_amdgcn_readfirstlane(r.n0);
            tl.m0 = 0;
            tl.k_begin = 0;
            tl.k_end = p.K;
        } else {
            const int per = ntm * ntn;
            const int slot = t / per;
            const int r = t - slot * per;
            tl.e = __builtin_amdgcn_readfirstlane(s_tiles[slot]);
            // bands of 4 M tiles, M inner: an XCD's 32 consecutive tiles form a
            // 4 x 8 window of the expert's output (12 operand panels), not a 1 x 32 row
            constexpr int GK = 4;
            const int band = r / (GK * ntn);
            const int within = r - band * GK * ntn;
            const int bm = min(GK, ntm - band * GK);
            tl.m0 = (band * GK + within % bm) * BM;
            tl.n0 = (within / bm) * BN;
            tl.row0 = tl.row_end = 0;
            tl.k_begin = __builtin_amdgcn_readfirstlane(p.offsets[tl.e]);
            tl.k_end = __builtin_amdgcn_readfirstlane(p.offsets[tl.e + 1]);
        }
        return tl;
    };

    // ---------------------------------------------------------- operand sources
    // Buffer resources bound the readable bytes: rows past the expert's region
    // (ragged M) or past N read as zero; masked lanes use an offset past the end.
    // Copy i of wavefront w fills LDS block i * 8 + w (1 KiB) and lane l writes
    // chunk l of it, so the lane loads whichever global 16-byte chunk the
    // swizzled layout puts there. The swizzle depends only on wave and lane, so
    // a lane's source offset for copy i is its offset for copy 0 plus a
    // uniform stride of i blocks (64 K-major rows or 16 MN-major k rows).
    auto make_src = [&](const Tile& tl) -> SlabSrc {
        SlabSrc sr;
        const uint16_t*& a_base = sr.a_base;
        int64_t& a_bytes = sr.a_bytes;
        if constexpr (!RAGGED_K) {
            // a ragged-M tile reads at most BM rows of its expert
            a_base = p.A + (int64_t)tl.row0 * p.lda;
            a_bytes = (int64_t)min(tl.row_end - tl.row0, BM) * p.lda * 2;
            sr.a_step = BK * 2;
        } else {
            a_base = p.A + (int64_t)tl.k_begin * p.lda;
            a_bytes = (int64_t)(tl.k_end - tl.k_begin) * p.lda * 2;
            sr.a_step = (uint32_t)(BK * p.lda * 2);
        }
        const uint16_t*& b_base = sr.b_base;
        int64_t& b_bytes = sr.b_bytes;
        if constexpr (RAGGED_K) {
            b_base = p.B + (int64_t)tl.k_begin * p.ldb;
            b_bytes = (int64_t)(tl.k_end - tl.k_begin) * p.ldb * 2;
            sr.b_step = (uint32_t)(BK * p.ldb * 2);
        } else if constexpr (B_KMAJ) {
            b_base = p.B + (int64_t)tl.e * p.b_estride + (int64_t)tl.n0 * p.ldb;
            b_bytes = (int64_t)min(p.N - tl.n0, BN) * p.ldb * 2;
            sr.b_step = BK * 2;
        } else {
            b_base = p.B + (int64_t)tl.e * p.b_estride;
            b_bytes = (int64_t)p.K * p.ldb * 2;
            sr.b_step = (uint32_t)(BK * p.ldb * 2);
        }
        if constexpr (GATHER == 1) {  // A rows from the un-permuted tensor
            a_base = p.A;
            a_bytes = p.g_rows * p.lda * 2;
            sr.a_step = RAGGED_K ? 0u : (uint32_t)(BK * 2);  // ragged K: offsets are per slab
        }
        if constexpr (GATHER == 2) {
            b_base = p.B;
            b_bytes = p.g_rows * p.ldb * 2;
            sr.b_step = RAGGED_K ? 0u : (uint32_t)(BK * 2);
        }
        sr.g_col0 = GATHER == 2 ? tl.n0 : tl.m0;
        const int q = wave * 64 + lane;  // copy 0
        if constexpr (GATHER == 1 && !RAGGED_K) {
            // K-major A: copy i reads row (q >> 3) + 64 i of the tile; those rows
            // come from tokens src_of / k (-1: padding row, reads zeros)
            const int r0 = q >> 3, c = (q & 7) ^ kmaj_swz(r0);
#pragma unroll
            for (int i = 0; i < kLoads; ++i) {
                const int gr = tl.row0 + r0 + i * (kThreads / 8);
                const int src = gr < tl.row_end ? p.src_of[gr] : -1;
                sr.g_off[i] = src >= 0 ? (uint32_t)(((int64_t)token_of(src, p.gk, p.gk_magic) * p.lda + c * 8) * 2)
                                       : kMasked;
            }
        }
        if constexpr (A_KMAJ) {
            const int r = q >> 3, c = (q & 7) ^ kmaj_swz(r);
            sr.a_off = (uint32_t)((r * p.lda + c * 8) * 2);
            sr.a_istep = (uint32_t)(kThreads / 8 * p.lda * 2);
        } else {
            const int kr = q >> 5, c = (q & 31) ^ ((kr & 7) << 2);
            const int col = tl.m0 + c * 8;
            sr.a_off = col < p.M ? (uint32_t)((kr * p.lda + col) * 2) : kMasked;
            sr.a_istep = (uint32_t)(kThreads / 32 * p.lda * 2);
        }
        if constexpr (B_KMAJ) {
            const int r = q >> 3, c = (q & 7) ^ kmaj_swz(r);
            sr.b_off = (uint32_t)((r * p.ldb + c * 8) * 2);
            sr.b_istep = (uint32_t)(kThreads / 8 * p.ldb * 2);
        } else {
            const int kr = q >> 5, c = (q & 31) ^ ((kr & 7) << 2);
            const int col = tl.n0 + c * 8;
            sr.b_off = col < p.N ? (uint32_t)((kr * p.ldb + col) * 2) : kMasked;
            sr.b_istep = (uint32_t)(kThreads / 32 * p.ldb * 2);
        }
        return sr;
    };

    // Ragged-K gather: the token rows of a slab are fetched (one global load by
    // each of the first BK threads) while the slab before it is multiplied,
    // staged into a two-slot LDS table just before that slab's closing barrier,
    // and read from there by every lane that copies a row: the copies never
    // wait on the fetch, and each lane keeps one register for it, not four.
    // The table holds each row's byte offset in the gathered tensor (token *
    // leading dimension * 2), or kMasked for a padding row.
    __shared__ uint32_t s_tok[RAGGED_K && GATHER != 0 ? 2 : 1][BK];
    int tok_reg = -1;
    int n_issue = 0;  // copies issued so far: issue n reads slot n & 1
    auto fetch_toks = [&](const Tile& tl, int ks) {
        if (tid < BK) {
            const int gr = tl.k_begin + ks * BK + tid;
            tok_reg = gr < tl.k_end ? p.src_of[gr] : -1;
        }
    };
    // after a vector-memory wait, before a barrier: the table for the next issue
    auto stash_toks = [&]() {
        if constexpr (RAGGED_K && GATHER != 0) {
            if (tid < BK) {
                const int64_t ld = GATHER == 1 ? p.lda : p.ldb;
                s_tok[n_issue & 1][tid] =
                    tok_reg >= 0 ? (uint32_t)((int64_t)token_of(tok_reg, p.gk, p.gk_magic) * ld * 2) : kMasked;
            }
        }
    };
    auto issue = [&](const SlabSrc& sr, int ks_idx, int buf, int part = 2) {
        LDS_AS char* lds = (LDS_AS char*)(&s_ab[buf][0]);
        if constexpr (RAGGED_K && GATHER != 0) {
            // MN-major gathered operand: chunk (k row, column c) of token tok
            SlabSrc g = sr;
            const int q = wave * 64 + lane;
            const int kr = q >> 5, c = (q & 31) ^ ((kr & 7) << 2);
            const int col = sr.g_col0 + c * 8;
            const int lim = GATHER == 1 ? p.M : p.N;
            const uint32_t* tk = s_tok[n_issue & 1];
            ++n_issue;
            // a padding row's kMasked plus the column stays past the buffer end
            uint32_t ro[kLoads];
#pragma unroll
            for (int i = 0; i < kLoads; ++i) ro[i] = tk[kr + i * (kThreads / 32)];
#pragma unroll
            for (int i = 0; i < kLoads; ++i) g.g_off[i] = col < lim ? ro[i] + (uint32_t)(col * 2) : kMasked;
            issue_slab<GATHER>(g, ks_idx, lds, wave);  // the gathered operand's slab step is 0
        } else {
            issue_slab<GATHER>(sr, ks_idx, lds, wave, part);
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
    bf16x8_t fa[2][4], fb[2][TNW];
    // the first MFMA row's operands of K step ks (B fragments, A fragment 0);
    // the other A fragments are requested after that row's MFMAs are issued
    auto load_row0 = [&](int set, int buf, int ks) {
        const uint16_t* sa = s_ab[buf];
        const uint16_t* sb = s_ab[buf] + BM * BK;
        fb[set][0] = frag(sb, B_KMAJ, wn * WN, ks);
        fa[set][0] = frag(sa, A_KMAJ, wm * 128, ks);
#pragma unroll
        for (int j = 1; j < TNW; ++j) fb[set][j] = frag(sb, B_KMAJ, wn * WN + 32 * j, ks);
    };
    f32x16_t acc[4][TNW];

    // ---------------------------------------------------------- MX scales
    // The block scales of 4 slabs travel together: one 16-byte copy per A row
    // and per B row (wavefronts 0-3 the A rows, 4-7 the B rows) straight into
    // LDS, a group ahead; each lane then reads its rows' words one slab ahead.
    // Bytes past a row's valid K read whatever follows (or 0 past the region)
    // and are never used.
    auto make_scales = [&](const Tile& tl) -> ScaleSrc {
        ScaleSrc sc;
        sc.as_base = p.as + (int64_t)tl.row0 * p.kb;
        sc.as_bytes = (int64_t)min(tl.row_end - tl.row0, BM) * p.kb;
        sc.bs_base = p.bs + ((int64_t)tl.e * p.N + tl.n0) * p.kb;
        sc.bs_bytes = (int64_t)min(p.N - tl.n0, BN) * p.kb;
        return sc;
    };
    auto issue_scales = [&](const ScaleSrc& sr, int g, int sbuf) {
        if constexpr (MX) {
            const bool a_side = wave < kWaves / 2;
            const int row = (wave % (kWaves / 2)) * 64 + lane;
            const i32x4_t r = a_side ? rsrc_from(sr.as_base, sr.as_bytes, 0) : rsrc_from(sr.bs_base, sr.bs_bytes, 0);
            const uint32_t l = (uint32_t)(uintptr_t)(LDS_AS char*)(&s_sc[sbuf][0]) + wave * 1024;
            lds_copy16(r, l, (uint32_t)(row * p.kb + g * 16));
        }
    };
    uint32_t sa[4], sb[TNW], na[4], nb_[TNW];  // MX: this lane's scale words (current, next slab)
    auto read_scales = [&](int sbuf, int kt4) {
        const uint8_t* base = s_sc[sbuf] + kt4 * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) na[i] = *(const uint32_t*)(base + (wm * 128 + 32 * i + (lane & 31)) * 16);
#pragma unroll
        for (int j = 0; j < TNW; ++j)
            nb_[j] = *(const uint32_t*)(base + (BM + wn * WN + 32 * j + (lane & 31)) * 16);
    };
    // shifted by this half-wave's block: K step ks then finds its scale in
    // byte 0 after a further shift by 16 ks
    auto take_scales = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) sa[i] = na[i] >> (8 * (lane >> 5));
#pragma unroll
        for (int j = 0; j < TNW; ++j) sb[j] = nb_[j] >> (8 * (lane >> 5));
    };
    // one 128-byte slab on the scaled MFMA: a lane's operand for K step ks is
    // 16-byte chunks h and 2 + h of its row's 64 step bytes (h = lane half),
    // the scale of block b coming from lane half b
    auto mx_slab = [&](int buf) {
        const uint8_t* sA = (const uint8_t*)s_ab[buf];
        const uint8_t* sB = sA + BM * BK * 2;
        const int hh = lane >> 5;
        auto xfrag = [&](const uint8_t* s, int base, int ks) -> i32x8_t {
            const int r = base + (lane & 31);
            const i32x4_t lo = *(const i32x4_t*)(s + kmaj_byte(r, 4 * ks + hh));
            const i32x4_t hi = *(const i32x4_t*)(s + kmaj_byte(r, 4 * ks + 2 + hh));
            return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        // the first MFMA's operands (B, then A row 0) first; the MFMAs go column by
        // column (all A rows with B fragment 0, then with B fragment 1), so each
        // fragment of the next K step is requested right after its last MFMA of this
        // step: at least three MFMAs before its first use (every accumulator's MFMA
        // order unchanged)
        i32x8_t xa[4], xb[TNW];
#pragma unroll
        for (int j = 0; j < TNW; ++j) xb[j] = xfrag(sB, wn * WN + 32 * j, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) xa[i] = xfrag(sA, wm * 128 + 32 * i, 0);
        // no MFMA-phase issue priority here (measured 1.5% faster on MX FC1, unlike the
        // bf16 modes, where it gains 2.3%)
        static_for<2>([&](auto KS) {
            constexpr int ks = KS;
            static_for<TNW>([&](auto J) {
                static_for<4>([&](auto I) {
                    acc[I][J] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        xb[J], xa[I], acc[I][J], 0, 0, 0, (int)(sb[J] >> (16 * ks)), 0, (int)(sa[I] >> (16 * ks)));
                    if constexpr (ks == 0 && J + 1 == TNW) xa[I] = xfrag(sA, wm * 128 + 32 * I, 1);
                });
                if constexpr (ks == 0) xb[J] = xfrag(sB, wn * WN + 32 * J, 1);
            });
        });
        // keep the MFMAs above the slab barrier (left alone, the compiler sinks
        // them below it and serialises the copy wait with the multiply)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < TNW; ++j) asm volatile("" : "+v"(acc[i][j]));
    };

    // ---------------------------------------------------------- tile loop
    int round = 0;
    int t = logical(0);
    if (t >= total) return;
    Tile tl = get_tile(t);
    SlabSrc src = make_src(tl);
    int nk = (tl.k_end - tl.k_begin) / BK;
    int buf0 = 0;  // LDS buffer holding slab 0 of the current tile
    constexpr bool kTok = RAGGED_K && GATHER != 0;
    constexpr bool kSplitCopies = !kTok && !MX && EPI != EPI_DGLU;  // A and B copies in different K steps
    // (a non-empty ragged-K tile has at least two slabs: expert regions are
    // 128-row multiples, so the token prefetch below never runs past a tile)
    if (nk > 0) {
        if constexpr (kTok) {
            fetch_toks(tl, 0);
            __builtin_amdgcn_s_waitcnt(0);
            stash_toks();
            __syncthreads();
        }
        issue(src, 0, 0);
        if constexpr (MX) issue_scales(make_scales(tl), 0, 0);
        if constexpr (kTok) fetch_toks(tl, 1);
    }
    int sg0 = 0;  // MX: scale buffer holding group 0 of the current tile
    bool have_next = false;
    for (;;) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < TNW; ++j) acc[i][j] = (f32x16_t){};
        // the next tile of this workgroup; its first slab is fetched while the
        // current tile finishes, so its latency hides behind MFMAs and stores
        const int tn = logical(round + 1);
        have_next = tn < total;
        Tile tl_next = tl;
        SlabSrc src_next = src;
        int nk_next = 0;
        if (have_next) {
            tl_next = get_tile(tn);
            src_next = make_src(tl_next);
            nk_next = (tl_next.k_end - tl_next.k_begin) / BK;
        }
        int next_buf0 = buf0;
        const int ng = (nk + 3) / 4;  // MX: scale groups of this tile
        if (nk > 0) {
            __builtin_amdgcn_s_waitcnt(0);
            stash_toks();
            __syncthreads();
            if constexpr (MX) {
                read_scales(sg0, 0);
                take_scales();
            } else {
                load_row0(0, buf0, 0);
            }
            for (int kt = 0; kt < nk; ++kt) {
                // No vector-memory load is in flight here in the steady state (the
                // previous slab ended with a full wait), so this wait is free; it
                // makes registers reloaded from scratch before the loop ready on
                // entry, instead of the compiler waiting for them inside the loop,
                // where the same counter also tracks the slab copies.
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
                const int cur = (buf0 + kt) & 1;
                const bool last = kt + 1 == nk;
                // The next slab's copies (part: 0 = A, 1 = B, 2 = both). In the bf16
                // modes they are issued after the second MFMA row of the slab's
                // first K step (the B copies one step later when split), so that
                // the first MFMAs after the barrier do not wait behind the copies'
                // issue; they still have most of the slab to land.
                auto do_issue = [&](int part) {
                if (!last) {
                    issue(src, kt + 1, cur ^ 1, part);
                    if constexpr (kTok) {
                        if (kt + 2 < nk) fetch_toks(tl, kt + 2);
                        else if (nk_next > 0) fetch_toks(tl_next, 0);
                    }
                } else if (nk_next > 0) {
                    issue(src_next, 0, cur ^ 1, part);
                    if constexpr (MX) issue_scales(make_scales(tl_next), 0, (sg0 + ng) & 1);
                    if constexpr (kTok) fetch_toks(tl_next, 1);
                }
                };
                if constexpr (MX) do_issue(2);
                if constexpr (MX) {
                    // the next group's scales go to the buffer the previous group
                    // left (its last reads ended before the previous slab barrier);
                    // the next slab's words come from a group that landed at least
                    // one slab barrier ago
                    if ((kt & 3) == 0 && kt + 4 < nk) issue_scales(make_scales(tl), kt / 4 + 1, (sg0 + kt / 4 + 1) & 1);
                    if (!last) read_scales((sg0 + (kt + 1) / 4) & 1, (kt + 1) & 3);
                    mx_slab(cur);
                } else {
                const uint16_t* sa = s_ab[cur];
                const uint16_t* sb = s_ab[cur] + BM * BK;
                static_for<BK / 16>([&](auto KS) {
                    constexpr int ks = KS;
                    constexpr int c = ks & 1;
                    // The next step's fragments are requested after the first row of
                    // this step's MFMAs, not before them: right after the slab barrier
                    // all eight wavefronts ask LDS for fragments at once, and a first
                    // MFMA that also waits behind the next step's loads starts later.
                    // The first MFMA's operands (B0, A0) are requested first.
                    __builtin_amdgcn_s_setprio(1);  // the MFMA phase wins issue over the sibling wavefront
#pragma unroll
                    for (int j = 0; j < TNW; ++j)
                        acc[0][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[c][j], fa[c][0], acc[0][j], 0, 0, 0);
                    if constexpr (ks == 0) {  // the rest of step 0's A fragments (after the barrier
                                              // only the first row's operands were requested)
#pragma unroll
                        for (int i = 1; i < 4; ++i) fa[0][i] = frag(sa, A_KMAJ, wm * 128 + 32 * i, 0);
                    }
                    if constexpr (ks + 1 < BK / 16) {
                        fb[c ^ 1][0] = frag(sb, B_KMAJ, wn * WN, ks + 1);
                        fa[c ^ 1][0] = frag(sa, A_KMAJ, wm * 128, ks + 1);
#pragma unroll
                        for (int j = 1; j < TNW; ++j) fb[c ^ 1][j] = frag(sb, B_KMAJ, wn * WN + 32 * j, ks + 1);
#pragma unroll
                        for (int i = 1; i < 4; ++i) fa[c ^ 1][i] = frag(sa, A_KMAJ, wm * 128 + 32 * i, ks + 1);
                    }
#pragma unroll
                    for (int j = 0; j < TNW; ++j)
                        acc[1][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[c][j], fa[c][1], acc[1][j], 0, 0, 0);
                    // the next slab's A copies here and its B copies one K step later,
                    // spreading the copy issue and the LDS writes it causes (both at
                    // once with a token table, and for the dGLU epilogue kernel, which
                    // measured slower split)
                    if constexpr (ks == 0) do_issue(kSplitCopies ? 0 : 2);
                    if constexpr (ks == 1 && kSplitCopies) {
                        if (!last) issue(src, kt + 1, cur ^ 1, 1);
                        else if (nk_next > 0) issue(src_next, 0, cur ^ 1, 1);
                    }
#pragma unroll
                    for (int i = 2; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < TNW; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[c][j], fa[c][i], acc[i][j], 0, 0, 0);
                    __builtin_amdgcn_s_setprio(0);
                });
                }
                if (!last) {
                    __builtin_amdgcn_s_waitcnt(0);
                    stash_toks();
                    __syncthreads();
                    if constexpr (MX)
                        take_scales();
                    else
                        load_row0(0, cur ^ 1, 0);
                } else {
                    next_buf0 = cur ^ 1;
                }
            }
        } else if (nk_next > 0) {
            if constexpr (kTok) {
                fetch_toks(tl_next, 0);
                __builtin_amdgcn_s_waitcnt(0);
                stash_toks();
                __syncthreads();
            }
            issue(src_next, 0, buf0);
            if constexpr (MX) issue_scales(make_scales(tl_next), 0, sg0);
            if constexpr (kTok) fetch_toks(tl_next, 1);
        }
        const int e = tl.e, row0 = tl.row0, row_end = tl.row_end, n0 = tl.n0, m0 = tl.m0;
        (void)m0;
    // ---------------------------------------------------------- epilogue
    // lane holds row (l & 31) of each 32 x 32 tile and, in register 4q + s,
    // column 8q + 4h + s with h = l >> 5.
    const int h = lane >> 5;
    const int rbase = (RAGGED_K ? m0 : row0) + wm * 128 + (lane & 31);

    // EPI_F32 and EPI_BF16 store through this wavefront's 8 KiB of the LDS
    // stage the tile no longer reads (the next tile's first slab goes to the
    // other one): 32 rows at a time, written in the MFMA layout, read back in
    // whole-row runs. A store instruction then covers 4 rows x 256 B (fp32) or
    // 8 rows x 128 B (bf16) instead of 32 rows x 32 B or 16 B, a quarter of
    // the memory requests for the same bytes. The 16-byte chunks of a staged
    // row are XOR-swizzled by the row so both sides stay free of LDS bank
    // conflicts.
    if constexpr (EPI == EPI_F32 || EPI == EPI_BF16 || EPI == EPI_BF16_MX) {
        __syncthreads();  // the last slab and the previous tile's staging are read out
        uint8_t* stg = (uint8_t*)(&s_ab[next_buf0 ^ 1][0]) + wave * 8192;
        const int r = lane & 31;
        const int rband = (RAGGED_K ? m0 : row0) + wm * 128;
        const int col0 = n0 + wn * WN;
        static_for<4>([&](auto I) {
            if constexpr (EPI == EPI_F32) {
                // row r: 64 floats = 16 chunks, chunk 8J + 2Q + h from this lane
                static_for<TNW>([&](auto J) {
                    static_for<4>([&](auto Q) {
                        const int ch = 8 * J + 2 * Q + h;
                        *(float4*)(stg + r * 256 + ((ch ^ (r & 15)) << 4)) =
                            make_float4(acc[I][J][4 * Q], acc[I][J][4 * Q + 1], acc[I][J][4 * Q + 2],
                                        acc[I][J][4 * Q + 3]);
                    });
                });
                wave_lds_sync();
                float* out = p.outf + (int64_t)e * p.f_estride;
                static_for<8>([&](auto It) {
                    const int R = 4 * It + (lane >> 4), c = lane & 15;
                    const float4 v = *(const float4*)(stg + R * 256 + ((c ^ (R & 15)) << 4));
                    const int m = rband + 32 * I + R, col = col0 + 4 * c;
                    if (m < p.M && col < p.N) st_nt16(out + (int64_t)m * p.ldf + col, v);
                });
            } else {
                // row r: 64 bf16 = 8 chunks, half h of chunk 4J + Q from this lane
                uint32_t pk[TNW][8];  // EPI_BF16_MX: the lane's bf16 pairs of each 32-column block
                static_for<TNW>([&](auto J) {
                    static_for<4>([&](auto Q) {
                        const int ch = 4 * J + Q;
                        uint2 v;
                        v.x = pack_bf16x2(acc[I][J][4 * Q], acc[I][J][4 * Q + 1]);
                        v.y = pack_bf16x2(acc[I][J][4 * Q + 2], acc[I][J][4 * Q + 3]);
                        if constexpr (EPI == EPI_BF16_MX) {
                            pk[J][2 * Q] = v.x;
                            pk[J][2 * Q + 1] = v.y;
                        }
                        *(uint2*)(stg + r * 128 + ((ch ^ ((r >> 1) & 7)) << 4) + 8 * h) = v;
                    });
                });
                if constexpr (EPI == EPI_BF16_MX) {
                    // the row-wise MXFP8 copy of the bf16-rounded output (blocks of 32
                    // columns: lanes l and l ^ 32 share a row, so both take the branch)
                    // and, when asked, its column-wise copy stored transposed (blocks of
                    // 32 rows, which lie wholly inside or past a 128-row region, so the
                    // whole wavefront takes the branch)
                    const int m = rband + 32 * I + r;
                    const int mb = rband + 32 * I;
                    if (m < row_end) {
                        static_for<TNW>([&](auto J) {
                            const int cb = col0 + 32 * J;
                            if (cb < p.N) {
                                mx_rowq32(pk[J], lane, p.q_row + (int64_t)m * p.N + cb,
                                          p.s_row + (int64_t)m * (p.N / 32) + cb / 32);
                                if (p.q_col) {
                                    const int64_t ls = p.M_cap / 32;
                                    mx_colq32(pk[J], lane, p.q_col + (int64_t)cb * p.M_cap + mb, p.M_cap,
                                              p.s_col + (int64_t)cb * ls + mb / 32, ls);
                                }
                            }
                        });
                    }
                }
                wave_lds_sync();
                if (EPI == EPI_BF16 || p.out0) {  // the bf16 output is optional beside its MXFP8 copy
                    static_for<4>([&](auto It) {
                        const int R = 8 * It + (lane >> 3), c = lane & 7;
                        const uint4 v = *(const uint4*)(stg + R * 128 + ((c ^ ((R >> 1) & 7)) << 4));
                        const int m = rband + 32 * I + R, col = col0 + 8 * c;
                        if (m < row_end && col < p.N) st_nt16(p.out0 + (int64_t)m * p.ld0 + col, v);
                    });
                }
            }
            wave_lds_sync();  // read out before the next 32 rows overwrite it
        });
    } else if constexpr (EPI == EPI_GLU_MX) {
        // GLU as below, then the MXFP8 copies of the bf16-rounded A: row-wise
        // blocks (32 columns of a row: 16 in this lane, 16 in lane l ^ 32) and
        // column-wise blocks (32 rows of a column: one per lane of a half-wave).
        // 32-row blocks never straddle experts (regions are 128-row aligned).
        // H leaves through this wavefront's 8 KiB of the free LDS stage, as in
        // the bf16 GLU epilogue: whole 128-byte rows instead of 8-byte pieces.
        const int n = p.N / 2;
        __syncthreads();  // the last slab is read out
        uint8_t* stg = (uint8_t*)(&s_ab[next_buf0 ^ 1][0]) + wave * 8192;
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
                        uint32_t abp[8];  // bf16 A pairs: slots 2r, 2r + 1
                        uint32_t am = 0;
#pragma unroll
                        for (int r = 0; r < 8; ++r) {
                            abp[r] = pack_bf16x2(glu_gate<ACT>(G[2 * r]) * Up[2 * r],
                                                 glu_gate<ACT>(G[2 * r + 1]) * Up[2 * r + 1]);
                            am = max_u16x2(am, abp[r] & 0x7fff7fffu);
                        }
                        static_for<4>([&](auto Q) {
                            if (p.out1)  // the bf16 A is optional: the MX FC2 reads its codes
                                *(uint2*)(p.out1 + (int64_t)m * p.ld1 + ac + 4 * h + 8 * Q) =
                                    make_uint2(abp[2 * Q], abp[2 * Q + 1]);
                            if (p.out0) {
                                const int r = lane & 31;
                                uint2 g2, u2;
                                g2.x = pack_bf16x2(G[4 * Q], G[4 * Q + 1]);
                                g2.y = pack_bf16x2(G[4 * Q + 2], G[4 * Q + 3]);
                                u2.x = pack_bf16x2(Up[4 * Q], Up[4 * Q + 1]);
                                u2.y = pack_bf16x2(Up[4 * Q + 2], Up[4 * Q + 3]);
                                *(uint2*)(stg + r * 128 + ((Q ^ ((r >> 1) & 7)) << 4) + 8 * h) = g2;
                                *(uint2*)(stg + r * 128 + (((4 + Q) ^ ((r >> 1) & 7)) << 4) + 8 * h) = u2;
                            }
                        });
                        if (p.out0) {
                            wave_lds_sync();
                            static_for<4>([&](auto It) {  // H: 8 lanes x 16 B a row
                                const int R = 8 * It + (lane >> 3), c = lane & 7;
                                const uint4 v = *(const uint4*)(stg + R * 128 + ((c ^ ((R >> 1) & 7)) << 4));
                                st_nt16(p.out0 + (int64_t)(mb + R) * p.ld0 + hc + 8 * c, v);
                            });
                            wave_lds_sync();  // read out before the next 32 rows overwrite it
                        }
                        // row-wise block (16 values here, 16 in lane l ^ 32)
                        uint32_t amax = max(am & 0xffffu, am >> 16);
                        amax = max(amax, (uint32_t)__shfl_xor((int)amax, 32, 64));
                        const int er = mx_block_exp(amax);
                        const float invr = mx_inv_scale(er);
                        uint32_t cw[4];
                        static_for<4>([&](auto Q) {
                            cw[Q] = e4m3x4(bf16_lo(abp[2 * Q]) * invr, bf16_hi(abp[2 * Q]) * invr,
                                           bf16_lo(abp[2 * Q + 1]) * invr, bf16_hi(abp[2 * Q + 1]) * invr);
                        });
                        mx_store_row32(cw, lane, p.q_row + (int64_t)m * n + ac);
                        p.s_row[(int64_t)m * (n / 32) + ac / 32] = (uint8_t)(er + 127);  // same byte from both halves
                        // column-wise blocks, stored transposed
                        if (p.q_col) {
                            const int64_t ls = p.M_cap / 32;
                            mx_colq32(abp, lane, p.q_col + (int64_t)ac * p.M_cap + mb, p.M_cap,
                                      p.s_col + (int64_t)ac * ls + mb / 32, ls);
                        }
                    }
                });
            }
        });
    } else if constexpr (EPI == EPI_ACT) {
        // non-gated: A[m, c] = f(H[m, c]) from the fp32 accumulator, H stored when
        // asked. Staged through LDS like the GLU epilogue, 32 rows at a time: the
        // wavefront's 64 columns of A (128 B a row) at 0, of H at 4096, leaving
        // as whole rows.
        __syncthreads();  // the last slab and the previous tile's staging are read out
        uint8_t* stg = (uint8_t*)(&s_ab[next_buf0 ^ 1][0]) + wave * 8192;
        const int r = lane & 31;
        const int rband = row0 + wm * 128;
        const int cw0 = n0 + wn * WN;  // first column of the wavefront
        static_for<4>([&](auto I) {
            static_for<TNW>([&](auto J) {
                static_for<4>([&](auto Q) {
                    float av[4];
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        float f, df;
                        plain_act_grad<ACT>(acc[I][J][4 * Q + s], f, df);
                        av[s] = f;
                    }
                    const int ch = 4 * J + Q;
                    *(uint2*)(stg + r * 128 + ((ch ^ ((r >> 1) & 7)) << 4) + 8 * h) =
                        make_uint2(pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3]));
                    if (p.out0)
                        *(uint2*)(stg + 4096 + r * 128 + ((ch ^ ((r >> 1) & 7)) << 4) + 8 * h) =
                            make_uint2(pack_bf16x2(acc[I][J][4 * Q], acc[I][J][4 * Q + 1]),
                                       pack_bf16x2(acc[I][J][4 * Q + 2], acc[I][J][4 * Q + 3]));
                });
            });
            wave_lds_sync();
            static_for<4>([&](auto It) {  // 8 lanes x 16 B a row
                const int R = 8 * It + (lane >> 3), c = lane & 7;
                const int m = rband + 32 * I + R, col = cw0 + 8 * c;
                const int sw = (c ^ ((R >> 1) & 7)) << 4;
                if (m < row_end && col < p.N) {
                    *(uint4*)(p.out1 + (int64_t)m * p.ld1 + col) = *(const uint4*)(stg + R * 128 + sw);
                    if (p.out0) st_nt16(p.out0 + (int64_t)m * p.ld0 + col, *(const uint4*)(stg + 4096 + R * 128 + sw));
                }
            });
            wave_lds_sync();  // read out before the next 32 rows overwrite it
        });
    } else if constexpr (EPI == EPI_DACT) {
        // acc = dA' (unweighted) over columns c; H [M, n] holds the pre-activation.
        // Staged through LDS like the dGLU epilogue, 32 rows at a time: the
        // wavefront's 64 columns of H come in as whole rows (the next block's
        // loaded while this one is worked on), dH is written back in place and A'
        // at 4096, and both leave as whole rows.
        __syncthreads();  // the last slab and the previous tile's staging are read out
        uint8_t* stg = (uint8_t*)(&s_ab[next_buf0 ^ 1][0]) + wave * 8192;
        const int r = lane & 31;
        const int rband = row0 + wm * 128;
        const int cw0 = n0 + wn * WN;  // first column of the wavefront
        uint4 hv[4];
        auto load_h = [&](int I) {  // 8 lanes x 16 B a row, 8 rows per load
            const int col = cw0 + 8 * (lane & 7);
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int m = rband + 32 * I + 8 * it + (lane >> 3);
                hv[it] = make_uint4(0, 0, 0, 0);
                if (m < row_end && col < p.N) hv[it] = *(const uint4*)(p.aux + (int64_t)m * p.ld_aux + col);
            }
        };
        load_h(0);
        static_for<4>([&](auto I) {
            const int m = rbase + 32 * I;
            const bool row_ok = m < row_end;
            float w = 0.f;
            if (row_ok) {
                const int src = p.src_of[m];
                w = src >= 0 ? p.topk_w[src] : 0.f;
            }
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int R = 8 * it + (lane >> 3), c = lane & 7;
                *(uint4*)(stg + R * 128 + ((c ^ ((R >> 1) & 7)) << 4)) = hv[it];
            }
            if constexpr (I + 1 < 4) load_h(I + 1);
            wave_lds_sync();
            // rows past the region or columns past N hold zeros here and in acc:
            // they add nothing to dsum and are not stored
            float dsum = 0.f;
            static_for<TNW>([&](auto J) {
                static_for<4>([&](auto Q) {
                    const int ch = 4 * J + Q;
                    uint2* ph = (uint2*)(stg + r * 128 + ((ch ^ ((r >> 1) & 7)) << 4) + 8 * h);
                    float hf[4], dh[4], aw[4];
                    unpack_bf16x4(*ph, hf);
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        float f, df;
                        plain_act_grad<ACT>(hf[s], f, df);
                        const float dap = acc[I][J][4 * Q + s];
                        dsum = fmaf(dap, f, dsum);
                        dh[s] = w * dap * df;
                        aw[s] = w * f;
                    }
                    *ph = make_uint2(pack_bf16x2(dh[0], dh[1]), pack_bf16x2(dh[2], dh[3]));
                    *(uint2*)(stg + 4096 + r * 128 + ((ch ^ ((r >> 1) & 7)) << 4) + 8 * h) =
                        make_uint2(pack_bf16x2(aw[0], aw[1]), pack_bf16x2(aw[2], aw[3]));
                });
            });
            wave_lds_sync();
#pragma unroll
            for (int it = 0; it < 4; ++it) {  // dH and A': 8 lanes x 16 B a row
                const int R = 8 * it + (lane >> 3), c = lane & 7;
                const int mr = rband + 32 * I + R, col = cw0 + 8 * c;
                const int sw = (c ^ ((R >> 1) & 7)) << 4;
                if (mr < row_end && col < p.N) {
                    st_nt16(p.out0 + (int64_t)mr * p.ld0 + col, *(const uint4*)(stg + R * 128 + sw));
                    st_nt16(p.out1 + (int64_t)mr * p.ld1 + col, *(const uint4*)(stg + 4096 + R * 128 + sw));
                }
            }
            wave_lds_sync();  // read out before the next block overwrites it
            dsum += __shfl_xor(dsum, 32, 64);  // the partner lane holds the other half
            if (row_ok && h == 0) p.outf[(int64_t)m * p.n_part + (n0 / BN) * (BN / WN) + wn] = dsum;
        });
    } else if constexpr (EPI == EPI_GLU) {
        // Columns come in (gate 32, up 32) pairs: tiles 0 (gate) and 1 (up) of
        // the wavefront. Staged through LDS like EPI_BF16, 32 rows at a time:
        // the H rows of the pair (64 columns, 128 B) at 0, the A rows (32
        // columns, 64 B) at 4096.
        static_assert(TNW == 2, "one (gate, up) pair per wavefront");
        __syncthreads();  // the last slab and the previous tile's staging are read out
        uint8_t* stg = (uint8_t*)(&s_ab[next_buf0 ^ 1][0]) + wave * 8192;
        const int r = lane & 31;
        const int rband = row0 + wm * 128;
        const int hc = n0 + wn * WN;  // first gate column of the pair
        const bool pair_ok = hc < p.N;
        static_for<4>([&](auto I) {
            const f32x16_t& G = acc[I][0];
            const f32x16_t& Up = acc[I][1];
            static_for<4>([&](auto Q) {
                float av[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) av[s] = glu_gate<ACT>(G[4 * Q + s]) * Up[4 * Q + s];
                uint2 v;
                v.x = pack_bf16x2(av[0], av[1]);
                v.y = pack_bf16x2(av[2], av[3]);
                *(uint2*)(stg + 4096 + r * 64 + ((Q ^ ((r >> 1) & 3)) << 4) + 8 * h) = v;
                if (p.out0) {
                    uint2 g2, u2;
                    g2.x = pack_bf16x2(G[4 * Q], G[4 * Q + 1]);
                    g2.y = pack_bf16x2(G[4 * Q + 2], G[4 * Q + 3]);
                    u2.x = pack_bf16x2(Up[4 * Q], Up[4 * Q + 1]);
                    u2.y = pack_bf16x2(Up[4 * Q + 2], Up[4 * Q + 3]);
                    *(uint2*)(stg + r * 128 + ((Q ^ ((r >> 1) & 7)) << 4) + 8 * h) = g2;
                    *(uint2*)(stg + r * 128 + (((4 + Q) ^ ((r >> 1) & 7)) << 4) + 8 * h) = u2;
                }
            });
            wave_lds_sync();
            static_for<2>([&](auto It) {  // A: 4 lanes x 16 B a row
                const int R = 16 * It + (lane >> 2), c = lane & 3;
                const uint4 v = *(const uint4*)(stg + 4096 + R * 64 + ((c ^ ((R >> 1) & 3)) << 4));
                const int m = rband + 32 * I + R;
                if (m < row_end && pair_ok) *(uint4*)(p.out1 + (int64_t)m * p.ld1 + hc / 2 + 8 * c) = v;
            });
            if (p.out0) {
                static_for<4>([&](auto It) {  // H: 8 lanes x 16 B a row
                    const int R = 8 * It + (lane >> 3), c = lane & 7;
                    const uint4 v = *(const uint4*)(stg + R * 128 + ((c ^ ((R >> 1) & 7)) << 4));
                    const int m = rband + 32 * I + R;
                    if (m < row_end && pair_ok) st_nt16(p.out0 + (int64_t)m * p.ld0 + hc + 8 * c, v);
                });
            }
            wave_lds_sync();  // read out before the next 32 rows overwrite it
        });
    } else if constexpr (EPI == EPI_DGLU_MX) {
        // The dGLU epilogue below (its bf16 dH and A' stores are skipped when
        // out0 / out1 are null), then MXFP8 copies of the bf16-rounded dH
        // (row-wise: 32-column gate or up blocks, two lanes per row; column-wise:
        // 32-row blocks, stored transposed [2n, M_cap]) and of A' (column-wise,
        // transposed [n, M_cap]). A 32-row block lies wholly inside or wholly
        // past an expert region (regions are 128-row multiples), so whole blocks
        // are skipped together. The column-wise codes of a wavefront's 128-row
        // band are assembled in LDS (the last slab's buffer, free once every
        // wavefront is past it) and leave as whole 128-byte column lines.
        const int n2 = 2 * p.N;
        const int64_t ls = p.M_cap / 32;
        __syncthreads();
        uint8_t* stg = (uint8_t*)(&s_ab[next_buf0 ^ 1][0]) + wave * 8192;  // gate: 0, up: 4096
        const int band = row0 + wm * 128;                                  // first row of the band
        const int band_rows = min(max(row_end - band, 0), 128);
        // the row-wise codes of one 32-column block (16 bf16 here, 16 in lane l ^ 32)
        // as four words, word Q holding columns 8 Q + 4 h .. + 3; the scale is stored
        auto rowq = [&](const uint32_t* pk, int m, int col0, uint32_t* cw) {
            uint32_t am = 0;
#pragma unroll
            for (int r = 0; r < 8; ++r) am = max_u16x2(am, pk[r] & 0x7fff7fffu);
            uint32_t amax = max(am & 0xffffu, am >> 16);
            amax = max(amax, (uint32_t)__shfl_xor((int)amax, 32, 64));
            const int er = mx_block_exp(amax);
            const float inv = mx_inv_scale(er);
            static_for<4>([&](auto Q) {
                cw[Q] = e4m3x4(bf16_lo(pk[2 * Q]) * inv, bf16_hi(pk[2 * Q]) * inv, bf16_lo(pk[2 * Q + 1]) * inv,
                               bf16_hi(pk[2 * Q + 1]) * inv);
            });
            p.s_row[(int64_t)m * (n2 / 32) + col0 / 32] = (uint8_t)(er + 127);  // same byte from both halves
        };
        // the gate and up blocks of a row: lane half 0 writes the gate block's 32
        // codes, half 1 the up block's, each after trading the other block's four
        // words with lane l ^ 32 (every lane active here)
        auto rowq2 = [&](const uint32_t* pg, const uint32_t* pu, int m, int col0) {
            uint32_t cg[4], cu[4], got[4];
            rowq(pg, m, col0, cg);
            rowq(pu, m, col0 + 32, cu);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t give = h ? cg[q] : cu[q];
                const auto sw = __builtin_amdgcn_permlane32_swap(give, give, false, false);
                got[q] = h ? sw[0] : sw[1];
            }
            uint8_t* dst = p.q_row + (int64_t)m * n2 + col0 + 32 * h;
            if (h) {
                *(uint4*)dst = make_uint4(got[0], cu[0], got[1], cu[1]);
                *(uint4*)(dst + 16) = make_uint4(got[2], cu[2], got[3], cu[3]);
            } else {
                *(uint4*)dst = make_uint4(cg[0], got[0], cg[1], got[1]);
                *(uint4*)(dst + 16) = make_uint4(cg[2], got[2], cg[3], got[3]);
            }
        };
        float wI[4], dsum[4];
        static_for<4>([&](auto I) {
            const int m = rbase + 32 * I;
            wI[I] = 0.f;
            dsum[I] = 0.f;
            if (band + 32 * I < row_end) {
                const int src = p.src_of[m];
                wI[I] = src >= 0 ? p.topk_w[src] : 0.f;
            }
        });
        static_for<TNW>([&](auto J) {
            const int ct = n0 + wn * WN + 32 * J;  // first activation column of the tile
            if (ct < p.N) {
                const int gcol = 2 * ct;
                // One pass over H: dH (bf16 stores, row-wise codes, column-wise codes
                // staged) and A', whose bf16 pairs stay in registers until the dH
                // column codes have left the stage (a second H read for A' cost 8%).
                // Prefetching the next block's H as well made the kernel spill.
                uint32_t awp[4][8];  // A' bf16 pairs of the 4 blocks
                static_for<4>([&](auto I) {
                    const int m = rbase + 32 * I;
                    const int mb = band + 32 * I;  // first row of this 32-row block
                    if (mb < row_end) {
                        const float w = wI[I];
                        const int64_t hrow = (int64_t)m * p.ld_aux;
                        const int64_t drow = (int64_t)m * p.ld0;
                        // the block's H (this lane's 16 gate and 16 up values) requested
                        // at once: loading inside the loop below waited on each pair.
                        // Lane half h loads whole 16-byte chunks h and 2 + h of the gate
                        // and up columns (32 contiguous bytes a row per load, half the
                        // loads of 8-byte pieces) and trades the half it does not use
                        // with lane l ^ 32, which loaded the chunks next to them.
                        uint2 hg[4], hu[4];
                        {
                            uint4 ld[4];
#pragma unroll
                            for (int c = 0; c < 4; ++c)  // gate 8h, gate 16 + 8h, up 8h, up 16 + 8h
                                ld[c] = *(const uint4*)(p.aux + hrow + gcol + 32 * (c >> 1) + 16 * (c & 1) + 8 * h);
#pragma unroll
                            for (int c = 0; c < 4; ++c) {
                                const uint2 lo = make_uint2(ld[c].x, ld[c].y), hi = make_uint2(ld[c].z, ld[c].w);
                                const uint2 keep = h ? hi : lo, give = h ? lo : hi;
                                const auto s0 = __builtin_amdgcn_permlane32_swap(give.x, give.x, false, false);
                                const auto s1 = __builtin_amdgcn_permlane32_swap(give.y, give.y, false, false);
                                const uint2 got = h ? make_uint2(s0[0], s1[0]) : make_uint2(s0[1], s1[1]);
                                uint2* dst = (c >> 1) ? hu : hg;
                                const int q0 = 2 * (c & 1);  // chunks q0 (half 0) and q0 + 1 (half 1)
                                dst[q0] = h ? got : keep;
                                dst[q0 + 1] = h ? keep : got;
                            }
                        }
                        uint32_t dgp[8], dup[8];  // bf16 pairs, slots 2p, 2p + 1
                        static_for<4>([&](auto Q) {
                            const int cc = 8 * Q + 4 * h;
                            float g[4], uu[4], dg[4], du[4], aw[4];
                            unpack_bf16x4(hg[Q], g);
                            unpack_bf16x4(hu[Q], uu);
#pragma unroll
                            for (int s = 0; s < 4; ++s) {
                                float fg, dfg;
                                glu_gate_grad<ACT>(g[s], fg, dfg);
                                const float a = fg * uu[s];
                                const float dap = acc[I][J][4 * Q + s];
                                dsum[I] = fmaf(dap, a, dsum[I]);
                                const float da = w * dap;
                                dg[s] = da * uu[s] * dfg;
                                du[s] = da * fg;
                                aw[s] = w * a;
                            }
                            dgp[2 * Q] = pack_bf16x2(dg[0], dg[1]);
                            dgp[2 * Q + 1] = pack_bf16x2(dg[2], dg[3]);
                            dup[2 * Q] = pack_bf16x2(du[0], du[1]);
                            dup[2 * Q + 1] = pack_bf16x2(du[2], du[3]);
                            awp[I][2 * Q] = pack_bf16x2(aw[0], aw[1]);
                            awp[I][2 * Q + 1] = pack_bf16x2(aw[2], aw[3]);
                            if (p.out0) {  // the bf16 dH is optional: later MX stages read its codes
                                *(uint2*)(p.out0 + drow + gcol + cc) = make_uint2(dgp[2 * Q], dgp[2 * Q + 1]);
                                *(uint2*)(p.out0 + drow + gcol + 32 + cc) = make_uint2(dup[2 * Q], dup[2 * Q + 1]);
                            }
                            if (p.out1)  // the bf16 A' is optional as well
                                *(uint2*)(p.out1 + (int64_t)m * p.ld1 + ct + cc) =
                                    make_uint2(awp[I][2 * Q], awp[I][2 * Q + 1]);
                        });
                        rowq2(dgp, dup, m, gcol);
                        mx_colq32_stage(dgp, lane, stg, I, p.s_col + (int64_t)gcol * ls + mb / 32, ls);
                        mx_colq32_stage(dup, lane, stg + 4096, I, p.s_col + (int64_t)(gcol + 32) * ls + mb / 32, ls);
                    }
                });
                wave_lds_sync();
                mx_stage_flush(stg, lane, p.q_col + (int64_t)gcol * p.M_cap + band, p.M_cap, band_rows);
                mx_stage_flush(stg + 4096, lane, p.q_col + (int64_t)(gcol + 32) * p.M_cap + band, p.M_cap,
                               band_rows);
                wave_lds_sync();
                // A' column-wise codes from the kept pairs
                static_for<4>([&](auto I) {
                    const int mb = band + 32 * I;
                    if (mb < row_end) mx_colq32_stage(awp[I], lane, stg, I, p.s2_col + (int64_t)ct * ls + mb / 32, ls);
                });
                wave_lds_sync();
                mx_stage_flush(stg, lane, p.q2_col + (int64_t)ct * p.M_cap + band, p.M_cap, band_rows);
                wave_lds_sync();
            }
        });
        static_for<4>([&](auto I) {
            const int m = rbase + 32 * I;
            float d = dsum[I] + __shfl_xor(dsum[I], 32, 64);
            if (band + 32 * I < row_end && h == 0) p.outf[(int64_t)m * p.n_part + (n0 / BN) * (BN / WN) + wn] = d;
        });
    } else if constexpr (EPI == EPI_DGLU) {
        // acc = dA' over activation columns c; H holds (gate, up) interleaved by
        // 32-column block. Per 32 rows and 32-column block J, the block's H rows
        // (gate and up, 128 B) come in as whole-row loads into LDS, each lane
        // takes its values in the MFMA layout and writes dH back in place, and
        // dH and A' (64 B a row, at 4096) leave as whole-row stores. The H rows
        // of the next block are loaded while this one is worked on.
        __syncthreads();  // the last slab and the previous tile's staging are read out
        uint8_t* stg = (uint8_t*)(&s_ab[next_buf0 ^ 1][0]) + wave * 8192;
        const int r = lane & 31;
        const int rband = row0 + wm * 128;
        uint4 hv[4];
        auto load_h = [&](int I, int J) {  // 8 lanes x 16 B a row, 8 rows per load
            const int ct = n0 + wn * WN + 32 * J;
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int m = rband + 32 * I + 8 * it + (lane >> 3);
                hv[it] = make_uint4(0, 0, 0, 0);
                if (m < row_end && ct < p.N)
                    hv[it] = *(const uint4*)(p.aux + (int64_t)m * p.ld_aux + 2 * ct + 8 * (lane & 7));
            }
        };
        load_h(0, 0);
        static_for<4>([&](auto I) {
            const int m = rband + 32 * I + r;
            const bool row_ok = m < row_end;
            float w = 0.f;
            if (row_ok) {
                const int src = p.src_of[m];
                w = src >= 0 ? p.topk_w[src] : 0.f;
            }
            float dsum = 0.f;
            static_for<TNW>([&](auto J) {
                const int ct = n0 + wn * WN + 32 * J;  // first column of the block
                const bool blk_ok = ct < p.N;
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const int R = 8 * it + (lane >> 3), c = lane & 7;
                    *(uint4*)(stg + R * 128 + ((c ^ ((R >> 1) & 7)) << 4)) = hv[it];
                }
                if constexpr (J + 1 < TNW) load_h(I, J + 1);
                else if constexpr (I + 1 < 4) load_h(I + 1, 0);
                wave_lds_sync();
                // rows past the region or columns past N hold zeros here and in
                // acc, so they add nothing to dsum and are not stored
                static_for<4>([&](auto Q) {
                    uint2* pg = (uint2*)(stg + r * 128 + ((Q ^ ((r >> 1) & 7)) << 4) + 8 * h);
                    uint2* pu = (uint2*)(stg + r * 128 + (((4 + Q) ^ ((r >> 1) & 7)) << 4) + 8 * h);
                    float g[4], uu[4];
                    unpack_bf16x4(*pg, g);
                    unpack_bf16x4(*pu, uu);
                    float dg[4], du[4], aw[4];
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        float fg, dfg;
                        glu_gate_grad<ACT>(g[s], fg, dfg);
                        const float a = fg * uu[s];
                        const float dap = acc[I][J][4 * Q + s];
                        dsum = fmaf(dap, a, dsum);
                        const float da = w * dap;
                        dg[s] = da * uu[s] * dfg;
                        du[s] = da * fg;
                        aw[s] = w * a;
                    }
                    uint2 v;
                    v.x = pack_bf16x2(dg[0], dg[1]);
                    v.y = pack_bf16x2(dg[2], dg[3]);
                    *pg = v;
                    v.x = pack_bf16x2(du[0], du[1]);
                    v.y = pack_bf16x2(du[2], du[3]);
                    *pu = v;
                    v.x = pack_bf16x2(aw[0], aw[1]);
                    v.y = pack_bf16x2(aw[2], aw[3]);
                    *(uint2*)(stg + 4096 + r * 64 + ((Q ^ ((r >> 1) & 3)) << 4) + 8 * h) = v;
                });
                wave_lds_sync();
#pragma unroll
                for (int it = 0; it < 4; ++it) {  // dH: 8 lanes x 16 B a row
                    const int R = 8 * it + (lane >> 3), c = lane & 7;
                    const uint4 v = *(const uint4*)(stg + R * 128 + ((c ^ ((R >> 1) & 7)) << 4));
                    const int mr = rband + 32 * I + R;
                    if (mr < row_end && blk_ok) st_nt16(p.out0 + (int64_t)mr * p.ld0 + 2 * ct + 8 * c, v);
                }
#pragma unroll
                for (int it = 0; it < 2; ++it) {  // A': 4 lanes x 16 B a row
                    const int R = 16 * it + (lane >> 2), c = lane & 3;
                    const uint4 v = *(const uint4*)(stg + 4096 + R * 64 + ((c ^ ((R >> 1) & 3)) << 4));
                    const int mr = rband + 32 * I + R;
                    if (mr < row_end && blk_ok) st_nt16(p.out1 + (int64_t)mr * p.ld1 + ct + 8 * c, v);
                }
                wave_lds_sync();  // read out before the next block overwrites it
            });
            dsum += __shfl_xor(dsum, 32, 64);  // the partner lane holds the other half
            if (row_ok && h == 0) p.outf[(int64_t)m * p.n_part + (n0 / BN) * (BN / WN) + wn] = dsum;
        });
    }
        if (!have_next) break;
        ++round;
        tl = tl_next;
        src = src_next;
        nk = nk_next;
        buf0 = next_buf0;
        sg0 = (sg0 + ng) & 1;
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
template <bool RAGGED_K, bool A_KMAJ, bool B_KMAJ, int EPI, int ACT = 0, int GATHER = 0, bool MX = false>
static int run(const GemmArgs& a, int64_t tile_bound, hipStream_t s) {
    if (tile_bound <= 0) return 0;
    grouped_gemm_kernel<RAGGED_K, A_KMAJ, B_KMAJ, EPI, ACT, GATHER, MX>
        <<<persistent_grid(tile_bound), kThreads, 0, s>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

static GemmArgs zero_args() {
    GemmArgs a;
    __builtin_memset(&a, 0, sizeof(a));
    return a;
}

int ds_partials_per_row(int n) { return (BN / WN) * ((n + BN - 1) / BN); }

// A GLU-epilogue launch with the activation and gather chosen at run time.
template <bool B_KMAJ, int EPI>
static int run_glu(const GemmArgs& g, int act, bool gather, int64_t tile_bound, hipStream_t s) {
    if constexpr (EPI == EPI_GLU || EPI == EPI_DGLU) {
        if (act == 2) {  // non-gated squared ReLU
            constexpr int EA = EPI == EPI_GLU ? EPI_ACT : EPI_DACT;
            return gather ? run<false, true, B_KMAJ, EA, 2, 1>(g, tile_bound, s)
                          : run<false, true, B_KMAJ, EA, 2, 0>(g, tile_bound, s);
        }
    }
    if (gather)
        return act ? run<false, true, B_KMAJ, EPI, 1, 1>(g, tile_bound, s)
                   : run<false, true, B_KMAJ, EPI, 0, 1>(g, tile_bound, s);
    return act ? run<false, true, B_KMAJ, EPI, 1, 0>(g, tile_bound, s)
               : run<false, true, B_KMAJ, EPI, 0, 0>(g, tile_bound, s);
}

static void set_gather(GemmArgs& g, const GatherSpec& gs) {
    if (!gs.src_of) return;
    g.src_of = gs.src_of;
    g.gk = gs.k;
    g.gk_magic = gs.k > 1 ? ~0ull / (uint64_t)gs.k + 1 : 0;  // ceil(2^64 / k)
    g.g_rows = gs.rows;
}

int launch_fc1_glu(const uint16_t* x_perm, const uint16_t* w1, const int32_t* offsets, int E, int d,
                   int n, int64_t M_cap, int act, const GatherSpec& gx, uint16_t* h, uint16_t* a,
                   hipStream_t s) {
    const int n1 = act == 2 ? n : 2 * n;  // FC1 width: gate+up interleaved, or n (non-gated)
    GemmArgs g = zero_args();
    g.A = x_perm; g.lda = d;
    g.B = w1; g.ldb = n1; g.b_estride = (int64_t)d * n1;
    g.offsets = offsets; g.E = E; g.N = n1; g.K = d;
    g.out0 = h; g.ld0 = n1;
    g.out1 = a; g.ld1 = n;
    set_gather(g, gx);
    return run_glu<false, EPI_GLU>(g, act, gx.src_of != nullptr, ragged_m_grid(M_cap, E, n1), s);
}

int launch_fc1_glu_mx(const uint16_t* x_perm, const uint16_t* w1, const int32_t* offsets, int E,
                      int d, int n, int64_t M_cap, int act, const GatherSpec& gx, uint16_t* h,
                      uint16_t* a, uint8_t* a_q, uint8_t* a_s, uint8_t* at_q, uint8_t* at_s,
                      hipStream_t s) {
    GemmArgs g = zero_args();
    g.A = x_perm; g.lda = d;
    g.B = w1; g.ldb = 2 * n; g.b_estride = (int64_t)d * 2 * n;
    g.offsets = offsets; g.E = E; g.N = 2 * n; g.K = d;
    g.out0 = h; g.ld0 = 2 * n;
    g.out1 = a; g.ld1 = n;
    g.q_row = a_q; g.s_row = a_s; g.q_col = at_q; g.s_col = at_s; g.M_cap = M_cap;
    set_gather(g, gx);
    return run_glu<false, EPI_GLU_MX>(g, act, gx.src_of != nullptr, ragged_m_grid(M_cap, E, 2 * n), s);
}

// MXFP8 operands: codes are passed as 2-byte units (K, lda, ldb, b_estride
// halved), so the slab copies are the bf16 kernel's byte for byte.
int launch_fc1_glu_mxin(const uint8_t* x_q, const uint8_t* x_s, const uint8_t* w1t_q,
                        const uint8_t* w1t_s, const int32_t* offsets, int E, int d, int n,
                        int64_t M_cap, int act, uint16_t* h, uint16_t* a, uint8_t* a_q, uint8_t* a_s,
                        uint8_t* at_q, uint8_t* at_s, hipStream_t s) {
    GemmArgs g = zero_args();
    g.A = (const uint16_t*)x_q; g.lda = d / 2;
    g.B = (const uint16_t*)w1t_q; g.ldb = d / 2; g.b_estride = (int64_t)2 * n * (d / 2);
    g.offsets = offsets; g.E = E; g.N = 2 * n; g.K = d / 2;
    g.as = x_s; g.bs = w1t_s; g.kb = d / 32;
    g.out0 = h; g.ld0 = 2 * n;
    g.out1 = a; g.ld1 = n;
    g.q_row = a_q; g.s_row = a_s; g.q_col = at_q; g.s_col = at_s; g.M_cap = M_cap;
    const int64_t tb = ragged_m_grid(M_cap, E, 2 * n);
    return act ? run<false, true, true, EPI_GLU_MX, 1, 0, true>(g, tb, s)
               : run<false, true, true, EPI_GLU_MX, 0, 0, true>(g, tb, s);
}

int launch_fc2(const uint16_t* a, const uint16_t* w2, const int32_t* offsets, int E, int d, int n,
               int64_t M_cap, uint16_t* y, uint8_t* y_q, uint8_t* y_s, uint8_t* yt_q, uint8_t* yt_s,
               hipStream_t s) {
    GemmArgs g = zero_args();
    g.A = a; g.lda = n;
    g.B = w2; g.ldb = d; g.b_estride = (int64_t)n * d;
    g.offsets = offsets; g.E = E; g.N = d; g.K = n;
    g.out0 = y; g.ld0 = d;
    g.q_row = y_q; g.s_row = y_s;
    g.q_col = yt_q; g.s_col = yt_s; g.M_cap = M_cap;
    if (y_q) return run<false, true, false, EPI_BF16_MX>(g, ragged_m_grid(M_cap, E, d), s);
    return run<false, true, false, EPI_BF16>(g, ragged_m_grid(M_cap, E, d), s);
}

int launch_dgrad2_dglu(const uint16_t* dy_u, const uint16_t* w2, const uint16_t* h,
                       const float* topk_w, const int32_t* src_of, const int32_t* offsets, int E,
                       int d, int n, int64_t M_cap, int act, const GatherSpec& gdy, uint16_t* dh,
                       uint16_t* a_w, float* ds_part, hipStream_t s) {
    GemmArgs g = zero_args();
    g.A = dy_u; g.lda = d;
    g.B = w2; g.ldb = d; g.b_estride = (int64_t)n * d;  // row c of W2_e is column c of W2_e^T
    const int n1 = act == 2 ? n : 2 * n;  // width of H and dH
    g.offsets = offsets; g.E = E; g.N = n; g.K = d;
    g.out0 = dh; g.ld0 = n1;
    g.out1 = a_w; g.ld1 = n;
    g.outf = ds_part; g.n_part = ds_partials_per_row(n);
    g.aux = h; g.ld_aux = n1;
    g.topk_w = topk_w; g.src_of = src_of;
    set_gather(g, gdy);
    return run_glu<true, EPI_DGLU>(g, act, gdy.src_of != nullptr, ragged_m_grid(M_cap, E, n), s);
}

int launch_dgrad2_dglu_mx(const uint16_t* dy_u, const uint16_t* w2, const uint16_t* h,
                          const float* topk_w, const int32_t* src_of, const int32_t* offsets, int E,
                          int d, int n, int64_t M_cap, int act, const GatherSpec& gdy, uint16_t* dh,
                          uint16_t* a_w, float* ds_part, uint8_t* dh_q, uint8_t* dh_s,
                          uint8_t* dht_q, uint8_t* dht_s, uint8_t* awt_q, uint8_t* awt_s,
                          hipStream_t s) {
    GemmArgs g = zero_args();
    g.A = dy_u; g.lda = d;
    g.B = w2; g.ldb = d; g.b_estride = (int64_t)n * d;
    g.offsets = offsets; g.E = E; g.N = n; g.K = d;
    g.out0 = dh; g.ld0 = 2 * n;
    g.out1 = a_w; g.ld1 = n;
    g.outf = ds_part; g.n_part = ds_partials_per_row(n);
    g.aux = h; g.ld_aux = 2 * n;
    g.topk_w = topk_w; g.src_of = src_of;
    g.q_row = dh_q; g.s_row = dh_s; g.q_col = dht_q; g.s_col = dht_s;
    g.q2_col = awt_q; g.s2_col = awt_s; g.M_cap = M_cap;
    set_gather(g, gdy);
    return run_glu<true, EPI_DGLU_MX>(g, act, gdy.src_of != nullptr, ragged_m_grid(M_cap, E, n), s);
}

int launch_dgrad2_dglu_mxin(const uint8_t* dy_q, const uint8_t* dy_s, const uint8_t* w2_q,
                            const uint8_t* w2_s, const uint16_t* h, const float* topk_w,
                            const int32_t* src_of, const int32_t* offsets, int E, int d, int n,
                            int64_t M_cap, int act, uint16_t* dh, uint16_t* a_w, float* ds_part,
                            uint8_t* dh_q, uint8_t* dh_s, uint8_t* dht_q, uint8_t* dht_s,
                            uint8_t* awt_q, uint8_t* awt_s, hipStream_t s) {
    GemmArgs g = zero_args();
    g.A = (const uint16_t*)dy_q; g.lda = d / 2;
    g.B = (const uint16_t*)w2_q; g.ldb = d / 2; g.b_estride = (int64_t)n * (d / 2);
    g.offsets = offsets; g.E = E; g.N = n; g.K = d / 2;
    g.as = dy_s; g.bs = w2_s; g.kb = d / 32;
    g.out0 = dh; g.ld0 = 2 * n;
    g.out1 = a_w; g.ld1 = n;
    g.outf = ds_part; g.n_part = ds_partials_per_row(n);
    g.aux = h; g.ld_aux = 2 * n;
    g.topk_w = topk_w; g.src_of = src_of;
    g.q_row = dh_q; g.s_row = dh_s; g.q_col = dht_q; g.s_col = dht_s;
    g.q2_col = awt_q; g.s2_col = awt_s; g.M_cap = M_cap;
    const int64_t tb = ragged_m_grid(M_cap, E, n);
    return act ? run<false, true, true, EPI_DGLU_MX, 1, 0, true>(g, tb, s)
               : run<false, true, true, EPI_DGLU_MX, 0, 0, true>(g, tb, s);
}

int launch_ds_reduce(const float* ds_part, const int32_t* row_of, int T, int k, int n,
                     float* ds, hipStream_t s) {
    const int64_t P = (int64_t)T * k;
    ds_reduce_kernel<<<(int)((P + 255) / 256), 256, 0, s>>>(ds_part, row_of, P,
                                                           ds_partials_per_row(n), ds);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_dgrad1(const uint16_t* dh, const uint16_t* w1, const int32_t* offsets, int E, int d,
                  int n1, int64_t M_cap, uint16_t* dx_perm, hipStream_t s) {
    GemmArgs g = zero_args();
    g.A = dh; g.lda = n1;
    g.B = w1; g.ldb = n1; g.b_estride = (int64_t)d * n1;  // row r of W1_e = column r of W1_e^T
    g.offsets = offsets; g.E = E; g.N = d; g.K = n1;
    g.out0 = dx_perm; g.ld0 = d;
    return run<false, true, true, EPI_BF16>(g, ragged_m_grid(M_cap, E, d), s);
}

int launch_wgrad(const uint16_t* act, int Ma, const uint16_t* grad, int Nb, const int32_t* offsets,
                 int E, int gather, const GatherSpec& gs, float* dw, hipStream_t s) {
    GemmArgs g = zero_args();
    g.A = act; g.lda = Ma;
    g.B = grad; g.ldb = Nb;
    g.offsets = offsets; g.E = E; g.M = Ma; g.N = Nb;
    g.outf = dw; g.ldf = Nb; g.f_estride = (int64_t)Ma * Nb;
    const int64_t tiles = (int64_t)E * ((Ma + BM - 1) / BM) * ((Nb + BN - 1) / BN);
    if (gather && gs.src_of) {
        set_gather(g, gs);
        return gather == 1 ? run<true, false, false, EPI_F32, 0, 1>(g, tiles, s)
                           : run<true, false, false, EPI_F32, 0, 2>(g, tiles, s);
    }
    return run<true, false, false, EPI_F32>(g, tiles, s);
}

}  // namespace moe
