// MXFP8 kernels: standalone block quantization and the MX-scaled grouped FC2.
//
// [Dropless MoE 학습과 NVIDIA Transformer Engine 소개, three-components
// section: group-aware MXFP8 quantization and MXFP8 grouped GEMM; NVIDIA CuTe
// DSL fusion-kernel page, problem section: the BF16 -> MXFP8 pass writes a
// low-precision copy and a transposed copy.]
#include "gemm_common.hpp"
#include "mx_common.hpp"

namespace moe {

// ------------------------------------------------------------------ quant
// One workgroup quantizes a 128 x 128 bf16 tile straight from registers.
// Thread (w, l) of the 4 wavefronts holds 8 rows x 8 columns: columns
// 8 (l & 15) + [0, 8), rows 8 (4 w + (l >> 4)) + [0, 8), loaded as eight
// 16-byte row pieces (16 lanes cover a 256-byte row segment). A row-wise
// block (32 columns) spans 4 neighbouring lanes, a column-wise block (32 rows)
// the 4 lanes l, l ^ 16, l ^ 32, l ^ 48 of one wavefront, so both block maxima
// are two lane exchanges away (done on packed pairs of 16-bit magnitudes: two
// rows, or two columns, per exchange); the transposed copy is assembled in LDS and
// leaves in 16-byte pieces. Conversion uses gfx950's packed E4M3
// instruction, which rounds to nearest-even like the codec above (the scale
// keeps every value within +-448, so it never saturates).
constexpr int QT = 128;  // tile edge
typedef uint32_t nt_u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t nt_u32x4_t __attribute__((ext_vector_type(4)));

// largest magnitude bit pattern (sign cleared) among 8 bf16 values
__device__ __forceinline__ uint32_t abs_max_bf16x8(uint4 v) {
    const uint32_t m = 0x7fff7fffu;
    const u16x2_t a = __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, v.x & m), __builtin_bit_cast(u16x2_t, v.y & m));
    const u16x2_t c = __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, v.z & m), __builtin_bit_cast(u16x2_t, v.w & m));
    const u16x2_t d = __builtin_elementwise_max(a, c);
    return max((uint32_t)d.x, (uint32_t)d.y);
}

// GATHER: row r of the matrix is row src_of[r] / k of src [T, C] (the
// expert-major permutation, with zeros for padding rows, src_of[r] < 0), so
// the permuted bf16 copy is never written.
// NT: the codes leave as streaming (non-temporal) stores, which do not evict
// the source rows from the last-level cache: a gathered row is read k times,
// and a source that fits the cache (as one its producer just wrote does)
// stays there.
template <bool ROW, bool COL, bool GATHER, bool NT>
__global__ void __launch_bounds__(256) quant_mxfp8_kernel(const uint16_t* __restrict__ src, int64_t R,
                                                          int C, uint8_t* __restrict__ q_row,
                                                          uint8_t* __restrict__ s_row,
                                                          uint8_t* __restrict__ q_col,
                                                          uint8_t* __restrict__ s_col,
                                                          const int32_t* __restrict__ src_of, int k) {
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int cc = l & 15, rg = 4 * w + (l >> 4);
    const int64_t b = blockIdx.z;
    const int c = blockIdx.x * QT + 8 * cc;              // first column of this thread
    const int64_t r = (int64_t)blockIdx.y * QT + 8 * rg;  // first row
    const bool cok = c < C;
    src += b * R * C;
    // Scale bytes leave as whole 4-byte words (one per row, one per column of
    // the tile) through LDS when the column pass and its barrier run: 4 single
    // bytes to the same word were 4 separate partial writes. Words need a
    // tile's 4 blocks present and word-aligned scale arrays; else bytes.
    __shared__ __attribute__((aligned(16))) uint8_t s_rs[ROW && COL ? QT * 4 : 4];
    __shared__ __attribute__((aligned(16))) uint8_t s_cs[COL ? QT * 4 : 4];
    const bool rs_words = ROW && COL && (C % 128) == 0 && ((uintptr_t)s_row & 3) == 0;
    const bool cs_words = COL && (R % 128) == 0 && ((uintptr_t)s_col & 3) == 0;
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[i] = make_uint4(0, 0, 0, 0);
        if constexpr (GATHER) {
            const int sr = cok && r + i < R ? src_of[r + i] : -1;
            if (sr >= 0) v[i] = *(const uint4*)(src + (int64_t)(sr / k) * C + c);
        } else {
            if (cok && r + i < R) v[i] = *(const uint4*)(src + (r + i) * C + c);
        }
    }
    if constexpr (ROW) {
        uint8_t* qr = q_row + b * R * C;
        uint8_t* sr = s_row + b * R * (C / 32);
        // block maxima of rows (i, i + 1) travel together as one packed pair
        uint32_t pam[4];
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
            uint32_t pk = abs_max_bf16x8(v[2 * i2]) | (abs_max_bf16x8(v[2 * i2 + 1]) << 16);
            pk = max_u16x2(pk, (uint32_t)__shfl_xor((int)pk, 1, 64));
            pk = max_u16x2(pk, (uint32_t)__shfl_xor((int)pk, 2, 64));
            pam[i2] = pk;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t amax = (i & 1) ? pam[i >> 1] >> 16 : pam[i >> 1] & 0xffffu;
            const int e = mx_block_exp(amax);
            const float inv = mx_inv_scale(e);
            const uint4 x = v[i];
            uint2 q;
            q.x = e4m3x4(bf16_lo(x.x) * inv, bf16_hi(x.x) * inv, bf16_lo(x.y) * inv, bf16_hi(x.y) * inv);
            q.y = e4m3x4(bf16_lo(x.z) * inv, bf16_hi(x.z) * inv, bf16_lo(x.w) * inv, bf16_hi(x.w) * inv);
            if (cok && r + i < R) {
                if constexpr (NT)
                    __builtin_nontemporal_store(__builtin_bit_cast(nt_u32x2_t, q), (nt_u32x2_t*)(qr + (r + i) * C + c));
                else
                    *(uint2*)(qr + (r + i) * C + c) = q;
                if ((cc & 3) == 0) {
                    if (rs_words)
                        s_rs[(8 * rg + i) * 4 + (cc >> 2)] = (uint8_t)(e + 127);
                    else
                        sr[(r + i) * (C / 32) + c / 32] = (uint8_t)(e + 127);
                }
            }
        }
    }
    if constexpr (ROW && COL && GATHER) {
        // Left alone, the compiler keeps the 64 unpacked floats of the row pass
        // live into the column pass (123 VGPRs, 4 wavefronts per SIMD); opaque
        // words make the column pass unpack them again (70 VGPRs, 7 wavefronts).
        // Measured faster for the gathered form (-4 to -5%), slower for the
        // plain quantizer (+2 to +4%), which keeps the first schedule.
#pragma unroll
        for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(v[i].x), "+v"(v[i].y), "+v"(v[i].z), "+v"(v[i].w));
    }
    if constexpr (COL) {
        // R is a multiple of 32 here, so a wavefront's 32-row block is whole or
        // absent. The transposed codes go through LDS ([128 columns][128 rows]
        // bytes) so that they leave as 16-byte pieces, eight lanes per 128-row
        // column segment, instead of 8-byte pieces scattered over 16 columns
        // (which cost a third more time). A thread's 8-byte chunk (8 rows of a
        // column) is XOR-swizzled by its column group, keeping chunk pairs
        // adjacent for the 16-byte reads.
        __shared__ __attribute__((aligned(16))) uint8_t tq[QT * QT];
        uint8_t* qc = q_col + b * R * C;
        uint8_t* sc = s_col + b * R * (C / 32);
        const int64_t RB = R / 32;
        // word p (columns 2p, 2p + 1) of row i of this thread
        auto word = [&](int i, int p) -> uint32_t { return p == 0 ? v[i].x : p == 1 ? v[i].y : p == 2 ? v[i].z : v[i].w; };
        // element (row i, column j) of this thread
        auto elt = [&](int i, int j) -> float {
            const uint32_t w_ = word(i, j >> 1);
            return (j & 1) ? bf16_hi(w_) : bf16_lo(w_);
        };
        // block maxima of columns (2p, 2p + 1) travel together as one packed pair
        uint32_t cam[4];
#pragma unroll
        for (int p2 = 0; p2 < 4; ++p2) {
            uint32_t pk = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) pk = max_u16x2(pk, word(i, p2) & 0x7fff7fffu);
            pk = max_u16x2(pk, (uint32_t)__shfl_xor((int)pk, 16, 64));
            pk = max_u16x2(pk, (uint32_t)__shfl_xor((int)pk, 32, 64));
            cam[p2] = pk;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t amax = (j & 1) ? cam[j >> 1] >> 16 : cam[j >> 1] & 0xffffu;
            const int e = mx_block_exp(amax);
            const float inv = mx_inv_scale(e);
            uint2 q;
            q.x = e4m3x4(elt(0, j) * inv, elt(1, j) * inv, elt(2, j) * inv, elt(3, j) * inv);
            q.y = e4m3x4(elt(4, j) * inv, elt(5, j) * inv, elt(6, j) * inv, elt(7, j) * inv);
            *(uint2*)(tq + (8 * cc + j) * QT + ((rg ^ (2 * (cc & 7))) * 8)) = q;
            if ((l >> 4) == 0) {
                if (cs_words)
                    s_cs[(8 * cc + j) * 4 + w] = (uint8_t)(e + 127);
                else if (cok && r < R)
                    sc[(int64_t)(c + j) * RB + r / 32] = (uint8_t)(e + 127);
            }
        }
        __syncthreads();
        const int64_t r0 = (int64_t)blockIdx.y * QT;
        const int c0 = blockIdx.x * QT;
        if (rs_words && threadIdx.x < QT && r0 + threadIdx.x < R)
            *(uint32_t*)(s_row + b * R * (C / 32) + (r0 + threadIdx.x) * (C / 32) + c0 / 32) =
                *(const uint32_t*)(s_rs + 4 * threadIdx.x);
        if (cs_words && threadIdx.x >= QT && c0 + (int)threadIdx.x - QT < C)
            *(uint32_t*)(sc + (int64_t)(c0 + threadIdx.x - QT) * RB + r0 / 32) =
                *(const uint32_t*)(s_cs + 4 * (threadIdx.x - QT));
#pragma unroll
        for (int it = 0; it < QT * QT / (16 * 256); ++it) {
            const int idx = it * 256 + threadIdx.x;
            const int col = idx >> 3, pq = idx & 7;  // rows 16 pq .. 16 pq + 15 of the column
            const uint4 val = *(const uint4*)(tq + col * QT + (((2 * pq) ^ (2 * ((col >> 3) & 7))) * 8));
            if (c0 + col < C && r0 + 16 * pq < R) {
                uint4* dst = (uint4*)(qc + (int64_t)(c0 + col) * R + r0 + 16 * pq);
                if constexpr (NT)
                    __builtin_nontemporal_store(__builtin_bit_cast(nt_u32x4_t, val), (nt_u32x4_t*)dst);
                else
                    *dst = val;
            }
        }
    }
}

template <bool GATHER>
static void quant_dispatch(const uint16_t* src, int batch, int64_t R, int C, int mode, uint8_t* q_row,
                           uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, const int32_t* src_of, int k,
                           hipStream_t s) {
    const dim3 grid((C + QT - 1) / QT, (unsigned)((R + QT - 1) / QT), batch);
    // streaming code stores when the rows are gathered (each source row is read k
    // times) or the bf16 source fits the 256 MB last-level cache; a larger source
    // measured faster with normal stores
    const bool nt = GATHER || (int64_t)batch * R * C * 2 <= (256ll << 20);
    auto go = [&](auto kern) {
        kern<<<grid, 256, 0, s>>>(src, R, C, q_row, s_row, q_col, s_col, src_of, k);
    };
    if ((mode & 3) == 3)
        nt ? go(quant_mxfp8_kernel<true, true, GATHER, true>) : go(quant_mxfp8_kernel<true, true, GATHER, false>);
    else if (mode & 1)
        nt ? go(quant_mxfp8_kernel<true, false, GATHER, true>) : go(quant_mxfp8_kernel<true, false, GATHER, false>);
    else
        nt ? go(quant_mxfp8_kernel<false, true, GATHER, true>) : go(quant_mxfp8_kernel<false, true, GATHER, false>);
}

int launch_quant_mxfp8(const uint16_t* src, int batch, int64_t R, int C, int mode, uint8_t* q_row,
                       uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, hipStream_t s) {
    quant_dispatch<false>(src, batch, R, C, mode, q_row, s_row, q_col, s_col, nullptr, 1, s);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_permute_quant_mxfp8(const uint16_t* x, const int32_t* src_of, int k, int64_t M_cap, int d,
                               int mode, uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                               hipStream_t s) {
    quant_dispatch<true>(x, 1, M_cap, d, mode, q_row, s_row, q_col, s_col, src_of, k, s);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

// ------------------------------------------------------------------ MX GEMM
// Grouped GEMMs on v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, one E8M0
// scale per lane and 32-element K block), with the workgroup tile, wavefront
// grid and persistent XCD-aware schedule of the bf16 grouped GEMM. Both
// operands are K-major fp8 ([rows][K] bytes), streamed global -> LDS in
// 128-byte K slabs (two MFMA K steps of 64).
//  * ragged M (FC2 forward, FC1 dgrad): out[R_e] = A[R_e] x B_e^T, bf16,
//    A [M_cap, K], B [E, N, K];
//  * ragged K (both wgrads): out_e = A[:, R_e] x B[:, R_e]^T, fp32 [E, M, N],
//    A [M, ld] and B [N, ld] the column-wise (transposed) copies, whose K
//    runs over the expert's row region R_e (a 128-row multiple, so slabs
//    never straddle two experts); an empty expert's output is written as 0.
struct MxArgs {
    const uint8_t* A;    // codes: [M_cap, K] (ragged M) or [M, ld] (ragged K)
    const uint8_t* As;   // scales, one byte per 32 codes of a row
    const uint8_t* B;    // codes: [E, N, K] (ragged M) or [N, ld] (ragged K)
    const uint8_t* Bs;
    const int32_t* offsets;
    int E, M, N, K;      // ragged K: M unused by ragged M; K unused by ragged K
    int64_t ld;          // ragged K: bytes per code row (M_cap)
    uint16_t* out;       // ragged M: [M_cap, N] bf16 (nullable when q_row is given)
    float* outf;         // ragged K: [E, M, N] fp32
    uint8_t* q_row;      // ragged M, nullable: row-wise MXFP8 copy of out, codes [M_cap, N]
    uint8_t* s_row;      //   and scales [M_cap, N/32]
    uint8_t* q_col;      // ragged M, nullable (only beside q_row): column-wise copy, transposed,
    uint8_t* s_col;      //   codes [N, M_cap] and scales [N, M_cap/32]
    int64_t M_cap;
};

constexpr int MBK = 128;  // K bytes per LDS slab
constexpr int kMxLoads = BM * MBK / (kThreads * 16);

// Persistent: one workgroup per compute unit walks the tile order and fetches
// the next tile's first slab (codes and scales) during the current tile's
// last one. Ragged K takes the experts by descending row count, so the long
// tiles start first.
template <bool RAGGED_K>
__global__ void __launch_bounds__(kThreads, 1) mx_gemm_kernel(MxArgs p) {
    __shared__ __attribute__((aligned(1024))) uint8_t s_ab[2][(BM + BN) * MBK];
    // block scales of 4 consecutive slabs (a group): 16 bytes for each of the
    // BM A rows then the BN B rows, double-buffered by group
    __shared__ __attribute__((aligned(1024))) uint8_t s_sc[2][(BM + BN) * 16];
    __shared__ int s_tiles[MOE_MAX_E + 1];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / (kWaves / 2), wn = wave % (kWaves / 2);  // 2 x (kWaves / 2) wavefront grid
    const int h = lane >> 5;
    const int ntn = (p.N + BN - 1) / BN;
    const int ntm = RAGGED_K ? (p.M + BM - 1) / BM : 0;
    const int64_t rowb = RAGGED_K ? p.ld : (int64_t)p.K;  // bytes per code row
    const int KB = (int)(rowb / 32);                         // scale bytes per row
    int total;
    if constexpr (!RAGGED_K) {
        total = ragged_m_prefix(p.offsets, p.E, s_tiles) * ntn;
    } else {
        // sort keys in the operand stage, which no copy has touched yet
        experts_by_rows<kThreads>(p.offsets, p.E, (uint64_t*)&s_ab[0][0], s_tiles);
        total = p.E * ntm * ntn;
    }
    const int nb = gridDim.x;  // a multiple of 8
    auto logical = [&](int round) -> int {
        const int b = blockIdx.x;
        return round * nb + (b & 7) * (nb >> 3) + (b >> 3);
    };
    struct Tile {
        int e, row0, row_end, m0, n0, k_begin, nk;
    };
    auto get_tile = [&](int t) -> Tile {
        Tile tl;
        if constexpr (!RAGGED_K) {
            const RaggedTile r = ragged_m_decode(p.offsets, p.E, ntn, total / ntn, s_tiles, t);
            tl.e = __builtin_amdgcn_readfirstlane(r.e);
            tl.row0 = __builtin_amdgcn_readfirstlane(r.row0);
            tl.row_end = __builtin_amdgcn_readfirstlane(r.row_end);
            tl.n0 = __builtin_amdgcn_readfirstlane(r.n0);
            tl.m0 = 0;
            tl.k_begin = 0;
            tl.nk = p.K / MBK;
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
            tl.nk = (__builtin_amdgcn_readfirstlane(p.offsets[tl.e + 1]) - tl.k_begin) / MBK;
        }
        return tl;
    };
    // operand regions of a tile: codes and scales; rows past the region (ragged
    // M) or past M and N read as 0
    // (a tile reads at most BM rows of A and BN rows of B; byte counts are
    // formed in 64 bits and clamped to what a buffer resource holds)
    struct MxSrc {
        const uint8_t *a, *b, *as, *bs;
        uint32_t a_bytes, b_bytes, as_bytes, bs_bytes;
    };
    auto make_src = [&](const Tile& t) -> MxSrc {
        MxSrc s;
        if constexpr (!RAGGED_K) {
            s.a = p.A + (int64_t)t.row0 * p.K;
            s.a_bytes = clamp_records((int64_t)min(t.row_end - t.row0, BM) * p.K);
            s.b = p.B + ((int64_t)t.e * p.N + t.n0) * p.K;
            s.b_bytes = clamp_records((int64_t)min(p.N - t.n0, BN) * p.K);
            s.as = p.As + (int64_t)t.row0 * KB;
            s.as_bytes = clamp_records((int64_t)min(t.row_end - t.row0, BM) * KB);
            s.bs = p.Bs + ((int64_t)t.e * p.N + t.n0) * KB;
            s.bs_bytes = clamp_records((int64_t)min(p.N - t.n0, BN) * KB);
        } else {
            const int kb = t.k_begin / 32;
            s.a = p.A + (int64_t)t.m0 * rowb + t.k_begin;
            s.a_bytes = clamp_records((int64_t)min(p.M - t.m0, BM) * rowb - t.k_begin);
            s.b = p.B + (int64_t)t.n0 * rowb + t.k_begin;
            s.b_bytes = clamp_records((int64_t)min(p.N - t.n0, BN) * rowb - t.k_begin);
            s.as = p.As + (int64_t)t.m0 * KB + kb;
            s.as_bytes = clamp_records((int64_t)min(p.M - t.m0, BM) * KB - kb);
            s.bs = p.Bs + (int64_t)t.n0 * KB + kb;
            s.bs_bytes = clamp_records((int64_t)min(p.N - t.n0, BN) * KB - kb);
        }
        return s;
    };
    // this lane's source offset for copy 0 of a slab; copy i adds 64 rows
    const int q0 = wave * 64 + lane;
    const uint32_t off0 = (uint32_t)((q0 >> 3) * rowb + (((q0 & 7) ^ kmaj_swz(q0 >> 3)) * 16));
    const uint32_t istep = (uint32_t)(kThreads / 8 * rowb);
    auto issue = [&](const MxSrc& s, int kt, int buf) {
        const uint32_t l0 = (uint32_t)(uintptr_t)(LDS_AS char*)(&s_ab[buf][0]) + wave * 1024;
        const uint32_t o = off0 + (uint32_t)kt * MBK;
        const i32x4_t ra = rsrc_words(s.a, s.a_bytes), rb = rsrc_words(s.b, s.b_bytes);
#pragma unroll
        for (int i = 0; i < kMxLoads; ++i) lds_copy16(ra, l0 + i * kWaves * 1024, o + i * istep);
#pragma unroll
        for (int i = 0; i < kMxLoads; ++i) lds_copy16(rb, l0 + BM * MBK + i * kWaves * 1024, o + i * istep);
    };
    // Block scales travel by group of 4 slabs: one 16-byte copy per A row and
    // per B row (wavefronts 0-3 the A rows, 4-7 the B rows) straight into LDS.
    // Loading each lane's slab word from global memory instead touched one
    // cache line per row, per slab and per wavefront, and cost a third of the
    // kernel's time. Bytes past a row's valid K read whatever follows (or 0
    // past the region) and are never used.
    auto issue_scales = [&](const MxSrc& s, int g, int sbuf) {
        const bool a_side = wave < kWaves / 2;
        const int row = (wave % (kWaves / 2)) * 64 + lane;
        const i32x4_t r = a_side ? rsrc_words(s.as, s.as_bytes) : rsrc_words(s.bs, s.bs_bytes);
        const uint32_t l = (uint32_t)(uintptr_t)(LDS_AS char*)(&s_sc[sbuf][0]) + wave * 1024;
        lds_copy16(r, l, (uint32_t)(row * KB + g * 16));
    };
    // this lane's scale words of slab kt4 (0..3) of the group in buffer sbuf:
    // the 4 K blocks of the slab for its rows (A) and columns (B)
    auto read_scales = [&](int sbuf, int kt4, uint32_t* sa, uint32_t* sb) {
        const uint8_t* base = s_sc[sbuf] + kt4 * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) sa[i] = *(const uint32_t*)(base + (wm * 128 + 32 * i + (lane & 31)) * 16);
#pragma unroll
        for (int j = 0; j < TNW; ++j)
            sb[j] = *(const uint32_t*)(base + (BM + wn * WN + 32 * j + (lane & 31)) * 16);
    };
    // Operand fragment of row `base + (lane & 31)` for K step ks (64 bytes = K
    // blocks 2ks and 2ks+1): the instruction reads a lane's first 16 bytes as
    // part of the step's first 32-element block and its last 16 bytes as part
    // of the second, lane halves h = 0, 1 supplying 16-byte chunks h and 2 + h
    // (measured); the scale of block b comes from lane half b.
    auto frag = [&](const uint8_t* s, int base, int ks) -> i32x8_t {
        const int r = base + (lane & 31);
        const i32x4_t lo = *(const i32x4_t*)(s + kmaj_byte(r, 4 * ks + h));
        const i32x4_t hi = *(const i32x4_t*)(s + kmaj_byte(r, 4 * ks + 2 + h));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };

    int round = 0;
    int t = logical(0);
    if (t >= total) return;
    Tile tl = get_tile(t);
    MxSrc src = make_src(tl);
    uint32_t sa[4], sb[TNW], na[4], nb_[TNW];
    if (tl.nk > 0) {
        issue(src, 0, 0);
        issue_scales(src, 0, 0);
    }
    int buf0 = 0;  // LDS buffer holding slab 0 of the current tile
    int sg0 = 0;   // scale buffer holding group 0 of the current tile
    f32x16_t acc[4][TNW];
    for (;;) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < TNW; ++j) acc[i][j] = (f32x16_t){};
        const int tn = logical(round + 1);
        const bool have_next = tn < total;
        Tile tl_next = tl;
        MxSrc src_next = src;
        int nk_next = 0;
        if (have_next) {
            tl_next = get_tile(tn);
            src_next = make_src(tl_next);
            nk_next = tl_next.nk;
        }
        const int nk = tl.nk;
        const int ng = (nk + 3) / 4;  // scale groups of this tile
        int next_buf0 = buf0;
        if (nk > 0) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            read_scales(sg0, 0, na, nb_);
            // shifted by this half-wave's block: K step ks then finds its scale
            // in byte 0 after a further shift by 16 ks
#pragma unroll
            for (int i = 0; i < 4; ++i) sa[i] = na[i] >> (8 * h);
#pragma unroll
            for (int j = 0; j < TNW; ++j) sb[j] = nb_[j] >> (8 * h);
            for (int kt = 0; kt < nk; ++kt) {
                // No vector-memory load is in flight here in the steady state (the
                // previous slab ended with a full wait), so this wait is free; it
                // makes registers reloaded from scratch before the loop ready on
                // entry, instead of the compiler waiting for them inside the loop,
                // where the same counter also tracks the slab copies.
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
                const int cur = (buf0 + kt) & 1;
                if (kt + 1 < nk) {
                    issue(src, kt + 1, cur ^ 1);
                } else if (nk_next > 0) {
                    issue(src_next, 0, cur ^ 1);
                    issue_scales(src_next, 0, (sg0 + ng) & 1);
                }
                // the next group's scales, into the buffer the previous group
                // left (its last reads ended before the previous slab barrier)
                if ((kt & 3) == 0 && kt + 4 < nk) issue_scales(src, kt / 4 + 1, (sg0 + kt / 4 + 1) & 1);
                // the next slab's scale words: its group landed at least one
                // slab barrier ago
                if (kt + 1 < nk) read_scales((sg0 + (kt + 1) / 4) & 1, (kt + 1) & 3, na, nb_);
                const uint8_t* sA = s_ab[cur];
                const uint8_t* sB = s_ab[cur] + BM * MBK;
                // Fragments: the first MFMA's operands (B, then A row 0) are requested
                // first, so it starts while the other A rows still load. The MFMAs go
                // column by column (all A rows with B fragment 0, then with B fragment
                // 1), and each fragment of the next K step is requested as soon as
                // the last MFMA reading this step's is issued, so the loads of step 1
                // run under the MFMAs of step 0, at least three MFMAs ahead of their
                // use. The MFMA sequence of every accumulator is unchanged.
                i32x8_t fa[4], fb[TNW];
#pragma unroll
                for (int j = 0; j < TNW; ++j) fb[j] = frag(sB, wn * WN + 32 * j, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) fa[i] = frag(sA, wm * 128 + 32 * i, 0);
                static_for<MBK / 64>([&](auto KS) {
                    constexpr int ks = KS;
                    constexpr bool more = ks + 1 < MBK / 64;
                    __builtin_amdgcn_s_setprio(1);
                    static_for<TNW>([&](auto J) {
                        static_for<4>([&](auto I) {
                            // the instruction reads byte 0 of each scale register, so the
                            // block of this K step is shifted there (OPSEL stays 0)
                            acc[I][J] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                fb[J], fa[I], acc[I][J], 0, 0, 0, (int)(sb[J] >> (16 * ks)), 0,
                                (int)(sa[I] >> (16 * ks)));
                            if constexpr (more && J + 1 == TNW) fa[I] = frag(sA, wm * 128 + 32 * I, ks + 1);
                        });
                        if constexpr (more) fb[J] = frag(sB, wn * WN + 32 * J, ks + 1);
                    });
                    __builtin_amdgcn_s_setprio(0);
                });
                // Pin the MFMAs here: left alone, the compiler sinks them below the
                // barrier that waits for the next slab's copies (they touch no
                // memory), which serialises that wait with the multiply.
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < TNW; ++j) asm volatile("" : "+v"(acc[i][j]));
                if (kt + 1 < nk) {
                    __builtin_amdgcn_s_waitcnt(0);
                    __syncthreads();
#pragma unroll
                    for (int i = 0; i < 4; ++i) sa[i] = na[i] >> (8 * h);
#pragma unroll
                    for (int j = 0; j < TNW; ++j) sb[j] = nb_[j] >> (8 * h);
                } else {
                    next_buf0 = cur ^ 1;
                }
            }
        } else if (nk_next > 0) {
            // nothing to multiply (an empty expert): the buffers this tile would
            // have used take the next tile's first slab and scale group
            issue(src_next, 0, buf0);
            issue_scales(src_next, 0, sg0);
        }
        // Epilogue: lane = row (l & 31), columns 8q + 4h + s of each 32-wide
        // tile. Staged through this wavefront's 8 KiB of the LDS stage the tile
        // no longer reads, 32 rows at a time, so each store covers whole rows
        // (8 rows x 128 B of bf16, 4 rows x 256 B of fp32) instead of 32 rows
        // x 16 or 32 B; 16-byte chunks XOR-swizzled by row against bank
        // conflicts.
        __syncthreads();  // the last slab and the previous tile's staging are read out
        uint8_t* stg = &s_ab[next_buf0 ^ 1][0] + wave * 8192;
        const int r = lane & 31;
        const int col0 = tl.n0 + wn * WN;
        static_for<4>([&](auto I) {
            if constexpr (!RAGGED_K) {
                uint32_t pk[TNW][8];  // the lane's bf16 pairs of each 32-column block
                static_for<TNW>([&](auto J) {
                    static_for<4>([&](auto Q) {
                        uint2 v;
                        v.x = pack_bf16x2(acc[I][J][4 * Q], acc[I][J][4 * Q + 1]);
                        v.y = pack_bf16x2(acc[I][J][4 * Q + 2], acc[I][J][4 * Q + 3]);
                        pk[J][2 * Q] = v.x;
                        pk[J][2 * Q + 1] = v.y;
                        *(uint2*)(stg + r * 128 + (((4 * J + Q) ^ ((r >> 1) & 7)) << 4) + 8 * h) = v;
                    });
                });
                // GroupGemm + Quantize: the row-wise MXFP8 copy of the bf16 output
                // (lanes l and l ^ 32 share a row, so both take the branch) and,
                // when asked, its column-wise copy stored transposed (a 32-row block
                // lies wholly inside or past a 128-row region: the whole wavefront
                // takes the branch)
                const int mq = tl.row0 + wm * 128 + 32 * I + r;
                const int mb = tl.row0 + wm * 128 + 32 * I;
                if (p.q_row && mq < tl.row_end) {
                    static_for<TNW>([&](auto J) {
                        const int cb = col0 + 32 * J;
                        if (cb < p.N) {
                            mx_rowq32(pk[J], lane, p.q_row + (int64_t)mq * p.N + cb,
                                      p.s_row + (int64_t)mq * (p.N / 32) + cb / 32);
                            if (p.q_col) {
                                const int64_t ls = p.M_cap / 32;
                                mx_colq32(pk[J], lane, p.q_col + (int64_t)cb * p.M_cap + mb, p.M_cap,
                                          p.s_col + (int64_t)cb * ls + mb / 32, ls);
                            }
                        }
                    });
                }
                wave_lds_sync();
                if (p.out) {
                    static_for<4>([&](auto It) {
                        const int R = 8 * It + (lane >> 3), c = lane & 7;
                        const uint4 v = *(const uint4*)(stg + R * 128 + ((c ^ ((R >> 1) & 7)) << 4));
                        const int m = tl.row0 + wm * 128 + 32 * I + R, col = col0 + 8 * c;
                        if (m < tl.row_end && col < p.N) st_nt16(p.out + (int64_t)m * p.N + col, v);
                    });
                }
            } else {
                static_for<TNW>([&](auto J) {
                    static_for<4>([&](auto Q) {
                        const int ch = 8 * J + 2 * Q + h;
                        *(float4*)(stg + r * 256 + ((ch ^ (r & 15)) << 4)) =
                            make_float4(acc[I][J][4 * Q], acc[I][J][4 * Q + 1], acc[I][J][4 * Q + 2],
                                        acc[I][J][4 * Q + 3]);
                    });
                });
                wave_lds_sync();
                float* o = p.outf + (int64_t)tl.e * p.M * p.N;
                static_for<8>([&](auto It) {
                    const int R = 4 * It + (lane >> 4), c = lane & 15;
                    const float4 v = *(const float4*)(stg + R * 256 + ((c ^ (R & 15)) << 4));
                    const int m = tl.m0 + wm * 128 + 32 * I + R, col = col0 + 4 * c;
                    if (m < p.M && col < p.N) st_nt16(o + (int64_t)m * p.N + col, v);
                });
            }
            wave_lds_sync();  // read out before the next 32 rows overwrite it
        });
        if (!have_next) break;
        ++round;
        buf0 = next_buf0;
        sg0 = (sg0 + ng) & 1;
        tl = tl_next;
        src = src_next;
    }
}

int launch_mx_fc2(const uint8_t* a_q, const uint8_t* a_s, const uint8_t* w2t_q, const uint8_t* w2t_s,
                  const int32_t* offsets, int E, int d, int n, int64_t M_cap, uint16_t* y,
                  uint8_t* y_q, uint8_t* y_s, uint8_t* yt_q, uint8_t* yt_s, hipStream_t s) {
    return launch_mx_ragged_m(a_q, a_s, w2t_q, w2t_s, offsets, E, d, n, M_cap, y, y_q, y_s, yt_q, yt_s, s);
}

int launch_mx_ragged_m(const uint8_t* a_q, const uint8_t* a_s, const uint8_t* b_q, const uint8_t* b_s,
                       const int32_t* offsets, int E, int N, int K, int64_t M_cap, uint16_t* out,
                       uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, hipStream_t s) {
    MxArgs a;
    __builtin_memset(&a, 0, sizeof(a));
    a.A = a_q; a.As = a_s; a.B = b_q; a.Bs = b_s;
    a.offsets = offsets; a.E = E; a.N = N; a.K = K; a.ld = K;
    a.out = out;
    a.q_row = q_row; a.s_row = s_row;
    a.q_col = q_row ? q_col : nullptr; a.s_col = s_col; a.M_cap = M_cap;
    const int64_t tb = ragged_m_grid(M_cap, E, N);
    if (tb <= 0) return 0;
    mx_gemm_kernel<false><<<persistent_grid(tb), kThreads, 0, s>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_mx_wgrad(const uint8_t* at_q, const uint8_t* at_s, int M, const uint8_t* bt_q,
                    const uint8_t* bt_s, int N, const int32_t* offsets, int E, int64_t M_cap,
                    float* out, hipStream_t s) {
    MxArgs a;
    __builtin_memset(&a, 0, sizeof(a));
    a.A = at_q; a.As = at_s; a.B = bt_q; a.Bs = bt_s;
    a.offsets = offsets; a.E = E; a.M = M; a.N = N; a.ld = M_cap;
    a.outf = out;
    const int64_t tb = (int64_t)E * ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    if (tb <= 0) return 0;
    mx_gemm_kernel<true><<<persistent_grid(tb), kThreads, 0, s>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace moe
