// Pieces shared by the grouped-GEMM kernels (bf16 and MXFP8): the LDS slab
// layouts, the XCD-aware tile order, buffer resources and the ragged-M tile
// scheduler that turns device-side expert offsets into a tile.
#pragma once

#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int BM = 256, BN = 256;  // workgroup tile (rows x columns)
constexpr int kWaves = 8;          // 2 x 4 wavefronts, two per SIMD
constexpr int kThreads = kWaves * 64;
constexpr int WN = 64;             // columns per wavefront (two 32-column MFMA tiles)
constexpr int TNW = WN / 32;

// A K-major slab row holds 128 bytes (8 chunks of 16 B). Chunks are XOR-
// swizzled with row bits 1..3: a 256-byte LDS bank window holds two rows, so
// rows r and r + 2 must differ in chunk for conflict-free ds_read_b128.
__device__ __forceinline__ int kmaj_swz(int r) { return (r >> 1) & 7; }
// byte offset of 16-byte chunk `chunk` of row r in a [rows][128 B] slab
__device__ __forceinline__ int kmaj_byte(int r, int chunk) { return r * 128 + ((chunk ^ kmaj_swz(r)) << 4); }
// byte offset of chunk `chunk` of k-row k in an MN-major [64][512 B] slab
__device__ __forceinline__ int mnmaj_byte(int k, int chunk) { return k * 512 + ((chunk ^ ((k & 7) << 2)) << 4); }

// Workgroup order -> tile order: consecutive workgroups land on different
// XCDs (round robin over 8); give each XCD a contiguous range of tiles so
// tiles that share operands share an L2.
__device__ __forceinline__ int xcd_remap(int b, int total) {
    const int x = b & 7, i = b >> 3;
    const int q = total >> 3, r = total & 7;
    return x * q + min(x, r) + i;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// One 16-byte-per-lane direct global -> LDS copy: lane l's 16 bytes land at
// LDS byte address lds + 16 l. Written as inline assembly on purpose: the
// compiler cannot tell which LDS bytes the builtin form writes, so it waits
// for every outstanding copy before the next LDS read, which would serialise
// the prefetch of slab k + 1 with the multiply of slab k. Here the kernel
// owns the ordering: it waits on the vector-memory counter and a barrier
// before any wave reads a slab.
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4_t rsrc_words(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    i32x4_t r;
    r.x = (int32_t)(uint32_t)a;
    r.y = (int32_t)((uint32_t)(a >> 32) & 0xffffu);  // stride 0
    r.z = (int32_t)bytes;                            // reads at or past this offset return 0
    r.w = 0x00020000;
    return r;
}

// Readable bytes of a buffer resource from a 64-bit extent: at most 2^31 - 1
// (every lane offset the kernels form stays below 2^31), none if empty.
__device__ __forceinline__ uint32_t clamp_records(int64_t bytes) {
    return bytes <= 0 ? 0u : (bytes >= 0x7FFFFFFF ? 0x7FFFFFFFu : (uint32_t)bytes);
}

// Resource over bytes [skip, total) of an operand that starts at base: every
// K slab gets its own 64-bit base, so the 32-bit lane offsets only span one
// slab (or one tile's rows) and no operand size limits the GEMMs.
__device__ __forceinline__ i32x4_t rsrc_from(const void* base, int64_t total, int64_t skip) {
    return rsrc_words((const char*)base + skip, clamp_records(total - skip));
}

__device__ __forceinline__ void lds_copy16(i32x4_t rsrc, uint32_t lds, uint32_t voff) {
    // resource and LDS address are wave-uniform; readfirstlane pins them to
    // scalar registers when the compiler cannot prove it (free otherwise)
    i32x4_t r;
    r.x = __builtin_amdgcn_readfirstlane(rsrc.x);
    r.y = __builtin_amdgcn_readfirstlane(rsrc.y);
    r.z = __builtin_amdgcn_readfirstlane(rsrc.z);
    r.w = __builtin_amdgcn_readfirstlane(rsrc.w);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(r)
                 : "memory");
    // M0 is a reserved register the compiler would not preserve for us; these
    // kernels give it no other use (no compiler-issued LDS DMA, GWS or
    // message instructions), so the value written here is simply dead after.
}

// s_waitcnt vmcnt(0) alone (expcnt and lgkmcnt fields left at their maxima)
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr uint32_t kMasked = 0x80000000u;  // byte offset past every buffer: the load returns 0

struct RaggedTile {
    int e, row0, row_end, n0;
};

// Ragged-M scheduling: expert e owns rows [offsets[e], offsets[e+1]) split
// into ceil(rows / BM) M tiles. Every workgroup derives the prefix of M tiles
// from the device offsets (no host copy): s_tiles[e] = first M tile of expert
// e, s_tiles[E] = total. s_tiles: LDS scratch of E + 1 ints. Must be called by
// the whole workgroup; returns the total number of M tiles.
__device__ __forceinline__ int ragged_m_prefix(const int32_t* offsets, int E, int* s_tiles) {
    const int tid = threadIdx.x, lane = tid & 63;
    for (int i = tid; i < E; i += blockDim.x) {
        const int rows = offsets[i + 1] - offsets[i];
        s_tiles[i + 1] = (rows + BM - 1) / BM;
    }
    if (tid == 0) s_tiles[0] = 0;
    __syncthreads();
    if (tid < 64) {
        int carry = 0;
        for (int base = 0; base < E; base += 64) {
            const int i = base + lane;
            int v = (i < E) ? s_tiles[i + 1] : 0;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int u = __shfl_up(v, o, 64);
                if (lane >= o) v += u;
            }
            if (i < E) s_tiles[i + 1] = v + carry;
            carry += __shfl(v, 63, 64);
        }
    }
    __syncthreads();
    return s_tiles[E];
}

// Tile number tt (of mtiles * ntn) -> tile: bands of G M tiles with the M
// tiles inner, so that the 32 tiles one XCD runs at a time (a contiguous run)
// form a G x (32 / G) window whose operand panels its L2 shares; the expert is
// the last one whose first M tile is <= the tile's M index. The bf16 GEMMs
// use G = 4 (measured 1% faster on FC1 than 8, whose 8 x 4 window has the
// same panel count; 16 was 2% slower); the MXFP8 GEMMs keep G = 8 (1.5-3.5%
// slower with 4).
template <int G = 8>
__device__ __forceinline__ RaggedTile ragged_m_decode(const int32_t* offsets, int E, int ntn, int mtiles,
                                                      const int* s_tiles, int tt) {
    const int band = tt / (G * ntn);
    const int within = tt - band * G * ntn;
    const int bm = min(G, mtiles - band * G);
    const int mt = band * G + within % bm;
    const int nt = within / bm;
    int lo = 0, hi = E;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_tiles[mid] <= mt) lo = mid; else hi = mid;
    }
    RaggedTile t;
    t.e = lo;
    t.row0 = offsets[lo] + (mt - s_tiles[lo]) * BM;
    t.row_end = offsets[lo + 1];
    t.n0 = nt * BN;
    return t;
}

// One tile per workgroup: workgroups past the real tile count return false.
__device__ __forceinline__ bool ragged_m_tile(const int32_t* offsets, int E, int ntn, int* s_tiles,
                                              RaggedTile& t) {
    const int mtiles = ragged_m_prefix(offsets, E, s_tiles);
    const int total = mtiles * ntn;
    if ((int)blockIdx.x >= total) return false;
    t = ragged_m_decode(offsets, E, ntn, mtiles, s_tiles, xcd_remap(blockIdx.x, total));
    return true;
}

// Ragged-K scheduling: the experts ordered by descending row count (ties to
// the lower index), so the longest wgrad tiles start first and the short ones
// fill the tail. A bitonic sort of 64-bit keys (rows << 11 | 1024 | 1023 - e:
// the 1024 bit keeps every real key above the zero padding of the power-of-
// two array) in LDS scratch `key` of at least 1024 entries; order[0, E) gets
// the expert indices. log2(P) (log2(P) + 1) / 2 barrier steps for P >= E, one
// compare-exchange per thread and step at P = 1024. Must be called by the
// whole workgroup of NT threads.
template <int NT>
__device__ __forceinline__ void experts_by_rows(const int32_t* offsets, int E, uint64_t* key, int* order) {
    const int tid = threadIdx.x;
    int P = 1;
    while (P < E) P <<= 1;
    for (int i = tid; i < P; i += NT)
        key[i] = i < E ? ((uint64_t)(uint32_t)(offsets[i + 1] - offsets[i]) << 11) | 1024u | (uint32_t)(1023 - i)
                       : 0ull;
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < P; i += NT) {
                const int l = i ^ j;
                if (l > i) {
                    const uint64_t a = key[i], b = key[l];
                    const bool desc = (i & k) == 0;  // the last merge (k = P) is descending throughout
                    if (desc ? a < b : a > b) {
                        key[i] = b;
                        key[l] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    for (int i = tid; i < E; i += NT) order[i] = 1023 - (int)(key[i] & 1023u);
    __syncthreads();
}

// Compute units of the current device, cached per device on first use (the
// only state the library keeps; concurrent first calls store the same value).
inline int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// Persistent grid: one workgroup per compute unit (the LDS footprint allows
// one), never more than the upper bound on tiles, always a multiple of 8.
inline int persistent_grid(int64_t tile_bound) {
    const int64_t cus = (device_cus() + 7) & ~7;
    const int64_t bound = (tile_bound + 7) & ~(int64_t)7;
    return (int)std::max<int64_t>(8, std::min(cus, bound));
}

// Upper bound on ragged-M workgroups: every expert region is 128-row aligned,
// so sum_e ceil(rows_e / BM) <= M_cap / BM + E.
inline int ragged_m_grid(int64_t M_cap, int E, int N) {
    return (int)((M_cap / BM + E + 1) * ((N + BN - 1) / BN));
}

}  // namespace moe
