/*
 * moe.h -- C ABI of libmoe.so: the dropless MoE expert MLP on one MI355X
 * (gfx950), run as a sync-free ragged grouped GEMM with a fused GLU epilogue.
 *
 * Sources (web pages, cited by title and section):
 *   [P1] "NVIDIA CuTe DSL 융합 커널은 MoE 학습의 CPU·메모리 병목을 지운다"
 *   [P2] "SonicMoE로 보는 GPU 커널 최적화"
 *   [P3] "Dropless MoE 학습과 NVIDIA Transformer Engine 소개"
 *
 * Conventions shared by every entry point
 *   - bf16 tensors are passed as uint16_t* raw bit patterns; all sizes are
 *     element counts; every matrix is row-major and densely packed.
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise.
 *     The caller owns every buffer and keeps it alive until the stream work
 *     that uses it has completed. The library allocates nothing and keeps no
 *     pointer after a call returns. Its only mutable global state is two
 *     per-device caches filled on first use (the compute-unit count, and the
 *     device address of the static scratch of moe_route_counts_noalloc), so
 *     calls are reentrant and thread-safe, except that moe_route_counts_noalloc
 *     calls overlapping on one GPU share that scratch.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL = the
 *     legacy default stream). No call synchronises, allocates or copies
 *     device-to-host, so every call may be recorded into a hipGraph. Shapes
 *     that depend on the routing (per-expert counts and offsets) are read by
 *     the kernels from device memory only [P1, core-idea section: per-expert
 *     counts tracked on the GPU so no host shape query is needed].
 *   - Host-checkable errors (NULL pointers, bad sizes, misaligned pointers,
 *     a too-small workspace or capacity) return a negative status before any
 *     launch. A launch failure returns MOE_ERR_LAUNCH. Data-dependent
 *     problems never trap: they set bits in a caller-owned device error word.
 *
 * Layout of the expert-major ragged buffer [P3, sections on ragged tensors,
 * dropless MoE, grouped GEMM (128-token alignment) and the dropless
 * boundary (one slot per (token, expert) pair, expert regions padded)]:
 *   pair p = t*k + j (token t, slot j) goes to expert e = topk_idx[t, j];
 *   expert e owns rows [offsets[e], offsets[e+1]), offsets[0] = 0,
 *   offsets[e+1] - offsets[e] = 128 * ceil(counts[e] / 128) (0 if empty);
 *   its pairs sit in rows offsets[e] + rank in ascending p, the remaining
 *   rows of its region are padding and every permuted tensor the library
 *   writes holds zeros there; rows >= offsets[E] are never read or written.
 *   M_cap = moe_capacity_rows(T, k, E) rows always suffice, so nothing is
 *   ever dropped [P3, dropless-boundary section: a worst-case buffer never
 *   drops].
 *
 * FC1 weight layout [P3, grouped-GEMM section: prefused FC1 weight of shape
 * (experts, embed_dim, 2*mlp_dim); P1, core-idea section: gate and input
 * columns interleaved so one tile holds both halves]: w1 is [E, d, 2n];
 * column block b (32 wide) of each row holds gate columns [2*32b, 2*32b+32)
 * = gate[32b, 32b+32) followed by up columns = up[32b, 32b+32).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ALIGN 128          /* rows per expert-region alignment unit    */
#define MOE_MX_BLOCK 32        /* elements per MXFP8 scale block           */
#define MOE_GLU_INTERLEAVE 32  /* gate/up interleave granularity (columns) */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_WIDTH (1 << 20) /* largest d and FC1 width (2n, or n for sReLU) */

/* status codes */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1)  /* NULL/negative/misaligned argument      */
#define MOE_ERR_UNSUPPORTED (-2)  /* valid but unsupported shape or option  */
#define MOE_ERR_WORKSPACE (-3)    /* workspace or M_cap too small           */
#define MOE_ERR_LAUNCH (-4)       /* a kernel launch reported an error      */

/* activation of the expert MLP */
#define MOE_ACT_SWIGLU 0       /* silu(gate) * up, silu(x) = x / (1 + e^-x) */
#define MOE_ACT_GEGLU 1        /* gelu(gate) * up, gelu(x) = x * Phi(x) (exact, erf form) */
#define MOE_ACT_SRELU 2        /* relu(h)^2, non-gated: FC1 has n columns, w1 [E, d, n],
                                  h and dh [M_cap, n], dw1 [E, d, n] [P1, problem and
                                  published-evidence sections: the sReLU family] */

/* stage bits of moe_grouped_mlp_fwd / moe_grouped_mlp_bwd */
#define MOE_STAGE_FC1 0x01     /* H = X_perm W1_e, A = GLU(H)               */
#define MOE_STAGE_FC2 0x02     /* Y = A W2_e                                */
#define MOE_STAGE_DGRAD2 0x04  /* dA' = dY_u W2_e^T + dGLU epilogue, dS     */
#define MOE_STAGE_WGRAD2 0x08  /* dW2_e = A'^T dY_u                          */
#define MOE_STAGE_DGRAD1 0x10  /* dX_perm = dH W1_e^T                        */
#define MOE_STAGE_WGRAD1 0x20  /* dW1_e = X_perm^T dH                        */
#define MOE_STAGES_FWD (MOE_STAGE_FC1 | MOE_STAGE_FC2)
#define MOE_STAGES_BWD (MOE_STAGE_DGRAD2 | MOE_STAGE_WGRAD2 | MOE_STAGE_DGRAD1 | MOE_STAGE_WGRAD1)
/* mode bit for moe_grouped_mlp_fwd / _bwd: the x_perm argument (and dy_u in
 * the backward) is the un-permuted [T, d] tensor, and the GEMMs read its rows
 * through src_of (row r = token src_of[r] / k; padding rows read zeros), so
 * no expert-major copy is written or read [P2, IO-hiding section: gather
 * fused into the GEMM's loads] */
#define MOE_GATHER_ROWS 0x100

/* bits of the device error word */
#define MOE_ERRBIT_NONFINITE_LOGIT 0x1

/* moe_quant_mxfp8 mode bits */
#define MOE_QUANT_ROWWISE 0x1
#define MOE_QUANT_COLWISE 0x2

typedef void* moe_stream_t; /* hipStream_t */

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_str(int status);

/* Worst-case row count of the expert-major buffer for T tokens, top-k over E
 * experts: 128*ceil(T*k/128) + 128*E. Returns -1 for invalid arguments.
 * Host-only; touches no device. */
int64_t moe_capacity_rows(int T, int k, int E);

/* Device workspace (bytes) that moe_route_counts needs. Host-only. */
size_t moe_route_workspace_bytes(int T, int k, int E);

/* Device workspace (bytes) that moe_grouped_mlp_bwd needs (per-row router
 * gradient partials). Host-only. */
size_t moe_mlp_bwd_workspace_bytes(int n, int64_t M_cap);

/*
 * moe_route_counts -- softmax top-k routing plus the device-resident ragged
 * layout: per-expert counts, 128-aligned prefix offsets and both row maps.
 *   [P3, ragged-tensor section: a learned router sends each token to its
 *   top-K experts and the per-expert counts vary per batch; P1, core-idea
 *   section: counts stay in GPU memory; P3, grouped-GEMM section: 128-token
 *   alignment of expert regions.]
 * Routing: p = softmax over all E logits of a token (fp32); experts ranked by
 * raw logit, descending, ties to the lower expert index; slot j holds the
 * j-th best; topk_w[t, j] = p of that expert, renormalised over the k chosen
 * ones when renorm != 0.
 *   logits   [T, E] fp32 (in)
 *   topk_idx [T, k] int32 (out)    topk_w [T, k] fp32 (out)
 *   counts   [E] int32 (out)       offsets [E+1] int32 (out)
 *   row_of   [T*k] int32 (out): row of pair p in the expert-major buffer
 *   src_of   [M_cap] int32 (out): pair held by each row, -1 for padding and
 *            for rows >= offsets[E]
 *   err_word [1] int32 (in/out, device): MOE_ERRBIT_NONFINITE_LOGIT is OR-ed
 *            in when a logit is NaN or infinite (the routing of such a token
 *            is then unspecified but every output stays in range)
 *   workspace: >= moe_route_workspace_bytes(T, k, E) bytes, 16-byte aligned
 * Requires 1 <= k <= E <= MOE_MAX_EXPERTS, T >= 1, M_cap >= capacity rows.
 */
int moe_route_counts(const float* logits, int T, int E, int k, int renorm,
                     int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                     int32_t* row_of, int32_t* src_of, int64_t M_cap, int32_t* err_word,
                     void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* Bytes of the static device scratch behind moe_route_counts_noalloc (per GPU). */
#define MOE_ROUTE_STATIC_SCRATCH_BYTES (8u << 20)

/*
 * moe_route_counts_noalloc -- moe_route_counts with no workspace argument, for
 *   callers that cannot allocate device memory: code under hipGraph capture
 *   that may not call hipMalloc, tight serving loops, harnesses that forbid
 *   allocation. Same arguments (minus the workspace), the same kernels and
 *   bit-identical outputs. The layout scratch is a device array of
 *   MOE_ROUTE_STATIC_SCRATCH_BYTES that the library reserves statically; each
 *   GPU holds its own copy until the process ends, and its address is looked
 *   up once per device on the first call with that device current. The call
 *   allocates nothing (no hipMalloc/hipFree, no allocating library routine).
 *   Returns MOE_ERR_WORKSPACE, before launching anything, when
 *   moe_route_workspace_bytes(T, k, E) exceeds that size (at most 8 bytes per
 *   expert per 1024 routed pairs: e.g. T*k = 2^20 pairs with E = 1024 experts fit).
 *   Every call on one GPU shares the array and leaves its contents behind
 *   (nothing in it needs clearing between calls), so calls that overlap on a
 *   GPU (concurrent streams or host threads) race: the caller serialises them.
 */
int moe_route_counts_noalloc(const float* logits, int T, int E, int k, int renorm,
                             int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                             int32_t* row_of, int32_t* src_of, int64_t M_cap, int32_t* err_word,
                             moe_stream_t stream);

/*
 * moe_route_bwd -- router backward: gradient of the loss w.r.t. the router
 *   logits, given ds = dL/dtopk_w from moe_grouped_mlp_bwd, for the experts
 *   the forward chose (topk_idx). Without renormalisation
 *     dlogits[t, e] = p_e (g_e - sum_j p_{e_j} ds[t, j]),
 *   p = softmax(logits[t]) over all E, g_e = ds[t, j] if e = e_j else 0;
 *   with renorm != 0 (weights renormalised over the chosen k)
 *     dlogits[t, e_j] = w_j (ds[t, j] - sum_i w_i ds[t, i]), 0 elsewhere.
 *   Non-finite logits have probability 0 and gradient 0.
 *   [P2, backward-rewrite section: dS is the router-score gradient and flows
 *   on through the router.]
 *   logits [T, E] fp32, topk_idx [T, k] int32 (as written by
 *   moe_route_counts), ds [T, k] fp32 (in); dlogits [T, E] fp32 (out).
 * Requires 0 < k <= E <= MOE_MAX_EXPERTS, T > 0; else MOE_ERR_INVALID_ARG.
 */
int moe_route_bwd(const float* logits, const int32_t* topk_idx, const float* ds, int T, int E,
                  int k, int renorm, float* dlogits, moe_stream_t stream);

/*
 * moe_permute -- gather token rows into the expert-major buffer
 *   x_perm[row_of[t*k + j]] = x[t] for every token t and slot j, and
 *   x_perm[r] = 0 for the padding rows of every expert region (the rows
 *   r < offsets[E] with src_of[r] < 0). Each token row is read once and
 *   written to its k rows.
 *   [P2, SonicMoE section: the gather sub-kernel; P3, EP section: dispatch
 *   permutes tokens expert-major.] Used for activations (forward) and for the
 *   upstream gradient dO (backward; no weighting).
 *   x [T, d] bf16 (in); row_of [T*k], src_of [M_cap], offsets [E+1] (in, as
 *   written by moe_route_counts: row_of and src_of are inverse maps);
 *   x_perm [M_cap, d] bf16 (out; rows >= offsets[E] untouched).
 * Requires d % 8 == 0; x and x_perm 16-byte aligned.
 */
int moe_permute(const uint16_t* x, const int32_t* row_of, const int32_t* src_of,
                const int32_t* offsets, int T, int k, int E, int d, int64_t M_cap,
                uint16_t* x_perm, moe_stream_t stream);

/*
 * moe_combine -- weighted un-permute: out[t] = sum over j ascending of
 *   w[t, j] * y[row_of[t*k + j]], accumulated in fp32, rounded once to bf16.
 *   w == NULL means unit weights (the backward's dX = sum_j dX_perm rows).
 *   [P2, SonicMoE section: scatter + expert aggregation sub-kernels; P3, EP
 *   section: combine restores token order and accumulates per token.]
 *   y [M_cap, d] bf16, row_of [T*k], w [T, k] fp32 or NULL (in),
 *   out [T, d] bf16 (out). Requires d % 8 == 0, 16-byte aligned y and out.
 */
int moe_combine(const uint16_t* y, const int32_t* row_of, const float* w,
                int T, int k, int d, uint16_t* out, moe_stream_t stream);

/* MXFP8 side of the forward (all device pointers). E4M3 codes (OCP, bias 7,
 * round to nearest-even), E8M0 block scales (code = exponent + 127) over 32
 * elements: the shared exponent is the smallest e with amax <= 448 * 2^e, so
 * no element saturates; a zero block takes code 0. */
typedef struct moe_mx_fwd {
    uint8_t* a_q;          /* [M_cap, n]    row-wise codes of A (out)            */
    uint8_t* a_s;          /* [M_cap, n/32] row-wise scales of A (out)           */
    uint8_t* at_q;         /* [n, M_cap]    transposed (column-wise) codes, or NULL */
    uint8_t* at_s;         /* [n, M_cap/32] transposed scales, or NULL           */
    const uint8_t* w2t_q;  /* [E, d, n]     W2_e quantized along n, transposed (in) */
    const uint8_t* w2t_s;  /* [E, d, n/32]  its scales (in)                      */
    const uint8_t* x_q;    /* [M_cap, d]    X_perm row-wise codes (in), or NULL: FC1 in bf16 */
    const uint8_t* x_s;    /* [M_cap, d/32] its scales (in)                      */
    const uint8_t* w1t_q;  /* [E, 2n, d]    W1_e quantized along d, transposed (in) */
    const uint8_t* w1t_s;  /* [E, 2n, d/32] its scales (in)                      */
    uint8_t* y_q;          /* [M_cap, d]    row-wise codes of Y (out), or NULL    */
    uint8_t* y_s;          /* [M_cap, d/32] its scales (out)                     */
    uint8_t* yt_q;         /* [d, M_cap]    transposed (column-wise) codes of Y (out), or NULL */
    uint8_t* yt_s;         /* [d, M_cap/32] its scales (out)                     */
} moe_mx_fwd;

/*
 * moe_grouped_mlp_fwd -- grouped FC1 + GLU epilogue, then grouped FC2,
 * one launch each over all experts, tiles scheduled from device offsets;
 * empty experts take no tiles.
 *   [P1, problem and core-idea sections: the GLU activation fused into the
 *   FC1 GEMM epilogue over interleaved weights; P3, grouped-GEMM section: one
 *   call for all experts computing only the real rows.]
 *   FC1: H = X_perm[R_e] W1_e (fp32 accumulate); A = bf16(f(g) * u) from
 *        the fp32 accumulators, f = silu (act = MOE_ACT_SWIGLU) or exact
 *        gelu (act = MOE_ACT_GEGLU) [P1, problem section: SwiGLU and GeGLU
 *        epilogues]; H is stored (bf16) when h != NULL.
 *   FC2: Y = bf16(A[R_e] W2_e). With mx != NULL:
 *        - a_q != NULL: the FC1 epilogue also writes the MXFP8 row-wise (and,
 *          if at_q != NULL, transposed) copy of the bf16 A [P1, core-idea
 *          section: MXFP8 and transposed output fused in the GEMM];
 *        - w2t_q != NULL: FC2 runs on MX-scaled MFMA from a_q/a_s and
 *          w2t_q/w2t_s instead of a and w2 [P3, three-components section:
 *          MXFP8 grouped GEMM]; otherwise FC2 stays bf16 from a and w2;
 *        - y_q != NULL: the FC2 epilogue also writes the row-wise MXFP8 copy
 *          of the bf16 Y (blocks of 32 along d; the "GroupGemm + Quantize"
 *          fused kernel [P3, next-steps section], for an FP8 combine or
 *          all-to-all), and, if yt_q != NULL, its column-wise copy stored
 *          transposed (blocks of 32 rows of an expert region, as at_q); y may
 *          then be NULL;
 *        - x_q != NULL: FC1 also runs on MX-scaled MFMA, from x_q/x_s and
 *          w1t_q/w1t_s instead of x_perm and w1 (then a_q is required,
 *          d % 128 == 0 and no MOE_GATHER_ROWS).
 *   x_perm [M_cap, d], w1 [E, d, 2n], w2 [E, n, d] (bf16, in);
 *   offsets [E+1] (in); h [M_cap, 2n] (out, nullable), a [M_cap, n] (out;
 *   nullable when A's MXFP8 copy is written and FC2 reads only that copy),
 *   y [M_cap, d] (out; needed with MOE_STAGE_FC2 unless y_q is given).
 *   stages: MOE_STAGE_FC1 and/or MOE_STAGE_FC2 (FC2 alone reads a), plus
 *   optionally MOE_GATHER_ROWS: x_perm is then x [T, d] and FC1 reads its
 *   rows through src_of [M_cap] (T, k: the routing shape; both are ignored
 *   without the bit; T * d * 2 < 2^31).
 * With act = MOE_ACT_SRELU the MLP is non-gated: FC1 = X_perm[R_e] W1_e with
 * w1 [E, d, n], A = bf16(relu(H)^2), h [M_cap, n]; no MXFP8 form (mx must be
 * NULL).
 * Requires d % 64 == 0, n % 64 == 0, act MOE_ACT_SWIGLU, MOE_ACT_GEGLU or MOE_ACT_SRELU,
 * M_cap % 128 == 0, M_cap < 2^31, d and the FC1 width (2n; n for sReLU) at
 * most MOE_MAX_WIDTH; no limit on the size of any tensor (every GEMM tile
 * and K slab is addressed from its own 64-bit base). With MOE_GATHER_ROWS
 * the un-permuted x is addressed as a whole with 32-bit byte offsets:
 * T * d * 2 < 2^31. With mx != NULL: n % 128 == 0 (the MX FC2 reads whole
 * 128-byte K slabs of A's codes), and with mx->x_q also d % 128 == 0, so the
 * MXFP8 form needs d, n multiples of 128 (a 2880-wide model is refused).
 * 16-byte aligned pointers. Otherwise MOE_ERR_UNSUPPORTED.
 */
int moe_grouped_mlp_fwd(const uint16_t* x_perm, const uint16_t* w1, const uint16_t* w2,
                        const int32_t* offsets, const int32_t* src_of, int T, int k, int E, int d,
                        int n, int64_t M_cap, int act, unsigned stages, uint16_t* h, uint16_t* a,
                        uint16_t* y, const moe_mx_fwd* mx, moe_stream_t stream);

/* MXFP8 side of the backward (all device pointers; codes and scales as in
 * moe_mx_fwd). DGRAD2 writes the first six, the others are inputs the caller
 * quantizes with moe_quant_mxfp8 (column-wise dY_u and X_perm, row-wise W1). */
typedef struct moe_mx_bwd {
    uint8_t* dh_q;         /* [M_cap, 2n]     row-wise codes of dH (DGRAD2 out, DGRAD1 in) */
    uint8_t* dh_s;         /* [M_cap, 2n/32]  its scales                        */
    uint8_t* dht_q;        /* [2n, M_cap]     column-wise codes of dH, transposed (DGRAD2 out, WGRAD1 in) */
    uint8_t* dht_s;        /* [2n, M_cap/32]  its scales                        */
    uint8_t* awt_q;        /* [n, M_cap]      column-wise codes of A', transposed (DGRAD2 out, WGRAD2 in) */
    uint8_t* awt_s;        /* [n, M_cap/32]   its scales                        */
    const uint8_t* dyt_q;  /* [d, M_cap]      column-wise codes of dY_u, transposed (WGRAD2 in) */
    const uint8_t* dyt_s;  /* [d, M_cap/32]                                     */
    const uint8_t* xt_q;   /* [d, M_cap]      column-wise codes of X_perm, transposed (WGRAD1 in) */
    const uint8_t* xt_s;   /* [d, M_cap/32]                                     */
    const uint8_t* w1_q;   /* [E, d, 2n]      W1_e row-wise along 2n (DGRAD1 in) */
    const uint8_t* w1_s;   /* [E, d, 2n/32]                                     */
    const uint8_t* dy_q;   /* [M_cap, d]      dY_u row-wise codes (DGRAD2 in), or NULL: DGRAD2 in bf16 */
    const uint8_t* dy_s;   /* [M_cap, d/32]                                     */
    const uint8_t* w2_q;   /* [E, n, d]       W2_e row-wise along d (DGRAD2 in) */
    const uint8_t* w2_s;   /* [E, n, d/32]                                      */
    uint8_t* dx_q;         /* [M_cap, d]      row-wise codes of dX_perm (DGRAD1 out), or NULL */
    uint8_t* dx_s;         /* [M_cap, d/32]                                     */
    uint8_t* dxt_q;        /* [d, M_cap]      column-wise codes of dX_perm, transposed (DGRAD1 out), or NULL */
    uint8_t* dxt_s;        /* [d, M_cap/32]                                     */
} moe_mx_bwd;

/*
 * moe_grouped_mlp_bwd -- backward of the expert MLP for fixed routing.
 *   [P2, backward-rewrite section: dS_{t,e} = <dO_t, Y> = <dO_t W2^T, A>;
 *   GEMM-overlapping section: the dH kernel reloads H in its epilogue and
 *   stores dH, dS and A'; P1, published-evidence section: dSwiGLU and dGeGLU
 *   fused into the dgrad GEMM.]
 *   DGRAD2: dA' = dY_u[R_e] W2_e^T (fp32); epilogue with a = f(g) u from
 *           the stored H (f the gate activation selected by act) and
 *           w = topk_w of the row's pair (0 for padding):
 *           dS partials += dA' . a per row; dA = w dA';
 *           dg = dA u f'(g) (silu' = s (1 + g (1 - s)), s = sigmoid(g);
 *           gelu' = Phi(g) + g phi(g)); du = dA f(g);
 *           dH = bf16 interleaved (dg, du); A' = bf16(w a);
 *           then ds[t, j] = sum of the row's partials in a fixed order.
 *   WGRAD2: dW2_e = A'[R_e]^T dY_u[R_e] (fp32; exactly 0 for empty experts).
 *   DGRAD1: dX_perm[R_e] = bf16(dH[R_e] W1_e^T).
 *   WGRAD1: dW1_e = X_perm[R_e]^T dH[R_e] (fp32, interleaved like w1).
 *   Non-gated act = MOE_ACT_SRELU: dH = bf16(w dA' * 2 relu(h)), A' = w relu(h)^2,
 *   dS partials += dA' . relu(h)^2; h, dh [M_cap, n], w1 and dw1 [E, d, n].
 *   dy_u = moe_permute of dO (unweighted). Stages run in the order above.
 *   With MOE_GATHER_ROWS in stages, x_perm is x [T, d] and dy_u is dO [T, d]
 *   (un-permuted) and every GEMM reads their rows through src_of.
 *   x_perm, dy_u [M_cap, d]; w1 [E, d, 2n]; w2 [E, n, d]; h [M_cap, 2n]
 *   (bf16, in); topk_w [T, k] fp32, src_of [M_cap], row_of [T*k],
 *   offsets [E+1] (in); dh [M_cap, 2n], a_w [M_cap, n], dx_perm [M_cap, d]
 *   (bf16, out); ds [T, k] fp32 (out); dw1 [E, d, 2n], dw2 [E, n, d]
 *   (fp32, out). Outputs of stages not requested may be NULL.
 *   workspace: >= moe_mlp_bwd_workspace_bytes(n, M_cap) bytes.
 *   With mx != NULL [P1, core-idea and published-evidence sections:
 *   GroupGemm + dActivation + Quantize/Transpose; P3, three-components
 *   section: MXFP8 grouped GEMM]: DGRAD2 stays bf16 and its epilogue also
 *   writes the MXFP8 copies of the bf16 dH (row-wise, and column-wise
 *   transposed) and of A' (column-wise transposed); the other three GEMMs
 *   run on MX-scaled MFMA: DGRAD1 from dh_q x w1_q (with dx_q != NULL its
 *   epilogue also writes the row-wise MXFP8 copy of the bf16 dX_perm, the
 *   "GroupGemm + Quantize" kernel [P3, next-steps section], with dxt_q !=
 *   NULL also its column-wise copy stored transposed, and dx_perm may then
 *   be NULL), WGRAD2 from awt_q x
 *   dyt_q, WGRAD1 from xt_q x dht_q (K = the expert's row region). Only the
 *   rows of expert regions are written in the transposed copies; dh and
 *   a_w may then be NULL (their bf16 stores are skipped; no stage reads
 *   them). With
 *   dy_q != NULL DGRAD2 also runs on MX-scaled MFMA (dy_q x w2_q, then d %
 *   128 == 0 and no MOE_GATHER_ROWS), its dGLU epilogue taking that product
 *   as dA' and dS on the rewritten side as always.
 * Requires the shape constraints of moe_grouped_mlp_fwd; with mx != NULL also
 * M_cap < 2^23 (the MX wgrads address 256 rows of the transposed [rows,
 * M_cap] copies with 32-bit byte offsets).
 */
int moe_grouped_mlp_bwd(const uint16_t* x_perm, const uint16_t* w1, const uint16_t* w2,
                        const uint16_t* h, const uint16_t* dy_u, const float* topk_w,
                        const int32_t* src_of, const int32_t* row_of, const int32_t* offsets,
                        int T, int k, int E, int d, int n, int64_t M_cap, int act,
                        unsigned stages, uint16_t* dh, uint16_t* a_w, float* ds,
                        uint16_t* dx_perm, float* dw1, float* dw2,
                        void* workspace, size_t workspace_bytes, const moe_mx_bwd* mx,
                        moe_stream_t stream);

/*
 * moe_quant_mxfp8 -- standalone MXFP8 quantization of `batch` bf16 matrices
 * src [batch, R, C] [P3, three-components section: group-aware MXFP8
 * quantization; P1, problem section: the BF16 -> MXFP8 pass plus its
 * transposed copy].
 *   MOE_QUANT_ROWWISE: blocks of 32 consecutive columns;
 *     q_row [batch, R, C] codes, s_row [batch, R, C/32] scales.
 *   MOE_QUANT_COLWISE: blocks of 32 consecutive rows, stored transposed;
 *     q_col [batch, C, R] codes, s_col [batch, C, R/32] scales.
 *   Row-wise needs C % 32 == 0, column-wise R % 32 == 0. On the expert-major
 *   buffer every 32-row block lies inside one expert region (regions are
 *   128-row aligned), which is what makes the quantization group-aware.
 */
int moe_quant_mxfp8(const uint16_t* src, int batch, int64_t R, int C, int mode,
                    uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                    moe_stream_t stream);

/*
 * moe_permute_quant_mxfp8 -- the expert-major permutation of x [T, d] fused
 * with its MXFP8 quantization: row r of the permuted matrix is
 * x[src_of[r] / k] (zeros where src_of[r] < 0), and it is quantized as
 * moe_quant_mxfp8 would quantize X_perm [M_cap, d], without the bf16 copy
 * ever being written [P1, problem section: the BF16 -> MXFP8 pass and its
 * transposed copy; P3, three-components section: group-aware MXFP8
 * quantization on the expert-major buffer].
 *   x [T, d] bf16, src_of [M_cap] (in, from moe_route_counts); mode, q_row
 *   [M_cap, d] + s_row [M_cap, d/32], q_col [d, M_cap] + s_col [d, M_cap/32]
 *   as in moe_quant_mxfp8 (out, every row of [0, M_cap)).
 * Requires d % 32 == 0, M_cap % 128 == 0, M_cap >= moe_capacity_rows(T, k, E),
 * 16-byte aligned x and code buffers.
 */
int moe_permute_quant_mxfp8(const uint16_t* x, const int32_t* src_of, int T, int k, int E, int d,
                            int64_t M_cap, int mode, uint8_t* q_row, uint8_t* s_row,
                            uint8_t* q_col, uint8_t* s_col, moe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
