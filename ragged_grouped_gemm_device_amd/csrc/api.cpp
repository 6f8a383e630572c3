// extern "C" entry points of libmoe: host-side validation, then kernel launches
// on the caller's stream. Nothing here allocates, synchronises or reads device
// memory; every shape that depends on the routing stays on the device.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "../../include/moe.h"
#include "launch.hpp"

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline hipStream_t S(moe_stream_t s) { return reinterpret_cast<hipStream_t>(s); }
inline int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

int64_t capacity(int T, int k, int E) {
    if (T <= 0 || k <= 0 || E <= 0 || k > E || E > MOE_MAX_EXPERTS) return -1;
    return align_up((int64_t)T * k, MOE_ALIGN) + (int64_t)MOE_ALIGN * E;
}

// Shapes of the grouped MLP that the kernels support.
int check_mlp_shape(int E, int d, int n, int64_t M_cap, int act) {
    if (E <= 0 || E > MOE_MAX_EXPERTS || d <= 0 || n <= 0 || M_cap <= 0) return MOE_ERR_INVALID_ARG;
    if (act != MOE_ACT_SWIGLU && act != MOE_ACT_GEGLU && act != MOE_ACT_SRELU) return MOE_ERR_UNSUPPORTED;
    if (d % 64 || n % 64 || M_cap % MOE_ALIGN) return MOE_ERR_UNSUPPORTED;
    // row maps are int32; a GEMM tile's 32-bit buffer offsets span at most
    // 256 rows of one operand (each K slab and tile gets its own 64-bit base)
    const int64_t n1 = act == MOE_ACT_SRELU ? n : 2 * n;
    if (M_cap > INT32_MAX || d > MOE_MAX_WIDTH || n1 > MOE_MAX_WIDTH) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_str(int status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
        case MOE_ERR_LAUNCH: return "MOE_ERR_LAUNCH";
        default: return "MOE_ERR_UNKNOWN";
    }
}

int64_t moe_capacity_rows(int T, int k, int E) { return capacity(T, k, E); }

size_t moe_route_workspace_bytes(int T, int k, int E) {
    if (capacity(T, k, E) < 0) return 0;
    return moe::route_workspace_bytes(T, k, E);
}

size_t moe_mlp_bwd_workspace_bytes(int n, int64_t M_cap) {
    if (n <= 0 || M_cap <= 0) return 0;
    return (size_t)M_cap * moe::ds_partials_per_row(n) * sizeof(float);
}

int moe_route_counts(const float* logits, int T, int E, int k, int renorm, int32_t* topk_idx,
                     float* topk_w, int32_t* counts, int32_t* offsets, int32_t* row_of,
                     int32_t* src_of, int64_t M_cap, int32_t* err_word, void* workspace,
                     size_t workspace_bytes, moe_stream_t stream) {
    const int64_t cap = capacity(T, k, E);
    if (cap < 0) return MOE_ERR_INVALID_ARG;
    if (!logits || !topk_idx || !topk_w || !counts || !offsets || !row_of || !src_of || !workspace)
        return MOE_ERR_INVALID_ARG;
    if (!aligned16(workspace)) return MOE_ERR_INVALID_ARG;
    if (M_cap < cap || M_cap > ((int64_t)1 << 31) - 1) return MOE_ERR_WORKSPACE;
    if (workspace_bytes < moe::route_workspace_bytes(T, k, E)) return MOE_ERR_WORKSPACE;
    const int rc = moe::launch_route(logits, T, E, k, renorm, topk_idx, topk_w, counts, offsets,
                                     row_of, src_of, M_cap, err_word, workspace, S(stream));
    return rc ? MOE_ERR_LAUNCH : MOE_OK;
}

int moe_route_counts_noalloc(const float* logits, int T, int E, int k, int renorm, int32_t* topk_idx,
                             float* topk_w, int32_t* counts, int32_t* offsets, int32_t* row_of,
                             int32_t* src_of, int64_t M_cap, int32_t* err_word, moe_stream_t stream) {
    const int64_t cap = capacity(T, k, E);
    if (cap < 0) return MOE_ERR_INVALID_ARG;
    if (!logits || !topk_idx || !topk_w || !counts || !offsets || !row_of || !src_of) return MOE_ERR_INVALID_ARG;
    if (M_cap < cap || M_cap > ((int64_t)1 << 31) - 1) return MOE_ERR_WORKSPACE;
    if (moe::route_workspace_bytes(T, k, E) > moe::kRouteStaticScratch) return MOE_ERR_WORKSPACE;
    const int rc = moe::launch_route_noalloc(logits, T, E, k, renorm, topk_idx, topk_w, counts, offsets, row_of,
                                             src_of, M_cap, err_word, S(stream));
    return rc == 0 ? MOE_OK : rc == -3 ? MOE_ERR_WORKSPACE : MOE_ERR_LAUNCH;
}

int moe_route_bwd(const float* logits, const int32_t* topk_idx, const float* ds, int T, int E, int k,
                  int renorm, float* dlogits, moe_stream_t stream) {
    if (T <= 0 || E <= 0 || k <= 0 || k > E || E > MOE_MAX_EXPERTS) return MOE_ERR_INVALID_ARG;
    if (!logits || !topk_idx || !ds || !dlogits) return MOE_ERR_INVALID_ARG;
    const int rc = moe::launch_route_bwd(logits, T, E, k, renorm, topk_idx, ds, dlogits, S(stream));
    return rc ? MOE_ERR_LAUNCH : MOE_OK;
}

int moe_permute(const uint16_t* x, const int32_t* row_of, const int32_t* src_of,
                const int32_t* offsets, int T, int k, int E, int d, int64_t M_cap, uint16_t* x_perm,
                moe_stream_t stream) {
    const int64_t cap = capacity(T, k, E);
    if (cap < 0 || d <= 0) return MOE_ERR_INVALID_ARG;
    if (!x || !row_of || !src_of || !offsets || !x_perm) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_INVALID_ARG;
    if (d % 8) return MOE_ERR_UNSUPPORTED;
    if (M_cap < cap) return MOE_ERR_WORKSPACE;
    const int rc = moe::launch_permute(x, row_of, src_of, offsets, T, k, E, d, M_cap, x_perm, S(stream));
    return rc ? MOE_ERR_LAUNCH : MOE_OK;
}

int moe_combine(const uint16_t* y, const int32_t* row_of, const float* w, int T, int k, int d,
                uint16_t* out, moe_stream_t stream) {
    if (T <= 0 || k <= 0 || d <= 0 || k > MOE_MAX_EXPERTS) return MOE_ERR_INVALID_ARG;
    if (!y || !row_of || !out) return MOE_ERR_INVALID_ARG;
    if (!aligned16(y) || !aligned16(out)) return MOE_ERR_INVALID_ARG;
    if (d % 8) return MOE_ERR_UNSUPPORTED;
    const int rc = moe::launch_combine(y, row_of, w, T, k, d, out, S(stream));
    return rc ? MOE_ERR_LAUNCH : MOE_OK;
}

// Gathered rows of an un-permuted [T, d] tensor (MOE_GATHER_ROWS): the map,
// the routing shape and the 32-bit addressing limit of the whole tensor.
static int gather_spec(unsigned stages, const int32_t* src_of, int T, int k, int E, int d,
                       moe::GatherSpec& gs) {
    gs = moe::GatherSpec{nullptr, 0, 0};
    if (!(stages & MOE_GATHER_ROWS)) return MOE_OK;
    if (!src_of || capacity(T, k, E) < 0) return MOE_ERR_INVALID_ARG;
    if ((int64_t)T * d * 2 >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    gs = moe::GatherSpec{src_of, k, (int64_t)T};
    return MOE_OK;
}

int moe_grouped_mlp_fwd(const uint16_t* x_perm, const uint16_t* w1, const uint16_t* w2,
                        const int32_t* offsets, const int32_t* src_of, int T, int k, int E, int d,
                        int n, int64_t M_cap, int act, unsigned stages, uint16_t* h, uint16_t* a,
                        uint16_t* y, const moe_mx_fwd* mx, moe_stream_t stream) {
    int rc = check_mlp_shape(E, d, n, M_cap, act);
    if (rc) return rc;
    if (!offsets) return MOE_ERR_INVALID_ARG;
    if ((stages & ~(unsigned)(MOE_STAGES_FWD | MOE_GATHER_ROWS)) || !(stages & MOE_STAGES_FWD))
        return MOE_ERR_INVALID_ARG;
    moe::GatherSpec gx;
    if ((rc = gather_spec(stages, src_of, T, k, E, d, gx))) return rc;
    // with mx: FC1's epilogue writes A's MXFP8 copies when a_q is given (it must be
    // when FC1 runs on MXFP8 operands); FC2 runs on MXFP8 operands (A's codes x W2's)
    // when w2t_q is given, else in bf16 from a and w2; y_q asks FC2's epilogue for
    // the row-wise MXFP8 copy of Y (GroupGemm + Quantize), and then y may be NULL
    const bool fc2_mx = mx && mx->w2t_q;
    const bool y_mx = mx && mx->y_q;
    if (mx) {
        if (act == MOE_ACT_SRELU) return MOE_ERR_UNSUPPORTED;  // MXFP8 copies exist for the GLU forms
        if ((mx->a_q == nullptr) != (mx->a_s == nullptr)) return MOE_ERR_INVALID_ARG;
        if ((mx->at_q == nullptr) != (mx->at_s == nullptr) || (mx->at_q && !mx->a_q)) return MOE_ERR_INVALID_ARG;
        if ((mx->y_q == nullptr) != (mx->y_s == nullptr)) return MOE_ERR_INVALID_ARG;
        if ((mx->yt_q == nullptr) != (mx->yt_s == nullptr) || (mx->yt_q && !mx->y_q)) return MOE_ERR_INVALID_ARG;
        if ((mx->a_q && (!aligned16(mx->a_q) || !aligned16(mx->a_s))) ||
            (mx->at_q && (!aligned16(mx->at_q) || !aligned16(mx->at_s))) || (mx->y_q && !aligned16(mx->y_q)) ||
            (mx->yt_q && (!aligned16(mx->yt_q) || !aligned16(mx->yt_s))))
            return MOE_ERR_INVALID_ARG;
        if (fc2_mx && (stages & MOE_STAGE_FC2)) {
            if (n % 128) return MOE_ERR_UNSUPPORTED;  // whole 128-byte K slabs of the MX FC2
            if (!mx->a_q || !mx->w2t_s || !aligned16(mx->w2t_q) || !aligned16(mx->w2t_s))
                return MOE_ERR_INVALID_ARG;
        }
    }
    // A is read by a bf16 FC2 and is the FC1 output unless only its MXFP8 copy is kept
    if (!a && (!mx || !mx->a_q || ((stages & MOE_STAGE_FC2) && !fc2_mx))) return MOE_ERR_INVALID_ARG;
    const bool fc1_mx = mx && mx->x_q;  // FC1 on MXFP8 operands
    if (fc1_mx && (stages & MOE_STAGE_FC1)) {
        if (d % 128 || (stages & MOE_GATHER_ROWS)) return MOE_ERR_UNSUPPORTED;
        if (!mx->x_s || !mx->w1t_q || !mx->w1t_s || !aligned16(mx->x_q) || !aligned16(mx->w1t_q))
            return MOE_ERR_INVALID_ARG;
    }
    if (fc1_mx && (stages & MOE_STAGE_FC1) && !mx->a_q) return MOE_ERR_INVALID_ARG;
    if ((stages & MOE_STAGE_FC1) && !fc1_mx) {
        if (!x_perm || !w1 || !aligned16(x_perm) || !aligned16(w1)) return MOE_ERR_INVALID_ARG;
    }
    if ((stages & MOE_STAGE_FC1) && h && !aligned16(h)) return MOE_ERR_INVALID_ARG;
    if (a && !aligned16(a)) return MOE_ERR_INVALID_ARG;
    if (stages & MOE_STAGE_FC2) {
        if ((!y && !y_mx) || (y && !aligned16(y))) return MOE_ERR_INVALID_ARG;
        if (!fc2_mx && (!w2 || !aligned16(w2))) return MOE_ERR_INVALID_ARG;
    }
    hipStream_t s = S(stream);
    if (stages & MOE_STAGE_FC1) {
        const int rc1 = fc1_mx ? moe::launch_fc1_glu_mxin(mx->x_q, mx->x_s, mx->w1t_q, mx->w1t_s, offsets, E,
                                                          d, n, M_cap, act, h, a, mx->a_q, mx->a_s, mx->at_q,
                                                          mx->at_s, s)
                        : (mx && mx->a_q)
                            ? moe::launch_fc1_glu_mx(x_perm, w1, offsets, E, d, n, M_cap, act, gx, h, a, mx->a_q,
                                                     mx->a_s, mx->at_q, mx->at_s, s)
                            : moe::launch_fc1_glu(x_perm, w1, offsets, E, d, n, M_cap, act, gx, h, a, s);
        if (rc1) return MOE_ERR_LAUNCH;
    }
    if (stages & MOE_STAGE_FC2) {
        uint8_t* y_q = y_mx ? mx->y_q : nullptr;
        uint8_t* y_s = y_mx ? mx->y_s : nullptr;
        uint8_t* yt_q = y_mx ? mx->yt_q : nullptr;
        uint8_t* yt_s = y_mx ? mx->yt_s : nullptr;
        const int rc2 = fc2_mx ? moe::launch_mx_fc2(mx->a_q, mx->a_s, mx->w2t_q, mx->w2t_s, offsets, E, d, n,
                                                     M_cap, y, y_q, y_s, yt_q, yt_s, s)
                               : moe::launch_fc2(a, w2, offsets, E, d, n, M_cap, y, y_q, y_s, yt_q, yt_s, s);
        if (rc2) return MOE_ERR_LAUNCH;
    }
    return MOE_OK;
}

int moe_grouped_mlp_bwd(const uint16_t* x_perm, const uint16_t* w1, const uint16_t* w2,
                        const uint16_t* h, const uint16_t* dy_u, const float* topk_w,
                        const int32_t* src_of, const int32_t* row_of, const int32_t* offsets,
                        int T, int k, int E, int d, int n, int64_t M_cap, int act, unsigned stages,
                        uint16_t* dh, uint16_t* a_w, float* ds, uint16_t* dx_perm, float* dw1,
                        float* dw2, void* workspace, size_t workspace_bytes,
                        const moe_mx_bwd* mx, moe_stream_t stream) {
    int rc = check_mlp_shape(E, d, n, M_cap, act);
    if (rc) return rc;
    const int64_t cap = capacity(T, k, E);
    if (cap < 0) return MOE_ERR_INVALID_ARG;
    if (M_cap < cap) return MOE_ERR_WORKSPACE;
    if ((stages & ~(unsigned)(MOE_STAGES_BWD | MOE_GATHER_ROWS)) || !(stages & MOE_STAGES_BWD))
        return MOE_ERR_INVALID_ARG;
    if (!offsets) return MOE_ERR_INVALID_ARG;
    moe::GatherSpec gs;
    if ((rc = gather_spec(stages, src_of, T, k, E, d, gs))) return rc;
    const bool dgrad2_mx = mx && mx->dy_q;  // FC2 dgrad on MXFP8 operands
    if (stages & MOE_STAGE_DGRAD2) {
        // with mx the bf16 dH and A' are optional (the later stages read their MXFP8 copies)
        if (!h || !topk_w || !src_of || !row_of || !ds || !workspace || (!mx && (!dh || !a_w)))
            return MOE_ERR_INVALID_ARG;
        if (!aligned16(h) || (dh && !aligned16(dh)) || (a_w && !aligned16(a_w)) || !aligned16(workspace))
            return MOE_ERR_INVALID_ARG;
        if (dgrad2_mx) {
            if (d % 128 || (stages & MOE_GATHER_ROWS)) return MOE_ERR_UNSUPPORTED;
            if (!mx->dy_s || !mx->w2_q || !mx->w2_s || !aligned16(mx->dy_q) || !aligned16(mx->w2_q))
                return MOE_ERR_INVALID_ARG;
        } else if (!dy_u || !w2 || !aligned16(dy_u) || !aligned16(w2)) {
            return MOE_ERR_INVALID_ARG;
        }
        if (workspace_bytes < moe_mlp_bwd_workspace_bytes(n, M_cap)) return MOE_ERR_WORKSPACE;
    }
    // with mx the last three GEMMs read only the MXFP8 copies
    if (stages & MOE_STAGE_WGRAD2) {
        if (!dw2 || !aligned16(dw2)) return MOE_ERR_INVALID_ARG;
        if (!mx && (!a_w || !dy_u || !aligned16(a_w) || !aligned16(dy_u))) return MOE_ERR_INVALID_ARG;
    }
    if (stages & MOE_STAGE_DGRAD1) {
        // with mx->dx_q the FC1 dgrad also writes dX_perm's row-wise MXFP8 copy
        // (GroupGemm + Quantize) and dx_perm may be NULL
        const bool dx_mx = mx && mx->dx_q;
        if ((!dx_perm && !dx_mx) || (dx_perm && !aligned16(dx_perm))) return MOE_ERR_INVALID_ARG;
        if (mx && ((mx->dx_q == nullptr) != (mx->dx_s == nullptr) || (dx_mx && !aligned16(mx->dx_q))))
            return MOE_ERR_INVALID_ARG;
        if (mx && ((mx->dxt_q == nullptr) != (mx->dxt_s == nullptr) || (mx->dxt_q && !dx_mx) ||
                   (mx->dxt_q && (!aligned16(mx->dxt_q) || !aligned16(mx->dxt_s)))))
            return MOE_ERR_INVALID_ARG;
        if (!mx && (!dh || !w1 || !aligned16(dh) || !aligned16(w1))) return MOE_ERR_INVALID_ARG;
    }
    if (stages & MOE_STAGE_WGRAD1) {
        if (!dw1 || !aligned16(dw1)) return MOE_ERR_INVALID_ARG;
        if (!mx && (!x_perm || !dh || !aligned16(x_perm) || !aligned16(dh))) return MOE_ERR_INVALID_ARG;
    }
    if (mx && act == MOE_ACT_SRELU) return MOE_ERR_UNSUPPORTED;
    // MX wgrads: 256 rows of a transposed [rows, M_cap] copy per tile, 32-bit offsets
    if (mx && M_cap >= ((int64_t)1 << 23)) return MOE_ERR_UNSUPPORTED;
    const int n1 = act == MOE_ACT_SRELU ? n : 2 * n;  // FC1 width
    if (mx) {
        auto ok = [](const void* p, const void* q) { return p && q && aligned16(p); };
        if ((stages & MOE_STAGE_DGRAD2) &&
            (!ok(mx->dh_q, mx->dh_s) || !ok(mx->dht_q, mx->dht_s) || !ok(mx->awt_q, mx->awt_s)))
            return MOE_ERR_INVALID_ARG;
        if ((stages & MOE_STAGE_WGRAD2) && (!ok(mx->awt_q, mx->awt_s) || !ok(mx->dyt_q, mx->dyt_s)))
            return MOE_ERR_INVALID_ARG;
        if ((stages & MOE_STAGE_DGRAD1) && (!ok(mx->dh_q, mx->dh_s) || !ok(mx->w1_q, mx->w1_s)))
            return MOE_ERR_INVALID_ARG;
        if ((stages & MOE_STAGE_WGRAD1) && (!ok(mx->xt_q, mx->xt_s) || !ok(mx->dht_q, mx->dht_s)))
            return MOE_ERR_INVALID_ARG;
    }
    hipStream_t s = S(stream);
    float* part = static_cast<float*>(workspace);
    if (stages & MOE_STAGE_DGRAD2) {
        const int rc2 = dgrad2_mx
                            ? moe::launch_dgrad2_dglu_mxin(mx->dy_q, mx->dy_s, mx->w2_q, mx->w2_s, h, topk_w, src_of,
                                                           offsets, E, d, n, M_cap, act, dh, a_w, part, mx->dh_q,
                                                           mx->dh_s, mx->dht_q, mx->dht_s, mx->awt_q, mx->awt_s, s)
                        : mx ? moe::launch_dgrad2_dglu_mx(dy_u, w2, h, topk_w, src_of, offsets, E, d, n, M_cap,
                                                         act, gs, dh, a_w, part, mx->dh_q, mx->dh_s,
                                                         mx->dht_q, mx->dht_s, mx->awt_q, mx->awt_s, s)
                           : moe::launch_dgrad2_dglu(dy_u, w2, h, topk_w, src_of, offsets, E, d, n, M_cap,
                                                      act, gs, dh, a_w, part, s);
        if (rc2) return MOE_ERR_LAUNCH;
        if (moe::launch_ds_reduce(part, row_of, T, k, n, ds, s)) return MOE_ERR_LAUNCH;
    }
    if (stages & MOE_STAGE_WGRAD2) {
        const int rc2 = mx ? moe::launch_mx_wgrad(mx->awt_q, mx->awt_s, n, mx->dyt_q, mx->dyt_s, d, offsets,
                                                   E, M_cap, dw2, s)
                           : moe::launch_wgrad(a_w, n, dy_u, d, offsets, E, 2, gs, dw2, s);
        if (rc2) return MOE_ERR_LAUNCH;
    }
    if (stages & MOE_STAGE_DGRAD1) {
        const int rc1 = mx ? moe::launch_mx_ragged_m(mx->dh_q, mx->dh_s, mx->w1_q, mx->w1_s, offsets, E, d,
                                                      2 * n, M_cap, dx_perm, mx->dx_q, mx->dx_s, mx->dxt_q,
                                                      mx->dxt_s, s)
                           : moe::launch_dgrad1(dh, w1, offsets, E, d, n1, M_cap, dx_perm, s);
        if (rc1) return MOE_ERR_LAUNCH;
    }
    if (stages & MOE_STAGE_WGRAD1) {
        const int rc1 = mx ? moe::launch_mx_wgrad(mx->xt_q, mx->xt_s, d, mx->dht_q, mx->dht_s, 2 * n, offsets,
                                                   E, M_cap, dw1, s)
                           : moe::launch_wgrad(x_perm, d, dh, n1, offsets, E, 1, gs, dw1, s);
        if (rc1) return MOE_ERR_LAUNCH;
    }
    return MOE_OK;
}

int moe_quant_mxfp8(const uint16_t* src, int batch, int64_t R, int C, int mode, uint8_t* q_row,
                    uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, moe_stream_t stream) {
    if (!src || batch <= 0 || R <= 0 || C <= 0) return MOE_ERR_INVALID_ARG;
    if (mode <= 0 || (mode & ~(MOE_QUANT_ROWWISE | MOE_QUANT_COLWISE))) return MOE_ERR_INVALID_ARG;
    if ((mode & MOE_QUANT_ROWWISE) && (!q_row || !s_row)) return MOE_ERR_INVALID_ARG;
    if ((mode & MOE_QUANT_COLWISE) && (!q_col || !s_col)) return MOE_ERR_INVALID_ARG;
    if (C % MOE_MX_BLOCK) return MOE_ERR_UNSUPPORTED;
    if ((mode & MOE_QUANT_COLWISE) && R % MOE_MX_BLOCK) return MOE_ERR_UNSUPPORTED;
    if (!aligned16(src) || (q_row && !aligned16(q_row)) || (q_col && !aligned16(q_col)))
        return MOE_ERR_INVALID_ARG;
    if (R * C * batch >= ((int64_t)1 << 40) || (R + 127) / 128 > 65535 || batch > 65535)
        return MOE_ERR_UNSUPPORTED;
    const int rc = moe::launch_quant_mxfp8(src, batch, R, C, mode, q_row, s_row, q_col, s_col, S(stream));
    return rc ? MOE_ERR_LAUNCH : MOE_OK;
}

int moe_permute_quant_mxfp8(const uint16_t* x, const int32_t* src_of, int T, int k, int E, int d,
                            int64_t M_cap, int mode, uint8_t* q_row, uint8_t* s_row, uint8_t* q_col,
                            uint8_t* s_col, moe_stream_t stream) {
    if (!x || !src_of || d <= 0 || M_cap <= 0) return MOE_ERR_INVALID_ARG;
    const int64_t cap = capacity(T, k, E);
    if (cap < 0) return MOE_ERR_INVALID_ARG;
    if (M_cap < cap) return MOE_ERR_WORKSPACE;
    if (mode <= 0 || (mode & ~(MOE_QUANT_ROWWISE | MOE_QUANT_COLWISE))) return MOE_ERR_INVALID_ARG;
    if ((mode & MOE_QUANT_ROWWISE) && (!q_row || !s_row)) return MOE_ERR_INVALID_ARG;
    if ((mode & MOE_QUANT_COLWISE) && (!q_col || !s_col)) return MOE_ERR_INVALID_ARG;
    if (d % MOE_MX_BLOCK || M_cap % MOE_ALIGN) return MOE_ERR_UNSUPPORTED;
    if (!aligned16(x) || (q_row && !aligned16(q_row)) || (q_col && !aligned16(q_col)))
        return MOE_ERR_INVALID_ARG;
    if (M_cap * d >= ((int64_t)1 << 40) || (M_cap + 127) / 128 > 65535) return MOE_ERR_UNSUPPORTED;
    const int rc = moe::launch_permute_quant_mxfp8(x, src_of, k, M_cap, d, mode, q_row, s_row, q_col, s_col,
                                                   S(stream));
    return rc ? MOE_ERR_LAUNCH : MOE_OK;
}

}  // extern "C"
