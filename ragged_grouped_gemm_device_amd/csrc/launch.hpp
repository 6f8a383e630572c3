// Internal launcher declarations of libmoe (host side of the HIP kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#define MOE_MAX_E 1024
#define MOE_ALIGN_ROWS 128
#define MOE_ERRBIT_NONFINITE_LOGIT 0x1

namespace moe {

constexpr int kChunkPairs = 1024;  // pairs per wavefront chunk of the layout sort

int launch_route(const float* logits, int T, int E, int k, int renorm, int32_t* topk_idx,
                 float* topk_w, int32_t* counts, int32_t* offsets, int32_t* row_of,
                 int32_t* src_of, int64_t M_cap, int32_t* err_word, void* ws, hipStream_t s);
size_t route_workspace_bytes(int T, int k, int E);

// Allocation-free routing: the layout scratch is a static device array of
// kRouteStaticScratch bytes per GPU. Returns -3 when route_workspace_bytes
// exceeds it (nothing launched), -4 on a failed symbol lookup or launch.
constexpr size_t kRouteStaticScratch = (size_t)8 << 20;
constexpr int kMaxDevices = 64;
int launch_route_noalloc(const float* logits, int T, int E, int k, int renorm, int32_t* topk_idx,
                         float* topk_w, int32_t* counts, int32_t* offsets, int32_t* row_of,
                         int32_t* src_of, int64_t M_cap, int32_t* err_word, hipStream_t s);

int launch_route_bwd(const float* logits, int T, int E, int k, int renorm, const int32_t* topk_idx,
                     const float* ds, float* dlogits, hipStream_t s);
int launch_permute(const uint16_t* x, const int32_t* row_of, const int32_t* src_of,
                   const int32_t* offsets, int T, int k, int E, int d, int64_t M_cap, uint16_t* x_perm,
                   hipStream_t s);
int launch_combine(const uint16_t* y, const int32_t* row_of, const float* w, int T, int k, int d,
                   uint16_t* out, hipStream_t s);

// Grouped GEMMs. All take the device offsets [E+1] of the ragged layout.
// Rows of an operand read from an un-permuted [rows, cols] tensor through
// src_of (row r holds token src_of[r] / k; -1 reads zeros). src_of == nullptr:
// the operand is the expert-major copy itself.
struct GatherSpec {
    const int32_t* src_of;
    int k;
    int64_t rows;
};

// act: 0 = SwiGLU, 1 = GeGLU (the gate activation of the GLU epilogues)
int launch_fc1_glu(const uint16_t* x_perm, const uint16_t* w1, const int32_t* offsets, int E, int d,
                   int n, int64_t M_cap, int act, const GatherSpec& gx, uint16_t* h, uint16_t* a,
                   hipStream_t s);
int launch_fc1_glu_mx(const uint16_t* x_perm, const uint16_t* w1, const int32_t* offsets, int E,
                      int d, int n, int64_t M_cap, int act, const GatherSpec& gx, uint16_t* h,
                      uint16_t* a, uint8_t* a_q, uint8_t* a_s, uint8_t* at_q, uint8_t* at_s,
                      hipStream_t s);
// q_row / s_row (nullable): the row-wise MXFP8 copy of the bf16 output, written by
// the GEMM epilogue (GroupGemm + Quantize); the bf16 output is then nullable.
// q_col / s_col (nullable, only beside q_row): its column-wise copy, transposed
// (codes [N, M_cap], scales [N, M_cap / 32]).
int launch_mx_fc2(const uint8_t* a_q, const uint8_t* a_s, const uint8_t* w2t_q, const uint8_t* w2t_s,
                  const int32_t* offsets, int E, int d, int n, int64_t M_cap, uint16_t* y,
                  uint8_t* y_q, uint8_t* y_s, uint8_t* yt_q, uint8_t* yt_s, hipStream_t s);
// out[R_e] = MX(A[R_e]) x MX(B_e)^T (bf16 [M_cap, N]); A [M_cap, K], B [E, N, K]
int launch_mx_ragged_m(const uint8_t* a_q, const uint8_t* a_s, const uint8_t* b_q, const uint8_t* b_s,
                       const int32_t* offsets, int E, int N, int K, int64_t M_cap, uint16_t* out,
                       uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, hipStream_t s);
// out_e = MX(At[:, R_e]) x MX(Bt[:, R_e])^T (fp32 [E, M, N]); At [M, M_cap], Bt [N, M_cap]
int launch_mx_wgrad(const uint8_t* at_q, const uint8_t* at_s, int M, const uint8_t* bt_q,
                    const uint8_t* bt_s, int N, const int32_t* offsets, int E, int64_t M_cap,
                    float* out, hipStream_t s);
int launch_fc2(const uint16_t* a, const uint16_t* w2, const int32_t* offsets, int E, int d, int n,
               int64_t M_cap, uint16_t* y, uint8_t* y_q, uint8_t* y_s, uint8_t* yt_q, uint8_t* yt_s,
               hipStream_t s);
int launch_dgrad2_dglu(const uint16_t* dy_u, const uint16_t* w2, const uint16_t* h,
                       const float* topk_w, const int32_t* src_of, const int32_t* offsets, int E,
                       int d, int n, int64_t M_cap, int act, const GatherSpec& gdy, uint16_t* dh,
                       uint16_t* a_w, float* ds_part, hipStream_t s);
int launch_dgrad2_dglu_mx(const uint16_t* dy_u, const uint16_t* w2, const uint16_t* h,
                          const float* topk_w, const int32_t* src_of, const int32_t* offsets, int E,
                          int d, int n, int64_t M_cap, int act, const GatherSpec& gdy, uint16_t* dh,
                          uint16_t* a_w, float* ds_part, uint8_t* dh_q, uint8_t* dh_s,
                          uint8_t* dht_q, uint8_t* dht_s, uint8_t* awt_q, uint8_t* awt_s,
                          hipStream_t s);
// FC1 / FC2 dgrad on MXFP8 operands (codes + block scales along K = d)
int launch_fc1_glu_mxin(const uint8_t* x_q, const uint8_t* x_s, const uint8_t* w1t_q,
                        const uint8_t* w1t_s, const int32_t* offsets, int E, int d, int n,
                        int64_t M_cap, int act, uint16_t* h, uint16_t* a, uint8_t* a_q, uint8_t* a_s,
                        uint8_t* at_q, uint8_t* at_s, hipStream_t s);
int launch_dgrad2_dglu_mxin(const uint8_t* dy_q, const uint8_t* dy_s, const uint8_t* w2_q,
                            const uint8_t* w2_s, const uint16_t* h, const float* topk_w,
                            const int32_t* src_of, const int32_t* offsets, int E, int d, int n,
                            int64_t M_cap, int act, uint16_t* dh, uint16_t* a_w, float* ds_part,
                            uint8_t* dh_q, uint8_t* dh_s, uint8_t* dht_q, uint8_t* dht_s,
                            uint8_t* awt_q, uint8_t* awt_s, hipStream_t s);
int launch_ds_reduce(const float* ds_part, const int32_t* row_of, int T, int k, int n,
                     float* ds, hipStream_t s);
// n1: the FC1 width (2n gated, n non-gated), the K of this GEMM
int launch_dgrad1(const uint16_t* dh, const uint16_t* w1, const int32_t* offsets, int E, int d,
                  int n1, int64_t M_cap, uint16_t* dx_perm, hipStream_t s);
// gather: 0 none, 1 = the A operand (act) is gathered, 2 = the B operand (grad)
int launch_wgrad(const uint16_t* act, int Ma, const uint16_t* grad, int Nb, const int32_t* offsets,
                 int E, int gather, const GatherSpec& gs, float* dw, hipStream_t s);
int ds_partials_per_row(int n);

// MXFP8
int launch_quant_mxfp8(const uint16_t* src, int batch, int64_t R, int C, int mode, uint8_t* q_row,
                       uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, hipStream_t s);
int launch_permute_quant_mxfp8(const uint16_t* x, const int32_t* src_of, int k, int64_t M_cap, int d,
                               int mode, uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                               hipStream_t s);

}  // namespace moe
