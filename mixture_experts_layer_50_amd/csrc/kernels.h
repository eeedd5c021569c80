// Launchers of the token-level kernels (gate, permutation, combine).  Each
// enqueues on stream `s`, records itself in the kernel timer, and returns
// MOE_OK or MOE_ERR_HIP.
#pragma once

#include <algorithm>

#include "common.h"

namespace moe {

// route.hip
moe_status_t launch_balanced_gate(int T, int E, int k, int32_t* idx, float* w, hipStream_t s);
moe_status_t launch_topk_softmax(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                                 hipStream_t s);
// Tokens per workgroup of the router backward (one bias-gradient partial each).
constexpr int ROUTE_BWD_TOKENS = 32;
// logits / aux_w (both or neither): add the auxiliary loss's logit gradient.
moe_status_t launch_route_bwd_dl(const int32_t* idx, const float* g, const float* dg, int T, int E,
                                 int k, float* dl, bf16_t* dl_bf16, float* db_part,
                                 const float* logits, const float* aux_w, hipStream_t s);
// Load-balancing auxiliary loss: loss[0] and aux_w[E] (the backward's weights).
int64_t aux_loss_ws_bytes(int T, int E);
moe_status_t launch_aux_loss(const float* logits, const int32_t* idx, int T, int E, int k,
                             float alpha, float* loss, float* aux_w, void* ws, hipStream_t s);
moe_status_t launch_route_bwd_reduce(const float* dw_part, int nsplit, int64_t n_dw, bf16_t* dw,
                                     const float* db_part, int nblk, int E, float* db,
                                     hipStream_t s);
// Zeroes up to three buffers (null ones are skipped) in one launch.
moe_status_t launch_fill_zero(void* p0, int64_t bytes0, void* p1, int64_t bytes1, void* p2,
                              int64_t bytes2, hipStream_t s);

// permute.hip
constexpr int PERM_TOKENS = 256;  // tokens per block of the counting sort
int64_t permute_ws_bytes(int T, int E_loc);
moe_status_t launch_permute(const int32_t* idx, const void* x, int T, int d, int k, int e_lo,
                            int e_hi, int R_cap, int elt_bytes, int32_t* offsets, int32_t* perm,
                            int32_t* inv, void* xp, void* ws, hipStream_t s);
// y[t] = sum_j w[t,j] * src[inv[t*k+j]] (w == NULL: weight 1), fp32 accumulation.
moe_status_t launch_gather_sum(const void* src, const int32_t* inv, const float* w, int T, int d,
                               int k, int elt_bytes, void* y, hipStream_t s, const char* name);
moe_status_t launch_combine_bwd(const void* dy, const void* yp, const int32_t* inv, const float* w,
                                int T, int d, int k, int elt_bytes, void* dyp, float* dw,
                                hipStream_t s);

// small.hip: the small-batch FFN (no sort): y[t] = sum_j w[t,j] FFN_e(x[t]) over
// the local, first-occurrence slots.  Workspace: fp32 gate/up partial sums
// [T*k, KS, 2I] (KS splits of d), Yp [T*k, d], the slot map [T*k].  Needs T*k <= SMALL_MAX_PAIRS, d and I <= SMALL_MAX_WIDTH.
constexpr int64_t SMALL_MAX_PAIRS = 65535;
constexpr int SMALL_MAX_WIDTH = 12288;
int64_t small_ffn_ws_bytes(int T, int d, int k, int I, int elt_bytes);
moe_status_t launch_small_ffn(const void* x, const int32_t* idx, const float* w_topk,
                              const void* wg, const void* wu, const void* wd, int T, int d, int k,
                              int I, int e_lo, int e_hi, int elt_bytes, void* y, void* ws,
                              hipStream_t s);

}  // namespace moe
