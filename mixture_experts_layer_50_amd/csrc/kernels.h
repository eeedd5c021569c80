// Launchers of the token-level kernels (gate, permutation, combine).  Each
// enqueues on stream `s`, records itself in the kernel timer, and returns
// MOE_OK or MOE_ERR_HIP.
#pragma once

#include <algorithm>

#include "common.h"

namespace moe {

// route.hip
moe_status_t launch_balanced_gate(int T, int E, int k, int32_t* idx, float* w, hipStream_t s);
// The balanced gate with the expert sort in closed form (idx, w, offsets, perm, inv).
moe_status_t launch_balanced_route_permute(int T, int E, int k, int e_lo, int e_hi, int R_cap,
                                           int32_t* idx, float* w, int32_t* offsets,
                                           int32_t* perm, int32_t* inv, hipStream_t s);
// The row copy Xp[p] = x[perm[p] / k] of the permute (perm_gather_kernel).
moe_status_t launch_permute_gather(const void* x, const int32_t* inv, int T, int d, int k,
                                   int elt_bytes, void* xp, hipStream_t s);
moe_status_t launch_topk_softmax(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                                 hipStream_t s);
// The router for a few tokens (T <= SMALL_ROUTE_MAX_T): split over K in
// chunks of SMALL_ROUTE_KC rows of d (d % 64 == 0), then per token a
// fixed-order sum, the bias, the top k by rank and the softmax.  Workspace:
// the partial logits.
constexpr int SMALL_ROUTE_MAX_T = 16;
constexpr int SMALL_ROUTE_KC = 64;
int64_t small_router_ws_bytes(int T, int d, int E);
// The partial-logit kernel alone (the top-k then runs inside the small FFN's
// first kernel, see SmallRoute).
moe_status_t launch_small_router_part(const void* x, const void* wr, int T, int d, int E,
                                      int elt_bytes, float* part, hipStream_t s);
moe_status_t launch_small_router(const void* x, const void* wr, const float* bias, int T, int d,
                                 int E, int k, int elt_bytes, float* logits, int32_t* idx,
                                 float* w, float* part, hipStream_t s);
// moe_route's logits for T <= SMALL_ROUTE_MAX_T with no workspace (one
// workgroup per 16 bytes of a router row and up to 4 tokens walks all of d); when
// few_token_logits_fit.
bool few_token_logits_fit(int T, int E, int elt_bytes);
moe_status_t launch_few_token_logits(const void* x, const void* wr, const float* bias, int T,
                                     int d, int E, int elt_bytes, float* logits, hipStream_t s);
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
// The gate gradient from the dSwiGLU GEMM's shares: dw[s] = sum of the
// stride values part[inv[s]][0 .. stride) in order (0 when inv[s] < 0), only
// when *flag (device memory) is zero.
moe_status_t launch_gate_grad_sum(const int32_t* inv, const float* part, int stride, int slots,
                                  const int32_t* flag, float* dw, hipStream_t s);
// dyp[inv[t*k+j]] = w[t,j] dy[t] and dw[t,j] = <dy[t], yp[inv[t*k+j]]>; with
// dyp_flag (device memory), the kernel runs only when *dyp_flag is nonzero.
moe_status_t launch_combine_bwd(const void* dy, const void* yp, const int32_t* inv, const float* w,
                                int T, int d, int k, int elt_bytes, void* dyp, float* dw,
                                hipStream_t s, const int32_t* dyp_flag = nullptr);

// The routing-table check (moe_check_routing): range and repeat bits of the
// table into *flags; with offsets, also the group sizes (counts [E_loc],
// zeroed by the launcher) and the offsets compared with their prefix.
constexpr int CHECK_IDX_RANGE = 1, CHECK_IDX_REPEAT = 2, CHECK_OFFSETS = 4;
moe_status_t launch_check_routing(const int32_t* idx, int T, int k, int E, int e_lo, int e_hi,
                                  int R_cap, const int32_t* offsets, int32_t* counts,
                                  int32_t* flags, hipStream_t s);

// small.hip: the small-batch FFN (no sort): y[t] = sum_j w[t,j] FFN_e(x[t]) over
// the local, first-occurrence slots.  Workspace: fp32 gate/up partial sums
// [T*k, KS, 2I] (KS splits of d), Yp [T*k, d], the combine's arrival
// counters [T, d / (8 N)].  Needs T*k <= SMALL_MAX_PAIRS, d and I <=
// SMALL_MAX_WIDTH (the LDS the kernels' routing table and token rows take).
constexpr int64_t SMALL_MAX_PAIRS = 4096;
constexpr int SMALL_MAX_WIDTH = 8192;
// The gate folded into the small FFN's first kernel: every workgroup adds
// the router's partial logits [nsplit][T][E] itself (in split order, then the
// bias) and takes the top k by rank, as small_router_final_kernel does;
// workgroup 0 writes logits, idx and w.  For T*E <= SMALL_FUSED_ROUTE_MAX_TE
// and T*E*nsplit <= SMALL_FUSED_ROUTE_MAX (the partials one workgroup adds).
struct SmallRoute {
  const float* part;
  const float* bias;
  int nsplit, E;
  float* logits;
  int32_t* idx;
  float* w;
};
constexpr int SMALL_FUSED_ROUTE_MAX_TE = 1024;
constexpr int64_t SMALL_FUSED_ROUTE_MAX = 8192;
int64_t small_ffn_ws_bytes(int T, int d, int k, int I, int e_lo, int e_hi, int elt_bytes);
// route: the gate folded in (idx and w_topk are then its outputs), or null.
moe_status_t launch_small_ffn(const void* x, const int32_t* idx, const float* w_topk,
                              const void* wg, const void* wu, const void* wd, int T, int d, int k,
                              int I, int e_lo, int e_hi, int elt_bytes, void* y, void* ws,
                              hipStream_t s, const SmallRoute* route = nullptr);

}  // namespace moe
