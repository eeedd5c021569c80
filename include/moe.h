/*
 * moe.h -- C ABI of the MoE expert layer for AMD Instinct MI355X (gfx950).
 *
 * The layer: route every token to k of E experts, sort the (token, slot) rows
 * by expert, run each expert's SwiGLU FFN over its group as one grouped GEMM,
 * and sum the expert outputs back per token with the gate weights; plus the
 * backward pass of every step for full fine-tuning.
 *
 * Pages cited (by title and section):
 *   [P3] "Accelerating Transformers fine-tuning with NVIDIA NeMo AutoModel"
 *        (zh-CN translation on neows.pages.dev);
 *   [P1] "NVIDIA NeMo AutoModel MoE 微調的 3.7 倍加速突破" (digest).
 * [P3] section 背景 (background) states the problem: route tokens across
 * hundreds of experts and fuse the expert matmuls into a single kernel.
 * [P3] section 专家后端 (expert backends), grouped_mm row: sort tokens by their
 * assigned expert, then one grouped GEMM.  [P3] section 加速来源, DeepEP item:
 * token dispatch and combine are their own fused kernels.  Each entry point
 * below is one of those steps.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer is a DEVICE pointer (memory of the current HIP device) unless
 *   stated otherwise.  Matrices are row-major and dense (no padding).
 * - The caller owns every buffer.  The library never allocates, frees or keeps
 *   device memory; it keeps no state between calls except the optional kernel
 *   timer (moe_prof_*), a thread-local error string, and the one static
 *   scratch array of moe_grouped_ffn_fwd_gather_noalloc (4 MiB per device,
 *   part of the library image, held until the process ends).
 * - Every call enqueues its kernels on `stream` (a hipStream_t; NULL = the
 *   default stream) and returns without waiting for them.  Data-dependent sizes
 *   (group sizes, the routed row count R) stay on the device: buffers are sized
 *   for the capacity R_cap and kernels read the true counts from group_offsets.
 * - Arguments are validated before anything is launched.  On a non-OK status
 *   nothing was enqueued and no output was touched; moe_last_error() then
 *   holds a one-line description.  MOE_ERR_HIP means a launch failed after
 *   validation (earlier kernels of the same call may have run).
 * - dtype MOE_F32: every float tensor is fp32.  dtype MOE_BF16: activations,
 *   weights and their gradients are bf16 (uint16 bit patterns); logits, gate
 *   weights and their gradients are fp32; every accumulation is fp32 and every
 *   conversion to bf16 rounds to nearest even.
 * - Supported shapes: d % 64 == 0, I % 64 == 0, E <= 512 (and E % 8 == 0 for
 *   bf16), 1 <= k <= min(E, 32), T*k < 2^31, and every pointer 16-byte aligned
 *   (workspaces 256-byte aligned).  Others return MOE_ERR_UNSUPPORTED.
 * - Results are deterministic: no floating-point atomics; every sum has a fixed
 *   order, so two identical calls give bit-identical outputs.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = 1,         /* null pointer where one is required, k > E, bad enum, e_lo/e_hi out of range */
  MOE_ERR_SHAPE = 2,       /* non-positive or overflowing sizes */
  MOE_ERR_DTYPE = 3,       /* unknown dtype */
  MOE_ERR_WORKSPACE = 4,   /* workspace smaller than moe_workspace_size() */
  MOE_ERR_HIP = 5,         /* a HIP launch failed; moe_last_error() has the HIP message */
  MOE_ERR_UNSUPPORTED = 6  /* valid but outside the supported shapes listed above */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

/* The gate.  The pages fix neither the gate function nor tie-breaking:
 * MOE_GATE_SOFTMAX_TOPK takes the k largest logits (ties toward the lower
 * expert id, slots in descending-logit order) and softmax over those k.
 * MOE_GATE_BALANCED is the balanced routing gate of [P3] section
 * 单节点30B MoE基准测试 (note on the routing gate: tokens are forced evenly
 * over the experts): slot i of token t goes to expert (t mod P) + i*P with
 * P = E/k, weight 1/k.  It needs k | E. */
typedef enum { MOE_GATE_SOFTMAX_TOPK = 0, MOE_GATE_BALANCED = 1 } moe_gate_t;

/* Which call a workspace size is asked for. */
typedef enum {
  MOE_OP_ROUTE = 0, MOE_OP_PERMUTE = 1, MOE_OP_FFN_FWD = 2, MOE_OP_COMBINE = 3,
  MOE_OP_COMBINE_BWD = 4, MOE_OP_FFN_BWD = 5, MOE_OP_PERMUTE_BWD = 6, MOE_OP_ROUTE_BWD = 7,
  MOE_OP_SMALL_FWD = 8, MOE_OP_AUX_LOSS = 9, MOE_OP_FFN_FWD_FUSED = 10, MOE_OP_ROUTE_PERMUTE = 11,
  MOE_OP_SMALL_ROUTED_FWD = 12, MOE_OP_CHECK_ROUTING = 13
} moe_op_t;

typedef void* moe_stream_t; /* hipStream_t */

/* Layer shape.  E counts ALL experts; this GPU holds the local experts
 * [e_lo, e_hi) (expert parallelism shards experts along the expert dimension,
 * [P3] section 专家并行与DeepEP).  On one GPU holding every expert: 0, E.
 * R_cap is the row capacity of the permuted buffers (0 means T*k): rows whose
 * expert-sorted position is >= R_cap are dropped (see moe_permute). */
typedef struct {
  int32_t T, d, E, k, I;
  int32_t e_lo, e_hi;
  int32_t R_cap;
  moe_dtype_t dtype;
  moe_gate_t gate;
} moe_shape_t;

/* ---------------------------------------------------------------- utility */
const char* moe_status_string(moe_status_t s);    /* static string, never NULL */
const char* moe_last_error(void);                 /* thread-local, valid until the next call on this thread */
const char* moe_version(void);                    /* static string */

/* Host-side query: bytes of workspace `op` needs for `shape` (0 if none).
 * Errors: MOE_ERR_ARG if shape or bytes is NULL or op unknown; the shape
 * errors of the op itself. */
moe_status_t moe_workspace_size(const moe_shape_t* shape, int op, size_t* bytes);

/* ------------------------------------------------------------- forward */

/* a1 -- route.  [P3] section 背景: route tokens across many experts.
 * softmax_topk: logits = x * w_router (+ bias) with fp32 accumulation, then the
 *   k largest per token (ties -> lower id), topk_w = softmax over those k.
 *   For T <= 16 (and E * element bytes a multiple of 16) the logits come from
 *   a kernel that walks all of d per group of experts instead of the MFMA
 *   router: fixed-order sums in another order, so they may differ from the
 *   MFMA router's in the last bits; both are deterministic.
 * balanced: topk_idx/topk_w from the balanced gate; x, w_router, bias and
 *   logits are not read or written (they may be NULL).
 * x [T,d] (dtype); w_router [d,E] (dtype); bias [E] fp32 or NULL;
 * logits [T,E] fp32 (required for softmax_topk); topk_idx [T,k] int32 (global
 * expert ids); topk_w [T,k] fp32.  No workspace. */
moe_status_t moe_route(const moe_shape_t* shape, const void* x, const void* w_router,
                       const float* bias, float* logits, int32_t* topk_idx, float* topk_w,
                       moe_stream_t stream);

/* a2 -- permute: the rows sorted by their expert ([P3] section 专家后端, grouped_mm row).
 * Rows r = t*k + j whose expert e = topk_idx[t,j] is local (e_lo <= e < e_hi)
 * are ordered by expert and, inside an expert, by r (a stable sort; the
 * result is unique).  Outputs:
 *   group_offsets [E_loc+1] int32: exclusive prefix of the group sizes,
 *     clamped to R_cap; rows of local expert e_lo+i are [o_i, o_{i+1});
 *   perm [R_cap] int32: perm[p] = r of the row at sorted position p
 *     (positions >= group_offsets[E_loc] are left untouched);
 *   inv [T*k] int32: sorted position of row r, or -1 if r is not local, was
 *     dropped by the capacity, or repeats an expert id an earlier slot of the
 *     same token already holds (routing never produces repeats);
 *   xp [R_cap, d] (dtype): xp[p] = x[perm[p] / k] (rows past the end untouched).
 *     xp may be NULL (then x may be NULL too): only the sort runs, for the
 *     _gather forms of the FFN calls below, which read x through perm.
 * ws/ws_bytes: workspace of moe_workspace_size(MOE_OP_PERMUTE). */
moe_status_t moe_permute(const moe_shape_t* shape, const int32_t* topk_idx, const void* x,
                         int32_t* group_offsets, int32_t* perm, int32_t* inv, void* xp,
                         void* ws, size_t ws_bytes, moe_stream_t stream);

/* a1 + a2 in one call: moe_route followed by moe_permute, with the same
 * arguments, outputs and results (bit-identical).  Under the balanced gate
 * the sort has a closed form (expert e = (t mod P) + j*P receives the tokens
 * t = e mod P, e mod P + P, ... in token order), so idx, topk_w,
 * group_offsets, perm and inv come from one kernel and x, w_router, bias and
 * logits are not touched (xp, when given, is still filled from x).  Under the
 * softmax top-k gate the router kernels run, then the sort.  ws:
 * moe_workspace_size(MOE_OP_ROUTE_PERMUTE) (0 for the balanced gate, else
 * the permute's workspace). */
moe_status_t moe_route_permute(const moe_shape_t* shape, const void* x, const void* w_router,
                               const float* bias, float* logits, int32_t* topk_idx, float* topk_w,
                               int32_t* group_offsets, int32_t* perm, int32_t* inv, void* xp,
                               void* ws, size_t ws_bytes, moe_stream_t stream);

/* a3 + a4 -- expert FFN over the expert groups as grouped GEMMs (one grouped
 * GEMM over all groups, [P3] section 专家后端; experts are fused 3-D weight tensors,
 * [P3] note under the Qwen3 table).  For each local expert i and every row p
 * in [o_i, o_{i+1}):
 *   Hg = xp[p] * w_gate[i], Hu = xp[p] * w_up[i]      (fp32 accumulation)
 *   A  = silu(Hg) * Hu,  silu(z) = z / (1 + exp(-z))
 *   yp[p] = A * w_down[i]
 * xp [R_cap,d]; w_gate, w_up [E_loc,d,I]; w_down [E_loc,I,d];
 * h_save [R_cap,2I] receives [Hg | Hu] (NULL for inference);
 * a_save [R_cap,I] receives A (required: it also feeds the down GEMM);
 * yp [R_cap,d].  Rows past group_offsets[E_loc] are untouched.
 * ws: moe_workspace_size(MOE_OP_FFN_FWD). */
moe_status_t moe_grouped_ffn_fwd(const moe_shape_t* shape, const void* xp,
                                 const int32_t* group_offsets, const void* w_gate,
                                 const void* w_up, const void* w_down, void* h_save,
                                 void* a_save, void* yp, void* ws, size_t ws_bytes,
                                 moe_stream_t stream);

/* a2 + a3 + a4 fused -- the same FFN with the dispatch copy folded into the
 * gate/up GEMM's operand loads (the one-GPU counterpart of dispatch fused with
 * the expert computation, [P3] section 加速来源, DeepEP item): row p of Xp is
 * read as x[perm[p] / k] and Xp is never written.  Results are bit-identical
 * to moe_permute(xp) followed by moe_grouped_ffn_fwd.  x [T,d]; perm [R_cap]
 * as written by moe_permute (which may then skip xp); the other arguments and
 * the workspace as for moe_grouped_ffn_fwd.  Needs T*d*element bytes < 2^31
 * (else MOE_ERR_UNSUPPORTED). */
moe_status_t moe_grouped_ffn_fwd_gather(const moe_shape_t* shape, const void* x,
                                        const int32_t* perm, const int32_t* group_offsets,
                                        const void* w_gate, const void* w_up,
                                        const void* w_down, void* h_save, void* a_save,
                                        void* yp, void* ws, size_t ws_bytes,
                                        moe_stream_t stream);

/* moe_grouped_ffn_fwd_gather without a workspace, for callers that cannot
 * allocate (code under HIP-graph capture, serving loops, harnesses that
 * forbid allocation).  Same arguments, kernels and bit-identical results as
 * moe_grouped_ffn_fwd_gather minus ws/ws_bytes: the tile tables and the token
 * table live in a static device array of 4 MiB per device instead (enough
 * for R_cap up to about 900,000 rows; a shape whose tables need more returns
 * MOE_ERR_UNSUPPORTED before anything is launched).  The call allocates
 * nothing: on its first call on a device it looks up that device's copy of
 * the array (hipGetSymbolAddress, with the device current) and keeps the
 * address.  Every call rewrites the part of the array it reads, so nothing
 * needs clearing between calls; but every call on one device shares that
 * device's array, so calls that may overlap on one device (different
 * streams without ordering between them) race and give wrong results.  The
 * stream must belong to the current device. */
moe_status_t moe_grouped_ffn_fwd_gather_noalloc(const moe_shape_t* shape, const void* x,
                                                const int32_t* perm,
                                                const int32_t* group_offsets,
                                                const void* w_gate, const void* w_up,
                                                const void* w_down, void* h_save, void* a_save,
                                                void* yp, moe_stream_t stream);

/* a2 + a3 + a4 + a5 fused -- the gathered FFN forward with the combine run in
 * the down projection's epilogue, the one-GPU counterpart of dispatch and
 * combine fused with the expert computation ([P3] section 加速来源, DeepEP
 * item; the pages' DeepEP kernels move tokens between GPUs, here the rows stay
 * on one).  Row p of Xp is read as x[perm[p] / k] (as in
 * moe_grouped_ffn_fwd_gather), and
 *   y[t] = sum_j topk_w[t,j] * yp[inv[t*k+j]]   (slots with inv >= 0, ascending j)
 * is computed by the workgroup that writes the last of token t's row blocks of
 * yp (integer arrival counters per token and 64-column block; no
 * floating-point atomics): y is bit-identical to moe_combine after
 * moe_grouped_ffn_fwd_gather, and every other output is bit-identical to that
 * call's.  Tokens with no kept slot get y[t] = 0.  yp is still written (the
 * combine reads it back, and the backward needs it).  x [T,d]; perm [R_cap],
 * inv [T*k] as written by moe_permute; topk_w [T,k] fp32; y [T,d]; the other
 * arguments as for moe_grouped_ffn_fwd.  ws: moe_workspace_size(
 * MOE_OP_FFN_FWD_FUSED) (the tile tables, kept slots per token [T], arrival
 * counters [T, d/64]).  Needs T*d and R_cap*d element bytes < 2^31 (else
 * MOE_ERR_UNSUPPORTED).  fp32 layers run the same steps with the combine
 * kernel after the GEMM. */
moe_status_t moe_grouped_ffn_fwd_fused(const moe_shape_t* shape, const void* x,
                                       const int32_t* perm, const int32_t* inv,
                                       const float* topk_w, const int32_t* group_offsets,
                                       const void* w_gate, const void* w_up, const void* w_down,
                                       void* h_save, void* a_save, void* yp, void* y, void* ws,
                                       size_t ws_bytes, moe_stream_t stream);

/* a5 -- combine (the second of the two token-movement kernels, [P3] section 加速来源, DeepEP item):
 * y[t] = sum_j topk_w[t,j] * yp[inv[t*k+j]] over the slots with inv >= 0, in
 * ascending j, fp32 accumulation; a token with no local slot gets y[t] = 0.
 * yp [R_cap,d]; inv [T*k]; topk_w [T,k] fp32; y [T,d].  No workspace. */
moe_status_t moe_combine(const moe_shape_t* shape, const void* yp, const int32_t* inv,
                         const float* topk_w, void* y, moe_stream_t stream);

/* a3 + a4 + a5 for a few tokens -- the batched_mm expert backend ([P3] section
 * 专家后端, backend table: the routed pairs multiply by their experts' weights
 * in batched products, for small inputs).  No sort and no grouped GEMM: the
 * workgroups of each active local expert find that expert's (token, slot)
 * pairs (local, first-occurrence slots e = topk_idx[t,j]) in the table
 * themselves and read its weights once per column block, and
 *   y[t] = sum_j topk_w[t,j] * (silu(x[t] Wg[e]) * (x[t] Wu[e])) Wd[e]
 * in ascending j with fp32 accumulation (A rounded to the dtype, as in
 * moe_grouped_ffn_fwd); tokens with no local slot get y[t] = 0.  The same
 * result as moe_permute + moe_grouped_ffn_fwd + moe_combine within rounding
 * (the sums run in another order).  x [T,d]; topk_idx, topk_w [T,k];
 * weights as for moe_grouped_ffn_fwd; y [T,d].  ws:
 * moe_workspace_size(MOE_OP_SMALL_FWD) (fp32 partial sums of [Hg | Hu] over
 * up to 8 ranges of d, the per-slot outputs, the combine's counters).  The
 * combine runs inside the second kernel (the workgroup that writes a token's
 * last pair row of a column block, by an integer arrival counter, sums the
 * token's pairs in ascending slot order: deterministic).  With no tile
 * padding and no sort it is the faster form while T*k is below about
 * E_loc / 2 (the layer's size rule).  Needs T*k <= 4096, d and I <= 8192
 * and no row capacity (R_cap 0 or T*k); else MOE_ERR_UNSUPPORTED.  Forward
 * only. */
moe_status_t moe_ffn_small_fwd(const moe_shape_t* shape, const void* x, const int32_t* topk_idx,
                               const float* topk_w, const void* w_gate, const void* w_up,
                               const void* w_down, void* y, void* ws, size_t ws_bytes,
                               moe_stream_t stream);

/* a1 + a3 + a4 + a5 for a few tokens, in one call: the gate, then
 * moe_ffn_small_fwd's FFN and combine.  Under the softmax top-k gate with
 * T*E <= 1024 and T*E*d/64 <= 8192 (one or two tokens at E = 128, d = 2048)
 * the router runs split over d (partial logits of 64-row chunks of d in
 * parallel workgroups) and every workgroup of the FFN's first kernel adds
 * them in chunk order, adds the bias, takes the top k by rank -- the same
 * selection and tie rule as moe_route -- and the softmax over the k slots
 * (one launch less; the sums run in another order than moe_route's, so
 * logits may differ from it in the last bits).  Otherwise moe_route's
 * kernels run (for T <= 16 its few-token logits), or, for T <= 16 with E *
 * element bytes not a multiple of 16, the split router with one workgroup
 * per token for the top k.  Outputs
 * logits (softmax gate), topk_idx, topk_w and y as moe_route and
 * moe_ffn_small_fwd would; the same arguments and limits.  ws:
 * moe_workspace_size(MOE_OP_SMALL_ROUTED_FWD). */
moe_status_t moe_small_fwd(const moe_shape_t* shape, const void* x, const void* w_router,
                           const float* bias, float* logits, int32_t* topk_idx, float* topk_w,
                           const void* w_gate, const void* w_up, const void* w_down, void* y,
                           void* ws, size_t ws_bytes, moe_stream_t stream);

/* ---------------------------------------------------------------- checks */

/* Device-side check of a routing table and its group offsets: the layer's
 * debug check.  The kernels take any expert id outside [e_lo, e_hi) for
 * another GPU's expert and drop its row, so an id outside [0, E) in a caller's
 * table would otherwise pass unnoticed.  ORs into *flags (one device int32;
 * bits are only ever set, so the caller zeroes it once and may run several
 * checks into it; read it once the stream has finished):
 *   MOE_CHECK_IDX_RANGE   some topk_idx[t,j] < 0 or >= E;
 *   MOE_CHECK_IDX_REPEAT  some token names one expert in two slots (allowed:
 *                         only the first of those slots is routed, as in
 *                         moe_permute);
 *   MOE_CHECK_OFFSETS     group_offsets (when not NULL) is not what
 *                         moe_permute writes for this table: the exclusive
 *                         prefix of the local experts' group sizes (rows under
 *                         the first-slot rule), each entry clamped to R_cap.
 * The order of the expert-sorted rows ([P3] section 专家后端, grouped_mm row)
 * is not checked here: perm and inv follow from the table by moe_permute.
 * topk_idx [T,k] int32; group_offsets [E_loc+1] int32 or NULL; flags [1]
 * int32.  ws: moe_workspace_size(MOE_OP_CHECK_ROUTING) (the group sizes,
 * E_loc int32), needed only with group_offsets.  Errors: MOE_ERR_ARG for a
 * NULL topk_idx or flags, MOE_ERR_WORKSPACE for a short workspace. */
#define MOE_CHECK_IDX_RANGE 1
#define MOE_CHECK_IDX_REPEAT 2
#define MOE_CHECK_OFFSETS 4
moe_status_t moe_check_routing(const moe_shape_t* shape, const int32_t* topk_idx,
                               const int32_t* group_offsets, int32_t* flags, void* ws,
                               size_t ws_bytes, moe_stream_t stream);

/* ------------------------------------------------------------ backward */
/* Full-parameter fine-tuning needs every gradient ([P3] Qwen3 and Nemotron
 * tables report the backward pass on its own row). */

/* a6 -- combine backward.  For every slot with p = inv[t*k+j] >= 0:
 * dyp[p] = topk_w[t,j] * dy[t];  dtopk_w[t,j] = <dy[t], yp[p]> (fp32);
 * slots with inv < 0 get dtopk_w = 0.  dy [T,d]; dyp [R_cap,d]; dtopk_w [T,k]. */
moe_status_t moe_combine_bwd(const moe_shape_t* shape, const void* dy, const void* yp,
                             const int32_t* inv, const float* topk_w, void* dyp,
                             float* dtopk_w, moe_stream_t stream);

/* a7..a10 -- expert FFN backward (grouped GEMMs).  Per local expert i, rows
 * [o_i, o_{i+1}):
 *   dA = dyp * w_down[i]^T;  s = sigmoid(Hg)
 *   dHg = dA * Hu * s * (1 + Hg (1 - s)),  dHu = dA * Hg * s
 *   dxp = dHg * w_gate[i]^T + dHu * w_up[i]^T
 *   dw_down[i] = A^T dyp,  dw_gate[i] = xp^T dHg,  dw_up[i] = xp^T dHu
 * Experts with no rows get dw = 0 exactly.  h_save/a_save are the buffers
 * moe_grouped_ffn_fwd filled.  dxp [R_cap,d]; dw_gate, dw_up [E_loc,d,I];
 * dw_down [E_loc,I,d].  ws: moe_workspace_size(MOE_OP_FFN_BWD) (it holds
 * [dHg | dHu]). */
moe_status_t moe_grouped_ffn_bwd(const moe_shape_t* shape, const void* xp,
                                 const int32_t* group_offsets, const void* w_gate,
                                 const void* w_up, const void* w_down, const void* h_save,
                                 const void* a_save, const void* dyp, void* dxp,
                                 void* dw_gate, void* dw_up, void* dw_down, void* ws,
                                 size_t ws_bytes, moe_stream_t stream);

/* a7..a10 with the Xp rows of the gate/up weight gradient read as
 * x[perm[p] / k] (the backward of moe_grouped_ffn_fwd_gather; no Xp buffer).
 * Bit-identical to moe_grouped_ffn_bwd on the Xp that moe_permute writes.
 * x [T,d]; perm [R_cap]; the rest as for moe_grouped_ffn_bwd.  Needs
 * T*d*element bytes < 2^31 (else MOE_ERR_UNSUPPORTED). */
moe_status_t moe_grouped_ffn_bwd_gather(const moe_shape_t* shape, const void* x,
                                        const int32_t* perm, const int32_t* group_offsets,
                                        const void* w_gate, const void* w_up,
                                        const void* w_down, const void* h_save,
                                        const void* a_save, const void* dyp, void* dxp,
                                        void* dw_gate, void* dw_up, void* dw_down, void* ws,
                                        size_t ws_bytes, moe_stream_t stream);

/* a6..a10 in one call: moe_combine_bwd followed by moe_grouped_ffn_bwd_gather,
 * with dyp written only where a kernel reads it.  Same outputs, to rounding:
 * in bf16, while every local expert has at most 256 rows, dyp is never
 * written and the a6 kernel does not run: the rows g * dy[t] of dyp
 * (g = topk_w[t,j], t*k + j = perm[p]) are formed inside the kernels -- dA's
 * rows scaled by g in fp32 after the product dA0 = dy[t] w_down^T, the rows
 * of A scaled by g and rounded to bf16 in dw_down = sum_p (g A[p])^T dy[t]
 * -- and dtopk_w[t,j] = <dA0[p], silu(Hg[p]) * Hu[p]> (fp32, from the saved
 * H), which is <dy[t], yp[p]> = <dy[t], A[p] w_down> up to rounding; with a
 * larger expert, and in fp32, a6 runs as moe_combine_bwd (dyp written, the
 * same dtopk_w) and a7..a10 as moe_grouped_ffn_bwd_gather on that dyp (the
 * same bits).  The choice is made on the device from group_offsets.  dyp
 * [R_cap,d] is caller-owned scratch whose contents afterwards are
 * unspecified.  Arguments as for moe_combine_bwd and
 * moe_grouped_ffn_bwd_gather; the workspace is moe_workspace_size(
 * MOE_OP_FFN_BWD) (in bf16 it also holds fp32 [R_cap][I/32] shares of the
 * gate gradient).  Needs T*d*element bytes < 2^31 (else
 * MOE_ERR_UNSUPPORTED). */
moe_status_t moe_combine_ffn_bwd_gather(const moe_shape_t* shape, const void* x,
                                        const int32_t* perm, const int32_t* inv,
                                        const int32_t* group_offsets, const float* topk_w,
                                        const void* w_gate, const void* w_up,
                                        const void* w_down, const void* h_save,
                                        const void* a_save, const void* yp, const void* dy,
                                        void* dyp, float* dtopk_w, void* dxp, void* dw_gate,
                                        void* dw_up, void* dw_down, void* ws, size_t ws_bytes,
                                        moe_stream_t stream);

/* a11 -- permute backward: dx[t] = sum_j dxp[inv[t*k+j]] over slots with
 * inv >= 0, ascending j, fp32 accumulation (tokens with no slot get 0).
 * dxp [R_cap,d]; dx [T,d] (overwritten). */
moe_status_t moe_permute_bwd(const moe_shape_t* shape, const void* dxp, const int32_t* inv,
                             void* dx, moe_stream_t stream);

/* a12 -- route backward.
 * softmax_topk: dlogits[t, idx[t,j]] = g_j (dg_j - sum_i g_i dg_i), every other
 *   entry 0; dw_router = x^T dlogits; dbias = sum_t dlogits (if non-NULL);
 *   dx += dlogits * w_router^T (read-modify-write of dx, which moe_permute_bwd
 *   wrote first).
 * balanced: the gate weights are constants: dlogits (if non-NULL), dw_router
 *   and dbias (if non-NULL) are set to 0 and dx is not touched.
 * x [T,d]; w_router [d,E]; topk_idx, topk_w, dtopk_w [T,k]; dlogits [T,E] fp32
 * (required for softmax_topk); dw_router [d,E] (dtype); dbias [E] fp32;
 * dx [T,d].  ws: moe_workspace_size(MOE_OP_ROUTE_BWD) (0 for balanced; it
 * holds the bf16 copy of dlogits, column sums of dlogits per 32 tokens and,
 * for bf16, fp32 partials of dw_router over token ranges; every sum runs in a
 * fixed order, so results are deterministic). */
moe_status_t moe_route_bwd(const moe_shape_t* shape, const void* x, const void* w_router,
                           const int32_t* topk_idx, const float* topk_w,
                           const float* dtopk_w, float* dlogits, void* dw_router,
                           float* dbias, void* dx, void* ws, size_t ws_bytes,
                           moe_stream_t stream);

/* Load-balancing auxiliary loss of the router (softmax_topk gate).  The pages
 * name an auxiliary loss that keeps the naturally uneven routing even during
 * fine-tuning (page "NVIDIA NeMo AutoModel MoE 微調的 3.7 倍加速突破", section
 * 延伸觀點; [P3] section 单节点30B MoE基准测试, routing-gate note: a trained
 * model's balancing loss drives expert utilisation toward uniform) without a
 * formula; this is the Switch Transformer balancing loss with the k slots of
 * a token counted as k dispatches:
 *   f_e  = c_e / (T*k), c_e = routed slots on expert e (all E experts, from
 *          topk_idx, whichever experts are local),
 *   P_e  = (1/T) sum_t softmax(logits[t,:])_e (full softmax over E, fp32),
 *   loss = alpha * E * sum_e f_e P_e.
 * logits [T,E] fp32 (as moe_route wrote them); topk_idx [T,k]; loss [1] fp32
 * (written); aux_w [E] fp32 (written): alpha*E*f_e/T, the weights
 * moe_route_bwd_aux needs.  Every sum runs in a fixed order (deterministic).
 * ws: moe_workspace_size(MOE_OP_AUX_LOSS) (per-32-token partial sums).
 * MOE_ERR_ARG for the balanced gate (it has no router probabilities) or a
 * non-finite alpha. */
moe_status_t moe_aux_loss(const moe_shape_t* shape, const float* logits, const int32_t* topk_idx,
                          float alpha, float* loss, float* aux_w, void* ws, size_t ws_bytes,
                          moe_stream_t stream);

/* moe_route_bwd with the auxiliary loss's gradient added to dlogits before
 * dw_router, dbias and dx are formed: the counts c_e are piecewise constant,
 * so the gradient flows through P only:
 *   dlogits[t,e] += p[t,e] (aux_w[e] - sum_e' aux_w[e'] p[t,e']),
 * p = softmax(logits[t,:]).  logits [T,E] fp32 and aux_w [E] fp32 (from
 * moe_aux_loss) are required; the other arguments, the workspace
 * (MOE_OP_ROUTE_BWD) and the errors are those of moe_route_bwd, plus
 * MOE_ERR_ARG for the balanced gate. */
moe_status_t moe_route_bwd_aux(const moe_shape_t* shape, const void* x, const void* w_router,
                               const int32_t* topk_idx, const float* topk_w,
                               const float* dtopk_w, const float* logits, const float* aux_w,
                               float* dlogits, void* dw_router, float* dbias, void* dx, void* ws,
                               size_t ws_bytes, moe_stream_t stream);

/* ---------------------------------------------------------- kernel timer */
/* Optional per-kernel timing with HIP events recorded on the launch stream
 * around each kernel of the calls above.  Off by default.  Host-side calls;
 * moe_prof_read waits for the recorded events.
 * moe_prof_read(name, ...): total milliseconds and launch count of the kernels
 * whose name equals `name` since the last reset; unknown names read 0.
 * moe_prof_names(): the names recorded so far, comma-separated (static buffer
 * valid until the next moe_prof_* call). */
moe_status_t moe_prof_enable(int on);
/* Record only the kernels named in `names` (comma-separated); NULL or "" records
 * every kernel.  Each recorded launch adds two event records to its stream. */
moe_status_t moe_prof_select(const char* names);
moe_status_t moe_prof_reset(void);
moe_status_t moe_prof_read(const char* name, double* total_ms, int64_t* launches);
const char* moe_prof_names(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
