// Grouped GEMM engine of the MoE layer: problem description shared by the
// bf16 MFMA kernels and the fp32 kernels (gemm.hip), and the launchers the
// C ABI (abi.hip) calls.
//
// Every GEMM of the layer is C[m][n] = sum_k A(m,k) * B(k,n) with
//   A(m,k) stored k-contiguous (a[m*lda + k])  -- A_KC
//             or m-contiguous (a[k*lda + m])  -- A_MC
//   B(k,n) stored n-contiguous (b[k*ldb + n])  -- B_NC
//             or k-contiguous (b[n*ldb + k])  -- B_KC
// and one of three groupings:
//   G_DENSE  one plain GEMM of M x N x K;
//   G_MROWS  expert groups along M: the rows of local expert e are
//            [off[e], off[e+1]) of A and C, and B is expert e's weight matrix
//            (forward and input-gradient GEMMs: the rows sorted by expert
//            and one grouped GEMM over the groups, page "Accelerating
//            Transformers fine-tuning with NVIDIA NeMo AutoModel", section
//            专家后端, grouped_mm row);
//   G_KROWS  expert groups along K: C for expert e sums over the rows
//            [off[e], off[e+1]) of A and B (weight gradients); an expert
//            with no rows gets C = 0.
#pragma once

#include "common.h"

namespace moe {

enum AMode { A_KC = 0, A_MC = 1 };
enum BMode { B_NC = 0, B_KC = 1 };
enum GMode { G_DENSE = 0, G_MROWS = 1, G_KROWS = 2 };
// B with two sources: none; tile columns split in halves (gate | up); K split.
enum B2Mode { B2_NONE = 0, B2_NHALF = 1, B2_KSPLIT = 2 };
enum EpiMode {
  EPI_STORE = 0,      // C0[m,n] = acc  (cols >= n_split go to C1[m, n-n_split] when n_split > 0)
  EPI_ACCUM = 1,      // C0[m,n] += acc
  EPI_F32_BIAS = 2,   // fp32 C0[m,n] = acc + bias[n]
  EPI_SWIGLU = 3,     // gate/up pair -> H = [Hg|Hu] (C0, optional), A = silu(Hg)*Hu (C2)
  EPI_DSWIGLU = 4     // acc = dA; with H from `aux`: dH = [dHg|dHu] into C0
};

struct GemmParams {
  const void* A;
  int64_t lda;
  const void* B0;
  const void* B1;
  int64_t ldb;
  int64_t b_estride;   // element stride between experts' B (G_MROWS)
  int M, N, K;         // G_DENSE: all; G_MROWS: N, K (M = row capacity); G_KROWS: M, N
  int k_split;         // B2_KSPLIT: k < k_split from B0, else B1 at k - k_split
  const int32_t* off;  // group offsets [groups+1] (G_MROWS, G_KROWS); NULL in G_KROWS: see k_chunk
  int k_chunk;         // G_KROWS without offsets: group g sums K rows [g*k_chunk, (g+1)*k_chunk)
                       // (a split of K into partial results); 0 = one group [0, K)
  int k_strip;         // G_KROWS with offsets and kcost: nonzero when the strip kernel ran
                       // first; the tile kernels then neither read nor write the experts of
                       // zero K cost (the strip kernel's)
  int col_parts;       // strip kernel: parts (of whole column tiles) a row block is split in
  // R_DOWN_DGRAD_GATHER and the strip kernel's dY form: the gate weight of
  // routed row p is row_gate[row_slot[p]] (row_slot = perm: t*k + j)
  const float* row_gate;
  const int32_t* row_slot;
  // R_DOWN_DGRAD_GATHER: the materialised dYp.  When the tile-table launch
  // gave the weight gradients' tile kernels any expert (kcost[groups] > 0),
  // the combine backward has written it and the kernel reads its rows in
  // order, with no gate weight; else A = dY through a_rows, scaled by row_gate.
  const void* a_alt;
  // R_DOWN_DGRAD_GATHER reading dY (not a_alt): the gate gradient's shares,
  // dg_part[p * dg_stride + b] = sum over the 32 columns i of block b of
  // dA0[p,i] * silu(Hg[p,i]) Hu[p,i], with dA0 = dY[t] Wd^T before the gate
  // weight (so that dG = <dY[t], A Wd> = sum_b dg_part[p, b]); NULL: none
  float* dg_part;
  int dg_stride;       // I / 32
  const int32_t* tiles;// G_MROWS tile table: tiles[0] = count, then (expert, first row) pairs
  const int32_t* kcost;// G_KROWS (optional): prefix sums [groups+1] of the per-expert tile cost
                       // (K slices + a fixed part), for balancing the persistent kernels; all
                       // zero when every expert fits the strip kernel (R_DOWN_DGRAD_GATHER
                       // reads kcost[groups] to pick its A source)
  int groups;          // number of local experts
  int m_tiles, n_tiles;
  void* C0;
  void* C1;
  void* C2;
  int64_t ldc;
  int64_t c_estride;   // element stride between experts' C (G_KROWS)
  int n_split;         // EPI_STORE: columns >= n_split go to C1
  int I;               // EPI_SWIGLU / EPI_DSWIGLU: expert width (H row stride is 2I)
  const void* aux;     // EPI_DSWIGLU: saved H
  const float* bias;   // EPI_F32_BIAS (may be NULL)
  const int32_t* a_rows;  // gather roles: A row p (the M index for G_MROWS, the K index for
  int a_rows_div;         // G_KROWS) is row a_rows[p] / a_rows_div of the matrix at A (the
                          // bf16 kernels take a table of rows: a_rows_div must be 1)
  // R_DOWN_FWD_COMBINE: the combine y[t] = sum_j w[t,j] C0[inv[t*k+j]] run by the
  // workgroup that writes a token's last row block (see CombinePrep)
  const int32_t* cmb_tok;   // token of every routed row [R_cap]
  const int32_t* cmb_inv;   // [T*k]
  const float* cmb_w;       // gate weights [T*k]
  const int32_t* cmb_kept;  // kept slots per token [T]
  int32_t* cmb_cnt;         // arrival counters [T][N/64], zero on entry
  void* cmb_y;              // [T][N]
  int cmb_k;
};

// Preparation of the fused combine, done by the tile-table launch before the
// FFN's GEMMs: kept[t] = slots of token t with inv >= 0, the token's arrival
// counters zeroed, and y[t] = 0 for a token with no kept slot (no row block of
// it is ever written, so no workgroup would write it).
struct CombinePrep {
  const int32_t* inv;
  int T, k;
  int32_t* kept;
  int32_t* cnt;
  int ncb;          // counters per token (N / 64)
  void* y;
  int y_row_bytes;  // N * element bytes (a multiple of 16)
};

// Tile shapes of the bf16 MFMA kernels.
enum TileCfg { TILE_256x256 = 0, TILE_256x128 = 1, TILE_64x64 = 2, TILE_128x128 = 3, TILE_128x256 = 4 };

// The GEMMs of the layer.  Each role fixes the operand layouts, the grouping
// and the epilogue, and is its own kernel instance (so profilers tell them apart).
enum GemmRole {
  R_ROUTE_LOGITS = 0,   // logits = x Wr (+ b)
  R_GATEUP_FWD = 1,     // [Hg | Hu] = Xp [Wg | Wu], A = silu(Hg) Hu
  R_DOWN_FWD = 2,       // Yp = A Wd
  R_DOWN_DGRAD = 3,     // dA = dYp Wd^T, then dSwiGLU -> [dHg | dHu]
  R_GATEUP_DGRAD = 4,   // dXp = dHg Wg^T + dHu Wu^T
  R_DOWN_WGRAD = 5,     // dWd = A^T dYp
  R_GATEUP_WGRAD = 6,   // [dWg | dWu] = Xp^T [dHg | dHu]
  R_ROUTE_DW = 7,       // dWr = x^T dL
  R_ROUTE_DX = 8,       // dX += dL Wr^T
  // R_GATEUP_FWD and R_GATEUP_WGRAD with the rows of Xp read from x through
  // perm (Xp is never written): a_rows = perm, a_rows_div = k
  R_GATEUP_FWD_GATHER = 9,
  R_GATEUP_WGRAD_GATHER = 10,
  // R_DOWN_FWD with the combine in its epilogue (dispatch's counterpart, the
  // combine, fused into the expert GEMM)
  R_DOWN_FWD_COMBINE = 11,
  // R_DOWN_DGRAD on the rows g * dY[t] of dYp formed in the kernel: dY read
  // through the token table (a_rows), the accumulator rows scaled by g in the
  // epilogue; or on dYp itself (a_alt), as the device decides (bf16 only)
  R_DOWN_DGRAD_GATHER = 12
};

// Tile shape each role runs with (bf16), for a GEMM with n output columns
// (n = 0: the role's usual shape).
TileCfg role_tile(GemmRole role, int n = 0);
int tile_bm(TileCfg cfg);
int tile_bn(TileCfg cfg);
const char* role_name(GemmRole role);

// Launch one GEMM: the bf16 MFMA kernel of the role, or the fp32 kernel.  For
// G_MROWS the caller has built the tile table (launch_tile_tables) for
// tile_bm(role_tile(role)); max_m_tiles bounds its entries (fp32: the row count).
moe_status_t launch_gemm(bool is_bf16, GemmRole role, const GemmParams& p, int max_m_tiles,
                         hipStream_t s);

// The down projection's weight gradient with dYp never written (bf16):
// dWd = sum_p (g_p A[p])^T dY[tok[p]].  The strip kernel reads dY through the
// token table (p.a_rows) and scales its A fragments by the gate weights
// (p.row_gate / p.row_slot); when the device gave the tile kernels any expert
// (one has more than STRIP_K rows), they run R_DOWN_WGRAD on `dyp`, which
// the combine backward has then written.  p: R_DOWN_WGRAD's parameters with
// B0 = dY.
moe_status_t launch_down_wgrad_dy(const GemmParams& p, const void* dyp, int max_m_tiles,
                                  hipStream_t s);

// Tile tables for G_MROWS, for 256-row and for 128-row tiles (one launch):
// tiles[0] = number of M tiles, then for each tile (expert, first row) in
// expert order; and the K-cost prefix of the weight gradients (kcost above).
// With perm, the same launch also writes the token row of every routed row,
// tok[p] = perm[p] / k for p < off[groups] (the A rows of the gather roles).
moe_status_t launch_tile_tables(const int32_t* off, int groups, int32_t* tiles256,
                                int32_t* tiles128, int32_t* kcost, hipStream_t s,
                                const int32_t* perm = nullptr, int k = 1, int32_t* tok = nullptr,
                                int rows_cap = 0, const CombinePrep* cmb = nullptr);
// Per-tile cost of a weight-gradient tile beyond its K slices (its epilogue).
constexpr int KCOST_FIXED = 2;
// When every expert has at most STRIP_K rows, the weight gradients run in the
// strip kernel (gemm.hip), whose workgroups hold all of an expert's K rows:
// the tile-table launch then gives every expert zero K cost, and the tile
// kernels leave them all out.  With a larger expert the tile kernels run
// every expert (two kernels splitting the experts ran slower, one after the
// other).  Build-time tunable: 0 turns the strip kernel off.
#ifndef MOE_STRIP_K
#define MOE_STRIP_K 256
#endif
constexpr int STRIP_K = MOE_STRIP_K;

}  // namespace moe
