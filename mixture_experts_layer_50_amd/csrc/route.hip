// Gate kernels of the MoE layer: balanced gate, wavefront top-k + softmax,
// and the router backward (softmax Jacobian, bias column sums).
//
// Routing tokens over many experts is the first problem the page "Accelerating
// Transformers fine-tuning with NVIDIA NeMo AutoModel" lists (section 背景);
// its balanced gate (section 单节点30B MoE基准测试, routing-gate note) forces
// tokens evenly over the experts.  The gate function itself is not on the
// pages: top-k by logit (ties toward the lower expert id) with softmax over
// the k selected logits.
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------- balanced
__global__ void balanced_gate_kernel(int T, int E, int k, int32_t* idx, float* w) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * k) return;
  int t = (int)(i / k), j = (int)(i - (int64_t)t * k);
  int P = E / k;
  idx[i] = (t % P) + j * P;
  w[i] = 1.0f / (float)k;
}

moe_status_t launch_balanced_gate(int T, int E, int k, int32_t* idx, float* w, hipStream_t s) {
  ProfScope prof("route_balanced", s);
  int64_t n = (int64_t)T * k;
  balanced_gate_kernel<<<(unsigned)ceil_div(n, 256), 256, 0, s>>>(T, E, k, idx, w);
  return check_launch("balanced_gate_kernel");
}

// Balanced gate and the expert sort in one kernel.  Expert e = (t mod P) +
// j*P (P = E/k) receives the tokens t = e mod P + m*P, m = 0, 1, ..., in
// token order, so a row's sorted position has a closed form: the rows of the
// local experts before e, plus m = t div P.  With c(r) = the number of tokens
// t < T with t mod P = r, the rows of experts [0, n) number
//   F(n) = (n div P) T + (T div P) (n mod P) + min(T mod P, n mod P),
// and local expert e starts at F(e) - F(e_lo).  Positions >= R_cap are
// dropped (inv = -1), as in the sort.
__device__ __forceinline__ int64_t balanced_rows_before(int64_t n, int T, int P) {
  const int64_t q = n / P, r = n % P;
  return q * T + (int64_t)(T / P) * r + min((int64_t)(T % P), r);
}

__global__ void balanced_route_permute_kernel(int T, int E, int k, int e_lo, int e_hi, int R_cap,
                                              int32_t* idx, float* w, int32_t* offsets,
                                              int32_t* perm, int32_t* inv) {
  const int P = E / k;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t base = balanced_rows_before(e_lo, T, P);
  if (i <= e_hi - e_lo)  // group offsets of the local experts
    offsets[i] = (int32_t)min(balanced_rows_before(e_lo + i, T, P) - base, (int64_t)R_cap);
  if (i >= (int64_t)T * k) return;
  const int t = (int)(i / k), j = (int)(i - (int64_t)t * k);
  const int e = (t % P) + j * P;
  idx[i] = e;
  w[i] = 1.0f / (float)k;
  int pos = -1;
  if (e >= e_lo && e < e_hi) {
    const int64_t p = balanced_rows_before(e, T, P) - base + t / P;
    if (p < R_cap) {
      pos = (int)p;
      perm[pos] = (int32_t)i;
    }
  }
  inv[i] = pos;
}

moe_status_t launch_balanced_route_permute(int T, int E, int k, int e_lo, int e_hi, int R_cap,
                                           int32_t* idx, float* w, int32_t* offsets,
                                           int32_t* perm, int32_t* inv, hipStream_t s) {
  ProfScope prof("route_permute_balanced", s);
  const int64_t n = std::max<int64_t>((int64_t)T * k, e_hi - e_lo + 1);
  balanced_route_permute_kernel<<<(unsigned)ceil_div(n, 256), 256, 0, s>>>(
      T, E, k, e_lo, e_hi, R_cap, idx, w, offsets, perm, inv);
  return check_launch("balanced_route_permute_kernel");
}

// ---------------------------------------------------------------- top-k
// One wavefront per token.  Lane l holds the logits of experts l + 64 v.
// k rounds: every lane proposes its best untaken expert, a butterfly over the
// wavefront keeps the larger logit (the lower id on equal logits), the owner
// marks it taken.  Lane j keeps the j-th winner; softmax over lanes < k.
__device__ __forceinline__ bool better(float v, int id, float bv, int bid) {
  return v > bv || (v == bv && id < bid);
}

// Top-k and softmax of one token's logits, held by one wavefront (lane l:
// experts l + 64 q in v[q], -inf past E); writes the token's k slots.
template <int VPL>
__device__ __forceinline__ void topk_softmax_wave(const float (&v)[VPL], int E, int k, int lane,
                                                  int32_t* idx_t, float* w_t) {
  bool taken[VPL];
#pragma unroll
  for (int q = 0; q < VPL; ++q) taken[q] = lane + 64 * q >= E;
  float my_v = -INFINITY;
  int my_id = 0x7fffffff;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bid = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
      int e = lane + 64 * q;
      if (!taken[q] && better(v[q], e, bv, bid)) { bv = v[q]; bid = e; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      float ov = __shfl_xor(bv, off, 64);
      int oid = __shfl_xor(bid, off, 64);
      if (better(ov, oid, bv, bid)) { bv = ov; bid = oid; }
    }
#pragma unroll
    for (int q = 0; q < VPL; ++q)
      if (lane + 64 * q == bid) taken[q] = true;
    if (lane == j) { my_v = bv; my_id = bid; }
  }
  const float vmax = __shfl(my_v, 0, 64);
  float z = lane < k ? expf(my_v - vmax) : 0.f;
  float sum = z;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if (lane < k) {
    idx_t[lane] = my_id;
    w_t[lane] = z / sum;
  }
}

template <int VPL>
__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* logits, int T, int E, int k,
                                                           int32_t* idx, float* w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (int64_t)t * E;
  float v[VPL];
#pragma unroll
  for (int q = 0; q < VPL; ++q) {
    int e = lane + 64 * q;
    v[q] = e < E ? row[e] : -INFINITY;
  }
  topk_softmax_wave<VPL>(v, E, k, lane, idx + (int64_t)t * k, w + (int64_t)t * k);
}

// ---------------------------------------------------------------- few tokens
// The router for a few tokens, split over K: workgroup s computes the partial
// logits of every token over rows [s*64, s*64 + 64) of d into part[s][t][e];
// then one workgroup per token adds the d/64 partials in split order, adds
// the bias, writes the logits and runs the top-k and softmax.  With a few
// tokens the MFMA router's two column tiles each walk all of d on one CU;
// here d/64 workgroups share the router weights.  (The sums run in another
// order than the MFMA router's, so the logits may differ from it in the last
// bits.)
//
// In a workgroup, G = 256 / (columns per pass) row groups split the 64 rows:
// thread (g, e) loads its 64/G weights of column e before using any, then
// the G group sums are added in group order through LDS.
template <typename ELT, int G>
__global__ __launch_bounds__(256) void small_router_part_kernel(const ELT* x, const ELT* wr, int T,
                                                                int d, int E, float* part) {
  constexpr int KC = SMALL_ROUTE_KC, RPG = KC / G, EW = 256 / G, MT = SMALL_ROUTE_MAX_T;
  __shared__ float sx[MT * KC];
  __shared__ float red[G > 1 ? G * MT * EW : 1];
  const int s = blockIdx.x, k0 = s * KC;
  const int g = threadIdx.x / EW, el = threadIdx.x % EW, r0 = g * RPG;
  // weight loads unconditional (a clamped column past E, its sums never
  // stored), all RPG in flight together; the first pass's go out before x
  // is staged
  float wv[RPG];
  {
    const ELT* wc = wr + (int64_t)(k0 + r0) * E + min(el, E - 1);
#pragma unroll
    for (int r = 0; r < RPG; ++r) wv[r] = Elt<ELT>::load(wc + (int64_t)r * E);
  }
  for (int i = threadIdx.x; i < T * KC; i += 256)
    sx[i] = Elt<ELT>::load(x + (int64_t)(i / KC) * d + k0 + i % KC);
  __syncthreads();
  for (int e0 = 0; e0 < E; e0 += EW) {
    const int e = e0 + el;
    if (e0 > 0) {
      const ELT* wc = wr + (int64_t)(k0 + r0) * E + min(e, E - 1);
#pragma unroll
      for (int r = 0; r < RPG; ++r) wv[r] = Elt<ELT>::load(wc + (int64_t)r * E);
    }
    float acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      acc[t] = 0.f;
      if (t < T)
#pragma unroll
        for (int r = 0; r < RPG; ++r) acc[t] = fmaf(sx[t * KC + r0 + r], wv[r], acc[t]);
    }
    if constexpr (G == 1) {
      if (e < E)
#pragma unroll
        for (int t = 0; t < MT; ++t)
          if (t < T) part[((int64_t)s * T + t) * E + e] = acc[t];
    } else {
#pragma unroll
      for (int t = 0; t < MT; ++t)
        if (t < T) red[(g * MT + t) * EW + el] = acc[t];
      __syncthreads();
      for (int i = threadIdx.x; i < T * EW; i += 256) {
        const int t = i / EW, ec = i % EW;
        if (e0 + ec >= E) continue;
        float v = 0.f;
#pragma unroll
        for (int gg = 0; gg < G; ++gg) v += red[(gg * MT + t) * EW + ec];
        part[((int64_t)s * T + t) * E + e0 + ec] = v;
      }
      __syncthreads();
    }
  }
}

// One workgroup per token: the logits (partials added in split order, then
// the bias), then the top k by rank -- value e's slot is the number of
// values that come before it (a larger logit, or an equal one with a lower
// id), so slots run in the order of the wavefront top-k above with no chain
// of cross-lane steps -- and the softmax over the k slots in slot order.
__global__ __launch_bounds__(256) void small_router_final_kernel(const float* part, int nsplit,
                                                                 const float* bias, int T, int E,
                                                                 int k, float* logits, int32_t* idx,
                                                                 float* w) {
  constexpr int SB = 32;  // split partials in flight per thread
  __shared__ __align__(16) float sl[512];
  __shared__ float sv[512];
  __shared__ int sid[512];
  const int t = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 256) {
    float a = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += SB) {
      // unconditional loads (a clamped split past the last, never added)
      float pv[SB];
#pragma unroll
      for (int j = 0; j < SB; ++j) pv[j] = part[((int64_t)min(s0 + j, nsplit - 1) * T + t) * E + e];
#pragma unroll
      for (int j = 0; j < SB; ++j)
        if (s0 + j < nsplit) a += pv[j];
    }
    if (bias) a += bias[e];
    logits[(int64_t)t * E + e] = a;
    sl[e] = a;
  }
  const int E4 = (E + 3) & ~3;  // the row padded to whole float4s with -inf
  if (threadIdx.x < E4 - E) sl[E + threadIdx.x] = -INFINITY;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    const float v = sl[e];
    int rank = 0;
#pragma unroll 8
    for (int o = 0; o < E4; o += 4) {
      const float4 u = *reinterpret_cast<const float4*>(sl + o);
      rank += (u.x > v || (u.x == v && o < e)) + (u.y > v || (u.y == v && o + 1 < e)) +
              (u.z > v || (u.z == v && o + 2 < e)) + (u.w > v || (u.w == v && o + 3 < e));
    }
    if (rank < k) {
      sv[rank] = v;
      sid[rank] = e;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const float vmax = sv[0];
    float sum = 0.f;
    for (int j = 0; j < k; ++j) sum += expf(sv[j] - vmax);
    for (int j = 0; j < k; ++j) {
      idx[(int64_t)t * k + j] = sid[j];
      w[(int64_t)t * k + j] = expf(sv[j] - vmax) / sum;
    }
  }
}

int64_t small_router_ws_bytes(int T, int d, int E) {
  return round_up((int64_t)(d / SMALL_ROUTE_KC) * T * E * 4, 256);
}

moe_status_t launch_small_router_part(const void* x, const void* wr, int T, int d, int E,
                                      int elt_bytes, float* part, hipStream_t s) {
  const int nsplit = d / SMALL_ROUTE_KC;
  {
    ProfScope prof("small_route_part", s);
    // row groups: as many as leave one pass of at least E columns
    const int G = E <= 8 ? 32 : E <= 16 ? 16 : E <= 32 ? 8 : E <= 64 ? 4 : E <= 128 ? 2 : 1;
#define L_(E_, G_)                                                                 \
  small_router_part_kernel<E_, G_><<<nsplit, 256, 0, s>>>(static_cast<const E_*>(x), \
                                                          static_cast<const E_*>(wr), T, d, E, part)
#define LG_(E_)                  \
  switch (G) {                   \
    case 32: L_(E_, 32); break;  \
    case 16: L_(E_, 16); break;  \
    case 8: L_(E_, 8); break;    \
    case 4: L_(E_, 4); break;    \
    case 2: L_(E_, 2); break;    \
    default: L_(E_, 1); break;   \
  }
    if (elt_bytes == 2) { LG_(bf16_t) } else { LG_(float) }
#undef LG_
#undef L_
    return check_launch("small_router_part_kernel");
  }
}

moe_status_t launch_small_router(const void* x, const void* wr, const float* bias, int T, int d,
                                 int E, int k, int elt_bytes, float* logits, int32_t* idx,
                                 float* w, float* part, hipStream_t s) {
  const int nsplit = d / SMALL_ROUTE_KC;
  const moe_status_t st = launch_small_router_part(x, wr, T, d, E, elt_bytes, part, s);
  if (st != MOE_OK) return st;
  ProfScope prof("small_route_topk", s);
  small_router_final_kernel<<<T, 256, 0, s>>>(part, nsplit, bias, T, E, k, logits, idx, w);
  return check_launch("small_router_final_kernel");
}

// moe_route's logits for a few tokens (T <= SMALL_ROUTE_MAX_T), with no
// workspace: the MFMA router's two column tiles would each walk all of d on
// one CU, one K slice after another.  Here one workgroup per (16-byte chunk
// of a router row: N experts, group of up to MT tokens) walks all of d: lane
// l of wave w takes 8 consecutive rows of each 2048-row pass, all its weight
// and x loads of a pass in flight together, and accumulates them in row
// order; the lanes' sums are added by a butterfly, then the four waves' in
// wave order, then the bias: deterministic (another order than the MFMA
// router's, so the logits may differ from it in the last bits).  Needs
// E % N == 0 (16-byte row chunks).  MT: at most 4 tokens a workgroup (the
// butterfly's work grows with MT * N).
template <typename ELT, int MT>
__global__ __launch_bounds__(256) void few_token_logits_kernel(const ELT* x, const ELT* wr,
                                                               const float* bias, int T, int d,
                                                               int E, float* logits) {
  constexpr int N = 16 / sizeof(ELT);  // experts of the workgroup
  constexpr int RP = 8;                // rows of d per lane and pass
  __shared__ float red[4][MT][N];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e0 = blockIdx.x * N, t0 = blockIdx.y * MT;
  x += (int64_t)t0 * d;
  logits += (int64_t)t0 * E;
  T = min(T - t0, MT);  // tokens of this workgroup
  float acc[MT][N];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int n = 0; n < N; ++n) acc[t][n] = 0.f;
  for (int r0 = threadIdx.x * RP; r0 < d; r0 += 256 * RP) {
    uint4 wq[RP];
#pragma unroll
    for (int i = 0; i < RP; ++i)
      wq[i] = *reinterpret_cast<const uint4*>(wr + (int64_t)(r0 + i) * E + e0);
    uint4 xq[MT][RP / (16 / sizeof(ELT))];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int v = 0; v < RP / N; ++v)
        xq[t][v] = *reinterpret_cast<const uint4*>(x + (int64_t)min(t, T - 1) * d + r0 + v * N);
#pragma unroll
    for (int i = 0; i < RP; ++i) {
      float wv[N];
      if constexpr (sizeof(ELT) == 2) {
        const uint32_t q[4] = {wq[i].x, wq[i].y, wq[i].z, wq[i].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          wv[2 * h] = __uint_as_float(q[h] << 16);
          wv[2 * h + 1] = __uint_as_float(q[h] & 0xffff0000u);
        }
      } else {
        wv[0] = __uint_as_float(wq[i].x); wv[1] = __uint_as_float(wq[i].y);
        wv[2] = __uint_as_float(wq[i].z); wv[3] = __uint_as_float(wq[i].w);
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const uint4 xv = xq[t][i / N];
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
        float xf;
        if constexpr (sizeof(ELT) == 2) {
          const uint32_t u = xw[(i % N) / 2];
          xf = __uint_as_float((i % 2) ? (u & 0xffff0000u) : (u << 16));
        } else {
          xf = __uint_as_float(xw[i % N]);
        }
#pragma unroll
        for (int n = 0; n < N; ++n) acc[t][n] = fmaf(xf, wv[n], acc[t][n]);
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int n = 0; n < N; ++n) acc[t][n] += __shfl_xor(acc[t][n], off, 64);
  if (lane == 0)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int n = 0; n < N; ++n) red[w][t][n] = acc[t][n];
  __syncthreads();
  if (threadIdx.x < T * N) {
    const int t = threadIdx.x / N, n = threadIdx.x % N;
    float v = red[0][t][n];
    v += red[1][t][n];
    v += red[2][t][n];
    v += red[3][t][n];
    if (bias) v += bias[e0 + n];
    logits[(int64_t)t * E + e0 + n] = v;
  }
}

bool few_token_logits_fit(int T, int E, int elt_bytes) {
  return T >= 1 && T <= SMALL_ROUTE_MAX_T && E % (16 / elt_bytes) == 0;
}

moe_status_t launch_few_token_logits(const void* x, const void* wr, const float* bias, int T,
                                     int d, int E, int elt_bytes, float* logits, hipStream_t s) {
  ProfScope prof("route_logits", s);
  const int mt = T <= 1 ? 1 : T <= 2 ? 2 : 4;
  const dim3 grid((unsigned)(E / (16 / elt_bytes)), (unsigned)ceil_div(T, mt));
#define L_(E_, MT_)                                                                       \
  few_token_logits_kernel<E_, MT_><<<grid, 256, 0, s>>>(static_cast<const E_*>(x),        \
                                                        static_cast<const E_*>(wr), bias, T, d, \
                                                        E, logits)
#define LM_(E_)                                   \
  if (mt == 1) L_(E_, 1);                         \
  else if (mt == 2) L_(E_, 2);                    \
  else L_(E_, 4);
  if (elt_bytes == 2) { LM_(bf16_t) } else { LM_(float) }
#undef LM_
#undef L_
  return check_launch("few_token_logits_kernel");
}

moe_status_t launch_topk_softmax(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                                 hipStream_t s) {
  ProfScope prof("route_topk", s);
  unsigned grid = (unsigned)ceil_div(T, 4);
  if (E <= 64) topk_softmax_kernel<1><<<grid, 256, 0, s>>>(logits, T, E, k, idx, w);
  else if (E <= 128) topk_softmax_kernel<2><<<grid, 256, 0, s>>>(logits, T, E, k, idx, w);
  else if (E <= 256) topk_softmax_kernel<4><<<grid, 256, 0, s>>>(logits, T, E, k, idx, w);
  else topk_softmax_kernel<8><<<grid, 256, 0, s>>>(logits, T, E, k, idx, w);
  return check_launch("topk_softmax_kernel");
}

// ---------------------------------------------------------------- backward
// dL[t, idx[t,j]] = g_j (dg_j - sum_i g_i dg_i); all other logits get 0.
// One workgroup per 64 tokens, one wavefront per 16 of them in token order;
// lane l owns experts l + 64 q.  The optional bf16 copy feeds the bf16
// router-gradient GEMMs.  Each workgroup also writes its column sums of dL
// (tokens in order, then its four waves in order) to db_part[block][E].
//
// AUX adds the gradient of the load-balancing auxiliary loss:
// dL[t, e] += p[t, e] (w[e] - sum_e' w[e'] p[t, e']), p = softmax of the
// token's full logit row (fp32, max subtracted), w = aux_w.
template <int VPL, bool AUX>
__global__ __launch_bounds__(256) void route_bwd_dl_kernel(const int32_t* idx, const float* g,
                                                           const float* dg, int T, int E, int k,
                                                           float* dl, bf16_t* dl_bf16,
                                                           float* db_part, const float* logits,
                                                           const float* aux_w) {
  __shared__ float part[4][64 * VPL];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int TPW = ROUTE_BWD_TOKENS / 4;  // tokens per wave
  const int t0 = blockIdx.x * ROUTE_BWD_TOKENS + wave * TPW;
  float aw[VPL];
#pragma unroll
  for (int q = 0; q < VPL; ++q) aw[q] = AUX && q * 64 + lane < E ? aux_w[q * 64 + lane] : 0.f;
  // every token's slot data first (the loads in flight together)
  float gq[TPW], dgq[TPW];
  int iq[TPW];
  float lq[AUX ? TPW : 1][VPL];  // AUX: the tokens' logit rows
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const bool ok = t0 + i < T && lane < k;
    const int64_t o = (int64_t)(t0 + i) * k + lane;
    gq[i] = ok ? g[o] : 0.f;
    dgq[i] = ok ? dg[o] : 0.f;
    iq[i] = ok ? idx[o] : -1;
    if constexpr (AUX) {
#pragma unroll
      for (int q = 0; q < VPL; ++q)
        lq[i][q] = t0 + i < T && q * 64 + lane < E ? logits[(int64_t)(t0 + i) * E + q * 64 + lane]
                                                   : -INFINITY;
    }
  }
  float col[VPL];
#pragma unroll
  for (int q = 0; q < VPL; ++q) col[q] = 0.f;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int t = t0 + i;
    if (t >= T) break;  // uniform per wave
    const float gj = gq[i], dgj = dgq[i];
    const int ij = iq[i];
    float sum = gj * dgj;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
    const float val = gj * (dgj - sum);
    float pa[VPL], pdot = 0.f;  // AUX: the token's probabilities and sum_e w_e p_e
    if constexpr (AUX) {
      float m = -INFINITY;
      const float* lv = lq[i];
#pragma unroll
      for (int q = 0; q < VPL; ++q) m = fmaxf(m, lv[q]);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
      float z = 0.f;
#pragma unroll
      for (int q = 0; q < VPL; ++q) {
        pa[q] = q * 64 + lane < E ? expf(lv[q] - m) : 0.f;
        z += pa[q];
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off, 64);
#pragma unroll
      for (int q = 0; q < VPL; ++q) {
        pa[q] = pa[q] / z;
        pdot += aw[q] * pa[q];
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) pdot += __shfl_xor(pdot, off, 64);
    }
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
      const int e = q * 64 + lane;
      float out = 0.f;
      for (int j = 0; j < k; ++j) {
        const int ej = __shfl(ij, j, 64);
        const float vj = __shfl(val, j, 64);
        if (ej == e) out = vj;
      }
      if constexpr (AUX) out += pa[q] * (aw[q] - pdot);
      if (e < E) {
        dl[(int64_t)t * E + e] = out;
        if (dl_bf16) dl_bf16[(int64_t)t * E + e] = f2bf(out);
        col[q] += out;
      }
    }
  }
#pragma unroll
  for (int q = 0; q < VPL; ++q) part[wave][q * 64 + lane] = col[q];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    db_part[(int64_t)blockIdx.x * E + e] = ((part[0][e] + part[1][e]) + part[2][e]) + part[3][e];
}

template <bool AUX>
static void route_bwd_dl_launch(const int32_t* idx, const float* g, const float* dg, int T, int E,
                                int k, float* dl, bf16_t* dl_bf16, float* db_part,
                                const float* logits, const float* aux_w, hipStream_t s) {
  const unsigned grid = (unsigned)ceil_div(T, ROUTE_BWD_TOKENS);
#define L_(V) route_bwd_dl_kernel<V, AUX><<<grid, 256, 0, s>>>(idx, g, dg, T, E, k, dl, dl_bf16, db_part, logits, aux_w)
  if (E <= 64) L_(1);
  else if (E <= 128) L_(2);
  else if (E <= 256) L_(4);
  else L_(8);
#undef L_
}

moe_status_t launch_route_bwd_dl(const int32_t* idx, const float* g, const float* dg, int T, int E,
                                 int k, float* dl, bf16_t* dl_bf16, float* db_part,
                                 const float* logits, const float* aux_w, hipStream_t s) {
  ProfScope prof(aux_w ? "route_bwd_dlogits_aux" : "route_bwd_dlogits", s);
  if (aux_w) route_bwd_dl_launch<true>(idx, g, dg, T, E, k, dl, dl_bf16, db_part, logits, aux_w, s);
  else route_bwd_dl_launch<false>(idx, g, dg, T, E, k, dl, dl_bf16, db_part, nullptr, nullptr, s);
  return check_launch("route_bwd_dl_kernel");
}

// ---------------------------------------------------------------- aux loss
// Load-balancing auxiliary loss, loss = alpha E sum_e f_e P_e with
// f_e = c_e / (T k) (routed rows on expert e) and P_e = mean_t softmax(L[t,:])_e
// (the Switch Transformer balancing loss; the pages name an auxiliary
// balancing loss without its formula).  Pass 1: one workgroup per
// ROUTE_BWD_TOKENS tokens, one wavefront per quarter of them in token order,
// lane l owns experts l + 64 q; writes the block's column sums of p and its
// expert counts (waves added in a fixed order).  Pass 2, one workgroup: per
// expert the block partials in block order, then the loss over the experts in
// order.  fp32 throughout.
template <int VPL>
__global__ __launch_bounds__(256) void aux_loss_part_kernel(const float* logits, const int32_t* idx,
                                                            int T, int E, int k, float* pp_part,
                                                            int32_t* cnt_part) {
  __shared__ float pp[4][64 * VPL];
  __shared__ int cn[64 * VPL];  // the block's expert counts (integer adds: order-free)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int TPW = ROUTE_BWD_TOKENS / 4;
  const int t0 = blockIdx.x * ROUTE_BWD_TOKENS + wave * TPW;
  for (int e = threadIdx.x; e < 64 * VPL; e += blockDim.x) cn[e] = 0;
  __syncthreads();
  // every token's logit row and slots first (the loads in flight together)
  float lv[TPW][VPL];
  int iq[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
#pragma unroll
    for (int q = 0; q < VPL; ++q)
      lv[i][q] = t0 + i < T && q * 64 + lane < E ? logits[(int64_t)(t0 + i) * E + q * 64 + lane]
                                                 : -INFINITY;
    iq[i] = t0 + i < T && lane < k ? idx[(int64_t)(t0 + i) * k + lane] : -1;
  }
  float col[VPL];
#pragma unroll
  for (int q = 0; q < VPL; ++q) col[q] = 0.f;
#pragma unroll
  for (int i = 0; i < TPW; ++i)
    if (iq[i] >= 0 && iq[i] < E) atomicAdd(&cn[iq[i]], 1);
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    if (t0 + i >= T) break;  // uniform per wave
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < VPL; ++q) m = fmaxf(m, lv[i][q]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    float z = 0.f, ev[VPL];
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
      ev[q] = q * 64 + lane < E ? expf(lv[i][q] - m) : 0.f;
      z += ev[q];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off, 64);
#pragma unroll
    for (int q = 0; q < VPL; ++q) col[q] += ev[q] / z;
  }
#pragma unroll
  for (int q = 0; q < VPL; ++q) pp[wave][q * 64 + lane] = col[q];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    pp_part[(int64_t)blockIdx.x * E + e] = ((pp[0][e] + pp[1][e]) + pp[2][e]) + pp[3][e];
    cnt_part[(int64_t)blockIdx.x * E + e] = cn[e];
  }
}

// One workgroup: thread e adds expert e's block partials in block order
// (neighbouring threads read neighbouring words, so the loads of a block row
// coalesce and stay in flight together), then wavefront 0 adds the experts'
// terms in order.
__global__ __launch_bounds__(512) void aux_loss_final_kernel(const float* pp_part,
                                                             const int32_t* cnt_part, int nblk,
                                                             int T, int E, int k, float alpha,
                                                             float* loss, float* aux_w) {
  __shared__ float term[512];
  const int e = threadIdx.x;
  if (e < E) {
    float ps = 0.f;
    int c = 0;
    constexpr int U = 32;  // block partials loaded together, then added in order
    int b = 0;
    for (; b + U <= nblk; b += U) {
      float pv[U];
      int cv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        pv[u] = pp_part[(int64_t)(b + u) * E + e];
        cv[u] = cnt_part[(int64_t)(b + u) * E + e];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        ps += pv[u];
        c += cv[u];
      }
    }
    for (; b < nblk; ++b) {
      ps += pp_part[(int64_t)b * E + e];
      c += cnt_part[(int64_t)b * E + e];
    }
    const float f = (float)c / ((float)T * (float)k);
    term[e] = f * (ps / (float)T);
    aux_w[e] = alpha * (float)E * f / (float)T;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    float v = 0.f;
    for (int i = lane; i < E; i += 64) v += term[i];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0) loss[0] = alpha * (float)E * v;
  }
}

int64_t aux_loss_ws_bytes(int T, int E) {
  const int64_t nblk = ceil_div(T, ROUTE_BWD_TOKENS);
  return 2 * round_up(nblk * E * 4, 256);
}

moe_status_t launch_aux_loss(const float* logits, const int32_t* idx, int T, int E, int k,
                             float alpha, float* loss, float* aux_w, void* ws, hipStream_t s) {
  const int nblk = (int)ceil_div(T, ROUTE_BWD_TOKENS);
  float* pp_part = static_cast<float*>(ws);
  int32_t* cnt_part = reinterpret_cast<int32_t*>(static_cast<char*>(ws) +
                                                 round_up((int64_t)nblk * E * 4, 256));
  {
  ProfScope prof("aux_loss_part", s);
  if (E <= 64) aux_loss_part_kernel<1><<<nblk, 256, 0, s>>>(logits, idx, T, E, k, pp_part, cnt_part);
  else if (E <= 128) aux_loss_part_kernel<2><<<nblk, 256, 0, s>>>(logits, idx, T, E, k, pp_part, cnt_part);
  else if (E <= 256) aux_loss_part_kernel<4><<<nblk, 256, 0, s>>>(logits, idx, T, E, k, pp_part, cnt_part);
  else aux_loss_part_kernel<8><<<nblk, 256, 0, s>>>(logits, idx, T, E, k, pp_part, cnt_part);
  const moe_status_t st = check_launch("aux_loss_part_kernel");
  if (st != MOE_OK) return st;
  }
  ProfScope prof("aux_loss_final", s);
  aux_loss_final_kernel<<<1, 512, 0, s>>>(pp_part, cnt_part, nblk, T, E, k, alpha, loss, aux_w);
  return check_launch("aux_loss_final_kernel");
}

// Final sums of the router backward, each in a fixed order:
// dw[i] = sum_s dw_part[s][i] (split-K partials of x^T dL, when nsplit > 0),
// db[e] = sum_b db_part[b][e] (per-workgroup column sums of dL, when db).
// dw[i] = sum of the nsplit partials (in split order), for the first nb_dw
// workgroups; db[e] = sum over the nblk block partials, one wavefront per
// expert: lane l adds blocks l, l + 64, ... in order, then the lanes are
// combined by a fixed butterfly.  Deterministic either way.
__global__ __launch_bounds__(256) void route_bwd_reduce_kernel(const float* dw_part, int nsplit,
                                                               int64_t n_dw, bf16_t* dw,
                                                               const float* db_part, int nblk,
                                                               int E, float* db, int nb_dw) {
  if ((int)blockIdx.x < nb_dw) {
    const int64_t stride = (int64_t)nb_dw * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_dw; i += stride) {
      float v = 0.f;
      for (int sp = 0; sp < nsplit; ++sp) v += dw_part[(int64_t)sp * n_dw + i];
      dw[i] = f2bf(v);
    }
    return;
  }
  const int lane = threadIdx.x & 63;
  const int e = ((int)blockIdx.x - nb_dw) * 4 + (threadIdx.x >> 6);
  if (e >= E) return;  // uniform per wave
  float v = 0.f;
  for (int b = lane; b < nblk; b += 64) v += db_part[(int64_t)b * E + e];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  if (lane == 0) db[e] = v;
}

moe_status_t launch_route_bwd_reduce(const float* dw_part, int nsplit, int64_t n_dw, bf16_t* dw,
                                     const float* db_part, int nblk, int E, float* db,
                                     hipStream_t s) {
  const int nb_dw = nsplit > 0 ? (int)std::min<int64_t>(ceil_div(n_dw, 256), 2048) : 0;
  const int nb_db = db ? (int)ceil_div(E, 4) : 0;
  if (nb_dw + nb_db == 0) return MOE_OK;
  ProfScope prof("route_bwd_reduce", s);
  route_bwd_reduce_kernel<<<nb_dw + nb_db, 256, 0, s>>>(dw_part, nsplit, n_dw, dw, db_part, nblk,
                                                        E, db, nb_dw);
  return check_launch("route_bwd_reduce_kernel");
}

// ---------------------------------------------------------------- fill
// Zeroes up to three buffers in one launch.
struct ZeroList {
  uint32_t* p[3];
  int64_t n[3];  // 4-byte words
};

__global__ void fill_zero_kernel(ZeroList z) {
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
#pragma unroll
  for (int b = 0; b < 3; ++b)
    for (int64_t i = i0; i < z.n[b]; i += stride) z.p[b][i] = 0u;
}

moe_status_t launch_fill_zero(void* p0, int64_t bytes0, void* p1, int64_t bytes1, void* p2,
                              int64_t bytes2, hipStream_t s) {
  ZeroList z{};
  void* ps[3] = {p0, p1, p2};
  const int64_t bs[3] = {bytes0, bytes1, bytes2};
  int64_t most = 0;
  for (int b = 0; b < 3; ++b) {
    z.p[b] = static_cast<uint32_t*>(ps[b]);
    z.n[b] = ps[b] ? bs[b] / 4 : 0;  // every buffer here is a multiple of 4 bytes
    most = std::max(most, z.n[b]);
  }
  if (most <= 0) return MOE_OK;
  ProfScope prof("fill_zero", s);
  const unsigned grid = (unsigned)std::min<int64_t>(ceil_div(most, 256), 4096);
  fill_zero_kernel<<<grid, 256, 0, s>>>(z);
  return check_launch("fill_zero_kernel");
}

}  // namespace moe
