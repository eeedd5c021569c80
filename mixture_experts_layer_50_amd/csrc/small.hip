// Small-batch expert FFN: the batched_mm expert backend of page "Accelerating
// Transformers fine-tuning with NVIDIA NeMo AutoModel", section 专家后端 (table
// of backends: the routed (token, slot) pairs multiply by their experts'
// weights in batched products, with no grouping kernels; meant for small
// inputs).  Nothing is sorted: each workgroup finds its expert's pairs in the
// routing table itself, so for a few tokens the whole FFN is two memory-bound
// matrix-vector kernels, instead of the sort, the tile tables and two grouped
// GEMMs.
//
// Expert-major: grid row y takes the y-th active local expert (ascending id;
// rows past the number of active experts exit), and lists that expert's
// pairs in ascending pair order (at most one per token: the local,
// first-occurrence slots, as in the permute).  The expert's weights are read
// once per column block however many of its tokens there are, in groups of
// up to TG tokens per pass.
// Kernel 1, one workgroup per (column block of the expert width, active
// expert, K split): partial sums of Hg = x[t] Wg[e] and Hu = x[t] Wu[e] over
// the block's columns and one of KS ranges of d (ranges of at most 512
// rows), into part[pair][ks].  It also
// zeroes the combine's counters and the output rows of tokens with no kept
// slot (strided over the whole grid).  For one or two tokens it can also take
// the gate's last step (SmallRoute): every workgroup adds the router's
// partial logits and takes the top k itself before it builds its table.
// Kernel 2, one workgroup per (column block of d, active expert): adds the KS
// partials in order, A = silu(Hg) Hu (rounded to the dtype), then
// Yp[pair] = A Wd[e] over the block's columns.  The combine runs inside
// kernel 2: the workgroup that writes the last of a token's pair rows for a
// column block (an integer arrival counter per token and column block, its
// increment after the block's stores are complete) sums the token's pairs in
// ascending slot order from the stored rows, the operations and order of the
// combine kernel.
// Inside a workgroup, in each batch of 32 U rows lane (rs, c) of wave w
// accumulates the U consecutive rows from (8w + rs) U on for its 16-byte
// column chunk c (its factors then come in one vector load); a column's 32
// partial sums are added by a butterfly over rs within the wave, then over
// the four waves in order: results are deterministic.  Every load of a batch
// is unconditional (clamped addresses, zero factors past the end), so that
// all of them are in flight together.
#include "kernels.h"

namespace moe {

namespace {

template <typename ELT> struct Vec16;
template <> struct Vec16<bf16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void unpack(const uint4& v, float (&f)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void unpack(const uint4& v, float (&f)[4]) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
};

// A lane's rows of a row-major [K][ld] matrix (ld elements per row) at
// column chunk c (16 bytes): in each batch of 32 U rows, lane (rs, c) of wave
// w takes the U consecutive rows from (8w + rs) U on (so its factors are
// consecutive too).  issue_rows loads the block that starts at row r (a
// block at or past K, which K % U == 0 keeps whole, reads row 0 instead),
// all U rows in flight together; use_rows adds them, scaled by v[tg][u] for
// TG vectors, into acc.  The caller gives a block past K the factors 0: with
// no branch between them the loads stay ahead of their uses.
template <typename ELT, int NM, int U>
__device__ __forceinline__ void issue_rows(uint4 (&q)[U][NM], const ELT* const (&m)[NM], int64_t ld,
                                           int r, int K, int c) {
  constexpr int N = Vec16<ELT>::N;
  const int r0 = r < K ? r : 0;
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int h = 0; h < NM; ++h)
      q[u][h] = *reinterpret_cast<const uint4*>(m[h] + (int64_t)(r0 + u) * ld + c * N);
}

template <typename ELT, int NM, int TG, int U>
__device__ __forceinline__ void use_rows(const uint4 (&q)[U][NM], const float (&v)[TG][U],
                                         float (&acc)[TG][NM][Vec16<ELT>::N]) {
  constexpr int N = Vec16<ELT>::N;
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int h = 0; h < NM; ++h) {
      float f[N];
      Vec16<ELT>::unpack(q[u][h], f);
#pragma unroll
      for (int tg = 0; tg < TG; ++tg)
#pragma unroll
        for (int i = 0; i < N; ++i) acc[tg][h][i] = fmaf(v[tg][u], f[i], acc[tg][h][i]);
    }
  }
}

// U consecutive elements of a row from p (16-byte aligned) as fp32.
template <typename ELT, int U>
__device__ __forceinline__ void load_block(const ELT* p, float (&f)[U]) {
  constexpr int N = Vec16<ELT>::N;
  static_assert(U % N == 0, "whole 16-byte chunks");
#pragma unroll
  for (int v = 0; v < U / N; ++v) {
    float g[N];
    Vec16<ELT>::unpack(reinterpret_cast<const uint4*>(p)[v], g);
#pragma unroll
    for (int i = 0; i < N; ++i) f[v * N + i] = g[i];
  }
}

// Sums acc over the eight row slots rs of the wave (lanes 8 apart): a
// butterfly, so every lane ends with the same, order-fixed sum.
template <int TG, int NM, int N>
__device__ __forceinline__ void sum_row_slots(float (&acc)[TG][NM][N]) {
#pragma unroll
  for (int off = 8; off < 64; off <<= 1)
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
      for (int h = 0; h < NM; ++h)
#pragma unroll
        for (int i = 0; i < N; ++i) acc[tg][h][i] += __shfl_xor(acc[tg][h][i], off, 64);
}

// Device-coherent stores and loads of one element (sc1: through to the point
// every XCD reads from), for the rows the combine reads back from other
// workgroups.
constexpr int SMALL_CPOL = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t small_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff,
                                           0x00020000);
}
__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, int off, bf16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16((short)v, r, off * 2, 0, SMALL_CPOL);
}
__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, int off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off * 4, 0, SMALL_CPOL);
}
template <typename ELT> __device__ __forceinline__ float load_coherent(__amdgpu_buffer_rsrc_t r, int off);
template <> __device__ __forceinline__ float load_coherent<bf16_t>(__amdgpu_buffer_rsrc_t r, int off) {
  return bf2f((bf16_t)__builtin_amdgcn_raw_buffer_load_b16(r, off * 2, 0, SMALL_CPOL));
}
template <> __device__ __forceinline__ float load_coherent<float>(__amdgpu_buffer_rsrc_t r, int off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off * 4, 0, SMALL_CPOL));
}

// The workgroup's view of the routing table, in LDS: every pair's local
// expert (pe), the set of active experts, and the pairs of one expert.
struct PairTable {
  int16_t pe[SMALL_MAX_PAIRS];
  uint16_t list[SMALL_MAX_PAIRS];
  uint32_t mask[16];  // local experts 0..511
  int wcnt[4];
  int expert;
};

// Fills pe (the pair's expert as a local index, or -1 when the slot is not
// local or repeats an expert an earlier slot of the token holds, as in the
// permute) and mask, then takes the nth active expert (ascending) and lists
// its pairs in ascending order.  Returns the number of pairs (0 when there is
// no nth active expert); the same value in every thread.
__device__ int find_expert_pairs(PairTable& pt, const int32_t* idx, int npairs, int k, int e_lo,
                                 int e_hi, int nth) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid < 16) pt.mask[tid] = 0;
  // the table's local ids (-1: not local) staged in list, one load a thread
  int16_t* loc = reinterpret_cast<int16_t*>(pt.list);
  for (int p = tid; p < npairs; p += 256) {
    const int e = idx[p];
    loc[p] = (int16_t)(e >= e_lo && e < e_hi ? e - e_lo : -1);
  }
  __syncthreads();
  for (int p = tid; p < npairs; p += 256) {
    const int t = p / k, j = p % k;
    int le = loc[p];
    for (int jj = 0; jj < j && le >= 0; ++jj)
      if (loc[t * k + jj] == le) le = -1;
    pt.pe[p] = (int16_t)le;
    if (le >= 0) atomicOr(&pt.mask[le >> 5], 1u << (le & 31));
  }
  __syncthreads();
  if (tid == 0) {
    int rem = nth, e = -1;
    for (int wi = 0; wi < 16; ++wi) {
      uint32_t m = pt.mask[wi];
      const int c = __popc(m);
      if (rem < c) {
        for (int r = 0; r < rem; ++r) m &= m - 1;
        e = wi * 32 + __ffs(m) - 1;
        break;
      }
      rem -= c;
    }
    pt.expert = e;
  }
  __syncthreads();
  const int le = pt.expert;
  if (le < 0) return 0;
  int total = 0;
  for (int base = 0; base < npairs; base += 256) {
    const int p = base + tid;
    const bool hit = p < npairs && pt.pe[p] == le;
    const unsigned long long b = __ballot(hit);
    if (lane == 0) pt.wcnt[w] = __popcll(b);
    __syncthreads();
    int off = total;
    for (int ww = 0; ww < w; ++ww) off += pt.wcnt[ww];
    if (hit) pt.list[off + __popcll(b & ((1ull << lane) - 1))] = (uint16_t)p;
    total += pt.wcnt[0] + pt.wcnt[1] + pt.wcnt[2] + pt.wcnt[3];
    __syncthreads();
  }
  return total;
}

// The gate inside the workgroup (SmallRoute): logits of all T tokens from
// the router's partials (split order, then the bias), the top k by rank
// (a larger logit, or an equal one with a lower id, comes first) and the
// softmax in slot order, the operations of small_router_final_kernel.  The
// table lands in sidx [T*k]; `write`: also to the outputs.
__device__ void route_in_block(const SmallRoute& r, int T, int k, float* sl, int32_t* sidx,
                               float* sv, bool write) {
  const int E = r.E, ns = r.nsplit, tid = threadIdx.x;
  constexpr int SB = 32;  // partials in flight per item
  for (int i = tid; i < T * E; i += 256) {
    const int t = i / E, e = i % E;
    float a = 0.f;
    for (int s0 = 0; s0 < ns; s0 += SB) {
      float pv[SB];
#pragma unroll
      for (int j = 0; j < SB; ++j) pv[j] = r.part[((int64_t)min(s0 + j, ns - 1) * T + t) * E + e];
#pragma unroll
      for (int j = 0; j < SB; ++j)
        if (s0 + j < ns) a += pv[j];
    }
    if (r.bias) a += r.bias[e];
    sl[i] = a;
    if (write) r.logits[i] = a;
  }
  __syncthreads();
  for (int i = tid; i < T * E; i += 256) {
    const int t = i / E, e = i % E;
    const float v = sl[i];
    const float* row = sl + t * E;
    int rank = 0;
#pragma unroll 8
    for (int o = 0; o < E; ++o) rank += row[o] > v || (row[o] == v && o < e);
    if (rank < k) {
      sidx[t * k + rank] = e;
      sv[t * k + rank] = v;
    }
  }
  __syncthreads();
  if (tid < T) {
    const int t = tid;
    const float vmax = sv[t * k];
    float sum = 0.f;
    for (int j = 0; j < k; ++j) sum += expf(sv[t * k + j] - vmax);
    if (write)
      for (int j = 0; j < k; ++j) {
        r.idx[t * k + j] = sidx[t * k + j];
        r.w[t * k + j] = expf(sv[t * k + j] - vmax) / sum;
      }
  }
  __syncthreads();
}

template <typename ELT, int TG, bool ROUTE>
__global__ __launch_bounds__(256) void small_gateup_kernel(const ELT* x, const int32_t* idx,
                                                           SmallRoute route, const ELT* wg,
                                                           const ELT* wu, int T, int d, int I,
                                                           int k, int e_lo, int e_hi, float* part,
                                                           int32_t* cnt, ELT* y) {
  constexpr int N = Vec16<ELT>::N, CB = 8 * N;
  constexpr int RT = ROUTE ? SMALL_FUSED_ROUTE_MAX_TE : 1;
  __shared__ PairTable pt;
  __shared__ float r_logit[RT], r_val[RT];
  __shared__ int32_t r_idx[RT];
  const int npairs = T * k, ks = blockIdx.z, KS = gridDim.z;
  const int32_t* table = idx;
  if constexpr (ROUTE) {
    route_in_block(route, T, k, r_logit, r_idx, r_val,
                   blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0);
    table = r_idx;
  }
  const int n = find_expert_pairs(pt, table, npairs, k, e_lo, e_hi, blockIdx.y);
  // the combine's counters, and y = 0 for tokens with no kept slot, strided
  // over the grid
  {
    const int nwg = gridDim.x * gridDim.y * gridDim.z;
    const int wid = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int ncb = d / CB;
    for (int64_t i = (int64_t)wid * 256 + threadIdx.x; i < (int64_t)T * ncb; i += (int64_t)nwg * 256)
      cnt[i] = 0;
    for (int t = wid; t < T; t += nwg) {
      bool any = false;
      for (int j = 0; j < k; ++j) any = any || pt.pe[t * k + j] >= 0;
      if (!any)
        for (int c = threadIdx.x; c < d; c += 256) Elt<ELT>::store(y + (int64_t)t * d + c, 0.f);
    }
  }
  if (n == 0) return;
  const int le = pt.expert;
  extern __shared__ float red[];  // the wave sums: [4 waves][TG][2][CB]
  const int Kc = d / KS, k0 = ks * Kc;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, rs = lane >> 3, c = lane & 7;
  const int n0 = blockIdx.x * CB;
  const int64_t base = ((int64_t)le * d + k0) * I + n0;
  const ELT* const m[2] = {wg + base, wu + base};
  constexpr int U = 8;
  for (int g0 = 0; g0 < n; g0 += TG) {
    // the group's x rows over the K range, read by each lane at its own rows
    // (a token past the group's end repeats the last one: computed, not stored)
    const ELT* xr[TG];
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
      xr[tg] = x + (int64_t)(pt.list[min(g0 + tg, n - 1)] / k) * d + k0;
    float acc[TG][2][N];
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < N; ++i) acc[tg][h][i] = 0.f;
    for (int b0 = 0; b0 < Kc; b0 += 32 * U) {
      const int r = b0 + (8 * w + rs) * U;
      const bool ok = r < Kc;
      uint4 q[U][2];
      float xv[TG][U];
      issue_rows<ELT, 2, U>(q, m, I, r, Kc, c);
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {
        load_block<ELT, U>(xr[tg] + (ok ? r : 0), xv[tg]);
#pragma unroll
        for (int u = 0; u < U; ++u) xv[tg][u] = ok ? xv[tg][u] : 0.f;
      }
      use_rows<ELT, 2, TG, U>(q, xv, acc);
    }
    sum_row_slots(acc);
    if (rs == 0)
#pragma unroll
      for (int tg = 0; tg < TG; ++tg)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < N; ++i) red[((w * TG + tg) * 2 + h) * CB + c * N + i] = acc[tg][h][i];
    __syncthreads();
    for (int o = threadIdx.x; o < TG * 2 * CB; o += 256) {
      const int tg = o / (2 * CB), h = (o / CB) % 2, col = o % CB;
      if (g0 + tg >= n) continue;
      float sum = 0.f;
      for (int ww = 0; ww < 4; ++ww) sum += red[((ww * TG + tg) * 2 + h) * CB + col];
      const int pair = pt.list[g0 + tg];
      part[(((int64_t)pair * KS + ks) * 2 + h) * I + n0 + col] = sum;
    }
    __syncthreads();
  }
}

template <typename ELT, int TG>
__global__ __launch_bounds__(256) void small_down_kernel(const float* part, int KS,
                                                         const int32_t* idx, const ELT* wd, int T,
                                                         int d, int I, int k, int e_lo, int e_hi,
                                                         ELT* yp, const float* w_topk,
                                                         int32_t* cnt, ELT* y) {
  constexpr int N = Vec16<ELT>::N, CB = 8 * N;
  __shared__ PairTable pt;
  __shared__ int last[TG];
  const int npairs = T * k;
  const int n = find_expert_pairs(pt, idx, npairs, k, e_lo, e_hi, blockIdx.y);
  if (n == 0) return;
  const int le = pt.expert;
  extern __shared__ float smem[];  // A rows of TG pairs (fp32 of the rounded values), then the wave sums
  float* sa = smem;
  float* red = smem + TG * I;  // [4 waves][TG][CB]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, rs = lane >> 3, c = lane & 7;
  const int cb = blockIdx.x, n0 = cb * CB, ncb = d / CB;
  const ELT* const m[1] = {wd + (int64_t)le * I * d + n0};
  const __amdgpu_buffer_rsrc_t ryp = small_rsrc(yp);
  constexpr int U = 8;
  for (int g0 = 0; g0 < n; g0 += TG) {
    // the first batch of Wd rows is in flight while A is formed
    int b0 = 0, r = (8 * w + rs) * U;
    uint4 q[U][1];
    issue_rows<ELT, 1, U>(q, m, d, r, I, c);
    const int iq = I / 4;  // float4 groups of a row
    // A for float4 group i of the pass's rows: the KS partials in order
    auto a_group = [&](int i) {
      const int tg = i / iq, qi = i % iq;
      float av[4] = {0.f, 0.f, 0.f, 0.f};
      if (g0 + tg < n) {
        const float* p = part + (int64_t)pt.list[g0 + tg] * KS * 2 * I + qi * 4;
        // unconditional loads (a clamped split past KS, never added), all in
        // flight together
        float4 gv[8], uv[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const float* ps = p + (int64_t)min(s, KS - 1) * 2 * I;
          gv[s] = *reinterpret_cast<const float4*>(ps);
          uv[s] = *reinterpret_cast<const float4*>(ps + I);
        }
        float g[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 8; ++s)
          if (s < KS) {
            g[0] += gv[s].x; g[1] += gv[s].y; g[2] += gv[s].z; g[3] += gv[s].w;
            u[0] += uv[s].x; u[1] += uv[s].y; u[2] += uv[s].z; u[3] += uv[s].w;
          }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float a;
          if constexpr (sizeof(ELT) == 2) a = g[j] * __builtin_amdgcn_rcpf(1.0f + __expf(-g[j])) * u[j];
          else a = g[j] / (1.0f + expf(-g[j])) * u[j];
          ELT rv;
          Elt<ELT>::store(&rv, a);  // A is rounded to the dtype, as the grouped path stores it
          av[j] = Elt<ELT>::load(&rv);
        }
      }
      *reinterpret_cast<float4*>(sa + tg * I + qi * 4) = make_float4(av[0], av[1], av[2], av[3]);
    };
    // the thread's first group in straight-line code, so that its partial
    // loads go out while the Wd rows are still in flight; the rest in a loop
    if (threadIdx.x < TG * iq) a_group(threadIdx.x);
    for (int i = threadIdx.x + 256; i < TG * iq; i += 256) a_group(i);
    __syncthreads();
    float acc[TG][1][N];
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
      for (int i = 0; i < N; ++i) acc[tg][0][i] = 0.f;
    for (;;) {
      const bool ok = r < I;
      float av[TG][U];
#pragma unroll
      for (int tg = 0; tg < TG; ++tg)
#pragma unroll
        for (int u = 0; u < U; u += 4) {
          const float4 a4 = *reinterpret_cast<const float4*>(sa + tg * I + (ok ? r : 0) + u);
          av[tg][u] = ok ? a4.x : 0.f;
          av[tg][u + 1] = ok ? a4.y : 0.f;
          av[tg][u + 2] = ok ? a4.z : 0.f;
          av[tg][u + 3] = ok ? a4.w : 0.f;
        }
      use_rows<ELT, 1, TG, U>(q, av, acc);
      b0 += 32 * U;
      if (b0 >= I) break;
      r = b0 + (8 * w + rs) * U;
      issue_rows<ELT, 1, U>(q, m, d, r, I, c);
    }
    sum_row_slots(acc);
    if (rs == 0)
#pragma unroll
      for (int tg = 0; tg < TG; ++tg)
#pragma unroll
        for (int i = 0; i < N; ++i) red[(w * TG + tg) * CB + c * N + i] = acc[tg][0][i];
    __syncthreads();
    for (int o = threadIdx.x; o < TG * CB; o += 256) {
      const int tg = o / CB, col = o % CB;
      if (g0 + tg >= n) continue;
      float sum = 0.f;
      for (int ww = 0; ww < 4; ++ww) sum += red[(ww * TG + tg) * CB + col];
      ELT yv;
      Elt<ELT>::store(&yv, sum);
      store_coherent(ryp, (int)((int64_t)pt.list[g0 + tg] * d + n0 + col), yv);
    }
    // the group's rows of Yp are complete before the counters move
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (threadIdx.x < TG) {
      const int tg = threadIdx.x;
      int is_last = 0;
      if (g0 + tg < n) {
        const int t = pt.list[g0 + tg] / k;
        int kept = 0;
        for (int j = 0; j < k; ++j) kept += pt.pe[t * k + j] >= 0;
        const int old = __hip_atomic_fetch_add(cnt + (int64_t)t * ncb + cb, 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        is_last = old == kept - 1;
      }
      last[tg] = is_last;
    }
    __syncthreads();
    // the last writer of a token's rows: y[t] over this column block, slots
    // in ascending order
    for (int o = threadIdx.x; o < TG * CB; o += 256) {
      const int tg = o / CB, col = n0 + o % CB;
      if (g0 + tg >= n || !last[tg]) continue;
      const int t = pt.list[g0 + tg] / k;
      float sum = 0.f;
      for (int j = 0; j < k; ++j) {
        const int pj = t * k + j;
        if (pt.pe[pj] < 0) continue;
        sum = fmaf(w_topk[pj], load_coherent<ELT>(ryp, (int)((int64_t)pj * d + col)), sum);
      }
      Elt<ELT>::store(y + (int64_t)t * d + col, sum);
    }
    __syncthreads();
  }
}

}  // namespace

// Tokens per pass: two while the active experts average under two tokens
// each (fewer registers, more workgroups resident; an expert's third token
// re-reads its weights), else four; in the down kernel halved while their
// fp32 A rows would take more than 32 KB of LDS.
static int small_tg(int64_t pairs, int64_t nexp, int a_len) {
  int tg = pairs >= 2 * nexp ? 4 : 2;
  while (tg > 1 && (int64_t)tg * a_len * 4 > 32768) tg /= 2;
  return tg;
}

// K splits of the gate/up kernel: ranges of at most 512 rows of d (up to 8
// splits, each whole 64-row slices, at least 128 rows).  Measured at the
// Qwen3 shape (d = 2048, natural router), against splitting only while fewer
// than 512 workgroups would run: the same at T = 1 to 4, gate/up kernel
// 54 vs 63 us at T = 8 and 90 vs 102 us at T = 16; 256-row ranges were
// slower at T = 2 and 4 (each workgroup's table set-up is repeated per split).
static int small_ks(int d) {
  int ks = 1;
  while (ks < 8 && d / ks > 512 && d % (2 * ks * 64) == 0 && d / (2 * ks) >= 128) ks *= 2;
  return ks;
}

static int64_t small_nexp(int T, int k, int e_lo, int e_hi) {
  return std::min<int64_t>((int64_t)T * k, e_hi - e_lo);
}

// Workspace: gate/up partials [pairs][KS][2I] fp32, Yp [pairs][d], the
// combine's arrival counters [T][d / (8 N)].
int64_t small_ffn_ws_bytes(int T, int d, int k, int I, int e_lo, int e_hi, int elt_bytes) {
  const int64_t pairs = (int64_t)T * k;
  const int KS = small_ks(d);
  const int CB = 8 * (16 / elt_bytes);
  return round_up(pairs * KS * 2 * I * 4, 256) + round_up(pairs * d * elt_bytes, 256) +
         round_up((int64_t)T * (d / CB) * 4, 256);
}

moe_status_t launch_small_ffn(const void* x, const int32_t* idx, const float* w_topk,
                              const void* wg, const void* wu, const void* wd, int T, int d, int k,
                              int I, int e_lo, int e_hi, int elt_bytes, void* y, void* ws,
                              hipStream_t s, const SmallRoute* route) {
  const int64_t pairs = (int64_t)T * k, nexp = small_nexp(T, k, e_lo, e_hi);
  const int KS = small_ks(d);
  char* base = static_cast<char*>(ws);
  float* part = reinterpret_cast<float*>(base);
  const int64_t part_bytes = round_up(pairs * KS * 2 * I * 4, 256);
  void* yp = base + part_bytes;
  int32_t* cnt = reinterpret_cast<int32_t*>(base + part_bytes + round_up(pairs * d * elt_bytes, 256));
  const int N = 16 / elt_bytes, CB = 8 * N;
  moe_status_t st;
  {
    ProfScope prof("small_gateup", s);
    const dim3 grid((unsigned)(I / CB), (unsigned)nexp, (unsigned)KS);
    const int TG = small_tg(pairs, nexp, 0);
    const size_t lds = (size_t)(4 * TG * 2 * CB) * 4;
    const SmallRoute r = route ? *route : SmallRoute{nullptr, nullptr, 0, 0, nullptr, nullptr, nullptr};
#define L_(E_, TG_, R_)                                                                       \
  small_gateup_kernel<E_, TG_, R_><<<grid, 256, lds, s>>>(                                    \
      static_cast<const E_*>(x), idx, r, static_cast<const E_*>(wg),                          \
      static_cast<const E_*>(wu), T, d, I, k, e_lo, e_hi, part, cnt, static_cast<E_*>(y))
#define LR_(E_, TG_)        \
  if (route) L_(E_, TG_, true); \
  else L_(E_, TG_, false);
    if (elt_bytes == 2) { if (TG == 4) { LR_(bf16_t, 4) } else { LR_(bf16_t, 2) } }
    else { if (TG == 4) { LR_(float, 4) } else { LR_(float, 2) } }
#undef LR_
#undef L_
    if ((st = check_launch("small_gateup_kernel")) != MOE_OK) return st;
  }
  {
    ProfScope prof("small_down", s);
    const dim3 grid((unsigned)(d / CB), (unsigned)nexp);
    const int TG = small_tg(pairs, nexp, I);
    const size_t lds = (size_t)(TG * I + 4 * TG * CB) * 4;
#define L_(E_, TG_)                                                                          \
  small_down_kernel<E_, TG_><<<grid, 256, lds, s>>>(                                         \
      part, KS, idx, static_cast<const E_*>(wd), T, d, I, k, e_lo, e_hi, static_cast<E_*>(yp), \
      w_topk, cnt, static_cast<E_*>(y))
#define LT_(E_)                  \
  if (TG == 4) L_(E_, 4);        \
  else if (TG == 2) L_(E_, 2);   \
  else L_(E_, 1);
    if (elt_bytes == 2) { LT_(bf16_t) } else { LT_(float) }
#undef LT_
#undef L_
    if ((st = check_launch("small_down_kernel")) != MOE_OK) return st;
  }
  return MOE_OK;
}

}  // namespace moe
