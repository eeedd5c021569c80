// Token permutation and combine kernels of the MoE layer.
//
// The permutation sorts the (token, slot) rows by expert, so that one grouped
// GEMM can run over the expert groups (page "Accelerating Transformers
// fine-tuning with NVIDIA NeMo AutoModel", section 专家后端, grouped_mm row).
// It is a deterministic counting sort in three passes and two launches:
//   1. per block of 256 tokens, one 256-bit token mask per local expert is
//      built in LDS (atomic OR: order-free), and its popcounts are the
//      block's expert histogram;
//   2. (second launch) every block scans the histograms in (expert, block)
//      order for itself, giving its first position per expert (block 0 also
//      writes the group offsets);
//   3. each block rebuilds its masks and places row (t, j) of expert e at
//      base[block][e] + popcount(mask_e below t): stable by token, and since
//      a token's kept experts are distinct, stable by row t*k + j (a slot
//      repeating an earlier slot's expert is dropped).
// A fourth kernel copies each token's x row to its k sorted positions.
//
// Combine (the pages give token dispatch and combine kernels of their own:
// section 加速来源, DeepEP item) is a gather-weighted sum
// back to token order; its backward and the permutation's backward are the
// matching gather/scatter kernels.  All sums run in a fixed order.
#include "kernels.h"

namespace moe {

constexpr int MASK_WORDS = PERM_TOKENS / 32;

int64_t permute_ws_bytes(int T, int E_loc) {
  return ceil_div(T, PERM_TOKENS) * (int64_t)E_loc * 4;
}

constexpr int MAXK = 32;

// The expert ids of this thread's token (slots >= k, and tokens >= T, get -1),
// all loads in flight together.
__device__ __forceinline__ void load_ids(int (&ids)[MAXK], const int32_t* idx, int T, int k) {
  const int t = blockIdx.x * PERM_TOKENS + threadIdx.x;
#pragma unroll
  for (int j = 0; j < MAXK; ++j) ids[j] = (t < T && j < k) ? idx[(int64_t)t * k + j] : -1;
}

__device__ __forceinline__ void build_masks(uint32_t* mask, const int (&ids)[MAXK], int e_lo, int e_hi,
                                            int E_loc) {
  for (int i = threadIdx.x; i < E_loc * MASK_WORDS; i += blockDim.x) mask[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < MAXK; ++j) {
    const int e = ids[j];
    if (e >= e_lo && e < e_hi)
      atomicOr(&mask[(e - e_lo) * MASK_WORDS + (threadIdx.x >> 5)], 1u << (threadIdx.x & 31));
  }
  __syncthreads();
}

__global__ __launch_bounds__(PERM_TOKENS) void perm_count_kernel(const int32_t* idx, int T, int k,
                                                                 int e_lo, int e_hi,
                                                                 int32_t* counts) {
  extern __shared__ uint32_t mask[];
  const int E_loc = e_hi - e_lo;
  int ids[MAXK];
  load_ids(ids, idx, T, k);
  build_masks(mask, ids, e_lo, e_hi, E_loc);
  for (int e = threadIdx.x; e < E_loc; e += blockDim.x) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < MASK_WORDS; ++w) c += __popc(mask[e * MASK_WORDS + w]);
    counts[(int64_t)blockIdx.x * E_loc + e] = c;
  }
}

// Scatter with the scan folded in: workgroup b reads the block counts of all
// blocks (nb x E_loc, written by perm_count_kernel) and works out its own
// first position per expert: the expert's offset (exclusive scan of the
// experts' totals) plus its counts in the blocks before b.  Every workgroup
// repeats this small scan instead of waiting for a separate scan launch;
// workgroup 0 writes the group offsets.  Positions are those of the
// three-kernel path.
constexpr int SCAT_MAX_E = 512;  // local experts: the entry points allow E <= 512

__global__ __launch_bounds__(PERM_TOKENS) void perm_scan_scatter_kernel(
    const int32_t* idx, int T, int k, int e_lo, int e_hi, int R_cap, const int32_t* counts, int nb,
    int32_t* offsets, int32_t* perm, int32_t* inv) {
  extern __shared__ uint32_t mask[];
  __shared__ int32_t sbase[SCAT_MAX_E];
  __shared__ int32_t stot[SCAT_MAX_E];
  __shared__ int32_t wsum[PERM_TOKENS / 64];
  const int E_loc = e_hi - e_lo;
  const int b = blockIdx.x;
  // 1. per expert: counts of the blocks before b, and the total (U loads in flight)
  for (int e = threadIdx.x; e < E_loc; e += PERM_TOKENS) {
    constexpr int U = 8;
    int before = 0, total = 0;
    for (int b0 = 0; b0 < nb; b0 += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = b0 + u < nb ? counts[(int64_t)(b0 + u) * E_loc + e] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (b0 + u < b) before += v[u];
        total += v[u];
      }
    }
    sbase[e] = before;
    stot[e] = total;
  }
  __syncthreads();
  // 2. exclusive scan of the totals over experts: each thread a contiguous run
  //    of experts, then the runs' sums across the workgroup
  constexpr int NTH = PERM_TOKENS;
  const int per = (E_loc + NTH - 1) / NTH;
  const int lo = min(E_loc, (int)threadIdx.x * per), hi = min(E_loc, lo + per);
  int run = 0;
  for (int e = lo; e < hi; ++e) run += stot[e];
  // inclusive scan of run over the threads: within a wavefront, then waves
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int inc = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(inc, off, 64);
    if (lane >= off) inc += v;
  }
  if (lane == 63) wsum[wv] = inc;
  __syncthreads();
  int prev = 0;
  for (int w = 0; w < wv; ++w) prev += wsum[w];
  int o = prev + inc - run;  // exclusive prefix of this thread's first expert
  for (int e = lo; e < hi; ++e) {
    const int t_e = stot[e];
    sbase[e] += o;
    if (b == 0) offsets[e] = min(o, R_cap);
    o += t_e;
  }
  if (b == 0 && hi == E_loc && lo < hi) offsets[E_loc] = min(o, R_cap);
  // 3. the block's masks, ranks and positions
  int ids[MAXK];
  load_ids(ids, idx, T, k);
  build_masks(mask, ids, e_lo, e_hi, E_loc);  // starts and ends with a barrier
  const int t = blockIdx.x * PERM_TOKENS + threadIdx.x;
  if (t >= T) return;
  const int w = threadIdx.x >> 5;
  const uint32_t below = (1u << (threadIdx.x & 31)) - 1u;
#pragma unroll
  for (int j = 0; j < MAXK; ++j) {
    if (j >= k) continue;
    const int64_t r = (int64_t)t * k + j;
    const int e = ids[j];
    bool keep = e >= e_lo && e < e_hi;
#pragma unroll
    for (int jj = 0; jj < j; ++jj)  // a repeated expert keeps its first slot only
      if (ids[jj] == e) keep = false;
    int pos = -1;
    if (keep) {
      const uint32_t* m = mask + (e - e_lo) * MASK_WORDS;
      int rank = __popc(m[w] & below);
      for (int ww = 0; ww < w; ++ww) rank += __popc(m[ww]);
      pos = sbase[e - e_lo] + rank;
      if (pos >= R_cap) pos = -1;
      else perm[pos] = (int32_t)r;
    }
    inv[r] = pos;
  }
}

// One wavefront per token: read x[t] once, write it to every sorted position.
// Lane j < k holds the token's j-th sorted position; the chunk loop reads it
// back with a lane broadcast instead of reloading it.  The loop runs over
// whole wavefronts of chunks (lanes past the last chunk idle through it), so
// every broadcast executes with all lanes active, also when k > chunks.
__global__ __launch_bounds__(256) void perm_gather_kernel(const uint4* x, const int32_t* inv, int T,
                                                          int k, int chunks, uint4* xp) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int myp = lane < k ? inv[(int64_t)t * k + lane] : -1;
  for (int c0 = 0; c0 < chunks; c0 += 64) {
    const int c = c0 + lane;
    const bool ok = c < chunks;
    const uint4 v = ok ? x[(int64_t)t * chunks + c] : make_uint4(0u, 0u, 0u, 0u);
    for (int j = 0; j < k; ++j) {
      const int p = __builtin_amdgcn_readlane(myp, j);
      if (ok && p >= 0) xp[(int64_t)p * chunks + c] = v;
    }
  }
}

moe_status_t launch_permute(const int32_t* idx, const void* x, int T, int d, int k, int e_lo,
                            int e_hi, int R_cap, int elt_bytes, int32_t* offsets, int32_t* perm,
                            int32_t* inv, void* xp, void* ws, hipStream_t s) {
  const int E_loc = e_hi - e_lo;
  const int nb = (int)ceil_div(T, PERM_TOKENS);
  int32_t* counts = static_cast<int32_t*>(ws);
  const size_t lds = (size_t)E_loc * MASK_WORDS * 4;
  moe_status_t st;
  {
    ProfScope prof("permute_count", s);
    perm_count_kernel<<<nb, PERM_TOKENS, lds, s>>>(idx, T, k, e_lo, e_hi, counts);
    if ((st = check_launch("perm_count_kernel")) != MOE_OK) return st;
  }
  {  // the scan runs inside the scatter kernel (every workgroup its own part)
    ProfScope prof("permute_scatter", s);
    perm_scan_scatter_kernel<<<nb, PERM_TOKENS, lds, s>>>(idx, T, k, e_lo, e_hi, R_cap, counts, nb,
                                                          offsets, perm, inv);
    if ((st = check_launch("perm_scan_scatter_kernel")) != MOE_OK) return st;
  }
  if (xp)  // without xp only the sort runs (the gathered GEMMs read x through perm)
    return launch_permute_gather(x, inv, T, d, k, elt_bytes, xp, s);
  return MOE_OK;
}

moe_status_t launch_permute_gather(const void* x, const int32_t* inv, int T, int d, int k,
                                   int elt_bytes, void* xp, hipStream_t s) {
  ProfScope prof("permute_gather", s);
  const int chunks = d * elt_bytes / 16;
  perm_gather_kernel<<<(unsigned)ceil_div(T, 4), 256, 0, s>>>(
      static_cast<const uint4*>(x), inv, T, k, chunks, static_cast<uint4*>(xp));
  return check_launch("perm_gather_kernel");
}

// ---------------------------------------------------------------- combine
// 16-byte chunk helpers for both element types.
template <typename T> struct Chunk;
template <> struct Chunk<bf16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void unpack(const uint4& v, float (&f)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static uint4 pack(const float (&f)[8]) {
    return make_uint4(pack_bf2(f[0], f[1]), pack_bf2(f[2], f[3]), pack_bf2(f[4], f[5]),
                      pack_bf2(f[6], f[7]));
  }
};
template <> struct Chunk<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void unpack(const uint4& v, float (&f)[4]) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
  __device__ __forceinline__ static uint4 pack(const float (&f)[4]) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
};

// y[t] = sum_j w[t,j] * src[inv[t,j]] in ascending j (w NULL: weight 1).
// One wavefront per token; lane j < k holds slot j's position and weight,
// broadcast to the wavefront in the chunk loop; the k row loads of a chunk are
// all issued before the first is used.  The chunk loop runs over whole
// wavefronts of chunks, so the broadcasts execute with all lanes active.
template <typename T>
__global__ __launch_bounds__(256) void gather_sum_kernel(const uint4* src, const int32_t* inv,
                                                         const float* w, int Tn, int k, int chunks,
                                                         uint4* y) {
  constexpr int N = Chunk<T>::N;
  constexpr int G = 8;  // rows in flight per lane
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int myp = lane < k ? inv[(int64_t)t * k + lane] : -1;
  const float myw = lane < k ? (w ? w[(int64_t)t * k + lane] : 1.0f) : 0.0f;
  for (int c0 = 0; c0 < chunks; c0 += 64) {
    const int c = c0 + lane;
    const bool ok = c < chunks;
    float acc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.f;
    for (int j0 = 0; j0 < k; j0 += G) {
      uint4 v[G];
#pragma unroll
      for (int jj = 0; jj < G; ++jj) {
        const int j = j0 + jj;
        const int p = j < k ? __builtin_amdgcn_readlane(myp, j) : -1;
        v[jj] = (ok && p >= 0) ? src[(int64_t)p * chunks + c] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int jj = 0; jj < G; ++jj) {
        const int j = j0 + jj;
        const int p = j < k ? __builtin_amdgcn_readlane(myp, j) : -1;
        if (p < 0) continue;  // uniform over the wavefront
        const float g = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, myw), j));
        float f[N];
        Chunk<T>::unpack(v[jj], f);
#pragma unroll
        for (int i = 0; i < N; ++i) acc[i] = fmaf(g, f[i], acc[i]);
      }
    }
    if (ok) y[(int64_t)t * chunks + c] = Chunk<T>::pack(acc);
  }
}

moe_status_t launch_gather_sum(const void* src, const int32_t* inv, const float* w, int T, int d,
                               int k, int elt_bytes, void* y, hipStream_t s, const char* name) {
  ProfScope prof(name, s);
  const int chunks = d * elt_bytes / 16;
  const unsigned grid = (unsigned)ceil_div(T, 4);
  if (elt_bytes == 2)
    gather_sum_kernel<bf16_t><<<grid, 256, 0, s>>>(static_cast<const uint4*>(src), inv, w, T, k,
                                                   chunks, static_cast<uint4*>(y));
  else
    gather_sum_kernel<float><<<grid, 256, 0, s>>>(static_cast<const uint4*>(src), inv, w, T, k,
                                                  chunks, static_cast<uint4*>(y));
  return check_launch(name);
}

// dyp[inv[t,j]] = w[t,j] * dy[t];  dw[t,j] = <dy[t], yp[inv[t,j]]> (0 when
// dropped); nothing when dyp_flag points to a zero.
// One wavefront per token, slot data broadcast from lane j as above (the
// chunk loop over whole wavefronts of chunks, all lanes active).
template <typename T>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const uint4* dy, const uint4* yp,
                                                          const int32_t* inv, const float* w,
                                                          int Tn, int k, int chunks, uint4* dyp,
                                                          const int32_t* dyp_flag, float* dw) {
  constexpr int N = Chunk<T>::N;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  if (dyp_flag && *dyp_flag == 0) return;  // neither output is wanted from this kernel
  const int myp = lane < k ? inv[(int64_t)t * k + lane] : -1;
  const float myw = lane < k ? w[(int64_t)t * k + lane] : 0.0f;
  float part[MAXK];
#pragma unroll
  for (int j = 0; j < MAXK; ++j) part[j] = 0.f;
  for (int c0 = 0; c0 < chunks; c0 += 64) {
    const int c = c0 + lane;
    const bool ok = c < chunks;
    float fy[N];
    Chunk<T>::unpack(ok ? dy[(int64_t)t * chunks + c] : make_uint4(0u, 0u, 0u, 0u), fy);
#pragma unroll
    for (int j0 = 0; j0 < MAXK; j0 += 8) {
      if (j0 >= k) break;  // uniform
      uint4 v[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int j = j0 + jj;
        const int p = j < k ? __builtin_amdgcn_readlane(myp, j) : -1;
        v[jj] = (ok && p >= 0) ? yp[(int64_t)p * chunks + c] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int j = j0 + jj;
        const int p = j < k ? __builtin_amdgcn_readlane(myp, j) : -1;
        if (p < 0) continue;  // uniform over the wavefront
        const float g = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, myw), j));
        float f[N], o[N];
        Chunk<T>::unpack(v[jj], f);
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < N; ++i) {
          a = fmaf(fy[i], f[i], a);
          o[i] = g * fy[i];
        }
        part[j] += a;  // lanes past the last chunk add zeros
        if (ok) dyp[(int64_t)p * chunks + c] = Chunk<T>::pack(o);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < MAXK; ++j) {
    if (j < k) {  // k is uniform over the wavefront
      float v = part[j];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
      const bool kept = __builtin_amdgcn_readlane(myp, j) >= 0;  // all lanes active here
      if (lane == 0) dw[(int64_t)t * k + j] = kept ? v : 0.f;
    }
  }
}

// dw[s] = sum_b part[inv[s] * stride + b] in ascending b for every slot s
// with inv[s] >= 0, else 0; nothing when flag points to a nonzero value.
__global__ __launch_bounds__(256) void gate_grad_sum_kernel(const int32_t* inv, const float* part,
                                                            int stride, int slots,
                                                            const int32_t* flag, float* dw) {
  if (*flag != 0) return;
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= slots) return;
  const int p = inv[s];
  float v = 0.f;
  if (p >= 0) {  // stride is even (I / 32, I a multiple of 64): the row in 8-byte pairs
    const float2* row = reinterpret_cast<const float2*>(part + (int64_t)p * stride);
#pragma unroll 4
    for (int b = 0; b < stride / 2; ++b) {
      const float2 x = row[b];
      v += x.x;
      v += x.y;
    }
  }
  dw[s] = v;
}

moe_status_t launch_gate_grad_sum(const int32_t* inv, const float* part, int stride, int slots,
                                  const int32_t* flag, float* dw, hipStream_t s) {
  ProfScope prof("gate_grad_sum", s);
  if (slots <= 0) return MOE_OK;
  gate_grad_sum_kernel<<<(unsigned)ceil_div(slots, 256), 256, 0, s>>>(inv, part, stride, slots,
                                                                     flag, dw);
  return check_launch("gate_grad_sum_kernel");
}

moe_status_t launch_combine_bwd(const void* dy, const void* yp, const int32_t* inv, const float* w,
                                int T, int d, int k, int elt_bytes, void* dyp, float* dw,
                                hipStream_t s, const int32_t* dyp_flag) {
  ProfScope prof("combine_bwd", s);
  const int chunks = d * elt_bytes / 16;
  const unsigned grid = (unsigned)ceil_div(T, 4);
  if (elt_bytes == 2)
    combine_bwd_kernel<bf16_t><<<grid, 256, 0, s>>>(
        static_cast<const uint4*>(dy), static_cast<const uint4*>(yp), inv, w, T, k, chunks,
        static_cast<uint4*>(dyp), dyp_flag, dw);
  else
    combine_bwd_kernel<float><<<grid, 256, 0, s>>>(
        static_cast<const uint4*>(dy), static_cast<const uint4*>(yp), inv, w, T, k, chunks,
        static_cast<uint4*>(dyp), dyp_flag, dw);
  return check_launch("combine_bwd_kernel");
}

// ---------------------------------------------------------------------------
// Routing-table check (moe_check_routing).  check_table_kernel: one thread
// per token tests its k ids against [0, E) and against the token's earlier
// slots; with counts, the local ids under the first-slot rule go into the
// block's LDS histogram, whose nonzero bins are added into counts (integer
// adds: the totals do not depend on their order).  The block's bits are ORed
// in LDS, then once into *flags.  check_offsets_kernel (one wavefront) forms
// the exclusive prefix of counts, clamps each entry to R_cap as the permute
// does, and compares it with the caller's offsets.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void check_table_kernel(const int32_t* idx, int T, int k, int E,
                                                          int e_lo, int e_hi, int32_t* counts,
                                                          int32_t* flags) {
  __shared__ int hist[512];
  __shared__ int bits;
  const int E_loc = e_hi - e_lo;
  if (threadIdx.x == 0) bits = 0;
  if (counts)
    for (int i = threadIdx.x; i < E_loc; i += 256) hist[i] = 0;
  __syncthreads();
  const int t = blockIdx.x * 256 + threadIdx.x;
  int b = 0;
  if (t < T) {
    const int32_t* row = idx + (int64_t)t * k;
    for (int j = 0; j < k; ++j) {
      const int e = row[j];
      if (e < 0 || e >= E) b |= CHECK_IDX_RANGE;
      bool first = true;
      for (int jj = 0; jj < j; ++jj) first = first && row[jj] != e;
      if (!first) b |= CHECK_IDX_REPEAT;
      if (counts && first && e >= e_lo && e < e_hi) atomicAdd(&hist[e - e_lo], 1);
    }
  }
  if (b) atomicOr(&bits, b);
  __syncthreads();
  if (counts)
    for (int i = threadIdx.x; i < E_loc; i += 256)
      if (hist[i]) atomicAdd(&counts[i], hist[i]);
  if (threadIdx.x == 0 && bits) atomicOr(flags, bits);
}

__global__ __launch_bounds__(64) void check_offsets_kernel(const int32_t* counts, int E_loc,
                                                           int R_cap, const int32_t* offsets,
                                                           int32_t* flags) {
  const int lane = threadIdx.x;
  // (the counts add up to at most T*k < 2^31: int sums do not overflow)
  int run = 0;  // rows of the experts before this chunk of 64
  bool bad = false;
  for (int c0 = 0; c0 <= E_loc; c0 += 64) {
    const int i = c0 + lane;
    const int v = i < E_loc ? counts[i] : 0;
    // inclusive prefix over the wavefront, then exclusive for entry i
    int inc = v;
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(inc, o, 64);
      if (lane >= o) inc += u;
    }
    const int excl = run + inc - v;
    if (i <= E_loc) bad = bad || offsets[i] != (excl < R_cap ? excl : R_cap);
    run += __shfl(inc, 63, 64);
  }
  if (__any(bad) && lane == 0) atomicOr(flags, CHECK_OFFSETS);
}

moe_status_t launch_check_routing(const int32_t* idx, int T, int k, int E, int e_lo, int e_hi,
                                  int R_cap, const int32_t* offsets, int32_t* counts,
                                  int32_t* flags, hipStream_t s) {
  ProfScope prof("check_routing", s);
  const int E_loc = e_hi - e_lo;
  if (offsets) {
    const moe_status_t z = launch_fill_zero(counts, (int64_t)E_loc * 4, nullptr, 0, nullptr, 0, s);
    if (z != MOE_OK) return z;
  }
  check_table_kernel<<<(unsigned)ceil_div(T, 256), 256, 0, s>>>(idx, T, k, E, e_lo, e_hi,
                                                               offsets ? counts : nullptr, flags);
  moe_status_t st = check_launch("check_table_kernel");
  if (st != MOE_OK || !offsets) return st;
  check_offsets_kernel<<<1, 64, 0, s>>>(counts, E_loc, R_cap, offsets, flags);
  return check_launch("check_offsets_kernel");
}

}  // namespace moe
