// Token permutation and combine kernels of the MoE layer.
//
// The permutation sorts the (token, slot) rows by expert ("sort tokens by
// their assigned expert, then one grouped GEMM": page "Accelerating
// Transformers fine-tuning with NVIDIA NeMo AutoModel", section 专家后端).
// It is a deterministic counting sort in three passes:
//   1. per block of 256 tokens, one 256-bit token mask per local expert is
//      built in LDS (atomic OR: order-free), and its popcounts are the
//      block's expert histogram;
//   2. one workgroup scans the histograms in (expert, block) order, giving
//      each block its first position per expert and the group offsets;
//   3. each block rebuilds its masks and places row (t, j) of expert e at
//      base[block][e] + popcount(mask_e below t): stable by token, and since
//      a token's k experts are distinct, stable by row t*k + j.
// A fourth kernel copies each token's x row to its k sorted positions.
//
// Combine ("dispatch and combine", section 加速来源) is a gather-weighted sum
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

// One workgroup; E_loc <= 1024.  counts[b][e] becomes the first sorted
// position of block b's rows of expert e.  TPE = 1024 / E_loc (rounded down
// to a power of two) threads share an expert, each summing a contiguous run
// of blocks; the runs and then the experts are scanned in order.
__global__ __launch_bounds__(1024) void perm_scan_kernel(int32_t* counts, int nb, int E_loc, int R_cap,
                                                         int32_t* offsets) {
  __shared__ int32_t part[1024];
  __shared__ int32_t scan[1024];
  int tpe = 1;
  while (tpe * 2 * E_loc <= 1024) tpe *= 2;
  const int e = threadIdx.x / tpe, c = threadIdx.x % tpe;
  const int run = (nb + tpe - 1) / tpe;
  const int b_lo = min(nb, c * run), b_hi = min(nb, b_lo + run);
  constexpr int U = 8;  // block counts in flight per thread
  int sum = 0;
  if (e < E_loc) {
    for (int b0 = b_lo; b0 < b_hi; b0 += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = b0 + u < b_hi ? counts[(int64_t)(b0 + u) * E_loc + e] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u) sum += v[u];
    }
  }
  part[threadIdx.x] = sum;
  __syncthreads();
  int before = 0, total = 0;  // this run's start within its expert; the expert's total
  if (e < E_loc) {
    for (int cc = 0; cc < tpe; ++cc) {
      const int v = part[e * tpe + cc];
      if (cc < c) before += v;
      total += v;
    }
  }
  scan[threadIdx.x] = (e < E_loc && c == 0) ? total : 0;  // one entry per expert, at its first thread
  __syncthreads();
  for (int s = 1; s < 1024; s <<= 1) {  // inclusive Hillis-Steele scan
    const int v = threadIdx.x >= s ? scan[threadIdx.x - s] : 0;
    __syncthreads();
    scan[threadIdx.x] += v;
    __syncthreads();
  }
  if (e < E_loc) {
    const int o = scan[e * tpe] - total;  // exclusive prefix over experts
    int pos = o + before;
    for (int b0 = b_lo; b0 < b_hi; b0 += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = b0 + u < b_hi ? counts[(int64_t)(b0 + u) * E_loc + e] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (b0 + u < b_hi) {
          counts[(int64_t)(b0 + u) * E_loc + e] = pos;
          pos += v[u];
        }
    }
    if (c == 0) {
      offsets[e] = min(o, R_cap);
      if (e == E_loc - 1) offsets[E_loc] = min(o + total, R_cap);
    }
  }
}

__global__ __launch_bounds__(PERM_TOKENS) void perm_scatter_kernel(const int32_t* idx, int T, int k,
                                                                   int e_lo, int e_hi, int R_cap,
                                                                   const int32_t* base,
                                                                   int32_t* perm, int32_t* inv) {
  extern __shared__ uint32_t mask[];
  const int E_loc = e_hi - e_lo;
  int ids[MAXK];
  load_ids(ids, idx, T, k);
  build_masks(mask, ids, e_lo, e_hi, E_loc);
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
      pos = base[(int64_t)blockIdx.x * E_loc + (e - e_lo)] + rank;
      if (pos >= R_cap) pos = -1;
      else perm[pos] = (int32_t)r;
    }
    inv[r] = pos;
  }
}

// One wavefront per token: read x[t] once, write it to every sorted position.
// Lane j < k holds the token's j-th sorted position; the chunk loop reads it
// back with a lane broadcast instead of reloading it.
__global__ __launch_bounds__(256) void perm_gather_kernel(const uint4* x, const int32_t* inv, int T,
                                                          int k, int chunks, uint4* xp) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int myp = lane < k ? inv[(int64_t)t * k + lane] : -1;
  for (int c = lane; c < chunks; c += 64) {
    const uint4 v = x[(int64_t)t * chunks + c];
    for (int j = 0; j < k; ++j) {
      const int p = __builtin_amdgcn_readlane(myp, j);
      if (p >= 0) xp[(int64_t)p * chunks + c] = v;
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
  {
    ProfScope prof("permute_scan", s);
    perm_scan_kernel<<<1, 1024, 0, s>>>(counts, nb, E_loc, R_cap, offsets);
    if ((st = check_launch("perm_scan_kernel")) != MOE_OK) return st;
  }
  {
    ProfScope prof("permute_scatter", s);
    perm_scatter_kernel<<<nb, PERM_TOKENS, lds, s>>>(idx, T, k, e_lo, e_hi, R_cap, counts, perm, inv);
    if ((st = check_launch("perm_scatter_kernel")) != MOE_OK) return st;
  }
  if (xp) {  // without xp only the sort runs (the gathered GEMMs read x through perm)
    ProfScope prof("permute_gather", s);
    const int chunks = d * elt_bytes / 16;
    perm_gather_kernel<<<(unsigned)ceil_div(T, 4), 256, 0, s>>>(
        static_cast<const uint4*>(x), inv, T, k, chunks, static_cast<uint4*>(xp));
    if ((st = check_launch("perm_gather_kernel")) != MOE_OK) return st;
  }
  return MOE_OK;
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
// all issued before the first is used.
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
  for (int c = lane; c < chunks; c += 64) {
    float acc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.f;
    for (int j0 = 0; j0 < k; j0 += G) {
      uint4 v[G];
#pragma unroll
      for (int jj = 0; jj < G; ++jj) {
        const int j = j0 + jj;
        const int p = j < k ? __builtin_amdgcn_readlane(myp, j) : -1;
        v[jj] = p >= 0 ? src[(int64_t)p * chunks + c] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int jj = 0; jj < G; ++jj) {
        const int j = j0 + jj;
        const int p = j < k ? __builtin_amdgcn_readlane(myp, j) : -1;
        if (p < 0) continue;
        const float g = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, myw), j));
        float f[N];
        Chunk<T>::unpack(v[jj], f);
#pragma unroll
        for (int i = 0; i < N; ++i) acc[i] = fmaf(g, f[i], acc[i]);
      }
    }
    y[(int64_t)t * chunks + c] = Chunk<T>::pack(acc);
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

// dyp[inv[t,j]] = w[t,j] * dy[t];  dw[t,j] = <dy[t], yp[inv[t,j]]> (0 when dropped).
// One wavefront per token, slot data broadcast from lane j as above.
template <typename T>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const uint4* dy, const uint4* yp,
                                                          const int32_t* inv, const float* w,
                                                          int Tn, int k, int chunks, uint4* dyp,
                                                          float* dw) {
  constexpr int N = Chunk<T>::N;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int myp = lane < k ? inv[(int64_t)t * k + lane] : -1;
  const float myw = lane < k ? w[(int64_t)t * k + lane] : 0.0f;
  float part[MAXK];
#pragma unroll
  for (int j = 0; j < MAXK; ++j) part[j] = 0.f;
  for (int c = lane; c < chunks; c += 64) {
    float fy[N];
    Chunk<T>::unpack(dy[(int64_t)t * chunks + c], fy);
#pragma unroll
    for (int j0 = 0; j0 < MAXK; j0 += 8) {
      if (j0 >= k) break;  // uniform
      uint4 v[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int j = j0 + jj;
        const int p = j < k ? __builtin_amdgcn_readlane(myp, j) : -1;
        v[jj] = p >= 0 ? yp[(int64_t)p * chunks + c] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int j = j0 + jj;
        const int p = j < k ? __builtin_amdgcn_readlane(myp, j) : -1;
        if (p < 0) continue;
        const float g = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, myw), j));
        float f[N], o[N];
        Chunk<T>::unpack(v[jj], f);
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < N; ++i) {
          a = fmaf(fy[i], f[i], a);
          o[i] = g * fy[i];
        }
        part[j] += a;
        dyp[(int64_t)p * chunks + c] = Chunk<T>::pack(o);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < MAXK; ++j) {
    if (j < k) {  // k is uniform over the wavefront
      float v = part[j];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
      if (lane == 0) dw[(int64_t)t * k + j] = __builtin_amdgcn_readlane(myp, j) >= 0 ? v : 0.f;
    }
  }
}

moe_status_t launch_combine_bwd(const void* dy, const void* yp, const int32_t* inv, const float* w,
                                int T, int d, int k, int elt_bytes, void* dyp, float* dw,
                                hipStream_t s) {
  ProfScope prof("combine_bwd", s);
  const int chunks = d * elt_bytes / 16;
  const unsigned grid = (unsigned)ceil_div(T, 4);
  if (elt_bytes == 2)
    combine_bwd_kernel<bf16_t><<<grid, 256, 0, s>>>(
        static_cast<const uint4*>(dy), static_cast<const uint4*>(yp), inv, w, T, k, chunks,
        static_cast<uint4*>(dyp), dw);
  else
    combine_bwd_kernel<float><<<grid, 256, 0, s>>>(
        static_cast<const uint4*>(dy), static_cast<const uint4*>(yp), inv, w, T, k, chunks,
        static_cast<uint4*>(dyp), dw);
  return check_launch("combine_bwd_kernel");
}

}  // namespace moe
