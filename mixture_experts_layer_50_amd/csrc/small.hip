// Small-batch expert FFN: the batched_mm expert backend of page "Accelerating
// Transformers fine-tuning with NVIDIA NeMo AutoModel", section 专家后端 (table
// of backends: every routed (token, slot) pair multiplies by its own expert's
// weights in one batched product; meant for small inputs).  Nothing is sorted:
// each (token, slot) pair reads its expert's weights directly, so for a few
// tokens the whole FFN is two memory-bound matrix-vector kernels and the
// combine, instead of the sort, the tile tables and two grouped GEMMs.
//
// Kernel 1, one workgroup per (pair, column block of the expert width, K
// split): partial sums of Hg = x[t] Wg[e] and Hu = x[t] Wu[e] over the
// block's columns and one of KS ranges of d (KS > 1 only when there are too
// few pairs to fill the GPU).
// Kernel 2, one workgroup per (pair, column block of d): adds the KS partials
// in order, A = silu(Hg) Hu (rounded to the dtype), then Yp[pair] = A Wd[e].
// Then the combine kernel sums Yp over each token's slots in ascending slot
// order.  Inside a workgroup, lane (rs, c) of wave w accumulates the rows
// r = 8w + rs (mod 32) for its 16-byte column chunk c; the 32 partial sums of
// a column are added in a fixed order, so results are deterministic.
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

// Rows [0, K) of a row-major [K][ld] matrix (ld elements per row) at column
// n0 + 16-byte chunk c: lane (rs, c) of wave w adds rows 8w + rs + 32i,
// scaled by v[row], into acc.  K % 32 == 0.  NM matrices share the rows.
template <typename ELT, int NM>
__device__ __forceinline__ void gemv_rows(const ELT* const (&m)[NM], int64_t ld, int K,
                                          const float* v, int w, int rs, int c,
                                          float (&acc)[NM][Vec16<ELT>::N]) {
  constexpr int N = Vec16<ELT>::N;
  constexpr int U = 4;  // rows in flight per lane
  int r = 8 * w + rs;
  for (; r + 32 * (U - 1) < K; r += 32 * U) {
    uint4 q[U][NM];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int h = 0; h < NM; ++h)
        q[u][h] = *reinterpret_cast<const uint4*>(m[h] + (int64_t)(r + 32 * u) * ld + c * N);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float s = v[r + 32 * u];
#pragma unroll
      for (int h = 0; h < NM; ++h) {
        float f[N];
        Vec16<ELT>::unpack(q[u][h], f);
#pragma unroll
        for (int i = 0; i < N; ++i) acc[h][i] = fmaf(s, f[i], acc[h][i]);
      }
    }
  }
  for (; r < K; r += 32) {
    const float s = v[r];
#pragma unroll
    for (int h = 0; h < NM; ++h) {
      float f[N];
      Vec16<ELT>::unpack(*reinterpret_cast<const uint4*>(m[h] + (int64_t)r * ld + c * N), f);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[h][i] = fmaf(s, f[i], acc[h][i]);
    }
  }
}

// The workgroup's column sums: red holds [4 waves][8 rs][8 c][NM][N] partials.
template <int NM, int N>
__device__ __forceinline__ float column_sum(const float* red, int h, int col) {
  const int c = col / N, i = col % N;
  float s = 0.f;
  for (int w = 0; w < 4; ++w)
    for (int rs = 0; rs < 8; ++rs) s += red[(((w * 8 + rs) * 8 + c) * NM + h) * N + i];
  return s;
}

// The pair's expert as a local index, or -1 when the slot is not local or
// repeats an expert an earlier slot of the token holds (as in the permute).
__device__ __forceinline__ int pair_expert(const int32_t* idx, int pair, int k, int e_lo, int e_hi) {
  const int t = pair / k, j = pair % k;
  const int e = idx[pair];
  bool local = e >= e_lo && e < e_hi;
  for (int jj = 0; jj < j; ++jj) local = local && idx[(int64_t)t * k + jj] != e;
  return local ? e - e_lo : -1;
}

template <typename ELT>
__global__ __launch_bounds__(256) void small_gateup_kernel(const ELT* x, const int32_t* idx,
                                                           const ELT* wg, const ELT* wu, int d,
                                                           int I, int k, int e_lo, int e_hi,
                                                           float* part, int32_t* inv) {
  constexpr int N = Vec16<ELT>::N, CB = 8 * N;
  const int pair = blockIdx.y, ks = blockIdx.z, KS = gridDim.z;
  const int le = pair_expert(idx, pair, k, e_lo, e_hi);
  if (blockIdx.x == 0 && ks == 0 && threadIdx.x == 0) inv[pair] = le >= 0 ? pair : -1;
  if (le < 0) return;
  extern __shared__ float smem[];  // x[t] over the K range as fp32 (Kc), then the partial sums
  const int Kc = d / KS, k0 = ks * Kc;
  float* sx = smem;
  float* red = smem + Kc;
  const int t = pair / k;
  for (int i = threadIdx.x; i < Kc; i += 256) sx[i] = Elt<ELT>::load(x + (int64_t)t * d + k0 + i);
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, rs = lane >> 3, c = lane & 7;
  const int n0 = blockIdx.x * CB;
  const int64_t base = ((int64_t)le * d + k0) * I + n0;
  const ELT* const m[2] = {wg + base, wu + base};
  float acc[2][N];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < N; ++i) acc[h][i] = 0.f;
  gemv_rows<ELT, 2>(m, I, Kc, sx, w, rs, c, acc);
  // partials: [w][rs][c][h][i]
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < N; ++i) red[(((w * 8 + rs) * 8 + c) * 2 + h) * N + i] = acc[h][i];
  __syncthreads();
  if (threadIdx.x < 2 * CB) {
    const int h = threadIdx.x / CB, col = threadIdx.x % CB;
    part[(((int64_t)pair * KS + ks) * 2 + h) * I + n0 + col] = column_sum<2, N>(red, h, col);
  }
}

template <typename ELT>
__global__ __launch_bounds__(256) void small_down_kernel(const float* part, int KS,
                                                         const int32_t* idx, const ELT* wd, int d,
                                                         int I, int k, int e_lo, int e_hi,
                                                         ELT* yp) {
  constexpr int N = Vec16<ELT>::N, CB = 8 * N;
  const int pair = blockIdx.y;
  const int le = pair_expert(idx, pair, k, e_lo, e_hi);
  if (le < 0) return;
  extern __shared__ float smem[];  // A[pair] as fp32 (I), then the partial sums
  float* sa = smem;
  float* red = smem + I;
  for (int i = threadIdx.x; i < I; i += 256) {
    const float* p = part + (int64_t)pair * KS * 2 * I + i;
    float g = 0.f, u = 0.f;
    for (int ks = 0; ks < KS; ++ks) {
      g += p[(int64_t)ks * 2 * I];
      u += p[(int64_t)ks * 2 * I + I];
    }
    float av;
    if constexpr (sizeof(ELT) == 2) av = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
    else av = g / (1.0f + expf(-g)) * u;
    ELT q;
    Elt<ELT>::store(&q, av);  // A is rounded to the dtype, as the grouped path stores it
    sa[i] = Elt<ELT>::load(&q);
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, rs = lane >> 3, c = lane & 7;
  const int n0 = blockIdx.x * CB;
  const ELT* const m[1] = {wd + (int64_t)le * I * d + n0};
  float acc[1][N];
#pragma unroll
  for (int i = 0; i < N; ++i) acc[0][i] = 0.f;
  gemv_rows<ELT, 1>(m, d, I, sa, w, rs, c, acc);
#pragma unroll
  for (int i = 0; i < N; ++i) red[((w * 8 + rs) * 8 + c) * N + i] = acc[0][i];
  __syncthreads();
  if (threadIdx.x < CB) {
    const int col = threadIdx.x;
    Elt<ELT>::store(yp + (int64_t)pair * d + n0 + col, column_sum<1, N>(red, 0, col));
  }
}

}  // namespace

// K splits of the gate/up kernel: only when there are too few pairs to give
// every CU a workgroup (the split costs the down kernel a pass over the
// partials), each split at least 128 rows of d.
static int small_ks(int64_t pairs, int d, int I, int elt_bytes) {
  const int64_t blocks = pairs * (I / (8 * (16 / elt_bytes)));
  int ks = 1;
  while (ks < 8 && blocks * ks < 256 && d % (2 * ks * 128) == 0) ks *= 2;
  return ks;
}

int64_t small_ffn_ws_bytes(int T, int d, int k, int I, int elt_bytes) {
  const int64_t pairs = (int64_t)T * k;
  const int KS = small_ks(pairs, d, I, elt_bytes);
  return round_up(pairs * KS * 2 * I * 4, 256) + round_up(pairs * d * elt_bytes, 256) +
         round_up(pairs * 4, 256);
}

moe_status_t launch_small_ffn(const void* x, const int32_t* idx, const float* w_topk,
                              const void* wg, const void* wu, const void* wd, int T, int d, int k,
                              int I, int e_lo, int e_hi, int elt_bytes, void* y, void* ws,
                              hipStream_t s) {
  const int64_t pairs = (int64_t)T * k;
  const int KS = small_ks(pairs, d, I, elt_bytes);
  char* base = static_cast<char*>(ws);
  float* part = reinterpret_cast<float*>(base);
  const int64_t part_bytes = round_up(pairs * KS * 2 * I * 4, 256);
  void* yp = base + part_bytes;
  int32_t* inv = reinterpret_cast<int32_t*>(base + part_bytes + round_up(pairs * d * elt_bytes, 256));
  const int N = 16 / elt_bytes, CB = 8 * N;
  moe_status_t st;
  {
    ProfScope prof("small_gateup", s);
    const dim3 grid((unsigned)(I / CB), (unsigned)pairs, (unsigned)KS);
    const size_t lds = (size_t)(d / KS + 4 * 8 * 8 * 2 * N) * 4;
    if (elt_bytes == 2)
      small_gateup_kernel<bf16_t><<<grid, 256, lds, s>>>(
          static_cast<const bf16_t*>(x), idx, static_cast<const bf16_t*>(wg),
          static_cast<const bf16_t*>(wu), d, I, k, e_lo, e_hi, part, inv);
    else
      small_gateup_kernel<float><<<grid, 256, lds, s>>>(
          static_cast<const float*>(x), idx, static_cast<const float*>(wg),
          static_cast<const float*>(wu), d, I, k, e_lo, e_hi, part, inv);
    if ((st = check_launch("small_gateup_kernel")) != MOE_OK) return st;
  }
  {
    ProfScope prof("small_down", s);
    const dim3 grid((unsigned)(d / CB), (unsigned)pairs);
    const size_t lds = (size_t)(I + 4 * 8 * 8 * N) * 4;
    if (elt_bytes == 2)
      small_down_kernel<bf16_t><<<grid, 256, lds, s>>>(part, KS, idx,
                                                       static_cast<const bf16_t*>(wd), d, I, k,
                                                       e_lo, e_hi, static_cast<bf16_t*>(yp));
    else
      small_down_kernel<float><<<grid, 256, lds, s>>>(part, KS, idx, static_cast<const float*>(wd),
                                                      d, I, k, e_lo, e_hi,
                                                      static_cast<float*>(yp));
    if ((st = check_launch("small_down_kernel")) != MOE_OK) return st;
  }
  return launch_gather_sum(yp, inv, w_topk, T, d, k, elt_bytes, y, s, "small_combine");
}

}  // namespace moe
