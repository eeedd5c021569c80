// Grouped GEMM kernels of the MoE layer for gfx950.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 (fp32 accumulation) on LDS-staged
// 64-deep K slices in two LDS buffers, with several further slices in flight
// in registers, four waves per workgroup.  Operands stored k-contiguous sit in
// LDS the same way (16-byte chunks XOR-swizzled by row); operands stored
// n-contiguous (weights [K][N], activations read transposed) are copied as is
// and read back with the gfx950 LDS transpose read.  Workgroup ids are remapped
// so that consecutive tiles land on the same XCD (its own L2), and tiles that
// share an A row block or a weight column block run together (GROUP_M order).
//
// fp32 path: a plain fp32 kernel (one output per thread, fp32 FMA) used for
// fp32 layers, which are small parity workloads.
#include <utility>

#include "gemm.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;  // K extent of one LDS stage: 8 chunks of 8 bf16
constexpr int NXCD = 8;

// Physical 16-byte chunk of logical chunk c in LDS row r (conflict-free for
// 8 or 16 consecutive rows reading the same logical chunk).
__device__ __forceinline__ int swz(int r, int c) { return c ^ (r & 7) ^ ((r >> 3) & 1); }

// Hardware dispatches workgroup ids round-robin over the 8 XCDs.  Give each
// XCD a contiguous range of the `count` real tiles instead.
__device__ __forceinline__ int remap_xcd(int pid, int count) {
  int xcd = pid % NXCD, idx = pid / NXCD;
  int per = count / NXCD, rem = count % NXCD;
  return xcd * per + min(xcd, rem) + idx;
}

// Linear tile id -> (m tile, n tile), GM m tiles at a time over all n tiles.
__device__ __forceinline__ void group_order(int L, int mt_count, int nt_count, int& mt, int& nt) {
  constexpr int GM = 4;
  int per_group = GM * nt_count;
  int g = L / per_group;
  int first = g * GM;
  int gsize = min(mt_count - first, GM);
  int r = L - g * per_group;
  mt = first + r % gsize;
  nt = r / gsize;
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// ---------------------------------------------------------------------------
// LDS tile layouts.  One K slice is 64 deep.
//  k-contiguous operand ("KC"): [ROWS][64] bf16; 16-byte chunk c of row r sits
//    at chunk swz(r, c).  A lane reads its 8 k values with one 16-byte read.
//  k-major operand ("KN", stored n-contiguous in memory, e.g. a weight matrix
//    [K][N]): copied as is into [64][COLS]; chunk c of row k sits at
//    kn_swz(k, c).  A lane gathers 8 k values of one column with two
//    ds_read_b64_tr_b16 reads: in each group of 16 lanes, lane 4r+q addresses
//    row r, columns 4q..4q+3, and lane i receives column i of rows 0..3.
// ---------------------------------------------------------------------------
template <int COLS>
__device__ __forceinline__ int kn_swz(int k, int c) {
  return c ^ (((k & 3) << 2) & (COLS / 8 - 1));
}

// Buffer loads: the hardware returns zeros for a byte offset past num_records,
// so masked lanes get offset OOB and no lane branches around a load.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int OOB = (int)0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

// CPOL: cache-policy bits of the load (gfx950: 1 = sc0, 2 = nt, 16 = sc1).
template <int CPOL>
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, CPOL));
}

// Loader of a KC tile: row r of the tile is src[(row0 + r) * ld + k], rows
// r >= row_hi - row0 read as zeros.  With TWO, k < ksplit comes from s0 and
// k >= ksplit from s1 at k - ksplit (ksplit is a multiple of 64, so one K
// slice never straddles it).  The per-lane address state is kept once; the
// loaded data lives in a separate register array per pipeline stage.
template <int ROWS, bool TWO, int NT, int CPOL>
struct LoaderKC {
  static constexpr int CH = ROWS * 8;
  static constexpr int NR = (CH + NT - 1) / NT;
  struct Data { uint4 r[NR]; };
  int voff[NR];
  __amdgpu_buffer_rsrc_t rs0, rs1;
  int ksplit, k_lo, k_hi;
  __device__ __forceinline__ void init(const bf16_t* s0, const bf16_t* s1, int64_t ld, int row0,
                                       int row_hi, int k_lo_, int k_hi_, int ksplit_, int tid) {
    rs0 = make_rsrc(s0 + (int64_t)row0 * ld);
    rs1 = make_rsrc(TWO ? s1 + (int64_t)row0 * ld : s0);
    ksplit = ksplit_;
    k_lo = k_lo_;
    k_hi = k_hi_;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      int q = tid + NT * i;
      int row = q >> 3;
      bool ok = (CH % NT == 0 || q < CH) && row0 + row < row_hi;
      voff[i] = ok ? (int)(((int64_t)row * ld + (q & 7) * 8) * 2) : OOB;
    }
  }
  // K slice starting at k_lo + kofs
  __device__ __forceinline__ void load(Data& d, int kofs, int tid) const {
    int k0 = k_lo + kofs;
    __amdgpu_buffer_rsrc_t rs = rs0;
    int lim = k_hi - k0;
    if (TWO && k0 >= ksplit) { rs = rs1; k0 -= ksplit; lim = k_hi - ksplit - k0; }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int kc = ((tid + NT * i) & 7) * 8;
      d.r[i] = buf_load16<CPOL>(rs, kc < lim ? voff[i] : OOB, k0 * 2);
    }
  }
  __device__ __forceinline__ static void store(const Data& d, bf16_t* lds, int tid) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      int q = tid + NT * i;
      if (CH % NT == 0 || q < CH) {
        int row = q >> 3, c = q & 7;
        *reinterpret_cast<uint4*>(lds + row * BK + swz(row, c) * 8) = d.r[i];
      }
    }
  }
};

// Loader of a KN tile: element (k, c) of the tile is src[(k_lo + kofs + k) * ld
// + col0 + c]; rows at or past k_hi and columns at or past col_hi read as
// zeros.  HALF: tile columns [0, COLS/2) come from s0 at col0 + c, columns
// [COLS/2, COLS) from s1 at col0 + c - COLS/2 (the gate | up halves); each
// load instruction reads one half only, so its buffer descriptor is uniform.
template <int COLS, bool HALF, int NT, int CPOL>
struct LoaderKN {
  static constexpr int CPR = HALF ? COLS / 16 : COLS / 8;  // chunks per row and source
  static constexpr int CH = BK * CPR;                        // chunks per source
  static constexpr int NS = (CH + NT - 1) / NT;              // loads per source
  static constexpr int NR = HALF ? 2 * NS : NS;
  struct Data { uint4 r[NR]; };
  int voff[NS];
  __amdgpu_buffer_rsrc_t rs0, rs1;
  int64_t ld;
  int k_lo, k_hi;
  __device__ __forceinline__ void init(const bf16_t* s0, const bf16_t* s1, int64_t ld_, int col0,
                                       int col_hi, int k_lo_, int k_hi_, int, int tid) {
    ld = ld_;
    k_lo = k_lo_;
    k_hi = k_hi_;
    rs0 = make_rsrc(s0 + (int64_t)k_lo * ld + col0);
    rs1 = make_rsrc((HALF ? s1 : s0) + (int64_t)k_lo * ld + col0);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      int q = tid + NT * i;
      int col = (q % CPR) * 8;
      bool ok = (CH % NT == 0 || q < CH) && col0 + col < col_hi;
      voff[i] = ok ? (int)(((int64_t)(q / CPR) * ld + col) * 2) : OOB;
    }
  }
  __device__ __forceinline__ void load(Data& d, int kofs, int tid) const {
    const int lim = k_hi - k_lo - kofs;
    const int soff = (int)((int64_t)kofs * ld * 2);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int v = (tid + NT * i) / CPR < lim ? voff[i] : OOB;
      d.r[i] = buf_load16<CPOL>(rs0, v, soff);
      if (HALF) d.r[NS + i] = buf_load16<CPOL>(rs1, v, soff);
    }
  }
  __device__ __forceinline__ static void store(const Data& d, bf16_t* lds, int tid) {
#pragma unroll
    for (int h = 0; h < (HALF ? 2 : 1); ++h) {
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        int q = tid + NT * i;
        if (CH % NT == 0 || q < CH) {
          int k = q / CPR, c = q % CPR + h * CPR;
          *reinterpret_cast<uint4*>(lds + k * COLS + kn_swz<COLS>(k, c) * 8) = d.r[h * NS + i];
        }
      }
    }
  }
};

template <bool KC, int ROWS, bool TWO, int NT, int CPOL> struct PickLoader;
template <int ROWS, bool TWO, int NT, int CPOL> struct PickLoader<true, ROWS, TWO, NT, CPOL> { typedef LoaderKC<ROWS, TWO, NT, CPOL> type; };
template <int ROWS, bool TWO, int NT, int CPOL> struct PickLoader<false, ROWS, TWO, NT, CPOL> { typedef LoaderKN<ROWS, TWO, NT, CPOL> type; };

// MFMA operand fragment (32 rows x 16 k): lane l holds row base + (l & 31),
// k = 16 ks + 8 (l >> 5) + 0..7.
__device__ __forceinline__ bf16x8 frag_kc(const bf16_t* lds, int base, int ks, int lane) {
  const int row = base + (lane & 31);
  const int c = ks * 2 + (lane >> 5);
  return *reinterpret_cast<const bf16x8*>(lds + row * BK + swz(row, c) * 8);
}

template <int COLS>
__device__ __forceinline__ bf16x8 frag_kn(const bf16_t* lds, int base, int ks, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int col = base + ((g & 1) << 4) + ((j & 3) << 2);
  const int k = ks * 16 + ((g >> 1) << 3) + (j >> 2);
  const int off = k * COLS + kn_swz<COLS>(k, col >> 3) * 8 + (col & 7);  // k+4: same swizzle
  v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds + off));
  v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds + off + 4 * COLS));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Epilogue shared by the bf16 kernels.  Lane holds C[m][n..n+3] of every
// 32x32 block of its wave tile: m = row (lane & 31), n = 8q + 4 (lane >> 5).
template <int FM, int FN, int WTM, int WTN, int GMD, int EPI>
__device__ __forceinline__ void epilogue(const GemmParams& p, f32x16 (&acc)[FM][FN], int m_lo,
                                         int m_hi, int n0, int e, int wm, int wn, int lane) {
  const int half = lane >> 5;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m_lo + wm * WTM + i * 32 + (lane & 31);
    if (m >= m_hi) continue;
    if constexpr (EPI == EPI_SWIGLU) {
      bf16_t* H = static_cast<bf16_t*>(p.C0);
      bf16_t* Aout = static_cast<bf16_t*>(p.C2);
      const int64_t I = p.I;
#pragma unroll
      for (int jp = 0; jp < FN / 2; ++jp) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn * (WTN / 2) + jp * 32 + 8 * q + 4 * half;
          if (n >= I) continue;
          float g[4], u[4], a[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            g[s] = acc[i][jp][4 * q + s];
            u[s] = acc[i][jp + FN / 2][4 * q + s];
            a[s] = g[s] * __builtin_amdgcn_rcpf(1.0f + __expf(-g[s])) * u[s];
          }
          if (H) {
            *reinterpret_cast<uint2*>(H + m * 2 * I + n) = make_uint2(pack_bf2(g[0], g[1]), pack_bf2(g[2], g[3]));
            *reinterpret_cast<uint2*>(H + m * 2 * I + I + n) = make_uint2(pack_bf2(u[0], u[1]), pack_bf2(u[2], u[3]));
          }
          *reinterpret_cast<uint2*>(Aout + m * I + n) = make_uint2(pack_bf2(a[0], a[1]), pack_bf2(a[2], a[3]));
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          int n = n0 + wn * WTN + j * 32 + 8 * q + 4 * half;
          if (n >= p.N) continue;
          float v[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) v[s] = acc[i][j][4 * q + s];
          if constexpr (EPI == EPI_STORE) {
            bf16_t* C = static_cast<bf16_t*>(p.C0);
            if (p.n_split > 0 && n >= p.n_split) { C = static_cast<bf16_t*>(p.C1); n -= p.n_split; }
            if (GMD == G_KROWS) C += (int64_t)e * p.c_estride;
            *reinterpret_cast<uint2*>(C + (int64_t)m * p.ldc + n) =
                make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
          } else if constexpr (EPI == EPI_ACCUM) {
            bf16_t* C = static_cast<bf16_t*>(p.C0) + (int64_t)m * p.ldc + n;
            uint2 o = *reinterpret_cast<const uint2*>(C);
            float w0 = bf2f((bf16_t)(o.x & 0xffff)) + v[0], w1 = bf2f((bf16_t)(o.x >> 16)) + v[1];
            float w2 = bf2f((bf16_t)(o.y & 0xffff)) + v[2], w3 = bf2f((bf16_t)(o.y >> 16)) + v[3];
            *reinterpret_cast<uint2*>(C) = make_uint2(pack_bf2(w0, w1), pack_bf2(w2, w3));
          } else if constexpr (EPI == EPI_F32_BIAS) {
            float* C = static_cast<float*>(p.C0) + (int64_t)m * p.ldc + n;
            if (p.bias) {
#pragma unroll
              for (int s = 0; s < 4; ++s) v[s] += p.bias[n + s];
            }
            *reinterpret_cast<float4*>(C) = make_float4(v[0], v[1], v[2], v[3]);
          } else if constexpr (EPI == EPI_DSWIGLU) {
            const bf16_t* H = static_cast<const bf16_t*>(p.aux);
            bf16_t* dH = static_cast<bf16_t*>(p.C0);
            const int64_t I = p.I;
            uint2 hg = *reinterpret_cast<const uint2*>(H + (int64_t)m * 2 * I + n);
            uint2 hu = *reinterpret_cast<const uint2*>(H + (int64_t)m * 2 * I + I + n);
            float g[4] = {bf2f((bf16_t)(hg.x & 0xffff)), bf2f((bf16_t)(hg.x >> 16)),
                          bf2f((bf16_t)(hg.y & 0xffff)), bf2f((bf16_t)(hg.y >> 16))};
            float u[4] = {bf2f((bf16_t)(hu.x & 0xffff)), bf2f((bf16_t)(hu.x >> 16)),
                          bf2f((bf16_t)(hu.y & 0xffff)), bf2f((bf16_t)(hu.y >> 16))};
            float dg[4], du[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-g[s]));
              dg[s] = v[s] * u[s] * sg * (1.0f + g[s] * (1.0f - sg));
              du[s] = v[s] * g[s] * sg;
            }
            *reinterpret_cast<uint2*>(dH + (int64_t)m * 2 * I + n) =
                make_uint2(pack_bf2(dg[0], dg[1]), pack_bf2(dg[2], dg[3]));
            *reinterpret_cast<uint2*>(dH + (int64_t)m * 2 * I + I + n) =
                make_uint2(pack_bf2(du[0], du[1]), pack_bf2(du[2], du[3]));
          }
        }
      }
    }
  }
}

// Plain-store epilogue staged through LDS: the wave tiles are written to LDS
// as bf16, then every store instruction writes whole 16-byte chunks of
// consecutive columns (full cache lines per row) instead of 8-byte pieces
// scattered over 32 rows.  16-byte chunk c of LDS row r sits at c ^ (r & 15).
template <int BM, int BN, int FM, int FN, int WTM, int WTN, int NT, int GMD>
__device__ __forceinline__ void epilogue_store_staged(const GemmParams& p, f32x16 (&acc)[FM][FN],
                                                      bf16_t* lds, int m_lo, int m_hi, int n0,
                                                      int e, int wm, int wn, int lane, int tid) {
  constexpr int CPR = BN / 8;  // 16-byte chunks per tile row
  static_assert(CPR >= 16, "swizzle needs 16 chunks per row");
  const int half = lane >> 5;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = wm * WTM + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = wn * WTN + j * 32 + 8 * q + 4 * half;
        const int c = (n >> 3) ^ (r & 15);
        *reinterpret_cast<uint2*>(lds + r * BN + c * 8 + (n & 7)) =
            make_uint2(pack_bf2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                       pack_bf2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
      }
    }
  }
  __syncthreads();
  bf16_t* C0 = static_cast<bf16_t*>(p.C0);
  bf16_t* C1 = static_cast<bf16_t*>(p.C1);
  if (GMD == G_KROWS) {
    C0 += (int64_t)e * p.c_estride;
    if (C1) C1 += (int64_t)e * p.c_estride;
  }
#pragma unroll
  for (int q0 = 0; q0 < BM * CPR; q0 += NT) {
    const int q = q0 + tid;
    const int r = q / CPR, c = q % CPR;
    const int m = m_lo + r;
    int n = n0 + c * 8;
    if (m < m_hi && n < p.N) {
      bf16_t* C = C0;
      if (p.n_split > 0 && n >= p.n_split) { C = C1; n -= p.n_split; }
      *reinterpret_cast<uint4*>(C + (int64_t)m * p.ldc + n) =
          *reinterpret_cast<const uint4*>(lds + r * BN + (c ^ (r & 15)) * 8);
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA grouped GEMM.  WGM x WGN waves, each owning a (BM/WGM) x
// (BN/WGN) block of 32x32 MFMA tiles.  P register stages: while the
// MFMAs work on K slice kt from LDS, slice kt+1 is written to the other LDS
// buffer and the loads of slices kt+2 .. kt+P are in flight.
// With the gate|up halves (B2_NHALF) the first FN/2 column blocks of a wave
// are gate columns and the last FN/2 the matching up columns.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WGM, int WGN, int P, int AM, int BMD, int GMD, int B2, int EPI, int ROLE>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_bf16_kernel(GemmParams p) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(FM >= 1 && FN >= 1, "wave tile of at least 32x32");
  static_assert(B2 != B2_NHALF || FN % 2 == 0, "gate|up halves need an even block count");
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * (BM + BN) * BK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  // ---- which tile
  int mt_count = (GMD == G_MROWS) ? p.tiles[0] : p.m_tiles;
  int per_group = mt_count * p.n_tiles;
  int count = (GMD == G_KROWS) ? per_group * p.groups : per_group;
  if ((int)blockIdx.x >= count) return;
  int L = remap_xcd(blockIdx.x, count);
  int e = 0;
  if (GMD == G_KROWS) { e = L / per_group; L -= e * per_group; }
  int mt, nt;
  group_order(L, mt_count, p.n_tiles, mt, nt);
  int m_lo, m_hi, k_lo, k_hi;
  if (GMD == G_MROWS) {
    e = p.tiles[1 + 2 * mt];
    m_lo = p.tiles[2 + 2 * mt];
    m_hi = min(m_lo + BM, p.off[e + 1]);
    k_lo = 0;
    k_hi = p.K;
  } else {
    m_lo = mt * BM;
    m_hi = min(m_lo + BM, p.M);
    if (GMD == G_KROWS && p.off) { k_lo = p.off[e]; k_hi = p.off[e + 1]; }
    else { k_lo = 0; k_hi = p.K; }
  }
  const int n0 = nt * ((B2 == B2_NHALF) ? BN / 2 : BN);
  const int n_hi = p.N;  // column bound in the B source's column space

  const bf16_t* A = static_cast<const bf16_t*>(p.A);
  const bf16_t* B0 = static_cast<const bf16_t*>(p.B0);
  const bf16_t* B1 = static_cast<const bf16_t*>(p.B1);
  if (GMD == G_MROWS) {
    B0 += (int64_t)e * p.b_estride;
    if (B2 != B2_NONE) B1 += (int64_t)e * p.b_estride;
  }

#ifndef MOE_WEIGHT_CPOL
#define MOE_WEIGHT_CPOL 2
#endif
  // expert weights (B of the row-grouped GEMMs) stream through once; the
  // activation rows (A) are re-read by every column tile of the expert
  constexpr int BPOL = GMD == G_MROWS ? MOE_WEIGHT_CPOL : 0;
  typedef typename PickLoader<AM == A_KC, BM, false, NT, 0>::type LA;
  typedef typename PickLoader<BMD == B_KC, BN, B2 != B2_NONE, NT, BPOL>::type LB;
  LA la;
  LB lb;
  typename LA::Data da[P];
  typename LB::Data db[P];
  la.init(A, A, p.lda, m_lo, m_hi, k_lo, k_hi, 0, tid);
  lb.init(B0, B1, p.ldb, n0, n_hi, k_lo, k_hi, p.k_split, tid);

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (k_hi - k_lo + BK - 1) / BK;
#pragma unroll
  for (int s = 0; s < P; ++s) {
    if (s < nk) {
      la.load(da[s], s * BK, tid);
      lb.load(db[s], s * BK, tid);
    }
  }
  if (nk > 0) {
    LA::store(da[0], smem, tid);
    LB::store(db[0], smem + BM * BK, tid);
  }
  __syncthreads();

  // One K slice: refill the register slot of slice kt with slice kt+P, multiply
  // slice kt from LDS, write slice kt+1 (loaded P-1 slices ago) to the other
  // LDS buffer, barrier.  U = kt mod P is a compile-time constant.
  auto step = [&](auto Uc, int kt, bool do_load, bool do_store) __attribute__((always_inline)) {
    constexpr int U = decltype(Uc)::value;
    if (do_load) {
      la.load(da[U], (kt + P) * BK, tid);
      lb.load(db[U], (kt + P) * BK, tid);
    }
    // keep the refill loads at the top of the step: the scheduler would
    // otherwise sink them below the MFMAs and expose their latency
    __builtin_amdgcn_sched_barrier(0);
    const bf16_t* as = smem + (kt & 1) * (BM + BN) * BK;
    const bf16_t* bs = as + BM * BK;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[FM], bfg[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int base = wm * WTM + i * 32;
        if constexpr (AM == A_KC) af[i] = frag_kc(as, base, ks, lane);
        else af[i] = frag_kn<BM>(as, base, ks, lane);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        int base;
        if constexpr (B2 == B2_NHALF)
          base = (j < FN / 2) ? (wn * (WTN / 2) + j * 32) : (BN / 2 + wn * (WTN / 2) + (j - FN / 2) * 32);
        else
          base = wn * WTN + j * 32;
        if constexpr (BMD == B_KC) bfg[j] = frag_kc(bs, base, ks, lane);
        else bfg[j] = frag_kn<BN>(bs, base, ks, lane);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfg[j], af[i], acc[i][j], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (do_store) {
      bf16_t* nxt = smem + ((kt + 1) & 1) * (BM + BN) * BK;
      LA::store(da[(U + 1) % P], nxt, tid);
      LB::store(db[(U + 1) % P], nxt + BM * BK, tid);
    }
    __syncthreads();
  };

  int kt0 = 0;
  // steady state: every step loads and stores
  for (; kt0 + 2 * P <= nk; kt0 += P) {
    [&]<int... Us>(std::integer_sequence<int, Us...>) __attribute__((always_inline)) {
      (step(std::integral_constant<int, Us>{}, kt0 + Us, true, true), ...);
    }(std::make_integer_sequence<int, P>{});
  }
  // drain: at most 2P-1 slices left
  [&]<int... Us>(std::integer_sequence<int, Us...>) __attribute__((always_inline)) {
    ((kt0 + Us < nk ? step(std::integral_constant<int, Us % P>{}, kt0 + Us, kt0 + Us + P < nk,
                           kt0 + Us + 1 < nk)
                    : void()),
     ...);
  }(std::make_integer_sequence<int, 2 * P - 1>{});

#ifndef MOE_STAGED_STORE
#define MOE_STAGED_STORE 1
#endif
  if constexpr (EPI == EPI_STORE && MOE_STAGED_STORE && BN / 8 >= 16 && BM * BN <= (BM + BN) * BK * 2)
    epilogue_store_staged<BM, BN, FM, FN, WTM, WTN, NT, GMD>(p, acc, smem, m_lo, m_hi, n0, e, wm,
                                                             wn, lane, tid);
  else
    epilogue<FM, FN, WTM, WTN, GMD, EPI>(p, acc, m_lo, m_hi, n0, e, wm, wn, lane);
}

// ===========================================================================
// Direct-to-LDS variant.  Every K slice goes from HBM/L2 straight into LDS
// with the 16-byte buffer-load-to-LDS instruction (no register staging, no
// LDS store instructions).  Lane l of a load lands at LDS base + 16 l, so the
// swizzled layouts are produced by choosing each lane's source address.  Each
// pipeline stage is a separate __shared__ array so the compiler can tell that
// fragment reads of one stage do not alias loads into another.
// ===========================================================================
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, bf16_t* lds_dst, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)lds_dst, 16, voff, soff, 0, 0);
}

// KC tile [ROWS][64]: slot s (16 bytes) holds row s >> 3, physical chunk s & 7,
// i.e. logical chunk (s & 7) ^ swz(row).
template <int ROWS, bool TWO, int NT>
struct DmaKC {
  static constexpr int CH = ROWS * 8;
  static constexpr int NR = CH / NT;
  static_assert(CH % NT == 0, "whole load instructions");
  int voff[NR];
  int kcol[NR];
  __amdgpu_buffer_rsrc_t rs0, rs1;
  int ksplit, k_lo, k_hi;
  __device__ __forceinline__ void init(const bf16_t* s0, const bf16_t* s1, int64_t ld, int row0,
                                       int row_hi, int k_lo_, int k_hi_, int ksplit_, int tid) {
    rs0 = make_rsrc(s0 + (int64_t)row0 * ld);
    rs1 = make_rsrc(TWO ? s1 + (int64_t)row0 * ld : s0);
    ksplit = ksplit_;
    k_lo = k_lo_;
    k_hi = k_hi_;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int slot = tid + NT * i;
      const int row = slot >> 3;
      const int c = (slot & 7) ^ (row & 7) ^ ((row >> 3) & 1);  // inverse of swz
      kcol[i] = c * 8;
      voff[i] = row0 + row < row_hi ? (int)(((int64_t)row * ld + c * 8) * 2) : OOB;
    }
  }
  __device__ __forceinline__ void issue(bf16_t* tile, int kofs, int tid) const {
    int k0 = k_lo + kofs;
    __amdgpu_buffer_rsrc_t rs = rs0;
    int lim = k_hi - k0;
    if (TWO && k0 >= ksplit) { rs = rs1; k0 -= ksplit; lim = k_hi - ksplit - k0; }
    bf16_t* dst = tile + (tid >> 6) * 64 * 8;
#pragma unroll
    for (int i = 0; i < NR; ++i) dma16(rs, dst + i * NT * 8, kcol[i] < lim ? voff[i] : OOB, k0 * 2);
  }
};

// KN tile [64][COLS] (HALF: two sub-tiles [64][COLS/2], gate then up): slot s
// of a (sub-)tile of width W holds row s / (W/8), physical chunk s % (W/8).
template <int COLS, bool HALF, int NT>
struct DmaKN {
  static constexpr int W = HALF ? COLS / 2 : COLS;  // width of one (sub-)tile
  static constexpr int CPR = W / 8;
  static constexpr int CH = BK * CPR;
  static constexpr int NR = CH / NT;
  static_assert(CH % NT == 0, "whole load instructions");
  int voff[NR];
  int krow[NR];
  __amdgpu_buffer_rsrc_t rs0, rs1;
  int64_t ld;
  int k_lo, k_hi;
  __device__ __forceinline__ void init(const bf16_t* s0, const bf16_t* s1, int64_t ld_, int col0,
                                       int col_hi, int k_lo_, int k_hi_, int, int tid) {
    ld = ld_;
    k_lo = k_lo_;
    k_hi = k_hi_;
    rs0 = make_rsrc(s0 + (int64_t)k_lo * ld + col0);
    rs1 = make_rsrc((HALF ? s1 : s0) + (int64_t)k_lo * ld + col0);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int slot = tid + NT * i;
      const int k = slot / CPR;
      const int col = kn_swz<W>(k, slot % CPR) * 8;  // the swizzle is its own inverse
      krow[i] = k;
      voff[i] = col0 + col < col_hi ? (int)(((int64_t)k * ld + col) * 2) : OOB;
    }
  }
  __device__ __forceinline__ void issue(bf16_t* tile, int kofs, int tid) const {
    const int lim = k_hi - k_lo - kofs;
    const int soff = (int)((int64_t)kofs * ld * 2);
    bf16_t* dst = tile + (tid >> 6) * 64 * 8;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int v = krow[i] < lim ? voff[i] : OOB;
      dma16(rs0, dst + i * NT * 8, v, soff);
      if (HALF) dma16(rs1, dst + BK * W + i * NT * 8, v, soff);
    }
  }
};

template <bool KC, int ROWS, bool TWO, int NT> struct PickDma;
template <int ROWS, bool TWO, int NT> struct PickDma<true, ROWS, TWO, NT> { typedef DmaKC<ROWS, TWO, NT> type; };
template <int ROWS, bool TWO, int NT> struct PickDma<false, ROWS, TWO, NT> { typedef DmaKN<ROWS, TWO, NT> type; };

// s_waitcnt vmcnt(N), leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int BM, int BN, int WGM, int WGN, int S, int AM, int BMD, int GMD, int B2, int EPI, int ROLE>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_bf16_dma_kernel(GemmParams p) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int SZ = (BM + BN) * BK;  // elements per stage
  static_assert(FM >= 1 && FN >= 1, "wave tile of at least 32x32");
  static_assert(B2 != B2_NHALF || FN % 2 == 0, "gate|up halves need an even block count");
  static_assert(S == 2 || S == 3, "two or three LDS stages");
  __shared__ __attribute__((aligned(16))) bf16_t st0[SZ];
  __shared__ __attribute__((aligned(16))) bf16_t st1[SZ];
  __shared__ __attribute__((aligned(16))) bf16_t st2[S > 2 ? SZ : 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  // ---- which tile
  int mt_count = (GMD == G_MROWS) ? p.tiles[0] : p.m_tiles;
  int per_group = mt_count * p.n_tiles;
  int count = (GMD == G_KROWS) ? per_group * p.groups : per_group;
  if ((int)blockIdx.x >= count) return;
  int L = remap_xcd(blockIdx.x, count);
  int e = 0;
  if (GMD == G_KROWS) { e = L / per_group; L -= e * per_group; }
  int mt, nt;
  group_order(L, mt_count, p.n_tiles, mt, nt);
  int m_lo, m_hi, k_lo, k_hi;
  if (GMD == G_MROWS) {
    e = p.tiles[1 + 2 * mt];
    m_lo = p.tiles[2 + 2 * mt];
    m_hi = min(m_lo + BM, p.off[e + 1]);
    k_lo = 0;
    k_hi = p.K;
  } else {
    m_lo = mt * BM;
    m_hi = min(m_lo + BM, p.M);
    if (GMD == G_KROWS && p.off) { k_lo = p.off[e]; k_hi = p.off[e + 1]; }
    else { k_lo = 0; k_hi = p.K; }
  }
  const int n0 = nt * ((B2 == B2_NHALF) ? BN / 2 : BN);
  const int n_hi = p.N;

  const bf16_t* A = static_cast<const bf16_t*>(p.A);
  const bf16_t* B0 = static_cast<const bf16_t*>(p.B0);
  const bf16_t* B1 = static_cast<const bf16_t*>(p.B1);
  if (GMD == G_MROWS) {
    B0 += (int64_t)e * p.b_estride;
    if (B2 != B2_NONE) B1 += (int64_t)e * p.b_estride;
  }

  typedef typename PickDma<AM == A_KC, BM, false, NT>::type LA;
  typedef typename PickDma<BMD == B_KC, BN, B2 != B2_NONE, NT>::type LB;
  constexpr int LPS = LA::NR + LB::NR * ((B2 == B2_NHALF) ? 2 : 1);  // loads per thread per stage
  LA la;
  LB lb;
  la.init(A, A, p.lda, m_lo, m_hi, k_lo, k_hi, 0, tid);
  lb.init(B0, B1, p.ldb, n0, n_hi, k_lo, k_hi, p.k_split, tid);

  auto buf = [&](auto Ic) __attribute__((always_inline)) -> bf16_t* {
    constexpr int I = decltype(Ic)::value;
    if constexpr (I == 0) return st0;
    else if constexpr (I == 1) return st1;
    else return st2;
  };
  auto issue = [&](bf16_t* b, int s) __attribute__((always_inline)) {
    la.issue(b, s * BK, tid);
    lb.issue(b + BM * BK, s * BK, tid);
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (k_hi - k_lo + BK - 1) / BK;
  if (nk > 0) issue(st0, 0);
  if (S > 2 && nk > 1) {
    issue(st1, 1);
    wait_vmcnt<LPS>();  // slice 0 landed, slice 1 may still be in flight
  } else {
    wait_vmcnt<0>();
  }
  __syncthreads();

  // Fragment reads of operands in the k-major layout use the LDS transpose
  // read, which the compiler cannot tie to one stage buffer: it would wait for
  // every load in flight before such a read.  So a step reads all of them
  // first, then issues the next slice's loads, then runs the MFMAs (with the
  // plain reads of k-contiguous operands interleaved).
  constexpr bool A_TR = AM != A_KC, B_TR = BMD != B_KC;
  auto step = [&](auto Uc, int kt) __attribute__((always_inline)) {
    constexpr int U = decltype(Uc)::value;
    const bf16_t* as = buf(std::integral_constant<int, U>{});
    const bf16_t* bs = as + BM * BK;
    auto a_frag = [&](int i, int ks) __attribute__((always_inline)) -> bf16x8 {
      const int base = wm * WTM + i * 32;
      if constexpr (AM == A_KC) return frag_kc(as, base, ks, lane);
      else return frag_kn<BM>(as, base, ks, lane);
    };
    auto b_frag = [&](int j, int ks) __attribute__((always_inline)) -> bf16x8 {
      if constexpr (B2 == B2_NHALF) {
        const int h = j < FN / 2 ? 0 : 1;
        const int base = wn * (WTN / 2) + (j - h * (FN / 2)) * 32;
        return frag_kn<BN / 2>(bs + h * BK * (BN / 2), base, ks, lane);
      } else {
        const int base = wn * WTN + j * 32;
        if constexpr (BMD == B_KC) return frag_kc(bs, base, ks, lane);
        else return frag_kn<BN>(bs, base, ks, lane);
      }
    };
    bf16x8 apre[A_TR ? BK / 16 : 1][A_TR ? FM : 1];
    bf16x8 bpre[B_TR ? BK / 16 : 1][B_TR ? FN : 1];
    if constexpr (A_TR) {
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
        for (int i = 0; i < FM; ++i) apre[ks][i] = a_frag(i, ks);
    }
    if constexpr (B_TR) {
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
        for (int j = 0; j < FN; ++j) bpre[ks][j] = b_frag(j, ks);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (kt + S - 1 < nk) issue(buf(std::integral_constant<int, (U + S - 1) % S>{}), kt + S - 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[FM], bfg[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = A_TR ? apre[A_TR ? ks : 0][A_TR ? i : 0] : a_frag(i, ks);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfg[j] = B_TR ? bpre[B_TR ? ks : 0][B_TR ? j : 0] : b_frag(j, ks);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfg[j], af[i], acc[i][j], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < nk) {
      // slice kt+1 must have landed; slices after it may stay in flight
      if (S > 2 && kt + 2 < nk) wait_vmcnt<LPS>();
      else wait_vmcnt<0>();
      __syncthreads();
    }
  };

  int kt0 = 0;
  for (; kt0 + S <= nk; kt0 += S) {
    [&]<int... Us>(std::integer_sequence<int, Us...>) __attribute__((always_inline)) {
      (step(std::integral_constant<int, Us>{}, kt0 + Us), ...);
    }(std::make_integer_sequence<int, S>{});
  }
  [&]<int... Us>(std::integer_sequence<int, Us...>) __attribute__((always_inline)) {
    ((kt0 + Us < nk ? step(std::integral_constant<int, Us>{}, kt0 + Us) : void()), ...);
  }(std::make_integer_sequence<int, S - 1>{});

  epilogue<FM, FN, WTM, WTN, GMD, EPI>(p, acc, m_lo, m_hi, n0, e, wm, wn, lane);
}

// ---------------------------------------------------------------------------
// fp32 kernel: one output (or one gate/up pair) per thread, fp32 FMA.
// ---------------------------------------------------------------------------
template <int AM, int BMD, int GMD, int B2, int EPI, int ROLE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParams p) {
  const int n = blockIdx.x * 16 + (threadIdx.x & 15);
  const int m = blockIdx.y * 16 + (threadIdx.x >> 4);
  const float* A = static_cast<const float*>(p.A);
  const float* B0 = static_cast<const float*>(p.B0);
  const float* B1 = static_cast<const float*>(p.B1);
  int e = 0, k_lo = 0, k_hi = p.K;
  const int ncols = (EPI == EPI_SWIGLU || EPI == EPI_DSWIGLU) ? p.I : p.N;
  if (n >= ncols) return;
  if (GMD == G_MROWS) {
    if (m >= p.off[p.groups]) return;
    int lo = 0, hi = p.groups - 1;  // last e with off[e] <= m
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (p.off[mid] <= m) lo = mid; else hi = mid - 1;
    }
    e = lo;
    B0 += (int64_t)e * p.b_estride;
    if (B2 != B2_NONE) B1 += (int64_t)e * p.b_estride;
  } else {
    if (m >= p.M) return;
    if (GMD == G_KROWS) {
      e = blockIdx.z;
      if (p.off) { k_lo = p.off[e]; k_hi = p.off[e + 1]; }
    }
  }
  auto a_at = [&](int k) -> float {
    return AM == A_KC ? A[(int64_t)m * p.lda + k] : A[(int64_t)k * p.lda + m];
  };
  auto b_at = [&](const float* B, int k, int col) -> float {
    return BMD == B_NC ? B[(int64_t)k * p.ldb + col] : B[(int64_t)col * p.ldb + k];
  };
  float acc = 0.f, acc2 = 0.f;
  for (int k = k_lo; k < k_hi; ++k) {
    float a = a_at(k);
    if (B2 == B2_NHALF) {
      acc = fmaf(a, b_at(B0, k, n), acc);
      acc2 = fmaf(a, b_at(B1, k, n), acc2);
    } else if (B2 == B2_KSPLIT) {
      acc = fmaf(a, k < p.k_split ? b_at(B0, k, n) : b_at(B1, k - p.k_split, n), acc);
    } else {
      acc = fmaf(a, b_at(B0, k, n), acc);
    }
  }
  if constexpr (EPI == EPI_STORE) {
    float* C = static_cast<float*>(p.C0);
    int nn = n;
    if (p.n_split > 0 && nn >= p.n_split) { C = static_cast<float*>(p.C1); nn -= p.n_split; }
    if (GMD == G_KROWS) C += (int64_t)e * p.c_estride;
    C[(int64_t)m * p.ldc + nn] = acc;
  } else if constexpr (EPI == EPI_ACCUM) {
    static_cast<float*>(p.C0)[(int64_t)m * p.ldc + n] += acc;
  } else if constexpr (EPI == EPI_F32_BIAS) {
    static_cast<float*>(p.C0)[(int64_t)m * p.ldc + n] = acc + (p.bias ? p.bias[n] : 0.f);
  } else if constexpr (EPI == EPI_SWIGLU) {
    const int64_t I = p.I;
    float* H = static_cast<float*>(p.C0);
    if (H) { H[m * 2 * I + n] = acc; H[m * 2 * I + I + n] = acc2; }
    static_cast<float*>(p.C2)[m * I + n] = acc / (1.0f + expf(-acc)) * acc2;
  } else if constexpr (EPI == EPI_DSWIGLU) {
    const int64_t I = p.I;
    const float* H = static_cast<const float*>(p.aux);
    float g = H[m * 2 * I + n], u = H[m * 2 * I + I + n];
    float sg = 1.0f / (1.0f + expf(-g));
    float* dH = static_cast<float*>(p.C0);
    dH[m * 2 * I + n] = acc * u * sg * (1.0f + g * (1.0f - sg));
    dH[m * 2 * I + I + n] = acc * g * sg;
  }
}

// ---------------------------------------------------------------------------
// Tile table for row-grouped GEMMs.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void tile_table_kernel(const int32_t* off, int groups, int bm,
                                                          int32_t* tiles) {
  __shared__ int32_t scan[1024];
  __shared__ int32_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < groups; base += 1024) {
    int e = base + threadIdx.x;
    int cnt = 0, o = 0;
    if (e < groups) {
      o = off[e];
      cnt = (off[e + 1] - o + bm - 1) / bm;
    }
    scan[threadIdx.x] = cnt;
    __syncthreads();
    for (int s = 1; s < 1024; s <<= 1) {  // inclusive Hillis-Steele scan
      int v = threadIdx.x >= s ? scan[threadIdx.x - s] : 0;
      __syncthreads();
      scan[threadIdx.x] += v;
      __syncthreads();
    }
    int first = carry + scan[threadIdx.x] - cnt;
    for (int t = 0; t < cnt; ++t) {
      tiles[1 + 2 * (first + t)] = e;
      tiles[2 + 2 * (first + t)] = o + t * bm;
    }
    __syncthreads();
    if (threadIdx.x == 1023) carry += scan[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) tiles[0] = carry;
}

moe_status_t launch_tile_table(const int32_t* off, int groups, int bm, int32_t* tiles,
                               hipStream_t s) {
  ProfScope prof("tile_table", s);
  tile_table_kernel<<<1, 1024, 0, s>>>(off, groups, bm, tiles);
  return check_launch("tile_table_kernel");
}

int tile_bm(TileCfg cfg) { return cfg == TILE_64x64 ? 64 : cfg == TILE_128x128 ? 128 : 256; }
int tile_bn(TileCfg cfg) {
  return cfg == TILE_256x256 ? 256 : (cfg == TILE_256x128 || cfg == TILE_128x128) ? 128 : 64;
}

// ---------------------------------------------------------------------------
// Dispatch
// ---------------------------------------------------------------------------
// Tile shape of each expert GEMM (build-time tunable).
#ifndef MOE_TILE_GATEUP_FWD
#define MOE_TILE_GATEUP_FWD TILE_256x256
#endif
#ifndef MOE_TILE_DOWN_FWD
#define MOE_TILE_DOWN_FWD TILE_256x256
#endif
#ifndef MOE_TILE_DOWN_DGRAD
#define MOE_TILE_DOWN_DGRAD TILE_256x128
#endif
#ifndef MOE_TILE_GATEUP_DGRAD
#define MOE_TILE_GATEUP_DGRAD TILE_256x256
#endif
#ifndef MOE_WGRAD_TILE
#define MOE_WGRAD_TILE TILE_128x128
#endif
#ifndef MOE_GEMM_STAGES
#define MOE_GEMM_STAGES 2
#endif
#ifndef MOE_WIDE_WAVES
#define MOE_WIDE_WAVES 8
#endif
#ifndef MOE_GEMM_DMA
#define MOE_GEMM_DMA 0
#endif

// role, name, tile, A layout, B layout, grouping, two-source B, epilogue
#define MOE_GEMM_ROLES(X)                                                                          \
  X(R_ROUTE_LOGITS, "route_logits", TILE_64x64, A_KC, B_NC, G_DENSE, B2_NONE, EPI_F32_BIAS)        \
  X(R_GATEUP_FWD, "ffn_gateup_fwd", MOE_TILE_GATEUP_FWD, A_KC, B_NC, G_MROWS, B2_NHALF, EPI_SWIGLU) \
  X(R_DOWN_FWD, "ffn_down_fwd", MOE_TILE_DOWN_FWD, A_KC, B_NC, G_MROWS, B2_NONE, EPI_STORE)         \
  X(R_DOWN_DGRAD, "ffn_down_dgrad", MOE_TILE_DOWN_DGRAD, A_KC, B_KC, G_MROWS, B2_NONE, EPI_DSWIGLU) \
  X(R_GATEUP_DGRAD, "ffn_gateup_dgrad", MOE_TILE_GATEUP_DGRAD, A_KC, B_KC, G_MROWS, B2_KSPLIT,      \
    EPI_STORE)                                                                                     \
  X(R_DOWN_WGRAD, "ffn_down_wgrad", MOE_WGRAD_TILE, A_MC, B_NC, G_KROWS, B2_NONE, EPI_STORE)        \
  X(R_GATEUP_WGRAD, "ffn_gateup_wgrad", MOE_WGRAD_TILE, A_MC, B_NC, G_KROWS, B2_NONE, EPI_STORE)    \
  X(R_ROUTE_DW, "route_bwd_dw", TILE_64x64, A_MC, B_NC, G_KROWS, B2_NONE, EPI_STORE)               \
  X(R_ROUTE_DX, "route_bwd_dx", TILE_64x64, A_KC, B_KC, G_DENSE, B2_NONE, EPI_ACCUM)

TileCfg role_tile(GemmRole role) {
  switch (role) {
#define X(r, n, t, a, b, g, t2, e) \
  case r: return t;
    MOE_GEMM_ROLES(X)
#undef X
  }
  return TILE_64x64;
}

const char* role_name(GemmRole role) {
  switch (role) {
#define X(r, n, t, a, b, g, t2, e) \
  case r: return n;
    MOE_GEMM_ROLES(X)
#undef X
  }
  return "gemm";
}

template <int CFG> struct TileDims;
template <> struct TileDims<TILE_256x256> { static constexpr int BM = 256, BN = 256; };
template <> struct TileDims<TILE_256x128> { static constexpr int BM = 256, BN = 128; };
template <> struct TileDims<TILE_128x128> { static constexpr int BM = 128, BN = 128; };
template <> struct TileDims<TILE_64x64> { static constexpr int BM = 64, BN = 64; };

template <int CFG, int AM, int BMD, int GMD, int B2, int EPI, int ROLE>
static void launch_bf16(const GemmParams& p, int grid, hipStream_t s) {
  constexpr int BMt = TileDims<CFG>::BM, BNt = TileDims<CFG>::BN;
  constexpr int P = (BMt >= 128) ? MOE_GEMM_STAGES : 2;  // register stages in flight
  // 256x256 tiles: MOE_WIDE_WAVES = 8 runs two waves per SIMD (2 x 4 grid)
  constexpr int WGN = (BMt == 256 && BNt == 256 && MOE_WIDE_WAVES == 8) ? 4 : 2;
  if constexpr (MOE_GEMM_DMA) {
    constexpr int S = ((BMt + BNt) * BK * 2 * 3 <= 160 * 1024 && !(BMt == 128 && BNt == 128)) ? 3 : 2;
    gemm_bf16_dma_kernel<BMt, BNt, 2, WGN, S, AM, BMD, GMD, B2, EPI, ROLE>
        <<<grid, 64 * 2 * WGN, 0, s>>>(p);
  } else {
    gemm_bf16_kernel<BMt, BNt, 2, WGN, P, AM, BMD, GMD, B2, EPI, ROLE><<<grid, 64 * 2 * WGN, 0, s>>>(p);
  }
}

template <int AM, int BMD, int GMD, int B2, int EPI, int ROLE>
static void launch_f32(const GemmParams& p, int max_rows, hipStream_t s) {
  int ncols = (EPI == EPI_SWIGLU || EPI == EPI_DSWIGLU) ? p.I : p.N;
  dim3 grid((unsigned)ceil_div(ncols, 16), (unsigned)ceil_div(max_rows, 16),
            GMD == G_KROWS ? (unsigned)p.groups : 1u);
  gemm_f32_kernel<AM, BMD, GMD, B2, EPI, ROLE><<<grid, 256, 0, s>>>(p);
}

moe_status_t launch_gemm(bool is_bf16, GemmRole role, const GemmParams& p, int max_m_tiles,
                         hipStream_t s) {
  const char* name = role_name(role);
  ProfScope prof(name, s);
  if (!is_bf16) {
    // rows to cover: G_MROWS row capacity (passed as max_m_tiles), else M
    switch (role) {
#define X(r, n, t, a, b, g, t2, e)                        \
  case r: {                                               \
    const int rows = (g == G_MROWS) ? max_m_tiles : p.M;  \
    if (rows <= 0) return MOE_OK;                         \
    launch_f32<a, b, g, t2, e, r>(p, rows, s);            \
    break;                                                \
  }
      MOE_GEMM_ROLES(X)
#undef X
    }
    return check_launch(name);
  }
  switch (role) {
#define X(r, n, t, a, b, g, t2, e)                                                        \
  case r: {                                                                               \
    const int64_t per = (int64_t)max_m_tiles * p.n_tiles;                                 \
    const int64_t grid = (g == G_KROWS) ? per * p.groups : per;                           \
    if (grid <= 0) return MOE_OK;                                                         \
    if (grid > 0x7fffffff) {                                                              \
      set_error("GEMM %s: grid too large", name);                                         \
      return MOE_ERR_UNSUPPORTED;                                                         \
    }                                                                                     \
    launch_bf16<t, a, b, g, t2, e, r>(p, (int)grid, s);                                   \
    break;                                                                                \
  }
    MOE_GEMM_ROLES(X)
#undef X
  }
  return check_launch(name);
}

}  // namespace moe
